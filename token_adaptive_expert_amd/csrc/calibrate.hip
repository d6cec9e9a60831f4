// Per-layer thresholds by quantile mapping, on the device.
//
// Method: "ACE: Adaptive Calibration-Free Expert Skipping for MoE-based LLMs"
// (picx.dev summary page), Efficiency Results (Table 6: thresholds come from
// quantile mapping) with max-fusion and the top-1 rule of Methodology
// section 3; the article page on ACE adds that thresholds are matched to the
// workload's own tokens.
//
// Reading of "quantile mapping" (the page gives no detail): over the eligible
// slots (every routed slot but the top-1), each view's scores are ranked
// ascending (ties by slot order t, then i).  A slot's fused rank is the larger
// of its two view ranks, max-fusion applied to the two empirical quantiles.
// For a target skip rate ρ over all T*k slots, n = floor(ρ*T*k + 1/2); the
// level m is the largest with #{fused rank < m} <= n, and each view's
// threshold lies strictly between its (m-1)-th and m-th smallest score, so
// "both scores below their thresholds" selects exactly the slots of fused
// rank < m.
//
// A slot's rank in a view is the number of eligible slots with a smaller
// (score, slot) key: unique 64-bit keys (the score's order-preserving bits,
// then the slot index) make "ties by slot order" a plain comparison.
// Kernel 1 sorts the keys of each tile of CALIB_TILE slots in LDS (bitonic
// network); kernel 2 gives every slot its rank as the sum, over the tiles,
// of the number of keys below its own (a binary search in the tile, staged
// in LDS): O(N log N) work per tile pass instead of N^2 compares.  Kernel 3
// (one workgroup) binary-searches m and places the two thresholds.
#include "kernels.h"

namespace ace {

namespace {
constexpr int RT = 256;     // threads (and LDS tile) of the rank kernel
constexpr int FT = 1024;    // threads of the finishing kernel

__device__ __forceinline__ void slot_scores(const CalibArgs& a, int j, float* sg, float* sr) {
  const int km1 = a.k - 1;
  const int t = j / km1, i = 1 + j % km1;
  const int64_t o = int64_t(t) * a.k + i;
  const float g = a.gate[o];
  const int e = a.idx[o];
  *sg = g * a.a_gsp[e];
  *sr = g * a.a_rcr[e];
}
}  // namespace

// Order-preserving 32-bit image of a float (finite values and +-0).
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ void slot_keys(const CalibArgs& a, int j, uint64_t* kg, uint64_t* kr, float* sg,
                                          float* sr) {
  slot_scores(a, j, sg, sr);
  *kg = (uint64_t(ordered_bits(*sg)) << 32) | uint32_t(j);
  *kr = (uint64_t(ordered_bits(*sr)) << 32) | uint32_t(j);
}

// Kernel 1: keys of one tile sorted ascending in LDS (bitonic network, one
// compare-exchange pair per thread per stage); slots past N get the largest key.
__global__ __launch_bounds__(CALIB_TILE / 2) void calib_tile_sort_kernel(CalibArgs a) {
  constexpr int TL = CALIB_TILE;
  __shared__ uint64_t s_k[2][TL];
  const int tid = threadIdx.x;
  const int base = blockIdx.x * TL;
  for (int u = tid; u < TL; u += TL / 2) {
    uint64_t kg = ~uint64_t(0), kr = ~uint64_t(0);
    float sg, sr;
    if (base + u < a.N) slot_keys(a, base + u, &kg, &kr, &sg, &sr);
    s_k[0][u] = kg;
    s_k[1][u] = kr;
  }
  __syncthreads();
  for (int kk = 2; kk <= TL; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      const int i = (tid / jj) * 2 * jj + (tid % jj), ixj = i + jj;  // pair (i, i ^ jj), i < ixj
      const bool asc = (i & kk) == 0;
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const uint64_t x = s_k[v][i], y = s_k[v][ixj];
        if ((x > y) == asc) {
          s_k[v][i] = y;
          s_k[v][ixj] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int u = tid; u < TL; u += TL / 2) {
    a.ws_key_g[base + u] = s_k[0][u];
    a.ws_key_r[base + u] = s_k[1][u];
  }
}

// Number of keys below x in a sorted LDS tile of CALIB_TILE keys.
__device__ __forceinline__ int count_below(const uint64_t* s, uint64_t x) {
  int pos = 0;
#pragma unroll
  for (int step = CALIB_TILE; step > 0; step >>= 1)
    if (pos + step <= CALIB_TILE && s[pos + step - 1] < x) pos += step;
  return pos;
}

// Kernel 2: ranks in both views, and the scores in rank order.
__global__ __launch_bounds__(RT) void calib_rank_kernel(CalibArgs a) {
  __shared__ uint64_t s_k[2][CALIB_TILE];
  const int N = a.N;
  const int j = blockIdx.x * RT + threadIdx.x;
  uint64_t kg = 0, kr = 0;
  float mg = 0.f, mr = 0.f;
  if (j < N) slot_keys(a, j, &kg, &kr, &mg, &mr);
  int rg = 0, rr = 0;
  const int ntiles = (N + CALIB_TILE - 1) / CALIB_TILE;
  for (int t = 0; t < ntiles; ++t) {
    for (int u = threadIdx.x; u < CALIB_TILE; u += RT) {
      s_k[0][u] = a.ws_key_g[int64_t(t) * CALIB_TILE + u];
      s_k[1][u] = a.ws_key_r[int64_t(t) * CALIB_TILE + u];
    }
    __syncthreads();
    rg += count_below(s_k[0], kg);
    rr += count_below(s_k[1], kr);
    __syncthreads();
  }
  if (j < N) {
    a.ws_rank_g[j] = rg;
    a.ws_rank_r[j] = rr;
    a.ws_score_g[rg] = mg;   // ranks are a permutation: sorted scores
    a.ws_score_r[rr] = mr;
  }
}

__global__ __launch_bounds__(FT) void calib_finish_kernel(CalibArgs a) {
  __shared__ int s_cnt[FT / 64];
  __shared__ int s_lo, s_hi;
  const int N = a.N, n = a.n_target;
  const int tid = threadIdx.x;
  if (n == 0 || N == 0) {
    if (tid == 0) {
      a.tau_out[0] = 0.f;
      a.tau_out[1] = 0.f;
      if (a.level_out) {
        a.level_out[0] = 0;
        a.level_out[1] = n;
      }
    }
    return;
  }
  // largest m in [0, N] with #{max(rank_g, rank_r) < m} <= n
  if (tid == 0) {
    s_lo = 0;   // count(0) = 0 <= n
    s_hi = N;   // candidate upper end
  }
  __syncthreads();
  int m;
  if (n >= N) {
    m = N;
  } else {
    // invariant: count(lo) <= n < count(hi) (count(N) = N > n)
    while (true) {
      const int lo = s_lo, hi = s_hi;
      __syncthreads();
      if (hi - lo <= 1) {
        m = lo;
        break;
      }
      const int mid = (lo + hi) >> 1;
      int c = 0;
      for (int j = tid; j < N; j += FT) c += (max(a.ws_rank_g[j], a.ws_rank_r[j]) < mid) ? 1 : 0;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
      if ((tid & 63) == 0) s_cnt[tid >> 6] = c;
      __syncthreads();
      if (tid == 0) {
        int tot = 0;
        for (int w = 0; w < FT / 64; ++w) tot += s_cnt[w];
        if (tot <= n) s_lo = mid; else s_hi = mid;
      }
      __syncthreads();
    }
  }
  if (tid == 0) {
    float tau[2];
    for (int v = 0; v < 2; ++v) {
      const float* srt = v == 0 ? a.ws_score_g : a.ws_score_r;
      if (m >= N) {
        tau[v] = nextafterf(srt[N - 1], INFINITY);
      } else {
        const float lo = srt[m - 1], hi = srt[m];
        float t = float((double(lo) + double(hi)) * 0.5);
        if (!(t > lo)) t = nextafterf(lo, INFINITY);
        tau[v] = t;
      }
    }
    a.tau_out[0] = tau[0];
    a.tau_out[1] = tau[1];
    if (a.level_out) {
      a.level_out[0] = m;
      a.level_out[1] = n;
    }
  }
}

size_t calib_workspace_bytes(int T, int k) {
  const size_t N = size_t(T) * size_t(k > 1 ? k - 1 : 0);
  const size_t npad = (N + CALIB_TILE - 1) / CALIB_TILE * CALIB_TILE;
  return 4 * ((N * sizeof(int32_t) + 255) & ~size_t(255)) + 2 * npad * sizeof(uint64_t);
}

hipError_t launch_calibrate(CalibArgs a, void* workspace, hipStream_t s) {
  const size_t stride = (size_t(a.N) * sizeof(int32_t) + 255) & ~size_t(255);
  const size_t npad = (size_t(a.N) + CALIB_TILE - 1) / CALIB_TILE * CALIB_TILE;
  uint8_t* w = static_cast<uint8_t*>(workspace);
  a.ws_rank_g = reinterpret_cast<int32_t*>(w);
  a.ws_rank_r = reinterpret_cast<int32_t*>(w + stride);
  a.ws_score_g = reinterpret_cast<float*>(w + 2 * stride);
  a.ws_score_r = reinterpret_cast<float*>(w + 3 * stride);
  a.ws_key_g = reinterpret_cast<uint64_t*>(w + 4 * stride);
  a.ws_key_r = reinterpret_cast<uint64_t*>(w + 4 * stride + npad * sizeof(uint64_t));
  if (a.N > 0 && a.n_target > 0) {
    hipLaunchKernelGGL(calib_tile_sort_kernel, dim3(unsigned(npad / CALIB_TILE)), dim3(CALIB_TILE / 2), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(calib_rank_kernel, dim3((a.N + RT - 1) / RT), dim3(RT), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(calib_finish_kernel, dim3(1), dim3(FT), 0, s, a);
  return hipGetLastError();
}

}  // namespace ace
