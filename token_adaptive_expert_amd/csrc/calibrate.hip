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
// Kernel 1 ranks every eligible slot in both views by counting, against LDS
// tiles of all scores (O(N^2) compares, which is cheap at calibration sizes
// and needs no sort).  Kernel 2 (one workgroup) binary-searches m and places
// the two thresholds.
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

__global__ __launch_bounds__(RT) void calib_rank_kernel(CalibArgs a) {
  __shared__ float s_g[RT], s_r[RT];
  const int N = a.N;
  const int j = blockIdx.x * RT + threadIdx.x;
  float mg = 0.f, mr = 0.f;
  if (j < N) slot_scores(a, j, &mg, &mr);
  int rg = 0, rr = 0;
  for (int base = 0; base < N; base += RT) {
    const int jj = base + threadIdx.x;
    if (jj < N) slot_scores(a, jj, &s_g[threadIdx.x], &s_r[threadIdx.x]);
    __syncthreads();
    const int lim = min(RT, N - base);
    for (int u = 0; u < lim; ++u) {
      const int o = base + u;
      const float vg = s_g[u], vr = s_r[u];
      rg += (vg < mg || (vg == mg && o < j)) ? 1 : 0;
      rr += (vr < mr || (vr == mr && o < j)) ? 1 : 0;
    }
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
  return 4 * ((N * sizeof(int32_t) + 255) & ~size_t(255));
}

hipError_t launch_calibrate(CalibArgs a, void* workspace, hipStream_t s) {
  const size_t stride = (size_t(a.N) * sizeof(int32_t) + 255) & ~size_t(255);
  uint8_t* w = static_cast<uint8_t*>(workspace);
  a.ws_rank_g = reinterpret_cast<int32_t*>(w);
  a.ws_rank_r = reinterpret_cast<int32_t*>(w + stride);
  a.ws_score_g = reinterpret_cast<float*>(w + 2 * stride);
  a.ws_score_r = reinterpret_cast<float*>(w + 3 * stride);
  if (a.N > 0 && a.n_target > 0) {
    hipLaunchKernelGGL(calib_rank_kernel, dim3((a.N + RT - 1) / RT), dim3(RT), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(calib_finish_kernel, dim3(1), dim3(FT), 0, s, a);
  return hipGetLastError();
}

}  // namespace ace
