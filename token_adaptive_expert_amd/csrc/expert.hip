// Grouped expert GEMMs over the dispatched slots, on MFMA.
//
// Method: the SwiGLU expert f(x) = (SiLU(x̄ΓW^gate) ⊙ x̄ΓW^up) W^down
// ("ACE: Adaptive Calibration-Free Expert Skipping for MoE-based LLMs",
// picx.dev summary page, Theoretical Foundation), applied to each kept slot
// and scaled by its router gate.
//
// Work unit ("tile"): one expert, up to BM = 16*RB of its sorted slot rows,
// and NW*32 of its weight rows.  Each wave owns 32 weight rows (two 16-row
// groups): for gate/up the 16 gate rows and the 16 up rows of the same
// intermediate units, so SiLU(gate)*up is formed in registers; for down two
// adjacent groups of 16 output columns.  The contraction runs in chunks of
// 256 bytes per row (4 k-steps of one 16-byte lane load each):
//   - weight fragments are loaded straight from HBM into registers in MFMA
//     operand layout (each weight byte is read once per tile), one chunk
//     ahead of the MFMAs;
//   - the slot rows (gathered token rows of h, or act rows) are staged
//     through LDS, double-buffered, and shared by all waves of the tile.
// The grid is persistent: every workgroup derives the tile list from
// expert_offsets (experts with no kept slot produce no tile, so their
// weights are never read) and strides over it.
#include "kernels.h"

namespace ace {

namespace {

constexpr int ROWB = 256;        // bytes of one row per chunk
constexpr int LDS_PITCH = 272;   // padded row pitch in LDS (16 B pad: conflict-free fragment reads)

template <typename T, int RB, int NW, int KIND>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(RB == 1 ? 4 : 2)))
void expert_gemm_kernel(ExpertArgs a) {
  constexpr int EPL = St<T>::EPL;
  constexpr int KS = 4 * EPL;      // k values per k-step
  constexpr int KC = 4 * KS;       // k values per chunk
  constexpr int BM = 16 * RB;
  constexpr int NTHR = NW * 64;
  constexpr int UNITS = BM * (ROWB / 16);   // 16-byte units of one staged chunk
  constexpr int UPT = (UNITS + NTHR - 1) / NTHR;
  constexpr int ROWS_PER_WG = (KIND == 0) ? NW * 16 : NW * 32;  // output columns per tile

  __shared__ __attribute__((aligned(16))) uint8_t s_x[2][BM * LDS_PITCH];
  __shared__ int32_t s_pref[257];
  __shared__ int32_t s_off[257];

  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int q = l >> 4, r16 = l & 15;
  const int E = a.E, K = a.K, N = a.N;
  const int nch = K / KC;
  const int nb_count = N / ROWS_PER_WG;

  // tile list: per-expert m-tile counts, exclusive prefix (wave 0)
  if (w == 0) {
    int cnt[4], loc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = l * 4 + j;
      int c = 0;
      if (e < E) {
        const int o0 = a.offsets[e], o1 = a.offsets[e + 1];
        s_off[e] = o0;
        c = (o1 - o0 + BM - 1) / BM;
      }
      cnt[j] = c;
      loc += c;
    }
    int inc = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (l >= o) inc += v;
    }
    int run = inc - loc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = l * 4 + j;
      if (e < E) s_pref[e] = run;
      run += cnt[j];
    }
    if (l == 63) s_pref[E] = inc;
    if (l == 0) s_off[E] = a.offsets[E];
  }
  __syncthreads();

  const int total_mt = s_pref[E];
  const int ntiles = total_mt * nb_count;
  const T* A = reinterpret_cast<const T*>(a.A);

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int mt = tile % total_mt;
    const int nb = tile / total_mt;
    // expert of this m-tile: last e with s_pref[e] <= mt
    int lo = 0, hi = E;  // invariant: s_pref[lo] <= mt < s_pref[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= mt) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int row0 = s_off[e] + (mt - s_pref[e]) * BM;
    const int rows = min(BM, s_off[e + 1] - row0);
    const int nrb = (rows + 15) >> 4;

    // weight row pointers of this lane's two groups
    const T* W0 = reinterpret_cast<const T*>(a.W0);
    const T* W1 = reinterpret_cast<const T*>(a.W1);
    const T* wrow[2];
    int col0;
    if (KIND == 0) {
      col0 = nb * ROWS_PER_WG + w * 16;
      wrow[0] = W0 + (int64_t(e) * N + col0 + r16) * K + q * EPL;
      wrow[1] = W1 + (int64_t(e) * N + col0 + r16) * K + q * EPL;
    } else {
      col0 = nb * ROWS_PER_WG + w * 32;
      wrow[0] = W0 + (int64_t(e) * N + col0 + r16) * K + q * EPL;
      wrow[1] = W0 + (int64_t(e) * N + col0 + 16 + r16) * K + q * EPL;
    }

    // staged-row sources of this thread's units
    const T* xsrc[UPT];
    int xoff[UPT];
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = tid + u * NTHR;
      const int r = unit >> 4, seg = unit & 15;
      xoff[u] = r * LDS_PITCH + seg * 16;
      xsrc[u] = nullptr;
      if (unit < UNITS && r < rows) {
        const int64_t src_row = (KIND == 0) ? int64_t(a.sorted_token[row0 + r]) : int64_t(row0 + r);
        xsrc[u] = A + src_row * K + seg * EPL;
      }
    }

    f32x4 acc[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb][0] = acc[rb][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 wr[2][4], wn[2][4], xr[UPT];
    // prologue: chunk 0
#pragma unroll
    for (int u = 0; u < UPT; ++u) xr[u] = xsrc[u] ? ld16(xsrc[u]) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int s = 0; s < 4; ++s) wr[g][s] = ld16(wrow[g] + s * KS);
#pragma unroll
    for (int u = 0; u < UPT; ++u)
      if (tid + u * NTHR < UNITS) *reinterpret_cast<u32x4*>(&s_x[0][xoff[u]]) = xr[u];
    __syncthreads();

    int buf = 0;
    for (int c = 0; c < nch; ++c) {
      const bool more = c + 1 < nch;
      if (more) {
        const int koff = (c + 1) * KC;
#pragma unroll
        for (int u = 0; u < UPT; ++u) xr[u] = xsrc[u] ? ld16(xsrc[u] + koff) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int s = 0; s < 4; ++s) wn[g][s] = ld16(wrow[g] + koff + s * KS);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const u32x4 af =
              *reinterpret_cast<const u32x4*>(&s_x[buf][(rb * 16 + r16) * LDS_PITCH + s * 64 + q * 16]);
          acc[rb][0] = mma_step<T>(af, wr[0][s], acc[rb][0]);
          acc[rb][1] = mma_step<T>(af, wr[1][s], acc[rb][1]);
        }
      }
      if (more) {
#pragma unroll
        for (int u = 0; u < UPT; ++u)
          if (tid + u * NTHR < UNITS) *reinterpret_cast<u32x4*>(&s_x[buf ^ 1][xoff[u]]) = xr[u];
      }
      __syncthreads();
      if (more) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int s = 0; s < 4; ++s) wr[g][s] = wn[g][s];
      }
      buf ^= 1;
    }

    // epilogue
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (rb < nrb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = rb * 16 + 4 * q + j;
          if (r < rows) {
            const int64_t p = row0 + r;
            if (KIND == 0) {
              const float v = silu(acc[rb][0][j]) * acc[rb][1][j];
              reinterpret_cast<T*>(a.out)[p * N + col0 + r16] = St<T>::from_f32(v);
            } else {
              const float g = a.sorted_gate[p];
              float* o = reinterpret_cast<float*>(a.out) + p * N + col0 + r16;
              o[0] = g * acc[rb][0][j];
              o[16] = g * acc[rb][1][j];
            }
          }
        }
      }
    }
  }
}

template <typename T, int RB, int NW, int KIND>
hipError_t launch_one(const ExpertArgs& a, int ntok, int k, int num_cu, int wg_per_cu, hipStream_t s) {
  constexpr int BM = 16 * RB;
  constexpr int ROWS_PER_WG = (KIND == 0) ? NW * 16 : NW * 32;
  const int64_t slots = int64_t(ntok) * k;
  const int64_t mt_bound = (slots + BM - 1) / BM + std::min<int64_t>(a.E, slots);
  const int64_t tiles_bound = mt_bound * (a.N / ROWS_PER_WG);
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(tiles_bound, int64_t(num_cu) * wg_per_cu));
  hipLaunchKernelGGL((expert_gemm_kernel<T, RB, NW, KIND>), dim3(unsigned(grid)), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expert(int dtype, int kind, bool stream_path, const ExpertArgs& a, int T, int k, int num_cu,
                         hipStream_t s) {
  if (dtype == 1) {
    if (stream_path)
      return kind == 0 ? launch_one<bf16_t, 1, 2, 0>(a, T, k, num_cu, 8, s)
                       : launch_one<bf16_t, 1, 2, 1>(a, T, k, num_cu, 8, s);
    return kind == 0 ? launch_one<bf16_t, 4, 4, 0>(a, T, k, num_cu, 2, s)
                     : launch_one<bf16_t, 4, 4, 1>(a, T, k, num_cu, 2, s);
  }
  if (stream_path)
    return kind == 0 ? launch_one<float, 1, 2, 0>(a, T, k, num_cu, 8, s)
                     : launch_one<float, 1, 2, 1>(a, T, k, num_cu, 8, s);
  return kind == 0 ? launch_one<float, 4, 4, 0>(a, T, k, num_cu, 2, s)
                   : launch_one<float, 4, 4, 1>(a, T, k, num_cu, 2, s);
}

}  // namespace ace
