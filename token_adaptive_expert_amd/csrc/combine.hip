// Gated combine: y[t] = residual[t] + sum over the kept slots of token t, in
// slot order, of their gate-scaled expert outputs (the MoE layer output, the
// gate-weighted sum of expert maps f in "ACE: Adaptive Calibration-Free
// Expert Skipping for MoE-based LLMs", picx.dev summary page).  Skipped slots
// add nothing; the kept gates are not renormalised.  The slot rows are in the
// layer's dtype; float32 accumulation in a fixed order, so the result is
// deterministic.
#include "kernels.h"

namespace ace {

namespace {
constexpr int NTHR = 256;

// 16 bytes of T (8 bf16 or 4 float32 values) as float32, and back (the
// store rounds to nearest even).
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float (&v)[N]) {
    const f32x4 r = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = r[j];
  }
  __device__ static void store(float* p, const float (&v)[N]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  }
};
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  __device__ static void load(const bf16_t* p, float (&v)[N]) {
    const u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_to_f32(uint16_t(r[j] & 0xFFFFu));
      v[2 * j + 1] = bf16_to_f32(uint16_t(r[j] >> 16));
    }
  }
  __device__ static void store(bf16_t* p, const float (&v)[N]) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = uint32_t(f32_to_bf16(v[2 * j])) | (uint32_t(f32_to_bf16(v[2 * j + 1])) << 16);
    *reinterpret_cast<u32x4*>(p) = r;
  }
};
}  // namespace

// grid: (T, ceil(H / (256 * C))); each thread owns C = 16 / sizeof(T)
// columns of one token (one 16-byte load per slot row).  The slot positions
// are read first (one scalar load), then every kept slot's row is requested
// before the ordered sum, so the loads overlap.
template <typename T, int KMAX>
__global__ __launch_bounds__(NTHR) void combine_kernel(CombineArgs a) {
  using V = Vec16<T>;
  constexpr int C = V::N;
  const int t = blockIdx.x;
  const int col = (blockIdx.y * NTHR + threadIdx.x) * C;
  const int H = a.H, k = a.k;
  if (col >= H) return;
  const int32_t* sp = a.slot_pos + int64_t(t) * k;
  int p[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) p[i] = sp[min(i, k - 1)];
  const T* so = reinterpret_cast<const T*>(a.slot_out);
  float v[KMAX][C];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    if (i < k && p[i] >= 0) {
      V::load(so + int64_t(p[i]) * H + col, v[i]);
    } else {
#pragma unroll
      for (int j = 0; j < C; ++j) v[i][j] = 0.f;
    }
  }
  const T* res = reinterpret_cast<const T*>(a.residual);
  float acc[C];
  if (res) {
    V::load(res + int64_t(t) * H + col, acc);
  } else {
#pragma unroll
    for (int j = 0; j < C; ++j) acc[j] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < KMAX; ++i)
#pragma unroll
    for (int j = 0; j < C; ++j) acc[j] += v[i][j];
  V::store(reinterpret_cast<T*>(a.y) + int64_t(t) * H + col, acc);
}

template <typename T>
hipError_t launch_combine_t(const CombineArgs& a, hipStream_t s) {
  constexpr int C = Vec16<T>::N;
  const dim3 grid(a.T, (a.H + NTHR * C - 1) / (NTHR * C)), block(NTHR);
  if (a.k <= 4)
    hipLaunchKernelGGL((combine_kernel<T, 4>), grid, block, 0, s, a);
  else if (a.k <= 8)
    hipLaunchKernelGGL((combine_kernel<T, 8>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((combine_kernel<T, 16>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(int dtype, const CombineArgs& a, hipStream_t s) {
  return dtype == 1 ? launch_combine_t<bf16_t>(a, s) : launch_combine_t<float>(a, s);
}

}  // namespace ace
