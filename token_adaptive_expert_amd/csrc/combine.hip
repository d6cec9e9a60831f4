// Gated combine: y[t] = residual[t] + sum over the kept slots of token t, in
// slot order, of their gate-scaled expert outputs (the MoE layer output, the
// gate-weighted sum of expert maps f in "ACE: Adaptive Calibration-Free
// Expert Skipping for MoE-based LLMs", picx.dev summary page).  Skipped slots
// add nothing; the kept gates are not renormalised.  Float32 accumulation in
// a fixed order, so the result is deterministic.
#include "kernels.h"

namespace ace {

namespace {
constexpr int NTHR = 256;

template <typename T> __device__ __forceinline__ f32x4 load4(const T* p);
template <> __device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <> __device__ __forceinline__ f32x4 load4<bf16_t>(const bf16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return f32x4{bf16_to_f32(uint16_t(v.x & 0xFFFFu)), bf16_to_f32(uint16_t(v.x >> 16)),
               bf16_to_f32(uint16_t(v.y & 0xFFFFu)), bf16_to_f32(uint16_t(v.y >> 16))};
}
template <typename T> __device__ __forceinline__ void store4(T* p, f32x4 v);
template <> __device__ __forceinline__ void store4<float>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t* p, f32x4 v) {
  uint2 o;
  o.x = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
  o.y = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = o;
}
}  // namespace

// grid: (T, ceil(H / 1024)); each thread owns 4 columns of one token.  The
// slot positions are read first (one scalar load), then every kept slot's
// row is requested before the ordered sum, so the loads overlap.
template <typename T, int KMAX>
__global__ __launch_bounds__(NTHR) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.x;
  const int col = (blockIdx.y * NTHR + threadIdx.x) * 4;
  const int H = a.H, k = a.k;
  if (col >= H) return;
  const int32_t* sp = a.slot_pos + int64_t(t) * k;
  int p[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) p[i] = sp[min(i, k - 1)];
  f32x4 v[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < k && p[i] >= 0) v[i] = *reinterpret_cast<const f32x4*>(a.slot_out + int64_t(p[i]) * H + col);
  }
  const T* res = reinterpret_cast<const T*>(a.residual);
  f32x4 acc = res ? load4<T>(res + int64_t(t) * H + col) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    acc[0] += v[i][0];
    acc[1] += v[i][1];
    acc[2] += v[i][2];
    acc[3] += v[i][3];
  }
  store4<T>(reinterpret_cast<T*>(a.y) + int64_t(t) * H + col, acc);
}

template <typename T>
hipError_t launch_combine_t(const CombineArgs& a, hipStream_t s) {
  const dim3 grid(a.T, (a.H + NTHR * 4 - 1) / (NTHR * 4)), block(NTHR);
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
