// Gated combine: y[t] = residual[t] + sum over the kept slots of token t, in
// slot order, of their gate-scaled expert outputs (the MoE layer output, the
// gate-weighted sum of expert maps f in "ACE: Adaptive Calibration-Free
// Expert Skipping for MoE-based LLMs", picx.dev summary page).  Skipped slots
// add nothing; the kept gates are not renormalised.  Float32 accumulation in
// a fixed order, so the result is deterministic.
#include "kernels.h"

namespace ace {

namespace {
constexpr int NW = 4;

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

template <typename T>
__global__ __launch_bounds__(NW * 64) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.x * NW + wave_id();
  if (t >= a.T) return;
  const int l = lane_id(), H = a.H, k = a.k;
  const T* res = reinterpret_cast<const T*>(a.residual);
  T* y = reinterpret_cast<T*>(a.y);
  for (int col = l * 4; col < H; col += 256) {
    f32x4 acc = res ? load4<T>(res + int64_t(t) * H + col) : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < k; ++i) {
      const int p = a.slot_pos[int64_t(t) * k + i];
      if (p >= 0) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(a.slot_out + int64_t(p) * H + col);
        acc[0] += v[0];
        acc[1] += v[1];
        acc[2] += v[2];
        acc[3] += v[3];
      }
    }
    store4<T>(y + int64_t(t) * H + col, acc);
  }
}

hipError_t launch_combine(int dtype, const CombineArgs& a, hipStream_t s) {
  const dim3 grid((a.T + NW - 1) / NW), block(NW * 64);
  if (dtype == 1)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace ace
