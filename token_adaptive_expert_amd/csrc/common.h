// Shared device helpers for the gfx950 kernels: storage types, bf16 rounding,
// wave reductions and the MFMA fragment types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ace {

// bf16 is stored as its 16-bit pattern (the upper half of an IEEE float32).
struct bf16_t {
  uint16_t bits;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float32 -> bf16, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Storage traits: a 16-byte lane load holds EPL elements of the type.
template <typename T> struct St;
template <> struct St<float> {
  static constexpr int EPL = 4;
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};
template <> struct St<bf16_t> {
  static constexpr int EPL = 8;
  __device__ static float to_f32(bf16_t v) { return bf16_to_f32(v.bits); }
  __device__ static bf16_t from_f32(float v) { return bf16_t{f32_to_bf16(v)}; }
};

// Wave64 reductions (all lanes get the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Wave64 sum through DPP row shifts (inclusive scan within each row of 16
// lanes) and the four row totals read from lanes 15, 31, 47, 63, added in
// that order; every lane gets the result.  No LDS round trips.
__device__ __forceinline__ float wave_sum_dpp(float v) {
#define ACE_DPP_ADD(CTRL) \
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false))
  ACE_DPP_ADD(0x111);
  ACE_DPP_ADD(0x112);
  ACE_DPP_ADD(0x114);
  ACE_DPP_ADD(0x118);
#undef ACE_DPP_ADD
  const int b = __float_as_int(v);
  return ((__int_as_float(__builtin_amdgcn_readlane(b, 15)) + __int_as_float(__builtin_amdgcn_readlane(b, 31))) +
          __int_as_float(__builtin_amdgcn_readlane(b, 47))) +
         __int_as_float(__builtin_amdgcn_readlane(b, 63));
}

// Inclusive prefix sum of an int over the 64 lanes of a wave (lane order):
// DPP row shifts build the sums within rows of 16 lanes, then two row
// broadcasts carry the totals of rows 0 and 0-1 forward.  No LDS round
// trips; all lanes must be active.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Buffer resource for raw (untyped) buffer loads: base address and size in
// bytes; loads past the size return zero.  The last dword holds the gfx9-family
// raw-buffer format bits.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}
// 16-byte buffer load at byte offset voff (per lane) + soff (uniform).
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// 16-byte buffer load straight into LDS (no registers): lane l's 16 bytes from
// byte offset voff (per lane) + soff (uniform) land at lds + 16*l, lds being
// wave-uniform.  Completion is counted by vmcnt like any vector memory load.
// (A plain function, not a template, so that the host pass of a kernel
// template that calls it still emits the kernel's launch stub.)
__device__ __forceinline__ void buf_ld16_lds(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// MFMA wrappers.  Fragment layouts (checked on gfx950):
//  16x16x32 bf16: lane l holds A[l%16][8*(l/16)+j] and B[8*(l/16)+j][l%16], j<8;
//  16x16x4 f32:   lane l holds A[l%16][l/16] and B[l/16][l%16];
//  both:          lane l holds D[4*(l/16)+j][l%16], j<4.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One 16-byte fragment pair -> MFMA accumulate.  A 16-byte lane load covers a
// "k-step": 32 bf16 values (one 16x16x32 MFMA) or 16 f32 values (four 16x16x4
// MFMAs; lane group q holds k = 4q..4q+3 and MFMA j takes element j, the same
// k permutation on both operands, so the sum over k is unchanged).
template <typename T> __device__ __forceinline__ f32x4 mma_step(u32x4 a, u32x4 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mma_step<bf16_t>(u32x4 a, u32x4 b, f32x4 c) { return mfma_bf16(a, b, c); }
template <> __device__ __forceinline__ f32x4 mma_step<float>(u32x4 a, u32x4 b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c = mfma_f32(__uint_as_float(a[j]), __uint_as_float(b[j]), c);
  return c;
}

// Exact three-term bf16 split of 8 float32 values: v = hi + mid + lo, each
// term rounded to nearest even.  24 significant bits = 3 x 8, and each residual
// is exact in float32, so bf16 MFMAs against the three planes form exact
// float32 products.  planes[p] holds term p of the 8 values, packed in order.
__device__ __forceinline__ void split3_f8(const float (&ww)[8], u32x4* planes) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint16_t h2[2], m2[2], l2[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float v = ww[2 * j + p];
      h2[p] = f32_to_bf16(v);
      const float r1 = v - bf16_to_f32(h2[p]);
      m2[p] = f32_to_bf16(r1);
      const float r2 = r1 - bf16_to_f32(m2[p]);
      l2[p] = f32_to_bf16(r2);
    }
    planes[0][j] = uint32_t(h2[0]) | (uint32_t(h2[1]) << 16);
    planes[1][j] = uint32_t(m2[0]) | (uint32_t(m2[1]) << 16);
    planes[2][j] = uint32_t(l2[0]) | (uint32_t(l2[1]) << 16);
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace ace
