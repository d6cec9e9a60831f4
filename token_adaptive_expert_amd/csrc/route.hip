// RMSNorm + router + top-k gates + ACE skip mask, one workgroup per 16 tokens.
//
// Method: "ACE: Adaptive Calibration-Free Expert Skipping for MoE-based LLMs"
// (picx.dev summary page).  h = x̄Γ is the RMSNorm output (Theoretical
// Foundation); the slot scores are g·A^GSP(e) and g·A^RCR(e) (Methodology
// sections 1 and 2); a slot is skipped only when both fall below their
// thresholds, and the top-1 slot is always kept (Methodology section 3).
#include "kernels.h"

namespace ace {

namespace {

constexpr int TB = 16;        // tokens per workgroup
constexpr int NTHR = 256;     // 4 waves
constexpr int EMAX = 256;

// h for EPL consecutive hidden units of one token, rounded to the storage type.
// The same function feeds h_out and the router's A operand, so both see the
// same values.
template <typename T> __device__ __forceinline__ u32x4 make_h(u32x4 xr, float inv, const float* gamma_k);

template <> __device__ __forceinline__ u32x4 make_h<bf16_t>(u32x4 xr, float inv, const float* g) {
  const f32x4 g0 = *reinterpret_cast<const f32x4*>(g);
  const f32x4 g1 = *reinterpret_cast<const f32x4*>(g + 4);
  float gg[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = (bf16_to_f32(uint16_t(xr[j] & 0xFFFFu)) * inv) * gg[2 * j];
    const float hi = (bf16_to_f32(uint16_t(xr[j] >> 16)) * inv) * gg[2 * j + 1];
    out[j] = uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
  }
  return out;
}

template <> __device__ __forceinline__ u32x4 make_h<float>(u32x4 xr, float inv, const float* g) {
  const f32x4 g0 = *reinterpret_cast<const f32x4*>(g);
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = __float_as_uint((__uint_as_float(xr[j]) * inv) * g0[j]);
  return out;
}

template <typename T> __device__ __forceinline__ float sumsq16(u32x4 v);
template <> __device__ __forceinline__ float sumsq16<bf16_t>(u32x4 v) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = bf16_to_f32(uint16_t(v[j] & 0xFFFFu)), b = bf16_to_f32(uint16_t(v[j] >> 16));
    s += a * a;
    s += b * b;
  }
  return s;
}
template <> __device__ __forceinline__ float sumsq16<float>(u32x4 v) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += __uint_as_float(v[j]) * __uint_as_float(v[j]);
  return s;
}

// Router product for one 16-token x 16-expert block and one k-step.
// bf16: each float32 router weight w is split exactly into three bf16 terms
// (w = hi + mid + lo; 24 significant bits = 3 x 8), so the three bf16 MFMAs
// form exact products of the bf16 h with the full float32 weight and
// accumulate them in float32.
template <typename T> __device__ __forceinline__ f32x4 router_step(u32x4 a, const float* wrow, bool ok, f32x4 acc);

template <> __device__ __forceinline__ f32x4 router_step<bf16_t>(u32x4 a, const float* w, bool ok, f32x4 acc) {
  f32x4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = {0.f, 0.f, 0.f, 0.f};
  if (ok) {
    w0 = *reinterpret_cast<const f32x4*>(w);
    w1 = *reinterpret_cast<const f32x4*>(w + 4);
  }
  float ww[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
  u32x4 hi, mid, lo;
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
    hi[j] = uint32_t(h2[0]) | (uint32_t(h2[1]) << 16);
    mid[j] = uint32_t(m2[0]) | (uint32_t(m2[1]) << 16);
    lo[j] = uint32_t(l2[0]) | (uint32_t(l2[1]) << 16);
  }
  acc = mfma_bf16(a, hi, acc);
  acc = mfma_bf16(a, mid, acc);
  acc = mfma_bf16(a, lo, acc);
  return acc;
}

template <> __device__ __forceinline__ f32x4 router_step<float>(u32x4 a, const float* w, bool ok, f32x4 acc) {
  u32x4 b = {0u, 0u, 0u, 0u};
  if (ok) b = ld16(w);
  return mma_step<float>(a, b, acc);
}

}  // namespace

template <typename T>
__global__ __launch_bounds__(NTHR) void route_skip_kernel(RouteArgs a) {
  __shared__ float s_inv[TB];
  __shared__ float s_logit[TB][EMAX + 1];
  __shared__ double s_z[NTHR / 64][EMAX];

  constexpr int EPL = St<T>::EPL;
  const int w = wave_id(), l = lane_id();
  const int tok0 = blockIdx.x * TB;
  const int H = a.H, E = a.E, k = a.k;
  const T* x = reinterpret_cast<const T*>(a.x);

  // 1. inverse RMS of each token (wave w: tokens 4w..4w+3)
  for (int r = 0; r < 4; ++r) {
    const int tl = w * 4 + r, t = tok0 + tl;
    float ss = 0.f;
    if (t < a.T) {
      const T* row = x + int64_t(t) * H;
      for (int j = l * EPL; j < H; j += 64 * EPL) ss += sumsq16<T>(ld16(row + j));
    }
    ss = wave_sum(ss);
    if (l == 0) s_inv[tl] = 1.0f / sqrtf(ss / float(H) + a.eps);
  }
  __syncthreads();

  // 2. h_out rows of this workgroup
  {
    const int segs = H / EPL;  // 16-byte segments per row
    for (int u = threadIdx.x; u < TB * segs; u += NTHR) {
      const int tl = u / segs, j = (u % segs) * EPL, t = tok0 + tl;
      if (t < a.T) {
        const u32x4 hv = make_h<T>(ld16(x + int64_t(t) * H + j), s_inv[tl], a.gamma + j);
        st16(reinterpret_cast<T*>(a.h_out) + int64_t(t) * H + j, hv);
      }
    }
  }

  // 3. logits into LDS
  if (a.logits_in != nullptr) {
    for (int u = threadIdx.x; u < TB * E; u += NTHR) {
      const int tl = u / E, e = u % E, t = tok0 + tl;
      s_logit[tl][e] = (t < a.T) ? a.logits_in[int64_t(t) * E + e] : 0.f;
    }
  } else {
    const int ncb = (E + 15) / 16;  // 16-expert column blocks, round-robin over waves
    const int q = l >> 4, r16 = l & 15;
    const int t = tok0 + r16;
    const bool tok_ok = t < a.T;
    const float inv = s_inv[r16];
    const T* xrow = x + int64_t(tok_ok ? t : 0) * H;
    f32x4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk < H; kk += 4 * EPL) {
      const int kb = kk + q * EPL;
      u32x4 af = {0u, 0u, 0u, 0u};
      if (tok_ok) af = make_h<T>(ld16(xrow + kb), inv, a.gamma + kb);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int cb = w + 4 * c;
        if (cb < ncb) {
          const int e = cb * 16 + r16;
          acc[c] = router_step<T>(af, a.w_router + int64_t(e < E ? e : 0) * H + kb, e < E, acc[c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int cb = w + 4 * c;
      const int e = cb * 16 + r16;
      if (cb < ncb && e < E) {
        const float b = a.bias ? a.bias[e] : 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) s_logit[4 * q + j][e] = acc[c][j] + b;
      }
    }
  }
  __syncthreads();

  if (a.logits_out != nullptr) {
    for (int u = threadIdx.x; u < TB * E; u += NTHR) {
      const int tl = u / E, e = u % E, t = tok0 + tl;
      if (t < a.T) a.logits_out[int64_t(t) * E + e] = s_logit[tl][e];
    }
  }

  // 4. top-k, gates, skip mask: one wave per token
  const int R = (E + 63) / 64;
  for (int r = 0; r < 4; ++r) {
    const int tl = w * 4 + r, t = tok0 + tl;
    if (t >= a.T) break;
    float v[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int e = l + 64 * rr;
      v[rr] = (rr < R && e < E) ? s_logit[tl][e] : 0.f;
    }
    uint32_t taken = 0;
    int my_e = 0;
    float my_logit = 0.f, top_logit = 0.f;
    for (int i = 0; i < k; ++i) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int e = l + 64 * rr;
        if (rr < R && e < E && !((taken >> rr) & 1u)) {
          if (v[rr] > bv || (v[rr] == bv && e < bi)) {
            bv = v[rr];
            bi = e;
          }
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & 63) == l) taken |= 1u << (bi >> 6);
      if (l == i) {
        my_e = bi;
        my_logit = bv;
      }
      if (i == 0) top_logit = bv;
    }
    // softmax in float64, shifted by the top-1 logit
    const double m = double(top_logit);
    const double z = (l < k) ? exp(double(my_logit) - m) : 0.0;
    double s = 0.0;
    if (a.norm_topk) {
      for (int i = 0; i < k; ++i) s += __shfl(z, i, 64);
    } else {
      for (int e = l; e < E; e += 64) s_z[w][e] = exp(double(s_logit[tl][e]) - m);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int e = 0; e < E; ++e) s += s_z[w][e];
      __builtin_amdgcn_wave_barrier();
    }
    if (l < k) {
      const float g = float(z / s);
      bool keep = true;
      if (l > 0) {
        const float sg = g * a.a_gsp[my_e];
        const float sr = g * a.a_rcr[my_e];
        const bool lg = sg < a.tau_gsp, lr = sr < a.tau_rcr;
        bool skip;
        switch (a.fusion) {
          case 1: skip = lg || lr; break;
          case 2:
            skip = a.tau_gsp > 0.f && a.tau_rcr > 0.f &&
                   0.5 * (double(sg) / double(a.tau_gsp) + double(sr) / double(a.tau_rcr)) < 1.0;
            break;
          case 3: skip = lg; break;
          case 4: skip = lr; break;
          case 5: skip = g < a.tau_gsp; break;
          default: skip = lg && lr; break;
        }
        keep = !skip;
      }
      const int64_t o = int64_t(t) * k + l;
      a.topk_idx[o] = my_e;
      a.topk_gate[o] = g;
      a.keep[o] = keep ? 1 : 0;
    }
  }
}

int route_tokens_per_block() { return TB; }

hipError_t launch_route(int dtype, const RouteArgs& a, hipStream_t s) {
  const dim3 grid((a.T + TB - 1) / TB), block(NTHR);
  if (dtype == 1)
    hipLaunchKernelGGL(route_skip_kernel<bf16_t>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(route_skip_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace ace
