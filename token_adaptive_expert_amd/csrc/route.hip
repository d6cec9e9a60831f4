// RMSNorm + router, then top-k gates + ACE skip mask (two kernels).
//
// Method: "ACE: Adaptive Calibration-Free Expert Skipping for MoE-based LLMs"
// (picx.dev summary page).  h = x̄Γ is the RMSNorm output (Theoretical
// Foundation); the slot scores are g·A^GSP(e) and g·A^RCR(e) (Methodology
// sections 1 and 2); a slot is skipped only when both fall below their
// thresholds, and the top-1 slot is always kept (Methodology section 3).
#include "kernels.h"

namespace ace {

namespace {

constexpr int TB = 16;        // tokens per workgroup (router kernel)
constexpr int ECB = 32;       // experts per workgroup (router kernel)
constexpr int RW = 16;        // waves of the router kernel (split the hidden dimension)
constexpr int RNTHR = RW * 64;
constexpr int NTHR = 256;     // 4 waves (top-k kernel)
constexpr int EMAX = 256;

// h for EPL consecutive hidden units of one token, rounded to the storage
// type (gamma values passed in).  The same function feeds h_out and the
// router's A operand, so both see the same values.
template <typename T> __device__ __forceinline__ u32x4 make_h(u32x4 xr, float inv, const f32x4* g);

template <> __device__ __forceinline__ u32x4 make_h<bf16_t>(u32x4 xr, float inv, const f32x4* g) {
  float gg[8] = {g[0][0], g[0][1], g[0][2], g[0][3], g[1][0], g[1][1], g[1][2], g[1][3]};
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = (bf16_to_f32(uint16_t(xr[j] & 0xFFFFu)) * inv) * gg[2 * j];
    const float hi = (bf16_to_f32(uint16_t(xr[j] >> 16)) * inv) * gg[2 * j + 1];
    out[j] = uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
  }
  return out;
}

template <> __device__ __forceinline__ u32x4 make_h<float>(u32x4 xr, float inv, const f32x4* g) {
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = __float_as_uint((__uint_as_float(xr[j]) * inv) * g[0][j]);
  return out;
}

// Operands of one router k-step for one lane: x (16 bytes), gamma, and the
// float32 router weights of its two experts (8 values each for bf16 h, 4 for f32).
template <typename T> struct RouterFrag {
  static constexpr int EPL = St<T>::EPL;
  static constexpr int NG = EPL / 4;  // float4 pieces per EPL values
  u32x4 x;
  f32x4 g[NG], w0[NG], w1[NG];
  __device__ __forceinline__ void load_x(const T* xrow, const float* gamma, int k) {
    x = ld16(xrow + k);
#pragma unroll
    for (int i = 0; i < NG; ++i) g[i] = *reinterpret_cast<const f32x4*>(gamma + k + 4 * i);
  }
  __device__ __forceinline__ void load(const T* xrow, const float* gamma, const float* r0, const float* r1, int k) {
    load_x(xrow, gamma, k);
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      w0[i] = *reinterpret_cast<const f32x4*>(r0 + k + 4 * i);
      w1[i] = *reinterpret_cast<const f32x4*>(r1 + k + 4 * i);
    }
  }
};

// Router product for one 16-token x 16-expert block and one k-step.
// bf16: each float32 router weight w is split exactly into three bf16 terms
// (w = hi + mid + lo; 24 significant bits = 3 x 8), so the three bf16 MFMAs
// form exact products of the bf16 h with the full float32 weight and
// accumulate them in float32.
template <typename T> __device__ __forceinline__ f32x4 router_mma(u32x4 a, const f32x4* w, f32x4 acc);

// Exact three-term bf16 split of the 8 float32 weights of one k-step.
__device__ __forceinline__ void split3(const f32x4* w, u32x4* planes) {
  const float ww[8] = {w[0][0], w[0][1], w[0][2], w[0][3], w[1][0], w[1][1], w[1][2], w[1][3]};
  split3_f8(ww, planes);
}

__device__ __forceinline__ f32x4 mma3(u32x4 a, const u32x4* planes, f32x4 acc) {
  acc = mfma_bf16(a, planes[0], acc);
  acc = mfma_bf16(a, planes[1], acc);
  acc = mfma_bf16(a, planes[2], acc);
  return acc;
}

template <> __device__ __forceinline__ f32x4 router_mma<bf16_t>(u32x4 a, const f32x4* w, f32x4 acc) {
  u32x4 planes[3];
  split3(w, planes);
  return mma3(a, planes, acc);
}

template <> __device__ __forceinline__ f32x4 router_mma<float>(u32x4 a, const f32x4* w, f32x4 acc) {
  return mma_step<float>(a, __builtin_bit_cast(u32x4, w[0]), acc);
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

}  // namespace

// Kernel 1: RMSNorm (+ h_out) and the router product for 16 tokens x 32
// experts.  Sixteen waves split the hidden dimension: wave w takes k-steps
// w, w+16, w+32, ...  Their partial logits are summed in a fixed wave order,
// so the result does not depend on timing.  Loads are issued for two
// k-steps before either is used; token rows past T and expert rows past E
// read a clamped valid row whose results are never stored.
template <typename T>
__global__ __launch_bounds__(RNTHR) void norm_router_kernel(RouteArgs a) {
  __shared__ float s_inv[TB];
  __shared__ float s_part[RW][TB][ECB + 1];

  constexpr int EPL = St<T>::EPL;
  constexpr int KS = 4 * EPL;
  const int w = wave_id(), l = lane_id();
  const int tok0 = blockIdx.x * TB;
  const int H = a.H, E = a.E;
  const T* x = reinterpret_cast<const T*>(a.x);

  // inverse RMS: wave w owns token tok0 + w; a row is read 8 segments of
  // 64 lanes x 16 bytes at a time, all in flight together
  {
    const T* row = x + int64_t(min(tok0 + w, a.T - 1)) * H;
    constexpr int SEG = 64 * EPL;
    float ss = 0.f;
    for (int j0 = 0; j0 < H; j0 += 8 * SEG) {
      u32x4 v[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) v[b] = ld16(row + min(j0 + b * SEG + l * EPL, H - EPL));
#pragma unroll
      for (int b = 0; b < 8; ++b)
        if (j0 + b * SEG + l * EPL < H) ss += sumsq16<T>(v[b]);
    }
    ss = wave_sum(ss);
    if (l == 0) s_inv[w] = 1.0f / sqrtf(ss / float(H) + a.eps);
  }
  __syncthreads();

  const int q = l >> 4, r16 = l & 15;
  const int tt = tok0 + r16;
  const int t = min(tt, a.T - 1);
  const float inv = s_inv[r16];
  const T* xrow = x + int64_t(t) * H;
  T* hrow = reinterpret_cast<T*>(a.h_out) + int64_t(t) * H;
  const bool write_h = blockIdx.y == 0 && tt < a.T;
  const bool do_router = a.logits_in == nullptr;
  const int e0 = min(blockIdx.y * ECB + r16, E - 1), e1 = min(blockIdx.y * ECB + 16 + r16, E - 1);
  const float* w0 = a.w_router + int64_t(e0) * H;
  const float* w1 = a.w_router + int64_t(e1) * H;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int nks = H / KS;
  if constexpr (sizeof(T) == 2) {
    if (do_router && a.router_packed) {
      // pre-split planes: [3][CB][nks][64][16 B]; this workgroup's two
      // 16-expert column blocks
      const int CB = (E + 15) / 16;
      const int cb0 = min(int(blockIdx.y) * 2, CB - 1), cb1 = min(int(blockIdx.y) * 2 + 1, CB - 1);
      const uint8_t* wp = reinterpret_cast<const uint8_t*>(a.w_router);
      const int64_t plane_bytes = int64_t(CB) * nks * 1024;
      auto ldp = [&](int cb, int j, u32x4* out) {
#pragma unroll
        for (int p = 0; p < 3; ++p) out[p] = ld16(wp + p * plane_bytes + (int64_t(cb) * nks + j) * 1024 + l * 16);
      };
      for (int j0 = w; j0 < nks; j0 += 2 * RW) {
        const int j1 = min(j0 + RW, nks - 1);
        const int k0 = j0 * KS + q * EPL, k1 = j1 * KS + q * EPL;
        RouterFrag<T> f0, f1;
        u32x4 p00[3], p01[3], p10[3], p11[3];
        f0.load_x(xrow, a.gamma, k0);
        f1.load_x(xrow, a.gamma, k1);
        ldp(cb0, j0, p00);
        ldp(cb1, j0, p01);
        ldp(cb0, j1, p10);
        ldp(cb1, j1, p11);
        const u32x4 h0 = make_h<T>(f0.x, inv, f0.g);
        if (write_h) st16(hrow + k0, h0);
        acc0 = mma3(h0, p00, acc0);
        acc1 = mma3(h0, p01, acc1);
        if (j0 + RW < nks) {
          const u32x4 h1 = make_h<T>(f1.x, inv, f1.g);
          if (write_h) st16(hrow + k1, h1);
          acc0 = mma3(h1, p10, acc0);
          acc1 = mma3(h1, p11, acc1);
        }
      }
      goto reduce;
    }
  }
  if (do_router || blockIdx.y == 0) {
    for (int j0 = w; j0 < nks; j0 += 2 * RW) {
      const int j1 = j0 + RW;
      const int k0 = j0 * KS + q * EPL, k1 = min(j1, nks - 1) * KS + q * EPL;
      RouterFrag<T> f0, f1;
      if (do_router) {
        f0.load(xrow, a.gamma, w0, w1, k0);
        f1.load(xrow, a.gamma, w0, w1, k1);
      } else {
        f0.load_x(xrow, a.gamma, k0);
        f1.load_x(xrow, a.gamma, k1);
      }
      const u32x4 h0 = make_h<T>(f0.x, inv, f0.g);
      if (write_h) st16(hrow + k0, h0);
      if (do_router) {
        acc0 = router_mma<T>(h0, f0.w0, acc0);
        acc1 = router_mma<T>(h0, f0.w1, acc1);
      }
      if (j1 < nks) {
        const u32x4 h1 = make_h<T>(f1.x, inv, f1.g);
        if (write_h) st16(hrow + k1, h1);
        if (do_router) {
          acc0 = router_mma<T>(h1, f1.w0, acc0);
          acc1 = router_mma<T>(h1, f1.w1, acc1);
        }
      }
    }
  }
  if (!do_router) return;
reduce:
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s_part[w][4 * q + j][r16] = acc0[j];
    s_part[w][4 * q + j][16 + r16] = acc1[j];
  }
  __syncthreads();
  for (int u = threadIdx.x; u < TB * ECB; u += RNTHR) {
    const int tl = u / ECB, c = u % ECB, e = blockIdx.y * ECB + c, to = tok0 + tl;
    if (to < a.T && e < E) {
      float v = s_part[0][tl][c];
#pragma unroll
      for (int ww = 1; ww < RW; ++ww) v += s_part[ww][tl][c];
      if (a.bias) v += a.bias[e];
      a.logits_out[int64_t(to) * E + e] = v;
    }
  }
}

// Kernel 2: top-k, gates and skip mask, one wave per token.
__global__ __launch_bounds__(NTHR) void topk_skip_kernel(RouteArgs a) {
  __shared__ double s_z[NTHR / 64][EMAX];
  const int w = wave_id(), l = lane_id();
  const int t = blockIdx.x * (NTHR / 64) + w;
  if (t >= a.T) return;
  const int E = a.E, k = a.k;
  const float* lrow = (a.logits_in ? a.logits_in : a.logits_out) + int64_t(t) * E;
  const int R = (E + 63) / 64;
  // lane l holds experts l, l+64, ...: logits and both tables, loaded together
  // (indices clamped so every load is in bounds)
  float v[4], tg[4], tr[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int e = min(l + 64 * rr, E - 1);
    v[rr] = lrow[e];
    tg[rr] = a.a_gsp[e];
    tr[rr] = a.a_rcr[e];
  }
  if (a.logits_in != nullptr) {
    float* orow = a.logits_out + int64_t(t) * E;
    for (int rr = 0; rr < R; ++rr)
      if (l + 64 * rr < E) orow[l + 64 * rr] = v[rr];
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
  // softmax in float64, shifted by the top-1 logit; sums in ascending order
  const double m = double(top_logit);
  const double z = (l < k) ? exp(double(my_logit) - m) : 0.0;
  double s = 0.0;
  if (a.norm_topk) {
    for (int i = 0; i < k; ++i) s += __shfl(z, i, 64);
  } else {
    for (int rr = 0; rr < R; ++rr) {
      const int e = l + 64 * rr;
      if (e < E) s_z[w][e] = exp(double(v[rr]) - m);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int e = 0; e < E; ++e) s += s_z[w][e];
  }
  // table values of this lane's selected expert, from the lane that owns it
  float ag = 0.f, ar = 0.f;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const float gq = __shfl(tg[rr], my_e & 63, 64), rq = __shfl(tr[rr], my_e & 63, 64);
    if ((my_e >> 6) == rr) {
      ag = gq;
      ar = rq;
    }
  }
  if (l < k) {
    const float g = float(z / s);
    bool keep = true;
    if (l > 0) {
      const float sg = g * ag;
      const float sr = g * ar;
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

// Router pre-split for bf16 activations: [3 planes][CB][H/32][64 lanes][8 bf16];
// the unit of lane l in (plane p, column block cb, k-step j) holds plane p of
// w_router[16*cb + l%16][32*j + 8*(l/16) .. +8] (zero for experts >= E).
__global__ __launch_bounds__(256) void pack_router_kernel(const float* __restrict__ w, uint8_t* __restrict__ dst,
                                                          int E, int H) {
  const int nks = H / 32, CB = (E + 15) / 16;
  const int64_t units = int64_t(CB) * nks * 64;
  const int64_t u = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (u >= units) return;
  const int l = int(u & 63);
  const int64_t frag = u >> 6;
  const int j = int(frag % nks), cb = int(frag / nks);
  const int e = cb * 16 + (l & 15), k = j * 32 + (l >> 4) * 8;
  f32x4 v[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  if (e < E) {
    v[0] = *reinterpret_cast<const f32x4*>(w + int64_t(e) * H + k);
    v[1] = *reinterpret_cast<const f32x4*>(w + int64_t(e) * H + k + 4);
  }
  u32x4 planes[3];
  split3(v, planes);
  const int64_t plane_bytes = units * 16;
#pragma unroll
  for (int p = 0; p < 3; ++p) st16(dst + p * plane_bytes + u * 16, planes[p]);
}

size_t router_packed_bytes(int E, int H) { return size_t(3) * ((E + 15) / 16) * 16 * size_t(H) * 2; }

hipError_t launch_pack_router(const float* w, void* dst, int E, int H, hipStream_t s) {
  const int64_t units = int64_t((E + 15) / 16) * (H / 32) * 64;
  hipLaunchKernelGGL(pack_router_kernel, dim3(unsigned((units + 255) / 256)), dim3(256), 0, s, w,
                     static_cast<uint8_t*>(dst), E, H);
  return hipGetLastError();
}

hipError_t launch_route(int dtype, const RouteArgs& a, hipStream_t s) {
  const dim3 grid1((a.T + TB - 1) / TB, a.logits_in ? 1 : (a.E + ECB - 1) / ECB), block1(RNTHR), block(NTHR);
  if (dtype == 1)
    hipLaunchKernelGGL(norm_router_kernel<bf16_t>, grid1, block1, 0, s, a);
  else
    hipLaunchKernelGGL(norm_router_kernel<float>, grid1, block1, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid2((a.T + NTHR / 64 - 1) / (NTHR / 64));
  hipLaunchKernelGGL(topk_skip_kernel, grid2, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace ace
