// RMSNorm + router, then top-k gates + ACE skip mask (two kernels).
//
// Method: "ACE: Adaptive Calibration-Free Expert Skipping for MoE-based LLMs"
// (picx.dev summary page).  h = x̄Γ is the RMSNorm output (Theoretical
// Foundation); the slot scores are g·A^GSP(e) and g·A^RCR(e) (Methodology
// sections 1 and 2); a slot is skipped only when both fall below their
// thresholds, and the top-1 slot is always kept (Methodology section 3).
#include "kernels.h"
#include "topk.h"

namespace ace {

namespace {

constexpr int TB = 16;        // tokens per workgroup (router kernel)
constexpr int RW = 16;        // waves of the router kernel (split the hidden dimension)
constexpr int RNTHR = RW * 64;
constexpr int NTHR = 256;     // 4 waves (top-k kernel)
constexpr int EMAX = 256;
constexpr int NARROW_HMAX = 8192;  // hidden size limit of the small-batch router variant
constexpr int XL_HMAX = 2048;      // hidden size limit of the router's x rows in LDS
constexpr int XL_PITCH = XL_HMAX + 8;  // bf16 elements per LDS row
#ifndef ACE_ROUTER_WIDE_T
#define ACE_ROUTER_WIDE_T 2048     // batch from which the 32/64-token router variant is used
#endif
#ifndef ACE_ROUTER_WIDE_MT4_T
#define ACE_ROUTER_WIDE_MT4_T (2 * ACE_ROUTER_WIDE_T)  // batch from which the 64-token variant is used
#endif
#ifndef ACE_ROUTER_WIDE_NBK4
#define ACE_ROUTER_WIDE_NBK4 1     // k-steps per load batch of the 64-token variant
#endif
#ifndef ACE_ROUTER_H_T
#define ACE_ROUTER_H_T 4096        // batch from which the RMS and the router product run as two kernels
#endif
#ifndef ACE_ROUTER_H_PA
#define ACE_ROUTER_H_PA 4          // k-steps of router planes in flight per wave (two-kernel router)
#endif
#ifndef ACE_ROUTER_H_SD
#define ACE_ROUTER_H_SD 2          // classes of h fragments staged ahead (two-kernel router)
#endif
#ifndef ACE_ROUTER_NARROW_WG
#define ACE_ROUTER_NARROW_WG 64    // workgroups aimed at by the small-batch variant's expert sub-blocks
#endif
#ifndef ACE_ROUTER_NARROW_GX
#define ACE_ROUTER_NARROW_GX 8     // token blocks up to which the 16-expert router variant is used
#endif

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

// Kernel 1: RMSNorm (+ h_out) and the router product for 16 tokens x 16*NCB
// experts.  Sixteen waves split the hidden dimension: wave w takes k-steps
// w, w+16, w+32, ...  Their partial logits are summed in a fixed wave order,
// so a logit does not depend on timing, on NCB or on the batch size.  Token
// rows past T load nothing (zeros) and expert rows past E read a clamped
// valid row; their results are never stored.  For small batches (NCB = 1:
// more workgroups share the pre-split router planes) gamma is staged in LDS;
// with
// SUB > 1 the column block is further cut into SUB sub-blocks of 16/SUB
// experts, one per workgroup (lanes of other experts load nothing and their
// MFMA columns are discarded: an output column depends only on its own
// weights), so that the plane bytes of a decode batch spread over SUB times
// more compute units.
template <typename T, int NCB, int SUB = 1, bool XL = false>
__global__ __launch_bounds__(RNTHR) void norm_router_kernel(RouteArgs a) {
  static_assert(SUB == 1 || NCB == 1, "sub-blocks of one column block only");
  static_assert(!XL || sizeof(T) == 2, "x rows in LDS: bf16 only");
  constexpr int ECBW = 16 * NCB;          // experts per workgroup
  constexpr int NBK = NCB == 1 ? 4 : 2;   // k-steps per wave per load batch (pre-split planes)
  __shared__ float s_inv[TB];
  __shared__ float s_part[RW][TB][ECBW + 1];
  __shared__ __attribute__((aligned(16))) float s_gam[NCB == 1 ? NARROW_HMAX : 4];
  // XL (H <= XL_HMAX): the RMS prologue keeps the 16 x rows in LDS and the
  // MFMA operands are read from there instead of a second pass over global
  // memory (each vector-memory instruction costs the CU the same time however
  // few of its lanes are active); rows padded by 16 bytes (no bank conflicts)
  __shared__ __attribute__((aligned(16))) uint16_t s_x[XL ? TB * XL_PITCH : 8];

  constexpr int EPL = St<T>::EPL;
  constexpr int KS = 4 * EPL;
  const int w = wave_id(), l = lane_id();
  const int tok0 = blockIdx.x * TB;
  const int H = a.H, E = a.E;
  const T* x = reinterpret_cast<const T*>(a.x);
  const int q = l >> 4, r16 = l & 15;
  const int tt = tok0 + r16;
  const int t = min(tt, a.T - 1);
  const T* xrow = x + int64_t(t) * H;
  T* hrow = reinterpret_cast<T*>(a.h_out) + int64_t(t) * H;
  // h_out: every column-block workgroup of a token block computes the same h
  // fragments; k-step j is written by workgroup j % gridDim.y, so the stores
  // (whose completion later load waits include) are spread evenly
  const bool do_router = a.logits_in == nullptr;
  const bool row_ok = tt < a.T;
  auto write_h = [&](int j) -> bool {
    return row_ok && (do_router ? j % int(gridDim.y) == int(blockIdx.y) : blockIdx.y == 0);
  };
  const int nks = H / KS;
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};

  // pre-split planes: [3][CB][nks][64][16 B]; this workgroup's column blocks
  const bool packed = sizeof(T) == 2 && do_router && a.router_packed;
  const int CB = (E + 15) / 16;
  const int ycb = int(blockIdx.y) / SUB;                 // column block (pair) index
  const int sub = int(blockIdx.y) % SUB;                 // sub-block of 16/SUB experts
  const bool lane_e = SUB == 1 || r16 / (16 / SUB) == sub;  // this lane's expert is computed here
  int cb[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) cb[c] = min(ycb * NCB + c, CB - 1);
  const uint8_t* wp = reinterpret_cast<const uint8_t*>(a.w_router);
  const int64_t plane_bytes = int64_t(CB) * nks * 1024;
  const int nki = w < nks ? (nks - 1 - w) / RW + 1 : 0;  // this wave's k-steps
  u32x4 pl[NBK][NCB][3];
  u32x4 px[NBK];
  // Loads that some lanes skip are buffer loads whose skipped lanes get an
  // offset past the buffer (they return zero and touch no memory), so no
  // load sits in a divergent branch and each wait covers only the loads it
  // needs.
  constexpr int OOB = int(0x7FFFFFF0u);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, uint32_t(int64_t(a.T) * H * int(sizeof(T))));
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(wp, packed ? uint32_t(3 * plane_bytes) : 0u);
  auto issue = [&](int i0) {
#pragma unroll
    for (int b = 0; b < NBK; ++b) {
      const int j = w + RW * min(i0 + b, nki - 1);
      px[b] = u32x4{0u, 0u, 0u, 0u};
      if (!XL)  // rows past the batch: no loads
        px[b] = buf_ld16(xr, tt < a.T && nki > 0 ? (tt * H + j * KS + q * EPL) * int(sizeof(T)) : OOB, 0);
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int p = 0; p < 3; ++p)
          pl[b][c][p] = buf_ld16(pr, lane_e && nki > 0 ? int(p * plane_bytes + (int64_t(cb[c]) * nks + j) * 1024) + l * 16 : OOB, 0);
    }
  };
  constexpr int GQ = NARROW_HMAX / (RNTHR * 4);  // gamma quads per thread for the LDS copy
  // one column block (the small-batch variants, launched only with the
  // pre-split router): gamma is copied to LDS once (read there by every
  // k-step of the MFMA loop)
  constexpr bool gam_lds = NCB == 1;
  // router bias of this thread's output (read after the last barrier)
  float bias_v = 0.f;
  if (do_router && a.bias != nullptr && threadIdx.x < TB * ECBW)
    bias_v = a.bias[min(ycb * ECBW + int(threadIdx.x) % ECBW, E - 1)];

  // inverse RMS: wave w owns token tok0 + w; a row is read 8 segments of
  // 64 lanes x 16 bytes at a time, all in flight together (segments past H
  // are not loaded), then the gamma quads for the LDS copy (one column block:
  // H <= NARROW_HMAX).  One column block with every k-step of a wave in one
  // load batch (the decode variant): the router plane loads go out while the
  // rows are in flight, but only after a bare barrier that follows every
  // wave's row and gamma loads, so that they queue behind those in the CU's
  // vector-memory pipe (planes issued first hold up the RMS); the RMS waits
  // for the rows alone and the planes arrive during it.
  // (XL: H <= 2048, so nks <= 64 = RW * NBK and every wave has at most NBK k-steps)
  constexpr bool early_planes = NCB == 1 && XL;
  {
    const int row_t = __builtin_amdgcn_readfirstlane(tok0 + w);
    const bool row_valid = row_t < a.T;  // waves past the batch load no row
    constexpr int SEG = 64 * EPL;
    // segments per batch (the per-lane sum runs over them in order); with
    // the rows in LDS (H <= 2048) one batch of 4 covers the row
    constexpr int RSEG = XL ? 4 : 8;
    const __amdgpu_buffer_rsrc_t gr = make_rsrc(a.gamma, uint32_t(H * 4));
    float ss = 0.f;
    for (int j0 = 0; j0 < H; j0 += RSEG * SEG) {
      u32x4 v[RSEG];
#pragma unroll
      for (int b = 0; b < RSEG; ++b) {
        const int col = j0 + b * SEG + l * EPL;
        v[b] = u32x4{0u, 0u, 0u, 0u};
        if (row_valid && j0 + b * SEG < H)  // wave-uniform
          v[b] = buf_ld16(xr, col < H ? (row_t * H + col) * int(sizeof(T)) : OOB, 0);
      }
      if (j0 == 0 && gam_lds) {
        f32x4 gq[GQ];
#pragma unroll
        for (int i = 0; i < GQ; ++i) {
          const int h = (int(threadIdx.x) + i * RNTHR) * 4;
          gq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (__builtin_amdgcn_readfirstlane(h) < H)  // waves wholly past H load nothing
            gq[i] = __builtin_bit_cast(f32x4, buf_ld16(gr, h < H ? h * 4 : OOB, 0));
        }
        if (early_planes) {
          __builtin_amdgcn_s_barrier();  // every wave's row and gamma loads are issued
          issue(0);                      // (waves without k-steps load nothing)
        }
#pragma unroll
        for (int i = 0; i < GQ; ++i) {
          const int h = (int(threadIdx.x) + i * RNTHR) * 4;
          if (h < H) *reinterpret_cast<f32x4*>(&s_gam[h]) = gq[i];  // read back after the barrier
        }
      }
#pragma unroll
      for (int b = 0; b < RSEG; ++b)
        if (j0 + b * SEG + l * EPL < H) {
          ss += sumsq16<T>(v[b]);
          if constexpr (XL) *reinterpret_cast<u32x4*>(&s_x[w * XL_PITCH + j0 + b * SEG + l * EPL]) = v[b];
        }
    }
    ss = wave_sum_dpp(ss);
    if (l == 0) s_inv[w] = 1.0f / sqrtf(ss / float(H) + a.eps);
  }
  __syncthreads();
  const float inv = s_inv[r16];

  if constexpr (sizeof(T) == 2) {
    if (packed) {
      for (int i0 = 0; i0 < nki; i0 += NBK) {
        if (!early_planes || i0 > 0) issue(i0);
#pragma unroll
        for (int b = 0; b < NBK; ++b) {
          if (i0 + b < nki) {
            const int jb = w + RW * (i0 + b);
            const int k0 = jb * KS + q * EPL;
            const float* gp = gam_lds ? s_gam + k0 : a.gamma + k0;
            f32x4 g[2];
            g[0] = *reinterpret_cast<const f32x4*>(gp);
            g[1] = *reinterpret_cast<const f32x4*>(gp + 4);
            u32x4 xv = px[b];
            if constexpr (XL) xv = *reinterpret_cast<const u32x4*>(&s_x[r16 * XL_PITCH + k0]);
            const u32x4 h = make_h<T>(xv, inv, g);
            if (write_h(jb)) st16(hrow + k0, h);
#pragma unroll
            for (int c = 0; c < NCB; ++c) acc[c] = mma3(h, pl[b][c], acc[c]);
          }
        }
      }
      goto reduce;
    }
  }
  if constexpr (NCB == 2) {
    const int e0 = min(blockIdx.y * ECBW + r16, E - 1), e1 = min(blockIdx.y * ECBW + 16 + r16, E - 1);
    const float* w0 = a.w_router + int64_t(e0) * H;
    const float* w1 = a.w_router + int64_t(e1) * H;
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
        if (write_h(j0)) st16(hrow + k0, h0);
        if (do_router) {
          acc[0] = router_mma<T>(h0, f0.w0, acc[0]);
          acc[1] = router_mma<T>(h0, f0.w1, acc[1]);
        }
        if (j1 < nks) {
          const u32x4 h1 = make_h<T>(f1.x, inv, f1.g);
          if (write_h(j1)) st16(hrow + k1, h1);
          if (do_router) {
            acc[0] = router_mma<T>(h1, f1.w0, acc[0]);
            acc[1] = router_mma<T>(h1, f1.w1, acc[1]);
          }
        }
      }
    }
  }
  if (!do_router) return;
reduce:
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int c = 0; c < NCB; ++c) s_part[w][4 * q + j][16 * c + r16] = acc[c][j];
  __syncthreads();
  static_assert(TB * ECBW <= RNTHR, "one output per thread");
  if (threadIdx.x < TB * ECBW) {
    const int u = threadIdx.x;
    const int tl = u / ECBW, c = u % ECBW, e = ycb * ECBW + c, to = tok0 + tl;
    if (to < a.T && e < E && (SUB == 1 || c / (16 / SUB) == sub)) {
      float v = s_part[0][tl][c];
#pragma unroll
      for (int ww = 1; ww < RW; ++ww) v += s_part[ww][tl][c];
      if (a.bias) v += bias_v;
      a.logits_out[int64_t(to) * E + e] = v;
    }
  }
}

// Kernel 1, large batches (bf16 with the pre-split router): 16*MT tokens x
// 32 experts per workgroup, so that each plane fragment read feeds MT token
// blocks instead of one.  Every step that fixes a value is the one of
// norm_router_kernel: the inverse RMS of a row (same lane split, same wave
// sum), h = make_h, the wave classes of k-steps (wave w takes k-steps w,
// w+16, ...), the MFMA chain of each class in k order with planes 0, 1, 2,
// and the sum of the 16 class partials in wave order, then the bias.  So a
// logit is bit-identical to the one the other variants compute, whatever the
// batch.  Workgroup L serves token block 8*(L/(8*ncb)) + L%8 and column
// block (L/8) % ncb: a token block's column blocks run on one XCD, eight
// launch slots apart, and share its x rows through that XCD's L2.
template <int MT, int NBK>
__global__ __launch_bounds__(RNTHR) void norm_router_wide_kernel(RouteArgs a, int gxw) {
  static_assert(MT % 2 == 0, "rows of the RMS prologue go in pairs");
  constexpr int TBW = TB * MT;
  constexpr int ECBW = 32;
  constexpr int EPL = 8, KS = 32;
  __shared__ float s_inv[TBW];
  __shared__ float s_part[RW][TBW][ECBW + 1];
  const int E = a.E, H = a.H;
  const int ncb = (E + ECBW - 1) / ECBW;
  const int L = blockIdx.x;
  const int cbk = (L / 8) % ncb;
  const int tbk = 8 * (L / (8 * ncb)) + L % 8;
  if (tbk >= gxw) return;  // padding of the grid to whole groups of 8
  const int w = wave_id(), l = lane_id();
  const int tok0 = tbk * TBW;
  const int q = l >> 4, r16 = l & 15;
  const bf16_t* x = reinterpret_cast<const bf16_t*>(a.x);
  bf16_t* hout = reinterpret_cast<bf16_t*>(a.h_out);
  const int nks = H / KS;
  const int CB = (E + 15) / 16;
  const int cb0 = min(2 * cbk, CB - 1), cb1 = min(2 * cbk + 1, CB - 1);
  const uint8_t* wp = reinterpret_cast<const uint8_t*>(a.w_router);
  const int64_t plane_bytes = int64_t(CB) * nks * 1024;
  const int nki = w < nks ? (nks - 1 - w) / RW + 1 : 0;
  float bias_v = 0.f;
  if (a.bias != nullptr) bias_v = a.bias[min(cbk * ECBW + int(threadIdx.x) % ECBW, E - 1)];

  // inverse RMS: wave w owns tokens tok0 + w + 16*m, all MT rows in flight,
  // 4 segments of 512 values per row and batch (each row's sum runs over its
  // segments in order, as in the other router variants)
  {
    constexpr int SEG = 64 * EPL, NSEG = 4;
    float ss[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) ss[m] = 0.f;
    for (int j0 = 0; j0 < H; j0 += NSEG * SEG) {
      u32x4 v[MT][NSEG];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bf16_t* row = x + int64_t(min(tok0 + w + 16 * m, a.T - 1)) * H;
#pragma unroll
        for (int b = 0; b < NSEG; ++b) v[m][b] = ld16(row + min(j0 + b * SEG + l * EPL, H - EPL));
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int b = 0; b < NSEG; ++b)
          if (j0 + b * SEG + l * EPL < H) ss[m] += sumsq16<bf16_t>(v[m][b]);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float t = wave_sum_dpp(ss[m]);
      if (l == 0) s_inv[w + 16 * m] = 1.0f / sqrtf(t / float(H) + a.eps);
    }
  }
  __syncthreads();
  float inv[MT];
  const bf16_t* xrow[MT];
  bf16_t* hrow[MT];
  bool wr[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    inv[m] = s_inv[16 * m + r16];
    const int tt = tok0 + 16 * m + r16;
    const int t = min(tt, a.T - 1);
    xrow[m] = x + int64_t(t) * H;
    hrow[m] = hout + int64_t(t) * H;
    wr[m] = tt < a.T;  // k-step j of h is written by column block j % ncb (stores spread evenly)
  }

  f32x4 acc[MT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m][0] = acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 px[NBK][MT], pl[NBK][2][3];
  for (int i0 = 0; i0 < nki; i0 += NBK) {
#pragma unroll
    for (int b = 0; b < NBK; ++b) {
      const int j = w + RW * min(i0 + b, nki - 1);
#pragma unroll
      for (int m = 0; m < MT; ++m) px[b][m] = ld16(xrow[m] + j * KS + q * EPL);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        pl[b][0][p] = ld16(wp + p * plane_bytes + (int64_t(cb0) * nks + j) * 1024 + l * 16);
        pl[b][1][p] = ld16(wp + p * plane_bytes + (int64_t(cb1) * nks + j) * 1024 + l * 16);
      }
    }
#pragma unroll
    for (int b = 0; b < NBK; ++b) {
      if (i0 + b < nki) {
        const int jb = w + RW * (i0 + b);
        const int k0 = jb * KS + q * EPL;
        const bool wj = jb % ncb == cbk;
        f32x4 g[2];
        g[0] = *reinterpret_cast<const f32x4*>(a.gamma + k0);
        g[1] = *reinterpret_cast<const f32x4*>(a.gamma + k0 + 4);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4 h = make_h<bf16_t>(px[b][m], inv[m], g);
          if (wr[m] && wj) st16(hrow[m] + k0, h);
          acc[m][0] = mma3(h, pl[b][0], acc[m][0]);
          acc[m][1] = mma3(h, pl[b][1], acc[m][1]);
        }
      }
    }
  }

  // class partials summed in wave order, all MT token blocks at once (the
  // partials of the 16·MT tokens fit in LDS; thread u sums entries u,
  // u + RNTHR, ..., whose expert column is the same, u % ECBW)
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 2; ++c) s_part[w][16 * m + 4 * q + j][16 * c + r16] = acc[m][c][j];
  __syncthreads();
  static_assert(RNTHR % ECBW == 0, "a thread's entries share one expert column");
  for (int u = threadIdx.x; u < TBW * ECBW; u += RNTHR) {
    const int tl = u / ECBW, c = u % ECBW, e = cbk * ECBW + c, to = tok0 + tl;
    if (to < a.T && e < E) {
      float v = s_part[0][tl][c];
#pragma unroll
      for (int ww = 1; ww < RW; ++ww) v += s_part[ww][tl][c];
      if (a.bias) v += bias_v;
      a.logits_out[int64_t(to) * E + e] = v;
    }
  }
}

// Workgroup barrier that orders LDS only (this wave's LDS operations
// complete, then s_barrier): unlike __syncthreads() it leaves the router
// plane loads in flight.
__device__ __forceinline__ void lds_only_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Large batches, H a multiple of 512 (bf16, pre-split router; launched at
// H = 2048): the RMSNorm and the router product as two kernels, each step
// the one of the other variants.  Kernel 1a: one wave per row, lane l holding x values 8l .. 8l+7
// of every 512-value segment, the per-lane sum over the segments in order,
// the same 64-lane reduction, h = make_h; x is read and h written once, at
// the streaming rate (R rows of a wave in flight together).
template <int NSEG, int R>
__global__ __launch_bounds__(256) void rms_h_kernel(RouteArgs a) {
  constexpr int EPL = 8, SEG = 64 * EPL;
  const int H = a.H;  // == NSEG * SEG (checked by the launcher)
  const int l = lane_id();
  const int nw = int(gridDim.x) * 4;
  const int gw = int(blockIdx.x) * 4 + wave_id();
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, uint32_t(a.T * H * 2));
  const __amdgpu_buffer_rsrc_t gr = make_rsrc(a.gamma, uint32_t(H * 4));
  f32x4 g[NSEG][2];
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    g[s][0] = __builtin_bit_cast(f32x4, buf_ld16(gr, (s * SEG + l * EPL) * 4, 0));
    g[s][1] = __builtin_bit_cast(f32x4, buf_ld16(gr, (s * SEG + l * EPL) * 4 + 16, 0));
  }
  bf16_t* hout = reinterpret_cast<bf16_t*>(a.h_out);
  for (int r0 = gw * R; r0 < a.T; r0 += nw * R) {
    u32x4 v[R][NSEG];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(r0 + r, a.T - 1);
#pragma unroll
      for (int s = 0; s < NSEG; ++s) v[r][s] = buf_ld16(xr, (row * H + s * SEG + l * EPL) * 2, 0);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < NSEG; ++s) ss += sumsq16<bf16_t>(v[r][s]);
      const float inv = 1.0f / sqrtf(wave_sum_dpp(ss) / float(H) + a.eps);
      if (r0 + r < a.T) {
        bf16_t* hrow = hout + int64_t(r0 + r) * H + l * EPL;
#pragma unroll
        for (int s = 0; s < NSEG; ++s) st16(hrow + s * SEG, make_h<bf16_t>(v[r][s], inv, g[s]));
      }
    }
  }
}

// Kernel 1b: the router product from h for 16·MT tokens x 4·NCW column
// blocks of 16 experts (one wave per NCW column blocks).  The logit of the
// other variants is the sum, in class order, of 16 class partials, class c
// being the MFMA chain (planes 0, 1, 2 per k-step) over k-steps c, c+16, ...
// in order, started from zero.  Here each wave walks the classes in turn
// for its own outputs and keeps that sum in registers (total = partial for
// class 0, total + partial after), so no partials go through LDS and the
// result is the same bit for bit.  The h fragments of a class (16·MT tokens
// x NKI k-steps) are staged in LDS fragment by fragment (lane order, so the
// operand reads are contiguous), loaded SD classes ahead into registers; the
// router plane fragments go straight into registers, PA k-steps ahead.  At
// T = 32768 this pair takes ~130 µs where the one-kernel variant took ~215:
// that one read x twice, in phases that every workgroup went through in
// step (1 workgroup per compute unit, 8 rounds).
template <int MT, int NKI, int NCW, int PA, int SD>
__global__ __launch_bounds__(256, 2) void router_from_h_kernel(RouteArgs a) {
  constexpr int NW = 4, KS = 32, EPL = 8;
  constexpr int NKS = 16 * NKI;      // k-steps of a row
  constexpr int TT = 16 * MT;        // tokens of the workgroup
  constexpr int FR = MT * NKI;       // h fragments (1 KB) of a class
  constexpr int FPW = FR / NW;       // staged by each wave
  static_assert(FR % NW == 0, "the class's fragments split evenly over the waves");
  static_assert(NKI % PA == 0, "the plane ring index is the k-step's index in its class modulo PA");
  static_assert(16 % SD == 0, "the class loop runs in groups of SD");
  __shared__ u32x4 s_a[2][FR * 64];
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id();
  const int q = l >> 4, r16 = l & 15;
  const int H = a.H, E = a.E;
  const int tok0 = int(blockIdx.x) * TT;
  const int nrows = min(TT, a.T - tok0);
  const int CB = (E + 15) / 16;
  int cb[NCW];
#pragma unroll
  for (int n = 0; n < NCW; ++n) cb[n] = min((int(blockIdx.y) * NW + w) * NCW + n, CB - 1);
  const int plane_bytes = CB * NKS * 1024;
  const __amdgpu_buffer_rsrc_t hr =
      make_rsrc(reinterpret_cast<const bf16_t*>(a.h_out) + int64_t(tok0) * H, uint32_t(nrows * H * 2));
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.w_router, uint32_t(3 * plane_bytes));

  // staging: fragment f = w + NW·i is (token block f / NKI, k-step f % NKI of
  // the class); lane (r16, q) fetches 8 h values of token 16·(f/NKI) + r16.
  // The fragments of class c + SD are requested while class c runs (held in
  // registers), and stored to LDS at the end of class c + SD - 1.
  int ho[FPW];
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    const int f = w + NW * i;
    ho[i] = (min(16 * (f / NKI) + r16, nrows - 1) * H + q * EPL) * 2;
  }
  u32x4 st[SD][FPW];
  auto stage_load = [&](int slot, int c) {
#pragma unroll
    for (int i = 0; i < FPW; ++i) st[slot][i] = buf_ld16(hr, ho[i], (c + 16 * ((w + NW * i) % NKI)) * KS * 2);
  };
  auto stage_store = [&](int slot, int buf) {
#pragma unroll
    for (int i = 0; i < FPW; ++i) s_a[buf][(w + NW * i) * 64 + l] = st[slot][i];
  };
  u32x4 pl[PA][NCW][3];
  auto issue = [&](int c, int s) {  // k-step s of class c (a clamped repeat past the last)
    const int idx = min(c * NKI + s, NKS - 1);
    const int j = idx / NKI + 16 * (idx % NKI);
#pragma unroll
    for (int n = 0; n < NCW; ++n)
#pragma unroll
      for (int p = 0; p < 3; ++p) pl[s % PA][n][p] = buf_ld16(pr, l * 16, p * plane_bytes + (cb[n] * NKS + j) * 1024);
  };

#pragma unroll
  for (int d = 0; d < SD; ++d) stage_load(d, d);  // class k is held in slot k % SD
  stage_store(0, 0);
#pragma unroll
  for (int s = 0; s < PA; ++s) issue(0, s);
  lds_only_barrier();
  f32x4 tot[MT][NCW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NCW; ++n) tot[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < 16; c0 += SD) {
#pragma unroll
    for (int d = 0; d < SD; ++d) {
      const int c = c0 + d;
      // slot d held class c, already in LDS, and now receives class c + SD
      // (past the last class: a repeat of it, never stored where it is read)
      stage_load(d, min(c + SD, 15));
      __builtin_amdgcn_sched_barrier(0);
      f32x4 acc[MT][NCW];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NCW; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKI; ++s) {
        u32x4 hf[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) hf[m] = s_a[c & 1][(m * NKI + s) * 64 + l];
        // plane fragment (n, p) feeds the MT MFMAs of column block n (each
        // accumulator still takes planes 0, 1, 2 in order), then is reloaded
        // at once with k-step s + PA's fragment: loads go out one per MT
        // MFMAs instead of in a burst (pinned by the group barriers)
        const int idx = min(c * NKI + s + PA, NKS - 1);
        const int jn = idx / NKI + 16 * (idx % NKI);
#pragma unroll
        for (int n = 0; n < NCW; ++n)
#pragma unroll
          for (int p = 0; p < 3; ++p) {
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m][n] = mfma_bf16(hf[m], pl[s % PA][n][p], acc[m][n]);
            pl[s % PA][n][p] = buf_ld16(pr, l * 16, p * plane_bytes + (cb[n] * NKS + jn) * 1024);
          }
#pragma unroll
        for (int g = 0; g < 3 * NCW; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, MT, 0);  // MT MFMAs
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one vector-memory read
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NCW; ++n) tot[m][n] = c == 0 ? acc[m][n] : tot[m][n] + acc[m][n];  // no 0 + (-0)
      stage_store((d + 1) % SD, (c + 1) & 1);
      lds_only_barrier();
    }
  }

#pragma unroll
  for (int n = 0; n < NCW; ++n) {
    const int e = cb[n] * 16 + r16;
    const bool e_ok = (int(blockIdx.y) * NW + w) * NCW + n < CB && e < E;
    const float bv = a.bias != nullptr && e_ok ? a.bias[e] : 0.f;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tl = 16 * m + 4 * q + j;
        float v = tot[m][n][j];
        if (a.bias) v += bv;
        if (e_ok && tl < nrows) a.logits_out[int64_t(tok0 + tl) * E + e] = v;
      }
  }
}

// Kernel 2: top-k, gates and skip mask, one wave per token (topk_slots).
__global__ __launch_bounds__(NTHR) void topk_skip_kernel(RouteArgs a) {
  constexpr int NWV = NTHR / 64;
  __shared__ float s_tg[EMAX], s_tr[EMAX];
  __shared__ double s_z[NWV][EMAX];
  const int w = wave_id(), l = lane_id();
  const int t_raw = blockIdx.x * NWV + w;
  const bool valid = t_raw < a.T;
  const int t = min(t_raw, a.T - 1);
  const int E = a.E, k = a.k;
  const int R = topk_per_lane(E);
  const float* lrow = (a.logits_in ? a.logits_in : a.logits_out) + int64_t(t) * E;
  // lane l holds experts l*R .. l*R + R-1 (indices clamped: every load in bounds)
  float v[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) v[rr] = rr < R ? lrow[min(l * R + rr, E - 1)] : 0.f;
  {
    // tables, shared by the workgroup's tokens (entries >= E are never read)
    const int e = min(int(threadIdx.x), E - 1);
    s_tg[threadIdx.x] = a.a_gsp[e];
    s_tr[threadIdx.x] = a.a_rcr[e];
  }
  if (valid && a.logits_in != nullptr) {
    float* orow = a.logits_out + int64_t(t) * E;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      if (rr < R && l * R + rr < E) orow[l * R + rr] = v[rr];
  }
  __syncthreads();
  const TopkParams p{E, k, a.norm_topk, a.fusion, a.tau_gsp, a.tau_rcr};
  int my_e;
  float g;
  bool keep;
  topk_slots(v, p, s_tg, s_tr, s_z[w], my_e, g, keep);
  if (valid && l < k) {
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

hipError_t launch_route(int dtype, const RouteArgs& a, hipStream_t s, bool with_topk) {
  static_assert(NTHR == EMAX, "the top-k kernel loads one table entry per thread");
  const dim3 block1(RNTHR), block(NTHR);
  const unsigned gx = unsigned((a.T + TB - 1) / TB);
  // small batches with the pre-split router: one 16-expert column block per
  // workgroup, so that more workgroups share the router weights
  const bool narrow =
      dtype == 1 && a.router_packed && a.logits_in == nullptr && gx <= ACE_ROUTER_NARROW_GX && a.H <= NARROW_HMAX;
  // large batches with the pre-split router: 32 or 64 tokens per workgroup
  const bool wide = dtype == 1 && a.router_packed && a.logits_in == nullptr && a.T >= ACE_ROUTER_WIDE_T;
  // from ACE_ROUTER_H_T tokens at H = 2048: RMS + h, then the router product
  // from h (32-bit buffer offsets: the batch's x fits in 2 GB).  At
  // H = 4096 the two kernels measured no faster than the wide one.
  const bool two = wide && a.T >= ACE_ROUTER_H_T && a.H == 2048 && int64_t(a.T) * a.H * 2 < (int64_t(1) << 31);
  if (two) {
    const unsigned CB = unsigned((a.E + 15) / 16);
    hipLaunchKernelGGL((rms_h_kernel<4, 4>), dim3(unsigned((a.T + 15) / 16)), block, 0, s, a);
    hipLaunchKernelGGL((router_from_h_kernel<4, 4, 2, ACE_ROUTER_H_PA, ACE_ROUTER_H_SD>),
                       dim3(unsigned((a.T + 63) / 64), (CB + 7) / 8), block, 0, s, a);
  } else if (wide) {
    const int mt = a.T >= ACE_ROUTER_WIDE_MT4_T ? 4 : 2;
    const int gxw = (a.T + TB * mt - 1) / (TB * mt);
    const unsigned nwg = unsigned((gxw + 7) / 8 * 8 * ((a.E + 31) / 32));
    if (mt == 4)
      hipLaunchKernelGGL((norm_router_wide_kernel<4, ACE_ROUTER_WIDE_NBK4>), dim3(nwg), block1, 0, s, a, gxw);
    else
      hipLaunchKernelGGL((norm_router_wide_kernel<2, 2>), dim3(nwg), block1, 0, s, a, gxw);
  } else if (narrow) {
    // sub-blocks: about ACE_ROUTER_NARROW_WG workgroups in all
    const unsigned cb = unsigned((a.E + 15) / 16);
    const unsigned sub = std::max(1u, std::min(4u, unsigned(ACE_ROUTER_NARROW_WG) / (gx * cb)));
    const bool xl = a.H <= XL_HMAX;
    if (sub >= 4 && xl)
      hipLaunchKernelGGL((norm_router_kernel<bf16_t, 1, 4, true>), dim3(gx, cb * 4), block1, 0, s, a);
    else if (sub >= 4)
      hipLaunchKernelGGL((norm_router_kernel<bf16_t, 1, 4>), dim3(gx, cb * 4), block1, 0, s, a);
    else if (sub >= 2 && xl)
      hipLaunchKernelGGL((norm_router_kernel<bf16_t, 1, 2, true>), dim3(gx, cb * 2), block1, 0, s, a);
    else if (sub >= 2)
      hipLaunchKernelGGL((norm_router_kernel<bf16_t, 1, 2>), dim3(gx, cb * 2), block1, 0, s, a);
    else if (xl)
      hipLaunchKernelGGL((norm_router_kernel<bf16_t, 1, 1, true>), dim3(gx, cb), block1, 0, s, a);
    else
      hipLaunchKernelGGL((norm_router_kernel<bf16_t, 1, 1>), dim3(gx, cb), block1, 0, s, a);
  } else {
    const dim3 grid1(gx, a.logits_in ? 1 : unsigned((a.E + 31) / 32));
    if (dtype == 1 && a.router_packed && a.logits_in == nullptr && a.H <= XL_HMAX)
      hipLaunchKernelGGL((norm_router_kernel<bf16_t, 2, 1, true>), grid1, block1, 0, s, a);
    else if (dtype == 1)
      hipLaunchKernelGGL((norm_router_kernel<bf16_t, 2>), grid1, block1, 0, s, a);
    else
      hipLaunchKernelGGL((norm_router_kernel<float, 2>), grid1, block1, 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !with_topk) return e;
  const dim3 grid2((a.T + NTHR / 64 - 1) / (NTHR / 64));
  hipLaunchKernelGGL(topk_skip_kernel, grid2, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace ace

