// Per-token top-k, router gates and ACE skip decision, computed by one wave.
// Shared by the routing kernel and the fused small-batch expert kernel, so
// both produce the same bits.
//
// Method: "ACE: Adaptive Calibration-Free Expert Skipping for MoE-based LLMs"
// (picx.dev summary page): slot scores g·A^GSP(e) and g·A^RCR(e)
// (Methodology sections 1 and 2); a slot is skipped only when both fall
// below their thresholds; the top-1 slot is always kept (Methodology
// section 3).  The alternative fusion rules are the page's ablations
// (Tables 4 and 5).
#pragma once

#include "common.h"

namespace ace {

// Wave-wide max / min through DPP row shifts (within rows of 16 lanes) and a
// combine of the four row results read from lanes 15, 31, 47 and 63; every
// lane gets the result.  No LDS round trips on the dependency chain.
template <int CTRL> __device__ __forceinline__ int dpp_shr(int v, int ident) {
  return __builtin_amdgcn_update_dpp(ident, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float wave_max_f(float v) {
  const int ni = __float_as_int(-INFINITY);
  v = fmaxf(v, __int_as_float(dpp_shr<0x111>(__float_as_int(v), ni)));
  v = fmaxf(v, __int_as_float(dpp_shr<0x112>(__float_as_int(v), ni)));
  v = fmaxf(v, __int_as_float(dpp_shr<0x114>(__float_as_int(v), ni)));
  v = fmaxf(v, __int_as_float(dpp_shr<0x118>(__float_as_int(v), ni)));
  const int b = __float_as_int(v);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 15)), __int_as_float(__builtin_amdgcn_readlane(b, 31))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 47)), __int_as_float(__builtin_amdgcn_readlane(b, 63))));
}
__device__ __forceinline__ int wave_min_i(int v) {
  constexpr int big = 0x7FFFFFFF;
  v = min(v, dpp_shr<0x111>(v, big));
  v = min(v, dpp_shr<0x112>(v, big));
  v = min(v, dpp_shr<0x114>(v, big));
  v = min(v, dpp_shr<0x118>(v, big));
  return min(min(__builtin_amdgcn_readlane(v, 15), __builtin_amdgcn_readlane(v, 31)),
             min(__builtin_amdgcn_readlane(v, 47), __builtin_amdgcn_readlane(v, 63)));
}

// Make this wave's LDS writes visible to its own later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct TopkParams {
  int E, k, norm_topk, fusion;
  float tau_gsp, tau_rcr;
};

// One token, one wave.  v[rr]: this lane's logit of expert l + 64*rr (entries
// for experts >= E are ignored).  k rounds of arg-max: the wave-wide largest
// remaining logit, then the lowest expert index among the lanes holding it
// (order: value descending, index ascending).  Gates: softmax in float64
// shifted by the top-1 logit, over the k selected (norm_topk) or all E,
// sums in ascending order, rounded once to float32.  Lane i < k gets slot i:
// its expert, gate and keep flag.  tg / tr: the two tables (any address
// space); zrow: EMAX doubles of LDS owned by this wave.
__device__ __forceinline__ void topk_slots(const float (&v)[4], const TopkParams& p, const float* tg,
                                           const float* tr, double* zrow, int& my_e, float& gate, bool& keep) {
  const int l = lane_id();
  const int E = p.E, k = p.k;
  const int R = (E + 63) / 64;
  uint32_t avail = 0;  // bit rr: value rr of this lane is a real, not yet taken expert
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
    if (rr < R && l + 64 * rr < E) avail |= 1u << rr;
  my_e = 0;
  float my_logit = 0.f, top_logit = 0.f;
  for (int i = 0; i < k; ++i) {
    // this lane's candidate: largest available value, lowest index on ties
    float cv = -INFINITY;
    int ce = 0x7FFFFFFF;
    int crr = -1;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      if (((avail >> rr) & 1u) && (crr < 0 || v[rr] > cv)) {
        cv = v[rr];
        ce = l + 64 * rr;
        crr = rr;
      }
    }
    const float m = wave_max_f(cv);
    const int be = wave_min_i(crr >= 0 && cv == m ? ce : 0x7FFFFFFF);
    if (ce == be) avail &= ~(1u << crr);
    if (l == i) {
      my_e = be;
      my_logit = m;
    }
    if (i == 0) top_logit = m;
  }
  const double mx = double(top_logit);
  const double z = (l < k) ? exp(double(my_logit) - mx) : 0.0;
  if (p.norm_topk) {
    if (l < k) zrow[l] = z;
  } else {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int e = l + 64 * rr;
      if (rr < R && e < E) zrow[e] = exp(double(v[rr]) - mx);
    }
  }
  wave_lds_sync();
  double s = 0.0;
  const int nsum = p.norm_topk ? k : E;
  for (int i = 0; i < nsum; ++i) s += zrow[i];
  wave_lds_sync();  // zrow may be rewritten by this wave's next token
  gate = float(z / s);
  keep = true;
  if (l > 0 && l < k) {
    const float sg = gate * tg[my_e];
    const float sr = gate * tr[my_e];
    const bool lg = sg < p.tau_gsp, lr = sr < p.tau_rcr;
    bool skip;
    switch (p.fusion) {
      case 1: skip = lg || lr; break;
      case 2:
        skip = p.tau_gsp > 0.f && p.tau_rcr > 0.f &&
               0.5 * (double(sg) / double(p.tau_gsp) + double(sr) / double(p.tau_rcr)) < 1.0;
        break;
      case 3: skip = lg; break;
      case 4: skip = lr; break;
      case 5: skip = gate < p.tau_gsp; break;
      default: skip = lg && lr; break;
    }
    keep = !skip;
  }
}

}  // namespace ace
