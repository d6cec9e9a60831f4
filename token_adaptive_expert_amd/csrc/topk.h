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

// Order-preserving map of a float32 logit to a uint32 key: a larger logit
// gives a larger key, -0 is folded onto +0 (they compare equal), NaN maps
// to 1 (below every number) and 0 is left free to mark a taken entry.
__device__ __forceinline__ uint32_t logit_key(float v) {
  if (v != v) return 1u;
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t kk) {
  return __uint_as_float((kk & 0x80000000u) ? (kk & 0x7FFFFFFFu) : ~kk);
}

// Wave-wide maximum: DPP row shifts within rows of 16 lanes (lane 15 of a
// row then holds the row maximum), two row broadcasts that carry it into
// lane 63, and one read of lane 63 (a uniform value).
template <int CTRL, int ROWS> __device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
  v = max(v, dpp_u<0x111, 0xF>(v));  // row_shr:1
  v = max(v, dpp_u<0x112, 0xF>(v));  // row_shr:2
  v = max(v, dpp_u<0x114, 0xF>(v));  // row_shr:4
  v = max(v, dpp_u<0x118, 0xF>(v));  // row_shr:8
  v = max(v, dpp_u<0x142, 0xA>(v));  // row_bcast:15 into rows 1 and 3
  v = max(v, dpp_u<0x143, 0xC>(v));  // row_bcast:31 into rows 2 and 3
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}

// Lane `lane`'s double (a uniform value).
__device__ __forceinline__ double readlane_d(double x, int lane) {
  const uint64_t u = uint64_t(__double_as_longlong(x));
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u)), lane));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u >> 32)), lane));
  return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
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

// Experts per lane for E experts (at most 4): lane l holds the logits of
// experts l*R .. l*R + R-1, so that a lower lane always means a lower index.
__device__ __forceinline__ int topk_per_lane(int E) { return (E + 63) / 64; }

// k rounds of selection over order-preserving keys, NR registers per lane
// (R <= NR of them used): each lane's candidate is its largest remaining key
// (the lower slot on ties), the wave-wide largest candidate wins, and the
// lowest lane holding it has the lowest expert index (order: value
// descending, index ascending).  Lane i < k receives round i's expert and
// key; top_key is round 0's.
template <int NR>
__device__ __forceinline__ void topk_rounds(const float (&v)[4], int E, int R, int k, int& my_e, uint32_t& my_key,
                                            uint32_t& top_key) {
  const int l = lane_id();
  uint32_t key[NR];
#pragma unroll
  for (int rr = 0; rr < NR; ++rr) key[rr] = (rr < R && l * R + rr < E) ? logit_key(v[rr]) : 0u;
  my_e = 0;
  my_key = 0u;
  top_key = 0u;
  for (int i = 0; i < k; ++i) {
    uint32_t cv = key[0];
    int cr = 0;
#pragma unroll
    for (int rr = 1; rr < NR; ++rr)
      if (key[rr] > cv) {
        cv = key[rr];
        cr = rr;
      }
    const uint32_t m = wave_max_u(cv);
    const int lsel = __builtin_ctzll(__builtin_amdgcn_ballot_w64(cv == m));  // k <= E: m is a real key
    const int esel = lsel * R + __builtin_amdgcn_readlane(cr, lsel);
#pragma unroll
    for (int rr = 0; rr < NR; ++rr)
      if (l == lsel && cr == rr) key[rr] = 0u;
    if (l == i) {
      my_e = esel;
      my_key = m;
    }
    if (i == 0) top_key = m;
  }
}

// One token, one wave.  v[rr]: this lane's logit of expert l*R + rr with
// R = topk_per_lane(E) (entries for experts >= E are ignored).  Selection as
// in topk_rounds.  Gates: softmax in float64 shifted by the top-1 logit, over
// the k selected (norm_topk) or all E, sums in ascending order, rounded once
// to float32.  Lane i < k gets slot i: its expert, gate and keep flag.
// tg / tr: the two tables (any address space); zrow: EMAX doubles of LDS
// owned by this wave (used when the softmax runs over all E).
__device__ __forceinline__ void topk_slots(const float (&v)[4], const TopkParams& p, const float* tg,
                                           const float* tr, double* zrow, int& my_e, float& gate, bool& keep) {
  const int l = lane_id();
  const int E = p.E, k = p.k;
  const int R = topk_per_lane(E);
  uint32_t my_key, top_key;
  if (R == 1)
    topk_rounds<1>(v, E, R, k, my_e, my_key, top_key);
  else if (R == 2)
    topk_rounds<2>(v, E, R, k, my_e, my_key, top_key);
  else
    topk_rounds<4>(v, E, R, k, my_e, my_key, top_key);
  const double mx = double(key_logit(top_key));
  const double z = (l < k) ? exp(double(key_logit(my_key)) - mx) : 0.0;
  double s = 0.0;
  if (p.norm_topk) {
    for (int i = 0; i < k; ++i) s += readlane_d(z, i);
  } else {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int e = l * R + rr;
      if (rr < R && e < E) zrow[e] = exp(double(v[rr]) - mx);
    }
    wave_lds_sync();
    for (int i = 0; i < E; ++i) s += zrow[i];
    wave_lds_sync();  // zrow may be rewritten by this wave's next token
  }
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
