/*
 * ace_moe.h -- C ABI of the MI355X (gfx950) library for one routed SwiGLU
 * Mixture-of-Experts layer forward with ACE per-token expert-slot skipping.
 *
 * Method source: "ACE: Adaptive Calibration-Free Expert Skipping for
 * MoE-based LLMs" (picx.dev summary page).  The layer input is x = x̄Γ
 * (Theoretical Foundation), each expert is the SwiGLU map f of that section,
 * each routed slot i of token t has gate g_{t,i}, and ACE skips a slot when
 * both g·A^GSP(e) and g·A^RCR(e) fall below their thresholds (Methodology,
 * sections 1-3), never skipping the top-1 slot.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers, row-major, owned by the caller,
 *     16-byte aligned (torch allocations are); a misaligned pointer is
 *     rejected with ACE_EINVAL naming it.
 *     The library never allocates, frees or synchronises; every call only
 *     enqueues kernels on `stream` (a hipStream_t, NULL = default stream).
 *   - Activations (x, h, act, slot outputs, y) and expert weights use
 *     desc->dtype (ACE_F32: float, ACE_BF16: bf16 bit patterns, 2 bytes).
 *     Router weights, logits, gates and tables are float32.
 *   - Expert weights follow the nn.Linear layout (out x in, K contiguous):
 *     w_gate, w_up: [E, I, H]; w_down: [E, H, I].  The page's H x I matrix
 *     W^gate is w_gate[e] transposed.
 *   - Arguments are checked before anything is enqueued.  On error nothing
 *     is launched, the status is returned and moe_last_error() (a
 *     thread-local string, valid until the next call on that thread) names
 *     the offending argument.  ACE_EHIP means a launch failed; the HIP error
 *     text is in moe_last_error().  No C++ exception crosses this ABI.
 *   - T = 0 is a valid empty batch: the call returns ACE_OK and launches
 *     nothing.
 *   - Limits: 1 <= k <= min(E, 16); 1 <= E <= 256; H and I multiples of 128;
 *     one expert's matrix (H*I elements) and the slot activations
 *     (T*k*max(H, I) elements) each under 2 GiB.  Outside them:
 *     ACE_EUNSUPPORTED.
 *   - Calls on one stream run in order; calls that share output or workspace
 *     buffers must not run concurrently on different streams.
 */
#ifndef ACE_MOE_H
#define ACE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ACE_MOE_ABI_VERSION 3

typedef enum {
  ACE_OK = 0,
  ACE_EINVAL = 1,       /* null required pointer, negative size, bad enum */
  ACE_EUNSUPPORTED = 2, /* valid request outside the limits above */
  ACE_EWORKSPACE = 3,   /* workspace smaller than moe_workspace_bytes() */
  ACE_EHIP = 4          /* a HIP launch or runtime call failed */
} ace_status;

typedef enum { ACE_F32 = 0, ACE_BF16 = 1 } ace_dtype;

/* Expert-GEMM schedule.  GROUPED tiles 32 to 128 slot rows per weight tile
 * (prefill and most decode batches); STREAM tiles 16 rows and splits the
 * contraction over the waves of a tile, for the smallest batches, whose cost
 * is reading the retained experts' weights with little work per byte.  AUTO
 * takes STREAM for T*k <= 64 routed slots, GROUPED above. */
typedef enum { ACE_PATH_AUTO = 0, ACE_PATH_GROUPED = 1, ACE_PATH_STREAM = 2 } ace_path;
/* Optional bits or-ed into the path argument of moe_expert_forward to run
 * only one of its two kernels (for timing a stage alone); no bit = both. */
#define ACE_STAGE_GATEUP 0x100
#define ACE_STAGE_DOWN 0x200

/* How the two views are fused into the skip decision (Methodology section 3;
 * the alternatives are the page's ablations, Tables 4 and 5).  With
 * sG = g*A^GSP(e), sR = g*A^RCR(e) (float32 products), a non-top-1 slot is
 * skipped when:
 *   MAX   : sG < tau_gsp && sR < tau_rcr   (ACE: intersection of skip sets)
 *   MIN   : sG < tau_gsp || sR < tau_rcr   (union)
 *   MEAN  : (sG/tau_gsp + sR/tau_rcr)/2 < 1, in float64 (never if a tau is 0)
 *   GSP   : sG < tau_gsp                   (single view)
 *   RCR   : sR < tau_rcr                   (single view)
 *   SCORE : g < tau_gsp                    (bare router gate)            */
typedef enum {
  ACE_FUSE_MAX = 0, ACE_FUSE_MIN = 1, ACE_FUSE_MEAN = 2,
  ACE_FUSE_GSP = 3, ACE_FUSE_RCR = 4, ACE_FUSE_SCORE = 5
} ace_fusion;

/* Layout of the expert weights passed to moe_expert_forward.
 * LINEAR: nn.Linear [E, N, K] (w_gate/w_up: N = I, K = H; w_down: N = H, K = I).
 * PACKED: the same values as made by moe_pack_weights, grouped so that each
 *   wave load reads one contiguous 1 KB block:
 *   [E][N/16][K/KS][64][V] with V = 16 bytes / element size (8 bf16, 4 f32)
 *   and KS = 4*V; entry [e][g][j][l][v] = linear[e][16*g + l%16][KS*j + V*(l/16) + v]. */
typedef enum { ACE_LAYOUT_LINEAR = 0, ACE_LAYOUT_PACKED = 1 } ace_weight_layout;

typedef struct {
  int32_t T;         /* tokens in the batch (rows of x) */
  int32_t H;         /* hidden size */
  int32_t E;         /* routed experts */
  int32_t I;         /* expert intermediate size */
  int32_t k;         /* routed slots per token (top-k) */
  int32_t dtype;     /* ace_dtype */
  int32_t norm_topk; /* 1: gates renormalised over the k selected experts */
  int32_t fusion;    /* ace_fusion */
  float rms_eps;     /* RMSNorm epsilon, added to the mean square */
  int32_t weight_layout; /* ace_weight_layout of w_gate, w_up, w_down */
  int32_t router_layout; /* ACE_LAYOUT_LINEAR: w_router is float32 [E, H];
                            ACE_LAYOUT_PACKED (bf16 only): the planes made by
                            moe_pack_router */
  int32_t expert_pool;   /* 0: off.  m >= 1: batch-level expert-pool cap in
                            moe_dispatch (see there); T*k <= 8192 */
} ace_moe_desc;

int moe_abi_version(void);
const char* moe_last_error(void);

/* Bytes of device workspace that moe_dispatch and moe_expert_forward need
 * (both take one; they may share it).  Calls sharing a workspace must not
 * overlap.  Returns 0 for an invalid descriptor. */
size_t moe_workspace_bytes(const ace_moe_desc* d);

/*
 * moe_route_skip -- RMSNorm, router, top-k gates and the ACE skip mask.
 *   h[t]      = x[t] / sqrt(mean_j x[t,j]^2 + rms_eps) * gamma   (x = x̄Γ, Theoretical
 *               Foundation), stored in dtype.
 *   logits[t] = h[t] . w_router^T (+ router_bias), float32 accumulation in a
 *               fixed order (deterministic), the same for every batch size
 *               and layout: a token's h and logits do not depend on the
 *               other rows of x.
 *   topk_idx  = the k largest logits, descending, equal logits to the lower
 *               expert index; slot 0 is the top-1 expert.
 *   topk_gate = softmax of the logits in float64 (over all E, or over the k
 *               selected when norm_topk), rounded to float32.
 *   keep      = the fusion rule above with (tau_gsp, tau_rcr); keep[t,0] = 1.
 * In:  x [T,H] dtype; gamma [H] f32; w_router [E,H] f32, or the packed
 *      planes when desc->router_layout is PACKED (may be NULL when logits_in
 *      is given); router_bias [E] f32 or NULL; logits_in [T,E] f32
 *      or NULL (when given, used instead of the router product, which is then
 *      not computed); a_gsp, a_rcr [E] f32, > 0; tau_gsp, tau_rcr >= 0.
 * Out: h_out [T,H] dtype; logits_out [T,E] f32 (required: the router writes
 *      its logits there, or logits_in is copied there; must not alias
 *      logits_in); topk_idx [T,k] i32; topk_gate [T,k] f32; keep [T,k] u8.
 * Logits must be finite; results for NaN logits are unspecified.
 */
ace_status moe_route_skip(const ace_moe_desc* d, const void* x, const float* gamma, const float* w_router,
                          const float* router_bias, const float* logits_in, float* logits_out, const float* a_gsp,
                          const float* a_rcr, float tau_gsp, float tau_rcr, void* h_out, int32_t* topk_idx,
                          float* topk_gate, uint8_t* keep, void* stream);

/*
 * moe_dispatch -- group the kept slots by expert ("expert dispatch" on the
 * article page about ACE).  Deterministic: within an expert, slots follow
 * token order; no floating-point atomics are used.
 * In:  topk_idx [T,k] (each row k distinct experts, as moe_route_skip
 *      writes them; rows with a repeated expert give unspecified results),
 *      topk_gate [T,k], keep [T,k].
 * Out: expert_offsets [E+1] i32 (segment starts; [E] = n_kept);
 *      sorted_token [T*k] i32 and sorted_gate [T*k] f32, first n_kept
 *      entries valid; slot_pos [T*k] i32: the sorted row of slot (t,i), or
 *      -1 when the slot is skipped.
 * Expert-pool cap (desc->expert_pool = m >= 1; decode batches): the batch's
 * retained experts are every expert that is some token's top-1, plus, up to
 * m experts in all, the others with the largest S_e = sum of the gates of
 * the kept slots routed to e (float32, slot order), lower index first on
 * ties; kept slots of other experts are skipped as well (slot_pos -1,
 * nothing folded or renormalised).  Reading of the decode pool of "ExFold:
 * Unified Expert Folding for Training-Free MoE Prefill-Decode Acceleration"
 * (abstract; Tables 1, 5, 6) without its folding.  The keep array is not
 * modified: slot_pos >= 0 marks the slots that run.
 * workspace: >= moe_workspace_bytes(d) bytes of device memory (batches of
 *      more than 32768 slots keep per-block expert counts there: 8 bytes per
 *      expert per 4096 slots; smaller ones use none of it).
 */
ace_status moe_dispatch(const ace_moe_desc* d, const int32_t* topk_idx, const float* topk_gate, const uint8_t* keep,
                        int32_t* expert_offsets, int32_t* sorted_token, float* sorted_gate, int32_t* slot_pos,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_expert_forward -- the SwiGLU experts over the dispatched slots (expert
 * equation f, Theoretical Foundation), gate-weighted.  For sorted row p of
 * expert e with token t = sorted_token[p]:
 *   act[p]      = SiLU(h[t] . w_gate[e]^T) * (h[t] . w_up[e]^T)   (dtype)
 *   slot_out[p] = sorted_gate[p] * (act[p] . w_down[e]^T)          (dtype)
 * Both are accumulated in float32 and rounded once to dtype on store.
 * Only rows p < expert_offsets[E] are written; only experts with at least
 * one kept slot have their weights read.
 * In:  h [T,H] dtype (from moe_route_skip); weights as above.
 * Out: act [T*k, I] dtype (scratch rows); slot_out [T*k, H] dtype.
 * workspace: >= moe_workspace_bytes(d) bytes.
 */
ace_status moe_expert_forward(const ace_moe_desc* d, int32_t path, const void* h, const void* w_gate,
                              const void* w_up, const void* w_down, const int32_t* expert_offsets,
                              const int32_t* sorted_token, const float* sorted_gate, void* act, void* slot_out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_combine -- the layer output as the gate-weighted sum of the routed
 * experts' maps ("ACE: Adaptive Calibration-Free Expert Skipping for
 * MoE-based LLMs", picx.dev summary page: Introduction and Theoretical
 * Foundation, where each token is routed to a few SwiGLU experts f, and
 * Methodology section 1, where a routed slot's share is its router gate g;
 * ACE drops the skipped slots' terms, Methodology section 3):
 *   y[t] = residual[t] + sum over kept slots i = 0..k-1 (in that order) of
 *          slot_out[slot_pos[t,i]] (= g_{t,i} f_{e_i}(x_t) from
 *          moe_expert_forward), accumulated in float32, stored in dtype.
 * Skipped slots contribute nothing and the kept gates are not renormalised.
 * residual is not part of the layer (the pages define none); it lets a stack
 * of layers add x_{l+1} = x_l + y_l in the same pass.
 * In:  slot_pos [T*k] i32 (row-major [T,k], -1 = skipped, as moe_dispatch
 *      writes it); slot_out [T*k, H] dtype; residual [T,H] dtype or NULL (may
 *      equal y: each element is read before it is written).
 * Out: y [T,H] dtype.
 */
ace_status moe_combine(const ace_moe_desc* d, const int32_t* slot_pos, const void* slot_out, const void* residual,
                       void* y, void* stream);

/*
 * moe_forward -- the whole layer in one call: moe_route_skip, moe_dispatch,
 * moe_expert_forward (path) and moe_combine with the arguments of those four
 * calls (same meanings, layouts and outputs; residual may be NULL).  For
 * decode-sized batches (1 <= T <= 8 with T*k <= 64 for path AUTO, or path
 * STREAM; desc->expert_pool = 0; logits_in NULL) the top-k, gates, skip
 * rule and dispatch run inside
 * the gate/up kernel's workgroups (two fewer dependent launches); every
 * output is bit-identical to the four separate calls.  All arguments are
 * validated before anything is launched.
 */
ace_status moe_forward(const ace_moe_desc* d, int32_t path, const void* x, const float* gamma, const float* w_router,
                       const float* router_bias, const float* logits_in, float* logits_out, const float* a_gsp,
                       const float* a_rcr, float tau_gsp, float tau_rcr, const void* w_gate, const void* w_up,
                       const void* w_down, const void* residual, void* h_out, int32_t* topk_idx, float* topk_gate,
                       uint8_t* keep, int32_t* expert_offsets, int32_t* sorted_token, float* sorted_gate,
                       int32_t* slot_pos, void* act, void* slot_out, void* y, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * moe_forward_static -- moe_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments, results and kernels as moe_forward,
 * except that the slot activations (act), the slot outputs (slot_out) and
 * the dispatch workspace live in a static device buffer of
 * the library instead of caller memory.  Every output that moe_forward
 * writes to caller memory (h_out, logits_out, topk_idx, topk_gate, keep,
 * expert_offsets, sorted_token, sorted_gate, slot_pos, y) is written here
 * too, bit-identical to moe_forward's.
 *   - Limit: the call needs round256(T*k*I*dtype bytes) +
 *     round256(T*k*H*dtype bytes) + round256(dispatch workspace) <=
 *     ACE_STATIC_SCRATCH_BYTES (80 MiB; e.g. T = 1024 and T = 1536 at
 *     H = 2048, I = 768, k = 8 in bf16 fit, T = 2048 does not).  Larger batches are rejected with ACE_EUNSUPPORTED before anything
 *     is launched.
 *   - The buffer is a file-scope __device__ array: each device that runs the
 *     library holds its own 80 MiB copy until the process ends.  The first
 *     call on a device (with a non-empty batch) looks its address up once
 *     (hipGetSymbolAddress, a host query that allocates nothing); make that
 *     first call outside graph capture.  The call itself never calls hipMalloc,
 *     hipFree or any allocating routine.
 *   - Every call on one device shares that device's buffer and it keeps the
 *     last call's contents; nothing in it needs to start at zero (every
 *     kernel writes the rows it later reads).  Calls that overlap on one
 *     device (different streams or threads without ordering) race on the
 *     buffer and give undefined results: serialise them.
 */
#define ACE_STATIC_SCRATCH_BYTES (80u << 20)
ace_status moe_forward_static(const ace_moe_desc* d, int32_t path, const void* x, const float* gamma,
                              const float* w_router, const float* router_bias, const float* logits_in,
                              float* logits_out, const float* a_gsp, const float* a_rcr, float tau_gsp,
                              float tau_rcr, const void* w_gate, const void* w_up, const void* w_down,
                              const void* residual, void* h_out, int32_t* topk_idx, float* topk_gate, uint8_t* keep,
                              int32_t* expert_offsets, int32_t* sorted_token, float* sorted_gate, int32_t* slot_pos,
                              void* y, void* stream);

/*
 * moe_calibrate_thresholds -- per-layer thresholds (tau_gsp, tau_rcr) by
 * quantile mapping (Efficiency Results, Table 6) for a target skip rate over
 * all T*k routed slots, matched to the given batch's own routing.
 * Reading used: eligible slots are all but the top-1; each view ranks their
 * scores g*A(e) ascending (ties by slot order); a slot's fused rank is the
 * larger of its two ranks (max-fusion); with n = floor(skip_rate*T*k + 1/2),
 * m is the largest level with #{fused rank < m} <= n, and tau_v lies strictly
 * between view v's (m-1)-th and m-th smallest score (float32 midpoint).  Then
 * moe_route_skip with these thresholds skips n-1 or n slots of this batch.
 * n = 0 gives (0, 0); skipping every eligible slot gives just above the
 * largest scores.
 * In:  topk_idx, topk_gate [T,k] (from moe_route_skip; thresholds passed to
 *      it do not matter); a_gsp, a_rcr [E]; skip_rate in [0, (k-1)/k].
 * Out: tau_out [2] f32 (device); level_out [2] i32 (m, n) or NULL.
 * workspace: >= moe_calibrate_workspace_bytes(d) bytes.
 */
size_t moe_calibrate_workspace_bytes(const ace_moe_desc* d);
ace_status moe_calibrate_thresholds(const ace_moe_desc* d, const int32_t* topk_idx, const float* topk_gate,
                                    const float* a_gsp, const float* a_rcr, float skip_rate, float* tau_out,
                                    int32_t* level_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_pack_weights -- copy expert weights from the LINEAR layout into the
 * PACKED layout (see ace_weight_layout), typically once when a checkpoint is
 * loaded.  which = 0: a gate or up projection [E, I, H]; which = 1: the down
 * projection [E, H, I].  src and dst hold E*N*K elements of desc->dtype and
 * must not overlap.  desc->weight_layout is ignored here.
 */
ace_status moe_pack_weights(const ace_moe_desc* d, int32_t which, const void* src, void* dst, void* stream);

/*
 * moe_pack_router -- split float32 router weights w_router [E, H] exactly into
 * three bf16 planes (w = hi + mid + lo, each rounded to nearest even, the
 * residuals exact) laid out for the router's MFMA operand:
 * [3][ceil(E/16)][H/32][64][8 bf16], entry [p][c][j][l][v] = plane p of
 * w_router[16c + l%16][32j + 8(l/16) + v] (zero for rows >= E).  Typically
 * once per checkpoint; moe_route_skip then reads it when
 * desc->router_layout = ACE_LAYOUT_PACKED.  bf16 activations only (the split
 * gives exact float32 products with bf16 h).  dst holds
 * moe_router_packed_bytes(d) bytes.
 */
size_t moe_router_packed_bytes(const ace_moe_desc* d);
ace_status moe_pack_router(const ace_moe_desc* d, const float* w_router, void* dst, void* stream);

/*
 * moe_build_tables -- the offline per-expert tables from the layer's own
 * weights ("ACE: Adaptive Calibration-Free Expert Skipping for MoE-based
 * LLMs", Methodology sections 1 and 2), typically once per checkpoint.
 * With W^gate = w_gate[e]^T, W^up = w_up[e]^T (H x I), W^down = w_down[e]^T
 * (I x H) and Gamma = diag(gamma):
 *   GSP: a_up = |Gamma W^up|_F * |Gamma W^gate W^down|_F,
 *        a_gate = |Gamma W^gate|_F * |Gamma W^up W^down|_F,
 *        raw_e = sqrt(a_up * a_gate);
 *   RCR: q_e = (w_router[e] - mean_j w_router[j]) / (RMS(that) + eps)
 *        (prototype scale 1), raw_e = |f_e(q_e)| / (|q_e| + eps) where f_e is
 *        the SwiGLU expert applied to q_e in the role of the normalised token,
 *        i.e. to q_e * gamma;
 *   both: a[e] = raw_e / (mean over experts of raw + eps).
 * Computed on the device: the Frobenius norms through I x I Gram matrices
 * (bf16 MFMA with exact products, float32 accumulation, float64 sums); RCR
 * in float32 with float64 final sums.  Deterministic.
 * In:  gamma [H] f32; w_router [E,H] f32 (plain rows); w_gate, w_up [E,I,H]
 *      and w_down [E,H,I] of desc->dtype in the LINEAR layout (a PACKED
 *      desc->weight_layout is rejected); eps >= 0 (1e-6 is the usual value).
 * Out: a_gsp [E], a_rcr [E] f32 (device).  T, k, fusion and router_layout of
 *      the descriptor are not used.
 * workspace: moe_tables_workspace_bytes(d) bytes is the preferred size
 *      (transposed w_down for a batch of experts, at most 512 MiB of it, plus
 *      per-expert partials).  A smaller workspace is accepted down to the
 *      size for batches of one expert (else ACE_EWORKSPACE): the builder then
 *      uses the largest batch that fits.  The result does not depend on it.
 */
size_t moe_tables_workspace_bytes(const ace_moe_desc* d);
ace_status moe_build_tables(const ace_moe_desc* d, float eps, const float* gamma, const float* w_router,
                            const void* w_gate, const void* w_up, const void* w_down, float* a_gsp, float* a_rcr,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_hbm_read_probe -- a measuring aid, not a step of the layer: reads
 * `bytes` (a multiple of 16) of device memory at `buf` once, with 16-byte
 * loads spread over `workgroups` workgroups of 256 threads (a grid-stride
 * loop, eight independent loads in flight per thread), and writes one
 * 32-bit fold of the words read per workgroup to sink [workgroups] (device).
 * Timing it gives the streaming HBM read rate that the weight-streaming
 * expert kernels are compared with, beside the datasheet peak.
 */
ace_status moe_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream);

/*
 * moe_l2_load_probe -- a measuring aid, not a step of the layer: each wave of
 * `workgroups` workgroups of 256 threads runs `rounds` rounds of `loads`
 * (6 or 8) 1 KB loads (lane l reads 16 bytes at 16 l of a block) from `buf`
 * (`bytes` a power of two in [2 MiB, 1 GiB], small enough to stay in L2 at
 * 2 MiB), the next round's loads issued before this round's blocks are
 * used; each block feeds `mfma_per_load` (0, 4 or 8) bf16 MFMAs as their B
 * operand.  stride_mode 0: a round's blocks are consecutive; 1: block j sits
 * at (j % 3) * 512 KB + (j / 3) * 64 KB past the round's base.  Each wave
 * writes one 32-bit fold to sink [workgroups * 4] (device).  Timing it gives
 * the load rate a compute unit sustains from L2 with and without MFMAs.
 */
ace_status moe_l2_load_probe(const void* buf, size_t bytes, int32_t rounds, int32_t loads, int32_t mfma_per_load,
                             int32_t stride_mode, uint32_t* sink, int32_t workgroups, void* stream);

/*
 * moe_set_kernel_events -- for profiling callers: the next moe_expert_forward
 * on this thread records `start` (a hipEvent_t) on its stream just before the
 * gate/up kernel and `stop` just after it, then forgets both.  NULL clears.
 */
ace_status moe_set_kernel_events(void* start, void* stop);

#ifdef __cplusplus
}
#endif
#endif /* ACE_MOE_H */
