// C ABI of the ACE MoE layer library: argument checks, path choice and
// kernel launches.  Declarations and contracts: include/ace_moe.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/ace_moe.h"
#include "kernels.h"

// Device scratch of moe_forward_static: the slot activations, the float32
// slot outputs and the dispatch workspace of one call, for callers that
// cannot allocate.  Each device that runs the library holds its own copy
// until the process ends.  Host code must never pass `scratch` itself to a
// kernel (on the host it names a stand-in, not device memory): it uses the
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[ACE_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;

ace_status fail(ace_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

ace_status ok() {
  g_err.clear();
  return ACE_OK;
}

ace_status hip_fail(const char* what, hipError_t e) {
  return fail(ACE_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), int(e));
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cu[kMaxDevices];

// Compute units of the current device (cached per device).
ace_status num_cu(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) return fail(ACE_EUNSUPPORTED, "device index %d out of range", dev);
  int n = g_num_cu[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail("hipDeviceGetAttribute", e);
    g_num_cu[dev].store(n, std::memory_order_relaxed);
  }
  *out = n;
  return ACE_OK;
}

ace_status check_desc(const ace_moe_desc* d) {
  if (d == nullptr) return fail(ACE_EINVAL, "desc is NULL");
  if (d->T < 0) return fail(ACE_EINVAL, "T=%d is negative", d->T);
  if (d->H <= 0 || d->E <= 0 || d->I <= 0 || d->k <= 0)
    return fail(ACE_EINVAL, "H=%d E=%d I=%d k=%d must be positive", d->H, d->E, d->I, d->k);
  if (d->dtype != ACE_F32 && d->dtype != ACE_BF16) return fail(ACE_EINVAL, "dtype=%d is not an ace_dtype", d->dtype);
  if (d->fusion < ACE_FUSE_MAX || d->fusion > ACE_FUSE_SCORE)
    return fail(ACE_EINVAL, "fusion=%d is not an ace_fusion", d->fusion);
  if (d->norm_topk != 0 && d->norm_topk != 1) return fail(ACE_EINVAL, "norm_topk=%d must be 0 or 1", d->norm_topk);
  if (!(d->rms_eps >= 0.f)) return fail(ACE_EINVAL, "rms_eps must be >= 0");
  if (d->weight_layout != ACE_LAYOUT_LINEAR && d->weight_layout != ACE_LAYOUT_PACKED)
    return fail(ACE_EINVAL, "weight_layout=%d is not an ace_weight_layout", d->weight_layout);
  if (d->router_layout != ACE_LAYOUT_LINEAR && d->router_layout != ACE_LAYOUT_PACKED)
    return fail(ACE_EINVAL, "router_layout=%d is not an ace_weight_layout", d->router_layout);
  if (d->router_layout == ACE_LAYOUT_PACKED && d->dtype != ACE_BF16)
    return fail(ACE_EUNSUPPORTED, "router_layout=PACKED needs bf16 activations");
  if (d->expert_pool < 0) return fail(ACE_EINVAL, "expert_pool=%d must be >= 0", d->expert_pool);
  if (d->expert_pool > 0 && int64_t(d->T) * d->k > 8192)
    return fail(ACE_EUNSUPPORTED, "expert_pool needs T*k <= 8192 (got %lld)", (long long)(int64_t(d->T) * d->k));
  if (d->E > 256) return fail(ACE_EUNSUPPORTED, "E=%d > 256", d->E);
  if (d->k > 16 || d->k > d->E) return fail(ACE_EUNSUPPORTED, "k=%d must be <= min(E, 16)", d->k);
  if (d->H % 128 != 0) return fail(ACE_EUNSUPPORTED, "H=%d is not a multiple of 128", d->H);
  if (d->I % 128 != 0) return fail(ACE_EUNSUPPORTED, "I=%d is not a multiple of 128", d->I);
  if (int64_t(d->T) * d->k >= (int64_t(1) << 31)) return fail(ACE_EUNSUPPORTED, "T*k >= 2^31");
  {
    const int64_t es = d->dtype == ACE_BF16 ? 2 : 4;
    const int64_t lim = (int64_t(1) << 31) - 1;
    if (int64_t(d->H) * d->I * es > lim) return fail(ACE_EUNSUPPORTED, "H*I too large for one expert");
    if (int64_t(d->T) * d->k * std::max(d->H, d->I) * es > lim)
      return fail(ACE_EUNSUPPORTED, "T*k*max(H,I) activations exceed 2 GiB");
  }
  return ACE_OK;
}

// Device pointers: required ones must be non-NULL; all must be 16-byte
// aligned (the kernels use 16-byte vector loads and stores).
// Largest batch that moe_forward runs through the fused small-batch kernel
// (at most ace::FUSED_TMAX).
// AUTO path: batches of at most this many routed slots take the split-K
// ("stream") expert tiling, larger ones the grouped tiling.
#ifndef ACE_STREAM_MAX_SLOTS
#define ACE_STREAM_MAX_SLOTS 64
#endif
#ifndef ACE_FUSED_TOKENS
#define ACE_FUSED_TOKENS 8
#endif
static_assert(ACE_FUSED_TOKENS <= ace::FUSED_TMAX, "fused kernel: at most FUSED_TMAX tokens");

#define REQUIRE(p)                                                                                     \
  do {                                                                                                 \
    if ((p) == nullptr) return fail(ACE_EINVAL, "%s is NULL", #p);                                     \
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(ACE_EINVAL, "%s is not 16-byte aligned", #p); \
  } while (0)
#define ALIGNED_OR_NULL(p)                                                                           \
  do {                                                                                               \
    if ((p) != nullptr && reinterpret_cast<uintptr_t>(p) % 16 != 0)                                  \
      return fail(ACE_EINVAL, "%s is not 16-byte aligned", #p);                                      \
  } while (0)

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
ace_status static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) return fail(ACE_EUNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", e);
    if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0)
      return fail(ACE_EHIP, "hipGetSymbolAddress(scratch) gave an unusable address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ACE_OK;
}

// Arguments of moe_forward other than its scratch (act, slot_out, workspace);
// shared with moe_forward_static.  Every argument is checked before anything
// is launched.
ace_status check_forward_args(const ace_moe_desc* d, int32_t path, const void* x, const float* gamma,
                              const float* w_router, const float* router_bias, const float* logits_in,
                              const float* logits_out, const float* a_gsp, const float* a_rcr, float tau_gsp,
                              float tau_rcr, const void* w_gate, const void* w_up, const void* w_down,
                              const void* residual, const void* h_out, const int32_t* topk_idx,
                              const float* topk_gate, const uint8_t* keep, const int32_t* expert_offsets,
                              const int32_t* sorted_token, const float* sorted_gate, const int32_t* slot_pos,
                              const void* y) {
  ace_status st = check_desc(d);
  if (st != ACE_OK) return st;
  if (path < ACE_PATH_AUTO || path > ACE_PATH_STREAM) return fail(ACE_EINVAL, "path=%d is not an ace_path", path);
  REQUIRE(x);
  REQUIRE(gamma);
  if (logits_in == nullptr) REQUIRE(w_router);
  REQUIRE(logits_out);
  if (logits_in == logits_out) return fail(ACE_EINVAL, "logits_in and logits_out must not alias");
  ALIGNED_OR_NULL(router_bias);
  ALIGNED_OR_NULL(logits_in);
  ALIGNED_OR_NULL(residual);
  REQUIRE(a_gsp);
  REQUIRE(a_rcr);
  REQUIRE(w_gate);
  REQUIRE(w_up);
  REQUIRE(w_down);
  REQUIRE(h_out);
  REQUIRE(topk_idx);
  REQUIRE(topk_gate);
  REQUIRE(keep);
  REQUIRE(expert_offsets);
  REQUIRE(sorted_token);
  REQUIRE(sorted_gate);
  REQUIRE(slot_pos);
  REQUIRE(y);
  if (!(tau_gsp >= 0.f) || !(tau_rcr >= 0.f))
    return fail(ACE_EINVAL, "thresholds must be >= 0 (got %g, %g)", double(tau_gsp), double(tau_rcr));
  return ACE_OK;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

extern "C" {

int moe_abi_version(void) { return ACE_MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_err.c_str(); }

size_t moe_workspace_bytes(const ace_moe_desc* d) {
  if (check_desc(d) != ACE_OK) return 0;
  return ace::dispatch_workspace_bytes(std::max(d->T, 1), d->E, d->k);
}

ace_status moe_route_skip(const ace_moe_desc* d, const void* x, const float* gamma, const float* w_router,
                          const float* router_bias, const float* logits_in, float* logits_out, const float* a_gsp,
                          const float* a_rcr, float tau_gsp, float tau_rcr, void* h_out, int32_t* topk_idx,
                          float* topk_gate, uint8_t* keep, void* stream) {
  try {
    ace_status st = check_desc(d);
    if (st != ACE_OK) return st;
    REQUIRE(x);
    REQUIRE(gamma);
    if (logits_in == nullptr) REQUIRE(w_router);
    REQUIRE(logits_out);
    if (logits_in == logits_out) return fail(ACE_EINVAL, "logits_in and logits_out must not alias");
    ALIGNED_OR_NULL(router_bias);
    ALIGNED_OR_NULL(logits_in);
    REQUIRE(a_gsp);
    REQUIRE(a_rcr);
    REQUIRE(h_out);
    REQUIRE(topk_idx);
    REQUIRE(topk_gate);
    REQUIRE(keep);
    if (!(tau_gsp >= 0.f) || !(tau_rcr >= 0.f)) return fail(ACE_EINVAL, "thresholds must be >= 0 (got %g, %g)",
                                                            double(tau_gsp), double(tau_rcr));
    if (d->T == 0) return ok();
    ace::RouteArgs a;
    a.x = x;
    a.gamma = gamma;
    a.w_router = w_router;
    a.bias = router_bias;
    a.logits_in = logits_in;
    a.logits_out = logits_out;
    a.a_gsp = a_gsp;
    a.a_rcr = a_rcr;
    a.tau_gsp = tau_gsp;
    a.tau_rcr = tau_rcr;
    a.h_out = h_out;
    a.topk_idx = topk_idx;
    a.topk_gate = topk_gate;
    a.keep = keep;
    a.T = d->T;
    a.H = d->H;
    a.E = d->E;
    a.k = d->k;
    a.norm_topk = d->norm_topk;
    a.fusion = d->fusion;
    a.eps = d->rms_eps;
    a.router_packed = d->router_layout == ACE_LAYOUT_PACKED ? 1 : 0;
    hipError_t e = ace::launch_route(d->dtype, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("route_skip launch", e);
    return ok();
  } catch (...) {
    return fail(ACE_EHIP, "unexpected host exception in moe_route_skip");
  }
}

ace_status moe_dispatch(const ace_moe_desc* d, const int32_t* topk_idx, const float* topk_gate, const uint8_t* keep,
                        int32_t* expert_offsets, int32_t* sorted_token, float* sorted_gate, int32_t* slot_pos,
                        void* workspace, size_t workspace_bytes, void* stream) {
  try {
    ace_status st = check_desc(d);
    if (st != ACE_OK) return st;
    REQUIRE(topk_idx);
    REQUIRE(topk_gate);
    REQUIRE(keep);
    REQUIRE(expert_offsets);
    REQUIRE(sorted_token);
    REQUIRE(sorted_gate);
    REQUIRE(slot_pos);
    REQUIRE(workspace);
    const size_t need = ace::dispatch_workspace_bytes(std::max(d->T, 1), d->E, d->k);
    if (workspace_bytes < need)
      return fail(ACE_EWORKSPACE, "workspace_bytes=%zu < %zu needed", workspace_bytes, need);
    if (d->T == 0) return ok();
    ace::DispatchArgs a;
    a.idx = topk_idx;
    a.gate = topk_gate;
    a.keep = keep;
    a.offsets = expert_offsets;
    a.sorted_token = sorted_token;
    a.sorted_gate = sorted_gate;
    a.slot_pos = slot_pos;
    a.T = d->T;
    a.E = d->E;
    a.k = d->k;
    a.pool = d->expert_pool;
    a.ws = static_cast<int32_t*>(workspace);
    hipError_t e = ace::launch_dispatch(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("dispatch launch", e);
    return ok();
  } catch (...) {
    return fail(ACE_EHIP, "unexpected host exception in moe_dispatch");
  }
}

ace_status moe_expert_forward(const ace_moe_desc* d, int32_t path, const void* h, const void* w_gate,
                              const void* w_up, const void* w_down, const int32_t* expert_offsets,
                              const int32_t* sorted_token, const float* sorted_gate, void* act, void* slot_out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  try {
    ace_status st = check_desc(d);
    if (st != ACE_OK) return st;
    const int stages = path & (ACE_STAGE_GATEUP | ACE_STAGE_DOWN);
    const bool run_gu = stages == 0 || (stages & ACE_STAGE_GATEUP);
    const bool run_dn = stages == 0 || (stages & ACE_STAGE_DOWN);
    path &= ~(ACE_STAGE_GATEUP | ACE_STAGE_DOWN);
    if (path < ACE_PATH_AUTO || path > ACE_PATH_STREAM) return fail(ACE_EINVAL, "path=%d is not an ace_path", path);
    REQUIRE(h);
    REQUIRE(w_gate);
    REQUIRE(w_up);
    REQUIRE(w_down);
    REQUIRE(expert_offsets);
    REQUIRE(sorted_token);
    REQUIRE(sorted_gate);
    REQUIRE(act);
    REQUIRE(slot_out);
    REQUIRE(workspace);
    if (workspace_bytes < ace::dispatch_workspace_bytes(d->T, d->E, d->k))
      return fail(ACE_EWORKSPACE, "workspace_bytes=%zu < %zu needed", workspace_bytes,
                  ace::dispatch_workspace_bytes(d->T, d->E, d->k));
    if (d->T == 0) return ok();
    int ncu = 0;
    st = num_cu(&ncu);
    if (st != ACE_OK) return st;
    const bool stream_path =
        path == ACE_PATH_STREAM || (path == ACE_PATH_AUTO && int64_t(d->T) * d->k <= ACE_STREAM_MAX_SLOTS);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t ev0 = g_ev_start, ev1 = g_ev_stop;
    g_ev_start = g_ev_stop = nullptr;

    ace::ExpertArgs gu;
    gu.A = h;
    gu.W0 = w_gate;
    gu.W1 = w_up;
    gu.offsets = expert_offsets;
    gu.sorted_token = sorted_token;
    gu.sorted_gate = sorted_gate;
    gu.out = act;
    gu.K = d->H;
    gu.N = d->I;
    gu.E = d->E;
    gu.packed = d->weight_layout == ACE_LAYOUT_PACKED ? 1 : 0;
    gu.A_rows = d->T;
    hipError_t e;
    if (ev0) {
      e = hipEventRecord(ev0, s);
      if (e != hipSuccess) return hip_fail("hipEventRecord", e);
    }
    if (run_gu) {
      e = ace::launch_expert(d->dtype, 0, stream_path, gu, d->T, d->k, ncu, s);
      if (e != hipSuccess) return hip_fail("gate/up launch", e);
    }
    if (ev1) {
      e = hipEventRecord(ev1, s);
      if (e != hipSuccess) return hip_fail("hipEventRecord", e);
    }
    ace::ExpertArgs dn = gu;
    dn.A = act;
    dn.W0 = w_down;
    dn.W1 = nullptr;
    dn.out = slot_out;
    dn.K = d->I;
    dn.N = d->H;
    dn.A_rows = d->T * d->k;
    if (run_dn) {
      e = ace::launch_expert(d->dtype, 1, stream_path, dn, d->T, d->k, ncu, s);
      if (e != hipSuccess) return hip_fail("down launch", e);
    }
    return ok();
  } catch (...) {
    return fail(ACE_EHIP, "unexpected host exception in moe_expert_forward");
  }
}

ace_status moe_combine(const ace_moe_desc* d, const int32_t* slot_pos, const void* slot_out, const void* residual,
                       void* y, void* stream) {
  try {
    ace_status st = check_desc(d);
    if (st != ACE_OK) return st;
    REQUIRE(slot_pos);
    REQUIRE(slot_out);
    REQUIRE(y);
    if (d->T == 0) return ok();
    ace::CombineArgs a;
    a.slot_pos = slot_pos;
    a.slot_out = slot_out;
    ALIGNED_OR_NULL(residual);
    a.residual = residual;
    a.y = y;
    a.T = d->T;
    a.H = d->H;
    a.k = d->k;
    hipError_t e = ace::launch_combine(d->dtype, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("combine launch", e);
    return ok();
  } catch (...) {
    return fail(ACE_EHIP, "unexpected host exception in moe_combine");
  }
}

size_t moe_calibrate_workspace_bytes(const ace_moe_desc* d) {
  if (check_desc(d) != ACE_OK) return 0;
  return std::max<size_t>(ace::calib_workspace_bytes(d->T, d->k), 256);
}

ace_status moe_calibrate_thresholds(const ace_moe_desc* d, const int32_t* topk_idx, const float* topk_gate,
                                    const float* a_gsp, const float* a_rcr, float skip_rate, float* tau_out,
                                    int32_t* level_out, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    ace_status st = check_desc(d);
    if (st != ACE_OK) return st;
    REQUIRE(topk_idx);
    REQUIRE(topk_gate);
    REQUIRE(a_gsp);
    REQUIRE(a_rcr);
    REQUIRE(tau_out);
    REQUIRE(workspace);
    const double max_rate = double(d->k - 1) / double(d->k);
    if (!(skip_rate >= 0.f) || double(skip_rate) > max_rate + 1e-7)
      return fail(ACE_EINVAL, "skip_rate=%g outside [0, (k-1)/k = %g]", double(skip_rate), max_rate);
    const size_t need = std::max<size_t>(ace::calib_workspace_bytes(d->T, d->k), 256);
    if (workspace_bytes < need)
      return fail(ACE_EWORKSPACE, "workspace_bytes=%zu < %zu needed", workspace_bytes, need);
    if (d->T == 0) return ok();
    const int64_t slots = int64_t(d->T) * d->k;
    const int64_t N = int64_t(d->T) * (d->k - 1);
    int64_t n = int64_t(std::floor(double(skip_rate) * double(slots) + 0.5));
    n = std::min(n, N);
    ace::CalibArgs a{};
    a.idx = topk_idx;
    a.gate = topk_gate;
    a.a_gsp = a_gsp;
    a.a_rcr = a_rcr;
    a.tau_out = tau_out;
    ALIGNED_OR_NULL(level_out);
    a.level_out = level_out;
    a.T = d->T;
    a.k = d->k;
    a.N = int(N);
    a.n_target = int(n);
    hipError_t e = ace::launch_calibrate(a, workspace, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("calibrate launch", e);
    return ok();
  } catch (...) {
    return fail(ACE_EHIP, "unexpected host exception in moe_calibrate_thresholds");
  }
}

ace_status moe_pack_weights(const ace_moe_desc* d, int32_t which, const void* src, void* dst, void* stream) {
  try {
    ace_status st = check_desc(d);
    if (st != ACE_OK) return st;
    if (which != 0 && which != 1) return fail(ACE_EINVAL, "which=%d must be 0 (gate/up) or 1 (down)", which);
    REQUIRE(src);
    REQUIRE(dst);
    const int N = which == 0 ? d->I : d->H, K = which == 0 ? d->H : d->I;
    const size_t bytes = size_t(d->E) * N * K * (d->dtype == ACE_BF16 ? 2 : 4);
    const uint8_t* s0 = static_cast<const uint8_t*>(src);
    const uint8_t* d0 = static_cast<const uint8_t*>(dst);
    if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(ACE_EINVAL, "src and dst overlap");
    hipError_t e = ace::launch_pack(d->dtype, src, dst, d->E, N, K, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("pack launch", e);
    return ok();
  } catch (...) {
    return fail(ACE_EHIP, "unexpected host exception in moe_pack_weights");
  }
}

size_t moe_router_packed_bytes(const ace_moe_desc* d) {
  if (check_desc(d) != ACE_OK) return 0;
  return ace::router_packed_bytes(d->E, d->H);
}

ace_status moe_pack_router(const ace_moe_desc* d, const float* w_router, void* dst, void* stream) {
  try {
    ace_status st = check_desc(d);
    if (st != ACE_OK) return st;
    if (d->dtype != ACE_BF16) return fail(ACE_EUNSUPPORTED, "the packed router needs bf16 activations");
    REQUIRE(w_router);
    REQUIRE(dst);
    const size_t sb = size_t(d->E) * d->H * 4, db = ace::router_packed_bytes(d->E, d->H);
    const uint8_t* s0 = reinterpret_cast<const uint8_t*>(w_router);
    const uint8_t* d0 = static_cast<const uint8_t*>(dst);
    if (s0 < d0 + db && d0 < s0 + sb) return fail(ACE_EINVAL, "w_router and dst overlap");
    hipError_t e = ace::launch_pack_router(w_router, dst, d->E, d->H, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("pack_router launch", e);
    return ok();
  } catch (...) {
    return fail(ACE_EHIP, "unexpected host exception in moe_pack_router");
  }
}

ace_status moe_forward(const ace_moe_desc* d, int32_t path, const void* x, const float* gamma, const float* w_router,
                       const float* router_bias, const float* logits_in, float* logits_out, const float* a_gsp,
                       const float* a_rcr, float tau_gsp, float tau_rcr, const void* w_gate, const void* w_up,
                       const void* w_down, const void* residual, void* h_out, int32_t* topk_idx, float* topk_gate,
                       uint8_t* keep, int32_t* expert_offsets, int32_t* sorted_token, float* sorted_gate,
                       int32_t* slot_pos, void* act, void* slot_out, void* y, void* workspace,
                       size_t workspace_bytes, void* stream) {
  try {
    ace_status st = check_forward_args(d, path, x, gamma, w_router, router_bias, logits_in, logits_out, a_gsp, a_rcr,
                                       tau_gsp, tau_rcr, w_gate, w_up, w_down, residual, h_out, topk_idx, topk_gate,
                                       keep, expert_offsets, sorted_token, sorted_gate, slot_pos, y);
    if (st != ACE_OK) return st;
    REQUIRE(act);
    REQUIRE(slot_out);
    REQUIRE(workspace);
    const size_t need = ace::dispatch_workspace_bytes(std::max(d->T, 1), d->E, d->k);
    if (workspace_bytes < need) return fail(ACE_EWORKSPACE, "workspace_bytes=%zu < %zu needed", workspace_bytes, need);
    if (d->T == 0) return ok();
    // the fused kernel is the split-K tiling: only where moe_expert_forward would take it too
    const bool fused = d->T <= ACE_FUSED_TOKENS && d->expert_pool == 0 && logits_in == nullptr &&
                       (path == ACE_PATH_STREAM || (path == ACE_PATH_AUTO && int64_t(d->T) * d->k <= ACE_STREAM_MAX_SLOTS));
    if (!fused) {
      st = moe_route_skip(d, x, gamma, w_router, router_bias, logits_in, logits_out, a_gsp, a_rcr, tau_gsp, tau_rcr,
                          h_out, topk_idx, topk_gate, keep, stream);
      if (st != ACE_OK) return st;
      st = moe_dispatch(d, topk_idx, topk_gate, keep, expert_offsets, sorted_token, sorted_gate, slot_pos, workspace,
                        workspace_bytes, stream);
      if (st != ACE_OK) return st;
      st = moe_expert_forward(d, path, h_out, w_gate, w_up, w_down, expert_offsets, sorted_token, sorted_gate, act,
                              slot_out, workspace, workspace_bytes, stream);
      if (st != ACE_OK) return st;
      return moe_combine(d, slot_pos, slot_out, residual, y, stream);
    }
    int ncu = 0;
    st = num_cu(&ncu);
    if (st != ACE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    ace::RouteArgs r{};
    r.x = x;
    r.gamma = gamma;
    r.w_router = w_router;
    r.bias = router_bias;
    r.logits_in = nullptr;
    r.logits_out = logits_out;
    r.h_out = h_out;
    r.T = d->T;
    r.H = d->H;
    r.E = d->E;
    r.k = d->k;
    r.eps = d->rms_eps;
    r.router_packed = d->router_layout == ACE_LAYOUT_PACKED ? 1 : 0;
    hipError_t e = ace::launch_route(d->dtype, r, s, false);
    if (e != hipSuccess) return hip_fail("router launch", e);
    ace::FusedArgs f{};
    f.g.A = h_out;
    f.g.W0 = w_gate;
    f.g.W1 = w_up;
    f.g.out = act;
    f.g.K = d->H;
    f.g.N = d->I;
    f.g.E = d->E;
    f.g.packed = d->weight_layout == ACE_LAYOUT_PACKED ? 1 : 0;
    f.g.A_rows = d->T;
    f.logits = logits_out;
    f.a_gsp = a_gsp;
    f.a_rcr = a_rcr;
    f.tau_gsp = tau_gsp;
    f.tau_rcr = tau_rcr;
    f.T = d->T;
    f.k = d->k;
    f.norm_topk = d->norm_topk;
    f.fusion = d->fusion;
    f.topk_idx = topk_idx;
    f.topk_gate = topk_gate;
    f.keep = keep;
    f.offsets = expert_offsets;
    f.sorted_token = sorted_token;
    f.sorted_gate = sorted_gate;
    f.slot_pos = slot_pos;
    e = ace::launch_fused_gateup(d->dtype, f, ncu, s);
    if (e != hipSuccess) return hip_fail("fused gate/up launch", e);
    ace::ExpertArgs dn{};
    dn.A = act;
    dn.W0 = w_down;
    dn.W1 = nullptr;
    dn.offsets = expert_offsets;
    dn.sorted_token = sorted_token;
    dn.sorted_gate = sorted_gate;
    dn.out = slot_out;
    dn.K = d->I;
    dn.N = d->H;
    dn.E = d->E;
    dn.packed = f.g.packed;
    dn.A_rows = d->T * d->k;
    e = ace::launch_expert(d->dtype, 1, true, dn, d->T, d->k, ncu, s);
    if (e != hipSuccess) return hip_fail("down launch", e);
    ace::CombineArgs c{};
    c.slot_pos = slot_pos;
    c.slot_out = slot_out;
    c.residual = residual;
    c.y = y;
    c.T = d->T;
    c.H = d->H;
    c.k = d->k;
    e = ace::launch_combine(d->dtype, c, s);
    if (e != hipSuccess) return hip_fail("combine launch", e);
    return ok();
  } catch (...) {
    return fail(ACE_EHIP, "unexpected host exception in moe_forward");
  }
}

ace_status moe_forward_static(const ace_moe_desc* d, int32_t path, const void* x, const float* gamma,
                              const float* w_router, const float* router_bias, const float* logits_in,
                              float* logits_out, const float* a_gsp, const float* a_rcr, float tau_gsp,
                              float tau_rcr, const void* w_gate, const void* w_up, const void* w_down,
                              const void* residual, void* h_out, int32_t* topk_idx, float* topk_gate, uint8_t* keep,
                              int32_t* expert_offsets, int32_t* sorted_token, float* sorted_gate, int32_t* slot_pos,
                              void* y, void* stream) {
  try {
    ace_status st = check_forward_args(d, path, x, gamma, w_router, router_bias, logits_in, logits_out, a_gsp, a_rcr,
                                       tau_gsp, tau_rcr, w_gate, w_up, w_down, residual, h_out, topk_idx, topk_gate,
                                       keep, expert_offsets, sorted_token, sorted_gate, slot_pos, y);
    if (st != ACE_OK) return st;
    const size_t es = d->dtype == ACE_BF16 ? 2 : 4;
    const size_t rows = size_t(d->T) * size_t(d->k);
    const size_t act_bytes = round256(rows * size_t(d->I) * es);
    const size_t out_bytes = round256(rows * size_t(d->H) * es);
    const size_t ws_bytes = round256(ace::dispatch_workspace_bytes(std::max(d->T, 1), d->E, d->k));
    const size_t need = act_bytes + out_bytes + ws_bytes;
    if (need > size_t(ACE_STATIC_SCRATCH_BYTES))
      return fail(ACE_EUNSUPPORTED,
                  "moe_forward_static: T=%d needs %zu bytes of scratch (slot activations, slot outputs, dispatch "
                  "workspace), more than the %zu of the static buffer; use moe_forward with caller memory",
                  d->T, need, size_t(ACE_STATIC_SCRATCH_BYTES));
    if (d->T == 0) return ok();
    void* base = nullptr;
    st = static_scratch(&base);
    if (st != ACE_OK) return st;
    unsigned char* b = static_cast<unsigned char*>(base);
    return moe_forward(d, path, x, gamma, w_router, router_bias, logits_in, logits_out, a_gsp, a_rcr, tau_gsp,
                       tau_rcr, w_gate, w_up, w_down, residual, h_out, topk_idx, topk_gate, keep, expert_offsets,
                       sorted_token, sorted_gate, slot_pos, b, b + act_bytes, y,
                       b + act_bytes + out_bytes, ws_bytes, stream);
  } catch (...) {
    return fail(ACE_EHIP, "unexpected host exception in moe_forward_static");
  }
}

size_t moe_tables_workspace_bytes(const ace_moe_desc* d) {
  if (check_desc(d) != ACE_OK) return 0;
  return ace::tables_workspace_bytes(d->E, d->H, d->I, d->dtype, false);
}

ace_status moe_build_tables(const ace_moe_desc* d, float eps, const float* gamma, const float* w_router,
                            const void* w_gate, const void* w_up, const void* w_down, float* a_gsp, float* a_rcr,
                            void* workspace, size_t workspace_bytes, void* stream) {
  try {
    ace_status st = check_desc(d);
    if (st != ACE_OK) return st;
    if (d->weight_layout != ACE_LAYOUT_LINEAR)
      return fail(ACE_EUNSUPPORTED, "moe_build_tables reads expert weights in the LINEAR layout");
    if (!(eps >= 0.f)) return fail(ACE_EINVAL, "eps must be >= 0");
    REQUIRE(gamma);
    REQUIRE(w_router);
    REQUIRE(w_gate);
    REQUIRE(w_up);
    REQUIRE(w_down);
    REQUIRE(a_gsp);
    REQUIRE(a_rcr);
    REQUIRE(workspace);
    const size_t need = ace::tables_workspace_bytes(d->E, d->H, d->I, d->dtype, true);
    if (workspace_bytes < need)
      return fail(ACE_EWORKSPACE, "workspace_bytes=%zu < %zu needed (batches of one expert)", workspace_bytes,
                  need);
    ace::TablesArgs a{};
    a.gamma = gamma;
    a.w_router = w_router;
    a.w_gate = w_gate;
    a.w_up = w_up;
    a.w_down = w_down;
    a.a_gsp = a_gsp;
    a.a_rcr = a_rcr;
    a.E = d->E;
    a.H = d->H;
    a.I = d->I;
    a.eps = eps;
    hipError_t e = ace::launch_tables(d->dtype, a, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("tables launch", e);
    return ok();
  } catch (...) {
    return fail(ACE_EHIP, "unexpected host exception in moe_build_tables");
  }
}

ace_status moe_l2_load_probe(const void* buf, size_t bytes, int32_t rounds, int32_t loads, int32_t mfma_per_load,
                             int32_t stride_mode, uint32_t* sink, int32_t workgroups, void* stream) {
  try {
    REQUIRE(buf);
    REQUIRE(sink);
    if (bytes < (size_t(2) << 20) || bytes > (size_t(1) << 30) || (bytes & (bytes - 1)) != 0)
      return fail(ACE_EINVAL, "bytes=%zu is not a power of two in [2 MiB, 1 GiB]", bytes);
    if (loads != 6 && loads != 8) return fail(ACE_EINVAL, "loads=%d is not 6 or 8", loads);
    if (mfma_per_load != 0 && mfma_per_load != 4 && mfma_per_load != 8)
      return fail(ACE_EINVAL, "mfma_per_load=%d is not 0, 4 or 8", mfma_per_load);
    if (stride_mode != 0 && stride_mode != 1) return fail(ACE_EINVAL, "stride_mode=%d is not 0 or 1", stride_mode);
    if (rounds < 1 || rounds > (1 << 24)) return fail(ACE_EINVAL, "rounds=%d outside [1, 2^24]", rounds);
    if (workgroups < 1 || workgroups > (1 << 20)) return fail(ACE_EINVAL, "workgroups=%d outside [1, 2^20]", workgroups);
    hipError_t e = ace::launch_l2_probe(buf, bytes, rounds, loads, mfma_per_load, stride_mode, sink, workgroups,
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("l2 probe launch", e);
    return ok();
  } catch (...) {
    return fail(ACE_EHIP, "unexpected host exception in moe_l2_load_probe");
  }
}

ace_status moe_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream) {
  try {
    REQUIRE(buf);
    REQUIRE(sink);
    if (bytes % 16 != 0) return fail(ACE_EINVAL, "bytes=%zu is not a multiple of 16", bytes);
    if (workgroups < 1 || workgroups > (1 << 20)) return fail(ACE_EINVAL, "workgroups=%d outside [1, 2^20]", workgroups);
    if (bytes == 0) return ok();
    hipError_t e = ace::launch_read_probe(buf, bytes, sink, workgroups, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("read probe launch", e);
    return ok();
  } catch (...) {
    return fail(ACE_EHIP, "unexpected host exception in moe_hbm_read_probe");
  }
}

ace_status moe_set_kernel_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr)) return fail(ACE_EINVAL, "start and stop must both be set or both NULL");
  g_ev_start = static_cast<hipEvent_t>(start);
  g_ev_stop = static_cast<hipEvent_t>(stop);
  return ok();
}

}  // extern "C"
