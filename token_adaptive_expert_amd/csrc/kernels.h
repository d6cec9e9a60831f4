// Kernel argument blocks and host-side launchers shared by the C ABI.
#pragma once

#include "common.h"

namespace ace {

struct RouteArgs {
  const void* x;
  const float* gamma;
  const float* w_router;
  const float* bias;
  const float* logits_in;
  float* logits_out;
  const float* a_gsp;
  const float* a_rcr;
  float tau_gsp, tau_rcr;
  void* h_out;
  int32_t* topk_idx;
  float* topk_gate;
  uint8_t* keep;
  int T, H, E, k, norm_topk, fusion;
  float eps;
  int router_packed;  // w_router holds the pre-split bf16 planes (bf16 activations only)
};

struct DispatchArgs {
  const int32_t* idx;
  const float* gate;
  const uint8_t* keep;
  int32_t* offsets;
  int32_t* sorted_token;
  float* sorted_gate;
  int32_t* slot_pos;
  int T, E, k;
  int pool;      // 0: off; m >= 1: batch-level expert-pool cap (T*k <= 8192)
  int32_t* ws;   // workspace: per-block expert counts and row bases (large batches)
};

struct ExpertArgs {
  const void* A;              // gate/up: h [T, H] (rows gathered by sorted_token); down: act [*, I]
  const void* W0;             // gate/up: w_gate; down: w_down
  const void* W1;             // gate/up: w_up; down: unused
  const int32_t* offsets;     // [E+1]
  const int32_t* sorted_token;
  const float* sorted_gate;
  void* out;                  // gate/up: act [*, I]; down: slot_out [*, H] (both dtype)
  int K;                      // contraction length: H (gate/up) or I (down)
  int N;                      // weight rows per expert: I (gate/up) or H (down)
  int E;
  int packed;                 // weights in the packed fragment layout
  int A_rows;                 // rows of A: T (gate/up) or T*k (down)
};

// Fused small-batch gate/up (T <= FUSED_TMAX tokens): routing and dispatch are
// derived from the router logits inside every workgroup; workgroup 0 writes them.
constexpr int FUSED_TMAX = 32;
struct FusedArgs {
  ExpertArgs g;               // gate/up GEMM (offsets / sorted_token unused: made in LDS)
  const float* logits;        // [T, E] f32
  const float* a_gsp;
  const float* a_rcr;
  float tau_gsp, tau_rcr;
  int T, k, norm_topk, fusion;
  int32_t* topk_idx;          // outputs, written by workgroup 0
  float* topk_gate;
  uint8_t* keep;
  int32_t* offsets;
  int32_t* sorted_token;
  float* sorted_gate;
  int32_t* slot_pos;
};

struct CombineArgs {
  const int32_t* slot_pos;
  const void* slot_out;       // [*, H] dtype
  const void* residual;
  void* y;
  int T, H, k;
};

struct CalibArgs {
  const int32_t* idx;
  const float* gate;
  const float* a_gsp;
  const float* a_rcr;
  float* tau_out;       // [2]
  int32_t* level_out;   // [2] (m, n) or null
  int32_t* ws_rank_g;
  int32_t* ws_rank_r;
  float* ws_score_g;    // scores in ascending rank order
  float* ws_score_r;
  uint64_t* ws_key_g;   // (score, slot) keys, sorted within tiles of CALIB_TILE
  uint64_t* ws_key_r;
  int T, k, N, n_target;
};
constexpr int CALIB_TILE = 1024;

struct TablesArgs {
  const float* gamma;     // [H]
  const float* w_router;  // [E, H] f32
  const void* w_gate;     // [E, I, H] dtype (linear layout)
  const void* w_up;       // [E, I, H]
  const void* w_down;     // [E, H, I]
  float* a_gsp;           // [E] out
  float* a_rcr;           // [E] out
  int E, H, I;
  float eps;
  // workspace regions, set by launch_tables
  void* ws_wdT;
  double* ws_part;
  float* ws_mean;
  float* ws_x;
  float* ws_qnorm;
  float* ws_v;
  double* ws_opart;
  double* ws_raw_gsp;
  double* ws_raw_rcr;
};

// Host launchers (return the launch status).
// with_topk false: RMSNorm and router logits only (the fused small-batch
// path derives the top-k itself).
hipError_t launch_route(int dtype, const RouteArgs& a, hipStream_t s, bool with_topk = true);
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);
size_t dispatch_workspace_bytes(int T, int E, int k);
// kind 0: gate/up, 1: down; stream_path selects the small-batch tiling.
hipError_t launch_expert(int dtype, int kind, bool stream_path, const ExpertArgs& a, int T, int k, int num_cu,
                         hipStream_t s);
hipError_t launch_combine(int dtype, const CombineArgs& a, hipStream_t s);
hipError_t launch_fused_gateup(int dtype, const FusedArgs& a, int num_cu, hipStream_t s);
size_t router_packed_bytes(int E, int H);
hipError_t launch_pack_router(const float* w, void* dst, int E, int H, hipStream_t s);
hipError_t launch_pack(int dtype, const void* src, void* dst, int E, int N, int K, hipStream_t s);
size_t calib_workspace_bytes(int T, int k);
hipError_t launch_calibrate(CalibArgs a, void* workspace, hipStream_t s);
// minimum: the smallest workspace (Gram batches of one expert); else the preferred size.
size_t tables_workspace_bytes(int E, int H, int I, int dtype, bool minimum);
// Uses the largest Gram batch that workspace_bytes holds.
hipError_t launch_tables(int dtype, TablesArgs a, void* workspace, size_t workspace_bytes, hipStream_t s);
// Streaming-read probe (measuring aid): reads bytes (a multiple of 16) of src,
// writes one word per workgroup to sink.
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t s);
hipError_t launch_l2_probe(const void* buf, size_t bytes, int rounds, int loads, int mfma_per_load, int stride_mode,
                           uint32_t* sink, int workgroups, hipStream_t s);

}  // namespace ace
