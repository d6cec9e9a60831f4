// Expert dispatch: group the kept routed slots by expert, in token order
// within each expert, with integer work only.
//
// The article page on ACE says only that surviving slots go through
// "optimized expert dispatch"; this grouping is the layout the expert GEMMs
// read.  Slots are numbered s = t*k + i.  A token routes to k distinct
// experts, so within one expert, slot order is token order.  One workgroup
// of 16 waves handles the batch; wave w owns a contiguous run of 64-slot
// chunks (so slot order is wave order, then chunk order, then lane order)
// and every load is one coalesced 64-lane read.  Everything stays in LDS:
//   1. each wave counts its kept slots per expert (LDS integer atomics:
//      order-independent totals);
//   2. expert totals -> expert_offsets (exclusive scan); per expert, the wave
//      counts -> each wave's first row inside the expert's segment;
//   3. each wave walks its chunks again in order: per chunk, the 64-bit mask
//      of its lanes holding each expert (LDS bitwise OR); a kept slot's row is
//      its wave's running row for that expert + the popcount of the mask bits
//      of lower lanes.
// Every result is a function of the inputs alone, independent of timing.
//
// With the batch-level expert-pool cap (POOL), step 3 keeps each kept slot's
// row (and expert) in LDS instead of writing it; then
//   4. per expert, S_e = the sum of its kept gates in row order (= slot
//      order), the number of experts that are some token's top-1, and the
//      rank of every other active expert by (S_e descending, index
//      ascending) among the compacted list of such experts; retained = top-1
//      expert or rank < m - #top-1; new offsets from the retained counts;
//   5. every slot's final row = its expert's new offset + its row inside the
//      expert's segment (unchanged: a retained expert keeps all its slots).
// Reading of the decode expert pool of "ExFold: Unified Expert Folding for
// Training-Free MoE Prefill-Decode Acceleration" (abstract; Tables 1, 5, 6),
// without the folding of excluded experts.
//
// Without the pool, batches of more than 1024 slots spread step 3 over
// several workgroups, each owning a block of consecutive slots:
//   * up to 32768 slots (recount mode): one workgroup per 1024 slots; each
//     counts the whole batch itself (per expert: all kept slots, and those
//     before its block), so one launch does the job;
//   * above that (block mode): one workgroup per 4096 slots, after
//     dispatch_count_kernel (each block's counts per expert) and
//     dispatch_scan_kernel (expert_offsets and each block's first row per
//     expert, kept in the workspace).
// The rows are the same as the one-workgroup kernel's (slot order within an
// expert, whatever the split).
#include "kernels.h"

namespace ace {

namespace {
constexpr int NW = 16;
constexpr int NTHR = NW * 64;
constexpr int EMAX = 256;
constexpr int POOL_SLOTS = 8192;  // slots (T*k) the pool variant keeps in LDS
// Launch modes of dispatch_kernel
constexpr int DSP_ONE = 0;       // one workgroup for the whole batch
constexpr int DSP_RECOUNT = 1;   // one workgroup per RBS slots; each counts the whole batch itself
constexpr int DSP_BLOCK = 2;     // one workgroup per DBS slots; counts and row bases from the workspace
constexpr int RBS = 64 * NW;     // slots per workgroup, recount mode (one 64-slot chunk per wave)
constexpr int RECOUNT_MAX = 32768;  // largest batch (slots) of the recount mode
constexpr int RC_BATCH = 2;      // slot quads in flight per thread while recounting
constexpr int DBS = 4096;        // slots per workgroup, block mode (64 chunks)

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct SlotVals {
  int e;
  int kept;
  float g;
};

// Slot s of chunk c for this lane (index clamped so the load is always in
// bounds; callers check s < nslots).
__device__ __forceinline__ SlotVals load_slot(const DispatchArgs& a, int64_t s, int64_t nslots, bool with_gate) {
  const int64_t sc = s < nslots ? s : nslots - 1;
  SlotVals v;
  v.e = a.idx[sc];
  v.kept = a.keep[sc];
  v.g = with_gate ? a.gate[sc] : 0.f;
  return v;
}
}  // namespace

// Exclusive scan of one int per thread over the workgroup (thread order);
// returns the exclusive prefix, total in *total.  Contains barriers: every
// thread of the workgroup must call it.
__device__ __forceinline__ int block_excl_scan(int v, int32_t* s_wsum, int* total) {
  const int w = wave_id(), l = lane_id();
  const int inc = wave_incl_scan(v);
  if (l == 63) s_wsum[w] = inc;
  __syncthreads();
  int base = 0, all = 0;
  for (int ww = 0; ww < NW; ++ww) {
    if (ww < w) base += s_wsum[ww];
    all += s_wsum[ww];
  }
  __syncthreads();
  *total = all;
  return base + inc - v;
}

template <bool POOL, int MODE>
__global__ __launch_bounds__(NTHR) void dispatch_kernel(DispatchArgs a) {
  __shared__ uint32_t s_bits[NW][EMAX][2];
  __shared__ int32_t s_run[NW][EMAX];
  __shared__ int32_t s_off[EMAX + 1];
  __shared__ int32_t s_wsum[NTHR / 64];
  // pool variant only
  __shared__ int32_t s_pos[POOL ? POOL_SLOTS : 1];  // (row << 8) | expert, or -1
  __shared__ float s_sg[POOL ? POOL_SLOTS : 1];     // gates by pre-cap row
  __shared__ float s_S[POOL ? EMAX : 1];
  __shared__ int32_t s_flag[POOL ? EMAX : 1];       // bit 0: top-1 expert; bit 1: retained
  __shared__ int32_t s_list[POOL ? EMAX : 1];
  __shared__ int32_t s_noff[POOL ? EMAX : 1];
  // recount mode only: kept slots per expert outside this block, and before it
  __shared__ int32_t s_tot[MODE == DSP_RECOUNT ? EMAX : 1];
  __shared__ int32_t s_pre[MODE == DSP_RECOUNT ? EMAX : 1];
  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int E = a.E, k = a.k;
  const int64_t nslots = int64_t(a.T) * k;
  const int nchunks = int((nslots + 63) / 64);
  // workgroup b owns chunks [b*BCH, (b+1)*BCH) (all of them in DSP_ONE)
  constexpr int BCH = MODE == DSP_RECOUNT ? RBS / 64 : DBS / 64;
  const int cb0 = MODE != DSP_ONE ? int(blockIdx.x) * BCH : 0;
  const int cb1 = MODE != DSP_ONE ? min(nchunks, cb0 + BCH) : nchunks;
  const int cpw = (cb1 - cb0 + NW - 1) / NW;
  const int c0 = cb0 + w * cpw, c1 = min(cb1, c0 + cpw);

  // 1. per-wave expert counts (and, with the pool, the top-1 experts)
  for (int e = l; e < E; e += 64) s_run[w][e] = 0;
  if (POOL && tid < EMAX) s_flag[tid] = 0;
  if (MODE == DSP_RECOUNT && tid < EMAX) {
    s_tot[tid] = 0;
    s_pre[tid] = 0;
  }
  __syncthreads();
  // recount mode: each wave owns one chunk of the block; its slots are loaded
  // once, before the recount, and serve steps 1 and 3
  SlotVals own{};
  if constexpr (MODE == DSP_RECOUNT) own = load_slot(a, int64_t(min(c0, nchunks - 1)) * 64 + l, nslots, true);
  if constexpr (MODE == DSP_RECOUNT) {
    // the slots outside this block: kept slots per expert, and those before
    // the block.  Counting ignores slot order, so each thread takes four
    // consecutive slots per load (16-byte and 4-byte loads: the ABI's
    // buffers are 16-byte aligned and block boundaries are multiples of 64
    // slots), RC_BATCH quads in flight; a quad that reaches past the end of
    // the batch is read slot by slot.
    auto count = [&](int64_t sb, int64_t se, bool before) {
      for (int64_t q0 = sb + 4 * int64_t(tid); q0 < se; q0 += int64_t(4) * NTHR * RC_BATCH) {
        int4 ev[RC_BATCH];
        uint32_t kv[RC_BATCH];
#pragma unroll
        for (int b = 0; b < RC_BATCH; ++b) {
          const int64_t q = q0 + int64_t(4) * NTHR * b;
          ev[b] = int4{0, 0, 0, 0};
          kv[b] = 0u;
          if (q + 4 <= nslots) {
            if (q < se) {
              ev[b] = *reinterpret_cast<const int4*>(a.idx + q);
              kv[b] = *reinterpret_cast<const uint32_t*>(a.keep + q);
            }
          } else if (q < se) {
            ev[b].x = a.idx[q];
            kv[b] = a.keep[q];
            if (q + 1 < nslots) { ev[b].y = a.idx[q + 1]; kv[b] |= uint32_t(a.keep[q + 1]) << 8; }
            if (q + 2 < nslots) { ev[b].z = a.idx[q + 2]; kv[b] |= uint32_t(a.keep[q + 2]) << 16; }
          }
        }
#pragma unroll
        for (int b = 0; b < RC_BATCH; ++b) {
          const int64_t q = q0 + int64_t(4) * NTHR * b;
          const int e4[4] = {ev[b].x, ev[b].y, ev[b].z, ev[b].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (q + j < se && ((kv[b] >> (8 * j)) & 0xFFu) && unsigned(e4[j]) < unsigned(E)) {
              atomicAdd(&s_tot[e4[j]], 1);
              if (before) atomicAdd(&s_pre[e4[j]], 1);
            }
          }
        }
      }
    };
    count(0, int64_t(cb0) * 64, true);
    count(int64_t(cb1) * 64, nslots, false);
  }
  if (c0 < c1) {
    SlotVals cur = MODE == DSP_RECOUNT ? own : load_slot(a, int64_t(c0) * 64 + l, nslots, false);
    for (int c = c0; c < c1; ++c) {
      const SlotVals nxt =
          MODE == DSP_RECOUNT ? cur : load_slot(a, int64_t(min(c + 1, c1 - 1)) * 64 + l, nslots, false);
      const int64_t s = int64_t(c) * 64 + l;
      if (s < nslots && unsigned(cur.e) < unsigned(E)) {
        if (cur.kept) atomicAdd(&s_run[w][cur.e], 1);
        if (POOL && s % k == 0) s_flag[cur.e] = 1;  // top-1 expert (kept or not)
      }
      cur = nxt;
    }
  }
  __syncthreads();

  // 2. expert totals and exclusive scan over experts (thread e < E owns expert e)
  int tot = 0;
  if (tid < E) {
    for (int ww = 0; ww < NW; ++ww) {
      const int v = s_run[ww][tid];
      s_run[ww][tid] = tot;  // exclusive prefix over waves, within the expert
      tot += v;
    }
  }
  if constexpr (MODE == DSP_BLOCK) {
    // this block's first row in each expert's segment (dispatch_scan_kernel)
    const int nblk = int((nslots + DBS - 1) / DBS);
    if (tid < E) s_off[tid] = a.ws[int64_t(nblk) * E + int64_t(blockIdx.x) * E + tid];
  } else if constexpr (MODE == DSP_RECOUNT) {
    // whole-batch totals -> offsets; this block starts after the slots before it
    int all = 0;
    const int excl = block_excl_scan(tot + (tid < E ? s_tot[tid] : 0), s_wsum, &all);
    if (tid < E) {
      s_off[tid] = excl + s_pre[tid];
      if (blockIdx.x == 0) a.offsets[tid] = excl;
    }
    if (tid == 0 && blockIdx.x == 0) a.offsets[E] = all;
  } else {
    int all = 0;
    const int excl = block_excl_scan(tot, s_wsum, &all);
    if (tid < E) {
      s_off[tid] = excl;
      if (!POOL) a.offsets[tid] = excl;
    }
    if (tid == 0) {
      s_off[E] = all;
      if (!POOL) a.offsets[E] = all;
    }
  }
  __syncthreads();
  for (int e = l; e < E; e += 64) s_run[w][e] += s_off[e];
  wave_sync_lds();

  // 3. rows, chunk by chunk in slot order
  if (c0 < c1) {
    const uint64_t below = (uint64_t(1) << l) - 1u;
    SlotVals cur = MODE == DSP_RECOUNT ? own : load_slot(a, int64_t(c0) * 64 + l, nslots, true);
    for (int c = c0; c < c1; ++c) {
      const SlotVals nxt =
          MODE == DSP_RECOUNT ? cur : load_slot(a, int64_t(min(c + 1, c1 - 1)) * 64 + l, nslots, true);
      const int64_t s = int64_t(c) * 64 + l;
      const bool live = s < nslots && cur.kept && unsigned(cur.e) < unsigned(E);
      for (int e = l; e < E; e += 64) {
        s_bits[w][e][0] = 0u;
        s_bits[w][e][1] = 0u;
      }
      wave_sync_lds();
      if (live) atomicOr(&s_bits[w][cur.e][l >> 5], 1u << (l & 31));
      wave_sync_lds();
      if (s < nslots) {
        if (live) {
          const uint64_t m = uint64_t(s_bits[w][cur.e][0]) | (uint64_t(s_bits[w][cur.e][1]) << 32);
          const int pos = s_run[w][cur.e] + __popcll(m & below);
          if (POOL) {
            s_pos[s] = (pos << 8) | cur.e;
            s_sg[pos] = cur.g;
          } else {
            a.sorted_token[pos] = int(s / k);
            a.sorted_gate[pos] = cur.g;
            a.slot_pos[s] = pos;
          }
        } else {
          if (POOL) s_pos[s] = -1;
          else a.slot_pos[s] = -1;
        }
      }
      wave_sync_lds();
      for (int e = l; e < E; e += 64) s_run[w][e] += __popc(s_bits[w][e][0]) + __popc(s_bits[w][e][1]);
      wave_sync_lds();
      cur = nxt;
    }
  }
  if constexpr (POOL) {
    __syncthreads();
    // 4. pool: scores, top-1 count, candidate ranks, retained experts
    const bool is_e = tid < E;
    const int n_e = is_e ? s_off[tid + 1] - s_off[tid] : 0;
    const bool top1 = is_e && (s_flag[tid] & 1);
    float S = 0.f;
    for (int p = 0; p < n_e; ++p) S += s_sg[s_off[tid] + p];
    if (is_e) s_S[tid] = S;
    const bool cand = is_e && n_e > 0 && !top1;
    int n_top1 = 0, n_cand = 0;
    const int ctop = block_excl_scan(top1 ? 1 : 0, s_wsum, &n_top1);
    (void)ctop;
    const int cpos = block_excl_scan(cand ? 1 : 0, s_wsum, &n_cand);
    if (cand) s_list[cpos] = tid;
    __syncthreads();
    const int budget = max(a.pool - n_top1, 0);
    bool keep_e = top1;
    if (cand && budget > 0) {
      int rank = 0;
      for (int j = 0; j < n_cand; ++j) {
        const int e2 = s_list[j];
        const float S2 = s_S[e2];
        rank += (S2 > S || (S2 == S && e2 < tid)) ? 1 : 0;
      }
      keep_e = rank < budget;
    }
    if (is_e) s_flag[tid] = keep_e ? 2 : 0;
    int kept_all = 0;
    const int nexcl = block_excl_scan(keep_e ? n_e : 0, s_wsum, &kept_all);
    if (is_e) {
      s_noff[tid] = nexcl;
      a.offsets[tid] = nexcl;
    }
    if (tid == 0) a.offsets[E] = kept_all;
    __syncthreads();
    // 5. final rows
    for (int64_t s = tid; s < nslots; s += NTHR) {
      const int v = s_pos[s];
      int out = -1;
      if (v >= 0) {
        const int e = v & 255, row = v >> 8;
        if (s_flag[e] & 2) {
          out = s_noff[e] + (row - s_off[e]);
          a.sorted_token[out] = int(s / k);
          a.sorted_gate[out] = s_sg[row];
        }
      }
      a.slot_pos[s] = out;
    }
  }
}

// Multi-workgroup path (large batches), kernel 1: kept slots per expert in
// each block of DBS slots -> ws[b][e] (order-independent integer totals).
__global__ __launch_bounds__(256) void dispatch_count_kernel(DispatchArgs a) {
  __shared__ int32_t s_c[EMAX];
  const int tid = threadIdx.x, E = a.E;
  const int64_t nslots = int64_t(a.T) * a.k;
  const int64_t s0 = int64_t(blockIdx.x) * DBS;
  for (int e = tid; e < EMAX; e += 256) s_c[e] = 0;
  __syncthreads();
  int ev[DBS / 256];
  bool kv[DBS / 256];
#pragma unroll
  for (int j = 0; j < DBS / 256; ++j) {
    const int64_t s = min(s0 + j * 256 + tid, nslots - 1);
    ev[j] = a.idx[s];
    kv[j] = a.keep[s] != 0 && s0 + j * 256 + tid < nslots;
  }
#pragma unroll
  for (int j = 0; j < DBS / 256; ++j)
    if (kv[j] && unsigned(ev[j]) < unsigned(E)) atomicAdd(&s_c[ev[j]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 256) a.ws[int64_t(blockIdx.x) * E + e] = s_c[e];
}

// Kernel 2 (one workgroup): expert totals -> expert_offsets (exclusive scan
// over experts); each block's first row per expert = offset + the counts of
// the earlier blocks -> ws[nblk + b][e].  Thread (g, e) owns expert e over
// the g-th contiguous run of blocks.
__global__ __launch_bounds__(NTHR) void dispatch_scan_kernel(DispatchArgs a, int nblk) {
  __shared__ int32_t s_wsum[NTHR / 64];
  __shared__ int32_t s_part[NTHR];
  const int tid = threadIdx.x, E = a.E;
  const int G = NTHR / E;
  const int g = tid / E, e = tid - g * E;
  const int bpg = (nblk + G - 1) / G;
  const int b0 = g * bpg, b1 = min(nblk, b0 + bpg);
  const int32_t* __restrict__ cnt = a.ws;
  int32_t* __restrict__ base = a.ws + int64_t(nblk) * E;
  int part = 0;
  if (g < G)
    for (int b = b0; b < b1; ++b) part += cnt[int64_t(b) * E + e];
  s_part[tid] = part;
  __syncthreads();
  int tot = 0;
  if (tid < E)
    for (int gg = 0; gg < G; ++gg) tot += s_part[gg * E + tid];
  int all = 0;
  const int excl = block_excl_scan(tot, s_wsum, &all);  // expert order (tid < E)
  if (tid < E) {
    a.offsets[tid] = excl;
    // exclusive prefix over groups, in place: s_part[gg*E + e] -> row base of group gg
    int run = excl;
    for (int gg = 0; gg < G; ++gg) {
      const int v = s_part[gg * E + tid];
      s_part[gg * E + tid] = run;
      run += v;
    }
  }
  __syncthreads();
  if (g < G) {
    int run = s_part[tid];
    for (int b = b0; b < b1; ++b) {
      base[int64_t(b) * E + e] = run;
      run += cnt[int64_t(b) * E + e];
    }
  }
  if (tid == 0) a.offsets[E] = all;
}

size_t dispatch_workspace_bytes(int T, int E, int k) {
  const int64_t nslots = int64_t(T) * k;
  if (nslots <= RECOUNT_MAX) return 256;
  const int64_t nblk = (nslots + DBS - 1) / DBS;
  return size_t((nblk * E * 2 * 4 + 255) / 256 * 256);
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  const int64_t nslots = int64_t(a.T) * a.k;
  if (a.pool > 0) {
    hipLaunchKernelGGL((dispatch_kernel<true, DSP_ONE>), dim3(1), dim3(NTHR), 0, s, a);
  } else if (nslots <= RBS) {
    hipLaunchKernelGGL((dispatch_kernel<false, DSP_ONE>), dim3(1), dim3(NTHR), 0, s, a);
  } else if (nslots <= RECOUNT_MAX) {
    hipLaunchKernelGGL((dispatch_kernel<false, DSP_RECOUNT>), dim3(int((nslots + RBS - 1) / RBS)), dim3(NTHR), 0,
                       s, a);
  } else {
    // large batches: per-block counts, one scan, per-block rows
    const int nblk = int((nslots + DBS - 1) / DBS);
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(nblk), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(NTHR), 0, s, a, nblk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dispatch_kernel<false, DSP_BLOCK>), dim3(nblk), dim3(NTHR), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ace
