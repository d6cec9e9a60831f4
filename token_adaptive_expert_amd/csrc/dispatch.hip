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
#include "kernels.h"

namespace ace {

namespace {
constexpr int NW = 16;
constexpr int NTHR = NW * 64;
constexpr int EMAX = 256;

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

__global__ __launch_bounds__(NTHR) void dispatch_kernel(DispatchArgs a) {
  __shared__ uint32_t s_bits[NW][EMAX][2];
  __shared__ int32_t s_run[NW][EMAX];
  __shared__ int32_t s_off[EMAX + 1];
  __shared__ int32_t s_wsum[NTHR / 64];
  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int E = a.E, k = a.k;
  const int64_t nslots = int64_t(a.T) * k;
  const int nchunks = int((nslots + 63) / 64);
  const int cpw = (nchunks + NW - 1) / NW;
  const int c0 = w * cpw, c1 = min(nchunks, c0 + cpw);

  // 1. per-wave expert counts
  for (int e = l; e < E; e += 64) s_run[w][e] = 0;
  wave_sync_lds();
  if (c0 < c1) {
    SlotVals cur = load_slot(a, int64_t(c0) * 64 + l, nslots, false);
    for (int c = c0; c < c1; ++c) {
      const SlotVals nxt = load_slot(a, int64_t(min(c + 1, c1 - 1)) * 64 + l, nslots, false);
      const int64_t s = int64_t(c) * 64 + l;
      if (s < nslots && cur.kept && unsigned(cur.e) < unsigned(E)) atomicAdd(&s_run[w][cur.e], 1);
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
  int inc = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o, 64);
    if (l >= o) inc += v;
  }
  if (l == 63) s_wsum[w] = inc;
  __syncthreads();
  if (tid < E) {
    int base = 0;
    for (int ww = 0; ww < w; ++ww) base += s_wsum[ww];
    const int excl = base + inc - tot;
    s_off[tid] = excl;
    a.offsets[tid] = excl;
    if (tid == E - 1) a.offsets[E] = excl + tot;
  }
  __syncthreads();
  for (int e = l; e < E; e += 64) s_run[w][e] += s_off[e];
  wave_sync_lds();

  // 3. scatter, chunk by chunk in slot order
  if (c0 < c1) {
    const uint64_t below = (uint64_t(1) << l) - 1u;
    SlotVals cur = load_slot(a, int64_t(c0) * 64 + l, nslots, true);
    for (int c = c0; c < c1; ++c) {
      const SlotVals nxt = load_slot(a, int64_t(min(c + 1, c1 - 1)) * 64 + l, nslots, true);
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
          a.sorted_token[pos] = int(s / k);
          a.sorted_gate[pos] = cur.g;
          a.slot_pos[s] = pos;
        } else {
          a.slot_pos[s] = -1;
        }
      }
      wave_sync_lds();
      for (int e = l; e < E; e += 64) s_run[w][e] += __popc(s_bits[w][e][0]) + __popc(s_bits[w][e][1]);
      wave_sync_lds();
      cur = nxt;
    }
  }
}

size_t dispatch_workspace_bytes(int T, int E) {
  (void)T;
  (void)E;
  return 256;
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace ace
