// Expert dispatch: group the kept (token, slot) pairs by expert, in token
// order within each expert, with integer work only.
//
// The article page on ACE says only that surviving slots go through
// "optimized expert dispatch"; this grouping is the layout the expert GEMMs
// read.  One workgroup of 16 waves handles the whole batch in three phases:
//   1. each 64-token chunk builds, per expert, the 64-bit mask of its tokens
//      that kept that expert (LDS bitwise OR: order-independent) and counts it;
//   2. per expert, chunk counts are prefix-summed into segment bases, and
//      expert totals into expert_offsets;
//   3. each kept slot's row = base[chunk][e] + popcount of the mask bits of
//      lower tokens in its chunk.
// Every result is a function of the inputs alone, independent of timing.
#include "kernels.h"

namespace ace {

namespace {
constexpr int NW = 16;
constexpr int NTHR = NW * 64;
constexpr int EMAX = 256;
}  // namespace

__global__ __launch_bounds__(NTHR) void dispatch_kernel(DispatchArgs a) {
  __shared__ uint32_t s_bits[NW][EMAX][2];
  __shared__ int32_t s_tot[EMAX];
  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int T = a.T, E = a.E, k = a.k;
  const int nchunks = (T + 63) / 64;
  const int iters = (nchunks + NW - 1) / NW;

  // phase 1: per-chunk expert masks and counts
  for (int it = 0; it < iters; ++it) {
    const int c = it * NW + w;
    for (int e = l; e < E; e += 64) {
      s_bits[w][e][0] = 0u;
      s_bits[w][e][1] = 0u;
    }
    __syncthreads();
    if (c < nchunks) {
      const int t = c * 64 + l;
      if (t < T) {
        for (int i = 0; i < k; ++i) {
          const int64_t o = int64_t(t) * k + i;
          const int e = a.idx[o];
          if (a.keep[o] && unsigned(e) < unsigned(E)) atomicOr(&s_bits[w][e][l >> 5], 1u << (l & 31));
        }
      }
    }
    __syncthreads();
    if (c < nchunks) {
      for (int e = l; e < E; e += 64) {
        const uint64_t m = uint64_t(s_bits[w][e][0]) | (uint64_t(s_bits[w][e][1]) << 32);
        a.ws_mask[int64_t(c) * E + e] = m;
        a.ws_cnt[int64_t(c) * E + e] = __popcll(m);
      }
    }
    __syncthreads();
  }
  __threadfence();
  __syncthreads();

  // phase 2: expert totals, offsets, per-chunk segment bases
  if (tid < E) {
    int s = 0;
    for (int c = 0; c < nchunks; ++c) s += a.ws_cnt[int64_t(c) * E + tid];
    s_tot[tid] = s;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      const int v = s_tot[e];
      s_tot[e] = run;
      a.offsets[e] = run;
      run += v;
    }
    a.offsets[E] = run;
  }
  __syncthreads();
  if (tid < E) {
    int run = s_tot[tid];
    for (int c = 0; c < nchunks; ++c) {
      const int64_t o = int64_t(c) * E + tid;
      const int v = a.ws_cnt[o];
      a.ws_cnt[o] = run;
      run += v;
    }
  }
  __threadfence();
  __syncthreads();

  // phase 3: scatter
  for (int c = w; c < nchunks; c += NW) {
    const int t = c * 64 + l;
    if (t >= T) continue;
    const uint64_t below = (uint64_t(1) << l) - 1u;
    for (int i = 0; i < k; ++i) {
      const int64_t o = int64_t(t) * k + i;
      const int e = a.idx[o];
      if (a.keep[o] && unsigned(e) < unsigned(E)) {
        const int64_t ce = int64_t(c) * E + e;
        const int pos = a.ws_cnt[ce] + __popcll(a.ws_mask[ce] & below);
        a.sorted_token[pos] = t;
        a.sorted_gate[pos] = a.gate[o];
        a.slot_pos[o] = pos;
      } else {
        a.slot_pos[o] = -1;
      }
    }
  }
}

size_t dispatch_workspace_bytes(int T, int E) {
  const size_t nchunks = (size_t(T) + 63) / 64;
  const size_t cnt = nchunks * size_t(E) * sizeof(int32_t);
  const size_t cnt_aligned = (cnt + 255) & ~size_t(255);
  return cnt_aligned + nchunks * size_t(E) * sizeof(uint64_t);
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace ace
