// Streaming-read probe: reads a device buffer once with 16-byte loads spread
// over every compute unit and folds the words into one value per workgroup
// (so no load can be dropped).  It measures the HBM read ceiling that the
// weight-streaming expert kernels are held against; it is a measuring aid,
// not a step of the layer.
#include "kernels.h"

namespace ace {

namespace {
constexpr int PROBE_THREADS = 256;
constexpr int PROBE_UNROLL = 8;  // independent 16-byte loads in flight per thread

__global__ __launch_bounds__(PROBE_THREADS) void read_probe_kernel(const uint4* __restrict__ src, int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = int64_t(gridDim.x) * PROBE_THREADS;
  int64_t i = int64_t(blockIdx.x) * PROBE_THREADS + threadIdx.x;
  uint32_t acc = 0;
  // full rounds: PROBE_UNROLL loads per thread, each `stride` words apart
  for (; i + (PROBE_UNROLL - 1) * stride < n16; i += PROBE_UNROLL * stride) {
    uint4 v[PROBE_UNROLL];
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // fold the wave, then the workgroup, into one word
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  __shared__ uint32_t part[PROBE_THREADS / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < PROBE_THREADS / 64; ++w) r ^= part[w];
    sink[blockIdx.x] = r;
  }
}

// Cache-resident load probe.  Every wave runs `rounds` rounds of LD loads of
// 1 KB (lane l: the 16 bytes at 16 l of a block) from a buffer that stays in
// L2; each block is the B operand of R bf16 MFMAs into R independent
// accumulators, and the next round's blocks are requested before this
// round's MFMAs.  Block j of a round sits at the next consecutive 1 KB
// (stride mode 0) or at (j % 3) * 512 KB + (j / 3) * 64 KB past the round's
// base (stride mode 1: the spacing of a router k-step's plane fragments).
// Each wave writes one fold of what it read and computed to sink.
template <int LD, int R>
__global__ __launch_bounds__(PROBE_THREADS) void l2_probe_kernel(const uint8_t* __restrict__ buf, uint32_t bytes,
                                                                 int rounds, int smode, uint32_t* __restrict__ sink) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(buf, bytes);
  const int l = lane_id();
  const uint32_t mask = bytes - 1024;  // block bases stay below bytes - 1 KB
  auto block = [&](uint32_t round, int j) -> int {
    return smode ? int(((round * 1024u) & 65535u) + uint32_t(j % 3) * 524288u + uint32_t(j / 3) * 65536u)
                 : int((round * LD * 1024u + uint32_t(j) * 1024u) & mask);
  };
  const u32x4 a = {uint32_t(l), 1u, 2u, 3u};
  f32x4 acc[R > 0 ? R : 1];
#pragma unroll
  for (int i = 0; i < (R > 0 ? R : 1); ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 cur[LD], nxt[LD];
#pragma unroll
  for (int j = 0; j < LD; ++j) cur[j] = buf_ld16(r, l * 16, block(0u, j));
  uint32_t x = 0;
  for (int it = 0; it < rounds; ++it) {
#pragma unroll
    for (int j = 0; j < LD; ++j) {
#pragma unroll
      for (int i = 0; i < R; ++i) acc[i] = mfma_bf16(a, cur[j], acc[i]);
      if (R == 0) x ^= cur[j][0] ^ cur[j][1] ^ cur[j][2] ^ cur[j][3];
      nxt[j] = buf_ld16(r, l * 16, block(uint32_t(it + 1), j));
    }
#pragma unroll
    for (int j = 0; j < LD; ++j) cur[j] = nxt[j];
  }
#pragma unroll
  for (int i = 0; i < (R > 0 ? R : 1); ++i) x ^= __float_as_uint(acc[i][0]) ^ __float_as_uint(acc[i][3]);
  x ^= cur[0][0];
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if (l == 0) sink[int64_t(blockIdx.x) * (PROBE_THREADS / 64) + wave_id()] = x;
}
}  // namespace

hipError_t launch_l2_probe(const void* buf, size_t bytes, int rounds, int loads, int mfma_per_load, int stride_mode,
                           uint32_t* sink, int workgroups, hipStream_t s) {
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  const dim3 grid(workgroups), block(PROBE_THREADS);
  const uint32_t n = uint32_t(bytes);
#define ACE_L2P(LDV, RV)                                                                          \
  if (loads == LDV && mfma_per_load == RV) {                                                     \
    hipLaunchKernelGGL((l2_probe_kernel<LDV, RV>), grid, block, 0, s, b, n, rounds, stride_mode, sink); \
    return hipGetLastError();                                                                     \
  }
  ACE_L2P(6, 0) ACE_L2P(6, 4) ACE_L2P(6, 8) ACE_L2P(8, 0) ACE_L2P(8, 4) ACE_L2P(8, 8)
#undef ACE_L2P
  return hipErrorInvalidValue;
}

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t s) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(workgroups), dim3(PROBE_THREADS), 0, s,
                     static_cast<const uint4*>(src), int64_t(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace ace
