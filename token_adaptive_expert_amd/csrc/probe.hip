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
}  // namespace

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t s) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(workgroups), dim3(PROBE_THREADS), 0, s,
                     static_cast<const uint4*>(src), int64_t(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace ace
