// Streaming-read probe: a plain read of a device buffer at full width, used
// by the benchmark to measure the read rate the memory system delivers on
// this GPU at a given size (the reference point for the decode kernels'
// achieved bandwidth).  Not part of the attention path.
#include "pagedattn_probe.h"

#include <hip/hip_runtime.h>

namespace {

// Each thread walks the buffer in 16-byte vectors, four loads in flight per
// iteration, and folds what it read into one word; the waves' words go to
// `sink` so that no load can be removed.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4 *buf, size_t n_vec,
                                                         uint32_t *sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n_vec; i += 4 * stride) {
    const uint4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^
           d.w;
  }
  for (; i < n_vec; i += stride) {
    const uint4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

}  // namespace

extern "C" int pa_read_probe(const void *buf, size_t bytes, uint32_t *sink, int num_workgroups,
                             void *stream) {
  if (!buf || !sink) return -1;
  if (bytes == 0 || bytes % 16 != 0 || num_workgroups <= 0) return -2;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)num_workgroups), dim3(256), 0,
                     (hipStream_t)stream, (const uint4 *)buf, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
