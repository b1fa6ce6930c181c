// Streaming-read probe for the benchmark (libpa_readprobe.so, not part of the
// attention library): a plain read of a device buffer at full width, used to
// measure what the memory system delivers on this GPU for a buffer of a given
// size, the reference next to the decode kernels' achieved bandwidth.
//
// Workgroup w reads the w-th contiguous slice of the buffer (whole 4 KiB
// pages per slice, so each DRAM page is opened by one workgroup); its 256
// threads read consecutive 16-byte vectors, U independent loads in flight
// per thread per step, and fold what they read into one word so that no load
// can be removed.  The benchmark sweeps the grid size and U and keeps the
// fastest.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4 *buf, size_t n_vec,
                                                         size_t slice_vec, uint32_t *sink) {
  const size_t begin = (size_t)blockIdx.x * slice_vec;
  const size_t end = begin + slice_vec < n_vec ? begin + slice_vec : n_vec;
  uint32_t acc = 0;
  size_t i = begin + threadIdx.x;
  for (; i + (U - 1) * 256 < end; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += 256) {
    const u32x4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) at `buf` once with num_workgroups
// workgroups of 256 threads and `unroll` (4, 8 or 16) loads in flight per
// thread; sink (uint32 [4 * num_workgroups], device) receives one XOR of the
// words each wave read.  Enqueued on `stream`.  Returns 0, -1 for a NULL
// pointer, -2 for a bad size, grid or unroll, -6 when the launch fails.
extern "C" int pa_bench_read_probe(const void *buf, size_t bytes, uint32_t *sink,
                                   int num_workgroups, int unroll, void *stream) {
  if (!buf || !sink) return -1;
  if (bytes == 0 || bytes % 16 != 0 || num_workgroups <= 0) return -2;
  const size_t n_vec = bytes / 16;
  // slices of whole 4 KiB pages (256 vectors)
  size_t slice = (n_vec + num_workgroups - 1) / num_workgroups;
  slice = (slice + 255) / 256 * 256;
  const dim3 grid((unsigned)num_workgroups);
  const hipStream_t s = (hipStream_t)stream;
  switch (unroll) {
    case 4: hipLaunchKernelGGL(read_probe_kernel<4>, grid, dim3(256), 0, s, (const u32x4 *)buf,
                               n_vec, slice, sink); break;
    case 8: hipLaunchKernelGGL(read_probe_kernel<8>, grid, dim3(256), 0, s, (const u32x4 *)buf,
                               n_vec, slice, sink); break;
    case 16: hipLaunchKernelGGL(read_probe_kernel<16>, grid, dim3(256), 0, s, (const u32x4 *)buf,
                                n_vec, slice, sink); break;
    default: return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
