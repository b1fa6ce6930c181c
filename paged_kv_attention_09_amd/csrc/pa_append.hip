// Slot-mapped KV append (reshape_and_cache) for gfx950.
//
// Token i's new K row (num_kv_heads * head_dim bf16) is copied to row
// slot_mapping[i] of the pool viewed as [num_blocks * block_size,
// num_kv_heads * head_dim]; a negative slot is padding and writes nothing.
// Source: "direct physical tensor gather with zero-overhead slot mapping",
// mini-infer docs (prajwal7-2002.github.io/mini-infer), "Core Capabilities at
// a Glance" table, row "Batched Paged Decode (v0.2.1)".
//
// A pure copy: each lane moves one 16-byte vector of K and the same vector
// of V, so a wave covers 1 KiB of a row and rows stay coalesced.  fp8 pools
// take the quantising variant below.
#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

namespace {

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a, int vec_per_row) {
  const int64_t total = a.num_tokens * vec_per_row;
  const uint4 *k = (const uint4 *)a.k;
  const uint4 *v = (const uint4 *)a.v;
  uint4 *kc = (uint4 *)a.k_cache;
  uint4 *vc = (uint4 *)a.v_cache;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = idx / vec_per_row;
    const int64_t e = idx - i * vec_per_row;
    const int64_t s = a.slot_mapping[i];
    if (s < 0) continue;
    const int64_t dst = s * vec_per_row + e;
    kc[dst] = k[idx];
    vc[dst] = v[idx];
  }
}

// fp8 pools ([NB, Hkv, bs, D], head-major): each lane reads 8 bf16 of K and
// of V (16 bytes each) and writes their 8 codes (quantize8: 8 bytes each) to
// the row of its kv head.

__global__ __launch_bounds__(256) void append_fp8_kernel(AppendArgs a, int vec_per_row) {
  const int64_t total = a.num_tokens * vec_per_row;
  const uint4 *k = (const uint4 *)a.k;
  const uint4 *v = (const uint4 *)a.v;
  uint2 *kc = (uint2 *)a.k_cache;
  uint2 *vc = (uint2 *)a.v_cache;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = idx / vec_per_row;
    const int64_t e = idx - i * vec_per_row;
    const int64_t s = a.slot_mapping[i];
    if (s < 0) continue;
    // head-major pool: row (block, head, offset), 8 codes per vector
    const int64_t h = e / a.head_vecs, ve = e - h * a.head_vecs;
    const int64_t nh = vec_per_row / a.head_vecs;
    const int64_t blk = s >> a.bs_shift, off = s & ((1 << a.bs_shift) - 1);
    const int64_t dst = (((blk * nh + h) << a.bs_shift) + off) * a.head_vecs + ve;
    kc[dst] = quantize8(k[idx], a.inv_k_scale);
    vc[dst] = quantize8(v[idx], a.inv_v_scale);
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, int head_dim, hipStream_t stream) {
  (void)head_dim;
  const int vec_per_row = a.row_elems / 8;
  const int64_t total = a.num_tokens * vec_per_row;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  if (a.fp8)
    hipLaunchKernelGGL(append_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a,
                       vec_per_row);
  else
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a,
                       vec_per_row);
  return hipGetLastError();
}

}  // namespace pa
