// Kernel argument blocks and host-side launchers shared by the C ABI
// (pa_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct AppendArgs {
  const uint16_t *k, *v;
  const int64_t *slot_mapping;
  void *k_cache, *v_cache;    // bf16 pools, or fp8 (e4m3) pools when fp8 is set
  int64_t num_tokens;
  int row_elems;              // num_kv_heads * head_dim
  int fp8;                    // fp8 pools, [NB, Hkv, bs, D] (bf16 pools: [NB, bs, Hkv, D])
  float inv_k_scale, inv_v_scale;  // fp8: 1 / scale, rounded to fp32
  int bs_shift;               // fp8: log2(block_size)
  int head_vecs;              // fp8: head_dim / 8
};

struct DecodeArgs {
  const uint16_t *q;          // [B, q_len, Hq, D]
  const void *k_cache;        // [NB, bs, Hkv, D], bf16, or fp8 (e4m3) codes when kv_fp8
  const void *v_cache;
  const int32_t *block_tables;  // [B, W]
  const int32_t *context_lens;  // [B], including the q_len query tokens
  const uint16_t *new_k;      // bf16 [B, Hkv, D] rows appended at token L_b - 1, or null (q_len 1)
  const uint16_t *new_v;
  uint16_t *out;              // [B, q_len, Hq, D]        (num_splits == 1)
  float *o_part;              // [B, q_len, Hq, S, D]     (num_splits > 1)
  float *lse_part;            // [B, q_len, Hq, S], base-2 log-sum-exp of scaled scores
  float scale_log2;           // scale * log2(e) (times k_scale for fp8 pools)
  int num_q_heads, num_kv_heads, max_blocks_per_seq;
  int bs_shift;               // log2(block_size)
  int split_len;              // tokens per split, multiple of 64
  int num_splits;
  int mirror_second;          // upper half of the pieces takes the units in mirrored order
  int q_len;                  // query tokens per sequence (1 = single-token decode)
  int kv_fp8;                 // pools hold fp8 codes, head-major [NB, Hkv, bs, D]
  float v_scale;              // fp8 pools: value of V = code value * v_scale
  float inv_k_scale, inv_v_scale;  // fp8 pools, fused append: 1 / scale, rounded to fp32
};

struct PrefillArgs {
  const uint16_t *q;          // [Tq, Hq, D]
  const int32_t *cu_seqlens_q;  // [B + 1]
  const void *k_cache, *v_cache;  // bf16 [NB, bs, Hkv, D], or fp8 [NB, Hkv, bs, D] (kv_fp8)
  const int32_t *block_tables;
  const int32_t *context_lens;
  uint16_t *out;              // [Tq, Hq, D]
  uint16_t *o_part;           // bf16 [B, max_q_len, Hq, S, D] when the key range is split, else null
  float *lse_part;            // [B, max_q_len, Hq, S]
  float scale_log2;
  int num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq, bs_shift;
  int max_q_len;
  int split_len;              // keys per piece, multiple of 64
  int num_splits;
  int kv_fp8;                 // pools hold fp8 codes, head-major [NB, Hkv, bs, D]
  float v_scale;              // fp8 pools: value of V = code value * v_scale
};

hipError_t launch_append(const AppendArgs &a, int head_dim, hipStream_t stream);
// Returns hipErrorInvalidValue for an unsupported (head_dim, group, q_len):
// group * q_len must not exceed kMaxDecodeRows.
constexpr int kMaxDecodeRows = 32;
constexpr int kMaxQueryTokens = 8;
hipError_t launch_decode_split(const DecodeArgs &a, int head_dim, int group, int num_seqs,
                               hipStream_t stream);
hipError_t launch_decode_combine(const DecodeArgs &a, int head_dim, int num_seqs,
                                 hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs &a, int head_dim, int group, hipStream_t stream);
hipError_t launch_prefill_merge(const PrefillArgs &a, int head_dim, hipStream_t stream);

}  // namespace pa
