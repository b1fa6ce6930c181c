// Host-side checks of the preconditions the attention calls leave to the
// caller (declared at the end of include/pagedattn.h).  Plain C++ over host
// copies of the integer inputs; no HIP call.
#include <cstdint>
#include <unordered_set>
#include <vector>

#include "pagedattn.h"

namespace {

bool power_of_two(int x) { return x > 0 && (x & (x - 1)) == 0; }

int fail(int kind, int64_t index, int64_t *bad_index) {
  if (bad_index) *bad_index = index;
  return kind;
}

}  // namespace

extern "C" int pa_check_tables(const int32_t *block_tables, const int32_t *context_lens,
                               int num_seqs, int max_blocks_per_seq, int block_size,
                               int64_t num_blocks, int fused_append, int64_t *bad_index) {
  if (bad_index) *bad_index = -1;
  if (num_seqs < 0 || max_blocks_per_seq < 1 || num_blocks < 1 || !power_of_two(block_size))
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_CHECK_OK;
  if (!block_tables || !context_lens) return PA_ERR_NULL;
  const int64_t capacity = (int64_t)max_blocks_per_seq * block_size;
  auto used_blocks = [&](int b) { return ((int64_t)context_lens[b] + block_size - 1) / block_size; };

  for (int b = 0; b < num_seqs; ++b) {
    const int64_t L = context_lens[b];
    if (L < 0 || L > capacity) return fail(PA_CHECK_LENGTH, b, bad_index);
    const int32_t *row = block_tables + (int64_t)b * max_blocks_per_seq;
    for (int64_t j = 0; j < used_blocks(b); ++j)
      if (row[j] < 0 || row[j] >= num_blocks) return fail(PA_CHECK_BLOCK_ID, b, bad_index);
  }
  if (!fused_append) return PA_CHECK_OK;

  // How often each block is read through the tables (saturating at 2).
  std::vector<uint8_t> refs((size_t)num_blocks, 0);
  for (int b = 0; b < num_seqs; ++b) {
    const int32_t *row = block_tables + (int64_t)b * max_blocks_per_seq;
    for (int64_t j = 0; j < used_blocks(b); ++j)
      if (refs[(size_t)row[j]] < 2) ++refs[(size_t)row[j]];
  }
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t L = context_lens[b];
    if (L == 0) continue;
    const int32_t blk = block_tables[(int64_t)b * max_blocks_per_seq + (L - 1) / block_size];
    if (refs[(size_t)blk] > 1) return fail(PA_CHECK_APPEND_SHARED, b, bad_index);
  }
  return PA_CHECK_OK;
}

extern "C" int pa_check_slots(const int64_t *slot_mapping, int64_t num_tokens, int64_t num_blocks,
                              int block_size, int64_t *bad_index) {
  if (bad_index) *bad_index = -1;
  if (num_tokens < 0 || num_blocks < 1 || !power_of_two(block_size)) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_CHECK_OK;
  if (!slot_mapping) return PA_ERR_NULL;
  const int64_t limit = num_blocks * block_size;
  std::unordered_set<int64_t> seen;
  seen.reserve((size_t)num_tokens);
  for (int64_t i = 0; i < num_tokens; ++i) {
    const int64_t s = slot_mapping[i];
    if (s < 0) continue;  // padding row
    if (s >= limit) return fail(PA_CHECK_SLOT_RANGE, i, bad_index);
    if (!seen.insert(s).second) return fail(PA_CHECK_SLOT_DUPLICATE, i, bad_index);
  }
  return PA_CHECK_OK;
}

extern "C" int pa_check_prefill(const int32_t *cu_seqlens_q, const int32_t *context_lens,
                                int num_seqs, int max_q_len, int64_t *bad_index) {
  if (bad_index) *bad_index = -1;
  if (num_seqs < 0 || max_q_len < 0) return PA_ERR_SHAPE;
  if (!cu_seqlens_q) return PA_ERR_NULL;
  if (cu_seqlens_q[0] != 0) return fail(PA_CHECK_QUERY_OFFSETS, 0, bad_index);
  if (num_seqs == 0) return PA_CHECK_OK;
  if (!context_lens) return PA_ERR_NULL;
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t n = (int64_t)cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    if (n < 0 || n > max_q_len || n > context_lens[b])
      return fail(PA_CHECK_QUERY_OFFSETS, b, bad_index);
  }
  return PA_CHECK_OK;
}
