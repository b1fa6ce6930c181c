// C ABI of libpagedattn.so: argument checking, split planning and dispatch.
// The operations are documented in include/pagedattn.h.  Nothing here
// allocates, synchronises or reads device memory; all work goes on the
// caller's stream, in the order the calls are made.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>
#include <vector>

#include "pa_kernels.hpp"
#include "pagedattn.h"

static_assert(PA_MAX_QUERY_TOKENS == pa::kMaxQueryTokens, "query token limit");

namespace {

bool supported_head_dim(int d) { return d == 64 || d == 128; }
bool supported_block_size(int bs) { return bs == 16 || bs == 256; }
// fp8 pools: a per-tensor scale is a finite fp32 value > 0 whose reciprocal
// is finite too.
bool valid_kv_scale(float s) { return std::isfinite(s) && s > 0.f && std::isfinite(1.0f / s); }
int log2_exact(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

int check_heads(int num_q_heads, int num_kv_heads, int head_dim) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads > PA_MAX_HEADS) return PA_ERR_SHAPE;
  if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  const int g = num_q_heads / num_kv_heads;
  if (g < 1 || g > 8) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int check_pool(int64_t num_blocks, int block_size, int max_blocks_per_seq) {
  if (!supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  // token indices are kept in 32-bit registers on the device
  if ((int64_t)max_blocks_per_seq * block_size > (int64_t)1 << 30) return PA_ERR_SHAPE;
  return PA_OK;
}

// Tokens per piece for S pieces over a table of `max_tokens` tokens.
int split_len_for(int64_t max_tokens, int num_splits) {
  int64_t c = (max_tokens + num_splits - 1) / num_splits;
  c = (c + 63) / 64 * 64;
  if (c < 64) c = 64;
  return (int)c;
}

int num_pieces(int64_t max_tokens, int split_len) {
  return (int)((max_tokens + split_len - 1) / split_len);
}

// The planners' pieces are at least 128 tokens: measured at ctx 4096 batch 1,
// 32 pieces of 128 tokens make the step 2% faster than 64 pieces of 64 (the
// split kernel is slower, the merge of half the pieces faster).  An explicit
// piece count may still ask for 64-token pieces.
constexpr int kMinPlanSplitLen = 128;
int plan_split_len(int64_t max_tokens, int num_splits) {
  const int c = split_len_for(max_tokens, num_splits);
  return c < kMinPlanSplitLen ? kMinPlanSplitLen : c;
}

// Whether a launch of `units` (sequence, kv head) units in `pieces` pieces
// hands the upper half of its pieces out in mirrored unit order: exactly when
// its workgroups are more than the compute units and at most two per compute
// unit, so that the second round of slots exists and is filled in one go.
int mirrored_launch(int64_t units, int pieces, int num_cus) {
  const int64_t wgs = units * pieces;
  return pieces >= 2 && wgs > num_cus && wgs <= 2 * (int64_t)num_cus ? 1 : 0;
}

constexpr int kMaxDevices = 64;
std::once_flag g_cu_once[kMaxDevices];
int g_cu_count[kMaxDevices];

int cu_count(int device) {
  if (device < 0 || device >= kMaxDevices) return -1;
  std::call_once(g_cu_once[device], [device] {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
      v = -1;
    g_cu_count[device] = v;
  });
  return g_cu_count[device];
}

// Split partials of pa_decode_noalloc: a static device array, one copy per
// device (each device that loads the library holds its own until the process
// ends).  Host code never passes this name to a kernel: on the host it is only
// a stand-in for the symbol; the device address comes from
// hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_addr[kMaxDevices];

// Device address of `device`'s copy of the scratch, or NULL; `device` must be
// the current device.
void *scratch_address(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[device], [device] {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) ptr = nullptr;
    g_scratch_addr[device] = ptr;
  });
  return g_scratch_addr[device];
}

}  // namespace

extern "C" {

int pa_version(void) { return 101; }

const char *pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: sizes inconsistent or out of range";
    case PA_ERR_UNSUPPORTED:
      return "PA_ERR_UNSUPPORTED: head_dim must be 64 or 128, block_size 16 or 256, group 1..8";
    case PA_ERR_SPLITS: return "PA_ERR_SPLITS: num_splits outside [0, PA_MAX_SPLITS]";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: a HIP call or kernel launch failed";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: the KV pool cannot supply the blocks";
    case PA_ERR_STATE: return "PA_ERR_STATE: unknown or duplicate sequence, or forbidden change";
    case PA_ERR_SCRATCH:
      return "PA_ERR_SCRATCH: the split partials exceed PA_NOALLOC_SCRATCH_BYTES; use fewer "
             "splits or pa_decode with a workspace";
    default: return "unknown pagedattn status";
  }
}

namespace {

int append_rows(const void *k, const void *v, const int64_t *slot_mapping, void *k_cache,
                void *v_cache, int64_t num_tokens, int64_t num_blocks, int block_size,
                int num_kv_heads, int head_dim, bool fp8, float k_scale, float v_scale,
                void *stream) {
  if (!k_cache || !v_cache) return PA_ERR_NULL;
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PA_ERR_SHAPE;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size))
    return PA_ERR_UNSUPPORTED;
  if (fp8 && !(valid_kv_scale(k_scale) && valid_kv_scale(v_scale))) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping) return PA_ERR_NULL;
  pa::AppendArgs a;
  a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v;
  a.slot_mapping = slot_mapping;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_tokens = num_tokens;
  a.row_elems = num_kv_heads * head_dim;
  a.fp8 = fp8 ? 1 : 0;
  a.inv_k_scale = fp8 ? 1.0f / k_scale : 1.0f;
  a.inv_v_scale = fp8 ? 1.0f / v_scale : 1.0f;
  a.bs_shift = log2_exact(block_size);
  a.head_vecs = head_dim / 8;
  return pa::launch_append(a, head_dim, (hipStream_t)stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

int pa_reshape_and_cache(const void *k, const void *v, const int64_t *slot_mapping, void *k_cache,
                         void *v_cache, int64_t num_tokens, int64_t num_blocks, int block_size,
                         int num_kv_heads, int head_dim, void *stream) {
  return append_rows(k, v, slot_mapping, k_cache, v_cache, num_tokens, num_blocks, block_size,
                     num_kv_heads, head_dim, false, 1.0f, 1.0f, stream);
}

int pa_reshape_and_cache_fp8(const void *k, const void *v, const int64_t *slot_mapping,
                             void *k_cache, void *v_cache, float k_scale, float v_scale,
                             int64_t num_tokens, int64_t num_blocks, int block_size,
                             int num_kv_heads, int head_dim, void *stream) {
  return append_rows(k, v, slot_mapping, k_cache, v_cache, num_tokens, num_blocks, block_size,
                     num_kv_heads, head_dim, true, k_scale, v_scale, stream);
}

size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int head_dim, int num_splits) {
  return pa_decode_multi_workspace_size(num_seqs, 1, num_q_heads, head_dim, num_splits);
}

size_t pa_decode_multi_workspace_size(int num_seqs, int q_len, int num_q_heads, int head_dim,
                                      int num_splits) {
  if (num_seqs <= 0 || q_len <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  if (num_splits <= 1 || num_splits > PA_MAX_SPLITS) return 0;
  const size_t rows = (size_t)num_seqs * q_len * num_q_heads * num_splits;
  const size_t o_bytes = (rows * head_dim * sizeof(float) + 255) / 256 * 256;
  return o_bytes + (rows * sizeof(float) + 255) / 256 * 256;
}

int pa_decode_plan_splits(int num_seqs, int num_kv_heads, int max_blocks_per_seq, int block_size,
                          int num_cus) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || num_cus <= 0) return PA_ERR_SHAPE;
  const int st = check_pool(1, block_size, max_blocks_per_seq);
  if (st != PA_OK) return st;
  const int64_t max_tokens = (int64_t)max_blocks_per_seq * block_size;
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  // Aim for about one workgroup per compute unit: measured on the
  // ctx-4096 batches, the 7B batch and the 64-sequence mixed decode, it beats
  // two per compute unit (fewer partials to merge, and no merge launch at
  // all once the (sequence, kv head) units alone fill the device).
  const int64_t target = (int64_t)num_cus;
  int64_t s = 1;
  if (units < target) s = (target + units - 1) / units;
  if (s > PA_MAX_SPLITS) s = PA_MAX_SPLITS;
  const int c = plan_split_len(max_tokens, (int)s);
  int n = num_pieces(max_tokens, c);
  if (n < 1) n = 1;
  if (n > PA_MAX_SPLITS) n = PA_MAX_SPLITS;
  return n;
}

int pa_decode_auto_splits(int num_seqs, int num_kv_heads, int max_blocks_per_seq, int block_size,
                          int device) {
  const int cus = cu_count(device);
  if (cus <= 0) return PA_ERR_HIP;
  return pa_decode_plan_splits(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, cus);
}

// The merge launch and its read of the partials cost about what a compute
// unit takes to read this many tokens of one kv head at the decode's rate
// (measured: ≈ 4 µs against ≈ 60 tokens per µs per compute unit).
constexpr int64_t kMergeTokens = 256;
// Largest compute-unit count the length-aware planner models (its per-unit
// table is one int64 per compute unit).
constexpr int kMaxPlanCus = 1 << 16;

int pa_decode_plan_splits_lengths(const int32_t *context_lens, int num_seqs, int num_kv_heads,
                                  int max_blocks_per_seq, int block_size, int num_cus) {
  const int base =
      pa_decode_plan_splits(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, num_cus);
  if (base < 0) return base;
  if (!context_lens) return PA_ERR_NULL;
  if (num_cus > kMaxPlanCus) return PA_ERR_SHAPE;
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  // several generations of workgroups: the shape-only plan
  if (units * base > 2 * (int64_t)num_cus) return base;
  const int64_t max_tokens = (int64_t)max_blocks_per_seq * block_size;
  auto len = [&](int64_t u) {
    const int64_t L = context_lens[u / num_kv_heads];
    return L < 0 ? (int64_t)0 : (L > max_tokens ? max_tokens : L);
  };
  // Predicted cost of n pieces: the most tokens of one kv head a compute unit
  // reads, plus the merge launch when there are pieces.  Workgroup id
  // s * units + x (piece s of unit x, or of the mirrored unit units - 1 - x
  // in the upper half of a mirrored launch) takes the compute unit
  // id mod num_cus: each round of dispatch gives every compute unit one
  // workgroup, in id order.
  // no exception crosses the C ABI: without memory for the table, the
  // shape-only plan
  std::vector<int64_t> load;
  try {
    load.resize(num_cus);
  } catch (const std::bad_alloc &) {
    return base;
  }
  auto cost = [&](int n) {
    const int h = split_len_for(max_tokens, n);
    const int mirror = mirrored_launch(units, n, num_cus);
    std::fill(load.begin(), load.end(), 0);
    for (int sp = 0; sp < n; ++sp)
      for (int64_t x = 0; x < units; ++x) {
        const int64_t u = (mirror && 2 * sp >= n) ? units - 1 - x : x;
        const int64_t t = std::min(std::max(len(u) - (int64_t)sp * h, (int64_t)0), (int64_t)h);
        load[(sp * units + x) % num_cus] += t;
      }
    return *std::max_element(load.begin(), load.end()) + (n > 1 ? kMergeTokens : 0);
  };
  // every piece count whose workgroups fit one generation of two per compute
  // unit; the shape-only plan unless another is predicted cheaper
  int best = base;
  int64_t best_cost = cost(base);
  int last = 0;
  for (int S = 1; S <= PA_MAX_SPLITS; ++S) {
    const int n = num_pieces(max_tokens, plan_split_len(max_tokens, S));  // non-decreasing in S
    if (n == last) continue;
    last = n;
    if (units * n > 2 * (int64_t)num_cus) break;
    if (n == base) continue;
    const int64_t c = cost(n);
    if (c < best_cost) {
      best = n;
      best_cost = c;
    }
  }
  return best;
}

int pa_decode_auto_splits_lengths(const int32_t *context_lens, int num_seqs, int num_kv_heads,
                                  int max_blocks_per_seq, int block_size, int device) {
  const int cus = cu_count(device);
  if (cus <= 0) return PA_ERR_HIP;
  return pa_decode_plan_splits_lengths(context_lens, num_seqs, num_kv_heads, max_blocks_per_seq,
                                       block_size, cus);
}

namespace {

// Shared argument resolution of the decode entry points.  Fills `a` except the
// output pointers; returns a status.
int resolve_decode(const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *block_tables, const int32_t *context_lens, float scale,
                   int num_splits, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                   int block_size, int64_t num_blocks, int max_blocks_per_seq, pa::DecodeArgs *a) {
  if (num_seqs < 0 || num_seqs > PA_MAX_SEQS) return PA_ERR_SHAPE;
  int st = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (st != PA_OK) return st;
  st = check_pool(num_blocks, block_size, max_blocks_per_seq);
  if (st != PA_OK) return st;
  if (num_splits < 0 || num_splits > PA_MAX_SPLITS) return PA_ERR_SPLITS;
  if (!(std::isfinite(scale))) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (num_splits == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
    num_splits = pa_decode_auto_splits(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, dev);
    if (num_splits < 0) return num_splits;
  }
  const int64_t max_tokens = (int64_t)max_blocks_per_seq * block_size;
  const int split_len = split_len_for(max_tokens, num_splits);
  a->q = (const uint16_t *)q;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->new_k = nullptr;
  a->new_v = nullptr;
  a->out = nullptr;
  a->o_part = nullptr;
  a->lse_part = nullptr;
  a->scale_log2 = scale * 1.4426950408889634f;
  if (!std::isfinite(a->scale_log2)) return PA_ERR_SHAPE;
  a->num_q_heads = num_q_heads;
  a->num_kv_heads = num_kv_heads;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->bs_shift = log2_exact(block_size);
  a->split_len = split_len;
  a->num_splits = num_pieces(max_tokens, split_len);
  a->mirror_second = 0;   // set at launch (split_launch)
  a->q_len = 1;
  a->kv_fp8 = 0;
  a->v_scale = 1.0f;
  a->inv_k_scale = a->inv_v_scale = 1.0f;
  return PA_OK;
}

int attach_workspace(pa::DecodeArgs *a, int num_seqs, int head_dim, const void *workspace,
                     size_t workspace_bytes) {
  const size_t need = pa_decode_multi_workspace_size(num_seqs, a->q_len, a->num_q_heads, head_dim,
                                                     a->num_splits);
  if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
  const size_t rows = (size_t)num_seqs * a->q_len * a->num_q_heads * a->num_splits;
  const size_t o_bytes = (rows * head_dim * sizeof(float) + 255) / 256 * 256;
  a->o_part = (float *)workspace;
  a->lse_part = (float *)((char *)workspace + o_bytes);
  return PA_OK;
}

// The split pass, after every argument check.  When the workgroups are more
// than the compute units but fit two to a compute unit (one generation with
// a second round of slots), the upper half of the pieces goes out in mirrored
// unit order (see decode_split_kernel).
int split_launch(pa::DecodeArgs a, int head_dim, int group, int num_seqs, hipStream_t s) {
  if (a.num_splits >= 2) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
    const int cus = cu_count(dev);
    if (cus <= 0) return PA_ERR_HIP;
    a.mirror_second = mirrored_launch((int64_t)num_seqs * a.num_kv_heads, a.num_splits, cus);
  }
  return pa::launch_decode_split(a, head_dim, group, num_seqs, s) == hipSuccess ? PA_OK
                                                                                : PA_ERR_HIP;
}

int launch_split_and_merge(const pa::DecodeArgs &a, int head_dim, int group, int num_seqs,
                           hipStream_t s) {
  const int st = split_launch(a, head_dim, group, num_seqs, s);
  if (st != PA_OK) return st;
  if (a.num_splits > 1 && pa::launch_decode_combine(a, head_dim, num_seqs, s) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

}  // namespace

namespace {

// What distinguishes the decode entry points: query tokens per sequence, fp8
// pools with their scales, and the fused append of each sequence's new row.
struct DecodeVariant {
  int q_len = 1;
  bool fp8 = false;
  float k_scale = 1.0f, v_scale = 1.0f;
  bool append = false;
  const void *new_k = nullptr, *new_v = nullptr;
};

// The decode entry points' shared body: argument checks in a fixed order
// (query tokens, fp8 scales, shapes, rows per workgroup, pointers, the fp8
// score scale), then the split pass and, with more than one piece, the merge.
int decode_entry(const void *q, const void *k_cache, const void *v_cache,
                 const int32_t *block_tables, const int32_t *context_lens, float scale,
                 int num_splits, void *out, int num_seqs, int num_q_heads, int num_kv_heads,
                 int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
                 void *workspace, size_t workspace_bytes, void *stream, const DecodeVariant &v) {
  if (v.q_len < 1 || v.q_len > PA_MAX_QUERY_TOKENS) return PA_ERR_SHAPE;
  if (v.fp8 && !(valid_kv_scale(v.k_scale) && valid_kv_scale(v.v_scale))) return PA_ERR_SHAPE;
  pa::DecodeArgs a;
  int st = resolve_decode(q, k_cache, v_cache, block_tables, context_lens, scale, num_splits,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                          max_blocks_per_seq, &a);
  if (st != PA_OK) return st;
  if ((num_q_heads / num_kv_heads) * v.q_len > pa::kMaxDecodeRows) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!out || (v.append && (!v.new_k || !v.new_v))) return PA_ERR_NULL;
  if (v.fp8) {
    // scores are q . (code k_scale) scale: k_scale joins the score scale
    a.scale_log2 = (scale * v.k_scale) * 1.4426950408889634f;
    if (!std::isfinite(a.scale_log2)) return PA_ERR_SHAPE;
    a.kv_fp8 = 1;
    a.v_scale = v.v_scale;
    if (v.append) {
      a.inv_k_scale = 1.0f / v.k_scale;
      a.inv_v_scale = 1.0f / v.v_scale;
    }
  }
  a.q_len = v.q_len;
  a.out = (uint16_t *)out;
  if (v.append) {
    a.new_k = (const uint16_t *)v.new_k;
    a.new_v = (const uint16_t *)v.new_v;
  }
  if (a.num_splits > 1) {
    st = attach_workspace(&a, num_seqs, head_dim, workspace, workspace_bytes);
    if (st != PA_OK) return st;
  }
  return launch_split_and_merge(a, head_dim, num_q_heads / num_kv_heads, num_seqs,
                                (hipStream_t)stream);
}

}  // namespace

int pa_decode(const void *q, const void *k_cache, const void *v_cache,
              const int32_t *block_tables, const int32_t *context_lens, float scale,
              int num_splits, void *out, int num_seqs, int num_q_heads, int num_kv_heads,
              int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
              void *workspace, size_t workspace_bytes, void *stream) {
  return decode_entry(q, k_cache, v_cache, block_tables, context_lens, scale, num_splits, out,
                      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, workspace, workspace_bytes, stream, DecodeVariant{});
}

int pa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens, float scale,
                      int num_splits, void *out, int num_seqs, int num_q_heads,
                      int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                      int max_blocks_per_seq, void *stream) {
  // argument checks and the split count first: a refused call touches no device
  pa::DecodeArgs a;
  int st = resolve_decode(q, k_cache, v_cache, block_tables, context_lens, scale, num_splits,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                          max_blocks_per_seq, &a);
  if (st != PA_OK || num_seqs == 0) return st;
  if (!out) return PA_ERR_NULL;
  void *ws = nullptr;
  size_t ws_bytes = 0;
  if (a.num_splits > 1) {
    if (pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, a.num_splits) >
        PA_NOALLOC_SCRATCH_BYTES)
      return PA_ERR_SCRATCH;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
    ws = scratch_address(dev);
    if (ws == nullptr) return PA_ERR_HIP;
    ws_bytes = PA_NOALLOC_SCRATCH_BYTES;
  }
  return decode_entry(q, k_cache, v_cache, block_tables, context_lens, scale, num_splits, out,
                      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, ws, ws_bytes, stream, DecodeVariant{});
}

int pa_append_decode(const void *q, const void *new_k, const void *new_v, void *k_cache,
                     void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                     float scale, int num_splits, void *out, int num_seqs, int num_q_heads,
                     int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                     int max_blocks_per_seq, void *workspace, size_t workspace_bytes,
                     void *stream) {
  DecodeVariant v;
  v.append = true;
  v.new_k = new_k;
  v.new_v = new_v;
  return decode_entry(q, k_cache, v_cache, block_tables, context_lens, scale, num_splits, out,
                      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, workspace, workspace_bytes, stream, v);
}

int pa_decode_multi(const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, const int32_t *context_lens, float scale,
                    int num_splits, void *out, int num_seqs, int q_len, int num_q_heads,
                    int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                    int max_blocks_per_seq, void *workspace, size_t workspace_bytes,
                    void *stream) {
  DecodeVariant v;
  v.q_len = q_len;
  return decode_entry(q, k_cache, v_cache, block_tables, context_lens, scale, num_splits, out,
                      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, workspace, workspace_bytes, stream, v);
}

int pa_decode_fp8(const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *block_tables, const int32_t *context_lens, float scale,
                  float k_scale, float v_scale, int num_splits, void *out, int num_seqs,
                  int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                  int64_t num_blocks, int max_blocks_per_seq, void *workspace,
                  size_t workspace_bytes, void *stream) {
  DecodeVariant v;
  v.fp8 = true;
  v.k_scale = k_scale;
  v.v_scale = v_scale;
  return decode_entry(q, k_cache, v_cache, block_tables, context_lens, scale, num_splits, out,
                      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, workspace, workspace_bytes, stream, v);
}

int pa_append_decode_fp8(const void *q, const void *new_k, const void *new_v, void *k_cache,
                         void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                         float scale, float k_scale, float v_scale, int num_splits, void *out,
                         int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                         int block_size, int64_t num_blocks, int max_blocks_per_seq,
                         void *workspace, size_t workspace_bytes, void *stream) {
  DecodeVariant v;
  v.fp8 = true;
  v.k_scale = k_scale;
  v.v_scale = v_scale;
  v.append = true;
  v.new_k = new_k;
  v.new_v = new_v;
  return decode_entry(q, k_cache, v_cache, block_tables, context_lens, scale, num_splits, out,
                      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, workspace, workspace_bytes, stream, v);
}

int pa_decode_multi_fp8(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *block_tables, const int32_t *context_lens, float scale,
                        float k_scale, float v_scale, int num_splits, void *out, int num_seqs,
                        int q_len, int num_q_heads, int num_kv_heads, int head_dim,
                        int block_size, int64_t num_blocks, int max_blocks_per_seq,
                        void *workspace, size_t workspace_bytes, void *stream) {
  DecodeVariant v;
  v.q_len = q_len;
  v.fp8 = true;
  v.k_scale = k_scale;
  v.v_scale = v_scale;
  return decode_entry(q, k_cache, v_cache, block_tables, context_lens, scale, num_splits, out,
                      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, workspace, workspace_bytes, stream, v);
}

int pa_decode_partials(const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, const int32_t *context_lens, float scale,
                       int num_splits, int num_seqs, int num_q_heads, int num_kv_heads,
                       int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
                       void *workspace, size_t workspace_bytes, void *stream) {
  pa::DecodeArgs a;
  int st = resolve_decode(q, k_cache, v_cache, block_tables, context_lens, scale, num_splits,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                          max_blocks_per_seq, &a);
  if (st != PA_OK || num_seqs == 0) return st;
  if (a.num_splits < 2) return PA_ERR_SPLITS;
  st = attach_workspace(&a, num_seqs, head_dim, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  const int group = num_q_heads / num_kv_heads;
  return split_launch(a, head_dim, group, num_seqs, (hipStream_t)stream);
}

int pa_decode_merge(const void *workspace, size_t workspace_bytes, const int32_t *context_lens,
                    void *out, int num_splits, int num_seqs, int num_q_heads, int num_kv_heads,
                    int head_dim, int block_size, int max_blocks_per_seq, void *stream) {
  pa::DecodeArgs a;
  // q and the pools are not used by the merge; pass placeholders through the
  // shared resolution so both passes agree on split_len and the piece count.
  const void *ph = (const void *)1;
  int st = resolve_decode(ph, ph, ph, (const int32_t *)ph, context_lens, 1.f, num_splits,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, 1,
                          max_blocks_per_seq, &a);
  if (st != PA_OK || num_seqs == 0) return st;
  if (!out) return PA_ERR_NULL;
  if (a.num_splits < 2) return PA_ERR_SPLITS;
  st = attach_workspace(&a, num_seqs, head_dim, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  a.q = nullptr;
  a.k_cache = a.v_cache = nullptr;
  a.block_tables = nullptr;
  a.out = (uint16_t *)out;
  return pa::launch_decode_combine(a, head_dim, num_seqs, (hipStream_t)stream) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

size_t pa_prefill_workspace_size(int num_seqs, int max_q_len, int num_q_heads, int head_dim,
                                 int num_splits) {
  if (num_seqs <= 0 || max_q_len <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  if (num_splits <= 1 || num_splits > PA_MAX_SPLITS) return 0;
  const size_t rows = (size_t)num_seqs * max_q_len * num_q_heads * num_splits;
  const size_t o_bytes = (rows * head_dim * sizeof(uint16_t) + 255) / 256 * 256;  // bf16 rows
  return o_bytes + (rows * sizeof(float) + 255) / 256 * 256;
}

int pa_prefill_plan_splits(int num_seqs, int max_q_len, int num_kv_heads, int max_blocks_per_seq,
                           int block_size, int num_cus) {
  if (num_seqs <= 0 || max_q_len <= 0 || num_kv_heads <= 0 || num_cus <= 0) return PA_ERR_SHAPE;
  const int st = check_pool(1, block_size, max_blocks_per_seq);
  if (st != PA_OK) return st;
  const int64_t max_tokens = (int64_t)max_blocks_per_seq * block_size;
  // One workgroup per 32 query positions and kv head; split the key range
  // until there is about one workgroup per compute unit.
  const int64_t units = (int64_t)num_seqs * num_kv_heads * ((max_q_len + 31) / 32);
  int64_t s = 1;
  if (units < num_cus) s = (num_cus + units - 1) / units;
  if (s > PA_MAX_SPLITS) s = PA_MAX_SPLITS;
  int n = num_pieces(max_tokens, split_len_for(max_tokens, (int)s));
  return n < 1 ? 1 : (n > PA_MAX_SPLITS ? PA_MAX_SPLITS : n);
}

namespace {

int prefill_impl(const void *q, const int32_t *cu_seqlens_q, const void *k_cache,
                 const void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                 float scale, bool fp8, float k_scale, float v_scale, int num_splits, void *out,
                 int num_seqs, int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                 int block_size, int64_t num_blocks, int max_blocks_per_seq, void *workspace,
                 size_t workspace_bytes, void *stream) {
  if (num_seqs < 0 || max_q_len < 0 || num_seqs > PA_MAX_SEQS) return PA_ERR_SHAPE;
  if (fp8 && !(valid_kv_scale(k_scale) && valid_kv_scale(v_scale))) return PA_ERR_SHAPE;
  int st = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (st != PA_OK) return st;
  st = check_pool(num_blocks, block_size, max_blocks_per_seq);
  if (st != PA_OK) return st;
  if (num_splits < 0 || num_splits > PA_MAX_SPLITS) return PA_ERR_SPLITS;
  if (!(std::isfinite(scale))) return PA_ERR_SHAPE;
  if (num_seqs == 0 || max_q_len == 0) return PA_OK;
  if (!q || !cu_seqlens_q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PA_ERR_NULL;
  if (num_splits == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
    const int cus = cu_count(dev);
    if (cus <= 0) return PA_ERR_HIP;
    num_splits = pa_prefill_plan_splits(num_seqs, max_q_len, num_kv_heads, max_blocks_per_seq,
                                        block_size, cus);
    if (num_splits < 0) return num_splits;
  }
  const int64_t max_tokens = (int64_t)max_blocks_per_seq * block_size;
  pa::PrefillArgs a;
  a.q = (const uint16_t *)q;
  a.cu_seqlens_q = cu_seqlens_q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = (uint16_t *)out;
  a.o_part = nullptr;
  a.lse_part = nullptr;
  // fp8 pools: scores are q . (code k_scale) scale
  a.scale_log2 = (fp8 ? scale * k_scale : scale) * 1.4426950408889634f;
  if (!std::isfinite(a.scale_log2)) return PA_ERR_SHAPE;
  a.kv_fp8 = fp8 ? 1 : 0;
  a.v_scale = fp8 ? v_scale : 1.0f;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.bs_shift = log2_exact(block_size);
  a.max_q_len = max_q_len;
  a.split_len = split_len_for(max_tokens, num_splits);
  a.num_splits = num_pieces(max_tokens, a.split_len);
  // launch grid: (kv head, piece) workgroups in y; query rows counted in int
  if ((int64_t)num_kv_heads * a.num_splits > 65535) return PA_ERR_SHAPE;
  if ((int64_t)num_seqs * max_q_len * num_q_heads > INT32_MAX) return PA_ERR_SHAPE;
  if (a.num_splits > 1) {
    const size_t need = pa_prefill_workspace_size(num_seqs, max_q_len, num_q_heads, head_dim,
                                                  a.num_splits);
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    const size_t rows = (size_t)num_seqs * max_q_len * num_q_heads * a.num_splits;
    a.o_part = (uint16_t *)workspace;
    a.lse_part = (float *)((char *)workspace + (rows * head_dim * sizeof(uint16_t) + 255) / 256 * 256);
  }
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = pa::launch_prefill(a, head_dim, num_q_heads / num_kv_heads, s);
  if (e == hipErrorInvalidValue) return PA_ERR_UNSUPPORTED;
  if (e != hipSuccess) return PA_ERR_HIP;
  if (a.num_splits > 1 &&
      pa::launch_prefill_merge(a, head_dim, s) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

}  // namespace

int pa_prefill(const void *q, const int32_t *cu_seqlens_q, const void *k_cache,
               const void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
               float scale, int num_splits, void *out, int num_seqs, int max_q_len,
               int num_q_heads, int num_kv_heads, int head_dim, int block_size,
               int64_t num_blocks, int max_blocks_per_seq, void *workspace,
               size_t workspace_bytes, void *stream) {
  return prefill_impl(q, cu_seqlens_q, k_cache, v_cache, block_tables, context_lens, scale, false,
                      1.0f, 1.0f, num_splits, out, num_seqs, max_q_len, num_q_heads, num_kv_heads,
                      head_dim, block_size, num_blocks, max_blocks_per_seq, workspace,
                      workspace_bytes, stream);
}

int pa_prefill_fp8(const void *q, const int32_t *cu_seqlens_q, const void *k_cache,
                   const void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                   float scale, float k_scale, float v_scale, int num_splits, void *out,
                   int num_seqs, int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                   int block_size, int64_t num_blocks, int max_blocks_per_seq, void *workspace,
                   size_t workspace_bytes, void *stream) {
  return prefill_impl(q, cu_seqlens_q, k_cache, v_cache, block_tables, context_lens, scale, true,
                      k_scale, v_scale, num_splits, out, num_seqs, max_q_len, num_q_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                      workspace, workspace_bytes, stream);
}

}  // extern "C"
