// Host-side manager of the paged KV pool; the operations and their rules are
// documented in include/pa_block_manager.h.  Plain C++ on host memory.
#include "pa_block_manager.h"

#include <algorithm>
#include <cstdint>
#include <limits>
#include <list>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

namespace {

struct Block {
  int32_t ref = 0;
  // Shareable content: a content id (never reused; 0 = not shareable), the
  // content id of the block before it, and the block's token ids.
  uint64_t cid = 0;
  uint64_t parent_cid = 0;
  std::vector<int32_t> tokens;
  bool cached = false;  // released while shareable: in the LRU list
  std::list<int32_t>::iterator lru_it;
};

struct Seq {
  std::vector<int32_t> blocks;
  std::vector<int32_t> tokens;  // token ids (kept only with prefix sharing)
  int64_t len = 0;
  int priority = 0;
  uint64_t order = 0;     // admission counter
  size_t keyed = 0;       // leading blocks that are shareable
  uint64_t last_cid = 0;  // content id of block keyed - 1 (0 before the first)
  bool chain_ok = true;   // false once a block could not be made shareable
};

// FNV-1a over the parent content id and the token ids.
uint64_t key_hash(uint64_t parent, const int32_t *t, int n) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&h](uint64_t v, int bytes) {
    for (int i = 0; i < bytes; ++i) {
      h ^= (v >> (8 * i)) & 0xffu;
      h *= 1099511628211ull;
    }
  };
  mix(parent, 8);
  for (int i = 0; i < n; ++i) mix((uint32_t)t[i], 4);
  return h;
}

}  // namespace

struct pa_block_manager {
  int64_t num_blocks = 0;
  int bs = 0, max_blocks = 0;
  bool prefix = false;
  std::vector<Block> blocks;
  std::set<int32_t> free_set;       // smallest id first
  std::list<int32_t> lru;           // cached blocks, least recently released first
  std::unordered_multimap<uint64_t, int32_t> index;  // key hash -> shareable block
  std::unordered_map<int64_t, Seq> seqs;
  uint64_t next_cid = 1, next_order = 1;
  int64_t used = 0;

  int64_t available() const { return (int64_t)free_set.size() + (int64_t)lru.size(); }

  int32_t find(uint64_t parent, const int32_t *t) const {
    auto range = index.equal_range(key_hash(parent, t, bs));
    for (auto it = range.first; it != range.second; ++it) {
      const Block &b = blocks[it->second];
      if (b.parent_cid == parent && std::equal(b.tokens.begin(), b.tokens.end(), t))
        return it->second;
    }
    return -1;
  }

  void unkey(int32_t id) {
    Block &b = blocks[id];
    if (b.cid == 0) return;
    auto range = index.equal_range(key_hash(b.parent_cid, b.tokens.data(), bs));
    for (auto it = range.first; it != range.second; ++it) {
      if (it->second == id) {
        index.erase(it);
        break;
      }
    }
    b.cid = 0;
    b.parent_cid = 0;
    b.tokens.clear();
  }

  // One block for new tokens (precondition: available() > 0): the smallest
  // free id, else the cached block released longest ago.
  int32_t take() {
    int32_t id;
    if (!free_set.empty()) {
      id = *free_set.begin();
      free_set.erase(free_set.begin());
    } else {
      id = lru.front();
      lru.pop_front();
      blocks[id].cached = false;
      unkey(id);
    }
    blocks[id].ref = 1;
    ++used;
    return id;
  }

  // One more holder of a shareable block.
  void reuse(int32_t id) {
    Block &b = blocks[id];
    if (b.cached) {
      lru.erase(b.lru_it);
      b.cached = false;
      ++used;
    }
    ++b.ref;
  }

  // One holder fewer.
  void drop(int32_t id) {
    Block &b = blocks[id];
    if (--b.ref > 0) return;
    --used;
    if (b.cid != 0) {
      b.cached = true;
      b.lru_it = lru.insert(lru.end(), id);
    } else {
      free_set.insert(id);
    }
  }

  // The full blocks behind the sequence's end become shareable.
  void register_full(Seq &s) {
    if (!prefix) return;
    const size_t full = (size_t)(s.len / bs);
    while (s.keyed < full && s.chain_ok) {
      const int32_t id = s.blocks[s.keyed];
      Block &b = blocks[id];
      const int32_t *t = s.tokens.data() + s.keyed * (size_t)bs;
      if (b.cid == 0) {
        if (find(s.last_cid, t) >= 0) {  // the same content is already shareable elsewhere
          s.chain_ok = false;
          break;
        }
        b.cid = next_cid++;
        b.parent_cid = s.last_cid;
        b.tokens.assign(t, t + bs);
        index.emplace(key_hash(b.parent_cid, t, bs), id);
      }
      s.last_cid = b.cid;
      ++s.keyed;
    }
  }

  void release(std::unordered_map<int64_t, Seq>::iterator it) {
    register_full(it->second);
    for (int32_t id : it->second.blocks) drop(id);
    seqs.erase(it);
  }
};

extern "C" {

pa_block_manager *pa_bm_create(int64_t num_blocks, int block_size, int max_blocks_per_seq,
                               int prefix_cache) {
  if (num_blocks < 1 || num_blocks > std::numeric_limits<int32_t>::max() || block_size < 1 ||
      max_blocks_per_seq < 1)
    return nullptr;
  try {
    auto *bm = new pa_block_manager();
    bm->num_blocks = num_blocks;
    bm->bs = block_size;
    bm->max_blocks = max_blocks_per_seq;
    bm->prefix = prefix_cache != 0;
    bm->blocks.resize((size_t)num_blocks);
    for (int64_t i = 0; i < num_blocks; ++i) bm->free_set.insert(bm->free_set.end(), (int32_t)i);
    return bm;
  } catch (const std::bad_alloc &) {
    return nullptr;
  }
}

void pa_bm_destroy(pa_block_manager *bm) { delete bm; }

int pa_bm_admit(pa_block_manager *bm, int64_t seq_id, int priority, const int32_t *tokens,
                int64_t n, int64_t *num_cached, int64_t *slots_out) {
  if (!bm || !num_cached || !slots_out) return PA_ERR_NULL;
  if (n < 1) return PA_ERR_SHAPE;
  if (bm->prefix && !tokens) return PA_ERR_NULL;
  const int64_t nblk = (n + bm->bs - 1) / bm->bs;
  if (nblk > bm->max_blocks) return PA_ERR_SHAPE;
  if (bm->seqs.count(seq_id)) return PA_ERR_STATE;
  try {
    // Leading full blocks of the prompt that the cache holds (never the
    // block of the last prompt token).
    std::vector<int32_t> hits;
    int64_t cached_hits = 0;
    if (bm->prefix) {
      uint64_t parent = 0;
      const int64_t cacheable = (n - 1) / bm->bs;
      for (int64_t i = 0; i < cacheable; ++i) {
        const int32_t id = bm->find(parent, tokens + i * bm->bs);
        if (id < 0) break;
        hits.push_back(id);
        cached_hits += bm->blocks[id].cached ? 1 : 0;
        parent = bm->blocks[id].cid;
      }
    }
    const int64_t need = nblk - (int64_t)hits.size();
    if (need > bm->available() - cached_hits) return PA_ERR_NO_BLOCKS;
    Seq s;
    s.blocks.reserve((size_t)nblk);
    for (int32_t id : hits) {
      bm->reuse(id);
      s.blocks.push_back(id);
    }
    for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
    if (bm->prefix) s.tokens.assign(tokens, tokens + n);
    s.len = n;
    s.priority = priority;
    s.order = bm->next_order++;
    s.keyed = hits.size();
    s.last_cid = hits.empty() ? 0 : bm->blocks[hits.back()].cid;
    const int64_t c = (int64_t)hits.size() * bm->bs;
    for (int64_t t = c; t < n; ++t)
      slots_out[t - c] = (int64_t)s.blocks[(size_t)(t / bm->bs)] * bm->bs + t % bm->bs;
    *num_cached = c;
    bm->seqs.emplace(seq_id, std::move(s));
    return PA_OK;
  } catch (const std::bad_alloc &) {
    return PA_ERR_NO_BLOCKS;
  }
}

int pa_bm_append(pa_block_manager *bm, int64_t seq_id, const int32_t *tokens, int64_t n,
                 int64_t *slots_out) {
  if (!bm || !slots_out) return PA_ERR_NULL;
  if (n < 1) return PA_ERR_SHAPE;
  if (bm->prefix && !tokens) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_STATE;
  Seq &s = it->second;
  const int64_t new_len = s.len + n;
  const int64_t nblk = (new_len + bm->bs - 1) / bm->bs;
  if (nblk > bm->max_blocks) return PA_ERR_SHAPE;
  const int64_t need = nblk - (int64_t)s.blocks.size();
  if (need > bm->available()) return PA_ERR_NO_BLOCKS;
  try {
    if (bm->prefix) s.tokens.reserve((size_t)new_len);
    s.blocks.reserve((size_t)nblk);
    bm->register_full(s);
    for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
    if (bm->prefix) s.tokens.insert(s.tokens.end(), tokens, tokens + n);
    for (int64_t t = s.len; t < new_len; ++t)
      slots_out[t - s.len] = (int64_t)s.blocks[(size_t)(t / bm->bs)] * bm->bs + t % bm->bs;
    s.len = new_len;
    return PA_OK;
  } catch (const std::bad_alloc &) {
    return PA_ERR_NO_BLOCKS;
  }
}

int pa_bm_decode_step(pa_block_manager *bm, const int64_t *seq_ids, int n_seqs,
                      const int32_t *tokens, int64_t *slots_out) {
  if (!bm) return PA_ERR_NULL;
  if (n_seqs < 0) return PA_ERR_SHAPE;
  if (n_seqs == 0) return PA_OK;
  if (!seq_ids || !slots_out || (bm->prefix && !tokens)) return PA_ERR_NULL;
  try {
    // Validate the whole batch and count the new blocks before changing anything.
    std::vector<Seq *> ss((size_t)n_seqs);
    std::unordered_map<int64_t, int> seen;
    seen.reserve((size_t)n_seqs * 2);
    for (int i = 0; i < n_seqs; ++i) {
      auto it = bm->seqs.find(seq_ids[i]);
      if (it == bm->seqs.end() || !seen.emplace(seq_ids[i], i).second) return PA_ERR_STATE;
      ss[(size_t)i] = &it->second;
    }
    int64_t need = 0;
    for (Seq *s : ss) {
      if (s->len % bm->bs == 0) {
        if ((int64_t)s->blocks.size() + 1 > bm->max_blocks) return PA_ERR_SHAPE;
        ++need;
      }
    }
    if (need > bm->available()) return PA_ERR_NO_BLOCKS;
    for (int i = 0; i < n_seqs; ++i) {
      Seq &s = *ss[(size_t)i];
      bm->register_full(s);
      if (s.len % bm->bs == 0) s.blocks.push_back(bm->take());
      if (bm->prefix) s.tokens.push_back(tokens[i]);
      slots_out[i] = (int64_t)s.blocks.back() * bm->bs + s.len % bm->bs;
      ++s.len;
    }
    return PA_OK;
  } catch (const std::bad_alloc &) {
    return PA_ERR_NO_BLOCKS;
  }
}

int pa_bm_truncate(pa_block_manager *bm, int64_t seq_id, int64_t new_len) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_STATE;
  Seq &s = it->second;
  if (new_len < 1 || new_len > s.len) return PA_ERR_SHAPE;
  const int64_t keep = (new_len + bm->bs - 1) / bm->bs;
  const bool partial = new_len % bm->bs != 0;
  if (partial && bm->blocks[s.blocks[(size_t)(keep - 1)]].ref > 1) return PA_ERR_STATE;
  for (size_t i = (size_t)keep; i < s.blocks.size(); ++i) bm->drop(s.blocks[i]);
  s.blocks.resize((size_t)keep);
  if (partial) bm->unkey(s.blocks[(size_t)(keep - 1)]);  // its later slots will change
  if (bm->prefix) s.tokens.resize((size_t)new_len);
  s.len = new_len;
  s.keyed = std::min(s.keyed, (size_t)(new_len / bm->bs));
  s.last_cid = s.keyed ? bm->blocks[s.blocks[s.keyed - 1]].cid : 0;
  s.chain_ok = true;
  return PA_OK;
}

int pa_bm_release(pa_block_manager *bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_STATE;
  bm->release(it);
  return PA_OK;
}

int pa_bm_preempt(pa_block_manager *bm, int64_t *victim) {
  if (!bm || !victim) return PA_ERR_NULL;
  if (bm->seqs.empty()) return PA_ERR_STATE;
  auto pick = bm->seqs.begin();
  for (auto it = bm->seqs.begin(); it != bm->seqs.end(); ++it) {
    const Seq &a = it->second, &p = pick->second;
    if (a.priority < p.priority || (a.priority == p.priority && a.order > p.order)) pick = it;
  }
  *victim = pick->first;
  bm->release(pick);
  return PA_OK;
}

int pa_bm_block_tables(const pa_block_manager *bm, const int64_t *seq_ids, int n_seqs,
                       int32_t *tables_out, int32_t *lens_out) {
  if (!bm) return PA_ERR_NULL;
  if (n_seqs < 0) return PA_ERR_SHAPE;
  if (n_seqs == 0) return PA_OK;
  if (!seq_ids || !tables_out || !lens_out) return PA_ERR_NULL;
  for (int i = 0; i < n_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PA_ERR_STATE;
    if (it->second.len > std::numeric_limits<int32_t>::max()) return PA_ERR_SHAPE;
  }
  for (int i = 0; i < n_seqs; ++i) {
    const Seq &s = bm->seqs.find(seq_ids[i])->second;
    int32_t *row = tables_out + (size_t)i * bm->max_blocks;
    std::fill(row, row + bm->max_blocks, 0);
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    lens_out[i] = (int32_t)s.len;
  }
  return PA_OK;
}

int pa_bm_order_longest_first(const pa_block_manager *bm, const int64_t *seq_ids, int n_seqs,
                              int64_t *order_out) {
  if (!bm) return PA_ERR_NULL;
  if (n_seqs < 0) return PA_ERR_SHAPE;
  if (n_seqs == 0) return PA_OK;
  if (!seq_ids || !order_out) return PA_ERR_NULL;
  std::vector<std::pair<int64_t, int>> keyed((size_t)n_seqs);  // (length, position)
  for (int i = 0; i < n_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PA_ERR_STATE;
    keyed[(size_t)i] = {it->second.len, i};
  }
  std::stable_sort(keyed.begin(), keyed.end(),
                   [](const std::pair<int64_t, int> &x, const std::pair<int64_t, int> &y) {
                     return x.first > y.first;
                   });
  for (int i = 0; i < n_seqs; ++i) order_out[i] = seq_ids[keyed[(size_t)i].second];
  return PA_OK;
}

int pa_bm_stats(const pa_block_manager *bm, int64_t *free_blocks, int64_t *cached_blocks,
                int64_t *used_blocks, int64_t *running) {
  if (!bm) return PA_ERR_NULL;
  if (free_blocks) *free_blocks = (int64_t)bm->free_set.size();
  if (cached_blocks) *cached_blocks = (int64_t)bm->lru.size();
  if (used_blocks) *used_blocks = bm->used;
  if (running) *running = (int64_t)bm->seqs.size();
  return PA_OK;
}

}  // extern "C"
