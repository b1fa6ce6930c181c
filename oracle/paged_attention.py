"""CPU oracle for paged-KV attention: plain, slow, fp64.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg do.  It shares no code with the HIP library.

What it computes, and where the pages state it:

* ``append`` - the slot-mapped write of new K/V rows into the block pool:
  "direct physical tensor gather with zero-overhead slot mapping", mini-infer
  docs (prajwal7-2002.github.io/mini-infer), "Core Capabilities at a Glance"
  table, row "Batched Paged Decode (v0.2.1)".  A slot is
  ``physical_block * block_size + offset``; a negative slot writes nothing.
* ``decode`` - one query token per sequence attending to every token the
  sequence holds in the paged cache, the unified ``[B, 1]`` paged forward pass
  of the same table row, with keys and values fetched through the per-request
  virtual-to-physical block table of the page's "Systems Architecture"
  figure (PagedAttention via block tables: psmarter/mini-infer summary on
  sourcepulse.org, "How It Works").  Attention is softmax(q K^T * scale) V;
  the pages name the mechanism but print no formula, so the oracle takes the
  plain definition.  Split-KV / flash decoding ("Triton split-K", feature 7 of
  the zingnex.cn mini-infer thread; "paged decode, split-KV" in the MiniInfer
  README's "Attention Backend" table) re-associates the same sum and is
  therefore not modelled here: the oracle is the unsplit definition.
* ``prefill`` - a chunk of a longer prompt attending causally to the cached
  prefix and to itself: "bounded 512-token chunks", mini-infer docs, "Core
  Capabilities at a Glance" table, row "Prompt Ingestion (v0.2.1)".  Query i
  of an n-token chunk of a sequence of total length L sits at position
  L - n + i and sees keys 0 .. L - n + i.
* ``decode_multi`` - several query tokens per sequence in one decode step,
  causal among themselves: the target model's parallel verification of a
  speculative draft ("Speculative Decoding: K-token draft proposals with
  parallel target verification", mini-infer docs, "Core Capabilities at a
  Glance" table, row "Generation Speed"; draft-model speculative decoding,
  zingnex.cn mini-infer thread, feature list item 5).  The draft tokens are
  already in the cache, so query token j of q_len sits at position
  L - q_len + j and sees keys 0 .. L - q_len + j; a position below 0 (a
  sequence shorter than its query window) sees no key and gives a zero row.

Readings taken where the pages are silent (listed with the rest in the design
notes): q head h reads kv head h // (Hq / Hkv); ``context_lens`` counts every
cached token including one appended this step; a sequence of length 0 gives a
zero output; scale is a float32 value widened to fp64.

Every parity claim rests on this file, so each function is pinned in
``tests/test_oracle.py`` against brute force, a library SDPA, closed forms and
invariants.  No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64.  bf16 is the top half of an IEEE float32,
    so shifting into the high 16 bits gives the exact float32, which widens to
    float64 exactly."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Grouped-query attention: consecutive groups of Hq / Hkv query heads share
    one kv head."""
    assert num_q_heads % num_kv_heads == 0
    return h // (num_q_heads // num_kv_heads)


def block_and_offset(t: int, block_size: int):
    """Logical token t of a sequence lives in its virtual block t // bs, at
    offset t % bs inside that block."""
    return t // block_size, t % block_size


def gather_sequence(cache: np.ndarray, table_row: np.ndarray, num_tokens: int) -> np.ndarray:
    """Logical [num_tokens, Hkv, D] view of one sequence, read through its block
    table.  ``cache`` is [num_blocks, bs, Hkv, D] (any dtype)."""
    bs = cache.shape[1]
    rows = []
    for t in range(num_tokens):
        j, off = block_and_offset(t, bs)
        rows.append(cache[int(table_row[j]), off])
    if not rows:
        return np.zeros((0,) + cache.shape[2:], dtype=cache.dtype)
    return np.stack(rows)


def attend(qvec: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * keys @ q) @ values for one query vector, in fp64.
    keys/values: [L, D]; returns [D] (zeros when L == 0)."""
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    s = float(scale) * (keys @ qvec)
    w = np.exp(s - s.max())
    return (w @ values) / w.sum()


def append(new_k: np.ndarray, new_v: np.ndarray, slot_mapping: np.ndarray,
           k_cache: np.ndarray, v_cache: np.ndarray):
    """Return copies of the pools with row i of new_k / new_v written to slot
    slot_mapping[i] (bit patterns copied as they are); negative slots skip."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    bs = kc.shape[1]
    for i, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0:
            continue
        kc[s // bs, s % bs] = new_k[i]
        vc[s // bs, s % bs] = new_v[i]
    return kc, vc


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
           context_lens: np.ndarray, scale) -> np.ndarray:
    """q: bf16 bits [B, Hq, D]; caches: bf16 bits [NB, bs, Hkv, D];
    block_tables int [B, W]; context_lens int [B]; returns fp64 [B, Hq, D]."""
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    sc = np.float64(np.float32(scale))
    qf = bf16_bits_to_f64(q)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        K = bf16_bits_to_f64(gather_sequence(k_cache, block_tables[b], L))
        V = bf16_bits_to_f64(gather_sequence(v_cache, block_tables[b], L))
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[b, h] = attend(qf[b, h], K[:, g, :], V[:, g, :], sc)
    return out


def decode_multi(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 block_tables: np.ndarray, context_lens: np.ndarray, scale) -> np.ndarray:
    """q: bf16 bits [B, q_len, Hq, D]; context_lens [B] count the q_len query
    tokens, whose K/V are already in the pool.  Returns fp64 [B, q_len, Hq, D]:
    query token j attends keys 0 .. context_lens[b] - q_len + j."""
    B, QL, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    sc = np.float64(np.float32(scale))
    qf = bf16_bits_to_f64(q)
    out = np.zeros((B, QL, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        K = bf16_bits_to_f64(gather_sequence(k_cache, block_tables[b], L))
        V = bf16_bits_to_f64(gather_sequence(v_cache, block_tables[b], L))
        for j in range(QL):
            p = L - QL + j                     # absolute position of query token j
            n_keys = p + 1 if p >= 0 else 0
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                out[b, j, h] = attend(qf[b, j, h], K[:n_keys, g, :], V[:n_keys, g, :], sc)
    return out


def prefill(q: np.ndarray, cu_seqlens_q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
            block_tables: np.ndarray, context_lens: np.ndarray, scale) -> np.ndarray:
    """q: bf16 bits [Tq, Hq, D] packed over sequences by cu_seqlens_q [B + 1];
    context_lens [B] are total lengths (cached prefix + chunk); the chunk's own
    K/V must already be in the pool.  Returns fp64 [Tq, Hq, D]."""
    Tq, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    sc = np.float64(np.float32(scale))
    qf = bf16_bits_to_f64(q)
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    for b in range(len(context_lens)):
        L = int(context_lens[b])
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        n = q1 - q0
        K = bf16_bits_to_f64(gather_sequence(k_cache, block_tables[b], L))
        V = bf16_bits_to_f64(gather_sequence(v_cache, block_tables[b], L))
        for i in range(n):
            p = L - n + i                      # absolute position of query i
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                out[q0 + i, h] = attend(qf[q0 + i, h], K[:p + 1, g, :], V[:p + 1, g, :], sc)
    return out
