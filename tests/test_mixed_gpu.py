"""GPU parity of the chunked-prefill mixed batch as one composed step.

The step serves a prompt chunk and active decodes together over one pool
(the mini-infer docs, "Core Capabilities at a Glance", row "Prompt
Ingestion": bounded 512-token chunks interleaved with active decodes; the
MiniInfer README's scheduler, which forms prefill, decode and mixed batches):

  1. slot-mapped append of the chunk's 512 K/V rows,
  2. chunked prefill of the 512 query rows over the 4096-token sequence,
  3. fused append + decode of the 64 decode sequences (one new row each),

all on one stream, in that order, over one 2048-block pool (28 q / 4 kv
heads, head_dim 128, block_size 256).  The same three calls are also
captured in a HIP graph and replayed, with the pools reset and the outputs
poisoned eagerly between replays.

Checked against the oracle: both pools bit for bit (every block, referenced
or not) against the oracle's append of all 576 rows; the prefill rows and the
decode rows elementwise within 1e-2 + 1e-2 |oracle|.  fp8 pools run the same
step through the quantising append, the fp8 prefill and the fused quantising
append + fp8 decode, against oracle/kv_fp8.py.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.kv_fp8 as O8
import paged_kv_attention_09_amd as pa
import workloads as W
from gpu_cases import DEV, assert_close, bf16_tensor, to_bits, to_f64

pytestmark = pytest.mark.gpu

K_SCALE, V_SCALE = 0.375, 0.25


def _compact_slots(pool: W.CompactPool, slots: np.ndarray, bs: int) -> np.ndarray:
    lut = {int(x): i for i, x in enumerate(pool.ids)}
    return np.array([lut[int(s) // bs] * bs + int(s) % bs for s in slots], np.int64)


def _full_pool(pool: W.CompactPool, k: np.ndarray, v: np.ndarray, fp8: bool):
    """Whole device pools: poison in every block the step does not reference,
    the given dense blocks at their physical ids."""
    shape = (pool.num_blocks,) + k.shape[1:]
    if fp8:
        kd = torch.full(shape, int(W.E4M3_NAN), dtype=torch.uint8, device=DEV)
        vd = torch.full(shape, int(W.E4M3_NAN), dtype=torch.uint8, device=DEV)
        src_k = torch.from_numpy(np.ascontiguousarray(k)).to(DEV)
        src_v = torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
    else:
        nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
        kd = torch.full(shape, nan, dtype=torch.bfloat16, device=DEV)
        vd = torch.full(shape, nan, dtype=torch.bfloat16, device=DEV)
        src_k, src_v = bf16_tensor(k), bf16_tensor(v)
    ids = torch.from_numpy(pool.ids).to(DEV)
    kd.index_copy_(0, ids, src_k)
    vd.index_copy_(0, ids, src_v)
    return kd, vd


def _same_bytes(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


class MixedStep:
    """Device tensors of the mixed step and the oracle's pools and outputs."""

    def __init__(self, fp8: bool):
        m = W.make_mixed_inputs(W.PREFILL_CONFIGS["c5p"], W.CONFIGS["c5d"])
        self.m, self.fp8 = m, fp8
        p, d = m.prefill, m.decode
        bs = p.spec.block_size
        # the inputs meet the preconditions the calls leave to the caller
        pa.check_tables(d.block_tables, d.context_lens, m.pool.num_blocks, bs, fused_append=True)
        pa.check_tables(p.block_tables, p.context_lens, m.pool.num_blocks, bs)
        pa.check_prefill(p.cu_seqlens_q, p.context_lens, int(max(p.spec.chunk_lens)))
        pa.check_slots(m.all_rows()[2], m.pool.num_blocks, bs)

        # ---- the oracle: all 576 rows appended, then prefill and decode ----
        nk, nv, slots = m.all_rows()
        cslots = _compact_slots(m.pool, slots, bs)
        pct = m.pool.compact_tables(p.block_tables, p.poison_block)
        dct = m.pool.compact_tables(d.block_tables, d.poison_block)
        if fp8:
            k8, v8 = W.fp8_codes_like(p)
            self.k0, self.v0 = _full_pool(m.pool, k8, v8, True)
            ka, va = O8.append_fp8(nk, nv, cslots, k8, v8, K_SCALE, V_SCALE)
            self.ref_prefill = O8.prefill_fp8(p.q, p.cu_seqlens_q, ka, va, pct, p.context_lens,
                                              p.scale, K_SCALE, V_SCALE)
            self.ref_decode = O8.decode_fp8(d.q, ka, va, dct, d.context_lens, d.scale, K_SCALE,
                                            V_SCALE)
        else:
            self.k0, self.v0 = _full_pool(m.pool, m.pool.k, m.pool.v, False)
            ka, va = oracle.append(nk, nv, cslots, m.pool.k, m.pool.v)
            self.ref_prefill = oracle.prefill(p.q, p.cu_seqlens_q, ka, va, pct, p.context_lens,
                                              p.scale)
            self.ref_decode = oracle.decode(d.q, ka, va, dct, d.context_lens, d.scale)
        self.k_want, self.v_want = _full_pool(m.pool, ka, va, fp8)

        # ---- device inputs of the three calls ----
        self.k_cache, self.v_cache = self.k0.clone(), self.v0.clone()
        self.chunk_k, self.chunk_v = bf16_tensor(p.new_k), bf16_tensor(p.new_v)
        self.chunk_slots = torch.from_numpy(p.slot_mapping).to(DEV)
        self.pq = bf16_tensor(p.q)
        self.cu = torch.from_numpy(p.cu_seqlens_q).to(DEV)
        self.ptables = torch.from_numpy(p.block_tables).to(DEV)
        self.plens = torch.from_numpy(p.context_lens).to(DEV)
        self.max_q = int(max(p.spec.chunk_lens))
        self.pout = torch.empty_like(self.pq)
        self.dq = bf16_tensor(d.q)
        self.dk, self.dv = bf16_tensor(d.new_k), bf16_tensor(d.new_v)
        self.dtables = torch.from_numpy(d.block_tables).to(DEV)
        self.dlens = torch.from_numpy(d.context_lens).to(DEV)
        self.dout = torch.empty_like(self.dq)
        s = d.spec
        self.pS = pa.prefill_auto_splits(1, self.max_q, s.num_kv_heads, p.spec.max_blocks_per_seq,
                                         bs, DEV)
        self.dS = pa.auto_splits(s.num_seqs, s.num_kv_heads, s.max_blocks_per_seq, bs, DEV)
        Hq, D = s.num_q_heads, s.head_dim
        self.pws = torch.empty(max(pa.prefill_workspace_size(1, self.max_q, Hq, D, self.pS), 256),
                               dtype=torch.uint8, device=DEV)
        self.dws = torch.empty(max(pa.decode_workspace_size(s.num_seqs, Hq, D, self.dS), 256),
                               dtype=torch.uint8, device=DEV)

    def step(self):
        """The three calls of the step, on the current stream."""
        p, d = self.m.prefill, self.m.decode
        if self.fp8:
            pa.reshape_and_cache_fp8(self.chunk_k, self.chunk_v, self.chunk_slots, self.k_cache,
                                     self.v_cache, K_SCALE, V_SCALE)
            pa.prefill_fp8(self.pq, self.cu, self.k_cache, self.v_cache, self.ptables, self.plens,
                           float(p.scale), K_SCALE, V_SCALE, self.pout, self.max_q,
                           num_splits=self.pS, workspace=self.pws)
            pa.append_decode_fp8(self.dq, self.dk, self.dv, self.k_cache, self.v_cache,
                                 self.dtables, self.dlens, float(d.scale), K_SCALE, V_SCALE,
                                 self.dS, self.dout, workspace=self.dws)
        else:
            pa.reshape_and_cache(self.chunk_k, self.chunk_v, self.chunk_slots, self.k_cache,
                                 self.v_cache)
            pa.prefill(self.pq, self.cu, self.k_cache, self.v_cache, self.ptables, self.plens,
                       float(p.scale), self.pout, self.max_q, num_splits=self.pS,
                       workspace=self.pws)
            pa.append_decode(self.dq, self.dk, self.dv, self.k_cache, self.v_cache, self.dtables,
                             self.dlens, float(d.scale), self.dS, self.dout, workspace=self.dws)

    def reset(self):
        """Pools back to their state before the step; outputs poisoned."""
        self.k_cache.copy_(self.k0)
        self.v_cache.copy_(self.v0)
        self.pout.fill_(float("nan"))
        self.dout.fill_(float("nan"))

    def order_decode(self, order, splits: int):
        """Launch the decode sequences in `order` (host indices) with `splits`
        pieces; the expected decode rows follow the order."""
        perm = torch.from_numpy(np.asarray(order, np.int64)).to(DEV)
        self.dq, self.dk, self.dv, self.dtables, self.dlens = (
            t[perm].contiguous() for t in (self.dq, self.dk, self.dv, self.dtables, self.dlens))
        self.ref_decode = self.ref_decode[np.asarray(order)]
        self.dS = splits
        s = self.m.decode.spec
        self.dws = torch.empty(max(pa.decode_workspace_size(s.num_seqs, s.num_q_heads,
                                                            s.head_dim, splits), 256),
                               dtype=torch.uint8, device=DEV)

    def check(self, what: str):
        torch.cuda.synchronize()
        assert _same_bytes(self.k_cache, self.k_want), f"{what}: K pool differs from the oracle"
        assert _same_bytes(self.v_cache, self.v_want), f"{what}: V pool differs from the oracle"
        e1 = assert_close(to_f64(self.pout), self.ref_prefill, what=f"{what}: prefill rows")
        e2 = assert_close(to_f64(self.dout), self.ref_decode, what=f"{what}: decode rows")
        print(f"{what}: prefill max abs {e1[0]:.2e} rms {e1[1]:.2e}; "
              f"decode max abs {e2[0]:.2e} rms {e2[1]:.2e}", flush=True)
        return to_bits(self.pout), to_bits(self.dout)


@pytest.fixture(scope="module", params=[False, True], ids=["bf16", "fp8"])
def mixed(request):
    step = MixedStep(request.param)
    yield step
    del step
    torch.cuda.empty_cache()


def test_mixed_step_eager(mixed):
    """The composed step on one stream matches the oracle: pools bit for bit,
    prefill and decode rows within tolerance."""
    mixed.reset()
    mixed.step()
    mixed.check("eager")


def test_mixed_step_graph_replays(mixed):
    """The step captured in one graph and replayed three times (pools reset
    and outputs poisoned eagerly before each replay) matches the oracle on
    every replay and equals the eager step bit for bit."""
    mixed.reset()
    mixed.step()
    eager = mixed.check("eager before capture")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mixed.step()
    torch.cuda.synchronize()
    for i in range(3):
        mixed.reset()
        torch.cuda.synchronize()
        g.replay()
        got = mixed.check(f"replay {i}")
        assert np.array_equal(got[0], eager[0]) and np.array_equal(got[1], eager[1]), i
    del g


def test_mixed_step_decode_longest_first(mixed):
    """The same step with the decode batch launched longest first (the block
    manager's order) and its split count from the host's lengths in that
    order: two pieces with mirrored second pieces for this batch of 64
    sequences x 4 kv heads on 256 compute units.  Pools bit for bit, rows
    within tolerance; then back to the drawn order."""
    d = mixed.m.decode
    s = d.spec
    bm = pa.BlockManager(s.num_blocks, s.block_size, s.max_blocks_per_seq, prefix_cache=False)
    for b, L in enumerate(d.context_lens):
        bm.admit(b, 0, np.zeros(int(L), np.int32))
    order = bm.order_longest_first(np.arange(s.num_seqs))
    del bm
    assert np.all(np.diff(d.context_lens[order]) <= 0)
    S = pa.auto_splits_lengths(d.context_lens[order], s.num_kv_heads, s.max_blocks_per_seq,
                               s.block_size, DEV)
    saved = (mixed.dq, mixed.dk, mixed.dv, mixed.dtables, mixed.dlens, mixed.ref_decode,
             mixed.dS, mixed.dws)
    try:
        mixed.order_decode(order, S)
        mixed.reset()
        mixed.step()
        mixed.check(f"decode longest first, S={S}")
    finally:
        (mixed.dq, mixed.dk, mixed.dv, mixed.dtables, mixed.dlens, mixed.ref_decode, mixed.dS,
         mixed.dws) = saved
