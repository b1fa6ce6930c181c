"""GPU parity of multi-token decode (the speculative verify step) against the
fp64 oracle.

Each sequence's q_len newest tokens are appended through slot_mapping first
(the library's append), then pa_decode_multi runs; query token j of a window
attends keys 0 .. L - q_len + j.  Tolerance as for decode:
|gpu - oracle| <= 1e-2 + 1e-2 |oracle| elementwise.  Cases cover one and two
16-column tiles (G * q_len up to 32), both head_dims and block sizes, ragged
lengths, several split counts, and sequences shorter than their window.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_09_amd as pa
import workloads as W
from gpu_cases import DEV, assert_close, bf16_tensor, device_pool, to_f64

pytestmark = pytest.mark.gpu


class MultiCase:
    def __init__(self, D, G, Hkv, bs, QL, lens, seed):
        B = len(lens)
        Wd = -(-max(lens) // bs)
        nb = sum(-(-L // bs) for L in lens) + 7
        spec = W.PrefillSpec(f"multi{D}_{G}_{QL}", G * Hkv, Hkv, D, bs, nb, Wd,
                             chunk_lens=(QL,) * B, total_lens=tuple(lens), seed=seed)
        inp = W.make_prefill_inputs(spec)
        self.inp, self.spec, self.QL = inp, spec, QL
        self.B, self.Hq, self.D = B, G * Hkv, D
        self.k_cache, self.v_cache = device_pool(inp.pool)
        self.q_bits = inp.q.reshape(B, QL, G * Hkv, D)
        self.q = bf16_tensor(self.q_bits)
        self.tables = torch.from_numpy(inp.block_tables).to(DEV)
        self.lens = torch.from_numpy(inp.context_lens).to(DEV)
        self.out = torch.empty_like(self.q)
        pa.reshape_and_cache(bf16_tensor(inp.new_k), bf16_tensor(inp.new_v),
                             torch.from_numpy(inp.slot_mapping).to(DEV), self.k_cache,
                             self.v_cache)
        self.kc, self.vc, self.ct = self._oracle_pools()
        self.ref = self.oracle(inp.context_lens)

    def _oracle_pools(self):
        p = self.inp.pool
        bs = self.spec.block_size
        lut = {int(x): i for i, x in enumerate(p.ids)}
        slots = np.array([lut[int(s) // bs] * bs + int(s) % bs for s in self.inp.slot_mapping],
                         np.int64)
        kc, vc = oracle.append(self.inp.new_k, self.inp.new_v, slots, p.k, p.v)
        return kc, vc, p.compact_tables(self.inp.block_tables, self.inp.poison_block)

    def oracle(self, lens):
        return oracle.decode_multi(self.q_bits, self.kc, self.vc, self.ct, np.asarray(lens),
                                   self.inp.scale)

    def run(self, S=0, lens=None):
        pa.decode_multi(self.q, self.k_cache, self.v_cache, self.tables,
                        self.lens if lens is None else lens, float(self.inp.scale), S, self.out)
        torch.cuda.synchronize()
        return to_f64(self.out)


CASES = {
    # D, G, Hkv, bs, q_len, lens
    "g7_q4_bs256": (128, 7, 4, 256, 4, (3001, 4, 700, 1800, 2049, 256)),   # 28 rows, 2 tiles
    "g6_q2_bs16": (128, 6, 2, 16, 2, (4096, 700, 33)),                     # 12 rows, 1 tile
    "g8_q4_full": (128, 8, 1, 256, 4, (600, 2049)),                        # 32 rows
    "g5_q6": (128, 5, 2, 16, 6, (100, 7)),                                  # 30 rows
    "d64_g2_q8": (64, 2, 2, 16, 8, (9, 300, 1000)),                         # 16 rows, G 2
    "d64_g1_q3": (64, 1, 2, 256, 3, (5, 513)),
    "d64_g4_q7": (64, 4, 1, 16, 7, (64, 65, 2000)),                         # 28 rows
}


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    D, G, Hkv, bs, QL, lens = CASES[request.param]
    return request.param, MultiCase(D, G, Hkv, bs, QL, lens, seed=7000 + D + 10 * G + QL)


def test_parity(case):
    name, c = case
    for S in (1, 2, 3, 0, 64):     # S = 2: second pieces in mirrored unit order
        maxe, rms = assert_close(c.run(S), c.ref, what=f"{name} S={S}")
    print(f"{name}: max abs err {maxe:.3e} rms {rms:.3e}")


def test_each_token_is_a_shorter_decode(case):
    """Query token j of the window equals a one-token decode of the same
    query over the sequence cut after position L - q_len + j."""
    name, c = case
    full = c.run(0)
    L = c.inp.context_lens.astype(np.int64)
    out1 = torch.empty((c.B, c.Hq, c.D), dtype=torch.bfloat16, device=DEV)
    for j in range(c.QL):
        cut = torch.from_numpy((L - c.QL + j + 1).astype(np.int32)).to(DEV)
        pa.decode(c.q[:, j].contiguous(), c.k_cache, c.v_cache, c.tables, cut,
                  float(c.inp.scale), 0, out1)
        torch.cuda.synchronize()
        one = to_f64(out1)
        assert (np.abs(full[:, j] - one) <= 2 ** -7 * np.abs(one) + 2e-3).all(), (name, j)


def test_sequences_shorter_than_the_window():
    """Context lengths below q_len: tokens whose position is negative get
    zero rows, the rest attend the few keys there are."""
    c = MultiCase(128, 7, 4, 256, 4, (300, 300, 300), seed=7100)
    short = np.array([1, 3, 4], np.int32)
    got = c.run(0, torch.from_numpy(short).to(DEV))
    ref = c.oracle(short)
    assert_close(got, ref, what="short windows")
    assert (got[0, :3] == 0).all() and (got[1, :1] == 0).all()


@pytest.mark.parametrize("name", ["g6_q2_bs16", "d64_g1_q3", "g7_q4_bs256"])
def test_one_token_window_is_decode_bit_for_bit(name):
    """q_len 1 takes the single-token kernels: identical bits to pa_decode."""
    D, G, Hkv, bs, _, lens = CASES[name]
    c = MultiCase(D, G, Hkv, bs, 1, lens, seed=7200 + G)
    out1 = torch.empty((c.B, c.Hq, c.D), dtype=torch.bfloat16, device=DEV)
    for S in (1, 5, 0):
        multi = c.run(S)
        pa.decode(c.q[:, 0].contiguous(), c.k_cache, c.v_cache, c.tables, c.lens,
                  float(c.inp.scale), S, out1)
        torch.cuda.synchronize()
        assert torch.equal(c.out[:, 0], out1), (name, S)
        assert_close(multi, c.ref, what=f"{name} q_len 1 S={S}")
