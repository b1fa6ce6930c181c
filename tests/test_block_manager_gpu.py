"""The device path fed by the native block manager: prompts with a shared
system prefix are admitted (cached prefix blocks reused), their uncached K/V
appended through the returned slots with pa_reshape_and_cache, decode steps
appended one token at a time, and a speculative round drafts 4 tokens,
verifies them with pa_decode_multi and rolls back the rejected ones.  Every
attention result is compared with the oracle run on a host copy of the same
pool (tolerance as for decode)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_09_amd as pa
import workloads as W
from gpu_cases import DEV, assert_close, bf16_tensor, to_f64

pytestmark = pytest.mark.gpu

BS, HQ, HKV, D, NB, WMAX = 16, 12, 2, 128, 256, 64


def _kv_row(prefix_tokens, which):
    """K or V row of a token, a function of the whole prefix up to it, so that
    identical prefixes give identical rows (as in a real model)."""
    h = (hash(tuple(prefix_tokens)) ^ which) & 0xFFFFFFFF
    x = np.random.default_rng(h).standard_normal((HKV, D), dtype=np.float32)
    return W.f32_to_bf16_bits(x)


class Pool:
    def __init__(self):
        self.kh = np.full((NB, BS, HKV, D), W.BF16_NAN, np.uint16)
        self.vh = self.kh.copy()
        self.kd = bf16_tensor(self.kh)
        self.vd = bf16_tensor(self.vh)

    def write(self, tokens, first, slots):
        """K/V of tokens[first:first+len(slots)] into the given slots, on the
        device through the library's append and on the host copy."""
        if len(slots) == 0:
            return
        k = np.stack([_kv_row(tokens[:first + j + 1], 0) for j in range(len(slots))])
        v = np.stack([_kv_row(tokens[:first + j + 1], 1) for j in range(len(slots))])
        s = np.asarray(slots, np.int64)
        pa.reshape_and_cache(bf16_tensor(k), bf16_tensor(v), torch.from_numpy(s).to(DEV), self.kd,
                             self.vd)
        self.kh, self.vh = oracle.append(k, v, s, self.kh, self.vh)


def test_decode_from_manager_layout():
    rng = np.random.default_rng(21)
    bm = pa.BlockManager(NB, BS, WMAX, prefix_cache=True)
    pool = Pool()
    system = [int(x) for x in rng.integers(0, 1000, 3 * BS + 5)]
    seqs = {}
    for k in range(1, 7):
        prompt = system + [int(x) for x in rng.integers(0, 1000, int(rng.integers(1, 40)))]
        cached, slots = bm.admit(k, 0, prompt)
        if k > 1:
            assert cached == 3 * BS          # the system prompt's full blocks are reused
        pool.write(prompt, cached, slots)
        if k == 1:
            # one decode step: sequence 1 moves past its prompt, whose full
            # blocks (the system prompt's among them) become shareable
            tok = [int(rng.integers(0, 1000))]
            slot = bm.append(k, tok)
            prompt = prompt + tok
            pool.write(prompt, len(prompt) - 1, slot)
        seqs[k] = prompt
    for step in range(3):
        for k in sorted(seqs):
            tok = [int(rng.integers(0, 1000))]
            slot = bm.append(k, tok)
            seqs[k] = seqs[k] + tok
            pool.write(seqs[k], len(seqs[k]) - 1, slot)
        ids = sorted(seqs)
        tables, lens = bm.block_tables(ids)
        q = W.f32_to_bf16_bits(rng.standard_normal((len(ids), HQ, D), dtype=np.float32))
        out = torch.empty((len(ids), HQ, D), dtype=torch.bfloat16, device=DEV)
        pa.decode(bf16_tensor(q), pool.kd, pool.vd, torch.from_numpy(tables).to(DEV),
                  torch.from_numpy(lens).to(DEV), 0.0883883461356163, 0, out)
        torch.cuda.synchronize()
        ref = oracle.decode(q, pool.kh, pool.vh, tables, lens, np.float32(0.0883883461356163))
        assert_close(to_f64(out), ref, what=f"step {step}")
    # device pool equals the host copy bit for bit wherever the host has data
    kd = pool.kd.view(torch.int16).cpu().numpy().view(np.uint16)
    written = pool.kh != W.BF16_NAN
    assert np.array_equal(kd[written], pool.kh[written])


def test_speculative_round_with_rollback():
    rng = np.random.default_rng(22)
    bm = pa.BlockManager(NB, BS, WMAX, prefix_cache=True)
    pool = Pool()
    seqs = {}
    for k in range(1, 5):
        prompt = [int(x) for x in rng.integers(0, 1000, int(rng.integers(20, 200)))]
        cached, slots = bm.admit(k, 0, prompt)
        pool.write(prompt, cached, slots)
        seqs[k] = prompt
    ids = sorted(seqs)
    QL = 4
    # draft QL tokens per sequence, append their K/V, verify in one pass
    for k in ids:
        draft = [int(x) for x in rng.integers(0, 1000, QL)]
        slots = bm.append(k, draft)
        seqs[k] = seqs[k] + draft
        pool.write(seqs[k], len(seqs[k]) - QL, slots)
    tables, lens = bm.block_tables(ids)
    q = W.f32_to_bf16_bits(rng.standard_normal((len(ids), QL, HQ, D), dtype=np.float32))
    out = torch.empty((len(ids), QL, HQ, D), dtype=torch.bfloat16, device=DEV)
    scale = 0.0883883461356163
    pa.decode_multi(bf16_tensor(q), pool.kd, pool.vd, torch.from_numpy(tables).to(DEV),
                    torch.from_numpy(lens).to(DEV), scale, 0, out)
    torch.cuda.synchronize()
    ref = oracle.decode_multi(q, pool.kh, pool.vh, tables, lens, np.float32(scale))
    assert_close(to_f64(out), ref, what="verify")
    # accept a different number of draft tokens per sequence, roll back the rest
    for k, accept in zip(ids, (0, 1, 2, 4)):
        new_len = len(seqs[k]) - QL + accept
        bm.truncate(k, new_len)
        seqs[k] = seqs[k][:new_len]
        tok = [int(rng.integers(0, 1000))]
        slot = bm.append(k, tok)
        seqs[k] = seqs[k] + tok
        pool.write(seqs[k], len(seqs[k]) - 1, slot)
    tables, lens = bm.block_tables(ids)
    assert lens.tolist() == [len(seqs[k]) for k in ids]
    q1 = W.f32_to_bf16_bits(rng.standard_normal((len(ids), HQ, D), dtype=np.float32))
    out1 = torch.empty((len(ids), HQ, D), dtype=torch.bfloat16, device=DEV)
    pa.decode(bf16_tensor(q1), pool.kd, pool.vd, torch.from_numpy(tables).to(DEV),
              torch.from_numpy(lens).to(DEV), scale, 0, out1)
    torch.cuda.synchronize()
    ref1 = oracle.decode(q1, pool.kh, pool.vh, tables, lens, np.float32(scale))
    assert_close(to_f64(out1), ref1, what="after rollback")
