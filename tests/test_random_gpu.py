"""Seeded random configurations against the oracle: head_dim, group, block
size, batch, ragged lengths (empty sequences included), split count, query
tokens per sequence and pool dtype drawn at random, each call checked
elementwise at the attention tolerance |gpu - oracle| <= 1e-2 + 1e-2 |oracle|.
Complements the structured cases with combinations nobody wrote down."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_09_amd as pa
import workloads as W
from gpu_cases import DEV, DecodeCase, assert_close, bf16_tensor, to_f64
from test_kv_fp8_gpu import _oracle_fp8, _run_fp8

pytestmark = pytest.mark.gpu


def _draw(seed):
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 128]))
    G = int(rng.integers(1, 9))
    Hkv = int(rng.choice([1, 2, 4]))
    bs = int(rng.choice([16, 256]))
    B = int(rng.integers(1, 13))
    Wt = int(rng.integers(1, 4097 // bs + 1))
    cap = Wt * bs
    lens = rng.integers(0, cap + 1, B)
    lens[rng.random(B) < 0.15] = 0
    S = int(rng.choice([0, 1, 2, 3, 7, 16, 64]))
    nb = int(((lens + bs - 1) // bs).sum()) + 3
    spec = W.DecodeSpec(f"rand{seed}", B, G * Hkv, Hkv, D, bs, nb, Wt,
                        context_lens=tuple(int(x) for x in lens), seed=seed)
    return spec, S, rng


@pytest.mark.parametrize("seed", range(20))
def test_random_decode(seed):
    spec, S, _ = _draw(1000 + seed)
    print(f"seed {seed}: D={spec.head_dim} Hq={spec.num_q_heads} Hkv={spec.num_kv_heads} "
          f"bs={spec.block_size} B={spec.num_seqs} W={spec.max_blocks_per_seq} S={S}", flush=True)
    case = DecodeCase(W.make_decode_inputs(spec))
    case.run(num_splits=S)
    torch.cuda.synchronize()
    assert_close(to_f64(case.out), case.ref, what=f"random decode {seed}")


@pytest.mark.parametrize("seed", range(10))
def test_random_decode_fp8(seed):
    spec, S, rng = _draw(2000 + seed)
    ks, vs = float(2.0 ** rng.integers(-4, 3) * rng.uniform(0.5, 1)), float(rng.uniform(0.05, 2))
    print(f"seed {seed}: D={spec.head_dim} Hq={spec.num_q_heads} Hkv={spec.num_kv_heads} "
          f"bs={spec.block_size} B={spec.num_seqs} S={S} ks={ks:.3g} vs={vs:.3g}", flush=True)
    inp = W.make_decode_inputs(spec, fill="zeros")
    k8, v8 = W.fp8_codes_like(inp)
    got = to_f64(_run_fp8(inp, k8, v8, ks, vs, S))
    assert_close(got, _oracle_fp8(inp, k8, v8, ks, vs), what=f"random fp8 {seed}")


@pytest.mark.parametrize("seed", range(10))
def test_random_decode_multi(seed):
    spec, S, rng = _draw(3000 + seed)
    G = spec.num_q_heads // spec.num_kv_heads
    QL = int(rng.integers(1, min(8, 32 // G) + 1))
    lens = np.maximum(np.asarray(spec.context_lens), QL)     # every window inside its sequence
    lens = np.minimum(lens, spec.max_blocks_per_seq * spec.block_size)
    print(f"seed {seed}: D={spec.head_dim} G={G} Hkv={spec.num_kv_heads} bs={spec.block_size} "
          f"B={spec.num_seqs} q_len={QL} S={S}", flush=True)
    from test_decode_multi_gpu import MultiCase
    case = MultiCase(spec.head_dim, G, spec.num_kv_heads, spec.block_size, QL,
                     tuple(int(x) for x in lens), 3000 + seed)
    case.run(S)
    torch.cuda.synchronize()
    assert_close(to_f64(case.out), case.ref, what=f"random multi {seed}")


@pytest.mark.parametrize("seed", range(10))
def test_random_prefill(seed):
    rng = np.random.default_rng(4000 + seed)
    D = int(rng.choice([64, 128]))
    G = int(rng.integers(1, 9))
    Hkv = int(rng.choice([1, 2, 4]))
    bs = int(rng.choice([16, 256]))
    B = int(rng.integers(1, 6))
    chunks = rng.integers(0, 200, B)
    chunks[0] = max(int(chunks[0]), 1)                       # at least one query row
    totals = chunks + rng.integers(0, 1500, B)
    Wt = int(-(-int(totals.max()) // bs)) + int(rng.integers(0, 3))
    nb = int(((totals + bs - 1) // bs).sum()) + 3
    S = int(rng.choice([0, 1, 2, 5]))
    max_q = int(chunks.max()) + int(rng.integers(0, 40))
    spec = W.PrefillSpec(f"rpre{seed}", G * Hkv, Hkv, D, bs, nb, max(Wt, 1),
                         chunk_lens=tuple(int(x) for x in chunks),
                         total_lens=tuple(int(x) for x in totals), seed=4000 + seed)
    print(f"seed {seed}: D={D} G={G} Hkv={Hkv} bs={bs} chunks={list(chunks)} "
          f"totals={list(totals)} S={S} max_q={max_q}", flush=True)
    from test_prefill_gpu import PrefillCase
    case = PrefillCase(spec)
    assert_close(case.run(S, max_q=max(max_q, 1)), case.ref, what=f"random prefill {seed}")
