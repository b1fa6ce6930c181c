"""GPU parity at the largest calls the C ABI accepts, against the fp64 oracle.

* PA_MAX_SEQS sequences in one call: the merge grid's sequence dimension at
  its limit (two pieces per sequence), the direct single-piece path and the
  fused append + decode, over ragged lengths that include empty sequences.
* PA_MAX_HEADS q heads: group 8 (matrix path), group 1 (vector path) and the
  multi-token decode, whose merge grid spans q_len * PA_MAX_HEADS rows.
* Both limits over fp8 pools too, and PA_MAX_SEQS prompt chunks in one prefill.

Tolerance as for every attention output here: |gpu - oracle| <= 1e-2 +
1e-2 |oracle| elementwise, and the append bit-exact over the whole pools.
One call past each limit is refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_09_amd as pa
import workloads as W
from gpu_cases import DEV, DecodeCase, assert_close, bf16_tensor, to_bits, to_f64
from test_decode_multi_gpu import MultiCase
from test_kv_fp8_gpu import _oracle_fp8, _run_fp8

pytestmark = pytest.mark.gpu


def _max_seq_lens():
    """PA_MAX_SEQS lengths: every 5th sequence empty, most 1..16 tokens (one
    block), and every 997th sequence 100..128 tokens (seven or eight blocks,
    so it spans both pieces of a two-piece split)."""
    b = np.arange(pa.PA_MAX_SEQS, dtype=np.int64)
    lens = 1 + (b * 7919) % 16
    lens[b % 997 == 1] = 100 + (b[b % 997 == 1] % 29)
    lens[b % 5 == 0] = 0
    return lens.astype(np.int32)


def _max_seq_spec(append=False):
    lens = _max_seq_lens()
    bs = 16
    nb = int(((lens + bs - 1) // bs).sum()) + 8
    return W.DecodeSpec("max-seqs", pa.PA_MAX_SEQS, 2, 1, 64, bs, nb, 8,
                        context_lens=tuple(int(x) for x in lens), seed=9100, append=append)


@pytest.fixture(scope="module")
def max_seq_case():
    return DecodeCase(W.make_decode_inputs(_max_seq_spec()))


@pytest.mark.parametrize("S", [1, 2])
def test_max_num_seqs_decode(max_seq_case, S):
    case = max_seq_case
    print(f"decode B={case.inp.spec.num_seqs} S={S}", flush=True)
    case.run(num_splits=S)
    torch.cuda.synchronize()
    got = to_f64(case.out)
    empty = case.inp.context_lens == 0
    assert (got[empty] == 0).all()
    assert_close(got, case.ref, what=f"B={case.inp.spec.num_seqs} S={S}")


def test_max_num_seqs_fused_append_decode():
    """Every non-empty sequence appends its newest token in the decode launch."""
    inp = W.make_decode_inputs(_max_seq_spec(append=True))
    case = DecodeCase(inp)
    B, Hkv, D = inp.spec.num_seqs, inp.spec.num_kv_heads, inp.spec.head_dim
    sel = np.nonzero(inp.context_lens > 0)[0]
    nk = np.zeros((B, Hkv, D), np.uint16)
    nv = np.zeros((B, Hkv, D), np.uint16)
    nk[sel], nv[sel] = inp.new_k, inp.new_v
    before_k, before_v = to_bits(case.k_cache), to_bits(case.v_cache)
    print(f"append_decode B={B} S=2", flush=True)
    pa.append_decode(case.q, bf16_tensor(nk), bf16_tensor(nv), case.k_cache, case.v_cache,
                     case.tables, case.lens, case.scale, 2, case.out)
    torch.cuda.synchronize()
    want_k, want_v = oracle.append(inp.new_k, inp.new_v, inp.slot_mapping, before_k, before_v)
    assert np.array_equal(to_bits(case.k_cache), want_k)
    assert np.array_equal(to_bits(case.v_cache), want_v)
    assert_close(to_f64(case.out), case.ref, what=f"fused B={B}")


@pytest.mark.parametrize("Hkv,D,lens", [(512, 64, (1, 40, 100)), (4096, 64, (3, 33))])
def test_max_heads_decode(Hkv, D, lens):
    """PA_MAX_HEADS q heads: group 8 on the matrix path, group 1 on the vector
    path, at S = 1, 2 and automatic."""
    bs = 16
    nb = sum(-(-L // bs) for L in lens) + 4
    spec = W.DecodeSpec("max-heads", len(lens), pa.PA_MAX_HEADS, Hkv, D, bs, nb, 8,
                        context_lens=lens, seed=9200 + Hkv)
    case = DecodeCase(W.make_decode_inputs(spec))
    for S in (1, 2, 0):
        print(f"decode Hq={spec.num_q_heads} Hkv={Hkv} S={S}", flush=True)
        case.run(num_splits=S)
        torch.cuda.synchronize()
        assert_close(to_f64(case.out), case.ref, what=f"Hq={spec.num_q_heads} Hkv={Hkv} S={S}")


def test_max_heads_multi_token_decode():
    """q_len 4 at PA_MAX_HEADS q heads (group 4): 16 query rows per workgroup,
    4 * PA_MAX_HEADS rows for the merge."""
    case = MultiCase(D=64, G=4, Hkv=pa.PA_MAX_HEADS // 4, bs=16, QL=4, lens=(5, 70), seed=9300)
    for S in (1, 2):
        print(f"decode_multi Hq={case.Hq} q_len=4 S={S}", flush=True)
        case.run(S)
        torch.cuda.synchronize()
        assert_close(to_f64(case.out), case.ref, what=f"multi Hq={case.Hq} S={S}")


@pytest.fixture(scope="module")
def max_seq_fp8():
    inp = W.make_decode_inputs(_max_seq_spec(), fill="zeros")
    k8, v8 = W.fp8_codes_like(inp)
    return inp, k8, v8, _oracle_fp8(inp, k8, v8, 0.3, 0.7)


@pytest.mark.parametrize("S", [1, 2])
def test_max_num_seqs_decode_fp8(max_seq_fp8, S):
    """PA_MAX_SEQS sequences over fp8 pools (head-major codes, per-pool scales)."""
    inp, k8, v8, ref = max_seq_fp8
    print(f"decode_fp8 B={inp.spec.num_seqs} S={S}", flush=True)
    got = to_f64(_run_fp8(inp, k8, v8, 0.3, 0.7, S))
    assert_close(got, ref, what=f"fp8 B={inp.spec.num_seqs} S={S}")


def test_max_heads_decode_fp8():
    """PA_MAX_HEADS q heads at group 8 over fp8 pools, S = 1, 2 and automatic."""
    lens = (1, 40, 100)
    nb = sum(-(-L // 16) for L in lens) + 4
    spec = W.DecodeSpec("max-heads-fp8", len(lens), pa.PA_MAX_HEADS, 512, 64, 16, nb, 8,
                        context_lens=lens, seed=9400)
    inp = W.make_decode_inputs(spec, fill="zeros")
    k8, v8 = W.fp8_codes_like(inp)
    ref = _oracle_fp8(inp, k8, v8, 0.5, 0.25)
    for S in (1, 2, 0):
        print(f"decode_fp8 Hq={spec.num_q_heads} S={S}", flush=True)
        assert_close(to_f64(_run_fp8(inp, k8, v8, 0.5, 0.25, S)), ref, what=f"fp8 heads S={S}")


def test_max_num_seqs_prefill():
    """PA_MAX_SEQS prompt chunks in one prefill call (the merge grid's sequence
    dimension at its limit): chunks of 0..3 tokens, most sequences 0..16
    tokens long and every 1000th 65..80 (two key pieces at S = 2), every
    cached token already in the pool.  Inputs are drawn here in bulk (one
    normal draw for the whole pool) since the pool has 66k blocks."""
    B, Hq, Hkv, D, bs, Wt = pa.PA_MAX_SEQS, 2, 1, 64, 16, 5
    rng = np.random.default_rng(9500)
    totals = rng.integers(0, 17, B)
    long = np.arange(B) % 1000 == 7
    totals[long] = rng.integers(65, 81, int(long.sum()))
    chunks = np.minimum(totals, rng.integers(0, 4, B))
    nblk = (totals + bs - 1) // bs
    NB = int(nblk.sum()) + 1
    poison = NB - 1
    ids = rng.permutation(NB - 1)
    tables = np.full((B, Wt), poison, np.int32)
    off = 0
    for b in np.nonzero(nblk)[0]:
        tables[b, :nblk[b]] = ids[off:off + nblk[b]]
        off += int(nblk[b])
    pools = []
    for _ in range(2):
        pool = np.empty((NB, bs, Hkv, D), np.uint16)
        for i in range(0, NB, 8192):
            j = min(NB, i + 8192)
            pool[i:j] = W.f32_to_bf16_bits(rng.standard_normal((j - i, bs, Hkv, D), np.float32))
        pool[poison] = W.BF16_NAN
        tail = np.nonzero(totals % bs)[0]       # slots past each sequence's length: NaN
        for b in tail:
            pool[tables[b, totals[b] // bs], totals[b] % bs:] = W.BF16_NAN
        pools.append(pool)
    kc, vc = pools
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(chunks)
    q = W.f32_to_bf16_bits(rng.standard_normal((int(cu[-1]), Hq, D), np.float32))
    lens = totals.astype(np.int32)
    scale = np.float32(0.125)
    pa.check_tables(tables, lens, NB, bs)
    pa.check_prefill(cu, lens, 3)
    ref = oracle.prefill(q, cu, kc, vc, tables, lens, scale)
    dk, dv = bf16_tensor(kc), bf16_tensor(vc)
    dq = bf16_tensor(q)
    out = torch.empty_like(dq)
    for S in (1, 2):
        print(f"prefill B={B} S={S}", flush=True)
        pa.prefill(dq, torch.from_numpy(cu).to(DEV), dk, dv, torch.from_numpy(tables).to(DEV),
                   torch.from_numpy(lens).to(DEV), float(scale), out, 3, num_splits=S)
        torch.cuda.synchronize()
        assert_close(to_f64(out), ref, what=f"prefill B={B} S={S}")


def test_one_past_each_limit_is_refused(max_seq_case):
    """A batch of PA_MAX_SEQS + 1 and PA_MAX_HEADS * 2 q heads fail with a
    shape error before any launch; the output buffer is left untouched."""
    case = max_seq_case
    q = torch.zeros((pa.PA_MAX_SEQS + 1, 2, 64), dtype=torch.bfloat16, device=DEV)
    out = torch.full_like(q, 7.0)
    tables = torch.zeros((pa.PA_MAX_SEQS + 1, 8), dtype=torch.int32, device=DEV)
    lens = torch.zeros(pa.PA_MAX_SEQS + 1, dtype=torch.int32, device=DEV)
    with pytest.raises(pa.PagedAttnError):
        pa.decode(q, case.k_cache, case.v_cache, tables, lens, 0.125, 1, out)
    q2 = torch.zeros((1, 2 * pa.PA_MAX_HEADS, 64), dtype=torch.bfloat16, device=DEV)
    out2 = torch.full_like(q2, 7.0)
    with pytest.raises(pa.PagedAttnError):
        pa.decode(q2, case.k_cache, case.v_cache, tables[:1], lens[:1], 0.125, 1, out2)
    torch.cuda.synchronize()
    assert (out == 7.0).all() and (out2 == 7.0).all()
