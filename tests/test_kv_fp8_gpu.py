"""FP8 KV pages on the device against the oracle (oracle/kv_fp8.py).  fp8
pools are head-major, [num_blocks, num_kv_heads, block_size, head_dim].

* The quantising append is compared bit for bit with the oracle's codes over
  every bf16 bit pattern, for several scales (powers of two and not).  A NaN
  input must store a NaN code (0x7F or 0xFF: the format has two and no page
  picks one); every other code must match exactly.
* Decode over fp8 pools is compared with oracle.decode_fp8 at the decode
  tolerance, over the same shape matrix as bf16 decode (head_dim, group,
  block size, split counts, ragged and empty sequences) and at the full
  sizes of the single-token workloads on sampled rows.
* With power-of-two scales, decode over fp8 codes and decode over a bf16 pool
  holding the codes' values times the scales run the same arithmetic on the
  matrix path (group of 3 or more); their outputs must agree bit for bit.
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


def u8_tensor(a: np.ndarray, device=DEV) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def device_pool8(inp: W.DecodeInputs, k8: np.ndarray, v8: np.ndarray, device=DEV):
    """Full fp8 pools on the device: NaN codes except the referenced blocks."""
    shape = (inp.pool.num_blocks,) + k8.shape[1:]
    k = torch.full(shape, int(W.E4M3_NAN), dtype=torch.uint8, device=device)
    v = torch.full(shape, int(W.E4M3_NAN), dtype=torch.uint8, device=device)
    ids = torch.from_numpy(inp.pool.ids).to(device)
    k.index_copy_(0, ids, u8_tensor(k8, device))
    v.index_copy_(0, ids, u8_tensor(v8, device))
    return k, v


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.0625, 4.0), (0.37, 0.0173),
                                             (3.1, 1e-3)])
def test_append_fp8_every_bf16_value(k_scale, v_scale):
    T, Hkv, D, NB, BS = 128, 4, 128, 16, 16
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    k = allbits.reshape(T, Hkv, D)
    v = allbits[::-1].copy().reshape(T, Hkv, D)
    rng = np.random.default_rng(5)
    slots = rng.permutation(NB * BS)[:T].astype(np.int64)
    slots[rng.choice(T, 9, replace=False)] = -1          # padding rows write nothing
    init = rng.integers(0, 256, (NB, Hkv, BS, D), dtype=np.uint8)     # head-major pool
    kc, vc = u8_tensor(init), u8_tensor(init)
    pa.reshape_and_cache_fp8(bf16_tensor(k), bf16_tensor(v), torch.from_numpy(slots).to(DEV),
                             kc, vc, k_scale, v_scale)
    torch.cuda.synchronize()
    want_k, want_v = O8.append_fp8(k, v, slots, init, init, k_scale, v_scale)
    for name, got, want, src in (("k", kc, want_k, k), ("v", vc, want_v, v)):
        got = got.cpu().numpy()
        # NaN inputs: any NaN code; the slots they land in
        src_f = W.bf16_bits_to_f32(src)
        nan_slot = np.zeros(got.shape, bool)
        for i, s in enumerate(slots):
            if s >= 0:
                nan_slot[s // BS, :, s % BS] = np.isnan(src_f[i])
        assert np.all((got[nan_slot] & 0x7F) == 0x7F), name
        diff = (got != want) & ~nan_slot
        assert not diff.any(), (name, np.argwhere(diff)[:5], got[diff][:5], want[diff][:5])


def test_append_fp8_then_decode_end_to_end():
    """A pool filled through the quantising append from bf16 rows, decoded:
    the device pool equals the oracle's bit for bit and the decode matches."""
    rng = np.random.default_rng(8)
    B, Hq, Hkv, D, BS, NB, WM = 5, 12, 2, 128, 16, 64, 12
    lens = np.array([1, 16, 37, 150, 191], np.int32)
    perm = rng.permutation(NB)
    tables = np.zeros((B, WM), np.int32)
    slots, off = [], 0
    for b, L in enumerate(lens):
        n = -(-int(L) // BS)
        tables[b, :n] = perm[off:off + n]
        off += n
        slots += [int(tables[b, t // BS]) * BS + t % BS for t in range(L)]
    slots = np.asarray(slots, np.int64)
    T = len(slots)
    kb = W.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32) * 3)
    vb = W.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32))
    ks, vs = 0.011, 0.0042
    init = np.full((NB, Hkv, BS, D), 0x7F, np.uint8)
    kc, vc = u8_tensor(init), u8_tensor(init)
    pa.reshape_and_cache_fp8(bf16_tensor(kb), bf16_tensor(vb), torch.from_numpy(slots).to(DEV),
                             kc, vc, ks, vs)
    k8, v8 = O8.append_fp8(kb, vb, slots, init, init, ks, vs)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), k8) and np.array_equal(vc.cpu().numpy(), v8)
    q = W.f32_to_bf16_bits(rng.standard_normal((B, Hq, D), dtype=np.float32))
    scale = np.float32(1 / np.sqrt(D))
    for S in (1, 3, 0):
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
        pa.decode_fp8(bf16_tensor(q), kc, vc, torch.from_numpy(tables).to(DEV),
                      torch.from_numpy(lens).to(DEV), float(scale), ks, vs, S, out)
        torch.cuda.synchronize()
        ref = O8.decode_fp8(q, k8, v8, tables, lens, scale, ks, vs)
        assert_close(to_f64(out), ref, what=f"S={S}")


# ---------------------------------------------------------------------------
# decode: shape matrix
# ---------------------------------------------------------------------------

LENS_MIX = (0, 1, 15, 16, 17, 255, 256, 257, 700, 1029)


def _small_spec(D, Hq, Hkv, bs, lens, seed):
    W_ = max(-(-max(lens) // bs), 1) + 1
    nb = sum(-(-L // bs) for L in lens) + 8
    return W.DecodeSpec(f"fp8-{D}-{Hq}-{Hkv}-{bs}", len(lens), Hq, Hkv, D, bs, nb, W_,
                        context_lens=tuple(lens), seed=seed)


def _run_fp8(inp, k8, v8, ks, vs, S):
    s = inp.spec
    kc, vc = device_pool8(inp, k8, v8)
    out = torch.empty((s.num_seqs, s.num_q_heads, s.head_dim), dtype=torch.bfloat16, device=DEV)
    pa.decode_fp8(bf16_tensor(inp.q), kc, vc, torch.from_numpy(inp.block_tables).to(DEV),
                  torch.from_numpy(inp.context_lens).to(DEV), float(inp.scale), ks, vs, S, out)
    torch.cuda.synchronize()
    return out


def _oracle_fp8(inp, k8, v8, ks, vs, rows=None):
    ct = inp.pool.compact_tables(inp.block_tables, inp.poison_block)
    if rows is None:
        return O8.decode_fp8(inp.q, k8, v8, ct, inp.context_lens, inp.scale, ks, vs)
    out = []
    for b in rows:
        out.append(O8.decode_fp8(inp.q[b:b + 1], k8, v8, ct[b:b + 1], inp.context_lens[b:b + 1],
                                 inp.scale, ks, vs)[0])
    return np.stack(out)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (6, 2), (8, 2), (16, 2)])
@pytest.mark.parametrize("bs", [16, 256])
def test_decode_fp8_shapes(D, Hq, Hkv, bs):
    inp = W.make_decode_inputs(_small_spec(D, Hq, Hkv, bs, LENS_MIX, seed=D + 7 * Hq + bs),
                               fill="zeros")
    k8, v8 = W.fp8_codes_like(inp)
    ks, vs = 0.21, 0.47
    ref = _oracle_fp8(inp, k8, v8, ks, vs)
    for S in (1, 2, 4, 0):     # S = 2: second pieces in mirrored unit order
        got = to_f64(_run_fp8(inp, k8, v8, ks, vs, S))
        assert_close(got, ref, what=f"D={D} Hq={Hq} Hkv={Hkv} bs={bs} S={S}")


def test_decode_fp8_many_splits_and_scales():
    inp = W.make_decode_inputs(_small_spec(128, 28, 4, 16, (3000, 1, 64, 2047), seed=31),
                               fill="zeros")
    k8, v8 = W.fp8_codes_like(inp)
    for ks, vs, S in ((2.0 ** -6, 16.0, 64), (0.9, 0.01, 17), (1.0, 1.0, 256)):
        ref = _oracle_fp8(inp, k8, v8, ks, vs)
        assert_close(to_f64(_run_fp8(inp, k8, v8, ks, vs, S)), ref, what=f"{ks} {vs} S={S}")


def test_decode_fp8_nan_code_in_context_propagates():
    inp = W.make_decode_inputs(_small_spec(128, 8, 2, 16, (40, 40), seed=41), fill="zeros")
    k8, v8 = W.fp8_codes_like(inp)
    ct = inp.pool.compact_tables(inp.block_tables, inp.poison_block)
    v8[ct[1, 1], 0, 3, 5] = 0xFF                   # sequence 1, token 19, kv head 0
    out = to_f64(_run_fp8(inp, k8, v8, 0.5, 0.5, 1))
    assert np.isnan(out[1, :4, 5]).all()           # the 4 q heads of kv head 0
    assert np.isfinite(out[0]).all() and np.isfinite(out[1, 4:]).all()


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 12, 4), (128, 16, 2), (64, 24, 4)])
def test_decode_fp8_equals_bf16_pool_of_its_values(D, Hq, Hkv):
    """Power-of-two scales: fp8 decode == bf16 decode over the dequantised
    pool, bit for bit (matrix path on both sides)."""
    inp = W.make_decode_inputs(_small_spec(D, Hq, Hkv, 16, LENS_MIX, seed=51 + D), fill="zeros")
    k8, v8 = W.fp8_codes_like(inp)
    ks, vs = 2.0 ** -3, 2.0 ** 2
    tm = lambda c: np.ascontiguousarray(np.transpose(c, (0, 2, 1, 3)))   # noqa: E731
    k8t, v8t = tm(k8), tm(v8)                       # token-major, the bf16 pool layout
    kb = W.f32_to_bf16_bits((O8.e4m3_decode(k8t) * ks).astype(np.float32))
    vb = W.f32_to_bf16_bits((O8.e4m3_decode(v8t) * vs).astype(np.float32))
    assert np.array_equal(W.bf16_bits_to_f32(kb).astype(np.float64)[k8t != 0x7F],
                          (O8.e4m3_decode(k8t) * ks)[k8t != 0x7F])      # exact in bf16
    for S in (1, 5):
        got8 = to_bits(_run_fp8(inp, k8, v8, ks, vs, S))
        pool = W.CompactPool(inp.pool.num_blocks, inp.pool.ids, kb, vb)
        shape = (pool.num_blocks,) + kb.shape[1:]
        nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
        kc = torch.full(shape, nan, dtype=torch.bfloat16, device=DEV)
        vc = torch.full(shape, nan, dtype=torch.bfloat16, device=DEV)
        ids = torch.from_numpy(pool.ids).to(DEV)
        kc.index_copy_(0, ids, bf16_tensor(kb))
        vc.index_copy_(0, ids, bf16_tensor(vb))
        out = torch.empty((len(LENS_MIX), Hq, D), dtype=torch.bfloat16, device=DEV)
        pa.decode(bf16_tensor(inp.q), kc, vc, torch.from_numpy(inp.block_tables).to(DEV),
                  torch.from_numpy(inp.context_lens).to(DEV), float(inp.scale), S, out)
        torch.cuda.synchronize()
        assert np.array_equal(got8, to_bits(out)), f"S={S}"


# ---------------------------------------------------------------------------
# decode: full-size workloads, sampled rows
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name", ["c2b8", "c3", "c5d"])
def test_decode_fp8_full_size_sampled(name):
    spec = W.CONFIGS[name].with_(append=False)
    inp = W.make_decode_inputs(spec, fill="zeros")
    k8, v8 = W.fp8_codes_like(inp)
    ks, vs = 0.3, 0.25
    got = to_f64(_run_fp8(inp, k8, v8, ks, vs, 0))
    rows = sorted(set(np.random.default_rng(61).choice(spec.num_seqs, 4, replace=False).tolist()))
    ref = _oracle_fp8(inp, k8, v8, ks, vs, rows)
    assert_close(got[rows], ref, what=name)


# ---------------------------------------------------------------------------
# multi-token decode over fp8 pools
# ---------------------------------------------------------------------------


def _run_multi_fp8(inp, q, k8, v8, ks, vs, S):
    s = inp.spec
    kc, vc = device_pool8(inp, k8, v8)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    pa.decode_multi_fp8(bf16_tensor(q), kc, vc, torch.from_numpy(inp.block_tables).to(DEV),
                        torch.from_numpy(inp.context_lens).to(DEV), float(inp.scale), ks, vs, S,
                        out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("D,Hq,Hkv,QL", [(128, 12, 2, 4), (128, 28, 4, 4), (128, 16, 2, 4),
                                         (64, 8, 2, 8), (128, 4, 4, 8), (64, 6, 2, 2)])
@pytest.mark.parametrize("bs", [16, 256])
def test_decode_multi_fp8(D, Hq, Hkv, QL, bs):
    """q_len query tokens (one or two tiles of 16 rows), causal inside the
    window, ragged lengths including sequences shorter than the window."""
    lens = (2, 5, 17, 300, 1029)
    inp = W.make_decode_inputs(_small_spec(D, Hq, Hkv, bs, lens, seed=900 + D + Hq + QL + bs),
                               fill="zeros")
    k8, v8 = W.fp8_codes_like(inp)
    q = W.f32_to_bf16_bits(np.random.default_rng(QL + Hq).standard_normal(
        (len(lens), QL, Hq, D), dtype=np.float32))
    ks, vs = 0.3, 0.2
    ct = inp.pool.compact_tables(inp.block_tables, inp.poison_block)
    ref = O8.decode_multi_fp8(q, k8, v8, ct, inp.context_lens, inp.scale, ks, vs)
    for S in (1, 3, 0):
        got = to_f64(_run_multi_fp8(inp, q, k8, v8, ks, vs, S))
        assert_close(got, ref, what=f"D={D} Hq={Hq} Hkv={Hkv} q_len={QL} bs={bs} S={S}")


def test_decode_multi_fp8_one_token_is_decode_fp8():
    """q_len 1 runs the single-token kernel: bit-identical to pa_decode_fp8."""
    inp = W.make_decode_inputs(_small_spec(128, 28, 4, 16, LENS_MIX, seed=77), fill="zeros")
    k8, v8 = W.fp8_codes_like(inp)
    q1 = inp.q[:, None]
    for S in (1, 5):
        a = to_bits(_run_multi_fp8(inp, q1, k8, v8, 0.4, 0.3, S))[:, 0]
        b = to_bits(_run_fp8(inp, k8, v8, 0.4, 0.3, S))
        assert np.array_equal(a, b), S


# ---------------------------------------------------------------------------
# chunked prefill over fp8 pools
# ---------------------------------------------------------------------------


class PrefillCase8:
    """A prompt chunk over an fp8 pool: the cached prefix holds random codes,
    the chunk's own K/V rows go in through the device's quantising append
    (and the oracle's on the host), then prefill runs."""

    def __init__(self, spec, ks, vs):
        inp = W.make_prefill_inputs(spec)
        self.inp, self.spec, self.ks, self.vs = inp, spec, ks, vs
        k8, v8 = W.fp8_codes_like(inp)
        self.k_cache, self.v_cache = device_pool8(inp, k8, v8)
        pa.reshape_and_cache_fp8(bf16_tensor(inp.new_k), bf16_tensor(inp.new_v),
                                 torch.from_numpy(inp.slot_mapping).to(DEV), self.k_cache,
                                 self.v_cache, ks, vs)
        bs = spec.block_size
        lut = {int(x): i for i, x in enumerate(inp.pool.ids)}
        slots = np.array([lut[int(s) // bs] * bs + int(s) % bs for s in inp.slot_mapping],
                         np.int64)
        k8, v8 = O8.append_fp8(inp.new_k, inp.new_v, slots, k8, v8, ks, vs)
        ct = inp.pool.compact_tables(inp.block_tables, inp.poison_block)
        self.ref = O8.prefill_fp8(inp.q, inp.cu_seqlens_q, k8, v8, ct, inp.context_lens,
                                  inp.scale, ks, vs)
        self.q = bf16_tensor(inp.q)
        self.cu = torch.from_numpy(inp.cu_seqlens_q).to(DEV)
        self.tables = torch.from_numpy(inp.block_tables).to(DEV)
        self.lens = torch.from_numpy(inp.context_lens).to(DEV)
        self.max_q = int(max(spec.chunk_lens))

    def run(self, S):
        out = torch.empty_like(self.q)
        pa.prefill_fp8(self.q, self.cu, self.k_cache, self.v_cache, self.tables, self.lens,
                       float(self.inp.scale), self.ks, self.vs, out, self.max_q, num_splits=S)
        torch.cuda.synchronize()
        return to_f64(out)


@pytest.mark.parametrize("D,G,bs,chunks,totals", [
    (128, 7, 256, (37, 1, 64), (300, 1, 64)),       # ragged; a 1-token chunk; prefix 0
    (128, 2, 16, (100, 33), (1000, 33)),
    (64, 1, 16, (65, 7), (129, 520)),
    (64, 8, 256, (31,), (2100,)),
    (128, 5, 16, (96,), (96,)),                       # whole prompt, no prefix
])
def test_prefill_fp8_shapes(D, G, bs, chunks, totals):
    W_ = -(-max(totals) // bs)
    nb = sum(-(-t // bs) for t in totals) + 5
    spec = W.PrefillSpec(f"p8{D}_{G}_{bs}", 2 * G, 2, D, bs, nb, W_, chunk_lens=chunks,
                         total_lens=totals, seed=D * 10 + G + 1)
    case = PrefillCase8(spec, 0.37, 0.029)
    for S in (1, 2, 0):
        assert_close(case.run(S), case.ref, what=f"fp8 prefill D{D} G{G} bs{bs} S{S}")


@pytest.mark.parametrize("S", [0, 3])
def test_prefill_fp8_chunk_512_of_4096(S):
    """The 512-token chunk over a 3584-token prefix (28 q / 4 kv heads, bs 256)
    on fp8 pools."""
    case = PrefillCase8(W.PREFILL_CONFIGS["c5p"], 0.5, 0.25)
    assert_close(case.run(S), case.ref, what=f"fp8 chunk512 S={S}")


# ---------------------------------------------------------------------------
# append fused into the decode launch, fp8 pools
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("D,Hq,Hkv,bs", [(128, 28, 4, 256), (128, 12, 2, 16), (64, 8, 8, 16),
                                         (64, 16, 2, 256)])
def test_append_decode_fp8_equals_separate_calls(D, Hq, Hkv, bs):
    """The fused quantising append + decode gives the pool bytes and the
    outputs of the quantising append followed by decode, bit for bit, and the
    oracle's values."""
    lens = (0, 1, 16, 17, 255, 256, 700)
    spec = _small_spec(D, Hq, Hkv, bs, lens, seed=3100 + D + Hq + bs).with_(append=True)
    inp = W.make_decode_inputs(spec, fill="zeros")
    k8, v8 = W.fp8_codes_like(inp)             # appended slots hold NaN codes
    ks, vs = 0.31, 0.043
    tables = torch.from_numpy(inp.block_tables).to(DEV)
    lens_t = torch.from_numpy(inp.context_lens).to(DEV)
    q = bf16_tensor(inp.q)
    sel = np.nonzero(inp.context_lens > 0)[0]
    nk = np.zeros((len(lens), Hkv, D), np.uint16)
    nv = np.zeros((len(lens), Hkv, D), np.uint16)
    nk[sel], nv[sel] = inp.new_k, inp.new_v
    for S in (1, 0):
        kc1, vc1 = device_pool8(inp, k8, v8)
        out1 = torch.empty((len(lens), Hq, D), dtype=torch.bfloat16, device=DEV)
        pa.append_decode_fp8(q, bf16_tensor(nk), bf16_tensor(nv), kc1, vc1, tables, lens_t,
                             float(inp.scale), ks, vs, S, out1)
        kc2, vc2 = device_pool8(inp, k8, v8)
        out2 = torch.empty_like(out1)
        pa.reshape_and_cache_fp8(bf16_tensor(inp.new_k), bf16_tensor(inp.new_v),
                                 torch.from_numpy(inp.slot_mapping).to(DEV), kc2, vc2, ks, vs)
        pa.decode_fp8(q, kc2, vc2, tables, lens_t, float(inp.scale), ks, vs, S, out2)
        torch.cuda.synchronize()
        assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2), S
        assert np.array_equal(to_bits(out1), to_bits(out2)), S
    bsz = spec.block_size
    lut = {int(x): i for i, x in enumerate(inp.pool.ids)}
    slots = np.array([lut[int(s) // bsz] * bsz + int(s) % bsz for s in inp.slot_mapping], np.int64)
    k8a, v8a = O8.append_fp8(inp.new_k, inp.new_v, slots, k8, v8, ks, vs)
    ref = _oracle_fp8(inp, k8a, v8a, ks, vs)
    assert_close(to_f64(out1), ref, what=f"fused fp8 D={D} Hq={Hq} Hkv={Hkv} bs={bs}")
