"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each ``pin_*`` function takes the oracle module, runs it on a small seeded
case and raises AssertionError when the result disagrees with brute force, a
library routine, a closed form or an invariant.  ``tests/test_oracle.py`` runs
them against the real oracle, and against copies with planted mistakes to
show that every plausible slip is caught by at least one pin.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import workloads as W


def _logical_case(rng, lens, Hq, Hkv, D):
    """Random logical (contiguous) K/V per sequence plus q, as bf16 bits."""
    Ks = [W.f32_to_bf16_bits(rng.standard_normal((L, Hkv, D), dtype=np.float32)) for L in lens]
    Vs = [W.f32_to_bf16_bits(rng.standard_normal((L, Hkv, D), dtype=np.float32)) for L in lens]
    q = W.f32_to_bf16_bits(rng.standard_normal((len(lens), Hq, D), dtype=np.float32))
    return q, Ks, Vs


def _page_blockwise(rng, seqs, bs, num_blocks, extra_poison=True):
    """Place logical sequences into a shuffled block pool by copying whole
    blocks (numpy slicing, not per-token indexing).  Returns pool, tables."""
    Hkv, D = seqs[0].shape[1:]
    pool = np.full((num_blocks, bs, Hkv, D), W.BF16_NAN, dtype=np.uint16)
    perm = rng.permutation(num_blocks)
    nblk = [(len(s) + bs - 1) // bs for s in seqs]
    width = max(max(nblk), 1)
    poison = int(perm[-1])
    tables = np.full((len(seqs), width), poison, dtype=np.int32)
    off = 0
    for b, s in enumerate(seqs):
        for j in range(nblk[b]):
            phys = int(perm[off])
            off += 1
            tables[b, j] = phys
            piece = s[j * bs:(j + 1) * bs]
            pool[phys, :len(piece)] = piece
    assert off < num_blocks
    return pool, tables


def _f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _sdpa_decode(q, Ks, Vs, scale):
    """torch fp64 scaled_dot_product_attention on contiguous K/V, GQA by
    torch's own head repetition."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        if len(Ks[b]) == 0:
            continue
        qt = torch.from_numpy(_f64(q[b]))[:, None, :]                   # [Hq, 1, D]
        kt = torch.from_numpy(_f64(Ks[b])).permute(1, 0, 2).contiguous()  # [Hkv, L, D]
        vt = torch.from_numpy(_f64(Vs[b])).permute(1, 0, 2).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(
            qt[None], kt[None], vt[None], scale=float(scale), enable_gqa=True)[0]
        out[b] = o[:, 0, :].numpy()
    return out


# ---------------------------------------------------------------------------


def pin_sdpa_decode(oracle, seed=11):
    """P1: paged oracle == library SDPA on the contiguous logical K/V."""
    rng = np.random.default_rng(seed)
    for (lens, Hq, Hkv, D, bs) in [((1, 5, 40, 17), 6, 2, 8, 4), ((33, 16), 3, 3, 4, 16),
                                   ((9, 2, 31), 7, 1, 16, 2)]:
        q, Ks, Vs = _logical_case(rng, lens, Hq, Hkv, D)
        nb = sum((L + bs - 1) // bs for L in lens) + 3
        kp, tables = _page_blockwise(np.random.default_rng(seed + 1), Ks, bs, nb)
        vp, tables_v = _page_blockwise(np.random.default_rng(seed + 1), Vs, bs, nb)
        assert (tables == tables_v).all()
        scale = np.float32(0.3)
        got = oracle.decode(q, kp, vp, tables, np.array(lens, np.int32), scale)
        ref = _sdpa_decode(q, Ks, Vs, np.float64(scale))
        assert np.abs(got - ref).max() < 1e-12, np.abs(got - ref).max()


def pin_loops_decode(oracle, seed=12):
    """P1: paged oracle == explicit Python loops over a contiguous cache
    (math.exp, running sums, no numpy reductions)."""
    rng = np.random.default_rng(seed)
    lens, Hq, Hkv, D, bs = (3, 7, 1), 4, 2, 3, 2
    q, Ks, Vs = _logical_case(rng, lens, Hq, Hkv, D)
    nb = 10
    kp, tables = _page_blockwise(np.random.default_rng(5), Ks, bs, nb)
    vp, _ = _page_blockwise(np.random.default_rng(5), Vs, bs, nb)
    scale = 0.7
    got = oracle.decode(q, kp, vp, tables, np.array(lens, np.int32), np.float32(scale))
    sc = float(np.float32(scale))
    for b, L in enumerate(lens):
        K, V, qq = _f64(Ks[b]), _f64(Vs[b]), _f64(q[b])
        for h in range(Hq):
            g = h // (Hq // Hkv)
            scores = []
            for t in range(L):
                dot = 0.0
                for d in range(D):
                    dot += qq[h, d] * K[t, g, d]
                scores.append(sc * dot)
            mx = max(scores)
            den = sum(math.exp(s - mx) for s in scores)
            for d in range(D):
                num = sum(math.exp(scores[t] - mx) * V[t, g, d] for t in range(L))
                assert abs(got[b, h, d] - num / den) < 1e-13


def pin_two_token_closed_form(oracle):
    """Two keys: out = (v0 + e^D v1) / (1 + e^D) with D = scale * q.(k1 - k0)."""
    D_ = 4
    q = np.array([[[1.0, 2.0, -1.0, 0.5]]], np.float32)
    k = np.array([[0.5, 0.0, 1.0, 2.0], [-1.0, 1.0, 0.25, 4.0]], np.float32)
    v = np.array([[1.0, -2.0, 3.0, 0.125], [4.0, 0.5, -1.0, 8.0]], np.float32)
    bs = 4
    pool_k = np.full((3, bs, 1, D_), W.BF16_NAN, np.uint16)
    pool_v = pool_k.copy()
    pool_k[2, :2, 0] = W.f32_to_bf16_bits(k)
    pool_v[2, :2, 0] = W.f32_to_bf16_bits(v)
    scale = np.float32(0.5)
    got = oracle.decode(W.f32_to_bf16_bits(q), pool_k, pool_v, np.array([[2]], np.int32),
                        np.array([2], np.int32), scale)
    s0 = 0.5 * (1 * 0.5 + 2 * 0 - 1 * 1 + 0.5 * 2)      # = 0.25
    s1 = 0.5 * (1 * -1 + 2 * 1 - 1 * 0.25 + 0.5 * 4)    # = 1.375
    e = math.exp(s1 - s0)
    want = [(float(v[0, d]) + e * float(v[1, d])) / (1 + e) for d in range(D_)]
    assert np.abs(got[0, 0] - np.array(want)).max() < 1e-14


def pin_permutation(oracle, seed=13):
    """P2: relabelling physical blocks (pool'[pi(i)] = pool[i], tables' =
    pi(tables)) leaves the output bit-identical."""
    inp = W.make_decode_inputs(W.CONFIGS["c1"].with_(seed=seed))
    kf, vf = inp.pool.full()
    base = oracle.decode(inp.q, kf, vf, inp.block_tables, inp.context_lens, inp.scale)
    pi = np.random.default_rng(seed).permutation(kf.shape[0])
    k2 = np.empty_like(kf)
    v2 = np.empty_like(vf)
    k2[pi] = kf
    v2[pi] = vf
    out = oracle.decode(inp.q, k2, v2, pi[inp.block_tables].astype(np.int32), inp.context_lens,
                        inp.scale)
    assert np.array_equal(base, out)


def pin_block_size(oracle, seed=14):
    """P3: the same logical KV paged with block sizes 1, 16 and 256 gives the
    same output."""
    rng = np.random.default_rng(seed)
    lens, Hq, Hkv, D = (1, 17, 300), 4, 2, 8
    q, Ks, Vs = _logical_case(rng, lens, Hq, Hkv, D)
    outs = []
    for bs in (1, 16, 256):
        nb = sum((L + bs - 1) // bs for L in lens) + 2
        kp, tables = _page_blockwise(np.random.default_rng(bs), Ks, bs, nb)
        vp, _ = _page_blockwise(np.random.default_rng(bs), Vs, bs, nb)
        outs.append(oracle.decode(q, kp, vp, tables, np.array(lens, np.int32), np.float32(0.25)))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


def pin_ctx1_returns_v(oracle):
    """P4: a single cached token gets weight exactly 1: out == V[0]."""
    inp = W.make_decode_inputs(W.CONFIGS["c1"])
    kf, vf = inp.pool.full()
    out = oracle.decode(inp.q, kf, vf, inp.block_tables, inp.context_lens, inp.scale)
    b = int(np.nonzero(inp.context_lens == 1)[0][0])
    v0 = _f64(vf[inp.block_tables[b, 0], 0, 0])
    assert np.array_equal(out[b, 0], v0) and np.array_equal(out[b, 1], v0)


def pin_constant_v(oracle):
    """P5: V == c everywhere gives out == c (weights sum to one)."""
    inp = W.make_decode_inputs(W.CONFIGS["c1"])
    kf, vf = inp.pool.full()
    vf = np.where(np.isnan(_f64(vf)), vf, W.f32_to_bf16_bits(np.float32(0.75))).astype(np.uint16)
    out = oracle.decode(inp.q, kf, vf, inp.block_tables, inp.context_lens, inp.scale)
    assert np.abs(out - 0.75).max() < 1e-15


def pin_histogram(oracle):
    """P6: with K == 0 every weight is 1/L; with V[t, d] = [d == t mod D] the
    output is out[h, d] = #{t < L : t mod D = d} / L exactly - a dropped,
    repeated or misplaced token moves some bin."""
    spec = W.CONFIGS["c1"]
    inp = W.make_decode_inputs(spec)
    kf, vf = inp.pool.full()
    kf = np.where(np.isnan(_f64(kf)), kf, np.uint16(0)).astype(np.uint16)
    D, bs = spec.head_dim, spec.block_size
    for b, L in enumerate(inp.context_lens):
        for t in range(int(L)):
            blk = inp.block_tables[b, t // bs]
            vf[blk, t % bs, :, :] = 0
            vf[blk, t % bs, :, t % D] = W.BF16_ONE
    out = oracle.decode(inp.q, kf, vf, inp.block_tables, inp.context_lens, inp.scale)
    for b, L in enumerate(inp.context_lens):
        L = int(L)
        want = np.array([len(range(d, L, D)) / L for d in range(D)])
        for h in range(spec.num_q_heads):
            assert np.abs(out[b, h] - want).max() < 1e-15


def pin_gqa_mapping(oracle):
    """P7: V == c_g on kv head g gives out[h] == c_{h // (Hq/Hkv)}."""
    spec = W.DecodeSpec("gqa", 3, 12, 4, 8, 4, 40, 8, context_lens=(5, 1, 29), seed=77)
    inp = W.make_decode_inputs(spec)
    kf, vf = inp.pool.full()
    consts = [0.5, -1.25, 2.0, 3.5]
    for g, c in enumerate(consts):
        vf[:, :, g, :] = np.where(np.isnan(_f64(vf[:, :, g, :])), vf[:, :, g, :],
                                  W.f32_to_bf16_bits(np.float32(c)))
    out = oracle.decode(inp.q, kf, vf, inp.block_tables, inp.context_lens, inp.scale)
    for h in range(12):
        assert np.abs(out[:, h] - consts[h // 3]).max() < 1e-15


def pin_poison_untouched(oracle):
    """P9: pools full of NaN outside the referenced tokens give a finite output."""
    for name in ("c1",):
        inp = W.make_decode_inputs(W.CONFIGS[name])
        kf, vf = inp.pool.full()
        out = oracle.decode(inp.q, kf, vf, inp.block_tables, inp.context_lens, inp.scale)
        assert np.isfinite(out).all()


def pin_empty_sequence(oracle):
    """A sequence with no cached tokens reads nothing and gives zeros."""
    inp = W.make_decode_inputs(W.CONFIGS["c1"].with_(context_lens=(0, 17, 0, 3)))
    kf, vf = inp.pool.full()
    out = oracle.decode(inp.q, kf, vf, inp.block_tables, inp.context_lens, inp.scale)
    assert (out[0] == 0).all() and (out[2] == 0).all() and np.isfinite(out).all()


def pin_append(oracle, seed=15):
    """P10: writing each token of logical sequences through its slot into an
    all-NaN pool, one call per token, rebuilds those sequences when read back
    block by block; negative slots write nothing; untouched bytes keep their
    values."""
    rng = np.random.default_rng(seed)
    bs, Hkv, D, nb = 4, 2, 3, 12
    lens = (6, 9)
    _, Ks, Vs = _logical_case(rng, lens, 1, Hkv, D)
    perm = rng.permutation(nb)
    tables = np.array([perm[0:2], perm[2:5]], dtype=object)
    kc = np.full((nb, bs, Hkv, D), W.BF16_NAN, np.uint16)
    vc = kc.copy()
    kc[perm[-1]] = 7    # a block no slot targets keeps its contents
    vc[perm[-1]] = 9
    for t in range(max(lens)):
        rows_k, rows_v, slots = [], [], []
        for b, L in enumerate(lens):
            if t < L:
                rows_k.append(Ks[b][t]); rows_v.append(Vs[b][t])
                slots.append(int(tables[b][t // bs]) * bs + t % bs)
            rows_k.append(np.zeros((Hkv, D), np.uint16)); rows_v.append(rows_k[-1])
            slots.append(-1)                     # padding row: skipped
        kc, vc = oracle.append(np.stack(rows_k), np.stack(rows_v), np.array(slots), kc, vc)
    for b, L in enumerate(lens):
        blocks_k = np.concatenate([kc[int(p)] for p in tables[b]])[:L]
        blocks_v = np.concatenate([vc[int(p)] for p in tables[b]])[:L]
        assert np.array_equal(blocks_k, Ks[b]) and np.array_equal(blocks_v, Vs[b])
    assert (kc[perm[-1]] == 7).all() and (vc[perm[-1]] == 9).all()
    # everything no slot addressed is still NaN
    written = np.zeros((nb, bs), bool)
    for b, L in enumerate(lens):
        for t in range(L):
            written[int(tables[b][t // bs]), t % bs] = True
    written[perm[-1]] = True
    assert (kc[~written] == W.BF16_NAN).all()


def _sdpa_causal(qb, Kb, Vb, scale):
    qt = torch.from_numpy(_f64(qb)).permute(1, 0, 2).contiguous()[None]   # [1, Hq, n, D]
    kt = torch.from_numpy(_f64(Kb)).permute(1, 0, 2).contiguous()[None]
    vt = torch.from_numpy(_f64(Vb)).permute(1, 0, 2).contiguous()[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                         scale=float(scale), enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


def pin_prefill(oracle, seed=16):
    """P11: (a) an empty prefix is ordinary causal attention (library SDPA,
    is_causal); (b) a one-token chunk equals decode; (c) processing a prompt as
    consecutive chunks gives the same rows as one whole-prompt chunk."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs, L = 6, 2, 8, 4, 23
    q, Ks, Vs = _logical_case(rng, (L,), Hq, Hkv, D)
    qs = W.f32_to_bf16_bits(rng.standard_normal((L, Hq, D), dtype=np.float32))
    kp, tables = _page_blockwise(np.random.default_rng(3), Ks, bs, 9)
    vp, _ = _page_blockwise(np.random.default_rng(3), Vs, bs, 9)
    sc = np.float32(0.4)
    lens = np.array([L], np.int32)
    whole = oracle.prefill(qs, np.array([0, L], np.int32), kp, vp, tables, lens, sc)
    ref = _sdpa_causal(qs, Ks[0], Vs[0], np.float64(sc))
    assert np.abs(whole - ref).max() < 1e-12
    # (c) chunks [0,5), [5,12), [12,23): each chunk sees the prefix before it
    for a, b_ in ((0, 5), (5, 12), (12, 23)):
        part = oracle.prefill(qs[a:b_], np.array([0, b_ - a], np.int32), kp, vp, tables,
                              np.array([b_], np.int32), sc)
        assert np.abs(part - whole[a:b_]).max() < 1e-13
    # (b) one-token chunk at the end == decode with the same q
    one = oracle.prefill(qs[L - 1:L], np.array([0, 1], np.int32), kp, vp, tables, lens, sc)
    dec = oracle.decode(qs[L - 1:L], kp, vp, tables, lens, sc)
    assert np.array_equal(one, dec)


def _sdpa_window(qb, Kb, Vb, scale):
    """torch fp64 SDPA of a window of query tokens at the end of one logical
    sequence: qb [QL, Hq, D], Kb/Vb [L, Hkv, D] (bf16 bits, L >= QL); token j
    may see keys 0 .. L - QL + j (explicit boolean mask)."""
    QL, Hq, D = qb.shape
    L, Hkv, _ = Kb.shape
    G = Hq // Hkv
    qt = torch.from_numpy(_f64(qb)).permute(1, 0, 2)[None]                         # [1, Hq, QL, D]
    kt = torch.from_numpy(_f64(Kb)).permute(1, 0, 2).repeat_interleave(G, 0)[None]  # [1, Hq, L, D]
    vt = torch.from_numpy(_f64(Vb)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    mask = torch.arange(L)[None, :] <= (L - QL + torch.arange(QL))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                         scale=float(scale))
    return o[0].permute(1, 0, 2).numpy()


def pin_decode_multi(oracle, seed=17):
    """P12: several query tokens per sequence (the speculative verify step):
    (a) against a masked library SDPA on the contiguous sequence, GQA by
    torch's head repetition, for ragged lengths and 4 query tokens; (b) one
    query token is decode, exactly; (c) a sequence shorter than its window:
    tokens before position 0 give zero rows, the token at position 0 returns
    V[0] exactly."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs, QL = 6, 2, 8, 4, 4
    lens = (4, 9, 17)
    _, Ks, Vs = _logical_case(rng, lens, Hq, Hkv, D)
    q = W.f32_to_bf16_bits(rng.standard_normal((len(lens), QL, Hq, D), dtype=np.float32))
    kp, tables = _page_blockwise(np.random.default_rng(4), Ks, bs, 16)
    vp, _ = _page_blockwise(np.random.default_rng(4), Vs, bs, 16)
    sc = np.float32(0.3)
    lens_a = np.array(lens, np.int32)
    got = oracle.decode_multi(q, kp, vp, tables, lens_a, sc)
    for b in range(len(lens)):
        ref = _sdpa_window(q[b], Ks[b], Vs[b], np.float64(sc))
        assert np.abs(got[b] - ref).max() < 1e-12, b
    one = oracle.decode_multi(q[:, :1], kp, vp, tables, lens_a, sc)
    assert np.array_equal(one[:, 0], oracle.decode(q[:, 0], kp, vp, tables, lens_a, sc))
    short = oracle.decode_multi(q[:1], kp, vp, tables, np.array([2], np.int32), sc)
    assert np.array_equal(short[0, :2], np.zeros((2, Hq, D)))
    for h in range(Hq):
        assert np.array_equal(short[0, 2, h], _f64(Vs[0][0, h // (Hq // Hkv)]))


ALL_PINS = [pin_sdpa_decode, pin_loops_decode, pin_two_token_closed_form, pin_permutation,
            pin_block_size, pin_ctx1_returns_v, pin_constant_v, pin_histogram, pin_gqa_mapping,
            pin_poison_untouched, pin_empty_sequence, pin_append, pin_prefill, pin_decode_multi]


# --------------------------------------------------------------------------
# FP8 KV pages (oracle/kv_fp8.py): pins take that module
# --------------------------------------------------------------------------

def _torch_e4m3(x32: np.ndarray) -> np.ndarray:
    """Library routine: torch's float8_e4m3fn conversion (round to nearest
    even), as uint8 codes."""
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def pin_fp8_codec(kv):
    """F1: every code decodes to torch's float8_e4m3fn value; encoding equals
    torch's conversion on every bf16 value in [-448, 448], on ties and on
    subnormals; every finite code survives a round trip."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = kv.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(ref)], ref[~np.isnan(ref)])
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 448)]
    assert np.array_equal(kv.e4m3_encode(x), _torch_e4m3(x))
    finite = ref[~np.isnan(ref)]
    mids = (np.sort(np.unique(finite))[1:] + np.sort(np.unique(finite))[:-1]) / 2   # exact ties
    ties = mids.astype(np.float32)
    ties = ties[ties.astype(np.float64) == mids]
    assert np.array_equal(kv.e4m3_encode(ties), _torch_e4m3(ties))
    fc = codes[~np.isnan(ref)]
    back = kv.e4m3_encode(kv.e4m3_decode(fc).astype(np.float32))
    zero = (fc == 0x80)                                   # -0 keeps its sign
    assert np.array_equal(back[~zero], fc[~zero]) and (back[zero] == 0x80).all()


def pin_fp8_quantize_and_append(kv, seed=18):
    """F2: the appended codes are torch's conversion of clamp(x * (1/scale))
    with the reciprocal and product in fp32, written at the slots of the
    head-major pools [NB, Hkv, bs, D] (negative slots skip)."""
    rng = np.random.default_rng(seed)
    Hkv, D, bs, NB = 2, 8, 4, 6
    nk = W.f32_to_bf16_bits(rng.standard_normal((5, Hkv, D), dtype=np.float32) * 300)
    nv = W.f32_to_bf16_bits(rng.standard_normal((5, Hkv, D), dtype=np.float32))
    kc = np.full((NB, Hkv, bs, D), 0x7F, np.uint8)
    vc = kc.copy()
    slots = np.array([3, -1, 9, 22, 4], np.int64)
    ks, vs = np.float32(0.37), np.float32(0.011)
    k2, v2 = kv.append_fp8(nk, nv, slots, kc, vc, ks, vs)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        for new, cache, sc in ((nk, k2, ks), (nv, v2, vs)):
            x = (new[i].astype(np.uint32) << np.uint32(16)).view(np.float32)
            y = np.clip(x * (np.float32(1) / sc), np.float32(-448), np.float32(448))
            for h in range(Hkv):
                assert np.array_equal(cache[s // bs, h, s % bs], _torch_e4m3(y[h]))
    untouched = np.ones((NB, Hkv, bs), bool)
    for s in slots[slots >= 0]:
        untouched[s // bs, :, s % bs] = False
    assert (k2[untouched] == 0x7F).all() and (v2[untouched] == 0x7F).all()
    assert (k2[~untouched] != 0x7F).any()
    # values beyond the range clamp to the largest finite code
    big = W.f32_to_bf16_bits(np.array([1e6, -1e6], np.float32))
    assert kv.quantize(big, np.float32(1.0)).tolist() == [0x7E, 0xFE]


def pin_fp8_decode_reduces_to_bf16(kv, seed=19):
    """F3: with power-of-two scales every dequantised value is exactly a bf16
    value, so decode over fp8 pools equals the (pinned) bf16 decode over the
    dequantised pools, bit for bit (the fp8 pools head-major
    [NB, Hkv, bs, D], the bf16 ones [NB, bs, Hkv, D])."""
    import oracle.paged_attention as pa_oracle
    rng = np.random.default_rng(seed)
    NB, bs, Hkv, D, B, Hq = 12, 4, 2, 8, 3, 6
    codes = rng.integers(0, 256, (NB, bs, Hkv, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                  # no NaN codes
    vcodes = rng.integers(0, 256, (NB, bs, Hkv, D)).astype(np.uint8)
    vcodes[(vcodes & 0x7F) == 0x7F] = 0x40
    ks, vs = 2.0 ** -4, 2.0 ** 3
    kbf = W.f32_to_bf16_bits((kv.e4m3_decode(codes) * ks).astype(np.float32))
    vbf = W.f32_to_bf16_bits((kv.e4m3_decode(vcodes) * vs).astype(np.float32))
    assert np.array_equal(_f64(kbf), kv.e4m3_decode(codes) * ks)       # exact in bf16
    tables = rng.permutation(NB)[:B * 4].reshape(B, 4).astype(np.int32)
    lens = np.array([1, 9, 16], np.int32)
    q = W.f32_to_bf16_bits(rng.standard_normal((B, Hq, D), dtype=np.float32))
    hm = lambda c: np.ascontiguousarray(np.transpose(c, (0, 2, 1, 3)))   # noqa: E731
    got = kv.decode_fp8(q, hm(codes), hm(vcodes), tables, lens, np.float32(0.3), ks, vs)
    want = pa_oracle.decode(q, kbf, vbf, tables, lens, np.float32(0.3))
    assert np.array_equal(got, want)


def pin_fp8_decode_multi(kv, seed=20):
    """F4: multi-token decode over fp8 pools - with power-of-two scales it
    equals the (pinned) bf16 multi-token decode over the dequantised pools
    bit for bit, and with one query token it equals fp8 decode exactly."""
    import oracle.paged_attention as pa_oracle
    rng = np.random.default_rng(seed)
    NB, bs, Hkv, D, B, Hq, QL = 12, 4, 2, 8, 3, 6, 3
    codes = rng.integers(0, 256, (NB, Hkv, bs, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    vcodes = rng.integers(0, 256, (NB, Hkv, bs, D)).astype(np.uint8)
    vcodes[(vcodes & 0x7F) == 0x7F] = 0x40
    ks, vs = 2.0 ** -3, 2.0 ** 2
    tm = lambda c: np.ascontiguousarray(np.transpose(c, (0, 2, 1, 3)))   # noqa: E731
    kbf = W.f32_to_bf16_bits((kv.e4m3_decode(tm(codes)) * ks).astype(np.float32))
    vbf = W.f32_to_bf16_bits((kv.e4m3_decode(tm(vcodes)) * vs).astype(np.float32))
    tables = rng.permutation(NB)[:B * 4].reshape(B, 4).astype(np.int32)
    lens = np.array([2, 9, 16], np.int32)                    # the first shorter than q_len
    q = W.f32_to_bf16_bits(rng.standard_normal((B, QL, Hq, D), dtype=np.float32))
    got = kv.decode_multi_fp8(q, codes, vcodes, tables, lens, np.float32(0.3), ks, vs)
    want = pa_oracle.decode_multi(q, kbf, vbf, tables, lens, np.float32(0.3))
    assert np.array_equal(got, want)
    assert (got[0, 0] == 0).all()                            # position -1: no keys
    one = kv.decode_multi_fp8(q[:, :1], codes, vcodes, tables, lens, np.float32(0.3), 0.37, 0.011)
    dec = kv.decode_fp8(q[:, 0], codes, vcodes, tables, lens, np.float32(0.3), 0.37, 0.011)
    assert np.array_equal(one[:, 0], dec)


def pin_fp8_prefill(kv, seed=21):
    """F5: chunked prefill over fp8 pools - with power-of-two scales it equals
    the (pinned) bf16 prefill over the dequantised pools bit for bit; a
    one-row chunk equals fp8 decode exactly."""
    import oracle.paged_attention as pa_oracle
    rng = np.random.default_rng(seed)
    NB, bs, Hkv, D, Hq = 12, 4, 2, 8, 6
    codes = rng.integers(0, 256, (NB, Hkv, bs, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30
    vcodes = rng.integers(0, 256, (NB, Hkv, bs, D)).astype(np.uint8)
    vcodes[(vcodes & 0x7F) == 0x7F] = 0x44
    ks, vs = 2.0 ** 2, 2.0 ** -5
    tm = lambda c: np.ascontiguousarray(np.transpose(c, (0, 2, 1, 3)))   # noqa: E731
    kbf = W.f32_to_bf16_bits((kv.e4m3_decode(tm(codes)) * ks).astype(np.float32))
    vbf = W.f32_to_bf16_bits((kv.e4m3_decode(tm(vcodes)) * vs).astype(np.float32))
    tables = rng.permutation(NB)[:8].reshape(2, 4).astype(np.int32)
    lens = np.array([13, 16], np.int32)
    cu = np.array([0, 5, 9], np.int32)                        # chunks of 5 and 4 rows
    q = W.f32_to_bf16_bits(rng.standard_normal((9, Hq, D), dtype=np.float32))
    got = kv.prefill_fp8(q, cu, codes, vcodes, tables, lens, np.float32(0.2), ks, vs)
    want = pa_oracle.prefill(q, cu, kbf, vbf, tables, lens, np.float32(0.2))
    assert np.array_equal(got, want)
    one = kv.prefill_fp8(q[:2], np.array([0, 1, 2], np.int32), codes, vcodes, tables, lens,
                         np.float32(0.2), 0.7, 0.3)
    dec = kv.decode_fp8(q[:2], codes, vcodes, tables, lens, np.float32(0.2), 0.7, 0.3)
    assert np.array_equal(one, dec)


FP8_PINS = [pin_fp8_codec, pin_fp8_quantize_and_append, pin_fp8_decode_reduces_to_bf16,
            pin_fp8_decode_multi, pin_fp8_prefill]
