"""FP8 KV pages for the CPU oracle: the e4m3 code, the quantising append and
decode over fp8 pools.  fp64 numpy, plain and slow.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only the tests, the
smoke check and the benchmark's CPU baseline leg use it, and it shares no code
with the library.

What it computes, and where the pages state it: K/V pages stored quantised
(the Mini-Infer production-engine page lists several quantisation schemes
among its engine features; no page fixes one).  Readings taken (also in the
design notes): the OCP 8-bit floating-point format E4M3 (1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities, codes
0x7F / 0xFF are NaN, largest finite value 448); one fp32 scale per tensor (K
and V separately), the stored code being e4m3(clamp(x * (1 / scale),
-448, 448)) rounded to nearest even, with 1 / scale and the product taken in
fp32; the K and V a read uses are code value * scale.  Pools are head-major,
[num_blocks, num_kv_heads, block_size, head_dim]: slot s is row s % bs of
block s // bs for every kv head.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import attend, gather_sequence, kv_head_of

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> fp64 values (NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m * 2.0 ** -9
    nrm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    val = sign * np.where(e == 0, sub, nrm)
    return np.where((e == 15) & (c & 0x7 == 7), np.nan, val)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """fp32 values with |x| <= 448 (or NaN) -> uint8 codes, rounding to the
    nearest representable value, ties to even mantissa."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    out = np.zeros(x.shape, dtype=np.uint8)
    flat, res = x.ravel(), out.ravel()
    for i, v in enumerate(flat):
        if np.isnan(v):
            res[i] = 0x7F
            continue
        assert abs(v) <= E4M3_MAX, v
        s = 0x80 if np.signbit(v) else 0
        a = abs(v)
        if a < 2.0 ** -6:                              # subnormal range: steps of 2^-9
            code = int(np.rint(a / 2.0 ** -9))         # 8 rounds up into the first normal
        else:
            f, ex = np.frexp(a)                        # a = f 2^ex, 0.5 <= f < 1, exact
            e = int(ex) - 1
            m = int(np.rint((2.0 * f - 1.0) * 8.0))
            if m == 8:
                e, m = e + 1, 0
            code = ((e + 7) << 3) | m
        res[i] = s | code
    return out


def quantize(x_bf16_bits: np.ndarray, scale) -> np.ndarray:
    """bf16 bit patterns -> e4m3 codes of clamp(x * (1 / scale), +-448), the
    reciprocal and the product in fp32."""
    x = (np.asarray(x_bf16_bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore", invalid="ignore"):     # inf and NaN inputs
        y = np.clip(x * inv, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(y)


def token_major(pool8: np.ndarray) -> np.ndarray:
    """View of a head-major pool [NB, Hkv, bs, D] as [NB, bs, Hkv, D], the
    layout the shared gather reads."""
    return np.transpose(pool8, (0, 2, 1, 3))


def append_fp8(new_k: np.ndarray, new_v: np.ndarray, slot_mapping: np.ndarray,
               k_cache8: np.ndarray, v_cache8: np.ndarray, k_scale, v_scale):
    """Copies of the fp8 pools [NB, Hkv, bs, D] with row i of new_k / new_v
    ([T, Hkv, D] bf16 bits), quantised, written to slot slot_mapping[i] of
    every kv head; negative slots skip."""
    kc, vc = k_cache8.copy(), v_cache8.copy()
    bs = kc.shape[2]
    for i, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0:
            continue
        kc[s // bs, :, s % bs] = quantize(new_k[i], k_scale)
        vc[s // bs, :, s % bs] = quantize(new_v[i], v_scale)
    return kc, vc


def _sequence_kv(k_cache8, v_cache8, table, L, ks, vs):
    """K and V of a sequence's first L tokens (token-major pool views), as
    code value times scale, fp64 [L, Hkv, D]."""
    K = e4m3_decode(gather_sequence(k_cache8, table, L)) * ks
    V = e4m3_decode(gather_sequence(v_cache8, table, L)) * vs
    return K, V


def decode_fp8(q: np.ndarray, k_cache8: np.ndarray, v_cache8: np.ndarray,
               block_tables: np.ndarray, context_lens: np.ndarray, scale, k_scale,
               v_scale) -> np.ndarray:
    """Decode over fp8 pools [NB, Hkv, bs, D]: K = code value * k_scale,
    V = code value * v_scale (scales widened from fp32), then plain attention.
    q bf16 bits [B, Hq, D]; returns fp64 [B, Hq, D]."""
    B, Hq, D = q.shape
    Hkv = k_cache8.shape[1]
    k_cache8, v_cache8 = token_major(k_cache8), token_major(v_cache8)
    sc = np.float64(np.float32(scale))
    ks, vs = np.float64(np.float32(k_scale)), np.float64(np.float32(v_scale))
    qf = (np.asarray(q, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32) \
        .astype(np.float64)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        K, V = _sequence_kv(k_cache8, v_cache8, block_tables[b], L, ks, vs)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[b, h] = attend(qf[b, h], K[:, g, :], V[:, g, :], sc)
    return out


def decode_multi_fp8(q: np.ndarray, k_cache8: np.ndarray, v_cache8: np.ndarray,
                     block_tables: np.ndarray, context_lens: np.ndarray, scale, k_scale,
                     v_scale) -> np.ndarray:
    """Multi-token decode over fp8 pools [NB, Hkv, bs, D]: q bf16 bits
    [B, q_len, Hq, D]; query token j of sequence b sits at position
    context_lens[b] - q_len + j and attends the dequantised keys up to it
    (none when the position is negative).  Returns fp64 [B, q_len, Hq, D]."""
    B, QL, Hq, D = q.shape
    Hkv = k_cache8.shape[1]
    k_cache8, v_cache8 = token_major(k_cache8), token_major(v_cache8)
    sc = np.float64(np.float32(scale))
    ks, vs = np.float64(np.float32(k_scale)), np.float64(np.float32(v_scale))
    qf = (np.asarray(q, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32) \
        .astype(np.float64)
    out = np.zeros((B, QL, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        K, V = _sequence_kv(k_cache8, v_cache8, block_tables[b], L, ks, vs)
        for j in range(QL):
            p = L - QL + j
            n_keys = p + 1 if p >= 0 else 0
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                out[b, j, h] = attend(qf[b, j, h], K[:n_keys, g, :], V[:n_keys, g, :], sc)
    return out


def prefill_fp8(q: np.ndarray, cu_seqlens_q: np.ndarray, k_cache8: np.ndarray,
                v_cache8: np.ndarray, block_tables: np.ndarray, context_lens: np.ndarray,
                scale, k_scale, v_scale) -> np.ndarray:
    """Chunked prefill over fp8 pools [NB, Hkv, bs, D]: q bf16 bits [Tq, Hq, D]
    packed by cu_seqlens_q [B + 1]; context_lens [B] are total lengths (cached
    prefix + chunk, the chunk's K/V already in the pool); query i of an n-row
    chunk sits at position L - n + i and attends the dequantised keys up to it.
    Returns fp64 [Tq, Hq, D]."""
    Tq, Hq, D = q.shape
    Hkv = k_cache8.shape[1]
    k_cache8, v_cache8 = token_major(k_cache8), token_major(v_cache8)
    sc = np.float64(np.float32(scale))
    ks, vs = np.float64(np.float32(k_scale)), np.float64(np.float32(v_scale))
    qf = (np.asarray(q, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32) \
        .astype(np.float64)
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    for b in range(len(context_lens)):
        L = int(context_lens[b])
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        n = q1 - q0
        K, V = _sequence_kv(k_cache8, v_cache8, block_tables[b], L, ks, vs)
        for i in range(n):
            p = L - n + i
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                out[q0 + i, h] = attend(qf[q0 + i, h], K[:p + 1, g, :], V[:p + 1, g, :], sc)
    return out
