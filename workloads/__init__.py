"""Seeded synthetic inputs for paged-KV attention, shared by the oracle tests,
the GPU parity tests and the benchmark.

This module holds no attention arithmetic.  It only draws numbers and lays
them out the way a paged KV cache stores them:

* a physical block pool ``[num_blocks, block_size, kv_heads, head_dim]`` of
  bf16 values (stored here as their raw ``uint16`` bit patterns), the layout of
  the fixed physical block pool in the mini-infer docs
  (prajwal7-2002.github.io/mini-infer, "Systems Architecture" figure, Paged
  KV-Cache Memory Manager box);
* a per-sequence block table (virtual block j -> physical block id), same
  figure, "Virtual-to-Physical Block Table per request";
* per-token slot ids (``slot = block * block_size + offset``) for the append,
  the "zero-overhead slot mapping" of the same page's "Core Capabilities at a
  Glance" table, row "Batched Paged Decode".

Values are fp32 N(0, 1) draws rounded to bf16 with round-to-nearest-even.
Every physical block draws from its own stream ``PCG64([seed, tag, block])``,
so a block's contents depend only on the seed and its id.  Pool storage that
no sequence references, cache slots past a sequence's length and padded
table entries are filled with NaN ("poison"), so a kernel that reads them
turns its output into NaN.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
BF16_ONE = np.uint16(0x3F80)

# Stream tags: each kind of draw gets its own SeedSequence branch.
_TAG_LENS, _TAG_PERM, _TAG_Q, _TAG_K, _TAG_V, _TAG_NEWK, _TAG_NEWV, _TAG_K8, _TAG_V8 = range(9)

# fp8 pools store 8-bit float codes (sign bit 7, exponent bits 6..3, mantissa
# bits 2..0); 0x7F is a NaN code and poisons fp8 storage as BF16_NAN poisons
# bf16 storage.
E4M3_NAN = np.uint8(0x7F)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and
    return the 16-bit patterns.  NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = BF16_NAN
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), *[int(t) for t in tags]]))


def normal_bf16(seed: int, tags: Sequence[int], shape) -> np.ndarray:
    return f32_to_bf16_bits(_rng(seed, *tags).standard_normal(size=shape, dtype=np.float32))


# ---------------------------------------------------------------------------
# Workload shapes (single-layer, synthetic).  Head counts follow the published
# attention shapes of the model families the pages serve (Qwen2.5-1.5B: 12 q /
# 2 kv heads, Qwen2.5-7B: 28 q / 4 kv, Qwen3-0.6B: 16 q / 8 kv; head_dim 128).
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class DecodeSpec:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    context_lens: Optional[tuple] = None      # explicit lengths, or
    len_range: Optional[tuple] = None         # inclusive uniform integer range
    scale: Optional[float] = None             # None -> float32(1/sqrt(head_dim))
    seed: int = 0
    append: bool = False                      # new token of each sequence appended by slot

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale_f32(self) -> np.float32:
        s = self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)
        return np.float32(s)

    def with_(self, **kw) -> "DecodeSpec":
        return dataclasses.replace(self, **kw)


def _c1(**kw):
    return DecodeSpec("tiny", 4, 2, 1, 64, 16, 64, 16, context_lens=(1, 17, 100, 255),
                      scale=0.125, seed=1000, **kw)


def _c2(batch: int):
    return DecodeSpec(f"qwen2.5-1.5b-ctx4096-b{batch}", batch, 12, 2, 128, 16, 4096, 256,
                      context_lens=(4096,) * batch, seed=2000 + batch)


def _c3():
    return DecodeSpec("qwen2.5-7b-b8", 8, 28, 4, 128, 256, 512, 16, len_range=(128, 4096),
                      seed=3000, append=True)


# 90% of a 20 GB budget for one layer's K and V at [256, 8, 128] bf16 per block:
# floor(18e9 / (2 * 256 * 8 * 128 * 2)) = 17166 blocks.
C4_NUM_BLOCKS = (18 * 10**9) // (2 * 256 * 8 * 128 * 2)


def _c4():
    return DecodeSpec("qwen3-0.6b-b256", 256, 16, 8, 128, 256, C4_NUM_BLOCKS, 5,
                      len_range=(256, 1280), seed=4000)


def _c5_decode():
    return DecodeSpec("qwen2.5-7b-mixed-decode64", 64, 28, 4, 128, 256, 2048, 16,
                      len_range=(512, 4096), seed=5000, append=True)


CONFIGS = {
    "c1": _c1(),
    "c2b1": _c2(1),
    "c2b8": _c2(8),
    "c3": _c3(),
    "c4": _c4(),
    "c5d": _c5_decode(),
}


@dataclasses.dataclass(frozen=True)
class PrefillSpec:
    """One causal query chunk at the end of a longer sequence whose earlier
    tokens already sit in the paged cache."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    chunk_lens: tuple          # query tokens per sequence
    total_lens: tuple          # cached prefix + chunk, per sequence
    scale: Optional[float] = None
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale_f32(self) -> np.float32:
        s = self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)
        return np.float32(s)

    def with_(self, **kw) -> "PrefillSpec":
        return dataclasses.replace(self, **kw)


PREFILL_CONFIGS = {
    # 512-token chunk over a 3584-token cached prefix (total 4096), 28 q / 4 kv.
    "c5p": PrefillSpec("qwen2.5-7b-chunk512-of-4096", 28, 4, 128, 256, 2048, 16,
                       chunk_lens=(512,), total_lens=(4096,), seed=5500),
}


# ---------------------------------------------------------------------------
# Drawing the inputs.
# ---------------------------------------------------------------------------


def draw_context_lens(spec: DecodeSpec) -> np.ndarray:
    if spec.context_lens is not None:
        lens = np.asarray(spec.context_lens, dtype=np.int32)
        assert lens.shape == (spec.num_seqs,)
        return lens
    lo, hi = spec.len_range
    return _rng(spec.seed, _TAG_LENS).integers(lo, hi + 1, size=spec.num_seqs).astype(np.int32)


def assign_blocks(seed: int, num_blocks: int, lens: np.ndarray, block_size: int,
                  max_blocks_per_seq: int):
    """Seeded random permutation of the physical pool; sequence b takes the next
    ceil(L_b / block_size) ids in permutation order.  Returns the table
    (padded entries point at a block no sequence uses, which stays poisoned),
    the list of used ids and that poison id."""
    perm = _rng(seed, _TAG_PERM).permutation(num_blocks).astype(np.int64)
    need = [(int(L) + block_size - 1) // block_size for L in lens]
    assert max(need, default=0) <= max_blocks_per_seq
    total = sum(need)
    assert total < num_blocks, "pool too small to keep a poison block"
    poison = int(perm[-1])
    tables = np.full((len(lens), max_blocks_per_seq), poison, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        tables[b, :n] = perm[off:off + n]
        off += n
    return tables, perm[:total].copy(), poison


@dataclasses.dataclass
class CompactPool:
    """The referenced blocks of a pool, stored densely.

    ``ids[i]`` is the physical id of ``k[i]`` / ``v[i]``; every other block of
    the ``num_blocks`` pool is NaN.  ``full()`` materialises the whole pool
    (only sensible for small pools); ``compact_tables()`` rewrites a block
    table into indices of the dense arrays, which addresses the same logical
    tokens."""
    num_blocks: int
    ids: np.ndarray       # int64 [n_used]
    k: np.ndarray         # uint16 [n_used, bs, Hkv, D]
    v: np.ndarray

    def full(self):
        shape = (self.num_blocks,) + self.k.shape[1:]
        kf = np.full(shape, BF16_NAN, dtype=np.uint16)
        vf = np.full(shape, BF16_NAN, dtype=np.uint16)
        kf[self.ids] = self.k
        vf[self.ids] = self.v
        return kf, vf

    def compact_tables(self, tables: np.ndarray, poison: int):
        lut = np.full(self.num_blocks, -1, dtype=np.int64)
        lut[self.ids] = np.arange(len(self.ids))
        out = lut[tables.astype(np.int64)]
        # padded entries point at the poison block, which is not stored: map
        # them to entry 0 (they are never part of a sequence's tokens).
        out[tables == poison] = 0
        assert (out >= 0).all()
        return out.astype(np.int32)


def fill_blocks(seed: int, ids: np.ndarray, block_size: int, num_kv_heads: int, head_dim: int,
                fill: str = "normal"):
    shape = (len(ids), block_size, num_kv_heads, head_dim)
    if fill == "zeros":
        z = np.zeros(shape, dtype=np.uint16)
        return z, z.copy()
    k = np.empty(shape, dtype=np.uint16)
    v = np.empty(shape, dtype=np.uint16)
    for i, p in enumerate(ids):
        k[i] = normal_bf16(seed, (_TAG_K, int(p)), shape[1:])
        v[i] = normal_bf16(seed, (_TAG_V, int(p)), shape[1:])
    return k, v


def poison_tails(pool: CompactPool, tables: np.ndarray, lens: np.ndarray, block_size: int):
    """NaN the slots at or past each sequence's length in its last block."""
    idx = {int(p): i for i, p in enumerate(pool.ids)}
    for b, L in enumerate(lens):
        L = int(L)
        if L % block_size == 0:
            continue
        last = int(tables[b, L // block_size])
        i = idx[last]
        pool.k[i, L % block_size:] = BF16_NAN
        pool.v[i, L % block_size:] = BF16_NAN


@dataclasses.dataclass
class DecodeInputs:
    spec: DecodeSpec
    q: np.ndarray                 # uint16 [B, Hq, D]
    pool: CompactPool
    block_tables: np.ndarray      # int32 [B, W]
    context_lens: np.ndarray      # int32 [B] (after the append, when there is one)
    poison_block: int
    scale: np.float32
    # append (only when spec.append): new K/V rows and their slots
    new_k: Optional[np.ndarray] = None   # uint16 [T, Hkv, D]
    new_v: Optional[np.ndarray] = None
    slot_mapping: Optional[np.ndarray] = None  # int64 [T]


def make_decode_inputs(spec: DecodeSpec, *, fill: str = "normal", lens=None) -> DecodeInputs:
    """Inputs of one decode call.  With ``spec.append`` the last token of each
    sequence is not yet in the pool (its slot holds NaN) and arrives as
    ``new_k``/``new_v`` with ``slot_mapping[b] = slot of token L_b - 1``."""
    lens = draw_context_lens(spec) if lens is None else np.asarray(lens, dtype=np.int32)
    tables, ids, poison = assign_blocks(spec.seed, spec.num_blocks, lens, spec.block_size,
                                        spec.max_blocks_per_seq)
    k, v = fill_blocks(spec.seed, ids, spec.block_size, spec.num_kv_heads, spec.head_dim, fill)
    pool = CompactPool(spec.num_blocks, ids, k, v)
    poison_tails(pool, tables, lens, spec.block_size)
    q = normal_bf16(spec.seed, (_TAG_Q,), (spec.num_seqs, spec.num_q_heads, spec.head_dim))
    out = DecodeInputs(spec, q, pool, tables, lens, poison, spec.scale_f32)
    if spec.append:
        bs = spec.block_size
        sel = np.nonzero(lens > 0)[0]
        slots = np.array([int(tables[b, (lens[b] - 1) // bs]) * bs + int((lens[b] - 1) % bs)
                          for b in sel], dtype=np.int64)
        kv_shape = (len(sel), spec.num_kv_heads, spec.head_dim)
        out.new_k = normal_bf16(spec.seed, (_TAG_NEWK,), kv_shape)
        out.new_v = normal_bf16(spec.seed, (_TAG_NEWV,), kv_shape)
        out.slot_mapping = slots
        # the slot the new token goes to is still empty (poison) in the pool
        idx = {int(p): i for i, p in enumerate(ids)}
        for s in slots:
            i = idx[int(s) // bs]
            pool.k[i, int(s) % bs] = BF16_NAN
            pool.v[i, int(s) % bs] = BF16_NAN
    return out


@dataclasses.dataclass
class PrefillInputs:
    spec: PrefillSpec
    q: np.ndarray                 # uint16 [Tq, Hq, D]
    cu_seqlens_q: np.ndarray      # int32 [B + 1]
    pool: CompactPool             # holds the cached prefix; chunk slots are NaN
    block_tables: np.ndarray      # int32 [B, W]
    context_lens: np.ndarray      # int32 [B] total lengths (prefix + chunk)
    poison_block: int
    scale: np.float32
    new_k: np.ndarray             # uint16 [Tq, Hkv, D]: the chunk's own K/V
    new_v: np.ndarray
    slot_mapping: np.ndarray      # int64 [Tq]


def make_prefill_inputs(spec: PrefillSpec, *, fill: str = "normal") -> PrefillInputs:
    lens = np.asarray(spec.total_lens, dtype=np.int32)
    chunks = np.asarray(spec.chunk_lens, dtype=np.int32)
    assert (chunks <= lens).all() and (chunks >= 0).all()
    tables, ids, poison = assign_blocks(spec.seed, spec.num_blocks, lens, spec.block_size,
                                        spec.max_blocks_per_seq)
    k, v = fill_blocks(spec.seed, ids, spec.block_size, spec.num_kv_heads, spec.head_dim, fill)
    pool = CompactPool(spec.num_blocks, ids, k, v)
    poison_tails(pool, tables, lens, spec.block_size)
    bs = spec.block_size
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(chunks)
    slots = []
    for b, (L, n) in enumerate(zip(lens, chunks)):
        for t in range(int(L) - int(n), int(L)):
            slots.append(int(tables[b, t // bs]) * bs + t % bs)
    slots = np.asarray(slots, dtype=np.int64)
    idx = {int(p): i for i, p in enumerate(ids)}
    for s in slots:
        i = idx[int(s) // bs]
        pool.k[i, int(s) % bs] = BF16_NAN
        pool.v[i, int(s) % bs] = BF16_NAN
    tq = int(cu[-1])
    q = normal_bf16(spec.seed, (_TAG_Q,), (tq, spec.num_q_heads, spec.head_dim))
    kv_shape = (tq, spec.num_kv_heads, spec.head_dim)
    if fill == "zeros":
        nk = np.zeros(kv_shape, np.uint16)
        nv = np.zeros(kv_shape, np.uint16)
    else:
        nk = normal_bf16(spec.seed, (_TAG_NEWK,), kv_shape)
        nv = normal_bf16(spec.seed, (_TAG_NEWV,), kv_shape)
    return PrefillInputs(spec, q, cu, pool, tables, lens, poison, spec.scale_f32, nk, nv, slots)


@dataclasses.dataclass
class MixedInputs:
    """One mixed-batch step over one shared pool: the prompt chunk(s) of
    ``prefill`` and the decode sequences of ``decode`` reference disjoint
    blocks of the same ``pool`` (both input objects hold that same pool).
    The chunk's rows and each decode sequence's new row arrive by slot and
    their slots hold poison until then."""
    prefill: PrefillInputs
    decode: DecodeInputs
    pool: CompactPool

    def all_rows(self):
        """Every row the step appends, chunk rows first: (new_k, new_v, slots)."""
        p, d = self.prefill, self.decode
        return (np.concatenate([p.new_k, d.new_k]), np.concatenate([p.new_v, d.new_v]),
                np.concatenate([p.slot_mapping, d.slot_mapping]))


def make_mixed_inputs(pspec: PrefillSpec, dspec: DecodeSpec) -> MixedInputs:
    """Inputs of the chunked-prefill mixed batch: prompt chunks (``pspec``)
    interleaved with active decodes (``dspec``, one new token each), in one
    pool of max(num_blocks) blocks.  One seeded permutation of that pool
    (seed ``pspec.seed``) hands the prompt sequences their blocks first, then
    the decode sequences.  The prompt side draws q and its chunk rows from
    ``pspec.seed``, the decode side from ``dspec.seed``."""
    key = lambda s: (s.num_q_heads, s.num_kv_heads, s.head_dim, s.block_size)   # noqa: E731
    assert key(pspec) == key(dspec), "prompt and decode sides must share the pool's shape"
    bs, Hkv, D, Hq = dspec.block_size, dspec.num_kv_heads, dspec.head_dim, dspec.num_q_heads
    plens = np.asarray(pspec.total_lens, dtype=np.int32)
    chunks = np.asarray(pspec.chunk_lens, dtype=np.int32)
    assert (chunks <= plens).all() and (chunks >= 0).all()
    dlens = draw_context_lens(dspec)
    assert (dlens > 0).all(), "every decode sequence appends one token"
    NB = max(pspec.num_blocks, dspec.num_blocks)
    W = max(pspec.max_blocks_per_seq, dspec.max_blocks_per_seq)
    lens = np.concatenate([plens, dlens])
    tables, ids, poison = assign_blocks(pspec.seed, NB, lens, bs, W)
    k, v = fill_blocks(pspec.seed, ids, bs, Hkv, D)
    pool = CompactPool(NB, ids, k, v)
    poison_tails(pool, tables, lens, bs)
    P = len(plens)
    ptab = np.ascontiguousarray(tables[:P, :pspec.max_blocks_per_seq])
    dtab = np.ascontiguousarray(tables[P:, :dspec.max_blocks_per_seq])
    cu = np.zeros(P + 1, dtype=np.int32)
    cu[1:] = np.cumsum(chunks)
    pslots = np.asarray([int(ptab[b, t // bs]) * bs + t % bs
                         for b, (L, n) in enumerate(zip(plens, chunks))
                         for t in range(int(L) - int(n), int(L))], dtype=np.int64)
    dslots = np.asarray([int(dtab[b, (L - 1) // bs]) * bs + int((L - 1) % bs)
                         for b, L in enumerate(dlens)], dtype=np.int64)
    idx = {int(p): i for i, p in enumerate(ids)}
    for s in np.concatenate([pslots, dslots]):
        i = idx[int(s) // bs]
        pool.k[i, int(s) % bs] = BF16_NAN
        pool.v[i, int(s) % bs] = BF16_NAN
    tq = int(cu[-1])
    pre = PrefillInputs(
        pspec, normal_bf16(pspec.seed, (_TAG_Q,), (tq, Hq, D)), cu, pool, ptab, plens, poison,
        pspec.scale_f32, normal_bf16(pspec.seed, (_TAG_NEWK,), (tq, Hkv, D)),
        normal_bf16(pspec.seed, (_TAG_NEWV,), (tq, Hkv, D)), pslots)
    B = len(dlens)
    dec = DecodeInputs(
        dspec.with_(append=True, num_blocks=NB), normal_bf16(dspec.seed, (_TAG_Q,), (B, Hq, D)),
        pool, dtab, dlens, poison, dspec.scale_f32,
        normal_bf16(dspec.seed, (_TAG_NEWK,), (B, Hkv, D)),
        normal_bf16(dspec.seed, (_TAG_NEWV,), (B, Hkv, D)), dslots)
    return MixedInputs(pre, dec, pool)


def random_e4m3_codes(seed: int, tags: Sequence[int], shape) -> np.ndarray:
    """Random fp8 codes: sign, exponent field uniform in 4..8 and mantissa
    field uniform in 0..7, so magnitudes lie in [2^-3, 3.75] and no code is
    NaN."""
    g = _rng(seed, *tags)
    sign = g.integers(0, 2, size=shape, dtype=np.uint8) << 7
    expo = g.integers(4, 9, size=shape, dtype=np.uint8) << 3
    mant = g.integers(0, 8, size=shape, dtype=np.uint8)
    return (sign | expo | mant).astype(np.uint8)


def fp8_codes_like(inp):
    """fp8 pools for the blocks, tables and lengths of ``inp`` (decode or
    prefill inputs): each referenced
    block draws its own codes (streams keyed by seed and block id), and every
    slot that ``inp``'s bf16 pool poisons holds E4M3_NAN.  Returns the K and V
    codes, stored densely like ``inp.pool`` but head-major, [n, Hkv, bs, D],
    the layout of fp8 pools."""
    s = inp.spec
    shape = inp.pool.k.shape
    k = np.empty(shape, dtype=np.uint8)
    v = np.empty(shape, dtype=np.uint8)
    for i, p in enumerate(inp.pool.ids):
        k[i] = random_e4m3_codes(s.seed, (_TAG_K8, int(p)), shape[1:])
        v[i] = random_e4m3_codes(s.seed, (_TAG_V8, int(p)), shape[1:])
    k[inp.pool.k == BF16_NAN] = E4M3_NAN
    v[inp.pool.v == BF16_NAN] = E4M3_NAN
    hm = lambda c: np.ascontiguousarray(np.transpose(c, (0, 2, 1, 3)))   # noqa: E731
    return hm(k), hm(v)


def algorithmic_decode_bytes(lens, num_q_heads, num_kv_heads, head_dim, block_size) -> int:
    """Bytes a paged decode call must move at minimum: every K and V element of
    every sequence's tokens once per kv head, q and out once, the table entries
    it uses and the lengths."""
    lens = np.asarray(lens, dtype=np.int64)
    kv = int(lens.sum()) * num_kv_heads * head_dim * 2 * 2
    qo = len(lens) * num_q_heads * head_dim * 2 * 2
    tab = int(((lens + block_size - 1) // block_size).sum()) * 4
    return kv + qo + tab + len(lens) * 4
