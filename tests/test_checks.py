"""The library's host-side precondition checks (pa_check_tables, pa_check_slots,
pa_check_prefill): valid layouts pass, every kind of planted violation is
reported with the right offending index, and on random layouts the checks
agree with a brute-force statement of the same rules, written out below from
the header's definitions.  Host code only: runs without a GPU."""
import numpy as np
import pytest

import paged_kv_attention_09_amd as pa
import workloads as W

LENGTH, BLOCK_ID, APPEND_SHARED, SLOT_RANGE, SLOT_DUPLICATE, QUERY_OFFSETS = range(1, 7)


def _kind(fn, *args, **kw):
    """(kind, index) of the first violation, (0, -1) when none."""
    try:
        fn(*args, **kw)
    except pa.PreconditionError as e:
        return e.kind, e.index
    return 0, -1


def brute_tables(tables, lens, num_blocks, bs, fused):
    W_ = tables.shape[1]
    for b, L in enumerate(lens):
        if L < 0 or L > W_ * bs:
            return LENGTH, b
        if any(not 0 <= tables[b, j] < num_blocks for j in range(-(-int(L) // bs))):
            return BLOCK_ID, b
    if fused:
        reads = [(b, j) for b, L in enumerate(lens) for j in range(-(-int(L) // bs))]
        for b, L in enumerate(lens):
            if L == 0:
                continue
            j_last = (L - 1) // bs
            blk = tables[b, j_last]
            if any(tables[c, j] == blk for c, j in reads if (c, j) != (b, j_last)):
                return APPEND_SHARED, b
    return 0, -1


def brute_slots(slots, num_blocks, bs):
    seen = set()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        if s >= num_blocks * bs:
            return SLOT_RANGE, i
        if s in seen:
            return SLOT_DUPLICATE, i
        seen.add(int(s))
    return 0, -1


def test_workload_layouts_pass():
    for name in ("c1", "c3", "c5d"):
        spec = W.CONFIGS[name].with_(append=True)
        inp = W.make_decode_inputs(spec, fill="zeros")
        for fused in (False, True):
            pa.check_tables(inp.block_tables, inp.context_lens, spec.num_blocks,
                            spec.block_size, fused_append=fused)
        pa.check_slots(inp.slot_mapping, spec.num_blocks, spec.block_size)
    p = W.make_prefill_inputs(W.PREFILL_CONFIGS["c5p"], fill="zeros")
    pa.check_prefill(p.cu_seqlens_q, p.context_lens, int(np.diff(p.cu_seqlens_q).max()))
    pa.check_slots(p.slot_mapping, p.spec.num_blocks, p.spec.block_size)


def test_block_manager_layout_passes_with_shared_prefixes():
    """Tables from the native block manager with prefix sharing: shared blocks
    are read by several sequences, yet no sequence appends into one."""
    bm = pa.BlockManager(64, 16, 8, prefix_cache=True)
    prompt = list(range(40))
    bm.admit(0, 0, prompt)
    bm.decode_step([0], [500])           # sequence 0's full blocks become shareable
    for sid in range(1, 4):
        bm.admit(sid, 0, prompt)
    bm.decode_step(list(range(4)), [501, 502, 503, 504])
    tables, lens = bm.block_tables(list(range(4)))
    pa.check_tables(tables, lens, 64, 16, fused_append=True)
    shared = set(tables[0, :2]) & set(tables[1, :2])
    assert shared, "the prompt's full blocks should be shared"


def test_planted_table_violations():
    t = np.array([[3, 4, 9], [5, 6, 9], [7, 9, 9]], np.int32)
    lens = np.array([20, 17, 5], np.int32)
    assert _kind(pa.check_tables, t, lens, 10, 16) == (0, -1)
    assert _kind(pa.check_tables, t, np.array([20, -1, 5], np.int32), 10, 16) == (LENGTH, 1)
    assert _kind(pa.check_tables, t, np.array([20, 17, 49], np.int32), 10, 16) == (LENGTH, 2)
    assert _kind(pa.check_tables, t, np.array([20, 17, 48], np.int32), 10, 16) == (0, -1)
    bad = t.copy(); bad[1, 1] = 10
    assert _kind(pa.check_tables, bad, lens, 10, 16) == (BLOCK_ID, 1)
    bad = t.copy(); bad[2, 0] = -3
    assert _kind(pa.check_tables, bad, lens, 10, 16) == (BLOCK_ID, 2)
    bad = t.copy(); bad[2, 2] = 123          # past sequence 2's length: never read
    assert _kind(pa.check_tables, bad, lens, 10, 16) == (0, -1)
    # fused append: sequence 2 appends into block 4, which sequence 0 reads
    sh = t.copy(); sh[2, 0] = 4
    assert _kind(pa.check_tables, sh, lens, 10, 16) == (0, -1)
    assert _kind(pa.check_tables, sh, lens, 10, 16, fused_append=True) == (APPEND_SHARED, 0)
    sh = t.copy(); sh[2, 0] = 3              # block 3 is read (not written) by sequence 0
    assert _kind(pa.check_tables, sh, lens, 10, 16, fused_append=True) == (APPEND_SHARED, 2)
    # empty sequences append nothing and read nothing
    assert _kind(pa.check_tables, t, np.array([0, 0, 0], np.int32), 10, 16,
                 fused_append=True) == (0, -1)


def test_planted_slot_violations():
    assert _kind(pa.check_slots, [5, -1, 7, -1, 0], 4, 2) == (0, -1)
    assert _kind(pa.check_slots, [5, 8, 7], 4, 2) == (SLOT_RANGE, 1)
    assert _kind(pa.check_slots, [5, 3, 7, 3], 4, 2) == (SLOT_DUPLICATE, 3)
    assert _kind(pa.check_slots, np.zeros(0, np.int64), 4, 2) == (0, -1)


def test_planted_prefill_violations():
    lens = [10, 3, 600]
    assert _kind(pa.check_prefill, [0, 4, 7, 519], lens, 512) == (0, -1)
    assert _kind(pa.check_prefill, [1, 4, 7, 519], lens, 512) == (QUERY_OFFSETS, 0)
    assert _kind(pa.check_prefill, [0, 4, 3, 519], lens, 512) == (QUERY_OFFSETS, 1)
    assert _kind(pa.check_prefill, [0, 4, 8, 519], lens, 512) == (QUERY_OFFSETS, 1)
    assert _kind(pa.check_prefill, [0, 4, 7, 520], lens, 512) == (QUERY_OFFSETS, 2)


@pytest.mark.parametrize("seed", range(12))
def test_random_layouts_agree_with_brute_force(seed):
    rng = np.random.default_rng(seed)
    B, W_, bs, NB = int(rng.integers(1, 9)), int(rng.integers(1, 6)), 16, 48
    lens = rng.integers(0, W_ * bs + 1, size=B).astype(np.int32)
    tables = rng.permutation(NB)[:B * W_].reshape(B, W_).astype(np.int32)
    for _ in range(int(rng.integers(0, 3))):     # plant a few faults
        r = int(rng.integers(0, 4))
        b, j = int(rng.integers(0, B)), int(rng.integers(0, W_))
        if r == 0:
            lens[b] = int(rng.choice([-1, W_ * bs + 1]))
        elif r == 1:
            tables[b, j] = int(rng.choice([-1, NB, NB + 5]))
        else:
            tables[b, j] = tables[int(rng.integers(0, B)), int(rng.integers(0, W_))]
    for fused in (False, True):
        assert _kind(pa.check_tables, tables, lens, NB, bs, fused_append=fused) == \
            brute_tables(tables, lens, NB, bs, fused)
    slots = rng.integers(-2, NB * bs + 3, size=int(rng.integers(0, 40)))
    assert _kind(pa.check_slots, slots, NB, bs) == brute_slots(slots, NB, bs)


def test_argument_errors():
    with pytest.raises(pa.PagedAttnError):
        pa.check_tables(np.zeros((1, 1), np.int32), np.zeros(1, np.int32), 0, 16)
    with pytest.raises(pa.PagedAttnError):
        pa.check_slots([0], 4, 12)               # block size not a power of two
    with pytest.raises(ValueError):
        pa.check_tables(np.zeros((2, 1), np.int32), np.zeros(3, np.int32), 4, 16)
    with pytest.raises(ValueError):
        pa.check_slots(np.array([2**40], np.float64) + 0.5, 4, 16)
    import torch
    with pytest.raises(TypeError):
        pa.check_slots(torch.zeros(3, dtype=torch.int32), 4, 16)
