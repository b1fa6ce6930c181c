"""The seeded input generators: reproducible, correctly rounded, poisoned
where nothing may be read."""
import numpy as np
import pytest

import workloads as W


def test_bf16_rounding_is_rne():
    # 1 + 2^-8 is exactly halfway between bf16 1.0 and 1 + 2^-7: ties go to even (1.0)
    x = np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -2.5, 0.0, np.inf],
                 np.float32)
    got = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
    assert list(got) == [1.0, 1.0 + 2**-6, 1.0 + 2**-7, -2.5, 0.0, np.inf]
    assert W.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == W.BF16_NAN


def test_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bf16_bits(x), ref)


@pytest.mark.parametrize("name", ["c1", "c2b1", "c3"])
def test_reproducible(name):
    a = W.make_decode_inputs(W.CONFIGS[name])
    b = W.make_decode_inputs(W.CONFIGS[name])
    assert np.array_equal(a.q, b.q) and np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.pool.k, b.pool.k) and np.array_equal(a.pool.v, b.pool.v)


@pytest.mark.parametrize("name", ["c1", "c2b8", "c3", "c5d"])
def test_tables_and_poison(name):
    spec = W.CONFIGS[name]
    inp = W.make_decode_inputs(spec)
    bs = spec.block_size
    lens = inp.context_lens
    used = []
    for b, L in enumerate(lens):
        n = (int(L) + bs - 1) // bs
        used += list(inp.block_tables[b, :n])
        assert (inp.block_tables[b, n:] == inp.poison_block).all()
    assert len(set(used)) == len(used), "a physical block is shared"
    assert inp.poison_block not in used
    assert sorted(used) == sorted(int(i) for i in inp.pool.ids)
    # poison exactly at slots >= L of each last block (and at appended slots)
    idx = {int(p): i for i, p in enumerate(inp.pool.ids)}
    appended = set() if inp.slot_mapping is None else {int(s) for s in inp.slot_mapping}
    for b, L in enumerate(lens):
        for t in range(0, int(L), max(1, int(L) // 7)):
            blk = int(inp.block_tables[b, t // bs])
            slot = blk * bs + t % bs
            row = inp.pool.k[idx[blk], t % bs]
            assert (row == W.BF16_NAN).all() == (slot in appended)
        if int(L) % bs:
            blk = int(inp.block_tables[b, int(L) // bs])
            assert (inp.pool.k[idx[blk], int(L) % bs:] == W.BF16_NAN).all()
            assert (inp.pool.v[idx[blk], int(L) % bs:] == W.BF16_NAN).all()


def test_config_shapes():
    c = W.CONFIGS
    assert W.C4_NUM_BLOCKS == 17166
    assert (c["c2b8"].group, c["c3"].group, c["c4"].group, c["c5d"].group) == (6, 7, 2, 7)
    lens = W.draw_context_lens(c["c4"])
    assert lens.min() >= 256 and lens.max() <= 1280 and len(lens) == 256
    assert float(c["c2b8"].scale_f32) == float(np.float32(1 / np.sqrt(128)))


def test_append_targets_last_token():
    spec = W.CONFIGS["c3"]
    inp = W.make_decode_inputs(spec)
    bs = spec.block_size
    for b, L in enumerate(inp.context_lens):
        s = int(inp.slot_mapping[b])
        assert s // bs == inp.block_tables[b, (L - 1) // bs] and s % bs == (L - 1) % bs


def test_compact_tables_address_same_tokens():
    inp = W.make_decode_inputs(W.CONFIGS["c1"])
    kf, _ = inp.pool.full()
    ct = inp.pool.compact_tables(inp.block_tables, inp.poison_block)
    bs = 16
    for b, L in enumerate(inp.context_lens):
        for t in range(int(L)):
            assert np.array_equal(kf[inp.block_tables[b, t // bs], t % bs],
                                  inp.pool.k[ct[b, t // bs], t % bs])


def test_prefill_inputs():
    spec = W.PREFILL_CONFIGS["c5p"].with_(total_lens=(300,), chunk_lens=(40,), num_blocks=8,
                                          max_blocks_per_seq=2)
    inp = W.make_prefill_inputs(spec)
    assert inp.q.shape == (40, 28, 128) and list(inp.cu_seqlens_q) == [0, 40]
    bs = 256
    assert [int(s) for s in inp.slot_mapping[:2]] == [
        int(inp.block_tables[0, 260 // bs]) * bs + 260 % bs,
        int(inp.block_tables[0, 261 // bs]) * bs + 261 % bs]


def test_algorithmic_bytes_c2():
    # 8 x 4096 tokens x 2 kv heads x 128 x 2 B x (K, V) + q + out + 2048 table entries + lens
    assert W.algorithmic_decode_bytes([4096] * 8, 12, 2, 128, 16) == \
        8 * 4096 * 2 * 128 * 2 * 2 + 2 * 8 * 12 * 128 * 2 + 2048 * 4 + 8 * 4


def test_mixed_inputs_share_one_pool():
    """The mixed-batch step's prompt chunk and decode sequences take disjoint
    blocks of one pool; every row the step appends lands on a poisoned slot
    of the right sequence and position."""
    pspec = W.PREFILL_CONFIGS["c5p"].with_(total_lens=(700,), chunk_lens=(200,), num_blocks=64,
                                          max_blocks_per_seq=4)
    dspec = W.CONFIGS["c5d"].with_(num_seqs=5, len_range=(1, 900), num_blocks=32,
                                   max_blocks_per_seq=4)
    m = W.make_mixed_inputs(pspec, dspec)
    p, d = m.prefill, m.decode
    assert p.pool is m.pool and d.pool is m.pool and m.pool.num_blocks == 64
    assert d.spec.num_blocks == 64 and d.spec.append
    bs = 256
    used = []
    for tab, lens in ((p.block_tables, p.context_lens), (d.block_tables, d.context_lens)):
        for b, L in enumerate(lens):
            n = -(-int(L) // bs)
            used += [int(x) for x in tab[b, :n]]
            assert (tab[b, n:] == p.poison_block).all()
    assert len(set(used)) == len(used) and sorted(used) == sorted(int(i) for i in m.pool.ids)
    idx = {int(x): i for i, x in enumerate(m.pool.ids)}
    # the chunk's slots are its last 200 positions, the decode slots each last token
    assert [int(s) for s in p.slot_mapping] == [
        int(p.block_tables[0, t // bs]) * bs + t % bs for t in range(500, 700)]
    assert [int(s) for s in d.slot_mapping] == [
        int(d.block_tables[b, (L - 1) // bs]) * bs + (int(L) - 1) % bs
        for b, L in enumerate(d.context_lens)]
    k, v, slots = m.all_rows()
    assert k.shape == (205, 4, 128) and v.shape == k.shape and len(slots) == 205
    assert len(set(int(s) for s in slots)) == 205
    for s in slots:
        assert (m.pool.k[idx[int(s) // bs], int(s) % bs] == W.BF16_NAN).all()
        assert (m.pool.v[idx[int(s) // bs], int(s) % bs] == W.BF16_NAN).all()
    # the cached prefix is data, not poison; the two sides draw different q
    assert not (m.pool.k[idx[int(p.block_tables[0, 0])], :100] == W.BF16_NAN).any()
    assert not np.array_equal(p.q[:5], d.q)
    again = W.make_mixed_inputs(pspec, dspec)
    assert np.array_equal(again.pool.k, m.pool.k) and np.array_equal(again.decode.q, d.q)
