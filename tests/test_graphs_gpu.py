"""Decode steps captured in HIP graphs at power-of-two padded batch sizes
(paged_kv_attention_09_amd.graphs): every replay, with fresh inputs, eager
work and synchronisations between replays, equals an eager call on the same
padded inputs bit for bit, matches the oracle on the real rows within the
decode tolerance, and leaves the padding rows zero."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_09_amd as pa
import workloads as W
from gpu_cases import DEV, DecodeCase, assert_close, to_f64
from paged_kv_attention_09_amd.graphs import PaddedDecodeGraphs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def setup():
    spec = W.DecodeSpec("graphs", 12, 12, 2, 128, 16, 1200, 64, len_range=(1, 1000), seed=8100,
                        append=True)
    case = DecodeCase(W.make_decode_inputs(spec))
    kc, vc, ct = case.oracle_pools()           # every sequence's new row appended
    ref = oracle.decode(case.inp.q, kc, vc, ct, case.inp.context_lens, case.inp.scale)
    graphs = PaddedDecodeGraphs(case.k_cache, case.v_cache, spec.num_q_heads, 8,
                                spec.max_blocks_per_seq, case.scale)
    return case, ref, graphs


def test_replays_match_eager_and_oracle(setup):
    case, ref, graphs = setup
    rng = np.random.default_rng(5)
    for trial, B in enumerate((3, 1, 8, 5, 2, 4, 7, 3)):
        idx = rng.permutation(case.inp.spec.num_seqs)[:B]
        sel = torch.from_numpy(idx).to(DEV)
        P = graphs.prepare(case.q[sel], case.new_k[sel], case.new_v[sel], case.tables[sel],
                           case.lens[sel])
        assert P == graphs.size_for(B) and P >= B
        got = graphs.replay(P).clone()
        torch.cuda.synchronize()
        assert_close(to_f64(got[:B]), ref[idx], what=f"trial {trial} B={B}")
        assert not got[B:].any(), "padding rows must be zero"
        # the same padded step, eagerly, with its own workspace
        b = graphs.buffers(P)
        eager = torch.empty_like(b["out"])
        pa.append_decode(b["q"], b["new_k"], b["new_v"], case.k_cache, case.v_cache, b["tables"],
                         b["lens"], case.scale, graphs.splits[P], eager)
        torch.cuda.synchronize()
        assert torch.equal(eager, got), f"trial {trial}: graph differs from eager"
        # unrelated eager work between replays
        x = torch.randn(4096, device=DEV)
        _ = (x * x).sum().item()


def test_replay_of_a_size_twice_in_a_row(setup):
    """Two replays of one graph with different inputs in between."""
    case, ref, graphs = setup
    for idx in (np.array([0, 5, 9]), np.array([11, 2, 7])):
        sel = torch.from_numpy(idx).to(DEV)
        P = graphs.prepare(case.q[sel], case.new_k[sel], case.new_v[sel], case.tables[sel],
                           case.lens[sel])
        got = graphs.replay(P).clone()
        torch.cuda.synchronize()
        assert P == 4
        assert_close(to_f64(got[:3]), ref[idx], what=f"seqs {idx}")
        assert not got[3:].any()


def test_batch_over_the_largest_size_is_refused(setup):
    _, _, graphs = setup
    with pytest.raises(ValueError):
        graphs.size_for(9)


def test_prepare_holds_caller_tensors_until_its_stream_read_them(setup):
    """prepare() copies on the graphs' stream.  With that stream still busy,
    the caller frees its tensors and fills fresh allocations of the same
    sizes on its own stream: the static buffers must still receive the
    original rows (the allocator may not recycle memory the graphs' stream
    has yet to read)."""
    case, ref, graphs = setup
    idx = np.array([4, 1, 10])
    sel = torch.from_numpy(idx).to(DEV)
    srcs = [t[sel].clone() for t in (case.q, case.new_k, case.new_v, case.tables, case.lens)]
    want = [t.clone() for t in srcs]
    torch.cuda.synchronize()
    with torch.cuda.stream(graphs.stream):
        torch.cuda._sleep(20_000_000)            # keeps the copies waiting
    P = graphs.prepare(*srcs)
    shapes = [(t.shape, t.dtype) for t in srcs]
    del srcs
    junk = [torch.full(s, 7, dtype=dt, device=DEV) for s, dt in shapes]
    torch.cuda.synchronize()
    b = graphs.buffers(P)
    for name, w in zip(("q", "new_k", "new_v", "tables", "lens"), want):
        assert torch.equal(b[name][:3], w), f"{name} was overwritten before the copy read it"
    del junk
