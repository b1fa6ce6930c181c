"""The allocation-free decode entry point (pa_decode_noalloc) against
pa_decode with a caller workspace, through the C ABI: two calls in a row on
one device (the second smaller, so it reuses the static scratch the first
one filled) give pa_decode's outputs bit for bit at the same split count and
the oracle's within 1e-2 + 1e-2 |oracle|; a call whose partials exceed the
scratch is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_attention_09_amd as pa
import workloads as W
from gpu_cases import DEV, DecodeCase, assert_close, to_bits, to_f64


def _raw_noalloc(case: DecodeCase, S: int, out: torch.Tensor) -> int:
    """pa_decode_noalloc called with raw pointers (no binding checks)."""
    s = case.inp.spec
    NB = int(case.k_cache.shape[0])
    return pa.lib().pa_decode_noalloc(
        case.q.data_ptr(), case.k_cache.data_ptr(), case.v_cache.data_ptr(),
        case.tables.data_ptr(), case.lens.data_ptr(), ctypes.c_float(case.scale), S,
        out.data_ptr(), s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim, s.block_size, NB,
        s.max_blocks_per_seq, torch.cuda.current_stream().cuda_stream)


def _with_workspace(case: DecodeCase, S: int) -> torch.Tensor:
    s = case.inp.spec
    ws = torch.empty(max(pa.decode_workspace_size(s.num_seqs, s.num_q_heads, s.head_dim, S), 256),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(case.out)
    pa.decode(case.q, case.k_cache, case.v_cache, case.tables, case.lens, case.scale, S, out,
              workspace=ws)
    return out


@pytest.mark.gpu
def test_noalloc_two_calls_match_decode_and_oracle():
    big = DecodeCase(W.make_decode_inputs(W.CONFIGS["c2b8"]))          # 16 pieces
    small = DecodeCase(W.make_decode_inputs(W.CONFIGS["c1"]))          # then 4 pieces
    for case, S in ((big, 0), (small, 4)):
        s = case.inp.spec
        S_used = S or pa.auto_splits(s.num_seqs, s.num_kv_heads, s.max_blocks_per_seq,
                                     s.block_size, DEV)
        need = pa.decode_workspace_size(s.num_seqs, s.num_q_heads, s.head_dim, S_used)
        assert 0 < need <= pa.PA_NOALLOC_SCRATCH_BYTES
        out = torch.full_like(case.out, float("nan"))
        assert _raw_noalloc(case, S, out) == pa.PA_OK
        want = _with_workspace(case, S_used)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(out), to_bits(want)), s.name
        assert_close(to_f64(out), case.ref, what=f"noalloc {s.name}")
    # the binding's wrapper, once more on the big case after the small one
    out = torch.full_like(big.out, float("nan"))
    pa.decode_noalloc(big.q, big.k_cache, big.v_cache, big.tables, big.lens, big.scale, 0, out)
    torch.cuda.synchronize()
    assert_close(to_f64(out), big.ref, what="noalloc binding")


@pytest.mark.gpu
def test_noalloc_one_piece_needs_no_scratch():
    case = DecodeCase(W.make_decode_inputs(W.CONFIGS["c3"].with_(append=False)))
    out = torch.full_like(case.out, float("nan"))
    assert _raw_noalloc(case, 1, out) == pa.PA_OK
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), to_bits(_with_workspace(case, 1)))
    assert_close(to_f64(out), case.ref, what="noalloc S=1")


@pytest.mark.gpu
def test_noalloc_refuses_partials_beyond_the_scratch():
    """A 1024-entry table (16,384 tokens of capacity) at 256 pieces of 64
    tokens for 64 sequences of 32 q heads needs far more than the scratch:
    refused with PA_ERR_SCRATCH, the output untouched; the same call at a
    split count that fits runs."""
    spec = W.DecodeSpec("wide-table", 64, 32, 4, 128, 16, 300, 1024, context_lens=(64,) * 64,
                        seed=92)
    case = DecodeCase(W.make_decode_inputs(spec))
    assert pa.decode_workspace_size(64, 32, 128, 256) > pa.PA_NOALLOC_SCRATCH_BYTES
    out = torch.full_like(case.out, 7.0)
    before = out.clone()
    assert _raw_noalloc(case, 256, out) == pa.PA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.equal(out, before), "a refused call wrote its output"
    with pytest.raises(pa.PagedAttnError):
        pa.decode_noalloc(case.q, case.k_cache, case.v_cache, case.tables, case.lens, case.scale,
                          256, out)
    assert pa.decode_workspace_size(64, 32, 128, 2) <= pa.PA_NOALLOC_SCRATCH_BYTES
    assert _raw_noalloc(case, 2, out) == pa.PA_OK
    torch.cuda.synchronize()
    assert_close(to_f64(out), case.ref, what="noalloc wide table S=2")


def test_noalloc_argument_checks_need_no_device():
    f = pa.lib().pa_decode_noalloc
    P = 256
    args = [P, P, P, P, P, ctypes.c_float(0.1), 4, P, 2, 12, 2, 128, 16, 100, 8, None]
    bad = list(args); bad[11] = 96
    assert f(*bad) == -3                       # head_dim 96 unsupported
    bad = list(args); bad[6] = 300
    assert f(*bad) == -4                       # splits out of range
    bad = list(args); bad[7] = None
    assert f(*bad) == -1                       # no output
    bad = list(args); bad[8] = 0
    assert f(*bad) == 0                        # no sequences: nothing to do
    assert pa.lib().pa_status_string(pa.PA_ERR_SCRATCH).decode().startswith("PA_ERR_SCRATCH")
