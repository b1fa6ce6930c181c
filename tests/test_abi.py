"""The C ABI without a GPU: the library loads, exports every symbol the
headers declare, and rejects bad arguments with the documented status codes
before touching the device.  Only argument-checking paths are called here."""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_attention_09_amd as pa

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))
OK, NULL, SHAPE, UNSUP, SPLITS, WS, HIP = 0, -1, -2, -3, -4, -5, -6
P = ctypes.c_void_p(16)     # a non-NULL pointer that is never dereferenced


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(pa_\w+)\s*\(", text))
    return sorted(names)


def test_header_symbols_exported():
    names = declared_functions()
    assert len(HEADERS) == 2 and len(names) == 37, names
    L = pa.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(pa.SIGNATURES) == names


def test_status_strings():
    L = pa.lib()
    for code in (OK, NULL, SHAPE, UNSUP, SPLITS, WS, HIP):
        assert L.pa_status_string(code).decode().startswith("PA_")
    assert L.pa_version() >= 100


def _decode(**kw):
    a = dict(q=P, k=P, v=P, tables=P, lens=P, scale=0.1, S=1, out=P, B=2, Hq=12, Hkv=2, D=128,
             bs=16, NB=100, W=8, ws=None, wsb=0, stream=None)
    a.update(kw)
    return pa.lib().pa_decode(a["q"], a["k"], a["v"], a["tables"], a["lens"], a["scale"], a["S"],
                              a["out"], a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"], a["W"],
                              a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), UNSUP), (dict(D=256), UNSUP), (dict(bs=32), UNSUP), (dict(bs=8), UNSUP),
    (dict(Hq=12, Hkv=5), SHAPE), (dict(Hq=18, Hkv=2), UNSUP), (dict(Hkv=0), SHAPE),
    (dict(S=-1), SPLITS), (dict(S=257), SPLITS), (dict(NB=0), SHAPE), (dict(W=0), SHAPE),
    (dict(B=-1), SHAPE), (dict(q=None), NULL), (dict(tables=None), NULL), (dict(out=None), NULL),
    (dict(S=4), WS), (dict(S=4, ws=P, wsb=100), WS), (dict(scale=float("nan")), SHAPE),
    (dict(B=0), OK), (dict(B=0, q=None), OK),
    (dict(scale=3e38), SHAPE),                     # scale * log2(e) overflows fp32
    (dict(B=65536), SHAPE), (dict(Hq=8192, Hkv=1024), SHAPE),   # launch grid limits
])
def test_decode_argument_checks(kw, code):
    assert _decode(**kw) == code


def _multi(**kw):
    a = dict(q=P, k=P, v=P, tables=P, lens=P, scale=0.1, S=1, out=P, B=2, QL=4, Hq=28, Hkv=4,
             D=128, bs=256, NB=100, W=16, ws=None, wsb=0, stream=None)
    a.update(kw)
    return pa.lib().pa_decode_multi(a["q"], a["k"], a["v"], a["tables"], a["lens"], a["scale"],
                                    a["S"], a["out"], a["B"], a["QL"], a["Hq"], a["Hkv"], a["D"],
                                    a["bs"], a["NB"], a["W"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(QL=0), SHAPE), (dict(QL=9), SHAPE), (dict(QL=-1), SHAPE),
    (dict(Hq=32, Hkv=4, QL=5), UNSUP),            # 8 heads x 5 tokens > 32 rows
    (dict(Hq=32, Hkv=4, QL=4, B=0), OK),         # 32 rows: supported
    (dict(Hq=28, Hkv=4, QL=5, B=0), UNSUP),       # 35 rows, even with nothing to do
    (dict(D=96), UNSUP), (dict(bs=32), UNSUP), (dict(S=300), SPLITS), (dict(out=None), NULL),
    (dict(q=None), NULL), (dict(S=4), WS), (dict(S=4, ws=P, wsb=1000), WS), (dict(B=0), OK),
])
def test_decode_multi_argument_checks(kw, code):
    assert _multi(**kw) == code


def test_decode_multi_workspace_size():
    ws = pa.lib().pa_decode_multi_workspace_size
    rows = 8 * 4 * 28 * 16
    want = (rows * 128 * 4 + 255) // 256 * 256 + (rows * 4 + 255) // 256 * 256
    assert ws(8, 4, 28, 128, 16) == want
    assert ws(8, 1, 28, 128, 16) == pa.lib().pa_decode_workspace_size(8, 28, 128, 16)
    assert ws(8, 0, 28, 128, 16) == 0 and ws(8, 4, 28, 128, 1) == 0


def test_partials_and_merge_argument_checks():
    L = pa.lib()
    part = [P, P, P, P, P, 0.1, 1, 2, 12, 2, 128, 16, 100, 8, P, 1 << 20, None]
    assert L.pa_decode_partials(*part) == SPLITS          # one piece: use pa_decode
    part[6] = 4
    bad = list(part); bad[15] = 10
    assert L.pa_decode_partials(*bad) == WS
    bad = list(part); bad[10] = 80
    assert L.pa_decode_partials(*bad) == UNSUP
    merge = [P, 1 << 20, P, P, 1, 2, 12, 2, 128, 16, 8, None]
    assert L.pa_decode_merge(*merge) == SPLITS
    merge[4] = 4
    bad = list(merge); bad[1] = 16
    assert L.pa_decode_merge(*bad) == WS
    bad = list(merge); bad[3] = None
    assert L.pa_decode_merge(*bad) == NULL


def test_append_argument_checks():
    f = pa.lib().pa_reshape_and_cache
    assert f(P, P, P, None, P, 1, 10, 16, 1, 64, None) == NULL
    assert f(P, P, P, P, P, -1, 10, 16, 1, 64, None) == SHAPE
    assert f(P, P, P, P, P, 1, 10, 32, 1, 64, None) == UNSUP
    assert f(P, P, P, P, P, 1, 10, 16, 1, 80, None) == UNSUP
    assert f(None, None, None, P, P, 0, 10, 16, 1, 64, None) == OK
    assert f(None, P, P, P, P, 3, 10, 16, 1, 64, None) == NULL


def test_append_fp8_argument_checks():
    f = pa.lib().pa_reshape_and_cache_fp8
    ok = [P, P, P, P, P, 0.5, 2.0, 0, 10, 16, 1, 64, None]      # no tokens: nothing to do
    assert f(*ok) == OK
    for i, bad_scale in [(5, 0.0), (6, -1.0), (5, float("inf")), (6, float("nan")),
                         (5, 1e-45)]:                         # 1 / 1e-45 overflows fp32
        bad = list(ok); bad[i] = bad_scale
        assert f(*bad) == SHAPE, (i, bad_scale)
    bad = list(ok); bad[3] = None
    assert f(*bad) == NULL
    bad = list(ok); bad[11] = 96
    assert f(*bad) == UNSUP
    bad = list(ok); bad[7] = 2; bad[0] = None
    assert f(*bad) == NULL


def _decode_fp8(**kw):
    a = dict(q=P, k=P, v=P, tables=P, lens=P, scale=0.1, ks=0.05, vs=0.02, S=1, out=P, B=2, Hq=12,
             Hkv=2, D=128, bs=16, NB=100, W=8, ws=None, wsb=0, stream=None)
    a.update(kw)
    return pa.lib().pa_decode_fp8(a["q"], a["k"], a["v"], a["tables"], a["lens"], a["scale"],
                                  a["ks"], a["vs"], a["S"], a["out"], a["B"], a["Hq"], a["Hkv"],
                                  a["D"], a["bs"], a["NB"], a["W"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(ks=0.0), SHAPE), (dict(vs=-2.0), SHAPE), (dict(ks=float("nan")), SHAPE),
    (dict(vs=float("inf")), SHAPE), (dict(scale=1e30, ks=1e30), SHAPE),   # product overflows
    (dict(D=96), UNSUP), (dict(bs=32), UNSUP), (dict(Hq=18, Hkv=2), UNSUP),
    (dict(S=300), SPLITS), (dict(out=None), NULL), (dict(k=None), NULL), (dict(S=4), WS),
    (dict(B=0), OK), (dict(B=0, ks=0.0), SHAPE),
])
def test_decode_fp8_argument_checks(kw, code):
    assert _decode_fp8(**kw) == code


def test_prefill_argument_checks():
    f = pa.lib().pa_prefill
    args = [P, P, P, P, P, P, 0.1, 1, P, 1, 512, 28, 4, 128, 256, 100, 16, None, 0, None]
    bad = list(args); bad[13] = 100
    assert f(*bad) == UNSUP
    bad = list(args); bad[11] = 30
    assert f(*bad) == SHAPE
    bad = list(args); bad[1] = None
    assert f(*bad) == NULL
    bad = list(args); bad[7] = 4                 # split without a workspace
    assert f(*bad) == WS
    bad = list(args); bad[7] = 300
    assert f(*bad) == SPLITS
    ok0 = list(args); ok0[10] = 0
    assert f(*ok0) == OK
    bad = list(args); bad[9] = 65536              # more sequences than the grid holds
    assert f(*bad) == SHAPE
    bad = list(args); bad[11], bad[12], bad[7], bad[16] = 2048, 256, 256, 256   # 256 x 256 pieces
    assert f(*bad) == SHAPE
    bad = list(args); bad[10] = 1 << 20; bad[11], bad[12] = 4096, 512   # 2^32 query rows
    assert f(*bad) == SHAPE


def test_prefill_planning():
    L = pa.lib()
    # one 512-token chunk, 4 kv heads: 64 units -> split the 4096 keys in 4
    assert L.pa_prefill_plan_splits(1, 512, 4, 16, 256, 256) == 4
    assert L.pa_prefill_plan_splits(8, 512, 8, 16, 256, 256) == 1
    rows = 1 * 512 * 28 * 4
    want = (rows * 128 * 2 + 255) // 256 * 256 + (rows * 4 + 255) // 256 * 256   # bf16 rows
    assert L.pa_prefill_workspace_size(1, 512, 28, 128, 4) == want
    assert L.pa_prefill_workspace_size(1, 512, 28, 128, 1) == 0


def test_workspace_size():
    ws = pa.lib().pa_decode_workspace_size
    assert ws(8, 12, 128, 1) == 0 and ws(8, 12, 128, 0) == 0
    rows = 8 * 12 * 32
    want = (rows * 128 * 4 + 255) // 256 * 256 + (rows * 4 + 255) // 256 * 256
    assert ws(8, 12, 128, 32) == want
    assert ws(0, 12, 128, 4) == 0 and ws(8, 12, 128, 300) == 0


def test_plan_splits():
    plan = pa.lib().pa_decode_plan_splits
    # many (sequence, kv head) units already fill the device: one piece each
    assert plan(256, 8, 5, 256, 256) == 1
    # few units: about one workgroup per compute unit, 64-token multiples
    assert plan(8, 2, 256, 16, 256) == 16        # 16 units x 16 pieces of 256 tokens
    assert plan(8, 4, 16, 256, 256) == 8         # 32 units x 8 pieces of 512 tokens
    assert plan(64, 4, 16, 256, 256) == 1        # 256 units fill 256 compute units
    assert plan(1, 2, 256, 16, 256) == 32        # planned pieces are at least 128 tokens
    assert plan(2, 2, 256, 16, 256) == 32        # 4 units: 64 pieces would be 64 tokens
    assert plan(4, 2, 256, 16, 256) == 32        # 8 units x 32 pieces of 128 tokens
    assert plan(1, 1, 1, 16, 256) == 1           # a 16-token table: one piece
    for args in [(4, 1, 16, 16, 256), (8, 4, 16, 256, 256), (64, 4, 16, 256, 256)]:
        s = plan(*args)
        assert 1 <= s <= 256
        max_tokens = args[2] * args[3]
        c = -(-max_tokens // s)
        assert s == -(-max_tokens // max(128, (c + 63) // 64 * 64))
    assert plan(0, 2, 256, 16, 256) == SHAPE and plan(1, 2, 256, 16, 0) == SHAPE
    assert plan(1, 2, 256, 32, 256) == UNSUP


def test_plan_splits_lengths():
    """The length-aware planner on hand-worked cases: 8 compute units, block
    size 256, 16 blocks per table (pieces of 4096 / n tokens rounded up to 64).
    Workgroup s * units + x sits on compute unit (s * units + x) mod 8; with
    more workgroups than compute units the upper half of the pieces belongs
    to the mirrored units; a split adds 256 tokens for its merge."""
    plan = pa.lib().pa_decode_plan_splits
    L = lambda *v: np.array(v, np.int32)                                      # noqa: E731

    def lp(lens, hkv, cus, w=16, bs=256):
        return pa.plan_splits_lengths(lens, hkv, w, bs, cus)

    # 8 units: 1 piece reads 4096 on one compute unit; 2 pieces (mirrored)
    # put the long tails (2048) beside the short heads (512) of units 6 and 7:
    # 2560 + 256
    assert plan(8, 1, 16, 256, 8) == 1
    assert lp(L(4096, 4096, 512, 512, 512, 512, 512, 512), 1, 8) == 2
    assert lp(L(4096, 512, 512, 512), 2, 8) == 2          # two kv heads per sequence
    # the long tails land beside half-length heads: 2048 + 2048 + 256 > 4096
    assert lp(L(4096, 4096, 4096, 4096, 2048, 2048, 2048, 2048), 1, 8) == 1
    # a saving below the merge's 256 tokens: heads 2048 beside tails <= 252
    assert lp(L(2300, 2200, 2200, 2200, 2200, 2200, 2200, 2200), 1, 8) == 1
    # 6 units, equal lengths: the shape-only plan takes 2 pieces, but they put
    # 2048 + 2048 on four compute units (+ 256), more than one piece each
    assert plan(6, 1, 16, 256, 8) == 2
    assert lp(L(*[4096] * 6), 1, 8) == 1
    # ... and 2 pieces when the lengths are uneven: 300 + 2048 + 256
    assert lp(L(4096, 4096, 300, 300, 300, 300), 1, 8) == 2
    # 4 units, one long: 4 pieces of 1024 (16 workgroups, pieces 2 and 3
    # mirrored) put at most 16 + 1024 on a compute unit, + 256 = 1296; 3
    # pieces of 1408 give 1408 + 256, 2 pieces 2048 + 256, 1 piece 4096
    assert plan(4, 1, 16, 256, 8) == 2
    assert lp(L(4096, 16, 16, 16), 1, 8) == 4
    # the same lengths without the long one: every plan reads at most 16
    # tokens on a compute unit, so no split and no merge
    assert lp(L(16, 16, 16, 16), 1, 8) == 1
    # workgroups of the shape-only plan beyond two per compute unit: that plan
    assert lp(L(*[4096] + [16] * 23), 1, 8) == plan(24, 1, 16, 256, 8) == 1
    # lengths beyond the table capacity count as the capacity
    assert lp(L(9999, 9999, 512, 512, 512, 512, 512, 512), 1, 8) == 2
    # errors: no lengths, and the shapes pa_decode_plan_splits refuses
    f = pa.lib().pa_decode_plan_splits_lengths
    assert f(None, 8, 1, 16, 256, 8) == NULL
    assert f(P, 0, 1, 16, 256, 8) == SHAPE and f(P, 8, 1, 16, 32, 8) == UNSUP
    # a compute-unit count beyond what the planner models
    lens = L(4096, 512)
    ptr = lens.ctypes.data_as(ctypes.c_void_p)
    assert f(ptr, 2, 1, 16, 256, 1 << 16) >= 1 and f(ptr, 2, 1, 16, 256, (1 << 16) + 1) == SHAPE


def test_binding_constants_match_header():
    text = open(os.path.join(INCLUDE, "pagedattn.h")).read()
    defines = dict(re.findall(r"#define (PA_MAX_\w+) (\d+)", text))
    assert set(defines) == {"PA_MAX_SPLITS", "PA_MAX_QUERY_TOKENS", "PA_MAX_SEQS", "PA_MAX_HEADS"}
    for name, value in defines.items():
        assert getattr(pa, name) == int(value), name
