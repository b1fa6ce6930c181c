"""GPU parity of the chunked-prefill MFMA kernel against the fp64 oracle.

The chunk's own K/V rows are appended through slot_mapping first (the
library's append), then pa_prefill runs.  Tolerance as for decode:
|gpu - oracle| <= 1e-2 + 1e-2 |oracle| elementwise.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_09_amd as pa
import workloads as W
from gpu_cases import DEV, assert_close, bf16_tensor, device_pool, to_f64

pytestmark = pytest.mark.gpu


class PrefillCase:
    def __init__(self, spec: W.PrefillSpec, with_oracle=True):
        inp = W.make_prefill_inputs(spec)
        self.inp, self.spec = inp, spec
        self.k_cache, self.v_cache = device_pool(inp.pool)
        self.q = bf16_tensor(inp.q)
        self.cu = torch.from_numpy(inp.cu_seqlens_q).to(DEV)
        self.tables = torch.from_numpy(inp.block_tables).to(DEV)
        self.lens = torch.from_numpy(inp.context_lens).to(DEV)
        self.out = torch.empty_like(self.q)
        self.max_q = int(max(spec.chunk_lens))
        pa.reshape_and_cache(bf16_tensor(inp.new_k), bf16_tensor(inp.new_v),
                             torch.from_numpy(inp.slot_mapping).to(DEV), self.k_cache,
                             self.v_cache)
        self.ref = self.oracle() if with_oracle else None

    def oracle(self):
        p = self.inp.pool
        bs = self.spec.block_size
        lut = {int(x): i for i, x in enumerate(p.ids)}
        slots = np.array([lut[int(s) // bs] * bs + int(s) % bs for s in self.inp.slot_mapping],
                         np.int64)
        kc, vc = oracle.append(self.inp.new_k, self.inp.new_v, slots, p.k, p.v)
        ct = p.compact_tables(self.inp.block_tables, self.inp.poison_block)
        return oracle.prefill(self.inp.q, self.inp.cu_seqlens_q, kc, vc, ct,
                              self.inp.context_lens, self.inp.scale)

    def run(self, S=0, max_q=None):
        pa.prefill(self.q, self.cu, self.k_cache, self.v_cache, self.tables, self.lens,
                   float(self.inp.scale), self.out, self.max_q if max_q is None else max_q,
                   num_splits=S)
        torch.cuda.synchronize()
        return to_f64(self.out)


@pytest.fixture(scope="module")
def chunk512():
    return PrefillCase(W.PREFILL_CONFIGS["c5p"])


@pytest.mark.parametrize("S", [0, 1, 2, 3, 8])
def test_chunk_512_of_4096(chunk512, S):
    """28 q / 4 kv heads, head_dim 128, bs 256: a 512-token chunk over a
    3584-token cached prefix, split counts automatic and explicit."""
    maxe, rms = assert_close(chunk512.run(S), chunk512.ref, what=f"chunk512 S={S}")
    print(f"S={S}: max abs err {maxe:.3e} rms {rms:.3e}")


@pytest.mark.parametrize("D,G,bs,chunks,totals", [
    (128, 7, 256, (37, 1, 64), (300, 1, 64)),       # ragged; a 1-token chunk; prefix 0
    (128, 2, 16, (100, 33), (1000, 33)),
    (64, 1, 16, (65, 7), (129, 520)),
    (64, 8, 256, (31,), (2100,)),
    (128, 5, 16, (96,), (96,)),                       # whole prompt, no prefix
])
def test_prefill_shapes(D, G, bs, chunks, totals):
    W_ = -(-max(totals) // bs)
    nb = sum(-(-t // bs) for t in totals) + 5
    spec = W.PrefillSpec(f"p{D}_{G}_{bs}", 2 * G, 2, D, bs, nb, W_, chunk_lens=chunks,
                         total_lens=totals, seed=D * 10 + G)
    case = PrefillCase(spec)
    for S in (1, 2, 0):
        assert_close(case.run(S), case.ref, what=f"D{D} G{G} bs{bs} S{S}")


def test_many_ragged_sequences():
    """40 sequences in one call: chunks of 0..100 tokens (empty chunks and
    empty sequences included) over prefixes of 0..500 tokens, bs 16, a
    max_q_len above every chunk, several split counts: every row of every
    sequence reaches the oracle, through one merge grid row per sequence."""
    rng = np.random.default_rng(40)
    chunks = [int(x) for x in rng.choice([0, 1, 5, 31, 32, 33, 64, 100], size=40)]
    totals = [c + int(rng.integers(0, 501)) * (i % 3 != 0) for i, c in enumerate(chunks)]
    chunks[7], totals[7] = 0, 0                        # an empty sequence
    bs = 16
    W_ = -(-max(totals) // bs)
    nb = sum(-(-t // bs) for t in totals) + 5
    spec = W.PrefillSpec("many", 12, 4, 128, bs, nb, W_, chunk_lens=tuple(chunks),
                         total_lens=tuple(totals), seed=41)
    case = PrefillCase(spec)
    pa.check_prefill(case.inp.cu_seqlens_q, case.inp.context_lens, max(chunks) + 7)
    pa.check_tables(case.inp.block_tables, case.inp.context_lens, nb, bs)
    for S in (1, 3, 0, 16):
        assert_close(case.run(S, max_q=max(chunks) + 7), case.ref, what=f"many S={S}")


@pytest.mark.parametrize("scale", [0.0, -0.0883883461356163])
def test_prefill_scale_sign(scale):
    """Zero and negative scales take the explicitly scaled (non-folded)
    softmax path on every tile."""
    spec = W.PrefillSpec("pscale", 14, 2, 128, 16, 60, 48, chunk_lens=(70, 3),
                         total_lens=(700, 40), scale=scale, seed=71)
    case = PrefillCase(spec)
    for S in (1, 3):
        assert_close(case.run(S), case.ref, what=f"prefill scale {scale} S{S}")


def test_prefill_workspace_needs_no_initialisation():
    """A prefill workspace full of NaN bytes: rows past each chunk and pieces
    past each row's causal end are never written and never read."""
    spec = W.PrefillSpec("wsnan", 14, 2, 128, 16, 200, 160, chunk_lens=(70, 0, 3, 33),
                         total_lens=(2500, 9, 40, 33), seed=81)
    case = PrefillCase(spec)
    max_q = 80
    for S in (2, 5):
        n = pa.prefill_workspace_size(4, max_q, 14, 128, S)
        ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=DEV)
        pa.prefill(case.q, case.cu, case.k_cache, case.v_cache, case.tables, case.lens,
                   float(case.inp.scale), case.out, max_q, num_splits=S, workspace=ws)
        torch.cuda.synchronize()
        assert_close(to_f64(case.out), case.ref, what=f"prefill NaN workspace S={S}")


def test_one_token_chunk_equals_decode():
    """A chunk of one query is a decode step."""
    spec = W.PrefillSpec("one", 28, 4, 128, 256, 40, 16, chunk_lens=(1, 1, 1),
                         total_lens=(4096, 513, 2), seed=5)
    case = PrefillCase(spec, with_oracle=False)
    got = case.run(0)
    out = torch.empty((3, 28, 128), dtype=torch.bfloat16, device=DEV)
    pa.decode(case.q, case.k_cache, case.v_cache, case.tables, case.lens, float(case.inp.scale),
              0, out)
    torch.cuda.synchronize()
    dec = to_f64(out)
    assert (np.abs(got - dec) <= 2 ** -7 * np.abs(dec) + 1e-3).all()


def test_chunking_invariance():
    """Prefilling a prompt as three chunks (each appended, then attended)
    matches prefilling it at once, row for row, within rounding."""
    spec = W.PrefillSpec("whole", 14, 2, 128, 16, 80, 64, chunk_lens=(700,),
                         total_lens=(700,), seed=17)
    case = PrefillCase(spec)
    whole = case.run(0)
    assert_close(whole, case.ref, what="whole prompt")
    parts = []
    for a, b in ((0, 200), (200, 450), (450, 700)):
        cu = torch.tensor([0, b - a], dtype=torch.int32, device=DEV)
        lens = torch.tensor([b], dtype=torch.int32, device=DEV)
        out = torch.empty((b - a, 14, 128), dtype=torch.bfloat16, device=DEV)
        pa.prefill(case.q[a:b].contiguous(), cu, case.k_cache, case.v_cache, case.tables, lens,
                   float(case.inp.scale), out, b - a)
        torch.cuda.synchronize()
        parts.append(to_f64(out))
    chunked = np.concatenate(parts)
    assert_close(chunked, case.ref, what="three chunks")
    assert (np.abs(chunked - whole) <= 2 ** -7 * np.abs(whole) + 2e-3).all()


def test_poison_not_read_and_finite(chunk512):
    """Pool blocks no sequence references, and slots past the context, hold
    NaN: the output stays finite."""
    assert np.isfinite(chunk512.run(0)).all()


def test_prefill_workspace_lives_on_the_call_stream(chunk512, monkeypatch):
    """As for decode: the binding's own prefill workspace is allocated on the
    call's stream when that stream is not the current one."""
    s = torch.cuda.Stream()
    seen = []
    real_empty = torch.empty

    def spy(*args, **kw):
        if kw.get("dtype") == torch.uint8:
            seen.append(torch.cuda.current_stream().cuda_stream)
        return real_empty(*args, **kw)

    s.wait_stream(torch.cuda.current_stream())
    out = torch.empty_like(chunk512.q)
    monkeypatch.setattr(torch, "empty", spy)
    pa.prefill(chunk512.q, chunk512.cu, chunk512.k_cache, chunk512.v_cache, chunk512.tables,
               chunk512.lens, float(chunk512.inp.scale), out, chunk512.max_q, num_splits=4,
               stream=s)
    monkeypatch.setattr(torch, "empty", real_empty)
    assert seen == [s.cuda_stream], seen
    junk = torch.full((8 << 20,), 3, dtype=torch.uint8, device=DEV)
    s.synchronize()
    torch.cuda.synchronize()
    assert_close(to_f64(out), chunk512.ref, what="prefill workspace on a non-current stream")
    del junk
