#!/usr/bin/env python3
"""Paged-KV decode benchmark on one MI355X.

One step = the decode hot path for one batch: append each sequence's new
K/V row at its last token's slot and run the paged split-KV decode over the
whole context (pa_append_decode: the append fused into the split pass, then
the log-sum-exp merge).  The same step as separate calls
(pa_reshape_and_cache, then pa_decode) is timed too and reported as
config.unfused_graph_us_per_step.

Default workload: 12 q / 2 kv heads (Qwen2.5-1.5B attention shape), head_dim
128, block_size 16, batch 8, every context 4096 tokens, bf16, automatic split
count.  Inputs are synthetic N(0,1) bf16 drawn on the device from a fixed
seed; block tables are random permutations of a shuffled pool.

Method
  * Cold HBM: steps rotate over R disjoint sets of blocks (at least
    --rotate-gib GiB of K/V between two uses of the same block), so no call
    finds its K/V in the 256 MB last-level cache; the timed steps continue
    the rotation where the warm-up stopped.  Building the inputs ends with
    one read of every rotation, so timed steps meet warm address
    translations, as in a running engine, and not first touches.
  * The K timed steps are issued from the host through the C ABI
    (pa_append_decode with prebuilt arguments) between two events, with
    torch.cuda.synchronize() on both sides, the queue primed by a device-side
    sleep (20 ms, or 20 us per step for more than 1000, time for the host to
    enqueue all K steps) so that the
    events bracket the K steps' GPU work.  The same K steps captured into one HIP graph and
    replayed are reported beside (config.graph_us_per_step); a replay adds a
    fixed cost of several microseconds, which few steps do not amortise.
  * The dominant kernel (the split-KV pass) is timed with HIP events around
    back-to-back launches on the current stream, the queue primed by a
    device-side sleep so the events bracket GPU work and not host gaps.
  * value = algorithmic bytes of a step / seconds per step, in GB/s.
    Algorithmic bytes: every K and V element of every context token once per
    kv head, q and out once, the table entries used, the lengths, plus the
    append's read and write of the new rows and its slot ids.
  * roofline.achieved = algorithmic decode bytes per launch / average
    split-kernel duration; peak = 8000 GB/s (MI355X HBM3E).
  * cpu_baseline: the fp64 numpy oracle on host copies of the same workload,
    one worker process per host core (at most 16), one BLAS thread each,
    for about --cpu-seconds; the whole call in one thread is nested.  The
    same leg checks the benchmarked calls' results against the oracle (the
    fused decode step and the mixed prefill + decode step).
  * split_kv_gain: the ctx-4096 batches at the automatic split count against
    one piece per (sequence, kv head).
  * device_pass: from the committed step trace (profiles/decode_<workload>_
    step_trace), the split and merge kernels' medians and p90s and their sum
    per step, when the trace matches the current kernels.
  * equal_share_bound: the random-length batches' tokens laid out as equal
    lengths, one workgroup per (compute unit, kv head): the fastest any split
    into equal token shares could run, beside the drawn lengths' kernel.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# steps timed, and warm-up steps, per extra workload (every workload but the
# headline one), whatever --steps and --warmup are: a replayed graph's fixed
# cost spread over this many steps is small
EXTRA_STEPS = 100
EXTRA_WARMUP = 20
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["paged_kv_attention_09_amd/csrc/pa_decode.hip",
                  "paged_kv_attention_09_amd/csrc/pa_device.hpp",
                  "paged_kv_attention_09_amd/csrc/pa_kernels.hpp"]
PREFILL_SOURCES = ["paged_kv_attention_09_amd/csrc/pa_prefill.hip",
                   "paged_kv_attention_09_amd/csrc/pa_device.hpp",
                   "paged_kv_attention_09_amd/csrc/pa_kernels.hpp"]
# a mixed step runs the append, prefill and decode kernels
MIXED_SOURCES = KERNEL_SOURCES + ["paged_kv_attention_09_amd/csrc/pa_prefill.hip",
                                  "paged_kv_attention_09_amd/csrc/pa_append.hip"]


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="c2b8",
                   choices=["c2b8", "c2b1", "c3", "c4", "c5d", "c5p", "c2b8f8", "c4f8"],
                   help="decode workload timed; c5p (the prefill chunk) and the fp8-pool "
                        "workloads only with --kernel-loop")
    p.add_argument("--splits", type=int, default=0, help="0 = automatic")
    p.add_argument("--rotate-gib", type=float, default=2.0)
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--others", default="c2b1,c3,c4,c5d,c5p,c5mix,c2b8q2,c2b8q4,c3q4,"
                                         "c2b8f8,c3f8,c4f8,c2b8q4f8,c5pf8,c5mixf8",
                   help="comma list of extra workloads measured into 'workloads' ('' = none)")
    p.add_argument("--kernel-loop", type=int, default=0,
                   help="profiling mode: launch only the split kernel this many times and exit")
    p.add_argument("--step-loop", type=int, default=0,
                   help="profiling mode: capture this many whole fused steps (append + split "
                        "pass + merge) in one HIP graph, replay it once and exit")
    p.add_argument("--graph", action="store_true",
                   help="with --kernel-loop: capture the launches in one HIP graph and replay it, "
                        "so they run back to back as in the timed region (a tracer's per-launch "
                        "host work then no longer spaces them out)")
    p.add_argument("--sweep-splits", default="",
                   help="tuning mode: comma list of split counts; prints us/step per workload")
    p.add_argument("--ingest-trace", nargs=3, metavar=("DIR", "NAME", "COMMAND"),
                   help="write profiles/NAME.md from a rocprofv3 --stats output directory")
    p.add_argument("--ingest-counters", nargs=7,
                   metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR",
                            "COPY_MIB", "KERNEL_CMD", "COPY_CMD"),
                   help="write profiles/decode_split_<workload>_hbm_counters.{json,md}")
    p.add_argument("--ingest-sq", nargs=4, metavar=("DIR", "KERNEL", "NAME", "COMMAND"),
                   help="write profiles/NAME.{md,json} from a rocprofv3 --pmc pass of SQ counters")
    p.add_argument("--copy-calibration", type=int, default=0,
                   help="profiling mode: run a plain device copy of this many MiB, 20 times")
    return p.parse_args(argv)


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    """Hash of the kernel sources' code: // comments and blank lines are left
    out, so that a comment edit does not mark counters as stale."""
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------


class DecodeWorkload:
    """Device-resident inputs of one decode workload with R block rotations."""

    def __init__(self, spec, rotate_gib: float, splits: int, seed: int = 1234, q_len: int = 1,
                 kv_fp8: bool = False):
        import numpy as np
        import torch

        import paged_kv_attention_09_amd as pa
        import workloads as W

        self.spec = spec
        dev = torch.device("cuda:0")
        self.dev = dev
        self.lens_np = W.draw_context_lens(spec)
        bs, Hkv, D, B, Hq = spec.block_size, spec.num_kv_heads, spec.head_dim, spec.num_seqs, \
            spec.num_q_heads
        nblk = [(int(L) + bs - 1) // bs for L in self.lens_np]
        per_rot = sum(nblk)
        elem = 1 if kv_fp8 else 2
        kv_bytes = int(self.lens_np.sum()) * Hkv * D * elem * 2
        self.R = max(1, math.ceil(rotate_gib * 2**30 / kv_bytes))
        NB = max(spec.num_blocks, self.R * per_rot + 1)
        self.NB = NB
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        shape = (NB, Hkv, bs, D) if kv_fp8 else (NB, bs, Hkv, D)   # fp8 pools are head-major
        self.kv_fp8 = kv_fp8
        self.k_scale, self.v_scale = 0.25, 0.25
        dt = torch.uint8 if kv_fp8 else torch.bfloat16
        self.k_cache = torch.empty(shape, dtype=dt, device=dev)
        self.v_cache = torch.empty(shape, dtype=dt, device=dev)
        step = max(1, (256 << 20) // (bs * Hkv * D * elem))
        for i in range(0, NB, step):
            j = min(NB, i + step)
            for t in (self.k_cache, self.v_cache):
                if kv_fp8:
                    # fp8 codes: random sign and mantissa, exponent field 4..8
                    # (magnitudes 2^-3 .. 3.75), never NaN
                    sm = torch.randint(0, 256, t[i:j].shape, generator=g, device=dev,
                                       dtype=torch.int16) & 0x87
                    ex = torch.randint(4, 9, t[i:j].shape, generator=g, device=dev,
                                       dtype=torch.int16) << 3
                    t[i:j] = (sm | ex).to(torch.uint8)
                else:
                    t[i:j].normal_(generator=g)
        perm = torch.randperm(NB, generator=g, device=dev).cpu().numpy()
        W_ = spec.max_blocks_per_seq
        tables, slots = [], []
        for r in range(self.R):
            ids = perm[r * per_rot:(r + 1) * per_rot]
            t = np.full((B, W_), int(perm[-1]), np.int32)
            off = 0
            for b, n in enumerate(nblk):
                t[b, :n] = ids[off:off + n]
                off += n
            L = self.lens_np.astype(np.int64)
            last = t[np.arange(B), (L - 1) // bs].astype(np.int64) * bs + (L - 1) % bs
            tables.append(torch.from_numpy(t).to(dev))
            slots.append(torch.from_numpy(last).to(dev))
        self.tables, self.slots = tables, slots
        self.lens = torch.from_numpy(self.lens_np).to(dev)
        self.q_len = q_len
        qshape = (B, Hq, D) if q_len == 1 else (B, q_len, Hq, D)
        self.q = torch.randn(qshape, generator=g, device=dev).to(torch.bfloat16)
        self.new_k = torch.randn((B, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
        self.new_v = torch.randn((B, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
        self.out = torch.empty(qshape, dtype=torch.bfloat16, device=dev)
        self.scale = float(spec.scale_f32)
        self.S = splits if splits > 0 else pa.auto_splits(B, Hkv, W_, bs, dev)
        ws = pa.decode_multi_workspace_size(B, q_len, Hq, D, self.S)
        self.ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
        self.pa = pa
        # q and out once per query token; the cache once whatever q_len; fp8
        # pools move one byte per K/V element
        self.decode_bytes = (W.algorithmic_decode_bytes(self.lens_np, Hq, Hkv, D, bs)
                             + (q_len - 1) * B * Hq * D * 2 * 2)
        if kv_fp8:
            self.decode_bytes -= int(self.lens_np.sum()) * Hkv * D * 2
        self.append_bytes = B * Hkv * D * 2 * 2 * 2 + B * 8
        self.decode_flop = 4 * D * Hq * int(self.lens_np.sum())
        self.read_every_rotation()

    def read_every_rotation(self):
        """Part of making the inputs resident: one read of every rotation's
        blocks through its tables (a decode of the workload's kind without
        the append, which writes only the output and the workspace), so that
        timed steps meet the address translations a running engine has
        rather than first touches."""
        import torch
        if self.q_len > 1:
            read = self.step_multi_fp8 if self.kv_fp8 else self.step_multi
        else:
            read = self.step_fp8 if self.kv_fp8 else self.kernel
        for r in range(self.R):
            read(r)
        torch.cuda.synchronize()

    def set_splits(self, S: int):
        import torch
        self.S = S
        ws = self.pa.decode_workspace_size(self.spec.num_seqs, self.spec.num_q_heads,
                                           self.spec.head_dim, S)
        self.ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=self.dev)

    def step_multi(self, r: int):
        """Multi-token decode: q_len query tokens per sequence, causal."""
        self.pa.decode_multi(self.q, self.k_cache, self.v_cache, self.tables[r], self.lens,
                             self.scale, self.S, self.out, workspace=self.ws)

    def step_fp8(self, r: int):
        """Single-token decode over fp8 pools."""
        self.pa.decode_fp8(self.q, self.k_cache, self.v_cache, self.tables[r], self.lens,
                           self.scale, self.k_scale, self.v_scale, self.S, self.out,
                           workspace=self.ws)

    def step_multi_fp8(self, r: int):
        """Multi-token decode over fp8 pools."""
        self.pa.decode_multi_fp8(self.q, self.k_cache, self.v_cache, self.tables[r], self.lens,
                                 self.scale, self.k_scale, self.v_scale, self.S, self.out,
                                 workspace=self.ws)

    def step_plain(self, r: int):
        """Single-token decode without the append."""
        self.pa.decode(self.q, self.k_cache, self.v_cache, self.tables[r], self.lens, self.scale,
                       self.S, self.out, workspace=self.ws)

    def step(self, r: int):
        """Append of each sequence's new row fused with the decode."""
        self.pa.append_decode(self.q, self.new_k, self.new_v, self.k_cache, self.v_cache,
                              self.tables[r], self.lens, self.scale, self.S, self.out,
                              workspace=self.ws)

    def step_unfused(self, r: int):
        """The same step as separate calls: slot-mapped append, then decode."""
        pa = self.pa
        pa.reshape_and_cache(self.new_k, self.new_v, self.slots[r], self.k_cache, self.v_cache)
        pa.decode(self.q, self.k_cache, self.v_cache, self.tables[r], self.lens, self.scale,
                  self.S, self.out, workspace=self.ws)

    def kernel(self, r: int):
        """The dominant kernel alone: the split pass (or the whole decode when
        there is a single piece, which is then one kernel)."""
        pa = self.pa
        if self.S > 1:
            pa.decode_partials(self.q, self.k_cache, self.v_cache, self.tables[r], self.lens,
                               self.scale, self.S, self.ws)
        else:
            pa.decode(self.q, self.k_cache, self.v_cache, self.tables[r], self.lens, self.scale,
                      1, self.out, workspace=self.ws)


class PrefillWorkload:
    """A prompt chunk (causal, over its cached prefix) and, optionally, the
    decode sequences that share the step with it, in one pool with R block
    rotations.  step() is the mixed-batch step: slot-mapped append of the
    chunk's K/V, the chunked prefill on MFMA, then the fused append + decode
    of the decode sequences."""

    def __init__(self, pspec, dspec, rotate_gib: float, seed: int = 4321, kv_fp8: bool = False):
        import numpy as np
        import torch

        import paged_kv_attention_09_amd as pa
        import workloads as W

        self.pa = pa
        self.kv_fp8 = kv_fp8
        self.k_scale, self.v_scale = 0.25, 0.25
        dev = torch.device("cuda:0")
        self.dev = dev
        bs, Hkv, D, Hq = pspec.block_size, pspec.num_kv_heads, pspec.head_dim, pspec.num_q_heads
        assert dspec is None or (dspec.block_size, dspec.num_kv_heads, dspec.head_dim,
                                 dspec.num_q_heads) == (bs, Hkv, D, Hq)
        self.plens = np.asarray(pspec.total_lens, np.int32)
        self.chunks = np.asarray(pspec.chunk_lens, np.int32)
        self.dlens = W.draw_context_lens(dspec) if dspec is not None else np.zeros(0, np.int32)
        P, B = len(self.plens), len(self.dlens)
        pblk = [-(-int(L) // bs) for L in self.plens]
        dblk = [-(-int(L) // bs) for L in self.dlens]
        per_rot = sum(pblk) + sum(dblk)
        elem = 1 if kv_fp8 else 2
        kv_bytes = (int(self.plens.sum()) + int(self.dlens.sum())) * Hkv * D * elem * 2
        self.R = max(1, math.ceil(rotate_gib * 2**30 / kv_bytes))
        NB = max(pspec.num_blocks, self.R * per_rot + 1)
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        shape = (NB, Hkv, bs, D) if kv_fp8 else (NB, bs, Hkv, D)   # fp8 pools are head-major
        dt = torch.uint8 if kv_fp8 else torch.bfloat16
        self.k_cache = torch.empty(shape, dtype=dt, device=dev)
        self.v_cache = torch.empty(shape, dtype=dt, device=dev)
        step = max(1, (256 << 20) // (bs * Hkv * D * elem))
        for i in range(0, NB, step):
            j = min(NB, i + step)
            for t in (self.k_cache, self.v_cache):
                if kv_fp8:
                    # fp8 codes: random sign and mantissa, exponent field 4..8
                    sm = torch.randint(0, 256, t[i:j].shape, generator=g, device=dev,
                                       dtype=torch.int16) & 0x87
                    ex = torch.randint(4, 9, t[i:j].shape, generator=g, device=dev,
                                       dtype=torch.int16) << 3
                    t[i:j] = (sm | ex).to(torch.uint8)
                else:
                    t[i:j].normal_(generator=g)
        perm = torch.randperm(NB, generator=g, device=dev).cpu().numpy()
        Wp, Wd = pspec.max_blocks_per_seq, (dspec.max_blocks_per_seq if dspec else 1)
        self.ptables, self.dtables, self.cslots, self.dslots = [], [], [], []
        for r in range(self.R):
            ids = perm[r * per_rot:(r + 1) * per_rot]
            tp = np.full((P, Wp), int(perm[-1]), np.int32)
            td = np.full((max(B, 1), Wd), int(perm[-1]), np.int32)
            off = 0
            for b, nblk in enumerate(pblk):
                tp[b, :nblk] = ids[off:off + nblk]
                off += nblk
            for b, nblk in enumerate(dblk):
                td[b, :nblk] = ids[off:off + nblk]
                off += nblk
            slots = []
            for b in range(P):
                for t in range(int(self.plens[b] - self.chunks[b]), int(self.plens[b])):
                    slots.append(int(tp[b, t // bs]) * bs + t % bs)
            self.ptables.append(torch.from_numpy(tp).to(dev))
            self.dtables.append(torch.from_numpy(td).to(dev))
            if B:
                L = self.dlens.astype(np.int64)
                last = td[np.arange(B), (L - 1) // bs].astype(np.int64) * bs + (L - 1) % bs
                self.dslots.append(torch.from_numpy(last).to(dev))
            self.cslots.append(torch.from_numpy(np.asarray(slots, np.int64)).to(dev))
        Tq = int(self.chunks.sum())
        self.Tq = Tq
        cu = np.zeros(P + 1, np.int32)
        cu[1:] = np.cumsum(self.chunks)
        self.cu = torch.from_numpy(cu).to(dev)
        self.plens_t = torch.from_numpy(self.plens).to(dev)
        self.max_q = int(self.chunks.max())
        self.q = torch.randn((Tq, Hq, D), generator=g, device=dev).to(torch.bfloat16)
        self.ck = torch.randn((Tq, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
        self.cv = torch.randn((Tq, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
        self.out = torch.empty_like(self.q)
        self.scale = float(pspec.scale_f32)
        self.S = pa.prefill_auto_splits(P, self.max_q, Hkv, Wp, bs, dev)
        self.ws = torch.zeros(max(pa.prefill_workspace_size(P, self.max_q, Hq, D, self.S), 256),
                              dtype=torch.uint8, device=dev)
        pos = np.concatenate([np.arange(int(L - n), int(L)) for L, n in zip(self.plens, self.chunks)])
        self.flop = 4 * D * Hq * int((pos + 1).sum())
        self.append_bytes = Tq * Hkv * D * 2 * 2 * 2 + Tq * 8
        self.prefill_bytes = (int(self.plens.sum()) * Hkv * D * elem * 2 + 2 * Tq * Hq * D * 2)
        if B:
            self.dlens_t = torch.from_numpy(self.dlens).to(dev)
            self.dq = torch.randn((B, Hq, D), generator=g, device=dev).to(torch.bfloat16)
            self.dk = torch.randn((B, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
            self.dv = torch.randn((B, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
            self.dout = torch.empty_like(self.dq)
            self.dS = pa.auto_splits(B, Hkv, Wd, bs, dev)
            self.dws = torch.zeros(max(pa.decode_workspace_size(B, Hq, D, self.dS), 256),
                                   dtype=torch.uint8, device=dev)
            # the decode's algorithmic bytes plus the fused append of one row per
            # sequence (bf16 rows read, written as bf16 or as fp8 codes); fp8
            # pools move one byte per K/V element
            self.decode_bytes = W.algorithmic_decode_bytes(self.dlens, Hq, Hkv, D, bs) + \
                B * Hkv * D * 2 * (2 + elem)
            if kv_fp8:
                self.decode_bytes -= int(self.dlens.sum()) * Hkv * D * 2
        self.B = B
        # the chunk's K/V must be in the pool before any prefill-only timing;
        # then one read of every rotation (prefill, and the decode, whose
        # fused append rewrites the same rows), as for the decode workloads
        for r in range(self.R):
            self.append_chunk(r)
        for r in range(self.R):
            self.prefill(r)
            if self.B:
                self.decode(r)
        torch.cuda.synchronize()

    def order_decode(self, order, splits: int):
        """Launch the decode sequences in `order` (host indices) with `splits`
        pieces: their rows of q, new K/V, tables and lengths permuted, the
        work unchanged."""
        import numpy as np
        import torch
        pa = self.pa
        perm = torch.from_numpy(np.asarray(order, np.int64)).to(self.dev)
        self.dq, self.dk, self.dv = (t[perm].contiguous() for t in (self.dq, self.dk, self.dv))
        self.dtables = [t[perm].contiguous() for t in self.dtables]
        self.dlens = self.dlens[np.asarray(order)]
        self.dlens_t = torch.from_numpy(self.dlens).to(self.dev)
        self.dS = splits
        B, Hq, D = (int(x) for x in self.dq.shape)
        self.dws = torch.zeros(max(pa.decode_workspace_size(B, Hq, D, splits), 256),
                               dtype=torch.uint8, device=self.dev)

    def append_chunk(self, r):
        if self.kv_fp8:
            self.pa.reshape_and_cache_fp8(self.ck, self.cv, self.cslots[r], self.k_cache,
                                          self.v_cache, self.k_scale, self.v_scale)
        else:
            self.pa.reshape_and_cache(self.ck, self.cv, self.cslots[r], self.k_cache,
                                      self.v_cache)

    def prefill(self, r):
        if self.kv_fp8:
            self.pa.prefill_fp8(self.q, self.cu, self.k_cache, self.v_cache, self.ptables[r],
                                self.plens_t, self.scale, self.k_scale, self.v_scale, self.out,
                                self.max_q, num_splits=self.S, workspace=self.ws)
        else:
            self.pa.prefill(self.q, self.cu, self.k_cache, self.v_cache, self.ptables[r],
                            self.plens_t, self.scale, self.out, self.max_q, num_splits=self.S,
                            workspace=self.ws)

    def decode(self, r):
        if self.kv_fp8:
            # fp8 pools: the quantising append fused into the decode launch
            self.pa.append_decode_fp8(self.dq, self.dk, self.dv, self.k_cache, self.v_cache,
                                      self.dtables[r], self.dlens_t, self.scale, self.k_scale,
                                      self.v_scale, self.dS, self.dout, workspace=self.dws)
        else:
            self.pa.append_decode(self.dq, self.dk, self.dv, self.k_cache, self.v_cache,
                                  self.dtables[r], self.dlens_t, self.scale, self.dS, self.dout,
                                  workspace=self.dws)

    def step(self, r):
        self.append_chunk(r)
        self.prefill(r)
        if self.B:
            self.decode(r)


def time_graph(fn, R: int, steps: int, warmup: int) -> float:
    """Average milliseconds per call of `steps` calls fn(r) captured in one
    HIP graph after `warmup` eager calls, r running over the R rotations
    without restarting (the timed calls continue where the warm-up stopped)."""
    import torch
    for i in range(warmup):
        fn(i % R)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn((warmup + i) % R)      # the rotation continues after the warm-up
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    return primed_events(g.replay) / steps


def measure_prefill(args, steps, warmup, with_decode: bool, kv_fp8: bool = False):
    import numpy as np
    import workloads as W
    wl = PrefillWorkload(W.PREFILL_CONFIGS["c5p"], W.CONFIGS["c5d"] if with_decode else None,
                         args.rotate_gib, kv_fp8=kv_fp8)
    ms_pf = time_graph(wl.prefill, wl.R, steps, warmup)
    name = W.PREFILL_CONFIGS["c5p"].name + (" with " + W.CONFIGS["c5d"].name if with_decode else "")
    rec = {"workload": name + (", fp8 pools" if kv_fp8 else ""),
           "prefill_us": ms_pf * 1e3, "prefill_tflops": wl.flop / (ms_pf * 1e-3) / 1e12,
           "prefill_splits": wl.S, "prefill_gflop": wl.flop / 1e9, "query_rows": wl.Tq,
           "rotations": wl.R}
    if with_decode:
        ms_step = time_graph(wl.step, wl.R, steps, warmup)
        ms_dec = time_graph(wl.decode, wl.R, steps, warmup)
        ms_app = time_graph(wl.append_chunk, wl.R, steps, warmup)
        rec.update({"us_per_step": ms_step * 1e3, "decode_us": ms_dec * 1e3,
                    "decode_gbps": wl.decode_bytes / (ms_dec * 1e-3) / 1e9,
                    "append_us": ms_app * 1e3, "decode_splits": wl.dS,
                    "step": ("quantising append of the 512-token chunk, MFMA prefill over fp8 "
                             "pools, fused quantising append + fp8 decode of 64") if kv_fp8 else
                            "append 512-token chunk, MFMA prefill, fused append + decode of 64"})
        # the same step with the decode batch launched longest first (the block
        # manager's order: lengths descending, ties in order) and its split
        # count from the host's lengths in that order
        dspec = W.CONFIGS["c5d"]
        order = np.argsort(-wl.dlens.astype(np.int64), kind="stable")
        S_lf = wl.pa.auto_splits_lengths(wl.dlens[order], dspec.num_kv_heads,
                                         dspec.max_blocks_per_seq, dspec.block_size, wl.dev)
        wl.order_decode(order, S_lf)
        ms_step_lf = time_graph(wl.step, wl.R, steps, warmup)
        ms_dec_lf = time_graph(wl.decode, wl.R, steps, warmup)
        rec.update({"longest_first_decode_splits": S_lf,
                    "longest_first_us_per_step": ms_step_lf * 1e3,
                    "longest_first_decode_us": ms_dec_lf * 1e3})
    if kv_fp8:
        rec["kv"] = "fp8 e4m3, per-tensor scales"
    return wl, rec


def sleep_cycles_for(ms: float) -> int:
    """Calibrate torch.cuda._sleep (device spin) to roughly `ms` milliseconds."""
    import torch
    n = 1_000_000
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    torch.cuda._sleep(n)
    e.record()
    torch.cuda.synchronize()
    per = max(s.elapsed_time(e), 1e-3) / n
    return int(ms / per)


_SLEEP_CYCLES = None


def primed_events(issue, sleep_ms: float = 20.0) -> float:
    """Milliseconds between two HIP events around the GPU work `issue()`
    enqueues on the current stream, the queue primed by a device-side sleep
    of about `sleep_ms` so that the host's enqueue time (a graph launch, or
    eager calls) is spent while the GPU sleeps and the events bracket GPU
    work only.  Synchronised on both sides."""
    import torch
    global _SLEEP_CYCLES
    if _SLEEP_CYCLES is None:
        _SLEEP_CYCLES = sleep_cycles_for(20.0)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(_SLEEP_CYCLES * max(1.0, sleep_ms / 20.0)))
    s.record()
    issue()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e)


def time_kernel_events(fn, n: int, rotations: int):
    """HIP events around n back-to-back launches of `fn(i)` on the current
    stream, the queue primed by a device-side sleep so that the launches run
    back to back on the GPU and host enqueue time is not measured.  Returns
    the average milliseconds per launch."""
    import torch
    fn(0)
    torch.cuda.synchronize()
    cyc = sleep_cycles_for(max(20.0, 0.1 * n))
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(cyc)
    s.record()
    for i in range(n):
        fn((1 + i) % rotations)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / n


def time_steps_eager(wl, steps: int, warmup: int) -> float:
    """The fused append + decode step launched from the host every time (no
    graph), through the raw C function with prebuilt ctypes arguments so the
    binding's Python checks are not timed.  Returns milliseconds per step
    (HIP events around the loop, the queue primed by a device-side sleep as
    for the graph) and the host's issue time per call."""
    import ctypes
    import torch
    f = wl.pa.lib().pa_append_decode
    sp = torch.cuda.current_stream().cuda_stream
    B, Hq, D = (int(x) for x in wl.q.shape)
    NB, bs, Hkv, _ = (int(x) for x in wl.k_cache.shape)
    W_ = int(wl.tables[0].shape[1])
    args = [(wl.q.data_ptr(), wl.new_k.data_ptr(), wl.new_v.data_ptr(), wl.k_cache.data_ptr(),
             wl.v_cache.data_ptr(), t.data_ptr(), wl.lens.data_ptr(), ctypes.c_float(wl.scale),
             wl.S, wl.out.data_ptr(), B, Hq, Hkv, D, bs, NB, W_, wl.ws.data_ptr(),
             wl.ws.numel(), sp) for t in wl.tables]
    for i in range(warmup):
        assert f(*args[i % wl.R]) == 0
    torch.cuda.synchronize()
    host = [0.0]

    def issue():
        t0 = time.perf_counter()
        for i in range(steps):
            f(*args[(warmup + i) % wl.R])      # the rotation continues after the warm-up
        host[0] = time.perf_counter() - t0

    # a head start in which the host enqueues all the steps (≈ 10 µs each)
    ms = primed_events(issue, sleep_ms=max(20.0, 0.02 * steps))
    return ms / steps, host[0] * 1e3 / steps


def measure_multilayer(args, layers: int = 28, steps: int = 20, warmup: int = 3):
    """A whole decode step's attention, as a model runs it: `layers` fused
    append + decode calls back to back, layer l over its own K/V (block set
    l of the workload's rotations).  Timed three ways: issued from Python
    through the binding (what an engine loop does), issued through the raw C
    function with prebuilt arguments (the least host work possible), and
    replayed from one captured graph.  Milliseconds come from HIP events
    around `steps` steps; host issue time from the host clock."""
    import ctypes
    import torch
    import workloads as W
    res = {}
    for name in ("c2b1", "c2b8"):
        wl = DecodeWorkload(W.CONFIGS[name], args.rotate_gib, 0)
        rots = [l % wl.R for l in range(layers)]
        f = wl.pa.lib().pa_append_decode
        sp = torch.cuda.current_stream().cuda_stream
        B, Hq, D = (int(x) for x in wl.q.shape)
        NB, bs, Hkv, _ = (int(x) for x in wl.k_cache.shape)
        W_ = int(wl.tables[0].shape[1])
        raw = [(wl.q.data_ptr(), wl.new_k.data_ptr(), wl.new_v.data_ptr(),
                wl.k_cache.data_ptr(), wl.v_cache.data_ptr(), wl.tables[r].data_ptr(),
                wl.lens.data_ptr(), ctypes.c_float(wl.scale), wl.S, wl.out.data_ptr(), B, Hq,
                Hkv, D, bs, NB, W_, wl.ws.data_ptr(), wl.ws.numel(), sp) for r in rots]

        def step_binding():
            for r in rots:
                wl.step(r)

        def step_raw():
            for a in raw:
                f(*a)

        def timed(fn):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            t0 = time.perf_counter()
            for _ in range(steps):
                fn()
            host = time.perf_counter() - t0
            e.record()
            torch.cuda.synchronize()
            return s.elapsed_time(e) * 1e3 / steps, host * 1e6 / steps

        eager_b, host_b = timed(step_binding)
        eager_r, host_r = timed(step_raw)
        step_binding()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step_binding()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            g.replay()
        e.record()
        torch.cuda.synchronize()
        graph_us = s.elapsed_time(e) * 1e3 / steps
        res[name] = {"workload": W.CONFIGS[name].name, "layers": layers, "splits": wl.S,
                     "eager_binding_us_per_step": round(eager_b, 2),
                     "eager_binding_host_us_per_step": round(host_b, 2),
                     "eager_raw_us_per_step": round(eager_r, 2),
                     "eager_raw_host_us_per_step": round(host_r, 2),
                     "graph_us_per_step": round(graph_us, 2),
                     "graph_saving_vs_binding": round(1 - graph_us / eager_b, 4),
                     "graph_saving_vs_raw": round(1 - graph_us / eager_r, 4)}
        print(f"[bench] {layers}-layer step {name}: graph {graph_us:.1f} us, eager through the "
              f"binding {eager_b:.1f} us (host {host_b:.1f}), raw C calls {eager_r:.1f} us",
              file=sys.stderr, flush=True)
        del g, wl
        torch.cuda.empty_cache()
    return res


def time_steps_graph(wl, steps: int, warmup: int, fused: bool = True):
    """Warm up eagerly, capture `steps` steps in one graph, replay it between events."""
    import torch
    step = wl.step if fused else wl.step_unfused
    for i in range(warmup):
        step(i % wl.R)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step((warmup + i) % wl.R)      # the rotation continues after the warm-up
    torch.cuda.synchronize()
    g.replay()          # first replay uploads the graph
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = primed_events(g.replay)
    wall = time.perf_counter() - t0
    return ms / steps, wall


def _short_kernel(name: str) -> str:
    for k in ("decode_split_kernel", "decode_combine64_kernel", "decode_combine_kernel",
              "append_fp8_kernel", "append_kernel",
              "prefill_kernel", "prefill_merge_kernel", "spin_kernel", "read_probe_kernel"):
        if k in name:
            tmpl = name[name.find(k):]
            return tmpl[:tmpl.find("(")] if "(" in tmpl else tmpl
    return name[:60]


def _read_csv(directory: str, suffix: str):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {directory}")
    return rows


def ingest_trace(directory: str, out_name: str, command: str):
    """rocprofv3 --stats CSV -> a short markdown summary under profiles/."""
    import statistics
    rows = _read_csv(directory, "kernel_stats.csv")
    # per-dispatch durations for the median and 90th percentile
    durs = {}
    for r in _read_csv(directory, "kernel_trace.csv"):
        k = _short_kernel(r["Kernel_Name"])
        durs.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    srcs = (MIXED_SOURCES if "mixed" in out_name else
            PREFILL_SOURCES if "prefill" in out_name else KERNEL_SOURCES)
    src_hash = kernel_source_hash(srcs)
    lines = [f"# Kernel durations: {out_name}", "", "Command (run from /tmp with TMPDIR=/tmp):", "",
             "```", command, "```", "",
             "| kernel | calls | avg us | median us | p90 us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|---|---|"]
    rec = {"command": command, "kernel_source_sha256_16": src_hash, "kernels": {}}
    for r in rows:
        k = _short_kernel(r["Name"])
        if not k.startswith(("decode", "append", "prefill", "read_probe")):
            continue
        d = sorted(durs.get(k, [float("nan")]))
        p90 = d[min(len(d) - 1, int(0.9 * len(d)))]
        lines.append(f"| `{k}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{statistics.median(d):.2f} | {p90:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
        rec["kernels"][k] = {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                             "median_us": statistics.median(d), "p90_us": p90}
    # a decode step's device time: each merge dispatch paired with the split
    # dispatch before it (trace order), as the sum of the two durations and as
    # the span from the split's start to the merge's end; only for a trace of
    # one split-kernel variant (one workload)
    trace = sorted(_read_csv(directory, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    splits = {_short_kernel(r["Kernel_Name"]) for r in trace
              if _short_kernel(r["Kernel_Name"]).startswith("decode_split")}
    if len(splits) != 1:
        trace = []
    sums, spans, last = [], [], None
    for r in trace:
        k = _short_kernel(r["Kernel_Name"])
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        if k.startswith("decode_split"):
            last = (t0, t1)
        elif k.startswith("decode_combine") and last is not None:
            sums.append(((last[1] - last[0]) + (t1 - t0)) / 1e3)
            spans.append((t1 - last[0]) / 1e3)
            last = None
    if sums:
        sums.sort()
        spans.sort()
        pick = lambda d, q: d[min(len(d) - 1, int(q * len(d)))]
        lines += ["", f"Per step ({len(sums)} split + merge pairs): split + merge durations median "
                      f"{statistics.median(sums):.2f} us, p90 {pick(sums, 0.9):.2f} us; from the "
                      f"split's start to the merge's end median {statistics.median(spans):.2f} us, "
                      f"p90 {pick(spans, 0.9):.2f} us."]
        rec["step"] = {"pairs": len(sums), "sum_median_us": statistics.median(sums),
                       "sum_p90_us": pick(sums, 0.9), "span_median_us": statistics.median(spans),
                       "span_p90_us": pick(spans, 0.9)}
    lines += ["", f"Kernel sources ({', '.join(os.path.basename(x) for x in srcs)}) "
                  f"sha256[:16], comments excluded: {src_hash}"]
    path = os.path.join(PROFILES, out_name + ".md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(PROFILES, out_name + ".json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(path)


def load_step_trace(out_name: str):
    """The per-step device pass of a committed step trace summary (split and
    merge kernels of graph-replayed fused steps), if its kernel sources match
    the current ones; else None."""
    path = os.path.join(PROFILES, out_name + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash() or "step" not in rec:
        return None
    res = {"summary": f"profiles/{out_name}.md"}
    for k, v in rec["kernels"].items():
        tag = "split" if k.startswith("decode_split") else (
            "merge" if k.startswith("decode_combine") else None)
        if tag:
            res[f"{tag}_median_us"] = round(v["median_us"], 3)
            res[f"{tag}_p90_us"] = round(v["p90_us"], 3)
    res.update({k: round(v, 3) if isinstance(v, float) else v for k, v in rec["step"].items()})
    return res


def load_trace(out_name: str, kernel_prefix: str):
    """(average, median) microseconds of the first kernel whose name starts
    with kernel_prefix in a committed trace summary, if its kernel sources
    match the current ones; else None."""
    path = os.path.join(PROFILES, out_name + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    for k, v in rec["kernels"].items():
        if k.startswith(kernel_prefix):
            return v["avg_us"], v["median_us"], k
    return None


def ingest_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib: int,
                    workload: str, command_kernel: str, command_copy: str):
    """FETCH_SIZE / WRITE_SIZE per dispatch of the split kernel, scaled by what
    the same counters read for a plain device copy of known size."""
    import statistics

    def med(rows, counter, pick):
        v = [float(r["Counter_Value"]) for r in rows
             if r["Counter_Name"] == counter and pick(r["Kernel_Name"])]
        if not v:
            raise SystemExit(f"no {counter} rows")
        return statistics.median(v)

    is_split = lambda n: "decode_split_kernel" in n                            # noqa: E731
    fetch = med(_read_csv(fetch_dir, "counter_collection.csv"), "FETCH_SIZE", is_split)
    write = med(_read_csv(write_dir, "counter_collection.csv"), "WRITE_SIZE", is_split)
    copy_rows_f = _read_csv(copy_fetch_dir, "counter_collection.csv")
    copy_rows_w = _read_csv(copy_write_dir, "counter_collection.csv")
    big = lambda rows, c: max(float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == c)  # noqa: E731
    copy_bytes = copy_mib << 20
    f_fetch = copy_bytes / (big(copy_rows_f, "FETCH_SIZE") * 1024)
    f_write = copy_bytes / (big(copy_rows_w, "WRITE_SIZE") * 1024)
    import workloads as W
    spec = W.CONFIGS[workload]
    alg = W.algorithmic_decode_bytes(W.draw_context_lens(spec), spec.num_q_heads,
                                     spec.num_kv_heads, spec.head_dim, spec.block_size)
    hbm = fetch * 1024 * f_fetch + write * 1024 * f_write
    rec = {"kernel": "decode_split_kernel", "workload": spec.name,
           "fetch_size_kib_per_dispatch": fetch, "write_size_kib_per_dispatch": write,
           "copy_calibration_bytes": copy_bytes, "fetch_scale": round(f_fetch, 4),
           "write_scale": round(f_write, 4), "hbm_bytes_per_launch": int(hbm),
           "algorithmic_bytes_per_launch": alg, "ratio_to_algorithmic": round(hbm / alg, 4),
           "kernel_source_sha256_16": kernel_source_hash(),
           "commands": [command_kernel.replace("PMC", "FETCH_SIZE"),
                        command_kernel.replace("PMC", "WRITE_SIZE"),
                        command_copy.replace("PMC", "FETCH_SIZE"),
                        command_copy.replace("PMC", "WRITE_SIZE")]}
    base = os.path.join(PROFILES, f"decode_split_{workload}_hbm_counters")
    with open(base + ".json", "w") as f:
        json.dump(rec, f, indent=1)
    with open(base + ".md", "w") as f:
        f.write(f"# HBM traffic of decode_split_kernel, {spec.name}\n\n"
                f"Counters per dispatch (median over the launches), each pass its own run:\n\n"
                + "".join(f"    {c}\n" for c in rec["commands"]) +
                f"\n| quantity | value |\n|---|---|\n"
                f"| FETCH_SIZE (KiB/dispatch, raw) | {fetch:.1f} |\n"
                f"| WRITE_SIZE (KiB/dispatch, raw) | {write:.1f} |\n"
                f"| plain copy of {copy_mib} MiB: bytes / (FETCH_SIZE x 1024) | {f_fetch:.3f} |\n"
                f"| plain copy of {copy_mib} MiB: bytes / (WRITE_SIZE x 1024) | {f_write:.3f} |\n"
                f"| HBM bytes per launch (scaled) | {int(hbm)} |\n"
                f"| algorithmic bytes per launch | {alg} |\n"
                f"| ratio | {hbm / alg:.3f} |\n"
                f"| kernel sources sha256[:16] | {rec['kernel_source_sha256_16']} |\n")
    print(base + ".json")


def ingest_sq(directory: str, kernel: str, out_name: str, command: str, flop_per_call=None):
    """Per-dispatch medians of SQ/GRBM counters for one kernel, from one
    rocprofv3 --pmc pass, with rocprofv3's own derived formulas:
    MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs) and
    MfmaFlopsBF16 = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512."""
    import statistics
    rows = [r for r in _read_csv(directory, "counter_collection.csv") if kernel in r["Kernel_Name"]]
    if not rows:
        raise SystemExit(f"no rows for {kernel}")
    per = {}
    for r in rows:
        per.setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
        per[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    med = {c: statistics.median(v.values()) for c, v in per.items()}
    # rocprofv3 writes each counter summed over its hardware instances; the
    # GRBM counters have one instance per XCD and rocprofv3's own formulas
    # take their maximum, i.e. about the sum over the XCD count.
    gpu = [a for a in _read_csv(directory, "agent_info.csv") if a.get("Agent_Type") == "GPU"][0]
    nxcc, simds, cus = int(gpu["Num_Xcc"]), int(gpu["Simd_Count"]), int(gpu["Cu_Count"])
    for c in list(med):
        if c.startswith("GRBM_"):
            med[c] = med[c] / nxcc
    durs = {}
    for r in rows:
        durs[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    med["dispatch_ns"] = statistics.median(durs.values())
    title = "SQ counters" if all(c.startswith(("SQ_", "GRBM_")) for c in per) else "Counters"
    lines = [f"# {title}: {out_name}", "", f"Kernel `{kernel}`; per-dispatch medians over "
             f"{len(next(iter(per.values())))} dispatches.", "", "Command (run from /tmp with "
             "TMPDIR=/tmp):", "", "```", command, "```", "", "| counter | value |", "|---|---|"]
    lines += [f"| {c}{' (per XCD)' if c.startswith('GRBM_') else ''} | {v:.0f} |"
              for c, v in sorted(med.items())]
    rec = {"kernel": kernel, "counters": med, "command": command}
    if "SQ_VALU_MFMA_BUSY_CYCLES" in med and "GRBM_GUI_ACTIVE" in med:
        util = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (med["GRBM_GUI_ACTIVE"] * simds)
        rec["mfma_util"] = util
        lines.append(f"| MfmaUtil = MFMA busy / (GUI active x {simds} SIMDs) | {100 * util:.1f} % |")
    if "SQ_BUSY_CU_CYCLES" in med:
        # SQ_BUSY_CU_CYCLES, summed over the CUs, counts the shader clocks each
        # CU has waves resident (a long kernel filling every CU reads ~0.9 x
        # CUs x its clocks).  GRBM_GUI_ACTIVE spans more than a short dispatch
        # under counter collection, so the fraction uses the dispatch's own
        # duration at the nominal 2.4 GHz shader clock.
        frac = med["SQ_BUSY_CU_CYCLES"] / (med["dispatch_ns"] * 2.4 * cus)
        rec["active_cu_frac"] = frac
        rec["cu_busy_cycles_per_ns"] = med["SQ_BUSY_CU_CYCLES"] / med["dispatch_ns"]
        lines.append(f"| active-CU fraction = SQ_BUSY_CU_CYCLES / (dispatch ns x 2.4 GHz x {cus} CUs) | "
                     f"{100 * frac:.1f} % |")
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in med:
        ex = med["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        rec["mfma_flop_executed"] = ex
        lines.append(f"| bf16 MFMA flop executed per dispatch (MOPS x 512) | {ex:.4g} |")
        lines.append(f"| executed MFMA rate over the dispatch | {ex / med['dispatch_ns'] / 1e3:.0f} "
                     "TFLOP/s |")
        if flop_per_call:
            rec["flop_algorithmic"] = flop_per_call
            lines.append(f"| algorithmic flop per call (unmasked pairs) | {flop_per_call:.4g} |")
            lines.append(f"| executed / algorithmic | {ex / flop_per_call:.3f} |")
            lines.append(f"| algorithmic rate over the dispatch | "
                         f"{flop_per_call / med['dispatch_ns'] / 1e3:.0f} TFLOP/s |")
    if "TCC_HIT_sum" in med and "TCC_MISS_sum" in med:
        h, m = med["TCC_HIT_sum"], med["TCC_MISS_sum"]
        rec["l2_hit_rate"] = h / max(h + m, 1.0)
        lines.append(f"| L2 hit rate = TCC_HIT / (TCC_HIT + TCC_MISS) | {100 * h / max(h + m, 1.0):.1f} % |")
    if "TCC_EA0_RDREQ_LEVEL_sum" in med and "TCC_EA0_RDREQ_sum" in med:
        # Little's law over the L2 -> memory read queue: the per-cycle sum of
        # outstanding reads over the requests gives their mean latency
        lat = med["TCC_EA0_RDREQ_LEVEL_sum"] / max(med["TCC_EA0_RDREQ_sum"], 1.0)
        rec["l2_read_latency_cycles"] = lat
        lines.append(f"| mean L2 -> memory read latency = RDREQ_LEVEL / RDREQ | {lat:.0f} cycles |")
        if "GRBM_GUI_ACTIVE" in med:
            inflight = med["TCC_EA0_RDREQ_LEVEL_sum"] / max(med["GRBM_GUI_ACTIVE"], 1.0)
            rec["l2_reads_in_flight"] = inflight
            lines.append(f"| mean L2 -> memory reads in flight, all L2 channels | {inflight:.0f} |")
    if "SQ_LDS_BANK_CONFLICT" in med and "SQ_LDS_IDX_ACTIVE" in med:
        c, a = med["SQ_LDS_BANK_CONFLICT"], med["SQ_LDS_IDX_ACTIVE"]
        rec["lds_bank_conflict_rate"] = c / max(a - c, 1.0)
        lines.append(f"| LDS bank conflict cycles / conflict-free LDS cycles | {c / max(a - c, 1.0):.4f} |")
    rec["kernel_source_sha256_16"] = kernel_source_hash(
        PREFILL_SOURCES if "prefill" in kernel else KERNEL_SOURCES)
    lines.append(f"| kernel sources sha256[:16] | {rec['kernel_source_sha256_16']} |")
    with open(os.path.join(PROFILES, out_name + ".md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(PROFILES, out_name + ".json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(os.path.join(PROFILES, out_name + ".md"))


def load_traffic(workload: str):
    path = os.path.join(PROFILES, f"decode_split_{workload}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline_single(spec, seconds: float):
    """The oracle, as it stands, on host copies of the whole workload call,
    in this process with one BLAS thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import workloads as W

    inp = W.make_decode_inputs(spec)
    ct = inp.pool.compact_tables(inp.block_tables, inp.poison_block)
    per_call = W.algorithmic_decode_bytes(inp.context_lens, spec.num_q_heads, spec.num_kv_heads,
                                          spec.head_dim, spec.block_size)
    n, t = 0, 0.0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            oracle.decode(inp.q, inp.pool.k, inp.pool.v, ct, inp.context_lens, inp.scale)
            n += 1
            t = time.perf_counter() - t0
            if t >= seconds:
                break
    return {"value": round(per_call * n / t / 1e9, 4), "unit": "GB/s", "cores": 1,
            "sample": f"fp64 numpy oracle decode of the full {spec.name} call "
                      f"({spec.num_seqs} seqs, {int(np.sum(inp.context_lens))} tokens), "
                      f"{n} calls in {t:.1f} s, 1 BLAS thread",
            "us_per_call": round(t / n * 1e6, 1)}


def parity_record(spec):
    """The benchmarked call (fused append + decode at the automatic split
    count) on host-drawn inputs of the same workload, against the oracle:
    error statistics for the JSON line.  Part of the oracle leg."""
    import numpy as np
    import torch

    import oracle
    import paged_kv_attention_09_amd as pa
    import workloads as W

    s = spec.with_(append=True)
    inp = W.make_decode_inputs(s)
    dev = torch.device("cuda:0")

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)

    shape = (s.num_blocks,) + inp.pool.k.shape[1:]
    kc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    vc = torch.full_like(kc, float("nan"))
    ids = torch.from_numpy(inp.pool.ids).to(dev)
    kc.index_copy_(0, ids, bf16(inp.pool.k))
    vc.index_copy_(0, ids, bf16(inp.pool.v))
    B, Hkv, D, bs = s.num_seqs, s.num_kv_heads, s.head_dim, s.block_size
    sel = np.nonzero(inp.context_lens > 0)[0]
    nk = np.zeros((B, Hkv, D), np.uint16)
    nv = np.zeros_like(nk)
    nk[sel], nv[sel] = inp.new_k, inp.new_v
    q = bf16(inp.q)
    out = torch.empty_like(q)
    tables = torch.from_numpy(inp.block_tables).to(dev)
    lens = torch.from_numpy(inp.context_lens).to(dev)
    S = pa.auto_splits(B, Hkv, s.max_blocks_per_seq, bs, dev)
    pa.append_decode(q, bf16(nk), bf16(nv), kc, vc, tables, lens, float(inp.scale), S, out)
    torch.cuda.synchronize()
    lut = {int(x): i for i, x in enumerate(inp.pool.ids)}
    slots = np.array([lut[int(t) // bs] * bs + int(t) % bs for t in inp.slot_mapping], np.int64)
    k2, v2 = oracle.append(inp.new_k, inp.new_v, slots, inp.pool.k, inp.pool.v)
    ct = inp.pool.compact_tables(inp.block_tables, inp.poison_block)
    ref = oracle.decode(inp.q, k2, v2, ct, inp.context_lens, inp.scale)
    got = oracle.bf16_bits_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    err = np.abs(got - ref)
    ratio = err / (1e-2 + 1e-2 * np.abs(ref))
    return {"call": "pa_append_decode", "splits": S, "outputs": int(ref.size),
            "max_abs_err": float(err.max()), "rms_err": float(np.sqrt((err ** 2).mean())),
            "max_err_over_tolerance": float(ratio.max()), "tolerance": "1e-2 + 1e-2 |oracle|",
            "within_tolerance": bool(np.isfinite(got).all() and (ratio <= 1.0).all()),
            "inputs": "the workload drawn on the host (workloads module), K/V bf16 N(0,1), "
                      "unreferenced pool NaN-poisoned; fp64 oracle"}


def mixed_parity_record(kv_fp8: bool):
    """The benchmarked mixed step (PrefillWorkload.step: append of the 512-row
    chunk, prefill, fused append + decode of the 64 sequences, one pool, one
    stream), run once outside any timed region on the benchmark's own
    device-drawn inputs (one rotation), against the oracle on host copies of
    those inputs: the referenced blocks of both pools bit for bit, the prefill
    and decode rows within 1e-2 + 1e-2 |oracle|.  Part of the oracle leg."""
    import numpy as np
    import torch

    import oracle
    import oracle.kv_fp8 as O8
    import workloads as W

    wl = PrefillWorkload(W.PREFILL_CONFIGS["c5p"], W.CONFIGS["c5d"], 0.0, kv_fp8=kv_fp8)
    bs = int(wl.k_cache.shape[2] if kv_fp8 else wl.k_cache.shape[1])
    host = lambda t: t.detach().cpu().numpy()                            # noqa: E731
    bits = lambda t: host(t.view(torch.int16)).view(np.uint16)           # noqa: E731
    ptab, dtab = host(wl.ptables[0]), host(wl.dtables[0])
    used = [int(x) for b, L in enumerate(wl.plens) for x in ptab[b, :-(-int(L) // bs)]]
    used += [int(x) for b, L in enumerate(wl.dlens) for x in dtab[b, :-(-int(L) // bs)]]
    ids = np.asarray(sorted(set(used)), np.int64)
    lut = np.full(int(wl.k_cache.shape[0]), 0, np.int64)
    lut[ids] = np.arange(len(ids))
    ids_t = torch.from_numpy(ids).to(wl.dev)
    pool = (lambda t: host(t[ids_t])) if kv_fp8 else (lambda t: bits(t[ids_t]))
    k0, v0 = pool(wl.k_cache), pool(wl.v_cache)
    wl.out.fill_(float("nan"))
    wl.dout.fill_(float("nan"))
    wl.step(0)
    torch.cuda.synchronize()
    k1, v1 = pool(wl.k_cache), pool(wl.v_cache)
    slots = np.concatenate([host(wl.cslots[0]), host(wl.dslots[0])])
    cslots = lut[slots // bs] * bs + slots % bs
    nk = np.concatenate([bits(wl.ck), bits(wl.dk)])
    nv = np.concatenate([bits(wl.cv), bits(wl.dv)])
    pct, dct = lut[ptab].astype(np.int32), lut[dtab].astype(np.int32)
    if kv_fp8:
        ka, va = O8.append_fp8(nk, nv, cslots, k0, v0, wl.k_scale, wl.v_scale)
        ref_p = O8.prefill_fp8(bits(wl.q), host(wl.cu), ka, va, pct, wl.plens, wl.scale,
                               wl.k_scale, wl.v_scale)
        ref_d = O8.decode_fp8(bits(wl.dq), ka, va, dct, wl.dlens, wl.scale, wl.k_scale,
                              wl.v_scale)
    else:
        ka, va = oracle.append(nk, nv, cslots, k0, v0)
        ref_p = oracle.prefill(bits(wl.q), host(wl.cu), ka, va, pct, wl.plens, wl.scale)
        ref_d = oracle.decode(bits(wl.dq), ka, va, dct, wl.dlens, wl.scale)
    rec = {"call": "append chunk, prefill, fused append + decode (one pool, one stream)",
           "kv": "fp8 e4m3" if kv_fp8 else "bf16",
           "pools_bit_exact": bool(np.array_equal(k1, ka) and np.array_equal(v1, va)),
           "tolerance": "1e-2 + 1e-2 |oracle|"}
    ok = rec["pools_bit_exact"]
    for part, got_t, ref in (("prefill", wl.out, ref_p), ("decode", wl.dout, ref_d)):
        got = oracle.bf16_bits_to_f64(bits(got_t))
        err = np.abs(got - ref)
        ratio = err / (1e-2 + 1e-2 * np.abs(ref))
        fin = bool(np.isfinite(got).all())
        rec[part] = {"outputs": int(ref.size), "max_abs_err": float(np.nanmax(err)),
                     "rms_err": float(np.sqrt(np.nanmean(err ** 2))),
                     "max_err_over_tolerance": float(np.nanmax(ratio)), "finite": fin}
        ok = ok and fin and bool((ratio <= 1.0).all())
    rec["within_tolerance"] = ok
    rec["inputs"] = ("the benchmark's own device-drawn mixed-step inputs (one rotation), copied "
                     "to the host before the step; fp64 oracle")
    del wl
    torch.cuda.empty_cache()
    return rec


def cpu_model() -> str:
    """The host CPU's model string and its family/model/stepping, from
    /proc/cpuinfo."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" in line:
                    k, v = (x.strip() for x in line.split(":", 1))
                    fields.setdefault(k, v)
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    extra = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping")
                      if k in fields)
    return f"{name} ({extra})" if extra else name


def oracle_job(name: str, pairs, seconds: float):
    """Worker body of the parallel CPU baseline, run in its own process: the
    oracle over each (sequence, kv head) sub-call in `pairs` of workload
    `name`, round robin, for about `seconds`.  A sub-call is the oracle's
    decode of one sequence restricted to one kv head and its group of q heads
    (the oracle itself, unchanged, on a slice of the inputs).  Prints one JSON
    line: the sub-calls' algorithmic bytes processed and the seconds taken."""
    from threadpoolctl import threadpool_limits

    import oracle
    import workloads as W
    spec = W.CONFIGS[name]
    inp = W.make_decode_inputs(spec)
    ct = inp.pool.compact_tables(inp.block_tables, inp.poison_block)
    G = spec.group
    subs = []
    for b, g in pairs:
        lens = inp.context_lens[b:b + 1]
        subs.append((inp.q[b:b + 1, g * G:(g + 1) * G], inp.pool.k[:, :, g:g + 1],
                     inp.pool.v[:, :, g:g + 1], ct[b:b + 1], lens,
                     W.algorithmic_decode_bytes(lens, G, 1, spec.head_dim, spec.block_size)))
    done, n = 0, 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            q, k, v, tab, lens, nbytes = subs[n % len(subs)]
            oracle.decode(q, k, v, tab, lens, inp.scale)
            done += nbytes
            n += 1
            t = time.perf_counter() - t0
            if t >= seconds and n >= len(subs):
                break
    print(json.dumps({"bytes": done, "seconds": t, "subcalls": n}), flush=True)


def cpu_baseline(spec, seconds: float):
    """The oracle timed on the host's cores: one worker process per core (at
    most 16), each with one BLAS thread,
    sharing the workload's (sequence, kv head) sub-calls; value = their
    algorithmic bytes over the slowest worker's time.  The same oracle on the
    whole call in one thread is nested as `single_thread`."""
    import subprocess
    name = _config_key(spec)
    pairs = [(b, g) for b in range(spec.num_seqs) for g in range(spec.num_kv_heads)]
    visible = len(os.sched_getaffinity(0))
    workers = max(1, min(visible, 16, len(pairs)))
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    procs = []
    for w in range(workers):
        mine = pairs[w::workers]
        code = (f"import bench; bench.oracle_job({name!r}, {mine!r}, {seconds!r})")
        procs.append(subprocess.Popen([sys.executable, "-c", code], cwd=ROOT, env=env,
                                      stdout=subprocess.PIPE, text=True))
    res = []
    try:
        for p in procs:
            out, _ = p.communicate()
            if p.returncode != 0:
                raise RuntimeError(f"oracle worker failed with status {p.returncode}")
            res.append(json.loads(out.strip().splitlines()[-1]))
    finally:
        # no worker outlives the call, also when one of them failed
        for p in procs:
            if p.poll() is None:
                p.kill()
                p.wait()
    total = sum(r["bytes"] for r in res)
    wall = max(r["seconds"] for r in res)
    rec = {"value": round(total / wall / 1e9, 4), "unit": "GB/s", "cores": workers,
           "kind": "oracle", "cpu_model": cpu_model(), "host_cores_visible": visible,
           "sample": f"fp64 numpy oracle over the {len(pairs)} (sequence, kv head) sub-calls of "
                     f"the {spec.name} call, {workers} worker processes with one BLAS thread "
                     f"each, about {seconds:.0f} s each ({sum(r['subcalls'] for r in res)} "
                     f"sub-calls); input generation not timed",
           "us_per_call": round(wall / (sum(r["subcalls"] for r in res) / len(pairs)) * 1e6, 1)}
    rec["single_thread"] = cpu_baseline_single(spec, seconds / 2)
    return rec


def _config_key(spec):
    import workloads as W
    return next(k for k, v in W.CONFIGS.items() if v == spec)


def measure(name, args, steps, warmup, with_kernel=True):
    import workloads as W
    spec = W.CONFIGS[name]
    wl = DecodeWorkload(spec, args.rotate_gib, args.splits)
    # the step issued through the C ABI from the host, exactly `steps` of them
    # between two events (the queue primed so the host's enqueue time stays
    # outside); the same steps replayed from one HIP graph are reported beside
    ms_step, _ = time_steps_eager(wl, steps, warmup)
    bytes_step = wl.decode_bytes + wl.append_bytes
    rec = {"workload": spec.name, "key": name, "ms_per_step": ms_step,
           "gbps": bytes_step / (ms_step * 1e-3) / 1e9,
           "us_per_call": ms_step * 1e3, "splits": wl.S, "rotations": wl.R,
           "decode_bytes": wl.decode_bytes, "append_bytes": wl.append_bytes,
           "context_tokens": int(wl.lens_np.sum())}
    ms_graph, _ = time_steps_graph(wl, steps, 2)
    rec["graph_us_per_step"] = ms_graph * 1e3
    ms_unfused, _ = time_steps_graph(wl, steps, 2, fused=False)
    rec["unfused_graph_us_per_step"] = ms_unfused * 1e3
    # graph against eager issue: two adjacent (eager, graph) pairs, so that a
    # drift of the GPU's pace between legs timed apart does not enter the
    # comparison
    pairs, hosts = [], []
    for _ in range(2):
        ms_e, ms_host = time_steps_eager(wl, steps, warmup)
        ms_g, _ = time_steps_graph(wl, steps, 2)
        pairs.append((ms_e, ms_g))
        hosts.append(ms_host)
    rec["eager_us_per_step"] = sum(e for e, _ in pairs) / 2 * 1e3
    rec["graph_us_per_step_paired"] = sum(g for _, g in pairs) / 2 * 1e3
    rec["host_issue_us_per_call"] = sum(hosts) / 2 * 1e3
    rec["graph_saving"] = sum(1.0 - g / e for e, g in pairs) / 2
    if with_kernel:
        avg = time_kernel_events(wl.kernel, min(200, max(50, steps)), wl.R)
        rec["kernel_avg_us"] = avg * 1e3
        rec["kernel_gbps"] = wl.decode_bytes / (avg * 1e-3) / 1e9
    if spec.len_range is not None:
        rec.update(measure_drawn_order_planned(wl, steps, warmup))
        rec.update(measure_longest_first(wl, steps, warmup))
    return wl, rec


def load_sq(out_name: str, key: str):
    """A derived value of a committed counter summary whose kernel sources
    match the current ones, else None."""
    path = os.path.join(PROFILES, out_name + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get(key)


def measure_split_gain(args, steps, warmup):
    """What split-KV buys at ctx 4096: the same batch at the automatic split
    count and at one piece per (sequence, kv head) (S = 1, no merge), the
    split kernel alone (HIP events) and the whole graph-replayed step; the
    active-CU fraction of each from committed counter summaries
    (profiles/split_gain_<workload>_s<S>_cu_counters) when they match the
    current kernels."""
    import torch
    import workloads as W
    res = {}
    for name in ("c2b1", "c2b8"):
        wl = DecodeWorkload(W.CONFIGS[name], args.rotate_gib, 0)
        auto = wl.S
        row = {"workload": W.CONFIGS[name].name, "auto_splits": auto}
        for label, S in (("auto", auto), ("s1", 1)):
            wl.set_splits(S)
            ms_step, _ = time_steps_eager(wl, steps, warmup)
            ms_k = time_kernel_events(wl.kernel, min(200, max(50, steps)), wl.R)
            row[f"{label}_step_us"] = round(ms_step * 1e3, 3)
            row[f"{label}_kernel_us"] = round(ms_k * 1e3, 3)
            cu = load_sq(f"split_gain_{name}_{'s1' if S == 1 else 'auto'}_cu_counters",
                         "active_cu_frac")
            if cu is not None:
                row[f"{label}_active_cu_frac"] = round(cu, 4)
        row["step_speedup"] = round(row["s1_step_us"] / row["auto_step_us"], 3)
        row["kernel_speedup"] = round(row["s1_kernel_us"] / row["auto_kernel_us"], 3)
        res[name] = row
        print(f"[bench] split-KV gain {name}: step S=1 {row['s1_step_us']:.2f} us vs S={auto} "
              f"{row['auto_step_us']:.2f} us (x{row['step_speedup']:.2f})", file=sys.stderr,
              flush=True)
        del wl
        torch.cuda.empty_cache()
    return res


def equal_share_lens(total: int, n: int):
    """n lengths summing to total, differing by at most one token."""
    base, extra = divmod(total, n)
    return tuple([base + 1] * extra + [base] * (n - extra))


def measure_equal_share(args, others, steps, warmup):
    """The best any split of a random-length batch into equal token shares
    can do: the same number of context tokens and the same heads, laid out
    as one sequence per (compute unit, kv head) with equal lengths, decoded
    at one piece per (sequence, kv head) so that every compute unit gets
    one workgroup with the same work and no merge runs.  Reported beside the
    drawn batch's own kernel and step times."""
    import torch
    import workloads as W
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {}
    for name in ("c3", "c5d", "c4"):
        if name not in others:
            continue
        spec = W.CONFIGS[name]
        total = int(W.draw_context_lens(spec).sum())
        n = max(spec.num_seqs, cus // spec.num_kv_heads)
        eq = spec.with_(num_seqs=n, context_lens=equal_share_lens(total, n), len_range=None,
                        num_blocks=max(spec.num_blocks, n * spec.max_blocks_per_seq))
        wl = DecodeWorkload(eq, args.rotate_gib, 1)
        ms_step, _ = time_steps_eager(wl, steps, warmup)
        ms_k = time_kernel_events(wl.kernel, min(200, max(50, steps)), wl.R)
        drawn = others[name]
        # the library's best for the drawn lengths: the drawn order at the
        # automatic split, or longest first at the split planned from the lengths
        drawn_k = min(drawn["kernel_avg_us"], drawn.get("longest_first_kernel_us", 1e30))
        row = {"workload": spec.name, "context_tokens": total, "equal_share_seqs": n,
               "equal_share_len": int(wl.lens_np.max()),
               "equal_share_kernel_us": round(ms_k * 1e3, 3),
               "equal_share_step_us": round(ms_step * 1e3, 3),
               "equal_share_kernel_frac": round(wl.decode_bytes / (ms_k * 1e-3) / 1e9
                                                / HBM_PEAK_GBS, 4),
               "best_kernel_us": round(drawn_k, 3),
               "best_kernel_frac": round(drawn["decode_bytes"] / (drawn_k * 1e-6) / 1e9
                                         / HBM_PEAK_GBS, 4)}
        res[name] = row
        print(f"[bench] equal-share bound {name}: kernel {row['equal_share_kernel_us']:.2f} us "
              f"(frac {row['equal_share_kernel_frac']:.3f}) against {row['best_kernel_us']:.2f} "
              f"us (frac {row['best_kernel_frac']:.3f}) for the drawn lengths", file=sys.stderr,
              flush=True)
        del wl
        torch.cuda.empty_cache()
    return res


def longest_first_order(wl):
    """Device permutation of a workload's sequences, longest first, as the
    library's block manager gives it (pa_bm_order_longest_first)."""
    import numpy as np
    import torch
    spec = wl.spec
    B, bs = spec.num_seqs, spec.block_size
    need = int(((wl.lens_np.astype(np.int64) + bs - 1) // bs).sum())
    bm = wl.pa.BlockManager(max(spec.num_blocks, need + 1), bs, spec.max_blocks_per_seq,
                            prefix_cache=False)
    for b, L in enumerate(wl.lens_np):
        bm.admit(b, 0, np.zeros(int(L), np.int32))
    order = bm.order_longest_first(np.arange(B))
    del bm
    return torch.from_numpy(order).to(wl.dev)


def measure_drawn_order_planned(wl, steps, warmup):
    """The batch in its drawn order at the split count planned from the
    host's lengths (pa_decode_auto_splits_lengths) instead of the shape-only
    automatic count; timed only where the two counts differ."""
    spec = wl.spec
    S_d = wl.pa.auto_splits_lengths(wl.lens_np, spec.num_kv_heads, spec.max_blocks_per_seq,
                                    spec.block_size, wl.dev)
    rec = {"lengths_planned_splits": S_d}
    if S_d == wl.S:
        return rec
    S0 = wl.S
    wl.set_splits(S_d)
    ms_step, _ = time_steps_eager(wl, steps, warmup)
    avg = time_kernel_events(wl.kernel, min(200, max(50, steps)), wl.R)
    wl.set_splits(S0)
    rec.update({"lengths_planned_us_per_call": ms_step * 1e3,
                "lengths_planned_kernel_us": avg * 1e3,
                "lengths_planned_kernel_gbps": wl.decode_bytes / (avg * 1e-3) / 1e9})
    return rec


def measure_longest_first(wl, steps, warmup):
    """The same batch launched longest sequence first, in the order the
    library's block manager gives (pa_bm_order_longest_first): the sequences'
    rows of tables and lengths permuted, the work unchanged; the split count
    from the host's lengths in that order (pa_decode_auto_splits_lengths)."""
    perm = longest_first_order(wl)
    saved = wl.tables, wl.lens, wl.S
    wl.tables = [t[perm].contiguous() for t in saved[0]]
    wl.lens = saved[1][perm].contiguous()
    spec = wl.spec
    S_lf = wl.pa.auto_splits_lengths(wl.lens_np[perm.cpu().numpy()], spec.num_kv_heads,
                                     spec.max_blocks_per_seq, spec.block_size, wl.dev)
    wl.set_splits(S_lf)
    ms_step, _ = time_steps_eager(wl, steps, warmup)
    avg = time_kernel_events(wl.kernel, min(200, max(50, steps)), wl.R)
    wl.tables, wl.lens = saved[:2]
    wl.set_splits(saved[2])
    return {"longest_first_splits": S_lf, "longest_first_us_per_call": ms_step * 1e3,
            "longest_first_gbps": (wl.decode_bytes + wl.append_bytes) / (ms_step * 1e-3) / 1e9,
            "longest_first_kernel_us": avg * 1e3,
            "longest_first_kernel_gbps": wl.decode_bytes / (avg * 1e-3) / 1e9}


def _read_probe_fn():
    """pa_bench_read_probe from the benchmark's own probe library
    (libpa_readprobe.so, built beside the attention library)."""
    import ctypes

    import paged_kv_attention_09_amd as pa
    f = ctypes.CDLL(os.path.join(os.path.dirname(pa.LIB_PATH), "libpa_readprobe.so")) \
        .pa_bench_read_probe
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    return f


def read_probe_gbps(nbytes: int):
    """Fastest plain read of `nbytes` the probe finds on this GPU: each
    workgroup reads one contiguous slice with 4, 8 or 16 independent 16-byte
    loads in flight per thread, over grids of 512 to 16384 workgroups; cold
    buffers (rotating over at least 2 GiB, so no read hits the last-level
    cache); HIP events over back-to-back launches.  Returns (GB/s, grid,
    unroll) of the best setting."""
    import torch
    f = _read_probe_fn()
    nbytes = max(16, nbytes // 16 * 16)
    sink = torch.empty(4 * 16384, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    nbuf = max(2, -(-(2 << 30) // nbytes))
    bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0") for _ in range(nbuf)]
    best = (0.0, 0, 0)
    for wgs in (512, 1024, 2048, 4096, 8192, 16384):
        for unroll in (4, 8, 16):
            def launch(i):
                st = f(bufs[i % nbuf].data_ptr(), nbytes, sink.data_ptr(), wgs, unroll, stream)
                if st != 0:
                    raise RuntimeError(f"pa_bench_read_probe failed with status {st}")
            ms = time_kernel_events(launch, max(2 * nbuf, 32), nbuf)
            best = max(best, (nbytes / (ms * 1e-3) / 1e9, wgs, unroll))
    del bufs
    torch.cuda.empty_cache()
    return best


def measure_read_ceiling():
    """The read rate a plain streaming read reaches on this GPU, for context
    next to the 8 TB/s peak: cold buffers of 32 MiB (the size of the ctx-4096
    batch-8 decode) and of 1 GiB."""
    res = {}
    for mib in (32, 1024):
        gbps, wgs, unroll = read_probe_gbps(mib << 20)
        res[f"read_{mib}MiB_gbps"] = round(gbps, 1)
        res[f"read_{mib}MiB_best_setting"] = {"workgroups": wgs, "loads_in_flight": unroll}
    res["probe"] = ("pa_bench_read_probe (libpa_readprobe.so): contiguous slice per workgroup, "
                    "16-byte loads, best of 512-16384 workgroups x 4/8/16 loads in flight, cold "
                    "buffers, HIP events over back-to-back launches")
    return res


def measure_block_manager(seed: int = 77):
    """Host cost of the native block manager on the 256-sequence pool shape
    (17166 blocks of 256 tokens, 5 blocks per sequence): admission of 256
    prompts that share a 512-token system prompt, then decode steps (one
    token for every sequence, pa_bm_decode_step) and the 256 block-table rows
    each step feeds to the kernels.  Microseconds per call, median of 200."""
    import statistics
    import numpy as np
    import paged_kv_attention_09_amd as pa
    import workloads as W
    rng = np.random.default_rng(seed)
    bm = pa.BlockManager(W.C4_NUM_BLOCKS, 256, 5, prefix_cache=True)
    system = rng.integers(0, 32000, 512).astype(np.int32)
    ids = np.arange(1, 257, dtype=np.int64)
    t_admit, cached = [], 0
    for k in ids:
        prompt = np.concatenate([system, rng.integers(0, 32000, int(rng.integers(1, 512)))])
        t0 = time.perf_counter()
        c, _ = bm.admit(int(k), 0, prompt)
        t_admit.append(time.perf_counter() - t0)
        cached += c
        if k == 1:
            bm.decode_step(ids[:1], np.zeros(1, np.int32))   # the system prompt becomes shareable
    t_step, t_tab = [], []
    for _ in range(200):
        toks = rng.integers(0, 32000, 256).astype(np.int32)
        t0 = time.perf_counter()
        bm.decode_step(ids, toks)
        t1 = time.perf_counter()
        bm.block_tables(ids)
        t2 = time.perf_counter()
        t_step.append(t1 - t0)
        t_tab.append(t2 - t1)
    free, cached_b, used, running = bm.stats()
    return {"admit_us": round(statistics.median(t_admit) * 1e6, 2),
            "decode_step_us_256_seqs": round(statistics.median(t_step) * 1e6, 2),
            "block_tables_us_256_seqs": round(statistics.median(t_tab) * 1e6, 2),
            "prefix_cached_tokens": int(cached), "used_blocks": used,
            "note": "host time through the Python binding (one ctypes call per operation)"}


MULTI_WORKLOADS = {"c2b8q2": ("c2b8", 2), "c2b8q4": ("c2b8", 4), "c3q4": ("c3", 4),
                   "c2b8q4f8": ("c2b8", 4, "fp8")}


def measure_multi(name, args, steps, warmup):
    """Multi-token decode (the speculative verify step) on a decode workload's
    shapes and lengths, against single-token decode of the same batch."""
    import torch
    import workloads as W
    base, q_len = MULTI_WORKLOADS[name][:2]
    fp8 = MULTI_WORKLOADS[name][2:] == ("fp8",)
    spec = W.CONFIGS[base]
    wl = DecodeWorkload(spec, args.rotate_gib, args.splits, q_len=q_len, kv_fp8=fp8)
    ms = time_graph(wl.step_multi_fp8 if fp8 else wl.step_multi, wl.R, steps, warmup)
    rec = {"workload": f"{spec.name}, {q_len} query tokens" + (", fp8 pools" if fp8 else ""),
           "key": name, "base_workload": base,
           "q_len": q_len,
           "kv": "fp8 e4m3, per-tensor scales" if fp8 else "bf16",
           "us_per_call": ms * 1e3, "gbps": wl.decode_bytes / (ms * 1e-3) / 1e9,
           "decode_bytes": wl.decode_bytes, "splits": wl.S, "rotations": wl.R}
    del wl
    torch.cuda.empty_cache()
    one = DecodeWorkload(spec, args.rotate_gib, args.splits, kv_fp8=fp8)
    ms1 = time_graph(one.step_fp8 if fp8 else one.step_plain, one.R, steps, warmup)
    rec["single_token_us_per_call"] = ms1 * 1e3
    rec["ratio_to_single_token"] = ms / ms1
    return one, rec


FP8_WORKLOADS = {"c2b8f8": "c2b8", "c3f8": "c3", "c4f8": "c4"}


def measure_fp8(name, args, steps, warmup):
    """Single-token decode over fp8 pools on a decode workload's shapes and
    lengths, against the same decode over bf16 pools."""
    import torch
    import workloads as W
    base = FP8_WORKLOADS[name]
    spec = W.CONFIGS[base]
    wl = DecodeWorkload(spec, args.rotate_gib, args.splits, kv_fp8=True)
    ms = time_graph(wl.step_fp8, wl.R, steps, warmup)
    rec = {"workload": f"{spec.name}, fp8 pools", "key": name, "base_workload": base,
           "kv": "fp8 e4m3, per-tensor scales",
           "us_per_call": ms * 1e3, "gbps": wl.decode_bytes / (ms * 1e-3) / 1e9,
           "decode_bytes": wl.decode_bytes, "splits": wl.S, "rotations": wl.R}
    if spec.len_range is not None:
        perm = longest_first_order(wl)
        wl.tables = [t[perm].contiguous() for t in wl.tables]
        wl.lens = wl.lens[perm].contiguous()
        ms_lf = time_graph(wl.step_fp8, wl.R, steps, warmup)
        rec["longest_first_us_per_call"] = ms_lf * 1e3
        rec["longest_first_gbps"] = wl.decode_bytes / (ms_lf * 1e-3) / 1e9
    del wl
    torch.cuda.empty_cache()
    one = DecodeWorkload(spec, args.rotate_gib, args.splits)
    ms1 = time_graph(one.step_plain, one.R, steps, warmup)
    rec["bf16_us_per_call"] = ms1 * 1e3
    rec["speedup_over_bf16"] = ms1 / ms
    return one, rec


def main(argv=None):
    args = parse_args(argv)
    if args.workload in ("c5p", "c2b8f8", "c4f8") and not args.kernel_loop:
        raise SystemExit(f"--workload {args.workload} is a profiling mode: use it with "
                         "--kernel-loop")
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a measured configuration.",
              file=sys.stderr)
        sys.exit(2)
    if args.ingest_trace:
        ingest_trace(*args.ingest_trace)
        return
    if args.ingest_sq:
        d, k, name, cmd = args.ingest_sq
        flop = None
        if k == "prefill_kernel":
            import numpy as np
            import workloads as W
            ps = W.PREFILL_CONFIGS["c5p"]
            pos = np.concatenate([np.arange(L - n, L) for L, n in zip(ps.total_lens, ps.chunk_lens)])
            flop = 4 * ps.head_dim * ps.num_q_heads * int((pos + 1).sum())
        ingest_sq(d, k, name, cmd, flop)
        return
    if args.ingest_counters:
        a = args.ingest_counters
        ingest_counters(a[0], a[1], a[2], a[3], int(a[4]), args.workload, a[5], a[6])
        return
    import torch
    import workloads as W

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(20):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n, "launches": 20}))
        return
    if args.kernel_loop and args.workload == "c5p":
        wl = PrefillWorkload(W.PREFILL_CONFIGS["c5p"], None, args.rotate_gib)
        for i in range(args.kernel_loop):
            wl.prefill(i % wl.R)
        torch.cuda.synchronize()
        print(json.dumps({"workload": "c5p", "kernel_launches": args.kernel_loop,
                          "splits": wl.S, "flop_per_call": wl.flop}))
        return
    if args.kernel_loop and args.workload in FP8_WORKLOADS:
        wl = DecodeWorkload(W.CONFIGS[FP8_WORKLOADS[args.workload]], args.rotate_gib, args.splits,
                            kv_fp8=True)
        for i in range(args.kernel_loop):
            wl.step_fp8(i % wl.R)
        torch.cuda.synchronize()
        print(json.dumps({"workload": args.workload, "calls": args.kernel_loop,
                          "splits": wl.S, "decode_bytes_per_call": wl.decode_bytes}))
        return
    if args.step_loop:
        wl = DecodeWorkload(W.CONFIGS[args.workload], args.rotate_gib, args.splits)
        for i in range(3):
            wl.step(i % wl.R)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(args.step_loop):
                wl.step(i % wl.R)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(json.dumps({"workload": args.workload, "steps": args.step_loop, "splits": wl.S,
                          "decode_bytes_per_step": wl.decode_bytes}))
        return
    if args.kernel_loop:
        wl = DecodeWorkload(W.CONFIGS[args.workload], args.rotate_gib, args.splits)
        if args.graph:
            for i in range(3):
                wl.kernel(i % wl.R)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(args.kernel_loop):
                    wl.kernel(i % wl.R)
            torch.cuda.synchronize()
            g.replay()
        else:
            for i in range(args.kernel_loop):
                wl.kernel(i % wl.R)
        torch.cuda.synchronize()
        print(json.dumps({"workload": args.workload, "kernel_launches": args.kernel_loop,
                          "splits": wl.S, "decode_bytes_per_launch": wl.decode_bytes}))
        return

    if args.sweep_splits:
        res = {}
        for name in [args.workload] + [x for x in args.others.split(",") if x]:
            if name == "c5p":
                wl = PrefillWorkload(W.PREFILL_CONFIGS["c5p"], None, args.rotate_gib)
                res[name] = {"auto": wl.S}
                for S in [int(x) for x in args.sweep_splits.split(",")]:
                    wl.S = S
                    n = wl.pa.prefill_workspace_size(1, wl.max_q, wl.q.shape[1], wl.q.shape[2], S)
                    wl.ws = torch.zeros(max(n, 256), dtype=torch.uint8, device=wl.dev)
                    ms = time_graph(wl.prefill, wl.R, min(args.steps, 50), 3)
                    res[name][S] = round(ms * 1e3, 2)
                    print(f"[sweep] {name} S={S}: {ms * 1e3:.2f} us ({wl.flop / ms / 1e9:.0f} "
                          f"TFLOP/s)", file=sys.stderr, flush=True)
                del wl
                torch.cuda.empty_cache()
                continue
            if name not in W.CONFIGS or name in res:
                continue    # the sweep covers the decode workloads and the prefill chunk
            wl = DecodeWorkload(W.CONFIGS[name], args.rotate_gib, args.splits)
            auto = wl.S
            res[name] = {"auto": auto}
            for S in [int(x) for x in args.sweep_splits.split(",")]:
                wl.set_splits(S)
                ms, _ = time_steps_eager(wl, min(args.steps, 100), 3)
                res[name][S] = round(ms * 1e3, 2)
                print(f"[sweep] {name} S={S}: {ms * 1e3:.2f} us/step", file=sys.stderr, flush=True)
            del wl
            torch.cuda.empty_cache()
        print(json.dumps(res))
        return

    print(f"[bench] {args.workload}: building inputs", file=sys.stderr, flush=True)
    wl, main_rec = measure(args.workload, args, args.steps, args.warmup)
    print(f"[bench] {args.workload}: {main_rec['us_per_call']:.2f} us/step, "
          f"{main_rec['gbps']:.1f} GB/s (graph replay {main_rec['graph_us_per_step']:.2f} us); "
          f"kernel {main_rec['kernel_avg_us']:.2f} us; eager "
          f"{main_rec['eager_us_per_step']:.2f} us against graph "
          f"{main_rec['graph_us_per_step_paired']:.2f} us in adjacent pairs (graph saves "
          f"{100 * main_rec['graph_saving']:.1f}%, host issue "
          f"{main_rec['host_issue_us_per_call']:.2f} us/call)", file=sys.stderr, flush=True)
    others = {}
    for name in [x for x in args.others.split(",") if x and x != args.workload]:
        del wl
        torch.cuda.empty_cache()
        if name in FP8_WORKLOADS:
            wl, rec = measure_fp8(name, args, EXTRA_STEPS, EXTRA_WARMUP)
            msg = (f"fp8 pools: {rec['us_per_call']:.2f} us/call, {rec['gbps']:.1f} GB/s; bf16 "
                   f"{rec['bf16_us_per_call']:.2f} us (x{rec['speedup_over_bf16']:.2f})")
            if "longest_first_us_per_call" in rec:
                msg += f"; longest first {rec['longest_first_us_per_call']:.2f} us"
        elif name in MULTI_WORKLOADS:
            wl, rec = measure_multi(name, args, EXTRA_STEPS, EXTRA_WARMUP)
            msg = (f"q_len {rec['q_len']}: {rec['us_per_call']:.2f} us/call, {rec['gbps']:.1f} GB/s;"
                   f" single-token {rec['single_token_us_per_call']:.2f} us "
                   f"(x{rec['ratio_to_single_token']:.2f})")
        elif name in ("c5p", "c5mix", "c5pf8", "c5mixf8"):
            wl, rec = measure_prefill(args, EXTRA_STEPS // 2, EXTRA_WARMUP,
                                      with_decode=name.startswith("c5mix"),
                                      kv_fp8=name.endswith("f8"))
            msg = f"prefill {rec['prefill_us']:.2f} us ({rec['prefill_tflops']:.0f} TFLOP/s)"
            if name.endswith("f8"):
                msg = "fp8 pools: " + msg
            if name.startswith("c5mix"):
                msg += (f"; mixed step {rec['us_per_step']:.2f} us (append {rec['append_us']:.2f}, "
                        f"decode {rec['decode_us']:.2f}); decode batch longest first "
                        f"(S={rec['longest_first_decode_splits']}): step "
                        f"{rec['longest_first_us_per_step']:.2f} us, decode "
                        f"{rec['longest_first_decode_us']:.2f} us")
        else:
            wl, rec = measure(name, args, EXTRA_STEPS, EXTRA_WARMUP)
            msg = (f"{rec['us_per_call']:.2f} us/step, {rec['gbps']:.1f} GB/s; "
                   f"kernel {rec['kernel_avg_us']:.2f} us ({rec['kernel_gbps']:.0f} GB/s); "
                   f"eager {rec['eager_us_per_step']:.2f} us against graph "
                   f"{rec['graph_us_per_step_paired']:.2f} us (graph saves "
                   f"{100 * rec['graph_saving']:.1f}%)")
            if "lengths_planned_us_per_call" in rec:
                msg += (f"; drawn order at S = {rec['lengths_planned_splits']} from the lengths "
                        f"{rec['lengths_planned_us_per_call']:.2f} us/step, kernel "
                        f"{rec['lengths_planned_kernel_us']:.2f} us")
            if "longest_first_us_per_call" in rec:
                msg += (f"; longest first {rec['longest_first_us_per_call']:.2f} us/step, kernel "
                        f"{rec['longest_first_kernel_us']:.2f} us "
                        f"({rec['longest_first_kernel_gbps']:.0f} GB/s)")
        others[name] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in rec.items()
                        if k not in ("wall_s",)}
        print(f"[bench] {name}: {msg}", file=sys.stderr, flush=True)

    split_gain = measure_split_gain(args, EXTRA_STEPS, EXTRA_WARMUP)
    equal_share = measure_equal_share(args, others, EXTRA_STEPS, EXTRA_WARMUP)
    multilayer = measure_multilayer(args)
    bm_rec = measure_block_manager()
    print(f"[bench] block manager: decode step {bm_rec['decode_step_us_256_seqs']:.1f} us, "
          f"tables {bm_rec['block_tables_us_256_seqs']:.1f} us for 256 sequences; admit "
          f"{bm_rec['admit_us']:.1f} us; {bm_rec['prefix_cached_tokens']} prompt tokens from the "
          "prefix cache", file=sys.stderr, flush=True)
    others["host_block_manager"] = bm_rec
    ceiling = measure_read_ceiling()
    # each decode workload's split kernel against a plain read of its own bytes
    for name, rec in others.items():
        if "kernel_gbps" in rec and "decode_bytes" in rec:
            probe = read_probe_gbps(int(rec["decode_bytes"]))[0]
            rec["read_probe_gbps_same_bytes"] = round(probe, 1)
            rec["kernel_frac_of_read_probe"] = round(rec["kernel_gbps"] / probe, 4)
    print(f"[bench] measured read rate (read probe, cold): 32 MiB {ceiling['read_32MiB_gbps']:.0f} "
          f"GB/s, 1 GiB {ceiling['read_1024MiB_gbps']:.0f} GB/s", file=sys.stderr, flush=True)

    spec = W.CONFIGS[args.workload]
    achieved = main_rec["kernel_gbps"]
    traffic = load_traffic(args.workload)
    trace = load_trace(f"decode_{args.workload}_kernel_trace", "decode_split_kernel")
    line = {
        "metric": "paged-decode achieved HBM GB/s (% of peak) and us/call at ctx 4096",
        "value": round(main_rec["gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_rec["ms_per_step"], 6),
        "us_per_call": round(main_rec["us_per_call"], 3),
        "pct_of_hbm_peak": round(100 * main_rec["gbps"] / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) bf16, seeded; random block tables; cold-HBM rotation",
        "config": {"workload": spec.name, "num_seqs": spec.num_seqs,
                   "num_q_heads": spec.num_q_heads, "num_kv_heads": spec.num_kv_heads,
                   "head_dim": spec.head_dim, "block_size": spec.block_size,
                   "context_tokens": main_rec["context_tokens"], "num_splits": main_rec["splits"],
                   "rotations": main_rec["rotations"], "step": "append fused into split-KV decode, then merge",
                   "graph_us_per_step": round(main_rec["graph_us_per_step"], 3),
                   "unfused_graph_us_per_step": round(main_rec["unfused_graph_us_per_step"], 3),
                   "eager_us_per_step": round(main_rec["eager_us_per_step"], 3),
                   "graph_us_per_step_paired": round(main_rec["graph_us_per_step_paired"], 3),
                   "host_issue_us_per_call": round(main_rec["host_issue_us_per_call"], 3),
                   "timing": "the timed steps issued through the C ABI between HIP events "
                             "behind a primed queue (graph_us_per_step: the same steps "
                             "replayed from one HIP graph); kernel: HIP events around "
                             "back-to-back launches behind a primed queue"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "decode_split_kernel", "kernel_avg_us": round(main_rec["kernel_avg_us"], 3),
                     "algorithmic_bytes_per_launch": main_rec["decode_bytes"],
                     "headline": "frac: split-kernel average from HIP events in this run",
                     "frac_of_measured_read_32MiB": round(achieved / ceiling["read_32MiB_gbps"], 4)},
        "measured_read_ceiling": ceiling,
        "split_kv_gain": split_gain,
        "equal_share_bound": equal_share,
        "multilayer_graph": multilayer,
        "workloads": others,
    }
    if trace is not None:
        avg_us, med_us, kname = trace
        line["roofline"]["trace"] = {
            "summary": f"profiles/decode_{args.workload}_kernel_trace.md", "kernel": kname,
            "avg_us": round(avg_us, 3), "median_us": round(med_us, 3),
            "frac_from_avg": round(main_rec["decode_bytes"] / (avg_us * 1e-6) / 1e9
                                   / HBM_PEAK_GBS, 4),
            "events_over_trace_avg": round(main_rec["kernel_avg_us"] / avg_us, 4)}
    device_pass = load_step_trace(f"decode_{args.workload}_step_trace")
    if device_pass is not None:
        line["device_pass"] = device_pass
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(spec, args.cpu_seconds)
        # the same oracle leg checks the benchmarked call's results on host-drawn inputs
        par = parity_record(spec)
        line["cpu_baseline"]["parity_of_benchmarked_call"] = par
        mixed_par = {}
        for name in ("c5mix", "c5mixf8"):
            if name in others:
                mixed_par[name] = mixed_parity_record(name.endswith("f8"))
                others[name]["parity"] = mixed_par[name]
                print(f"[bench] {name} parity against the oracle: pools bit-exact "
                      f"{mixed_par[name]['pools_bit_exact']}, within tolerance "
                      f"{mixed_par[name]['within_tolerance']}", file=sys.stderr, flush=True)
        print(f"[bench] parity against the oracle: max abs err {par['max_abs_err']:.2e}, "
              f"rms {par['rms_err']:.2e}, within tolerance: {par['within_tolerance']}",
              file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
