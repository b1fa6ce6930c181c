"""Decode steps captured in HIP graphs at power-of-two padded batch sizes.

An engine replays one captured graph per padded batch size instead of
launching the step's kernels from the host every time (decode_batch captured
statically in a CUDA graph: zingnex.cn mini-infer thread, feature list item
6; graph capture of the decode step in the MiniInfer README's optimisation
log).  A batch of B sequences runs in the graph of the smallest captured
size P >= B; rows B .. P-1 are padding with context length 0, which the
kernels neither read for nor append for, and whose output rows are zero.

Everything a graph touches is allocated once, before any capture: the
static inputs and outputs of every size and one split workspace sized for
the largest.  The graphs replay on one stream, one at a time, so they share
the workspace.  This module is host logic only: the work inside a graph is
the library's fused append + decode launch (pa_append_decode) and nothing
else.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import torch

from . import append_decode, auto_splits, decode_workspace_size


def padded_sizes(max_batch: int) -> List[int]:
    """1, 2, 4, ... up to the first power of two >= max_batch."""
    if max_batch < 1:
        raise ValueError("max_batch must be >= 1")
    sizes, p = [], 1
    while True:
        sizes.append(p)
        if p >= max_batch:
            return sizes
        p *= 2


class PaddedDecodeGraphs:
    """Captured fused append + decode steps over one paged KV pool.

    For every padded size P the static tensors are
      q      bf16 [P, Hq, D]      new_k, new_v  bf16 [P, Hkv, D]
      tables int32 [P, W]         lens          int32 [P]
      out    bf16 [P, Hq, D]
    Write a batch into them with `prepare` (or directly into `buffers(P)`,
    keeping lens of the padding rows at 0), then `replay`.
    """

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, num_q_heads: int,
                 max_batch: int, max_blocks_per_seq: int, scale: float, num_splits: int = 0):
        NB, bs, Hkv, D = (int(x) for x in k_cache.shape)
        dev = k_cache.device
        self.k_cache, self.v_cache = k_cache, v_cache
        self.Hq, self.Hkv, self.D, self.W = num_q_heads, Hkv, D, max_blocks_per_seq
        self.scale = float(scale)
        self.sizes = padded_sizes(max_batch)
        self.splits = {P: (num_splits if num_splits > 0 else
                           auto_splits(P, Hkv, max_blocks_per_seq, bs, dev)) for P in self.sizes}
        ws_bytes = max([decode_workspace_size(P, num_q_heads, D, S) for P, S in self.splits.items()]
                       + [256])
        self.workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        self._buf: Dict[int, Dict[str, torch.Tensor]] = {}
        for P in self.sizes:
            self._buf[P] = {
                "q": torch.zeros((P, num_q_heads, D), dtype=torch.bfloat16, device=dev),
                "new_k": torch.zeros((P, Hkv, D), dtype=torch.bfloat16, device=dev),
                "new_v": torch.zeros((P, Hkv, D), dtype=torch.bfloat16, device=dev),
                "tables": torch.zeros((P, max_blocks_per_seq), dtype=torch.int32, device=dev),
                "lens": torch.zeros((P,), dtype=torch.int32, device=dev),
                "out": torch.zeros((P, num_q_heads, D), dtype=torch.bfloat16, device=dev),
            }
        self.stream = torch.cuda.Stream(device=dev)
        self.graphs: Dict[int, torch.cuda.CUDAGraph] = {}
        torch.cuda.synchronize(dev)
        for P in self.sizes:
            b = self._buf[P]
            g = torch.cuda.CUDAGraph()
            # All lengths are 0 here, so neither the eager warm-up nor the
            # capture touches the pool.
            with torch.cuda.stream(self.stream):
                self._step(P)
            self.stream.synchronize()
            with torch.cuda.graph(g, stream=self.stream):
                self._step(P)
            self.graphs[P] = g
            b["out"].zero_()
        torch.cuda.synchronize(dev)

    def _step(self, P: int) -> None:
        b = self._buf[P]
        append_decode(b["q"], b["new_k"], b["new_v"], self.k_cache, self.v_cache, b["tables"],
                      b["lens"], self.scale, self.splits[P], b["out"], workspace=self.workspace)

    def size_for(self, batch: int) -> int:
        for P in self.sizes:
            if P >= batch:
                return P
        raise ValueError(f"batch {batch} exceeds the largest captured size {self.sizes[-1]}")

    def buffers(self, P: int) -> Dict[str, torch.Tensor]:
        return self._buf[P]

    def prepare(self, q, new_k, new_v, block_tables, context_lens) -> int:
        """Copy one batch (device tensors, B rows) into the static buffers of
        its padded size and mark the remaining rows as padding.  Returns P."""
        B = int(q.shape[0])
        P = self.size_for(B)
        b = self._buf[P]
        self.stream.wait_stream(torch.cuda.current_stream(self.stream.device))
        # the copies run on the graphs' stream: the caller's tensors must not be
        # recycled by the allocator before that stream has read them
        for t in (q, new_k, new_v, block_tables, context_lens):
            t.record_stream(self.stream)
        with torch.cuda.stream(self.stream):
            b["q"][:B].copy_(q)
            b["new_k"][:B].copy_(new_k)
            b["new_v"][:B].copy_(new_v)
            b["tables"][:B].copy_(block_tables)
            b["lens"][:B].copy_(context_lens)
            b["lens"][B:].zero_()
        return P

    def replay(self, P: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Replay the captured step of size P on the graphs' stream (ordered
        after the caller's current stream).  Returns the static output (all
        P rows; padding rows are zero) or copies its first rows into `out`."""
        caller = torch.cuda.current_stream(self.stream.device)
        self.stream.wait_stream(caller)
        with torch.cuda.stream(self.stream):
            self.graphs[P].replay()
        caller.wait_stream(self.stream)
        res = self._buf[P]["out"]
        if out is not None:
            out.copy_(res[:out.shape[0]])
            return out
        return res
