"""Python binding of libpagedattn.so (paged-KV attention for MI355X / gfx950).

Argument marshalling only: shapes, dtypes and devices of torch tensors are
checked, raw device pointers and the current HIP stream are handed to the C
ABI declared in include/pagedattn.h, and every step of the computation runs
in the library's HIP kernels.  There is no fallback: if the library is not
built, or no GPU is present, the calls raise.

Calls (argument order as in the C ABI):
  reshape_and_cache(k, v, slot_mapping, k_cache, v_cache, stream=None)
  decode(q, k_cache, v_cache, block_tables, context_lens, scale, num_splits, out,
         stream=None, workspace=None)
  append_decode(q, new_k, new_v, k_cache, v_cache, block_tables, context_lens, scale,
                num_splits, out, stream=None, workspace=None)
  decode_multi(q, k_cache, v_cache, block_tables, context_lens, scale, num_splits, out,
               stream=None, workspace=None): q_len query tokens per sequence, causal
  decode_partials(...), decode_merge(...): the two passes of decode
  reshape_and_cache_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale, stream=None)
  decode_fp8(q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale,
             num_splits, out, stream=None, workspace=None): fp8 (e4m3) pools
  append_decode_fp8(...): append_decode over fp8 pools (quantising fused append)
  decode_multi_fp8(...): decode_multi over fp8 pools
  prefill_fp8(q, cu_seqlens_q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
              v_scale, out, max_q_len, num_splits=0, stream=None, workspace=None)
  prefill(q, cu_seqlens_q, k_cache, v_cache, block_tables, context_lens, scale, out,
          max_q_len, num_splits=0, stream=None, workspace=None)
  decode_workspace_size(num_seqs, num_q_heads, head_dim, num_splits)
  decode_multi_workspace_size(num_seqs, q_len, num_q_heads, head_dim, num_splits)
  plan_splits(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, num_cus)
  auto_splits(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, device=None)
  plan_splits_lengths(context_lens, num_kv_heads, max_blocks_per_seq, block_size, num_cus),
  auto_splits_lengths(context_lens, num_kv_heads, max_blocks_per_seq, block_size, device=None):
      the same from the host's context lengths in launch order (host int32 array)
  BlockManager(num_blocks, block_size, max_blocks_per_seq, prefix_cache): the host-side
      pool manager (admit / append / truncate / release / preempt / block_tables / stats)
  check_tables(block_tables, context_lens, num_blocks, block_size, fused_append=False),
  check_slots(slot_mapping, num_blocks, block_size),
  check_prefill(cu_seqlens_q, context_lens, max_q_len): synchronous debug checks of the
      preconditions the calls above leave unchecked (host copies; raise PreconditionError)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libpagedattn.so")

PA_OK = 0
PA_MAX_SPLITS = 256
PA_MAX_QUERY_TOKENS = 8
PA_MAX_SEQS = 65535
PA_MAX_HEADS = 4096
PA_ERR_SCRATCH = -9
PA_NOALLOC_SCRATCH_BYTES = 8 << 20

# Every symbol include/pagedattn.h declares, with its ctypes signature.
_VP, _I, _I64, _SZ, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
SIGNATURES = {
    "pa_version": (_I, []),
    "pa_status_string": (ctypes.c_char_p, [_I]),
    "pa_reshape_and_cache": (_I, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _I, _I, _I, _VP]),
    "pa_decode": (_I, [_VP, _VP, _VP, _VP, _VP, _F, _I, _VP, _I, _I, _I, _I, _I, _I64, _I, _VP,
                       _SZ, _VP]),
    "pa_append_decode": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _F, _I, _VP, _I, _I, _I, _I, _I,
                              _I64, _I, _VP, _SZ, _VP]),
    "pa_decode_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "pa_decode_noalloc": (_I, [_VP, _VP, _VP, _VP, _VP, _F, _I, _VP, _I, _I, _I, _I, _I, _I64, _I,
                               _VP]),
    "pa_decode_multi": (_I, [_VP, _VP, _VP, _VP, _VP, _F, _I, _VP, _I, _I, _I, _I, _I, _I, _I64, _I,
                             _VP, _SZ, _VP]),
    "pa_decode_multi_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "pa_decode_plan_splits": (_I, [_I, _I, _I, _I, _I]),
    "pa_decode_auto_splits": (_I, [_I, _I, _I, _I, _I]),
    "pa_decode_plan_splits_lengths": (_I, [_VP, _I, _I, _I, _I, _I]),
    "pa_decode_auto_splits_lengths": (_I, [_VP, _I, _I, _I, _I, _I]),
    "pa_decode_partials": (_I, [_VP, _VP, _VP, _VP, _VP, _F, _I, _I, _I, _I, _I, _I, _I64, _I, _VP,
                                _SZ, _VP]),
    "pa_decode_merge": (_I, [_VP, _SZ, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _VP]),
    "pa_prefill": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _F, _I, _VP, _I, _I, _I, _I, _I, _I, _I64,
                        _I, _VP, _SZ, _VP]),
    "pa_prefill_fp8": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _F, _F, _F, _I, _VP, _I, _I, _I, _I, _I,
                            _I, _I64, _I, _VP, _SZ, _VP]),
    "pa_prefill_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "pa_prefill_plan_splits": (_I, [_I, _I, _I, _I, _I, _I]),
    "pa_reshape_and_cache_fp8": (_I, [_VP, _VP, _VP, _VP, _VP, _F, _F, _I64, _I64, _I, _I, _I,
                                      _VP]),
    "pa_decode_fp8": (_I, [_VP, _VP, _VP, _VP, _VP, _F, _F, _F, _I, _VP, _I, _I, _I, _I, _I, _I64,
                           _I, _VP, _SZ, _VP]),
    "pa_append_decode_fp8": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _F, _F, _F, _I, _VP, _I, _I,
                                  _I, _I, _I, _I64, _I, _VP, _SZ, _VP]),
    "pa_decode_multi_fp8": (_I, [_VP, _VP, _VP, _VP, _VP, _F, _F, _F, _I, _VP, _I, _I, _I, _I, _I,
                                 _I, _I64, _I, _VP, _SZ, _VP]),
    # host-side block manager (include/pa_block_manager.h)
    "pa_bm_create": (_VP, [_I64, _I, _I, _I]),
    "pa_bm_destroy": (None, [_VP]),
    "pa_bm_admit": (_I, [_VP, _I64, _I, _VP, _I64, _VP, _VP]),
    "pa_bm_append": (_I, [_VP, _I64, _VP, _I64, _VP]),
    "pa_bm_decode_step": (_I, [_VP, _VP, _I, _VP, _VP]),
    "pa_bm_truncate": (_I, [_VP, _I64, _I64]),
    "pa_bm_release": (_I, [_VP, _I64]),
    "pa_bm_preempt": (_I, [_VP, _VP]),
    "pa_bm_block_tables": (_I, [_VP, _VP, _I, _VP, _VP]),
    "pa_bm_stats": (_I, [_VP, _VP, _VP, _VP, _VP]),
    "pa_bm_order_longest_first": (_I, [_VP, _VP, _I, _VP]),
    # host-side precondition checks (end of include/pagedattn.h)
    "pa_check_tables": (_I, [_VP, _VP, _I, _I, _I, _I64, _I, _VP]),
    "pa_check_slots": (_I, [_VP, _I64, _I64, _I, _VP]),
    "pa_check_prefill": (_I, [_VP, _VP, _I, _I, _VP]),
}

_lib = None


class PagedAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().pa_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status} ({msg})")
        self.status = status


def lib():
    """Load libpagedattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_attention_09_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PagedAttnError(fn, status)


def _stream_ptr(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, ndim: int, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _pool_dims(k_cache, v_cache, dtype=torch.bfloat16):
    """(NB, bs, Hkv, D) of a pool pair: bf16 pools are [NB, bs, Hkv, D], fp8
    (uint8) pools head-major [NB, Hkv, bs, D]."""
    _need(k_cache, "k_cache", dtype, 4)
    _need(v_cache, "v_cache", dtype, 4, k_cache.device)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    NB, a, b, D = (int(x) for x in k_cache.shape)
    return (NB, b, a, D) if dtype == torch.uint8 else (NB, a, b, D)


def reshape_and_cache(k, v, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """Write k[i], v[i] ([T, Hkv, D] bf16) to pool row slot_mapping[i] (int64 [T];
    negative = skip)."""
    NB, bs, Hkv, D, T, dev = _append_dims(k, v, slot_mapping, k_cache, v_cache, torch.bfloat16)
    _check("pa_reshape_and_cache", lib().pa_reshape_and_cache(
        k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), T, NB, bs, Hkv, D, _stream_ptr(stream, dev)))


def reshape_and_cache_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale: float, v_scale: float,
                          stream=None) -> None:
    """As reshape_and_cache into fp8 pools (uint8 e4m3 codes [NB, Hkv, bs, D]):
    element x is stored as e4m3(clamp(x / scale, -448, 448)), per-tensor fp32
    scales."""
    NB, bs, Hkv, D, T, dev = _append_dims(k, v, slot_mapping, k_cache, v_cache, torch.uint8)
    _check("pa_reshape_and_cache_fp8", lib().pa_reshape_and_cache_fp8(
        k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), float(k_scale), float(v_scale), T, NB, bs, Hkv, D,
        _stream_ptr(stream, dev)))


def _append_dims(k, v, slot_mapping, k_cache, v_cache, pool_dtype):
    NB, bs, Hkv, D = _pool_dims(k_cache, v_cache, pool_dtype)
    dev = k_cache.device
    _need(k, "k", torch.bfloat16, 3, dev)
    _need(v, "v", torch.bfloat16, 3, dev)
    _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    T = int(k.shape[0])
    if tuple(k.shape) != (T, Hkv, D) or tuple(v.shape) != (T, Hkv, D):
        raise ValueError(f"k/v must be [{T}, {Hkv}, {D}]")
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping length differs from the token count")
    return NB, bs, Hkv, D, T, dev


def decode_workspace_size(num_seqs: int, num_q_heads: int, head_dim: int, num_splits: int) -> int:
    return int(lib().pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, num_splits))


def decode_multi_workspace_size(num_seqs: int, q_len: int, num_q_heads: int, head_dim: int,
                                num_splits: int) -> int:
    return int(lib().pa_decode_multi_workspace_size(num_seqs, q_len, num_q_heads, head_dim,
                                                    num_splits))


def plan_splits(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, num_cus) -> int:
    r = int(lib().pa_decode_plan_splits(num_seqs, num_kv_heads, max_blocks_per_seq, block_size,
                                        num_cus))
    _check("pa_decode_plan_splits", min(r, 0))
    return r


def _device_index(device) -> int:
    if isinstance(device, str):
        device = torch.device(device)
    if device is None:
        return torch.cuda.current_device()
    if isinstance(device, torch.device):
        return device.index if device.index is not None else torch.cuda.current_device()
    return int(device)


def auto_splits(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, device=None) -> int:
    r = int(lib().pa_decode_auto_splits(num_seqs, num_kv_heads, max_blocks_per_seq, block_size,
                                        _device_index(device)))
    _check("pa_decode_auto_splits", min(r, 0))
    return r


def _host_lens(context_lens):
    a = np.ascontiguousarray(np.asarray(context_lens), dtype=np.int32)
    if a.ndim != 1:
        raise ValueError("context_lens must be one-dimensional")
    return a


def plan_splits_lengths(context_lens, num_kv_heads, max_blocks_per_seq, block_size,
                        num_cus) -> int:
    a = _host_lens(context_lens)
    r = int(lib().pa_decode_plan_splits_lengths(a.ctypes.data_as(ctypes.c_void_p), len(a),
                                                num_kv_heads, max_blocks_per_seq, block_size,
                                                num_cus))
    _check("pa_decode_plan_splits_lengths", min(r, 0))
    return r


def auto_splits_lengths(context_lens, num_kv_heads, max_blocks_per_seq, block_size,
                        device=None) -> int:
    a = _host_lens(context_lens)
    r = int(lib().pa_decode_auto_splits_lengths(a.ctypes.data_as(ctypes.c_void_p), len(a),
                                                num_kv_heads, max_blocks_per_seq, block_size,
                                                _device_index(device)))
    _check("pa_decode_auto_splits_lengths", min(r, 0))
    return r


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, num_splits: int, out,
           stream=None, workspace: Optional[torch.Tensor] = None):
    """out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b over the first
    context_lens[b] tokens of sequence b, read through block_tables.
    num_splits = 0 picks the split count automatically.  The split workspace
    comes from torch's caching allocator unless `workspace` (uint8, on the
    device, of at least decode_workspace_size bytes) is given; its contents
    need no initialisation."""
    NB, bs, Hkv, D = _pool_dims(k_cache, v_cache)
    dev = k_cache.device
    _need(q, "q", torch.bfloat16, 3, dev)
    _need(out, "out", torch.bfloat16, 3, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, Hq, Dq = (int(x) for x in q.shape)
    if Dq != D or tuple(out.shape) != (B, Hq, D):
        raise ValueError(f"q/out must be [{B}, {Hq}, {D}]")
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables/context_lens batch differs from q")
    W = int(block_tables.shape[1])
    if num_splits == 0 and B > 0:
        num_splits = auto_splits(B, Hkv, W, bs, dev)
    ws_ptr, ws_bytes, workspace = _workspace(B, Hq, D, num_splits, dev, workspace, stream=stream)
    _check("pa_decode", lib().pa_decode(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), float(scale), int(num_splits), out.data_ptr(), B, Hq, Hkv, D,
        bs, NB, W, ws_ptr, ws_bytes, _stream_ptr(stream, dev)))
    return out


def decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                   num_splits: int, out, stream=None):
    """decode without a workspace and without any allocation: the split
    partials go to the library's static per-device scratch
    (PA_NOALLOC_SCRATCH_BYTES).  Calls that may overlap on one device race on
    that scratch.  A split count whose partials do not fit raises
    PagedAttnError with status PA_ERR_SCRATCH."""
    NB, bs, Hkv, D, B, Hq, W, dev = _decode_dims(q, k_cache, v_cache, block_tables, context_lens)
    _need(out, "out", torch.bfloat16, 3, dev)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError(f"out must be [{B}, {Hq}, {D}]")
    _check("pa_decode_noalloc", lib().pa_decode_noalloc(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), float(scale), int(num_splits), out.data_ptr(), B, Hq, Hkv, D,
        bs, NB, W, _stream_ptr(stream, dev)))
    return out


def decode_fp8(q, k_cache, v_cache, block_tables, context_lens, scale: float, k_scale: float,
               v_scale: float, num_splits: int, out, stream=None,
               workspace: Optional[torch.Tensor] = None):
    """decode over fp8 pools (uint8 e4m3 codes [NB, Hkv, bs, D]): K and V are
    the codes' values times k_scale and v_scale."""
    NB, bs, Hkv, D, B, Hq, W, dev = _decode_dims(q, k_cache, v_cache, block_tables, context_lens,
                                                 torch.uint8)
    _need(out, "out", torch.bfloat16, 3, dev)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError(f"out must be [{B}, {Hq}, {D}]")
    if num_splits == 0 and B > 0:
        num_splits = auto_splits(B, Hkv, W, bs, dev)
    ws_ptr, ws_bytes, workspace = _workspace(B, Hq, D, num_splits, dev, workspace, stream=stream)
    _check("pa_decode_fp8", lib().pa_decode_fp8(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), float(scale), float(k_scale), float(v_scale), int(num_splits),
        out.data_ptr(), B, Hq, Hkv, D, bs, NB, W, ws_ptr, ws_bytes, _stream_ptr(stream, dev)))
    return out


def append_decode_fp8(q, new_k, new_v, k_cache, v_cache, block_tables, context_lens,
                      scale: float, k_scale: float, v_scale: float, num_splits: int, out,
                      stream=None, workspace: Optional[torch.Tensor] = None):
    """append_decode over fp8 pools (uint8 e4m3 codes [NB, Hkv, bs, D]): the
    new rows (bf16 [B, Hkv, D]) are quantised into the row of token
    context_lens[b] - 1, then decode_fp8."""
    NB, bs, Hkv, D, B, Hq, W, dev = _decode_dims(q, k_cache, v_cache, block_tables, context_lens,
                                                 torch.uint8)
    _need(out, "out", torch.bfloat16, 3, dev)
    _need(new_k, "new_k", torch.bfloat16, 3, dev)
    _need(new_v, "new_v", torch.bfloat16, 3, dev)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError(f"out must be [{B}, {Hq}, {D}]")
    if tuple(new_k.shape) != (B, Hkv, D) or tuple(new_v.shape) != (B, Hkv, D):
        raise ValueError(f"new_k/new_v must be [{B}, {Hkv}, {D}]")
    if num_splits == 0 and B > 0:
        num_splits = auto_splits(B, Hkv, W, bs, dev)
    ws_ptr, ws_bytes, workspace = _workspace(B, Hq, D, num_splits, dev, workspace, stream=stream)
    _check("pa_append_decode_fp8", lib().pa_append_decode_fp8(
        q.data_ptr(), new_k.data_ptr(), new_v.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), float(scale), float(k_scale),
        float(v_scale), int(num_splits), out.data_ptr(), B, Hq, Hkv, D, bs, NB, W, ws_ptr,
        ws_bytes, _stream_ptr(stream, dev)))
    return out


def decode_multi_fp8(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                     k_scale: float, v_scale: float, num_splits: int, out, stream=None,
                     workspace: Optional[torch.Tensor] = None):
    """decode_multi over fp8 pools (uint8 e4m3 codes [NB, Hkv, bs, D]); q, out:
    [B, q_len, Hq, D]."""
    NB, bs, Hkv, D = _pool_dims(k_cache, v_cache, torch.uint8)
    dev = k_cache.device
    _need(q, "q", torch.bfloat16, 4, dev)
    _need(out, "out", torch.bfloat16, 4, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, QL, Hq, Dq = (int(x) for x in q.shape)
    if Dq != D or tuple(out.shape) != (B, QL, Hq, D):
        raise ValueError(f"q/out must be [{B}, {QL}, {Hq}, {D}]")
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables/context_lens batch differs from q")
    W = int(block_tables.shape[1])
    if num_splits == 0 and B > 0:
        num_splits = auto_splits(B, Hkv, W, bs, dev)
    ws_ptr, ws_bytes, workspace = _workspace(B, Hq, D, num_splits, dev, workspace, q_len=QL,
                                             stream=stream)
    _check("pa_decode_multi_fp8", lib().pa_decode_multi_fp8(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), float(scale), float(k_scale), float(v_scale), int(num_splits),
        out.data_ptr(), B, QL, Hq, Hkv, D, bs, NB, W, ws_ptr, ws_bytes, _stream_ptr(stream, dev)))
    return out


def decode_multi(q, k_cache, v_cache, block_tables, context_lens, scale: float, num_splits: int,
                 out, stream=None, workspace: Optional[torch.Tensor] = None):
    """q, out: [B, q_len, Hq, D].  Query token j of sequence b sits at position
    context_lens[b] - q_len + j and attends the keys up to that position (the
    q_len tokens' K/V must already be in the cache).  The cache is read once
    for all q_len tokens."""
    NB, bs, Hkv, D = _pool_dims(k_cache, v_cache)
    dev = k_cache.device
    _need(q, "q", torch.bfloat16, 4, dev)
    _need(out, "out", torch.bfloat16, 4, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, QL, Hq, Dq = (int(x) for x in q.shape)
    if Dq != D or tuple(out.shape) != (B, QL, Hq, D):
        raise ValueError(f"q/out must be [{B}, {QL}, {Hq}, {D}]")
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables/context_lens batch differs from q")
    W = int(block_tables.shape[1])
    if num_splits == 0 and B > 0:
        num_splits = auto_splits(B, Hkv, W, bs, dev)
    ws_ptr, ws_bytes, workspace = _workspace(B, Hq, D, num_splits, dev, workspace, q_len=QL,
                                             stream=stream)
    _check("pa_decode_multi", lib().pa_decode_multi(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), float(scale), int(num_splits), out.data_ptr(), B, QL, Hq, Hkv,
        D, bs, NB, W, ws_ptr, ws_bytes, _stream_ptr(stream, dev)))
    return out


def append_decode(q, new_k, new_v, k_cache, v_cache, block_tables, context_lens, scale: float,
                  num_splits: int, out, stream=None, workspace: Optional[torch.Tensor] = None):
    """One decode step with the append fused in: new_k[b], new_v[b] ([B, Hkv, D])
    are written to the cache row of token context_lens[b] - 1 of sequence b,
    then out = decode(...) over all context_lens[b] tokens."""
    NB, bs, Hkv, D, B, Hq, W, dev = _decode_dims(q, k_cache, v_cache, block_tables, context_lens)
    _need(out, "out", torch.bfloat16, 3, dev)
    _need(new_k, "new_k", torch.bfloat16, 3, dev)
    _need(new_v, "new_v", torch.bfloat16, 3, dev)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError(f"out must be [{B}, {Hq}, {D}]")
    if tuple(new_k.shape) != (B, Hkv, D) or tuple(new_v.shape) != (B, Hkv, D):
        raise ValueError(f"new_k/new_v must be [{B}, {Hkv}, {D}]")
    if num_splits == 0 and B > 0:
        num_splits = auto_splits(B, Hkv, W, bs, dev)
    ws_ptr, ws_bytes, workspace = _workspace(B, Hq, D, num_splits, dev, workspace, stream=stream)
    _check("pa_append_decode", lib().pa_append_decode(
        q.data_ptr(), new_k.data_ptr(), new_v.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), float(scale), int(num_splits),
        out.data_ptr(), B, Hq, Hkv, D, bs, NB, W, ws_ptr, ws_bytes, _stream_ptr(stream, dev)))
    return out


def _scratch(nbytes: int, dev, stream) -> torch.Tensor:
    """A workspace from torch's caching allocator, allocated on the stream the
    call is enqueued on (not necessarily the current one): the allocator then
    hands the block to later work only in that stream's order, so freeing it
    when the call returns cannot let other streams overwrite it while the
    kernels still use it.  No fill: the kernels read only what they wrote."""
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=dev)
    with torch.cuda.stream(stream):
        return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def _workspace(B, Hq, D, num_splits, dev, workspace, q_len=1, stream=None):
    need = decode_multi_workspace_size(B, q_len, Hq, D, num_splits) if B > 0 else 0
    if not need:
        return None, 0, workspace
    if workspace is None:
        workspace = _scratch(need, dev, stream)
    if workspace.device != dev or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes on {dev}")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace


def _decode_dims(q, k_cache, v_cache, block_tables, context_lens, pool_dtype=torch.bfloat16):
    NB, bs, Hkv, D = _pool_dims(k_cache, v_cache, pool_dtype)
    dev = k_cache.device
    _need(q, "q", torch.bfloat16, 3, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, Hq, Dq = (int(x) for x in q.shape)
    if Dq != D:
        raise ValueError(f"q head_dim {Dq} differs from the pool's {D}")
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables/context_lens batch differs from q")
    return NB, bs, Hkv, D, B, Hq, int(block_tables.shape[1]), dev


def decode_partials(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                    num_splits: int, workspace: torch.Tensor, stream=None) -> int:
    """Split pass only: per-piece normalised outputs and base-2 log-sum-exps
    into `workspace` (layout in include/pagedattn.h).  Needs at least two
    pieces.  Returns the resolved num_splits."""
    NB, bs, Hkv, D, B, Hq, W, dev = _decode_dims(q, k_cache, v_cache, block_tables, context_lens)
    if num_splits == 0:
        num_splits = auto_splits(B, Hkv, W, bs, dev)
    _check("pa_decode_partials", lib().pa_decode_partials(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), float(scale), int(num_splits), B, Hq, Hkv, D, bs, NB, W,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream_ptr(stream, dev)))
    return num_splits


def decode_merge(workspace: torch.Tensor, context_lens, out, num_splits: int, num_kv_heads: int,
                 block_size: int, max_blocks_per_seq: int, stream=None):
    """Merge pass only: combine the partials in `workspace` into bf16 `out`."""
    dev = out.device
    _need(out, "out", torch.bfloat16, 3, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, Hq, D = (int(x) for x in out.shape)
    _check("pa_decode_merge", lib().pa_decode_merge(
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        context_lens.data_ptr(), out.data_ptr(), int(num_splits), B, Hq, int(num_kv_heads), D,
        int(block_size), int(max_blocks_per_seq), _stream_ptr(stream, dev)))
    return out


def prefill(q, cu_seqlens_q, k_cache, v_cache, block_tables, context_lens, scale: float, out,
            max_q_len: int, num_splits: int = 0, stream=None,
            workspace: Optional[torch.Tensor] = None):
    """Causal attention of packed chunk queries q [Tq, Hq, D] (sequence b owns
    rows cu_seqlens_q[b]..cu_seqlens_q[b+1]) over each sequence's cached
    context_lens[b] tokens, chunk included; query i of an n-row chunk sits at
    position context_lens[b] - n + i.  num_splits = 0 picks the key split
    automatically."""
    return _prefill(q, cu_seqlens_q, k_cache, v_cache, block_tables, context_lens, scale, out,
                    max_q_len, num_splits, stream, workspace, None)


def prefill_fp8(q, cu_seqlens_q, k_cache, v_cache, block_tables, context_lens, scale: float,
                k_scale: float, v_scale: float, out, max_q_len: int, num_splits: int = 0,
                stream=None, workspace: Optional[torch.Tensor] = None):
    """prefill over fp8 pools (uint8 e4m3 codes [NB, Hkv, bs, D]): K and V are
    the codes' values times k_scale and v_scale."""
    return _prefill(q, cu_seqlens_q, k_cache, v_cache, block_tables, context_lens, scale, out,
                    max_q_len, num_splits, stream, workspace, (float(k_scale), float(v_scale)))


def _prefill(q, cu_seqlens_q, k_cache, v_cache, block_tables, context_lens, scale, out,
             max_q_len, num_splits, stream, workspace, fp8_scales):
    NB, bs, Hkv, D = _pool_dims(k_cache, v_cache,
                                torch.bfloat16 if fp8_scales is None else torch.uint8)
    dev = k_cache.device
    _need(q, "q", torch.bfloat16, 3, dev)
    _need(out, "out", torch.bfloat16, 3, dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    Tq, Hq, Dq = (int(x) for x in q.shape)
    B = int(context_lens.shape[0])
    if Dq != D or tuple(out.shape) != (Tq, Hq, D):
        raise ValueError(f"q/out must be [{Tq}, {Hq}, {D}]")
    if cu_seqlens_q.shape[0] != B + 1 or block_tables.shape[0] != B:
        raise ValueError("cu_seqlens_q must have num_seqs + 1 entries")
    W = int(block_tables.shape[1])
    if num_splits == 0 and B > 0 and max_q_len > 0:
        num_splits = prefill_auto_splits(B, int(max_q_len), Hkv, W, bs, dev)
    need = (int(lib().pa_prefill_workspace_size(B, int(max_q_len), Hq, D, int(num_splits)))
            if B > 0 and max_q_len > 0 else 0)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = _scratch(need, dev, stream)
        if workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace needs {need} bytes")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    ptrs = (q.data_ptr(), cu_seqlens_q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), float(scale))
    rest = (int(num_splits), out.data_ptr(), B, int(max_q_len), Hq, Hkv, D, bs, NB, W, ws_ptr,
            ws_bytes, _stream_ptr(stream, dev))
    if fp8_scales is None:
        _check("pa_prefill", lib().pa_prefill(*ptrs, *rest))
    else:
        _check("pa_prefill_fp8", lib().pa_prefill_fp8(*ptrs, *fp8_scales, *rest))
    return out

def prefill_workspace_size(num_seqs, max_q_len, num_q_heads, head_dim, num_splits) -> int:
    return int(lib().pa_prefill_workspace_size(num_seqs, max_q_len, num_q_heads, head_dim,
                                               num_splits))


def prefill_auto_splits(num_seqs, max_q_len, num_kv_heads, max_blocks_per_seq, block_size,
                        device=None) -> int:
    if isinstance(device, str):
        device = torch.device(device)
    if device is None:
        device = torch.cuda.current_device()
    elif isinstance(device, torch.device):
        device = device.index if device.index is not None else torch.cuda.current_device()
    cus = torch.cuda.get_device_properties(int(device)).multi_processor_count
    r = int(lib().pa_prefill_plan_splits(num_seqs, max_q_len, num_kv_heads, max_blocks_per_seq,
                                         block_size, cus))
    _check("pa_prefill_plan_splits", min(r, 0))
    return r


# Kinds of precondition violation reported by the pa_check_* calls.
PA_CHECK_OK = 0
PA_CHECK_KINDS = {
    1: "context length outside [0, max_blocks_per_seq * block_size]",
    2: "block table entry read by the sequence outside [0, num_blocks)",
    3: "the block receiving the fused append is also read through another table entry",
    4: "slot at or past num_blocks * block_size",
    5: "valid slot repeated",
    6: "query offsets: cu_seqlens_q[0] != 0, decreasing, or a chunk longer than max_q_len "
       "or than its context length",
}


class PreconditionError(ValueError):
    """A device-resident precondition of the attention calls does not hold."""

    def __init__(self, fn: str, kind: int, index: int, what: str):
        super().__init__(f"{fn}: {PA_CHECK_KINDS.get(kind, f'kind {kind}')} at {what} {index}")
        self.kind = kind
        self.index = index


def _host_ints(x, dtype, name: str):
    """A contiguous host numpy copy of an integer tensor or array-like
    (device tensors are copied synchronously)."""
    if isinstance(x, torch.Tensor):
        want = {np.int32: torch.int32, np.int64: torch.int64}[dtype]
        if x.dtype != want:
            raise TypeError(f"{name} must be {want}, got {x.dtype}")
        return np.ascontiguousarray(x.detach().cpu().numpy())
    a = np.asarray(x)
    out = np.ascontiguousarray(a.astype(dtype))
    if a.size and not np.array_equal(out, a):
        raise ValueError(f"{name} does not fit {np.dtype(dtype).name}")
    return out


def _raise_check(fn: str, r: int, bad, what: str) -> None:
    if r < 0:
        raise PagedAttnError(fn, r)
    if r != PA_CHECK_OK:
        raise PreconditionError(fn, r, int(bad.value), what)


def check_tables(block_tables, context_lens, num_blocks: int, block_size: int,
                 fused_append: bool = False) -> None:
    """Check, on host copies, what decode / decode_multi / decode_partials (and
    append_decode with fused_append=True) assume of their tables and lengths;
    raise PreconditionError naming the first offending sequence."""
    t = _host_ints(block_tables, np.int32, "block_tables")
    lens = _host_ints(context_lens, np.int32, "context_lens")
    if t.ndim != 2 or lens.ndim != 1 or t.shape[0] != lens.shape[0]:
        raise ValueError("block_tables must be [B, W] and context_lens [B]")
    bad = ctypes.c_int64(-1)
    r = lib().pa_check_tables(t.ctypes.data, lens.ctypes.data, int(t.shape[0]), int(t.shape[1]),
                              int(block_size), int(num_blocks), int(bool(fused_append)),
                              ctypes.byref(bad))
    _raise_check("pa_check_tables", r, bad, "sequence")


def check_slots(slot_mapping, num_blocks: int, block_size: int) -> None:
    """Check, on a host copy, what reshape_and_cache(_fp8) assumes of its slots;
    raise PreconditionError naming the first offending token."""
    s = _host_ints(slot_mapping, np.int64, "slot_mapping")
    if s.ndim != 1:
        raise ValueError("slot_mapping must be 1-D")
    bad = ctypes.c_int64(-1)
    r = lib().pa_check_slots(s.ctypes.data, int(s.shape[0]), int(num_blocks), int(block_size),
                             ctypes.byref(bad))
    _raise_check("pa_check_slots", r, bad, "token")


def check_prefill(cu_seqlens_q, context_lens, max_q_len: int) -> None:
    """Check, on host copies, what prefill(_fp8) assumes of its query offsets;
    raise PreconditionError naming the first offending sequence."""
    cu = _host_ints(cu_seqlens_q, np.int32, "cu_seqlens_q")
    lens = _host_ints(context_lens, np.int32, "context_lens")
    if cu.ndim != 1 or lens.ndim != 1 or cu.shape[0] != lens.shape[0] + 1:
        raise ValueError("cu_seqlens_q must be [B + 1] and context_lens [B]")
    bad = ctypes.c_int64(-1)
    r = lib().pa_check_prefill(cu.ctypes.data, lens.ctypes.data, int(lens.shape[0]),
                               int(max_q_len), ctypes.byref(bad))
    _raise_check("pa_check_prefill", r, bad, "sequence")


__all__ = ["reshape_and_cache", "decode", "append_decode", "decode_partials", "decode_merge", "prefill",
           "prefill_workspace_size", "prefill_auto_splits", "decode_workspace_size", "plan_splits",
           "auto_splits", "plan_splits_lengths", "auto_splits_lengths", "decode_multi", "decode_multi_workspace_size", "reshape_and_cache_fp8",
           "decode_fp8", "append_decode_fp8", "decode_multi_fp8", "prefill_fp8", "BlockManager", "lib", "LIB_PATH", "SIGNATURES", "PagedAttnError",
           "PA_MAX_SPLITS", "PA_MAX_QUERY_TOKENS", "PA_MAX_SEQS", "PA_MAX_HEADS",
           "check_tables", "check_slots", "check_prefill", "PreconditionError", "PA_CHECK_KINDS"]


class BlockManager:
    """The library's host-side KV pool manager (include/pa_block_manager.h):
    slots for pa_reshape_and_cache and block tables for the decode and prefill
    calls.  Token ids and results are numpy arrays in host memory.  Errors
    raise PagedAttnError with the status code."""

    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int,
                 prefix_cache: bool = True):
        import numpy as np
        self._np = np
        self.block_size, self.max_blocks_per_seq = block_size, max_blocks_per_seq
        h = lib().pa_bm_create(num_blocks, block_size, max_blocks_per_seq, int(bool(prefix_cache)))
        if not h:
            raise ValueError("pa_bm_create refused its arguments")
        self._h = ctypes.c_void_p(h)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.pa_bm_destroy(h)
            self._h = None

    def _tok(self, tokens):
        t = self._np.ascontiguousarray(tokens, dtype=self._np.int32)
        return t, t.ctypes.data_as(ctypes.c_void_p)

    def admit(self, seq_id: int, priority: int, tokens):
        """Returns (num_cached_tokens, slots of the uncached prompt tokens)."""
        t, tp = self._tok(tokens)
        slots = self._np.empty(max(len(t), 1), dtype=self._np.int64)
        cached = ctypes.c_int64(0)
        _check("pa_bm_admit", lib().pa_bm_admit(self._h, seq_id, priority, tp, len(t),
                                                ctypes.byref(cached),
                                                slots.ctypes.data_as(ctypes.c_void_p)))
        return int(cached.value), slots[:len(t) - cached.value]

    def append(self, seq_id: int, tokens):
        """Returns the slots of the new tokens."""
        t, tp = self._tok(tokens)
        slots = self._np.empty(max(len(t), 1), dtype=self._np.int64)
        _check("pa_bm_append", lib().pa_bm_append(self._h, seq_id, tp, len(t),
                                                  slots.ctypes.data_as(ctypes.c_void_p)))
        return slots[:len(t)]

    def decode_step(self, seq_ids, tokens=None):
        """One token per listed sequence (all or nothing); returns the slots."""
        ids = self._np.ascontiguousarray(seq_ids, dtype=self._np.int64)
        n = len(ids)
        slots = self._np.empty(max(n, 1), dtype=self._np.int64)
        tp = None
        if tokens is not None:
            t, tp = self._tok(tokens)
            if len(t) != n:
                raise ValueError("one token per sequence")
        _check("pa_bm_decode_step", lib().pa_bm_decode_step(
            self._h, ids.ctypes.data_as(ctypes.c_void_p), n, tp,
            slots.ctypes.data_as(ctypes.c_void_p)))
        return slots[:n]

    def truncate(self, seq_id: int, new_len: int) -> None:
        _check("pa_bm_truncate", lib().pa_bm_truncate(self._h, seq_id, new_len))

    def release(self, seq_id: int) -> None:
        _check("pa_bm_release", lib().pa_bm_release(self._h, seq_id))

    def preempt(self) -> int:
        v = ctypes.c_int64(0)
        _check("pa_bm_preempt", lib().pa_bm_preempt(self._h, ctypes.byref(v)))
        return int(v.value)

    def block_tables(self, seq_ids):
        """Returns (tables int32 [n, max_blocks_per_seq], lens int32 [n])."""
        ids = self._np.ascontiguousarray(seq_ids, dtype=self._np.int64)
        n = len(ids)
        tables = self._np.zeros((n, self.max_blocks_per_seq), dtype=self._np.int32)
        lens = self._np.zeros(n, dtype=self._np.int32)
        _check("pa_bm_block_tables", lib().pa_bm_block_tables(
            self._h, ids.ctypes.data_as(ctypes.c_void_p), n,
            tables.ctypes.data_as(ctypes.c_void_p), lens.ctypes.data_as(ctypes.c_void_p)))
        return tables, lens

    def order_longest_first(self, seq_ids):
        """The ids of seq_ids sorted by context length, longest first (ties keep
        their order): the launch order that keeps a large decode batch's last
        workgroups short."""
        ids = self._np.ascontiguousarray(seq_ids, dtype=self._np.int64)
        out = self._np.empty(len(ids), dtype=self._np.int64)
        _check("pa_bm_order_longest_first", lib().pa_bm_order_longest_first(
            self._h, ids.ctypes.data_as(ctypes.c_void_p), len(ids),
            out.ctypes.data_as(ctypes.c_void_p)))
        return out

    def stats(self):
        """(free, cached, used) blocks and the number of running sequences."""
        v = [ctypes.c_int64(0) for _ in range(4)]
        _check("pa_bm_stats", lib().pa_bm_stats(self._h, *[ctypes.byref(x) for x in v]))
        return tuple(int(x.value) for x in v)
