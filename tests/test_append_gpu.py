"""GPU slot-mapped append: bit-exact against the oracle over the whole pool."""
import numpy as np
import pytest
import torch

import golden_cases as G
import oracle
import paged_kv_attention_09_amd as pa
import workloads as W
from gpu_cases import DEV, bf16_tensor, device_pool, to_bits

pytestmark = pytest.mark.gpu


def _check_append(kc, vc, new_k, new_v, slots):
    """Read the pools back, run the oracle append on those bits, run the GPU
    append, and require every byte of both pools to match."""
    before_k, before_v = to_bits(kc), to_bits(vc)
    want_k, want_v = oracle.append(new_k, new_v, slots, before_k, before_v)
    pa.reshape_and_cache(bf16_tensor(new_k), bf16_tensor(new_v),
                         torch.from_numpy(np.asarray(slots, np.int64)).to(DEV), kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(kc), want_k)
    assert np.array_equal(to_bits(vc), want_v)


def test_append_golden():
    """The hand-worked fixture, embedded in a supported shape: a slot is a row
    of the pool viewed as [num_blocks * block_size, kv_heads * head_dim], so
    the fixture's 12 rows of 2 values become the first 12 rows (first 2
    columns) of a [1, 16, 1, 64] pool."""
    nk, nv, slots, kc, vc, ek, ev = G.append_case()

    def embed(rows, fill):
        out = np.full((16, 64), fill, np.uint16)
        r = rows.reshape(-1, rows.shape[-2] * rows.shape[-1])
        out[:r.shape[0], :r.shape[1]] = r
        return out

    z = np.uint16(0)
    k_dev = bf16_tensor(embed(kc, z).reshape(1, 16, 1, 64))
    v_dev = bf16_tensor(embed(vc, z).reshape(1, 16, 1, 64))
    new_k = np.zeros((len(slots), 1, 64), np.uint16)
    new_v = np.zeros((len(slots), 1, 64), np.uint16)
    new_k[:, 0, :2] = nk[:, 0, :]
    new_v[:, 0, :2] = nv[:, 0, :]
    pa.reshape_and_cache(bf16_tensor(new_k), bf16_tensor(new_v),
                         torch.from_numpy(slots).to(DEV), k_dev, v_dev)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(k_dev).reshape(16, 64), embed(ek, z))
    assert np.array_equal(to_bits(v_dev).reshape(16, 64), embed(ev, z))


def test_append_decode_step_tokens():
    """The 8 new tokens of the 28/4-head, bs-256 decode batch."""
    inp = W.make_decode_inputs(W.CONFIGS["c3"])
    kc, vc = device_pool(inp.pool)
    _check_append(kc, vc, inp.new_k, inp.new_v, inp.slot_mapping)


def test_append_prefill_chunk_and_decodes():
    """A 512-token prompt chunk plus 64 decode tokens in one call, with
    padding rows (slot -1) mixed in."""
    pin = W.make_prefill_inputs(W.PREFILL_CONFIGS["c5p"])
    dec = W.make_decode_inputs(W.CONFIGS["c5d"].with_(num_blocks=2048))
    # both use their own pools; append into the prefill pool with the decode
    # tokens redirected to free blocks of it
    free = np.setdiff1d(np.arange(2048), pin.pool.ids)[:64]
    dec_slots = free.astype(np.int64) * 256 + 7
    nk = np.concatenate([pin.new_k, dec.new_k, pin.new_k[:5]])
    nv = np.concatenate([pin.new_v, dec.new_v, pin.new_v[:5]])
    slots = np.concatenate([pin.slot_mapping, dec_slots, -np.ones(5, np.int64)])
    kc, vc = device_pool(pin.pool)
    _check_append(kc, vc, nk, nv, slots)


@pytest.mark.parametrize("D,bs", [(64, 16), (128, 16), (64, 256)])
def test_append_shapes(D, bs):
    rng = np.random.default_rng(D + bs)
    NB, Hkv, T = 37, 3, 50
    kc = bf16_tensor(W.f32_to_bf16_bits(rng.standard_normal((NB, bs, Hkv, D), dtype=np.float32)))
    vc = bf16_tensor(W.f32_to_bf16_bits(rng.standard_normal((NB, bs, Hkv, D), dtype=np.float32)))
    slots = rng.choice(NB * bs, size=T, replace=False).astype(np.int64)
    slots[::7] = -1
    nk = W.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32))
    nv = W.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32))
    _check_append(kc, vc, nk, nv, slots)


def test_append_zero_tokens_is_noop():
    kc = torch.zeros((4, 16, 1, 64), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    e = torch.empty((0, 1, 64), dtype=torch.bfloat16, device=DEV)
    pa.reshape_and_cache(e, e, torch.empty(0, dtype=torch.int64, device=DEV), kc, vc)
    torch.cuda.synchronize()
    assert (kc == 0).all()
