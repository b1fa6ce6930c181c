"""Loaders that turn the hand-worked fixtures under tests/golden/ into arrays."""
import json
import os

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bits(x):
    return W.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def decode_case(name):
    """Returns (q, k_cache, v_cache, tables, lens, scale, expected) as bf16 bits /
    int32 / float32 / float64."""
    g = load(name)
    nb, bs, hkv, d = g["num_blocks"], g["block_size"], g["num_kv_heads"], g["head_dim"]
    kc = np.full((nb, bs, hkv, d), W.BF16_NAN, np.uint16)
    vc = kc.copy()
    tables = np.array(g["block_tables"], np.int32)
    lens = np.array(g["context_lens"], np.int32)
    for b, L in enumerate(lens):
        for t in range(int(L)):
            kc[tables[b, t // bs], t % bs] = 0
    if "v_rows" in g:
        for key, row in g["v_rows"].items():
            blk, off = map(int, key.split(","))
            vc[blk, off, 0] = bits(row)
    else:
        for key, row in g["v_rows_by_head"].items():
            blk, off, h = map(int, key.split(","))
            vc[blk, off, h] = bits(row)
    q = bits(g["q"])
    return q, kc, vc, tables, lens, np.float32(g["scale"]), np.array(g["expected_out"], np.float64)


def append_case(name="append_slots.json"):
    g = load(name)
    nb, bs, hkv, d = g["num_blocks"], g["block_size"], g["num_kv_heads"], g["head_dim"]
    init = bits(g["initial_value"])
    kc = np.full((nb, bs, hkv, d), init, np.uint16)
    vc = kc.copy()
    ek, ev = kc.copy(), vc.copy()
    for key, row in g["expected_k_written"].items():
        blk, off = map(int, key.split(","))
        ek[blk, off, 0] = bits(row)
    for key, row in g["expected_v_written"].items():
        blk, off = map(int, key.split(","))
        ev[blk, off, 0] = bits(row)
    return (bits(g["new_k"]), bits(g["new_v"]), np.array(g["slot_mapping"], np.int64), kc, vc,
            ek, ev)
