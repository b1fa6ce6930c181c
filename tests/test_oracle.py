"""The oracle against its pins, and the pins against planted mistakes.

The mutation half plants one plausible slip at a time into a private copy of
the oracle's source (a wrong GQA mapping, a transposed block/offset, a lost
normalisation, an off-by-one in the causal window, ...) and requires that at
least one pin rejects the copy.  The real oracle is never modified.
"""
import inspect
import types

import pytest

import oracle.paged_attention as real
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(real)


MUTANTS = {
    "gqa_interleaved": ("return h // (num_q_heads // num_kv_heads)", "return h % num_kv_heads"),
    "block_offset_swapped": ("return t // block_size, t % block_size",
                             "return t % block_size, t // block_size"),
    "no_normalisation": ("return (w @ values) / w.sum()", "return (w @ values)"),
    "scale_dropped": ("s = float(scale) * (keys @ qvec)", "s = (keys @ qvec)"),
    "softmax_sign": ("w = np.exp(s - s.max())", "w = np.exp(s.max() - s)"),
    "token_dropped": ("for t in range(num_tokens):", "for t in range(num_tokens - 1):"),
    "bf16_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "q_head_fixed": ("attend(qf[b, h], K[:, g, :]", "attend(qf[b, 0], K[:, g, :]"),
    "prefill_top_left": ("p = L - n + i ", "p = i "),
    "prefill_excludes_self": ("K[:p + 1, g, :], V[:p + 1, g, :]", "K[:p, g, :], V[:p, g, :]"),
    "multi_window_shifted": ("p = L - QL + j ", "p = L - QL + j + 1 "),
    "multi_negative_wraps": ("n_keys = p + 1 if p >= 0 else 0", "n_keys = p + 1"),
    "multi_query_token_fixed": ("attend(qf[b, j, h]", "attend(qf[b, 0, h]"),
    "append_transposed": ("kc[s // bs, s % bs] = new_k[i]", "kc[s % bs, s // bs] = new_k[i]"),
    "append_negative_written": ("if s < 0:", "if s < -1:"),
    "append_v_from_k": ("vc[s // bs, s % bs] = new_v[i]", "vc[s // bs, s % bs] = new_k[i]"),
}


def _mutant(old, new):
    src = inspect.getsource(real)
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:          # AssertionError, or a crash the slip causes
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin rejects mutant {name}"


# --------------------------------------------------------------------------
# FP8 KV pages
# --------------------------------------------------------------------------

import oracle.kv_fp8 as real_fp8  # noqa: E402


@pytest.mark.parametrize("pin", P.FP8_PINS, ids=lambda f: f.__name__)
def test_fp8_pin(pin):
    pin(real_fp8)


FP8_MUTANTS = {
    "ties_away": ("code = int(np.rint(a / 2.0 ** -9))", "code = int(np.floor(a / 2.0 ** -9 + 0.5))"),
    "mantissa_ties_away": ("m = int(np.rint((2.0 * f - 1.0) * 8.0))",
                           "m = int(np.floor((2.0 * f - 1.0) * 8.0 + 0.5))"),
    "bias_8": ("code = ((e + 7) << 3) | m", "code = ((e + 8) << 3) | m"),
    "decode_bias_8": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "no_clamp": ("y = np.clip(x * inv, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))", "y = x * inv"),
    "scale_not_inverted": ("inv = np.float32(1.0) / np.float32(scale)", "inv = np.float32(scale)"),
    "k_scale_dropped": ("K = e4m3_decode(gather_sequence(k_cache8, table, L)) * ks",
                        "K = e4m3_decode(gather_sequence(k_cache8, table, L))"),
    "v_scale_dropped": ("V = e4m3_decode(gather_sequence(v_cache8, table, L)) * vs",
                        "V = e4m3_decode(gather_sequence(v_cache8, table, L))"),
    "fp8_multi_window_shifted": ("            p = L - QL + j\n            n_keys", "            p = L - QL + j - 1\n            n_keys"),
    "subnormal_step": ("sub = m * 2.0 ** -9", "sub = m * 2.0 ** -10"),
    "no_token_major_view": ("return np.transpose(pool8, (0, 2, 1, 3))", "return pool8"),
    "fp8_prefill_causal_off_by_one": ("            p = L - n + i\n", "            p = L - n + i - 1\n"),
    "append_wrong_head_axis": ("kc[s // bs, :, s % bs] = quantize(new_k[i], k_scale)",
                               "kc[s // bs, :, s % bs] = quantize(new_k[i], k_scale)[::-1]"),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_pins_catch_mutant(name):
    old, new = FP8_MUTANTS[name]
    src = inspect.getsource(real_fp8)
    assert src.count(old) == 1, f"anchor not unique/found: {old!r}"
    src = src.replace(old, new).replace("from .paged_attention import",
                                        "from oracle.paged_attention import")
    mod = types.ModuleType("fp8_mutant")
    exec(compile(src, "fp8_mutant", "exec"), mod.__dict__)
    caught = []
    for pin in P.FP8_PINS:
        try:
            pin(mod)
        except Exception as e:
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin rejects {name}"
