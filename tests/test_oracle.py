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
