"""The oracle against the hand-worked fixtures in tests/golden/."""
import numpy as np
import pytest

import golden_cases as G
import oracle


@pytest.mark.parametrize("name", ["paged_uniform_mean.json", "paged_gqa_mean.json"])
def test_decode_golden(name):
    q, kc, vc, tables, lens, scale, want = G.decode_case(name)
    got = oracle.decode(q, kc, vc, tables, lens, scale)
    assert np.array_equal(got, want)


def test_append_golden():
    nk, nv, slots, kc, vc, ek, ev = G.append_case()
    k2, v2 = oracle.append(nk, nv, slots, kc, vc)
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev)
