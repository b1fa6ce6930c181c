"""Host logic of the graph helper (no GPU)."""
import pytest

from paged_kv_attention_09_amd.graphs import padded_sizes


def test_padded_sizes():
    assert padded_sizes(1) == [1]
    assert padded_sizes(5) == [1, 2, 4, 8]
    assert padded_sizes(8) == [1, 2, 4, 8]
    assert padded_sizes(9) == [1, 2, 4, 8, 16]
    with pytest.raises(ValueError):
        padded_sizes(0)
