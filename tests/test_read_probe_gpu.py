"""The streaming-read probe the benchmark uses as its measured read
reference must read every byte it is given: the XOR of the words the waves
report equals the XOR of the whole buffer, for buffer sizes that are and are
not multiples of the grid's stride."""
import numpy as np
import pytest
import torch

import paged_kv_attention_09_amd as pa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,wgs", [(16, 1), (4096, 3), ((1 << 20) + 48, 64),
                                         (32 << 20, 4096)])
def test_read_probe_reads_every_byte(nbytes, wgs):
    rng = np.random.default_rng(nbytes % 1000 + wgs)
    words = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to("cuda:0")
    sink = torch.zeros(4 * wgs, dtype=torch.int32, device="cuda:0")
    st = pa.lib().pa_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), wgs,
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
