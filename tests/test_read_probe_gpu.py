"""The streaming-read probe the benchmark uses as its measured read
reference (libpa_readprobe.so, outside the attention library) must read
every byte it is given: the XOR of the words the waves report equals the XOR
of the whole buffer, for every unroll and for sizes that do and do not fill
the grid's slices.  Its argument checks run on the CPU."""
import ctypes
import os

import numpy as np
import pytest
import torch

import paged_kv_attention_09_amd as pa

PROBE = os.path.join(os.path.dirname(pa.LIB_PATH), "libpa_readprobe.so")


def probe():
    f = ctypes.CDLL(PROBE).pa_bench_read_probe
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    return f


def test_probe_argument_checks():
    f, P = probe(), 256
    assert f(None, 16, P, 1, 4, None) == -1 and f(P, 16, None, 1, 4, None) == -1
    assert f(P, 0, P, 1, 4, None) == -2 and f(P, 24, P, 1, 4, None) == -2
    assert f(P, 16, P, 0, 4, None) == -2 and f(P, 16, P, 1, 5, None) == -2


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes,wgs,unroll", [(16, 1, 4), (4096, 3, 8), ((1 << 20) + 48, 64, 16),
                                               ((1 << 20) + 48, 1000, 4), (32 << 20, 4096, 8)])
def test_read_probe_reads_every_byte(nbytes, wgs, unroll):
    rng = np.random.default_rng(nbytes % 1000 + wgs + unroll)
    words = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to("cuda:0")
    sink = torch.zeros(4 * wgs, dtype=torch.int32, device="cuda:0")
    st = probe()(buf.data_ptr(), nbytes, sink.data_ptr(), wgs, unroll,
                 torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
