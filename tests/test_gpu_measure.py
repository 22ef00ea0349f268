"""The streaming-read helper (include/qkv_measure.h) that the benchmark's read
ceiling comes from: it must read every byte once.  The XOR of the words it
writes to the sink equals the XOR of all 32-bit words of the buffer (XOR is
order-free), for sizes and workgroup counts whose ranges end inside a
thread's four-load step, and with more workgroups than 16-byte words."""
import ctypes

import numpy as np
import pytest
import torch

from quantized_kv_cache_amd import _lib

pytestmark = pytest.mark.gpu

MAX_WGS = 8192


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 2048 * 256 * 16 * 4 + 48, 3 * 2 ** 24 + 784])
@pytest.mark.parametrize("wgs", [1, 7, 256, 2048, MAX_WGS])
def test_measure_read_touches_every_word(nbytes, wgs):
    L = _lib.load()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(4 * wgs, dtype=torch.int32, device="cuda")
    st = L.qkv_measure_read(ctypes.c_void_p(buf.data_ptr()), nbytes, wgs, ctypes.c_void_p(sink.data_ptr()),
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _lib.QKV_OK, L.qkv_last_error()
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host), (nbytes, wgs)
