"""The streaming probe bench.py reads the HBM ceiling with (libpa_probe.so)
reads exactly the tiles it is given: each lane's XOR of the 32-bit words it
loaded, recomputed on the CPU."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _probe():
    L = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_78_amd", "libpa_probe.so"))
    L.pa_probe_stream.restype = ctypes.c_int
    i32 = ctypes.c_int32
    L.pa_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, i32, i32, i32,
                                  i32, i32, ctypes.c_void_p, ctypes.c_void_p]
    return L


@pytest.mark.parametrize("nontemporal,tile_bytes,in_flight", [(0, 4096, 3), (1, 4096, 3),
                                                             (1, 2048, 2), (1, 2048, 8),
                                                             (1, 4096, 6)])
def test_probe_reads_the_listed_tiles(nontemporal, tile_bytes, in_flight):
    num_tiles, waves, per = 300, 6, 70          # 70 tiles: two id windows and a ragged ring
    g = torch.Generator().manual_seed(3)
    pool = torch.randint(-2**31, 2**31 - 1, (num_tiles * tile_bytes // 4,), generator=g,
                         dtype=torch.int32)
    ids = torch.randint(0, num_tiles, (waves * per,), generator=g, dtype=torch.int32)
    ids[5] = num_tiles + 7                       # out of the pool: read as zeros, not read
    sink = torch.zeros(waves * 64, dtype=torch.int32, device=DEV)
    gp, gi = pool.to(DEV), ids.to(DEV)
    st = _probe().pa_probe_stream(gp.data_ptr(), num_tiles, gi.data_ptr(), waves, per, tile_bytes,
                                  in_flight, nontemporal, sink.data_ptr(), None)
    assert st == 0
    torch.cuda.synchronize()
    loads = tile_bytes // 1024
    words = pool.numpy().view(np.uint32).reshape(num_tiles, loads, 64, 4)   # [tile, load, lane, word]
    want = np.zeros((waves, 64), dtype=np.uint32)
    for w in range(waves):
        for t in ids[w * per:(w + 1) * per].tolist():
            if 0 <= t < num_tiles:
                want[w] ^= np.bitwise_xor.reduce(words[t].transpose(1, 0, 2).reshape(64, 4 * loads),
                                                 axis=1)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32).reshape(waves, 64), want)
