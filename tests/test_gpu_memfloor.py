"""The benchmark's memory-floor kernels (libsrftq_memfloor.so) move every
byte they are timed for: each 16-byte output chunk of a tile holds the XOR
of that lane's input chunks, so every input byte is read and every output
byte written, for one tile per block and for persistent grids."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MIX = {0: (16, 5), 1: (5, 16), 2: (16, 16)}   # KiB read, KiB written per tile


def _lib():
    L = ctypes.CDLL(os.path.join(ROOT, "kv_cache_quantization_srft_amd", "libsrftq_memfloor.so"))
    L.srftq_memfloor.restype = ctypes.c_int
    L.srftq_memfloor.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_int, ctypes.c_void_p]
    return L


def _expected(inp, R, W, n_tiles):
    """out[t, i, l] = (acc, acc + 1, acc + 2, acc + i) with acc the XOR of the
    four dwords of lane l's R input chunks of tile t."""
    a = inp.reshape(n_tiles, R, 64, 4)
    acc = np.bitwise_xor.reduce(np.bitwise_xor.reduce(a, axis=3), axis=1)      # [n_tiles, 64]
    out = np.empty((n_tiles, W, 64, 4), dtype=np.uint32)
    out[..., 0] = acc[:, None, :]
    out[..., 1] = acc[:, None, :] + np.uint32(1)
    out[..., 2] = acc[:, None, :] + np.uint32(2)
    out[..., 3] = acc[:, None, :] + np.arange(W, dtype=np.uint32)[None, :, None]
    return out.reshape(-1)


@pytest.mark.parametrize("mix", [0, 1, 2])
@pytest.mark.parametrize("grid", ["tiles", 7, 64])
@pytest.mark.parametrize("nt", [0, 1])
def test_memfloor_moves_every_byte(mix, grid, nt):
    R, W = MIX[mix]
    n_tiles = 301
    g = n_tiles if grid == "tiles" else grid
    rng = np.random.default_rng(100 + mix)
    inp = rng.integers(0, 2**32, size=n_tiles * R * 256, dtype=np.uint32)
    din = torch.from_numpy(inp.view(np.int32)).cuda()
    dout = torch.full((n_tiles * W * 256,), -1, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    rc = _lib().srftq_memfloor(mix, nt, din.data_ptr(), dout.data_ptr(), n_tiles, g, s.cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = dout.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, _expected(inp, R, W, n_tiles))
