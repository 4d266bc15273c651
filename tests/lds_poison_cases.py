"""Parity of the streaming kernels in the LDS-poison debug build
(libsrftq_poison.so, loaded through SRFTQ_LIBRARY): every kernel that stages
through LDS fills its buffers with 0xff bytes before each use, so a read of
LDS the kernel did not write for this tile turns into NaNs or wrong codes,
which the oracle comparison catches.  Run as a script by
test_gpu_lds_poison.py (one process for all cases); prints one line per case
and exits non-zero on the first mismatch."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

from kv_cache_quantization_srft_amd import srftq as S  # noqa: E402
from oracle import compare, oracle  # noqa: E402


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def case(B, T, H, d, g, bits, rot, lam_on, seed, variant="default"):
    r = np.random.default_rng(seed)
    x = (r.standard_normal((B, T, H, d)) * r.uniform(0.5, 3.0, (1, 1, H, d))).astype(np.float16)
    s = (1 - 2 * r.integers(0, 2, (B, H, d))).astype(np.int8)
    lam = r.uniform(0.5, 2.0, (B, H, d)).astype(np.float32) if lam_on else None
    c, sc = S.quantize(dev(x), dev(s), None if lam is None else dev(lam), g, bits, rot, variant)
    xh = S.dequantize(c, sc, dev(s), None if lam is None else dev(lam), g, bits, rot, variant)
    torch.cuda.synchronize()
    cg, sg = c.cpu().numpy(), sc.cpu().numpy().view(np.uint16)
    co, so, zo = oracle.quantize(x, s, lam, g, bits, rot, return_z=True)
    compare.check_quantize(cg, sg, co, so, zo, bits, g, d)
    xo = oracle.dequantize(cg, sg, s, lam, g, bits, rot, d=d)
    compare.check_dequantize(xh.cpu().numpy(), xo)
    print(f"ok B={B} T={T} H={H} d={d} g={g} bits={bits} rot={rot} variant={variant} lam={lam_on}", flush=True)


def main():
    assert "poison" in os.path.basename(S.LIB_PATH), S.LIB_PATH
    seed = 9000
    # ragged tiles (T not a multiple of 32 or 64), several heads and tensors,
    # tiles per block > 1 where the grid is persistent
    for d in (64, 128, 256):
        for rot in ("srft", "srht", "none"):
            for g, bits in ((16, 4), (32, 8), (d, 4)):
                seed += 1
                case(2, 173, 3, d, g, bits, rot, seed % 2 == 0, seed)
    for g in (8, 64, 128):
        seed += 1
        case(1, 301, 2, 256, g, 4, "srft", True, seed)
    seed += 1
    case(2, 77, 2, 256, 16, 4, "srft", True, seed, variant="paired")
    for g, bits in ((16, 4), (32, 8)):
        seed += 1
        case(2, 99, 3, 96, g, bits, "srft", True, seed)
    # a long tensor: many tiles per block on the persistent grid
    seed += 1
    case(1, 8192, 8, 256, 16, 4, "srft", True, seed)
    # appends into a larger cache at per-tensor positions
    B, T, H, d, g, bits, cap = 3, 45, 2, 256, 16, 4, 128
    r = np.random.default_rng(seed + 1)
    x = r.standard_normal((B, T, H, d)).astype(np.float16)
    s = (1 - 2 * r.integers(0, 2, (B, H, d))).astype(np.int8)
    pos = np.array([0, 17, 90], dtype=np.int32)
    cc = torch.zeros((B, H, cap, d * bits // 8), dtype=torch.uint8, device="cuda:0")
    cs = torch.zeros((B, H, cap, d // g), dtype=torch.float16, device="cuda:0")
    S.cache_append(dev(x), cc, cs, dev(pos), dev(s), None, g, bits)
    torch.cuda.synchronize()
    cg, sg = cc.cpu().numpy(), cs.cpu().numpy().view(np.uint16)
    co, so, zo = oracle.quantize(x, s, None, g, bits, "srft", return_z=True)   # [B, H, T, .]
    for b in range(B):
        n = min(T, cap - int(pos[b]))
        rows = slice(int(pos[b]), int(pos[b]) + n)
        compare.check_quantize(cg[b, :, rows], sg[b, :, rows], co[b, :, :n], so[b, :, :n], zo[b, :, :n], bits, g, d)
        keep = np.ones(cap, bool)
        keep[rows] = False
        assert not cg[b, :, keep].any() and not sg[b, :, keep].any(), "rows outside the append changed"
    print("ok append", flush=True)
    print("all cases passed", flush=True)


if __name__ == "__main__":
    main()
