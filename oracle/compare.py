"""Element-by-element comparison of GPU results with the oracle's.

TEST INFRASTRUCTURE ONLY (tests, smoke check).  Tolerances:

  rotation     fp32 GPU vs fp64 oracle: relative L2 per vector <= 1e-3 and
               max |diff| <= 1e-5 * ||x|| (fp32 accumulation).
  scales       every scale within 1e-3 relative (a one-ulp fp16 step when
               the fp32 absmax sits on an fp16 rounding boundary), zero
               scales exact.
  codes        bit-exact except +-1 at rounding ties; a mismatch is accepted
               only when its group's scale differs or the oracle's z/sigma
               lies within 1e-4 of a half-integer; at most 1e-4 of elements.
  dequantize   GPU vs oracle on the same codes and scales: every element
               within one fp16 ulp of the oracle's value plus the fp32
               transform's absolute budget 2^-18 * ||vector||, and relative
               L2 <= 1e-3.
"""
from __future__ import annotations

import numpy as np

TIE_WINDOW = 1e-4
MAX_CODE_MISMATCH = 1e-4


def decode_codes(codes, bits, d):
    c = np.asarray(codes, dtype=np.uint8)
    if bits == 8:
        return c.view(np.int8).astype(np.int64)
    lo = (c & 0xF).astype(np.int64)
    hi = (c >> 4).astype(np.int64)
    q = np.empty(c.shape[:-1] + (d,), dtype=np.int64)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    return np.where(q >= 8, q - 16, q)


def _f16(bits_or_half):
    a = np.asarray(bits_or_half)
    if a.dtype == np.uint16:
        a = a.view(np.float16)
    return a.astype(np.float64)


def check_quantize(codes_g, scales_g, codes_o, scales_o, z_o, bits, group, d):
    """Raise AssertionError on a parity violation; return statistics."""
    sg = _f16(scales_g).reshape(-1, d // group)
    so = _f16(scales_o).reshape(-1, d // group)
    zero_o = so == 0
    assert np.array_equal(sg[zero_o], so[zero_o]), "zero scales differ"
    nz = ~zero_o
    rel = np.zeros_like(so)
    rel[nz] = np.abs(sg[nz] - so[nz]) / so[nz]
    assert np.all(np.isfinite(sg)), "non-finite scale"
    assert rel.max(initial=0.0) <= 1e-3, f"scale rel diff {rel.max():.3g} > 1e-3"
    scale_mism = sg != so

    qg = decode_codes(codes_g, bits, d).reshape(-1, d)
    qo = decode_codes(codes_o, bits, d).reshape(-1, d)
    diff = qg - qo
    mism = diff != 0
    n_mism = int(mism.sum())
    if n_mism:
        assert np.max(np.abs(diff)) == 1, f"code differs by {np.max(np.abs(diff))}"
        z = np.asarray(z_o, dtype=np.float64).reshape(-1, d)
        sig = np.repeat(so, group, axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(sig > 0, z / sig, 0.0)
        near_tie = np.abs(np.abs(ratio - np.trunc(ratio)) - 0.5) <= TIE_WINDOW
        grp_scale_diff = np.repeat(scale_mism, group, axis=1)
        unexplained = mism & ~near_tie & ~grp_scale_diff
        assert not unexplained.any(), (
            f"{int(unexplained.sum())} code mismatches away from ties, e.g. z/sigma="
            f"{ratio[unexplained][:4]}")
    frac = n_mism / qo.size
    assert frac <= MAX_CODE_MISMATCH, f"code mismatch fraction {frac:.3g} > {MAX_CODE_MISMATCH}"
    return {"codes": int(qo.size), "code_mismatch": n_mism, "scale_mismatch": int(scale_mism.sum()),
            "scale_max_rel": float(rel.max(initial=0.0))}


FP32_ABS_BUDGET = 2.0 ** -18


def check_dequantize(x_g, x_o, exact=False):
    """x_g, x_o: fp16 (or their uint16 bits) of the same shape [..., d]."""
    a = np.asarray(x_g)
    b = np.asarray(x_o)
    a = a.view(np.float16) if a.dtype == np.uint16 else a
    b = b.view(np.float16) if b.dtype == np.uint16 else b
    if exact:
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), "dequantized values differ"
    af, bf = a.astype(np.float64), b.astype(np.float64)
    assert np.all(np.isfinite(af)), "non-finite output"
    # one ulp of the reference value (spacing of fp16 at |b|) plus the fp32
    # absolute error budget of the inverse transform for that vector
    ulp = np.spacing(np.abs(b)).astype(np.float64)
    vnorm = np.linalg.norm(bf, axis=-1, keepdims=True)
    tol = ulp * 1.0001 + FP32_ABS_BUDGET * vnorm
    err = np.abs(af - bf)
    bad = err > tol
    if bad.any():
        i = np.argmax(err / tol)
        raise AssertionError(f"{int(bad.sum())} outputs beyond one fp16 ulp + fp32 budget; worst: "
                             f"ref={bf.flat[i]:.6g} got={af.flat[i]:.6g} ulp={ulp.flat[i]:.3g} "
                             f"tol={tol.flat[i]:.3g}")
    den = np.linalg.norm(bf)
    rel = np.linalg.norm(af - bf) / den if den > 0 else np.linalg.norm(af)
    assert rel <= 1e-3, f"dequantize rel L2 {rel:.3g} > 1e-3"
    return {"elements": int(b.size), "ulp_mismatch": int((a.view(np.uint16) != b.view(np.uint16)).sum()),
            "rel_l2": float(rel)}


def check_rotate(y_g, y_o, x):
    yg = np.asarray(y_g, dtype=np.float64)
    yo = np.asarray(y_o, dtype=np.float64)
    d = yo.shape[-1]
    yg2, yo2 = yg.reshape(-1, d), yo.reshape(-1, d)
    xn = np.linalg.norm(np.asarray(x, dtype=np.float64).reshape(-1, d), axis=1)
    err = np.linalg.norm(yg2 - yo2, axis=1)
    live = xn > 0
    rel = np.zeros_like(err)
    rel[live] = err[live] / xn[live]
    assert np.all(err[~live] == 0), "zero vectors must rotate to zero"
    assert rel.max(initial=0.0) <= 1e-3, f"rotation rel L2 {rel.max():.3g} > 1e-3"
    mx = np.max(np.abs(yg2 - yo2), axis=1)
    assert np.all(mx <= 1e-5 * np.maximum(xn, 1e-30)), "rotation max error above fp32 budget"
    return {"vectors": int(yo2.shape[0]), "max_rel_l2": float(rel.max(initial=0.0))}
