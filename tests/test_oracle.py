"""Pins for the CPU oracle: each check ties it to something other than itself.

Sources: "When Quantization Is Free" (gist.science technical summary),
"Metodologia" 1 (SRFT(x) = pack(F diag(s) x), F the unitary DFT; SRHT as the
Hadamard alternative) and 2 (pipeline order, per-group absmax, signed int4 /
int8 rounding, two int4 per byte); HyperQuant summary, "Metodologia" 1 (the
per-tile RHT = H D x).  The pins are closed forms, library routines the
special cases reduce to (numpy's real FFT, scipy's Sylvester Hadamard,
numpy's IEEE half conversion), brute force on tiny inputs, and invariants.
"""
import math

import numpy as np
import pytest
import scipy.linalg

from oracle import oracle


def _f16(a):
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def _rand_x(rng, shape, scale=1.0):
    return _f16(rng.standard_normal(shape) * scale)


def _rand_signs(rng, B, H, d):
    return (1 - 2 * rng.integers(0, 2, size=(B, H, d))).astype(np.int8)


# --------------------------------------------------------------------------
# IEEE half conversions (the oracle's own, written from the format).
# --------------------------------------------------------------------------

def test_f16_to_f64_all_bit_patterns():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_f64_to_f16_round_to_nearest_even():
    rng = np.random.default_rng(1)
    parts = [
        rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 6, 200000),
        # exact halfway points between adjacent halves (ties)
        (np.arange(1 << 16, dtype=np.uint16).view(np.float16).astype(np.float64)),
    ]
    h = np.arange(0x0000, 0x7bff, dtype=np.uint16).view(np.float16).astype(np.float64)
    mid = (h[:-1] + np.diff(h) / 2.0)
    parts.append(mid)
    parts.append(-mid)
    v = np.concatenate(parts)
    v = v[np.isfinite(v)]
    ours = oracle.f64_to_f16(v)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("v,expect", [
    (2049.0, 2048.0),            # tie -> even significand
    (2051.0, 2052.0),
    (65519.0, 65504.0),
    (65520.0, np.inf),           # halfway to 2^16 rounds to even = overflow
    (2.0 ** -25, 0.0),           # tie between 0 and the smallest subnormal
    (3 * 2.0 ** -25, 2.0 ** -23),
    (1.0 + 2.0 ** -11, 1.0),
    (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),
])
def test_f64_to_f16_hand_cases(v, expect):
    got = oracle.f16_to_f64(oracle.f64_to_f16(np.array([v])))[0]
    assert got == expect


# --------------------------------------------------------------------------
# SRFT rotation.
# --------------------------------------------------------------------------

def _pack_rfft(x_signed):
    """Pack numpy's orthonormal rfft into the d-real layout (reading of the
    Hermitian unpack): [Re X0, sqrt2 Re X1..X_{N-1}, Re X_N, sqrt2 Im X1..]."""
    d = x_signed.shape[-1]
    N = d // 2
    X = np.fft.rfft(x_signed, norm="ortho")
    y = np.empty(x_signed.shape, dtype=np.float64)
    y[..., 0] = X[..., 0].real
    y[..., 1:N] = math.sqrt(2.0) * X[..., 1:N].real
    y[..., N] = X[..., N].real
    y[..., N + 1:] = math.sqrt(2.0) * X[..., 1:N].imag
    return y


@pytest.mark.parametrize("d", [8, 16, 64, 96, 128, 256])
def test_srft_matches_numpy_rfft(d):
    rng = np.random.default_rng(d)
    B, T, H = 2, 5, 3
    x = _rand_x(rng, (B, T, H, d))
    s = _rand_signs(rng, B, H, d)
    y = oracle.rotate(x, s, "srft")
    xs = x.astype(np.float64) * s[:, None, :, :]
    ref = _pack_rfft(xs)
    assert np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_srft_brute_force_d8():
    d, N = 8, 4
    rng = np.random.default_rng(8)
    x = _rand_x(rng, (1, 7, 1, d))
    s = _rand_signs(rng, 1, 1, d)
    y = oracle.rotate(x, s, "srft")
    F = np.array([[np.exp(-2j * np.pi * j * k / d) for j in range(d)] for k in range(d)]) / np.sqrt(d)
    for t in range(7):
        X = F @ (x[0, t, 0].astype(np.float64) * s[0, 0])
        r2 = np.sqrt(2.0)
        ref = np.array([X[0].real, r2 * X[1].real, r2 * X[2].real, r2 * X[3].real,
                        X[4].real, r2 * X[1].imag, r2 * X[2].imag, r2 * X[3].imag])
        assert np.allclose(y[0, t, 0], ref, atol=1e-13, rtol=0)


@pytest.mark.parametrize("rot,d", [(r, d) for r in ("srft", "srht") for d in (8, 32, 128, 256)]
                         + [("srft", 96), ("srft", 24)])
def test_rotation_is_orthogonal(rot, d):
    eye = np.eye(d).astype(np.float16).reshape(d, 1, d)          # d basis vectors
    M = oracle.rotate(eye, None, rot).reshape(d, d).T              # columns = M e_j
    assert np.max(np.abs(M.T @ M - np.eye(d))) < 1e-13
    assert np.max(np.abs(M @ M.T - np.eye(d))) < 1e-13


@pytest.mark.parametrize("rot,d", [(r, d) for r in ("srft", "srht", "none") for d in (16, 64, 128, 256)]
                         + [("srft", 96), ("none", 96)])
def test_parseval_and_inverse(rot, d):
    rng = np.random.default_rng(d + 7)
    x = _rand_x(rng, (2, 9, 2, d), scale=3.0)
    s = _rand_signs(rng, 2, 2, d)
    y = oracle.rotate(x, s, rot)
    xf = x.astype(np.float64)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(xf, axis=-1), rtol=1e-13, atol=0)
    back = oracle.unrotate(y, s, rot)
    assert np.max(np.abs(back - xf)) < 1e-12 * np.max(np.abs(xf))


@pytest.mark.parametrize("d", [8, 64, 128])
def test_srft_delta_closed_form(d):
    N = d // 2
    rng = np.random.default_rng(3 * d)
    s = _rand_signs(rng, 1, 1, d)
    for j0 in [0, 1, 5 % d, N - 1, N, d - 1]:
        x = np.zeros((1, 1, 1, d), dtype=np.float16)
        x[..., j0] = 1.0
        y = oracle.rotate(x, s, "srft")[0, 0, 0]
        k = np.arange(1, N)
        ref = np.concatenate([[1.0], np.sqrt(2) * np.cos(2 * np.pi * j0 * k / d),
                              [(-1.0) ** j0], -np.sqrt(2) * np.sin(2 * np.pi * j0 * k / d)])
        ref *= s[0, 0, j0] / np.sqrt(d)
        assert np.allclose(y, ref, atol=1e-14, rtol=0)


@pytest.mark.parametrize("d", [8, 64, 256])
def test_srft_constant_and_alternating(d):
    N = d // 2
    c = 1.5
    x = np.full((1, 1, 1, d), c, dtype=np.float16)
    y = oracle.rotate(x, None, "srft")[0, 0, 0]
    e = np.zeros(d)
    e[0] = c * np.sqrt(d)
    assert np.allclose(y, e, atol=1e-13, rtol=0)
    xa = (c * (-1.0) ** np.arange(d)).astype(np.float16).reshape(1, 1, 1, d)
    ya = oracle.rotate(xa, None, "srft")[0, 0, 0]
    e = np.zeros(d)
    e[N] = c * np.sqrt(d)
    assert np.allclose(ya, e, atol=1e-13, rtol=0)


# --------------------------------------------------------------------------
# SRHT rotation.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d", [2, 8, 64, 128, 256])
def test_srht_matches_scipy_hadamard(d):
    rng = np.random.default_rng(d + 11)
    x = _rand_x(rng, (1, 6, 2, d))
    s = _rand_signs(rng, 1, 2, d)
    y = oracle.rotate(x, s, "srht")
    H = scipy.linalg.hadamard(d).astype(np.float64) / np.sqrt(d)
    ref = (x.astype(np.float64) * s[:, None]) @ H.T
    assert np.max(np.abs(y - ref)) < 1e-13 * max(1.0, np.max(np.abs(ref)))


def test_srht_d2_explicit():
    x = np.array([3.0, 1.0], dtype=np.float16).reshape(1, 1, 1, 2)
    y = oracle.rotate(x, None, "srht")[0, 0, 0]
    assert np.allclose(y, [4.0 / np.sqrt(2), 2.0 / np.sqrt(2)], atol=1e-15)


def test_none_is_sign_only():
    rng = np.random.default_rng(5)
    x = _rand_x(rng, (1, 4, 3, 32))
    s = _rand_signs(rng, 1, 3, 32)
    y = oracle.rotate(x, s, "none")
    assert np.array_equal(y, x.astype(np.float64) * s[:, None])


# --------------------------------------------------------------------------
# Quantizer.
# --------------------------------------------------------------------------

def decode_codes(codes, bits, d):
    """Independent decoder of the documented layout: int8 bytes, or two's
    complement nibbles with the even coordinate in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    if bits == 8:
        return c.view(np.int8).astype(np.int64)
    lo = (c & 0xF).astype(np.int64)
    hi = (c >> 4).astype(np.int64)
    q = np.empty(c.shape[:-1] + (d,), dtype=np.int64)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    return np.where(q >= 8, q - 16, q)


def _groups(a, g):
    return a.reshape(a.shape[:-1] + (a.shape[-1] // g, g))


@pytest.mark.parametrize("rot", ["srft", "srht", "none"])
@pytest.mark.parametrize("bits,group", [(4, 16), (4, 32), (8, 32), (4, 8), (8, 128)])
def test_quantizer_invariants(rot, bits, group):
    d = 128
    qmax = 7 if bits == 4 else 127
    rng = np.random.default_rng(bits * 100 + group)
    x = _rand_x(rng, (2, 33, 2, d), scale=2.0)
    x[..., 3] *= 20
    s = _rand_signs(rng, 2, 2, d)
    lam = rng.uniform(0.5, 2.0, size=(2, 2, d)).astype(np.float32)
    codes, scales, z = oracle.quantize(x, s, lam, group, bits, rot, return_z=True)
    q = decode_codes(codes, bits, d)
    sig = scales.view(np.float16).astype(np.float64)
    assert np.all(np.abs(q) <= qmax)
    # z is lambda * y (the decision input), fp64
    y = oracle.rotate(x, s, rot)
    zref = lam[:, None].astype(np.float64) * y
    # codes, scales and z are head-major [B, H, T, .]; y is [B, T, H, d]
    assert np.array_equal(z, zref.transpose(0, 2, 1, 3))
    zg = _groups(z, group)
    qg = _groups(q, group)
    a = np.max(np.abs(zg), axis=-1)
    # sigma is numpy's correctly rounded fp16 of a / qmax
    assert np.array_equal(sig, (a / qmax).astype(np.float16).astype(np.float64))
    # every group reaches the end of the code range
    assert np.all(np.max(np.abs(qg), axis=-1) == qmax)
    # nearest code: |z - q sigma| <= sigma / 2
    err = np.abs(zg - qg * sig[..., None])
    assert np.all(err <= sig[..., None] * (0.5 + 2.0 ** -40))
    # brute force over every code value: the oracle's code is the nearest
    # one, and where two are equally near (an exact tie), the even one
    cand = np.arange(-qmax, qmax + 1, dtype=np.float64)
    dist = np.abs(zg[..., None] - cand * sig[..., None, None])
    dmin = np.min(dist, axis=-1, keepdims=True)
    nearest = dist == dmin                                   # one or two candidates
    n_near = nearest.sum(axis=-1)
    best = cand[np.argmax(nearest, axis=-1)]
    single = n_near == 1
    assert np.array_equal(best[single], qg[single].astype(np.float64))
    even = np.where(nearest & (cand % 2 == 0), cand, np.inf).min(axis=-1)
    assert np.array_equal(even[~single], qg[~single].astype(np.float64))


def test_quantizer_ties_round_half_even():
    d, g = 16, 16
    # rot none, lambda 1, s = +1: z = x exactly; absmax 7 gives sigma = 1
    vals = np.array([7.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 6.5, -0.5, -1.5, 4.5, 5.5, 0.0, 1.0, -7.0, -6.5])
    x = vals.astype(np.float16).reshape(1, 1, 1, d)
    codes, scales = oracle.quantize(x, None, None, g, 4, "none")
    assert scales.view(np.float16)[0, 0, 0, 0] == 1.0
    q = decode_codes(codes, 4, d)[0, 0, 0]
    expect = [7, 2, 4, -2, -4, 0, 2, 6, 0, -2, 4, 6, 0, 1, -7, -6]
    assert list(q) == expect


def test_quantizer_zero_group_and_subnormal_clamp():
    d, g = 32, 16
    x = np.zeros((1, 1, 1, d), dtype=np.float16)
    # group 1: absmax 7 * 1.4 * 2^-24 -> a/7 rounds to the smallest subnormal,
    # so a / sigma = 9.8 and the code clamps to 7
    x[..., 16] = np.float16(7 * 1.4 * 2.0 ** -24)
    codes, scales = oracle.quantize(x, None, None, g, 4, "none")
    sc = scales.view(np.float16)[0, 0, 0]
    assert sc[0] == 0.0
    q = decode_codes(codes, 4, d)[0, 0, 0]
    assert np.all(q[:16] == 0)
    xv = float(x[0, 0, 0, 16])
    assert sc[1] == np.float16(2.0 ** -24)
    assert xv / float(sc[1]) > 7.5 and q[16] == 7 and np.all(q[17:] == 0)


def test_quantizer_overflowing_scale_clamps():
    d, g = 16, 16
    x = np.zeros((1, 1, 1, d), dtype=np.float16)
    x[..., 0] = 60000.0
    x[..., 1] = -30000.0
    x[..., 2] = 1000.0
    # a / qmax = 6e7 / 127 exceeds the largest half: sigma clamps to 65504
    lam = np.full((1, 1, d), 1000.0, dtype=np.float32)
    codes, scales = oracle.quantize(x, None, lam, g, 8, "none")
    assert scales.view(np.float16)[0, 0, 0, 0] == np.float16(65504.0)
    q = decode_codes(codes, 8, d)[0, 0, 0]
    # 6e7/65504 and -3e7/65504 clamp; 1e6/65504 = 15.27 rounds to 15
    assert q[0] == 127 and q[1] == -127 and q[2] == 15


@pytest.mark.parametrize("bits", [4, 8])
def test_dequantize_rot_none_closed_form(bits):
    """rot none: x_hat = s * q * sigma / lambda, rounded once to fp16."""
    d, g = 64, 16
    rng = np.random.default_rng(bits)
    x = _rand_x(rng, (1, 20, 3, d), scale=4.0)
    s = _rand_signs(rng, 1, 3, d)
    codes, scales = oracle.quantize(x, s, None, g, bits, "none")
    out = oracle.dequantize(codes, scales, s, None, g, bits, "none", d=d)
    q = decode_codes(codes, bits, d).astype(np.float64)                 # [B, H, T, d]
    sig = np.repeat(scales.view(np.float16).astype(np.float64), g, axis=-1)
    ref = (s[:, :, None] * q * sig).transpose(0, 2, 1, 3)               # -> [B, T, H, d]
    assert np.array_equal(out, ref.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("rot", ["srft", "srht"])
def test_roundtrip_error_identity_and_bound(rot):
    """Orthogonality: ||x_hat - x|| = ||y_hat - y|| before fp16 output rounding,
    and the per-vector error is bounded by half a quantization step."""
    d, g, bits = 128, 16, 4
    rng = np.random.default_rng(17)
    x = _rand_x(rng, (1, 40, 2, d))
    s = _rand_signs(rng, 1, 2, d)
    lam = rng.uniform(0.5, 2.0, size=(1, 2, d)).astype(np.float32)
    codes, scales = oracle.quantize(x, s, lam, g, bits, rot)
    _, x64 = oracle.dequantize(codes, scales, s, lam, g, bits, rot, d=d, return_f64=True)
    q = decode_codes(codes, bits, d).astype(np.float64)
    sig = np.repeat(scales.view(np.float16).astype(np.float64), g, axis=-1)
    yhat = (q * sig / lam[:, :, None]).transpose(0, 2, 1, 3)           # [B, T, H, d]
    sig = sig.transpose(0, 2, 1, 3)
    y = oracle.rotate(x, s, rot)
    e_x = np.linalg.norm(x64 - x.astype(np.float64), axis=-1)
    e_y = np.linalg.norm(yhat - y, axis=-1)
    assert np.allclose(e_x, e_y, rtol=1e-9, atol=1e-12)
    bound = np.sqrt(np.sum((sig / (2 * lam[:, None])) ** 2, axis=-1))
    assert np.all(e_x <= bound * (1 + 1e-5))


def test_calibrated_lambda_gives_unit_rms():
    d = 64
    rng = np.random.default_rng(23)
    x = _rand_x(rng, (2, 50, 2, d)) * np.float16(3.0)
    x[0, :, 1, :] = 0                       # a silent head: lambda stays 1
    s = _rand_signs(rng, 2, 2, d)
    for rot in ("srft", "srht"):
        lam = oracle.calibrate_lambda(x, s, rot)
        y = oracle.rotate(x, s, rot)
        rms = np.sqrt(np.mean((lam[:, None].astype(np.float64) * y) ** 2, axis=1))
        live = np.ones((2, 2), dtype=bool)
        live[0, 1] = False
        assert np.allclose(rms[live], 1.0, rtol=1e-6)
        assert np.all(lam[0, 1] == 1.0)


def test_pages_quality_claims_on_synthetic_outliers():
    """The pages' two qualitative claims, on outlier-channel data: per-group
    scaling beats per-token scaling, and SRFT and SRHT are on a par."""
    d = 128
    rng = np.random.default_rng(31)
    x = rng.standard_normal((1, 256, 4, d))
    for h in range(4):
        x[0, :, h, rng.choice(d, 4, replace=False)] *= 20
    x = _f16(x)
    s = _rand_signs(rng, 1, 4, d)

    def err(rot, g):
        c, sc = oracle.quantize(x, s, None, g, 4, rot)
        xh = oracle.dequantize(c, sc, s, None, g, 4, rot, d=d).view(np.float16)
        xf = x.astype(np.float64)
        return np.linalg.norm(xh.astype(np.float64) - xf) / np.linalg.norm(xf)

    e16, etok, enone = err("srft", 16), err("srft", d), err("none", d)
    assert e16 < etok < enone
    assert abs(err("srht", 16) - e16) / e16 < 0.1


def test_byte_accounting_reproduces_pages_figures():
    """The packed format (bits per code + one fp16 scale per group) reproduces
    the compression figures the pages print: 3.56x and 41 GB -> 10.9 GB."""
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "compression_figures.json")))
    d = 128
    x = np.ones((1, 4, 1, d), dtype=np.float16)

    def ratio(g):
        codes, scales = oracle.quantize(x, None, None, g, 4, "none")
        return x.nbytes / (codes.nbytes + scales.nbytes)

    assert round(ratio(32), 2) == gold["compression_upper"]
    assert round(gold["llama3_70b_128k_fp16_GB"] / ratio(64), 1) == gold["llama3_70b_128k_int4_GB"]


def test_ties_follow_the_quotient_not_a_reciprocal():
    """At an exact tie with a scale that is not a power of two, rne(z / sigma)
    and rne(z * fp32(1 / sigma)) differ: the oracle gives the quotient's
    answer (round half to even), the definition in the pages' pipeline order
    (rescale, group absmax, rounding)."""
    d, g = 16, 16
    for bits, qmax in ((4, 7), (8, 127)):
        # rot none, lambda 1, s = +1: z = x exactly; absmax 3 * qmax -> sigma = 3
        vals = [3.0 * qmax, 7.5, -7.5, 10.5, 4.5, 1.5, -1.5, 16.5, -10.5, 0.0, 3.0, -3.0, 6.0, 9.0, 12.0, 4.0]
        x = np.array(vals, dtype=np.float16).reshape(1, 1, 1, d)
        assert np.array_equal(x.astype(np.float64).ravel(), np.array(vals))
        codes, scales = oracle.quantize(x, None, None, g, bits, "none")
        assert scales.view(np.float16)[0, 0, 0, 0] == 3.0
        q = decode_codes(codes, bits, d)[0, 0, 0]
        quotient = [qmax, 2, -2, 4, 2, 0, 0, 6, -4, 0, 1, -1, 2, 3, 4, 1]   # 4/3 -> 1
        assert list(q) == quotient
        # the reciprocal rule rounds the four ties 2.5, -2.5, 0.5 and -0.5 the other way
        r = np.float64(np.float32(1.0 / 3.0))
        recip = np.clip(np.rint(np.array(vals) * r), -qmax, qmax).astype(int)
        differ = np.nonzero(recip != np.array(quotient))[0]
        assert list(differ) == [1, 2, 5, 6]
        assert np.all(np.abs(recip[differ] - np.array(quotient)[differ]) == 1)


def test_fp32_reciprocal_of_every_fp16_is_correctly_rounded():
    """A fact about fp16 values that a fast decision rule can rely on: for
    every positive finite fp16 sigma, one rounding of the double quotient
    1/sigma to fp32 is the correctly rounded fp32 reciprocal, and 1/sigma is
    never an fp32 rounding tie (exact rational arithmetic)."""
    from fractions import Fraction
    sig = np.arange(1, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)
    r = (1.0 / sig).astype(np.float32)
    up = np.nextafter(r, np.float32(np.inf))
    dn = np.nextafter(r, np.float32(0))
    for s_, r_, u_, d_ in zip(sig.tolist(), r.astype(np.float64).tolist(),
                              up.astype(np.float64).tolist(), dn.astype(np.float64).tolist()):
        exact = 1 / Fraction(s_)
        e = abs(Fraction(r_) - exact)
        assert e <= abs(Fraction(u_) - exact) and e <= abs(Fraction(d_) - exact)
        assert e != abs(Fraction(u_) - exact) and e != abs(Fraction(d_) - exact)   # never a tie


def test_fp32_newton_reciprocal_of_every_fp16_is_correctly_rounded():
    """The kernels' reciprocal of an fp16 scale (quant.h recip_f16_value):
    r0 within a few ulps of 1/sigma (the hardware estimate), e = fl(1 -
    sigma r0) by one FMA, r = fl(r0 + r0 e) by another.  In exact rational
    arithmetic, for every positive finite fp16 sigma and every r0 up to two
    fp32 ulps off the correctly rounded reciprocal: e is exact, and r is the
    correctly rounded fp32 reciprocal."""
    from fractions import Fraction

    def rn32(q):
        # round a positive rational to the nearest fp32 (ties to even)
        f = np.float32(float(q))   # float() rounds once to fp64: adjust to exact nearest below
        cands = [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))]
        best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                         int(np.array(c, np.float32).view(np.uint32)) & 1))
        return best

    sig = np.arange(1, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)
    for s_ in sig.tolist():
        S_ = Fraction(s_)
        r = np.float32(1.0 / s_)
        want = Fraction(float(r))
        offs = [r]
        for _ in range(2):
            offs = [np.nextafter(offs[0], np.float32(0))] + offs + [np.nextafter(offs[-1], np.float32(np.inf))]
        for r0 in offs:
            R0 = Fraction(float(r0))
            e_exact = 1 - S_ * R0
            e = rn32(abs(e_exact)) if e_exact != 0 else np.float32(0)
            e = Fraction(float(e)) * (1 if e_exact >= 0 else -1)
            assert e == e_exact                     # the FMA's 1 - sigma r0 is exact
            got = rn32(R0 + R0 * e)
            assert Fraction(float(got)) == want, (s_, float(r0))


# --------------------------------------------------------------------------
# The growing cache: appending places per-vector results, nothing else.
# --------------------------------------------------------------------------

def _sentinel_cache(B, H, cap, d, g, bits):
    return (np.full((B, H, cap, d * bits // 8), 0xA5, dtype=np.uint8),
            np.full((B, H, cap, d // g), 0x5A5A, dtype=np.uint16))


def test_cache_grown_step_by_step_equals_one_quantize():
    """The quantizer acts on each vector alone, so a cache filled one decode
    step at a time (or in chunks of any length) holds exactly the codes of
    quantizing the whole sequence at once; rows never appended keep their
    contents, and reading the prefix is dequantizing those codes."""
    B, T, H, d, g, bits, cap = 3, 9, 2, 64, 32, 8, 12
    rng = np.random.default_rng(41)
    x = _rand_x(rng, (B, T, H, d))
    s = _rand_signs(rng, B, H, d)
    lam = rng.uniform(0.5, 2.0, size=(B, H, d)).astype(np.float32)
    whole_c, whole_s = oracle.quantize(x, s, lam, g, bits, "srft")

    cc, cs = _sentinel_cache(B, H, cap, d, g, bits)
    for t in range(T):
        oracle.cache_append(cc, cs, x[:, t:t + 1], np.full(B, t, np.int32), s, lam, g, bits, "srft")
    assert np.array_equal(cc[:, :, :T], whole_c) and np.array_equal(cs[:, :, :T], whole_s)
    assert np.all(cc[:, :, T:] == 0xA5) and np.all(cs[:, :, T:] == 0x5A5A)

    cc2, cs2 = _sentinel_cache(B, H, cap, d, g, bits)
    for a, b in ((0, 4), (4, 5), (5, 9)):
        oracle.cache_append(cc2, cs2, x[:, a:b], np.full(B, a, np.int32), s, lam, g, bits, "srft")
    assert np.array_equal(cc2, cc) and np.array_equal(cs2, cs)

    got = oracle.cache_read(cc, cs, T, s, lam, g, bits, "srft", d=d)
    assert np.array_equal(got, oracle.dequantize(whole_c, whole_s, s, lam, g, bits, "srft", d=d))


def test_cache_append_ragged_positions_and_dropped_rows():
    """Tensor b's token t lands in row pos[b] + t; a row before 0 or past
    the capacity is dropped.  The expected placement is written out by hand."""
    B, n, H, d, g, bits, cap = 4, 3, 2, 64, 16, 4, 6
    rng = np.random.default_rng(43)
    x = _rand_x(rng, (B, n, H, d))
    s = _rand_signs(rng, B, H, d)
    pos = np.array([0, 2, 5, -1], dtype=np.int32)
    qc, qs = oracle.quantize(x, s, None, g, bits, "srht")          # [B, H, n, .]
    cc, cs = _sentinel_cache(B, H, cap, d, g, bits)
    oracle.cache_append(cc, cs, x, pos, s, None, g, bits, "srht")
    ec, es = _sentinel_cache(B, H, cap, d, g, bits)
    placed = {(0, 0): 0, (0, 1): 1, (0, 2): 2,      # (tensor, token) -> row
              (1, 0): 2, (1, 1): 3, (1, 2): 4,
              (2, 0): 5,                            # tokens 1, 2 fall past row 5
              (3, 1): 0, (3, 2): 1}                 # token 0 falls before row 0
    for (b, t), r in placed.items():
        ec[b, :, r] = qc[b, :, t]
        es[b, :, r] = qs[b, :, t]
    assert np.array_equal(cc, ec) and np.array_equal(cs, es)


# --------------------------------------------------------------------------
# Decode attention over the quantized cache.
# --------------------------------------------------------------------------

def _attn_case(seed, B, T, H, R, d, g, bits, rot, lam=True):
    rng = np.random.default_rng(seed)
    k = _rand_x(rng, (B, T, H, d))
    v = _rand_x(rng, (B, T, H, d), 2.0)
    sk, sv = _rand_signs(rng, B, H, d), _rand_signs(rng, B, H, d)
    lk = rng.uniform(0.5, 2.0, size=(B, H, d)).astype(np.float32) if lam else None
    lv = rng.uniform(0.5, 2.0, size=(B, H, d)).astype(np.float32) if lam else None
    kc, ks = oracle.quantize(k, sk, lk, g, bits, rot)
    vc, vs = oracle.quantize(v, sv, lv, g, bits, rot)
    q = _rand_x(rng, (B, H * R, d))
    return q, (kc, ks, sk, lk), (vc, vs, sv, lv)


def _attn(q, K, V, g, bits, rot, **kw):
    return oracle.decode_attention(q, K[0], K[1], V[0], V[1], signs_k=K[2], lam_k=K[3], signs_v=V[2],
                                   lam_v=V[3], group=g, bits=bits, rot=rot, **kw)


@pytest.mark.parametrize("d,g", [(64, 16), (96, 32)])
def test_attention_matches_torch_sdpa(d, g):
    """Against torch's scaled_dot_product_attention (fp64, CPU) on the
    oracle's own reconstructions, with grouped query heads and a length mask
    (d = 96: the SRFT with its radix-3 step)."""
    import torch
    B, T, H, R, bits = 2, 37, 2, 3, 4
    q, K, V = _attn_case(61 + d, B, T, H, R, d, g, bits, "srft")
    lengths = np.array([37, 20], dtype=np.int32)
    got = _attn(q, K, V, g, bits, "srft", lengths=lengths)
    _, kh = oracle.dequantize(K[0], K[1], K[2], K[3], g, bits, "srft", d=d, return_f64=True)
    _, vh = oracle.dequantize(V[0], V[1], V[2], V[3], g, bits, "srft", d=d, return_f64=True)
    kt = torch.from_numpy(kh).permute(0, 2, 1, 3).repeat_interleave(R, dim=1)    # [B, H*R, T, d]
    vt = torch.from_numpy(vh).permute(0, 2, 1, 3).repeat_interleave(R, dim=1)
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None]                    # [B, H*R, 1, d]
    mask = torch.from_numpy(np.arange(T)[None, :] < lengths[:, None])[:, None, None]   # [B, 1, 1, T]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)[:, :, 0]
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    """One token returns its value; equal keys average the values; no tokens
    give zeros; rows past the length do not matter."""
    B, T, H, R, d, g, bits = 1, 24, 1, 2, 64, 32, 8
    q, K, V = _attn_case(62, B, T, H, R, d, g, bits, "srht")
    _, vh = oracle.dequantize(V[0], V[1], V[2], V[3], g, bits, "srht", d=d, return_f64=True)
    one = _attn(q, K, V, g, bits, "srht", lengths=np.array([1], np.int32))
    assert np.allclose(one, vh[0, 0, 0][None, None], rtol=1e-13, atol=1e-13)
    Ke = (np.repeat(K[0][:, :, :1], T, axis=2), np.repeat(K[1][:, :, :1], T, axis=2), K[2], K[3])
    avg = _attn(q, Ke, V, g, bits, "srht", lengths=np.array([10], np.int32))
    assert np.allclose(avg, vh[0, :10, 0].mean(axis=0)[None, None], rtol=1e-12, atol=1e-12)
    zero = _attn(q, K, V, g, bits, "srht", lengths=np.array([0], np.int32))
    assert np.all(zero == 0)
    K2 = (K[0].copy(), K[1].copy(), K[2], K[3])
    K2[0][:, :, 12:] ^= 0x5A
    a = _attn(q, K, V, g, bits, "srht", lengths=np.array([12], np.int32))
    b = _attn(q, K2, V, g, bits, "srht", lengths=np.array([12], np.int32))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("d", [128, 96])
def test_attention_scores_in_the_rotated_domain(d):
    """The identity the GPU path relies on: q . k^ = (M (s_k . q)) . y^ with
    y^_j = c_j sigma_G / lambda_j, since M is orthonormal."""
    from oracle.compare import decode_codes
    B, T, H, R, g, bits = 1, 9, 1, 1, 16, 4
    q, K, _ = _attn_case(63 + d, B, T, H, R, d, g, bits, "srft")
    _, kh = oracle.dequantize(K[0], K[1], K[2], K[3], g, bits, "srft", d=d, return_f64=True)
    direct = kh[0, :, 0] @ q[0, 0].astype(np.float64)
    u = oracle.rotate(q[:, None], K[2], "srft")[0, 0, 0]                       # M (s . q)
    c = decode_codes(K[0], bits, d)[0, 0].astype(np.float64)                   # [T, d]
    sig = np.repeat(K[1].view(np.float16).astype(np.float64)[0, 0], g, axis=-1)
    yh = c * sig / K[3][0, 0].astype(np.float64)
    assert np.allclose(yh @ u, direct, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Rotations given as matrices: learned and Householder rotations ("When
# Quantization Is Free", Metodologia 3: a learnable rotation R with lambda,
# and Householder rotations with k = d/2 reflectors at d = 256).
# --------------------------------------------------------------------------

def _srft_matrix(d):
    """Columns M e_i from the oracle's FFT-based rotation of the basis."""
    return oracle.rotate(np.eye(d, dtype=np.float16).reshape(d, 1, d), None, "srft")[:, 0, :].T


def test_householder_single_reflector_invariants():
    """k = 1: H v = -v, H w = w for w orthogonal to v, H symmetric and H^2 = I."""
    rng = np.random.default_rng(40)
    d = 64
    v = rng.standard_normal(d)
    H = oracle.householder_matrix(v[None])
    assert np.allclose(H @ v, -v, atol=1e-13)
    w = rng.standard_normal(d)
    w -= (w @ v) / (v @ v) * v
    assert np.allclose(H @ w, w, atol=1e-13)
    assert np.allclose(H, H.T, atol=1e-15)
    assert np.allclose(H @ H, np.eye(d), atol=1e-13)


def test_householder_product_matches_lapack_qr():
    """LAPACK's QR stores Q as H_1 H_2 ... H_n with H_i = I - tau_i v_i v_i^T,
    v_i = (0 .. 0, 1, below-diagonal of column i); for real reflections
    tau_i = 2 / (v_i . v_i).  Rebuilding Q from those vectors must give
    numpy's Q (an independent library routine)."""
    rng = np.random.default_rng(41)
    n = 48
    A = rng.standard_normal((n, n))
    Qref = np.linalg.qr(A)[0]
    h, tau = np.linalg.qr(A, mode="raw")
    F = h.T                                     # LAPACK's column-major factor
    V = np.zeros((n, n))
    for i in range(n):
        V[i, i] = 1.0
        V[i, i + 1:] = F[i + 1:, i]
        if tau[i] != 0.0:
            assert np.isclose(tau[i], 2.0 / (V[i] @ V[i]), rtol=1e-12)
        else:
            V[i] = 0.0
    assert np.allclose(oracle.householder_matrix(V), Qref, atol=1e-12)


@pytest.mark.parametrize("k", [128, 127])
def test_householder_rotation_orthogonal_d256(k):
    """k reflectors at d = 256: Q^T Q = I and det Q = (-1)^k; zero rows are
    the identity."""
    rng = np.random.default_rng(42 + k)
    V = rng.standard_normal((k, 256))
    Q = oracle.householder_matrix(V)
    assert np.abs(Q.T @ Q - np.eye(256)).max() < 1e-12
    sign, _ = np.linalg.slogdet(Q)
    assert sign == (-1) ** k
    V2 = np.concatenate([V[:5], np.zeros((3, 256)), V[5:]])
    assert np.allclose(oracle.householder_matrix(V2), Q, atol=1e-14)


@pytest.mark.parametrize("bits,group", [(4, 16), (8, 32)])
def test_dense_special_cases_reduce_to_the_transforms(bits, group):
    """Q = I is rot none; Q = the packed SRFT matrix is rot srft; Q = H_d /
    sqrt(d) from scipy is rot srht (quantize bit-exact, dequantize to fp64
    rounding)."""
    d = 64
    rng = np.random.default_rng(43)
    x = _rand_x(rng, (2, 30, 3, d))
    s = _rand_signs(rng, 2, 3, d)
    lam = rng.uniform(0.5, 2.0, size=(2, 3, d)).astype(np.float32)
    mats = {"none": np.eye(d), "srft": _srft_matrix(d),
            "srht": scipy.linalg.hadamard(d).astype(np.float64) / math.sqrt(d)}
    for rot, M in mats.items():
        c0, s0 = oracle.quantize(x, s, lam, group, bits, rot)
        c1, s1 = oracle.quantize_dense(x, M.astype(np.float32), s, lam, group, bits)
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1), rot
        _, a = oracle.dequantize(c0, s0, s, lam, group, bits, rot, d=d, return_f64=True)
        _, b = oracle.dequantize_dense(c0, s0, M.astype(np.float32), s, lam, group, bits, d=d,
                                       return_f64=True)
        assert np.allclose(a, b, rtol=1e-6, atol=1e-6 * np.abs(a).max()), rot


def test_dense_per_head_matrices_index_by_tensor_and_head():
    """Q [B, H, d, d]: each head uses its own matrix (checked head by head
    against single-matrix calls)."""
    d, B, H, T = 64, 2, 3, 17
    rng = np.random.default_rng(44)
    x = _rand_x(rng, (B, T, H, d))
    Q = oracle.householder_matrix(rng.standard_normal((B, H, d // 2, d))).astype(np.float32)
    codes, scales = oracle.quantize_dense(x, Q, None, None, 16, 4)
    xr = oracle.dequantize_dense(codes, scales, Q, None, None, 16, 4)
    for b in range(B):
        for h in range(H):
            c1, s1 = oracle.quantize_dense(x[b:b + 1, :, h:h + 1], Q[b, h], None, None, 16, 4)
            assert np.array_equal(c1[0, 0], codes[b, h]) and np.array_equal(s1[0, 0], scales[b, h])
            x1 = oracle.dequantize_dense(c1, s1, Q[b, h], None, None, 16, 4)
            assert np.array_equal(x1[0, :, 0], xr[b, :, h])


def test_dense_roundtrip_error_identity_and_bound():
    """A Householder rotation (not symmetric, so a transposed operand shows):
    ||x_hat - x|| = ||y_hat - y|| (orthogonality of Q), within half a
    quantization step per coordinate."""
    d, g, bits = 128, 16, 4
    rng = np.random.default_rng(45)
    x = _rand_x(rng, (1, 40, 2, d))
    s = _rand_signs(rng, 1, 2, d)
    lam = rng.uniform(0.5, 2.0, size=(1, 2, d)).astype(np.float32)
    Q = oracle.householder_matrix(rng.standard_normal((d // 2, d))).astype(np.float32)
    assert np.abs(Q - Q.T).max() > 0.1
    codes, scales = oracle.quantize_dense(x, Q, s, lam, g, bits)
    _, x64 = oracle.dequantize_dense(codes, scales, Q, s, lam, g, bits, d=d, return_f64=True)
    from oracle.compare import decode_codes
    q = decode_codes(codes, bits, d).astype(np.float64)
    sig = np.repeat(scales.view(np.float16).astype(np.float64), g, axis=-1)
    yhat = (q * sig / lam[:, :, None]).transpose(0, 2, 1, 3)
    sig = sig.transpose(0, 2, 1, 3)
    y = np.einsum("ij,bthj->bthi", Q.astype(np.float64), s[:, None] * x.astype(np.float64))
    e_x = np.linalg.norm(x64 - x.astype(np.float64), axis=-1)
    e_y = np.linalg.norm(yhat - y, axis=-1)
    # fp32 rounding of Q makes it orthogonal to ~1e-7 only
    assert np.allclose(e_x, e_y, rtol=1e-5, atol=1e-5)
    bound = np.sqrt(np.sum((sig / (2 * lam[:, None])) ** 2, axis=-1))
    assert np.all(e_x <= bound * (1 + 1e-4) + 1e-5)


# --------------------------------------------------------------------------
# Decode attention over caches written with a rotation matrix.
# --------------------------------------------------------------------------

def _attn_case_dense(seed, B, T, H, R, d, g, bits, Q, lam=True):
    rng = np.random.default_rng(seed)
    k = _rand_x(rng, (B, T, H, d))
    v = _rand_x(rng, (B, T, H, d), 2.0)
    sk, sv = _rand_signs(rng, B, H, d), _rand_signs(rng, B, H, d)
    lk = rng.uniform(0.5, 2.0, size=(B, H, d)).astype(np.float32) if lam else None
    lv = rng.uniform(0.5, 2.0, size=(B, H, d)).astype(np.float32) if lam else None
    kc, ks = oracle.quantize_dense(k, Q, sk, lk, g, bits)
    vc, vs = oracle.quantize_dense(v, Q, sv, lv, g, bits)
    q = _rand_x(rng, (B, H * R, d))
    return q, (kc, ks, sk, lk), (vc, vs, sv, lv)


@pytest.mark.parametrize("which", ["srft", "none"])
def test_attention_dense_reduces_to_the_transforms(which):
    """With Q the packed SRFT matrix (or the identity) the caches, and so the
    attention, are those of rot = srft (none): the dense path adds nothing
    but the matrix."""
    B, T, H, R, d, g, bits = 2, 29, 2, 3, 64, 16, 4
    Q = (_srft_matrix(d) if which == "srft" else np.eye(d)).astype(np.float32)
    q, K, V = _attn_case(64, B, T, H, R, d, g, bits, which)
    lengths = np.array([29, 11], dtype=np.int32)
    ref = _attn(q, K, V, g, bits, which, lengths=lengths)
    got = oracle.decode_attention_dense(q, K[0], K[1], V[0], V[1], Q, Q, lengths=lengths, signs_k=K[2],
                                        lam_k=K[3], signs_v=V[2], lam_v=V[3], group=g, bits=bits)
    # the SRFT matrix is the FFT's output rounded to fp32 (2^-24 relative per entry)
    tol = 1e-6 if which == "srft" else 1e-13
    assert np.allclose(got, ref, rtol=tol, atol=tol)


def test_attention_dense_matches_torch_sdpa():
    """Per-head Householder rotations for K and different ones for V, against
    torch's scaled_dot_product_attention (fp64, CPU) on the dense
    reconstructions, grouped query heads and a length mask."""
    import torch
    B, T, H, R, d, g, bits = 2, 31, 2, 2, 64, 32, 8
    rng = np.random.default_rng(65)
    Qk = oracle.householder_matrix(rng.standard_normal((B, H, d // 2, d))).astype(np.float32)
    Qv = oracle.householder_matrix(rng.standard_normal((B, H, d // 2, d))).astype(np.float32)
    q, K, _ = _attn_case_dense(66, B, T, H, R, d, g, bits, Qk)
    _, _, V = _attn_case_dense(67, B, T, H, R, d, g, bits, Qv)
    lengths = np.array([31, 7], dtype=np.int32)
    got = oracle.decode_attention_dense(q, K[0], K[1], V[0], V[1], Qk, Qv, lengths=lengths, signs_k=K[2],
                                        lam_k=K[3], signs_v=V[2], lam_v=V[3], group=g, bits=bits)
    _, kh = oracle.dequantize_dense(K[0], K[1], Qk, K[2], K[3], g, bits, d=d, return_f64=True)
    _, vh = oracle.dequantize_dense(V[0], V[1], Qv, V[2], V[3], g, bits, d=d, return_f64=True)
    kt = torch.from_numpy(kh).permute(0, 2, 1, 3).repeat_interleave(R, dim=1)
    vt = torch.from_numpy(vh).permute(0, 2, 1, 3).repeat_interleave(R, dim=1)
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None]
    mask = torch.from_numpy(np.arange(T)[None, :] < lengths[:, None])[:, None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)[:, :, 0]
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_dense_scores_in_the_rotated_domain():
    """q . k^ = (Q (s_k . q)) . y^ for an orthonormal Q: the identity that lets
    the GPU score the codes directly under a Householder rotation."""
    from oracle.compare import decode_codes
    B, T, H, R, d, g, bits = 1, 9, 1, 1, 128, 16, 4
    rng = np.random.default_rng(68)
    Q = oracle.householder_matrix(rng.standard_normal((d // 2, d))).astype(np.float32)
    q, K, _ = _attn_case_dense(69, B, T, H, R, d, g, bits, Q)
    _, kh = oracle.dequantize_dense(K[0], K[1], Q, K[2], K[3], g, bits, d=d, return_f64=True)
    direct = kh[0, :, 0] @ q[0, 0].astype(np.float64)
    xs = q[0, 0].astype(np.float64) * K[2][0, 0]
    u = Q.astype(np.float64) @ xs
    c = decode_codes(K[0], bits, d)[0, 0].astype(np.float64)
    sig = np.repeat(K[1].view(np.float16).astype(np.float64)[0, 0], g, axis=-1)
    yh = c * sig / K[3][0, 0].astype(np.float64)
    assert np.allclose(yh @ u, direct, rtol=1e-12, atol=1e-12)
