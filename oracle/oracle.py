"""Python face of the CPU oracle (``srftq_oracle.c``), via ctypes and numpy.

TEST INFRASTRUCTURE ONLY: imported by the test-suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library.  The oracle is a
plain fp64 implementation of the definition of the sign-randomized Fourier
(or Walsh-Hadamard) rotation followed by per-channel lambda scaling,
per-group absmax scaling and symmetric int4/int8 rounding, as described in
"When Quantization Is Free" (gist.science technical summary, "Metodologia"
sections 1-3).  Each C function documents the reading it takes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "srftq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ROT = {"srft": 0, "srht": 1, "none": 2}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.oracle_rotate.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp]
        L.oracle_unrotate.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp]
        L.oracle_quantize.argtypes = [i64, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_dequantize.argtypes = [i64, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_quantize_dense.argtypes = [i64, i64, i32, i32, i32, i32, vp, i64, vp, vp, vp, vp, vp, vp]
        L.oracle_dequantize_dense.argtypes = [i64, i64, i32, i32, i32, i32, vp, i64, vp, vp, vp, vp, vp, vp]
        L.oracle_calibrate_lambda.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp]
        L.oracle_f16_array_to_f64.argtypes = [vp, vp, i64]
        L.oracle_f64_array_to_f16.argtypes = [vp, vp, i64]
        L.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_f16.restype = ctypes.c_uint16
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = None
        for f in ("oracle_rotate", "oracle_unrotate", "oracle_quantize",
                  "oracle_dequantize", "oracle_quantize_dense", "oracle_dequantize_dense",
                  "oracle_calibrate_lambda", "oracle_num_threads"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as4(x, d=None):
    """Accept [T,H,d] or [B,T,H,d]; return the 4-D view and B, T, H, d."""
    if x.ndim == 3:
        x = x[None]
    assert x.ndim == 4
    B, T, H, dd = x.shape
    return x, B, T, H, dd


def _bits(x16: np.ndarray) -> np.ndarray:
    """fp16 array (or uint16 bit array) as contiguous uint16 bits."""
    if x16.dtype == np.float16:
        return np.ascontiguousarray(x16).view(np.uint16)
    assert x16.dtype == np.uint16
    return np.ascontiguousarray(x16)


def _signs(signs, B, H, d):
    if signs is None:
        return None
    s = np.ascontiguousarray(np.asarray(signs, dtype=np.int8)).reshape(B, H, d)
    return s


def _lam(lam, B, H, d):
    if lam is None:
        return None
    return np.ascontiguousarray(np.asarray(lam, dtype=np.float32)).reshape(B, H, d)


def _check(st, what):
    if st != 0:
        raise ValueError(f"{what}: oracle status {st}")


def rotate(x16, signs=None, rot="srft") -> np.ndarray:
    """fp64 rotated coordinates y = M (s . x), same shape as x."""
    x, B, T, H, d = _as4(_bits(x16))
    s = _signs(signs, B, H, d)
    y = np.empty((B, T, H, d), dtype=np.float64)
    _check(lib().oracle_rotate(B, T, H, d, ROT[rot], _ptr(x), _ptr(s), _ptr(y)), "rotate")
    return y.reshape(x16.shape)


def unrotate(y, signs=None, rot="srft") -> np.ndarray:
    """fp64 x = s . (M^T y), same shape as y."""
    y4, B, T, H, d = _as4(np.ascontiguousarray(y, dtype=np.float64))
    s = _signs(signs, B, H, d)
    out = np.empty((B, T, H, d), dtype=np.float64)
    _check(lib().oracle_unrotate(B, T, H, d, ROT[rot], _ptr(y4), _ptr(s), _ptr(out)), "unrotate")
    return out.reshape(np.shape(y))


def quantize(x16, signs=None, lam=None, group=16, bits=4, rot="srft", return_z=False):
    """Return (codes uint8, scales fp16-bits uint16[, z fp64]) in the
    head-major cache layout: [B, H, T, .] for x [B, T, H, d] ([H, T, .] for
    3-D x [T, H, d]).  z = lambda * y is the value each code was decided on:
    sigma = fp16(min(max_G |z| / qmax, 65504)), q = clamp(rne(z / sigma))."""
    x, B, T, H, d = _as4(_bits(x16))
    s = _signs(signs, B, H, d)
    l = _lam(lam, B, H, d)
    codes = np.empty((B, H, T, d * bits // 8), dtype=np.uint8)
    scales = np.empty((B, H, T, d // group), dtype=np.uint16)
    z = np.empty((B, H, T, d), dtype=np.float64) if return_z else None
    _check(lib().oracle_quantize(B, T, H, d, group, bits, ROT[rot], _ptr(x), _ptr(s), _ptr(l),
                                 _ptr(codes), _ptr(scales), _ptr(z)), "quantize")
    out = (codes, scales) + ((z,) if return_z else ())
    if x16.ndim == 3:
        out = tuple(a[0] for a in out)
    return out


def dequantize(codes, scales, signs=None, lam=None, group=16, bits=4, rot="srft", d=None,
               return_f64=False):
    """codes [B, H, T, .] (or [H, T, .]) -> fp16 bits (uint16) of the
    reconstruction [B, T, H, d] (or [T, H, d]), and its fp64 values."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    if d is None:
        d = codes.shape[-1] * 8 // bits
    c4 = codes if codes.ndim == 4 else codes[None]
    B, H, T = c4.shape[:3]
    s = _signs(signs, B, H, d)
    l = _lam(lam, B, H, d)
    x = np.empty((B, T, H, d), dtype=np.uint16)
    x64 = np.empty((B, T, H, d), dtype=np.float64) if return_f64 else None
    _check(lib().oracle_dequantize(B, T, H, d, group, bits, ROT[rot], _ptr(c4),
                                   _ptr(scales), _ptr(s), _ptr(l), _ptr(x), _ptr(x64)),
           "dequantize")
    if codes.ndim == 3:
        x = x[0]
        x64 = None if x64 is None else x64[0]
    return (x, x64) if return_f64 else x


def householder_matrix(V) -> np.ndarray:
    """Product of Householder reflections, fp64: Q = H_1 H_2 ... H_k with
    H_i = I - 2 v_i v_i^T / (v_i^T v_i) for the rows v_i of V [..., k, d]
    (a zero row is the identity).  The Householder rotations of "When
    Quantization Is Free" (Metodologia 3, Householder rotations: k = d/2
    reflectors at d = 256) parametrize an orthogonal d x d matrix this way.
    Returns [..., d, d]."""
    V = np.asarray(V, dtype=np.float64)
    lead, (k, d) = V.shape[:-2], V.shape[-2:]
    Vs = V.reshape(-1, k, d)
    out = np.empty((Vs.shape[0], d, d), dtype=np.float64)
    for m in range(Vs.shape[0]):
        Q = np.eye(d)
        for i in range(k):
            v = Vs[m, i]
            n2 = float(v @ v)
            if n2 == 0.0:
                continue
            # Q <- Q H_i = Q - (2 / v.v) (Q v) v^T
            Q = Q - np.outer(Q @ v, v) * (2.0 / n2)
        out[m] = Q
    return out.reshape(lead + (d, d))


def _dense_q(Q, B, H, d):
    """Q as fp32 [d, d] (one matrix, stride 0) or [B, H, d, d] (stride d*d)."""
    Q = np.ascontiguousarray(np.asarray(Q, dtype=np.float32))
    if Q.shape == (d, d):
        return Q, 0
    return Q.reshape(B, H, d, d), d * d


def quantize_dense(x16, Q, signs=None, lam=None, group=16, bits=4, return_z=False):
    """As quantize() with the rotation y = Q (s . x) for a given fp32 matrix
    Q (a learned or Householder rotation, "When Quantization Is Free",
    Metodologia 3): Q [d, d] for every head or [B, H, d, d] per head."""
    x, B, T, H, d = _as4(_bits(x16))
    s = _signs(signs, B, H, d)
    l = _lam(lam, B, H, d)
    q, qs = _dense_q(Q, B, H, d)
    codes = np.empty((B, H, T, d * bits // 8), dtype=np.uint8)
    scales = np.empty((B, H, T, d // group), dtype=np.uint16)
    z = np.empty((B, H, T, d), dtype=np.float64) if return_z else None
    _check(lib().oracle_quantize_dense(B, T, H, d, group, bits, _ptr(q), qs, _ptr(x), _ptr(s), _ptr(l),
                                       _ptr(codes), _ptr(scales), _ptr(z)), "quantize_dense")
    out = (codes, scales) + ((z,) if return_z else ())
    if x16.ndim == 3:
        out = tuple(a[0] for a in out)
    return out


def dequantize_dense(codes, scales, Q, signs=None, lam=None, group=16, bits=4, d=None,
                     return_f64=False):
    """As dequantize() with x = s . (Q^T yhat)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    if d is None:
        d = codes.shape[-1] * 8 // bits
    c4 = codes if codes.ndim == 4 else codes[None]
    B, H, T = c4.shape[:3]
    s = _signs(signs, B, H, d)
    l = _lam(lam, B, H, d)
    q, qs = _dense_q(Q, B, H, d)
    x = np.empty((B, T, H, d), dtype=np.uint16)
    x64 = np.empty((B, T, H, d), dtype=np.float64) if return_f64 else None
    _check(lib().oracle_dequantize_dense(B, T, H, d, group, bits, _ptr(q), qs, _ptr(c4), _ptr(scales),
                                         _ptr(s), _ptr(l), _ptr(x), _ptr(x64)), "dequantize_dense")
    if codes.ndim == 3:
        x = x[0]
        x64 = None if x64 is None else x64[0]
    return (x, x64) if return_f64 else x


def cache_append(codes_cache, scales_cache, x16, pos=None, signs=None, lam=None, group=16, bits=4,
                 rot="srft"):
    """Appending to a growing quantized cache (the pages run their fused
    kernel inside an int4 KV cache that grows by the new tokens of each
    step; "When Quantization Is Free", Metodologia section 2).  In place:
    x [B, n, H, d] is quantized as by ``quantize`` and token t of tensor b is
    written to row pos[b] + t of each head of codes_cache [B, H, t_cap, .]
    and scales_cache [B, H, t_cap, .]; a token whose row falls outside
    [0, t_cap) is not written, and no other row changes."""
    assert np.asarray(x16).ndim == 4
    codes, scales = quantize(x16, signs, lam, group, bits, rot)   # [B, H, n, .]
    B, H, n = codes.shape[:3]
    t_cap = codes_cache.shape[2]
    for b in range(B):
        start = 0 if pos is None else int(pos[b])
        for t in range(n):
            row = start + t
            if 0 <= row < t_cap:
                codes_cache[b, :, row] = codes[b, :, t]
                scales_cache[b, :, row] = scales[b, :, t]
    return codes_cache, scales_cache


def cache_read(codes_cache, scales_cache, T, signs=None, lam=None, group=16, bits=4, rot="srft",
               d=None):
    """The reconstruction (fp16 bits) of rows [0, T) of every head of a
    cache [B, H, t_cap, .]: ``dequantize`` of that prefix."""
    return dequantize(codes_cache[:, :, :T], scales_cache[:, :, :T], signs, lam, group, bits, rot, d=d)


def decode_attention(q16, k_codes, k_scales, v_codes, v_scales, T=None, lengths=None, signs_k=None,
                     lam_k=None, signs_v=None, lam_v=None, group=16, bits=4, rot="srft", scale=None):
    """Attention of one query token per tensor over quantized K/V caches, the
    consumer the pages' growing int4 cache is read by at every decode step
    ("When Quantization Is Free", Resultados Clave: the speed-up comes from
    reading a third of the fp16 bytes per step).  Plain definition, fp64:
      out[b, r] = sum_{t < L_b} softmax_t(scale * q[b, r] . k^[b, t, h]) v^[b, t, h]
    with h = r // R (R = query heads per KV head), L_b = lengths[b] clamped to
    [0, T] (T when lengths is None; T defaults to the caches' rows), k^ and v^
    the fp64 reconstructions of ``dequantize`` (before its fp16 rounding), and
    scale = 1/sqrt(d) by default.  A tensor with no tokens gives zeros.
    q16: fp16 [B, H*R, d]; caches [B, H, t_cap, .]."""
    q = f16_to_f64(_bits(np.asarray(q16)))
    d = q.shape[2]
    T = k_codes.shape[2] if T is None else int(T)
    _, k = dequantize(k_codes[:, :, :T], k_scales[:, :, :T], signs_k, lam_k, group, bits, rot, d=d,
                      return_f64=True)
    _, v = dequantize(v_codes[:, :, :T], v_scales[:, :, :T], signs_v, lam_v, group, bits, rot, d=d,
                      return_f64=True)                                    # [B, T, H, d]
    return _attend(q, k, v, T, lengths, scale)


def decode_attention_dense(q16, k_codes, k_scales, v_codes, v_scales, Qk, Qv, T=None, lengths=None,
                           signs_k=None, lam_k=None, signs_v=None, lam_v=None, group=16, bits=4,
                           scale=None):
    """decode_attention over caches written with a rotation given as a matrix
    (a learned or Householder rotation, "When Quantization Is Free",
    Metodologia 3): k^ and v^ are the fp64 reconstructions of
    ``dequantize_dense`` with Qk and Qv ([d, d] or [B, H, d, d])."""
    q = f16_to_f64(_bits(np.asarray(q16)))
    d = q.shape[2]
    T = k_codes.shape[2] if T is None else int(T)
    _, k = dequantize_dense(k_codes[:, :, :T], k_scales[:, :, :T], Qk, signs_k, lam_k, group, bits, d=d,
                            return_f64=True)
    _, v = dequantize_dense(v_codes[:, :, :T], v_scales[:, :, :T], Qv, signs_v, lam_v, group, bits, d=d,
                            return_f64=True)                              # [B, T, H, d]
    return _attend(q, k, v, T, lengths, scale)


def _attend(q, k, v, T, lengths, scale):
    """softmax(scale q . k) v per tensor b and query head r over the first
    L_b = clamp(lengths[b], 0, T) tokens of KV head r // R; zeros when L_b = 0."""
    B, HR, d = q.shape
    H = k.shape[2]
    R = HR // H
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((B, HR, d), dtype=np.float64)
    for b in range(B):
        L = T if lengths is None else min(max(int(lengths[b]), 0), T)
        if L == 0:
            continue
        for r in range(HR):
            h = r // R
            s = scale * (k[b, :L, h] @ q[b, r])
            p = np.exp(s - s.max())
            out[b, r] = (p / p.sum()) @ v[b, :L, h]
    return out


def calibrate_lambda(x16, signs=None, rot="srft") -> np.ndarray:
    """fp32 lambda [B,H,d] (or [H,d] for 3-D x) = 1/RMS over tokens of rotated coords."""
    x, B, T, H, d = _as4(_bits(x16))
    s = _signs(signs, B, H, d)
    lam = np.empty((B, H, d), dtype=np.float32)
    _check(lib().oracle_calibrate_lambda(B, T, H, d, ROT[rot], _ptr(x), _ptr(s), _ptr(lam)),
           "calibrate_lambda")
    return lam if x16.ndim == 4 else lam[0]


def f16_to_f64(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    lib().oracle_f16_array_to_f64(_ptr(h), _ptr(out), h.size)
    return out


def f64_to_f16(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_f64_array_to_f16(_ptr(v), _ptr(out), v.size)
    return out


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on."""
    lib().oracle_set_num_threads(int(n))
