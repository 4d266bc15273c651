"""Thin Python binding of libsrftq (include/srftq.h) over ctypes.

Argument marshalling only: every step of the quantize / dequantize path runs
in the library's HIP kernels.  Tensors are torch CUDA tensors (device memory
and the current stream come from torch); there is no CPU fallback, and a
missing library raises.

The C functions keep their names here (``srftq_quantize`` ...) and take the
same arguments, with a ``Shape`` in place of ``const srftq_shape*``.  The
convenience wrappers ``quantize`` / ``dequantize`` / ``cache_append`` /
``cache_read`` / ``decode_attention`` / ``rotate`` / ``unrotate`` /
``calibrate_lambda`` allocate outputs (and workspace) with torch.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# SRFTQ_LIBRARY: another build of the same library to load instead (the
# LDS-poison debug build, libsrftq_poison.so, in the tests)
LIB_PATH = os.environ.get("SRFTQ_LIBRARY") or os.path.join(_PKG, "libsrftq.so")

(SRFTQ_OK, SRFTQ_ERR_NULL, SRFTQ_ERR_SHAPE, SRFTQ_ERR_UNSUPPORTED, SRFTQ_ERR_ALIGN, SRFTQ_ERR_HIP,
 SRFTQ_ERR_CAPACITY) = range(7)
# size of the library's static attention scratch (srftq_decode_attention_noalloc)
ATTENTION_SCRATCH_BYTES = 16 << 20
ROT = {"srft": 0, "srht": 1, "none": 2}
VARIANT = {"default": 0, "real": 1, "paired": 2}


class SrftqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int32),
                ("d", ctypes.c_int32), ("group", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("rot", ctypes.c_int32), ("variant", ctypes.c_int32)]

    def __repr__(self):
        return (f"Shape(B={self.B}, T={self.T}, H={self.H}, d={self.d}, group={self.group}, "
                f"bits={self.bits}, rot={self.rot}, variant={self.variant})")


def make_shape(B, T, H, d, group=16, bits=4, rot="srft", variant="default") -> Shape:
    r = ROT[rot] if isinstance(rot, str) else int(rot)
    v = VARIANT[variant] if isinstance(variant, str) else int(variant)
    return Shape(int(B), int(T), int(H), int(d), int(group), int(bits), r, v)


class CacheView(ctypes.Structure):
    """srftq_cache_view: device pointers of one cache (codes, scales, signs, lambda)."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("signs", ctypes.c_void_p), ("lam", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kv_cache_quantization_srft_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        sp = ctypes.POINTER(Shape)
        vp = ctypes.c_void_p
        L.srftq_validate.argtypes = [sp]
        L.srftq_codes_bytes.argtypes = [sp]
        L.srftq_codes_bytes.restype = ctypes.c_size_t
        L.srftq_scales_count.argtypes = [sp]
        L.srftq_scales_count.restype = ctypes.c_size_t
        L.srftq_quantize.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        L.srftq_dequantize.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        L.srftq_rotate.argtypes = [sp, vp, vp, vp, vp]
        L.srftq_unrotate.argtypes = [sp, vp, vp, vp, vp]
        L.srftq_calibrate_lambda.argtypes = [sp, vp, vp, vp, vp]
        L.srftq_cache_append.argtypes = [sp, ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp]
        L.srftq_cache_read.argtypes = [sp, ctypes.c_int64, vp, vp, vp, vp, vp, vp]
        cv = ctypes.POINTER(CacheView)
        L.srftq_attention_workspace_bytes.argtypes = [sp, ctypes.c_int32]
        L.srftq_attention_workspace_bytes.restype = ctypes.c_size_t
        L.srftq_decode_attention.argtypes = [sp, ctypes.c_int64, ctypes.c_int32, vp, cv, cv, vp,
                                             ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
        L.srftq_decode_attention_noalloc.argtypes = [sp, ctypes.c_int64, ctypes.c_int32, vp, cv, cv, vp,
                                                     ctypes.c_float, vp, vp]
        L.srftq_householder_matrix.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, vp, vp, vp]
        L.srftq_quantize_dense.argtypes = [sp, vp, ctypes.c_int64, vp, vp, vp, vp, vp, vp]
        L.srftq_dequantize_dense.argtypes = [sp, vp, ctypes.c_int64, vp, vp, vp, vp, vp, vp]
        L.srftq_decode_attention_dense.argtypes = [sp, ctypes.c_int64, ctypes.c_int32, vp, vp, ctypes.c_int64,
                                                   vp, cv, cv, vp, ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
        L.srftq_status_string.argtypes = [ctypes.c_int]
        L.srftq_status_string.restype = ctypes.c_char_p
        L.srftq_version.argtypes = []
        for f in ("srftq_validate", "srftq_quantize", "srftq_dequantize", "srftq_rotate",
                  "srftq_unrotate", "srftq_calibrate_lambda", "srftq_cache_append",
                  "srftq_cache_read", "srftq_decode_attention", "srftq_decode_attention_noalloc",
                  "srftq_householder_matrix",
                  "srftq_quantize_dense", "srftq_dequantize_dense", "srftq_decode_attention_dense",
                  "srftq_version"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().srftq_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != SRFTQ_OK:
        raise SrftqError(status, where)


# ---------------------------------------------------------------------------
# The C functions, same names and arguments.
# ---------------------------------------------------------------------------

def srftq_validate(shape: Shape) -> int:
    return lib().srftq_validate(ctypes.byref(shape))


def srftq_codes_bytes(shape: Shape) -> int:
    return int(lib().srftq_codes_bytes(ctypes.byref(shape)))


def srftq_scales_count(shape: Shape) -> int:
    return int(lib().srftq_scales_count(ctypes.byref(shape)))


def srftq_version() -> int:
    return int(lib().srftq_version())


def _dp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def srftq_quantize(shape, x, signs, lam, codes, scales, stream=None) -> int:
    return lib().srftq_quantize(ctypes.byref(shape), _dp(x), _dp(signs), _dp(lam), _dp(codes),
                                _dp(scales), _stream(stream))


def srftq_dequantize(shape, codes, scales, signs, lam, x_out, stream=None) -> int:
    return lib().srftq_dequantize(ctypes.byref(shape), _dp(codes), _dp(scales), _dp(signs), _dp(lam),
                                  _dp(x_out), _stream(stream))


def srftq_cache_append(shape, t_cap, pos, x, signs, lam, codes, scales, stream=None) -> int:
    return lib().srftq_cache_append(ctypes.byref(shape), int(t_cap), _dp(pos), _dp(x), _dp(signs),
                                    _dp(lam), _dp(codes), _dp(scales), _stream(stream))


def srftq_cache_read(shape, t_cap, codes, scales, signs, lam, x_out, stream=None) -> int:
    return lib().srftq_cache_read(ctypes.byref(shape), int(t_cap), _dp(codes), _dp(scales), _dp(signs),
                                  _dp(lam), _dp(x_out), _stream(stream))


def srftq_attention_workspace_bytes(shape, q_per_kv) -> int:
    return int(lib().srftq_attention_workspace_bytes(ctypes.byref(shape), int(q_per_kv)))


def cache_view(codes, scales, signs=None, lam=None) -> CacheView:
    return CacheView(_dp(codes), _dp(scales), _dp(signs), _dp(lam))


def srftq_decode_attention(shape, t_cap, q_per_kv, q, k_view, v_view, lengths, scale, out, workspace,
                           workspace_bytes, stream=None) -> int:
    return lib().srftq_decode_attention(ctypes.byref(shape), int(t_cap), int(q_per_kv), _dp(q),
                                        None if k_view is None else ctypes.byref(k_view),
                                        None if v_view is None else ctypes.byref(v_view), _dp(lengths),
                                        float(scale), _dp(out), _dp(workspace), int(workspace_bytes),
                                        _stream(stream))


def srftq_decode_attention_noalloc(shape, t_cap, q_per_kv, q, k_view, v_view, lengths, scale, out,
                                   stream=None) -> int:
    return lib().srftq_decode_attention_noalloc(ctypes.byref(shape), int(t_cap), int(q_per_kv), _dp(q),
                                                None if k_view is None else ctypes.byref(k_view),
                                                None if v_view is None else ctypes.byref(v_view), _dp(lengths),
                                                float(scale), _dp(out), _stream(stream))


def srftq_decode_attention_dense(shape, t_cap, q_per_kv, Qk, Qv, q_stride, q, k_view, v_view, lengths, scale,
                                 out, workspace, workspace_bytes, stream=None) -> int:
    return lib().srftq_decode_attention_dense(ctypes.byref(shape), int(t_cap), int(q_per_kv), _dp(Qk), _dp(Qv),
                                              int(q_stride), _dp(q),
                                              None if k_view is None else ctypes.byref(k_view),
                                              None if v_view is None else ctypes.byref(v_view), _dp(lengths),
                                              float(scale), _dp(out), _dp(workspace), int(workspace_bytes),
                                              _stream(stream))


def srftq_householder_matrix(d, k, n, V, Q, stream=None) -> int:
    return lib().srftq_householder_matrix(int(d), int(k), int(n), _dp(V), _dp(Q), _stream(stream))


def srftq_quantize_dense(shape, Q, q_stride, x, signs, lam, codes, scales, stream=None) -> int:
    return lib().srftq_quantize_dense(ctypes.byref(shape), _dp(Q), int(q_stride), _dp(x), _dp(signs),
                                      _dp(lam), _dp(codes), _dp(scales), _stream(stream))


def srftq_dequantize_dense(shape, Q, q_stride, codes, scales, signs, lam, x_out, stream=None) -> int:
    return lib().srftq_dequantize_dense(ctypes.byref(shape), _dp(Q), int(q_stride), _dp(codes), _dp(scales),
                                        _dp(signs), _dp(lam), _dp(x_out), _stream(stream))


def srftq_rotate(shape, x, signs, y, stream=None) -> int:
    return lib().srftq_rotate(ctypes.byref(shape), _dp(x), _dp(signs), _dp(y), _stream(stream))


def srftq_unrotate(shape, y, signs, x_out, stream=None) -> int:
    return lib().srftq_unrotate(ctypes.byref(shape), _dp(y), _dp(signs), _dp(x_out), _stream(stream))


def srftq_calibrate_lambda(shape, x, signs, lam_out, stream=None) -> int:
    return lib().srftq_calibrate_lambda(ctypes.byref(shape), _dp(x), _dp(signs), _dp(lam_out),
                                        _stream(stream))


# ---------------------------------------------------------------------------
# torch conveniences.
# ---------------------------------------------------------------------------

def _dims(x):
    if x.dim() == 3:
        T, H, d = x.shape
        return 1, T, H, d
    if x.dim() == 4:
        return tuple(x.shape)
    raise ValueError("expected [T,H,d] or [B,T,H,d]")


def _req(t, dtype, name):
    import torch
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _head_rows(t, B, H, d, name, flat_ok=False, device=None):
    """signs / lambda must hold one row of d per (tensor, head): [B, H, d]
    (or [H, d] when B == 1 and flat_ok), on the data's device; the kernels
    index them as [B, H, d], so a shorter tensor would be read past its end."""
    if t is None:
        return None
    want = (B, H, d)
    ok = tuple(t.shape) == want or (flat_ok and B == 1 and tuple(t.shape) == (H, d))
    if not ok:
        raise ValueError(f"{name} must have shape {want}" + (f" or {(H, d)}" if flat_ok and B == 1 else "")
                         + f", got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the data on {device}")
    return t


def _same_device(device, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the data on {device}")


def _cache_lead(x):
    """Leading dims of the head-major cache for x [B,T,H,d] / [T,H,d]."""
    if x.dim() == 4:
        B, T, H, _ = x.shape
        return (B, H, T)
    T, H, _ = x.shape
    return (H, T)


def _out(t, shape, dtype, device, name):
    import torch
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _req(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def quantize(x, signs=None, lam=None, group=16, bits=4, rot="srft", variant="default",
             codes=None, scales=None, stream=None):
    """x fp16 [B,T,H,d] (or [T,H,d]) -> (codes uint8 [B,H,T,d*bits/8],
    scales fp16 [B,H,T,d/group]) in the head-major cache layout ([H,T,.]
    for 3-D x)."""
    import torch
    B, T, H, d = _dims(x)
    _req(x, torch.float16, "x")
    _req(signs, torch.int8, "signs")
    _req(lam, torch.float32, "lambda")
    _head_rows(signs, B, H, d, "signs", x.dim() == 3, x.device)
    _head_rows(lam, B, H, d, "lambda", x.dim() == 3, x.device)
    lead = _cache_lead(x)
    codes = _out(codes, lead + (d * bits // 8,), torch.uint8, x.device, "codes")
    scales = _out(scales, lead + (max(d // max(group, 1), 1),), torch.float16, x.device, "scales")
    _same_device(x.device, codes=codes, scales=scales)
    sh = make_shape(B, T, H, d, group, bits, rot, variant)
    _check(srftq_quantize(sh, x, signs, lam, codes, scales, stream), "srftq_quantize")
    return codes, scales


def dequantize(codes, scales, signs=None, lam=None, group=16, bits=4, rot="srft", variant="default",
               d=None, out=None, stream=None):
    """codes + scales, head-major [B,H,T,.] (or [H,T,.]) -> fp16 [B,T,H,d]
    (or [T,H,d])."""
    import torch
    _req(codes, torch.uint8, "codes")
    _req(scales, torch.float16, "scales")
    _req(signs, torch.int8, "signs")
    _req(lam, torch.float32, "lambda")
    if d is None:
        d = codes.shape[-1] * 8 // bits
    if codes.dim() == 3:
        H, T = codes.shape[:2]
        B, oshape = 1, (T, H, d)
    elif codes.dim() == 4:
        B, H, T = codes.shape[:3]
        oshape = (B, T, H, d)
    else:
        raise ValueError("codes must be [H,T,*] or [B,H,T,*]")
    _check_scales(scales, codes.shape[:-1], d, group)
    _head_rows(signs, B, H, d, "signs", codes.dim() == 3, codes.device)
    _head_rows(lam, B, H, d, "lambda", codes.dim() == 3, codes.device)
    out = _out(out, oshape, torch.float16, codes.device, "out")
    _same_device(codes.device, scales=scales, out=out)
    sh = make_shape(B, T, H, d, group, bits, rot, variant)
    _check(srftq_dequantize(sh, codes, scales, signs, lam, out, stream), "srftq_dequantize")
    return out


def _check_scales(scales, lead, d, group):
    want = tuple(lead) + (max(d // max(group, 1), 1),)
    if tuple(scales.shape) != want:
        raise ValueError(f"scales must have shape {want}, got {tuple(scales.shape)}")


def _cache_dims(codes, scales, d, bits, group, name="codes"):
    """(B, H, t_cap) of a cache pair [B,H,t_cap,d*bits/8] / [B,H,t_cap,d/group]."""
    if codes.dim() != 4:
        raise ValueError(f"{name} must be [B,H,t_cap,d*bits/8]")
    B, H, t_cap, cb = codes.shape
    if cb != d * bits // 8:
        raise ValueError(f"{name} rows must hold {d * bits // 8} bytes, got {cb}")
    want = (B, H, t_cap, max(d // max(group, 1), 1))
    if tuple(scales.shape) != want:
        raise ValueError(f"scales must have shape {want}, got {tuple(scales.shape)}")
    return B, H, t_cap


def cache_append(x, codes, scales, pos=None, signs=None, lam=None, group=16, bits=4, rot="srft",
                 variant="default", stream=None):
    """Quantize the new tokens x fp16 [B,T,H,d] into the caches codes uint8
    [B,H,t_cap,d*bits/8] / scales fp16 [B,H,t_cap,d/group] in place: token t
    of tensor b goes to row pos[b] + t (pos int32 [B] on the device, or None
    for row t); rows outside [0, t_cap) are dropped."""
    import torch
    if x.dim() != 4:
        raise ValueError("x must be [B,T,H,d]")
    B, T, H, d = x.shape
    _req(x, torch.float16, "x")
    _req(codes, torch.uint8, "codes")
    _req(scales, torch.float16, "scales")
    _req(signs, torch.int8, "signs")
    _req(lam, torch.float32, "lambda")
    _req(pos, torch.int32, "pos")
    Bc, Hc, t_cap = _cache_dims(codes, scales, d, bits, group)
    if (Bc, Hc) != (B, H):
        raise ValueError(f"cache is for B={Bc}, H={Hc}; x has B={B}, H={H}")
    if pos is not None and tuple(pos.shape) != (B,):
        raise ValueError(f"pos must have shape ({B},)")
    _head_rows(signs, B, H, d, "signs", device=x.device)
    _head_rows(lam, B, H, d, "lambda", device=x.device)
    _same_device(x.device, codes=codes, scales=scales, pos=pos)
    sh = make_shape(B, T, H, d, group, bits, rot, variant)
    _check(srftq_cache_append(sh, t_cap, pos, x, signs, lam, codes, scales, stream), "srftq_cache_append")
    return codes, scales


class CacheAppender:
    """srftq_cache_append with everything but the new tokens checked once.

    For decode loops, where the per-call checks of cache_append cost more host
    time than the kernel: the caches, positions, signs, lambda, sizes and
    stream are fixed at construction (stream None: the current stream at that
    moment); each call passes x fp16 [B, tokens, H, d] of the same shape
    every time and runs srftq_cache_append on it.  The positions are read by
    the kernel when it runs, so the caller may advance them on the device
    between calls.  Not for use inside a graph capture on another stream."""

    def __init__(self, codes, scales, pos, signs=None, lam=None, group=16, bits=4, rot="srft",
                 variant="default", tokens=1, stream=None):
        import torch
        for t, dt, n in ((codes, torch.uint8, "codes"), (scales, torch.float16, "scales"),
                         (pos, torch.int32, "pos"), (signs, torch.int8, "signs"),
                         (lam, torch.float32, "lambda")):
            _req(t, dt, n)
        if pos is None:
            raise ValueError("pos is required")
        d = codes.shape[-1] * 8 // bits
        B, H, t_cap = _cache_dims(codes, scales, d, bits, group)
        if tuple(pos.shape) != (B,):
            raise ValueError(f"pos must have shape ({B},)")
        _head_rows(signs, B, H, d, "signs", device=codes.device)
        _head_rows(lam, B, H, d, "lambda", device=codes.device)
        _same_device(codes.device, scales=scales, pos=pos)
        self._device = codes.device
        self._shape = make_shape(B, int(tokens), H, d, group, bits, rot, variant)
        st = srftq_validate(self._shape)
        if st != SRFTQ_OK:
            _check(st, "srftq_validate")
        self.x_shape = (B, int(tokens), H, d)
        self._keep = (codes, scales, pos, signs, lam)        # the tensors outlive the appender's calls
        self._fn = lib().srftq_cache_append
        self._args = (ctypes.byref(self._shape), int(t_cap), _dp(pos))
        self._rest = (_dp(signs), _dp(lam), _dp(codes), _dp(scales), _stream(stream))
        self._f16 = torch.float16

    def __call__(self, x):
        if (tuple(x.shape) != self.x_shape or x.dtype != self._f16 or not x.is_contiguous()
                or x.device != self._device):
            raise ValueError(f"x must be a contiguous fp16 tensor of shape {self.x_shape} on {self._device}")
        st = self._fn(*self._args, x.data_ptr(), *self._rest)
        if st != SRFTQ_OK:
            _check(st, "srftq_cache_append")


def _x_dims(x_shape):
    """(B, T, H, d, flat) of an fp16 x shape [B,T,H,d] or [T,H,d]."""
    x_shape = tuple(int(v) for v in x_shape)
    if len(x_shape) == 4:
        return x_shape + (False,)
    if len(x_shape) == 3:
        return (1,) + x_shape + (True,)
    raise ValueError("x must be [B,T,H,d] or [T,H,d]")


class Quantizer:
    """srftq_quantize with everything but x checked once.

    For small launches in a loop (decode steps), where quantize()'s per-call
    checks cost more host time than the kernel: the output codes and scales,
    signs, lambda, sizes and stream are fixed at construction (stream None:
    the current stream at that moment); each call passes x fp16 of shape
    x_shape ([B,T,H,d] or [T,H,d]) and overwrites codes and scales.  Not for
    use inside a graph capture on another stream."""

    def __init__(self, x_shape, codes, scales, signs=None, lam=None, group=16, bits=4, rot="srft",
                 variant="default", stream=None):
        import torch
        B, T, H, d, flat = _x_dims(x_shape)
        for t, dt, n in ((codes, torch.uint8, "codes"), (scales, torch.float16, "scales"),
                         (signs, torch.int8, "signs"), (lam, torch.float32, "lambda")):
            _req(t, dt, n)
        if codes is None or scales is None:
            raise ValueError("codes and scales are required")
        lead = (H, T) if flat else (B, H, T)
        if tuple(codes.shape) != lead + (d * bits // 8,):
            raise ValueError(f"codes must have shape {lead + (d * bits // 8,)}")
        _check_scales(scales, lead, d, group)
        _head_rows(signs, B, H, d, "signs", flat, codes.device)
        _head_rows(lam, B, H, d, "lambda", flat, codes.device)
        _same_device(codes.device, scales=scales)
        self._shape = make_shape(B, T, H, d, group, bits, rot, variant)
        st = srftq_validate(self._shape)
        if st != SRFTQ_OK:
            _check(st, "srftq_validate")
        self.x_shape = (T, H, d) if flat else (B, T, H, d)
        self._device = codes.device
        self._keep = (codes, scales, signs, lam)        # the tensors outlive the quantizer's calls
        self._fn = lib().srftq_quantize
        self._sh = ctypes.byref(self._shape)
        self._rest = (_dp(signs), _dp(lam), _dp(codes), _dp(scales), _stream(stream))
        self._f16 = torch.float16

    def __call__(self, x):
        if (tuple(x.shape) != self.x_shape or x.dtype != self._f16 or not x.is_contiguous()
                or x.device != self._device):
            raise ValueError(f"x must be a contiguous fp16 tensor of shape {self.x_shape} on {self._device}")
        st = self._fn(self._sh, x.data_ptr(), *self._rest)
        if st != SRFTQ_OK:
            _check(st, "srftq_quantize")


class Dequantizer:
    """srftq_dequantize with everything but the codes and scales checked once.

    The counterpart of Quantizer: the output out fp16 ([B,T,H,d] or
    [T,H,d]), signs, lambda, sizes and stream are fixed at construction; each
    call passes codes and scales of the head-major shapes that quantize()
    writes for out's shape, and overwrites out."""

    def __init__(self, out, signs=None, lam=None, group=16, bits=4, rot="srft", variant="default",
                 stream=None):
        import torch
        _req(out, torch.float16, "out")
        _req(signs, torch.int8, "signs")
        _req(lam, torch.float32, "lambda")
        if out is None:
            raise ValueError("out is required")
        B, T, H, d, flat = _x_dims(out.shape)
        _head_rows(signs, B, H, d, "signs", flat, out.device)
        _head_rows(lam, B, H, d, "lambda", flat, out.device)
        self._shape = make_shape(B, T, H, d, group, bits, rot, variant)
        st = srftq_validate(self._shape)
        if st != SRFTQ_OK:
            _check(st, "srftq_validate")
        lead = (H, T) if flat else (B, H, T)
        self.codes_shape = lead + (d * bits // 8,)
        self.scales_shape = lead + (max(d // max(group, 1), 1),)
        self._device = out.device
        self._keep = (out, signs, lam)
        self._fn = lib().srftq_dequantize
        self._sh = ctypes.byref(self._shape)
        self._mid = (_dp(signs), _dp(lam), _dp(out), _stream(stream))
        self._u8, self._f16 = torch.uint8, torch.float16

    def __call__(self, codes, scales):
        if (tuple(codes.shape) != self.codes_shape or codes.dtype != self._u8 or not codes.is_contiguous()
                or codes.device != self._device):
            raise ValueError(f"codes must be a contiguous uint8 tensor of shape {self.codes_shape} on {self._device}")
        if (tuple(scales.shape) != self.scales_shape or scales.dtype != self._f16 or not scales.is_contiguous()
                or scales.device != self._device):
            raise ValueError(f"scales must be a contiguous fp16 tensor of shape {self.scales_shape} "
                             f"on {self._device}")
        st = self._fn(self._sh, codes.data_ptr(), scales.data_ptr(), *self._mid)
        if st != SRFTQ_OK:
            _check(st, "srftq_dequantize")


def cache_read(codes, scales, T, signs=None, lam=None, group=16, bits=4, rot="srft", variant="default",
               d=None, out=None, stream=None):
    """Dequantize + unrotate rows [0, T) of every head of a cache
    [B,H,t_cap,.] -> fp16 [B,T,H,d]."""
    import torch
    _req(codes, torch.uint8, "codes")
    _req(scales, torch.float16, "scales")
    _req(signs, torch.int8, "signs")
    _req(lam, torch.float32, "lambda")
    if d is None:
        d = codes.shape[-1] * 8 // bits
    B, H, t_cap = _cache_dims(codes, scales, d, bits, group)
    _head_rows(signs, B, H, d, "signs", device=codes.device)
    _head_rows(lam, B, H, d, "lambda", device=codes.device)
    out = _out(out, (B, int(T), H, d), torch.float16, codes.device, "out")
    _same_device(codes.device, scales=scales, out=out)
    sh = make_shape(B, int(T), H, d, group, bits, rot, variant)
    _check(srftq_cache_read(sh, t_cap, codes, scales, signs, lam, out, stream), "srftq_cache_read")
    return out


def decode_attention(q, k_codes, k_scales, v_codes, v_scales, k_signs=None, k_lam=None, v_signs=None,
                     v_lam=None, lengths=None, T=None, scale=None, group=16, bits=4, rot="srft",
                     workspace=None, out=None, stream=None):
    """Attention of one new query token per tensor over quantized K/V caches.
    q fp16 [B, H*R, d]; caches [B, H, t_cap, .] (srftq_cache_append layout);
    lengths int32 [B] (device) or None (= T, default t_cap); scale defaults
    to 1/sqrt(d).  Returns fp32 [B, H*R, d]."""
    return _attention(None, q, k_codes, k_scales, v_codes, v_scales, k_signs, k_lam, v_signs, v_lam, lengths,
                      T, scale, group, bits, rot, workspace, out, stream)


def decode_attention_dense(q, k_codes, k_scales, v_codes, v_scales, Qk, Qv, k_signs=None, k_lam=None,
                           v_signs=None, v_lam=None, lengths=None, T=None, scale=None, group=16, bits=4,
                           workspace=None, out=None, stream=None):
    """decode_attention over caches written by quantize_dense: Qk, Qv fp32
    [d, d] (one matrix) or [B, H, d, d] (one per head)."""
    return _attention((Qk, Qv), q, k_codes, k_scales, v_codes, v_scales, k_signs, k_lam, v_signs, v_lam,
                      lengths, T, scale, group, bits, "none", workspace, out, stream)


def _attention(mats, q, k_codes, k_scales, v_codes, v_scales, k_signs, k_lam, v_signs, v_lam, lengths, T,
               scale, group, bits, rot, workspace, out, stream):
    import math

    import torch
    _req(q, torch.float16, "q")
    for t, dt, n in ((k_codes, torch.uint8, "k_codes"), (k_scales, torch.float16, "k_scales"),
                     (v_codes, torch.uint8, "v_codes"), (v_scales, torch.float16, "v_scales"),
                     (k_signs, torch.int8, "k_signs"), (v_signs, torch.int8, "v_signs"),
                     (k_lam, torch.float32, "k_lam"), (v_lam, torch.float32, "v_lam"),
                     (lengths, torch.int32, "lengths")):
        _req(t, dt, n)
    if q.dim() != 3:
        raise ValueError("q must be [B, H*R, d]")
    B, HR, d = q.shape
    Bc, H, t_cap = _cache_dims(k_codes, k_scales, d, bits, group, "k_codes")
    if _cache_dims(v_codes, v_scales, d, bits, group, "v_codes") != (Bc, H, t_cap) or Bc != B:
        raise ValueError("K and V caches must both be [B, H, t_cap, .] for q's B")
    if HR % H:
        raise ValueError(f"q has {HR} heads, not a multiple of the {H} KV heads")
    R = HR // H
    _head_rows(k_signs, B, H, d, "k_signs", device=q.device)
    _head_rows(k_lam, B, H, d, "k_lam", device=q.device)
    _head_rows(v_signs, B, H, d, "v_signs", device=q.device)
    _head_rows(v_lam, B, H, d, "v_lam", device=q.device)
    if lengths is not None and tuple(lengths.shape) != (B,):
        raise ValueError(f"lengths must have shape ({B},), got {tuple(lengths.shape)}")
    _same_device(q.device, k_codes=k_codes, k_scales=k_scales, v_codes=v_codes, v_scales=v_scales,
                 lengths=lengths, workspace=workspace, out=out)
    T = t_cap if T is None else int(T)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    sh = make_shape(B, T, H, d, group, bits, rot)
    need = srftq_attention_workspace_bytes(sh, R)
    if need == 0 and B * H > 0:
        _check(SRFTQ_ERR_SHAPE, "srftq_attention_workspace_bytes")
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    out = _out(out, (B, HR, d), torch.float32, q.device, "out")
    kv = cache_view(k_codes, k_scales, k_signs, k_lam)
    vv = cache_view(v_codes, v_scales, v_signs, v_lam)
    nbytes = workspace.numel() * workspace.element_size()
    if mats is None:
        _check(srftq_decode_attention(sh, t_cap, R, q, kv, vv, lengths, scale, out, workspace, nbytes, stream),
               "srftq_decode_attention")
    else:
        Qk, Qv = mats
        _req(Qk, torch.float32, "Qk")
        _req(Qv, torch.float32, "Qv")
        qs = _q_stride(Qk, B, H, d)
        if _q_stride(Qv, B, H, d) != qs:
            raise ValueError("Qk and Qv must both be [d, d] or both [B, H, d, d]")
        _check(srftq_decode_attention_dense(sh, t_cap, R, Qk, Qv, qs, q, kv, vv, lengths, scale, out, workspace,
                                            nbytes, stream), "srftq_decode_attention_dense")
    return out


class DecodeAttention:
    """srftq_decode_attention with every argument checked once.

    For decode loops, where decode_attention()'s per-call checks take a
    quarter of the kernels' time at a 28-layer, 32K-token step: the query
    buffer q, the K and V caches, their signs and lambda, lengths, scale,
    workspace, out and stream are fixed at construction (stream None: the
    current stream at that moment; workspace and out allocated here when
    None).  The caller refills q, appends to the caches and updates lengths
    on the device between calls (they are read when the kernels run); each
    call runs one step and returns out.  Not for use inside a graph capture
    on another stream."""

    def __init__(self, q, k_codes, k_scales, v_codes, v_scales, k_signs=None, k_lam=None, v_signs=None,
                 v_lam=None, lengths=None, T=None, scale=None, group=16, bits=4, rot="srft", workspace=None,
                 out=None, stream=None):
        import math

        import torch
        _req(q, torch.float16, "q")
        for t, dt, n in ((k_codes, torch.uint8, "k_codes"), (k_scales, torch.float16, "k_scales"),
                         (v_codes, torch.uint8, "v_codes"), (v_scales, torch.float16, "v_scales"),
                         (k_signs, torch.int8, "k_signs"), (v_signs, torch.int8, "v_signs"),
                         (k_lam, torch.float32, "k_lam"), (v_lam, torch.float32, "v_lam"),
                         (lengths, torch.int32, "lengths")):
            _req(t, dt, n)
        if q.dim() != 3:
            raise ValueError("q must be [B, H*R, d]")
        B, HR, d = q.shape
        Bc, H, t_cap = _cache_dims(k_codes, k_scales, d, bits, group, "k_codes")
        if _cache_dims(v_codes, v_scales, d, bits, group, "v_codes") != (Bc, H, t_cap) or Bc != B:
            raise ValueError("K and V caches must both be [B, H, t_cap, .] for q's B")
        if HR % H:
            raise ValueError(f"q has {HR} heads, not a multiple of the {H} KV heads")
        R = HR // H
        for t, n in ((k_signs, "k_signs"), (k_lam, "k_lam"), (v_signs, "v_signs"), (v_lam, "v_lam")):
            _head_rows(t, B, H, d, n, device=q.device)
        if lengths is not None and tuple(lengths.shape) != (B,):
            raise ValueError(f"lengths must have shape ({B},), got {tuple(lengths.shape)}")
        _same_device(q.device, k_codes=k_codes, k_scales=k_scales, v_codes=v_codes, v_scales=v_scales,
                     lengths=lengths, workspace=workspace, out=out)
        T = t_cap if T is None else int(T)
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        self._shape = make_shape(B, T, H, d, group, bits, rot)
        need = srftq_attention_workspace_bytes(self._shape, R)
        if need == 0 and B * H > 0:
            _check(SRFTQ_ERR_SHAPE, "srftq_attention_workspace_bytes")
        if workspace is None:
            workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous CUDA (HIP) tensor")
        nbytes = workspace.numel() * workspace.element_size()
        if nbytes < need:
            raise ValueError(f"workspace holds {nbytes} bytes, the call needs {need}")
        self.out = _out(out, (B, HR, d), torch.float32, q.device, "out")
        self._kv = cache_view(k_codes, k_scales, k_signs, k_lam)
        self._vv = cache_view(v_codes, v_scales, v_signs, v_lam)
        self._keep = (q, k_codes, k_scales, v_codes, v_scales, k_signs, k_lam, v_signs, v_lam, lengths,
                      workspace)      # the tensors outlive the calls
        self._fn = lib().srftq_decode_attention
        self._args = (ctypes.byref(self._shape), int(t_cap), int(R), _dp(q), ctypes.byref(self._kv),
                      ctypes.byref(self._vv), _dp(lengths), float(scale), _dp(self.out), _dp(workspace),
                      int(nbytes), _stream(stream))

    def __call__(self):
        st = self._fn(*self._args)
        if st != SRFTQ_OK:
            _check(st, "srftq_decode_attention")
        return self.out


def rotate(x, signs=None, rot="srft", variant="default", out=None, stream=None):
    """Rotated coordinates y = M (s . x), fp32, same shape as x."""
    import torch
    B, T, H, d = _dims(x)
    _req(x, torch.float16, "x")
    _req(signs, torch.int8, "signs")
    _head_rows(signs, B, H, d, "signs", x.dim() == 3, x.device)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    elif tuple(out.shape) != tuple(x.shape):
        raise ValueError(f"out must have shape {tuple(x.shape)}")
    _req(out, torch.float32, "out")
    sh = make_shape(B, T, H, d, 8, 4, rot, variant)
    _check(srftq_rotate(sh, x, signs, out, stream), "srftq_rotate")
    return out


def unrotate(y, signs=None, rot="srft", variant="default", out=None, stream=None):
    """fp16 s . (M^T y), same shape as y."""
    import torch
    B, T, H, d = _dims(y)
    _req(y, torch.float32, "y")
    _req(signs, torch.int8, "signs")
    _head_rows(signs, B, H, d, "signs", y.dim() == 3, y.device)
    if out is None:
        out = torch.empty(y.shape, dtype=torch.float16, device=y.device)
    elif tuple(out.shape) != tuple(y.shape):
        raise ValueError(f"out must have shape {tuple(y.shape)}")
    _req(out, torch.float16, "out")
    sh = make_shape(B, T, H, d, 8, 4, rot, variant)
    _check(srftq_unrotate(sh, y, signs, out, stream), "srftq_unrotate")
    return out


def calibrate_lambda(x, signs=None, rot="srft", variant="default", out=None, stream=None):
    """lambda [B,H,d] (or [H,d] for 3-D x) = 1/RMS over tokens of the rotated coordinates."""
    import torch
    B, T, H, d = _dims(x)
    _req(x, torch.float16, "x")
    _req(signs, torch.int8, "signs")
    _head_rows(signs, B, H, d, "signs", x.dim() == 3, x.device)
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float32, device=x.device)
    elif tuple(out.shape) != (B, H, d):
        raise ValueError(f"out must have shape {(B, H, d)}")
    _req(out, torch.float32, "out")
    sh = make_shape(B, T, H, d, 8, 4, rot, variant)
    _check(srftq_calibrate_lambda(sh, x, signs, out, stream), "srftq_calibrate_lambda")
    return out if x.dim() == 4 else out[0]


def householder_matrix(V, out=None, stream=None):
    """Products of Householder reflections: V fp32 [..., k, d] (device) ->
    Q fp32 [..., d, d], Q = H_1 ... H_k with H_i = I - 2 v_i v_i^T / |v_i|^2."""
    import torch
    _req(V, torch.float32, "V")
    *lead, k, d = V.shape
    n = 1
    for m in lead:
        n *= m
    out = _out(out, tuple(lead) + (d, d), torch.float32, V.device, "out")
    _check(srftq_householder_matrix(d, k, n, V, out, stream), "srftq_householder_matrix")
    return out


def _q_stride(Q, B, H, d):
    if tuple(Q.shape) == (d, d):
        return 0
    if tuple(Q.shape) == (B, H, d, d):
        return d * d
    raise ValueError(f"Q must be [d, d] or [B, H, d, d] = [{B}, {H}, {d}, {d}], got {tuple(Q.shape)}")


def quantize_dense(x, Q, signs=None, lam=None, group=16, bits=4, codes=None, scales=None, stream=None):
    """As quantize() with the rotation y = Q (s . x): Q fp32 [d, d] (every
    head) or [B, H, d, d] (per head), e.g. from householder_matrix()."""
    import torch
    B, T, H, d = _dims(x)
    _req(x, torch.float16, "x")
    _req(Q, torch.float32, "Q")
    _req(signs, torch.int8, "signs")
    _req(lam, torch.float32, "lambda")
    qs = _q_stride(Q, B, H, d)
    _head_rows(signs, B, H, d, "signs", x.dim() == 3, x.device)
    _head_rows(lam, B, H, d, "lambda", x.dim() == 3, x.device)
    _same_device(x.device, Q=Q)
    lead = _cache_lead(x)
    codes = _out(codes, lead + (d * bits // 8,), torch.uint8, x.device, "codes")
    scales = _out(scales, lead + (max(d // max(group, 1), 1),), torch.float16, x.device, "scales")
    sh = make_shape(B, T, H, d, group, bits, "none")
    _check(srftq_quantize_dense(sh, Q, qs, x, signs, lam, codes, scales, stream), "srftq_quantize_dense")
    return codes, scales


def dequantize_dense(codes, scales, Q, signs=None, lam=None, group=16, bits=4, d=None, out=None, stream=None):
    """As dequantize() with x = s . (Q^T yhat)."""
    import torch
    _req(codes, torch.uint8, "codes")
    _req(scales, torch.float16, "scales")
    _req(Q, torch.float32, "Q")
    _req(signs, torch.int8, "signs")
    _req(lam, torch.float32, "lambda")
    if d is None:
        d = codes.shape[-1] * 8 // bits
    if codes.dim() == 3:
        H, T = codes.shape[:2]
        B, oshape = 1, (T, H, d)
    elif codes.dim() == 4:
        B, H, T = codes.shape[:3]
        oshape = (B, T, H, d)
    else:
        raise ValueError("codes must be [H,T,*] or [B,H,T,*]")
    qs = _q_stride(Q, B, H, d)
    _check_scales(scales, codes.shape[:-1], d, group)
    _head_rows(signs, B, H, d, "signs", codes.dim() == 3, codes.device)
    _head_rows(lam, B, H, d, "lambda", codes.dim() == 3, codes.device)
    _same_device(codes.device, scales=scales, Q=Q)
    out = _out(out, oshape, torch.float16, codes.device, "out")
    sh = make_shape(B, T, H, d, group, bits, "none")
    _check(srftq_dequantize_dense(sh, Q, qs, codes, scales, signs, lam, out, stream), "srftq_dequantize_dense")
    return out
