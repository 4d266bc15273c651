"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/srftq.h declares, and rejects bad arguments before
anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

from kv_cache_quantization_srft_amd import srftq as S
from oracle import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    hdr = open(os.path.join(ROOT, "include", "srftq.h")).read()
    return sorted(set(re.findall(r"\b(srftq_[a-z_]+)\s*\(", hdr)))


def test_library_exports_every_declared_function():
    L = S.lib()
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert S.srftq_version() >= 100
    for st in range(7):
        assert isinstance(S.status_string(st), str) and S.status_string(st)
    assert S.status_string(7) == "unknown status"


@pytest.mark.parametrize("kw,expect", [
    (dict(B=1, T=10, H=8, d=128, group=16, bits=4), S.SRFTQ_OK),
    (dict(B=56, T=32768, H=2, d=128, group=16, bits=4), S.SRFTQ_OK),
    (dict(B=1, T=256, H=8, d=64, group=32, bits=8), S.SRFTQ_OK),
    (dict(B=1, T=0, H=8, d=128, group=16, bits=4), S.SRFTQ_OK),
    (dict(B=0, T=5, H=8, d=128, group=16, bits=4), S.SRFTQ_OK),
    (dict(B=1, T=10, H=8, d=128, group=128, bits=8), S.SRFTQ_OK),
    (dict(B=1, T=10, H=8, d=112, group=16, bits=4), S.SRFTQ_ERR_UNSUPPORTED),
    (dict(B=1, T=10, H=4, d=256, group=16, bits=4), S.SRFTQ_OK),
    (dict(B=1, T=10, H=4, d=256, group=256, bits=8), S.SRFTQ_OK),
    (dict(B=1, T=10, H=4, d=512, group=16, bits=4), S.SRFTQ_ERR_UNSUPPORTED),
    (dict(B=1, T=10, H=8, d=128, group=16, bits=3), S.SRFTQ_ERR_UNSUPPORTED),
    (dict(B=1, T=10, H=8, d=128, group=12, bits=4), S.SRFTQ_ERR_UNSUPPORTED),
    (dict(B=1, T=10, H=8, d=128, group=4, bits=4), S.SRFTQ_ERR_UNSUPPORTED),
    (dict(B=1, T=10, H=8, d=64, group=128, bits=4), S.SRFTQ_ERR_UNSUPPORTED),
    (dict(B=-1, T=10, H=8, d=128, group=16, bits=4), S.SRFTQ_ERR_SHAPE),
    (dict(B=1, T=-1, H=8, d=128, group=16, bits=4), S.SRFTQ_ERR_SHAPE),
    (dict(B=1, T=10, H=0, d=128, group=16, bits=4), S.SRFTQ_ERR_SHAPE),
    (dict(B=1 << 20, T=1 << 30, H=8, d=128, group=16, bits=4), S.SRFTQ_ERR_SHAPE),
    (dict(B=1, T=2, H=65535, d=64, group=32, bits=8), S.SRFTQ_OK),
    (dict(B=1, T=10, H=8, d=96, group=16, bits=4), S.SRFTQ_OK),
    (dict(B=1, T=10, H=8, d=96, group=32, bits=8, rot=2), S.SRFTQ_OK),
    (dict(B=1, T=10, H=8, d=96, group=64, bits=4), S.SRFTQ_ERR_UNSUPPORTED),
    (dict(B=1, T=10, H=8, d=96, group=16, bits=4, rot=1), S.SRFTQ_ERR_UNSUPPORTED),
    (dict(B=1, T=10, H=8, d=96, group=16, bits=4, variant=2), S.SRFTQ_ERR_UNSUPPORTED),
    (dict(B=1, T=10, H=8, d=80, group=16, bits=4), S.SRFTQ_ERR_UNSUPPORTED),
    (dict(B=1, T=2, H=65536, d=64, group=32, bits=8), S.SRFTQ_ERR_SHAPE),
])
def test_validate(kw, expect):
    assert S.srftq_validate(S.make_shape(**kw)) == expect


def test_validate_rot_and_variant_range():
    assert S.srftq_validate(S.make_shape(1, 1, 1, 128, rot=5)) == S.SRFTQ_ERR_UNSUPPORTED
    assert S.srftq_validate(S.make_shape(1, 1, 1, 128, variant=3)) == S.SRFTQ_ERR_UNSUPPORTED
    for r in ("srft", "srht", "none"):
        for v in ("default", "real", "paired"):
            assert S.srftq_validate(S.make_shape(1, 1, 1, 128, rot=r, variant=v)) == S.SRFTQ_OK


def test_null_shape_pointer():
    assert S.lib().srftq_validate(None) == S.SRFTQ_ERR_NULL


@pytest.mark.parametrize("d,group,bits", [(128, 16, 4), (64, 32, 8), (128, 128, 8), (64, 8, 4), (96, 16, 4),
                                          (96, 32, 8)])
def test_sizes_match_oracle_layout(d, group, bits):
    B, T, H = 2, 7, 3
    sh = S.make_shape(B, T, H, d, group, bits)
    x = np.zeros((B, T, H, d), dtype=np.float16)
    codes, scales = oracle.quantize(x, None, None, group, bits, "none")
    assert S.srftq_codes_bytes(sh) == codes.nbytes
    assert S.srftq_scales_count(sh) == scales.size


def test_sizes_zero_for_invalid_shape():
    sh = S.make_shape(1, 10, 8, 112, 16, 4)
    assert S.srftq_codes_bytes(sh) == 0 and S.srftq_scales_count(sh) == 0


class _Fake:
    """Stands in for a tensor: only data_ptr() is read by the raw bindings."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def test_argument_errors_return_before_launch():
    sh = S.make_shape(1, 64, 8, 128, 16, 4)
    a = _Fake(0x10000)
    mis = _Fake(0x10008)
    # NULL required pointers
    assert S.srftq_quantize(sh, None, None, None, a, a, stream=0) == S.SRFTQ_ERR_NULL
    assert S.srftq_quantize(sh, a, None, None, None, a, stream=0) == S.SRFTQ_ERR_NULL
    assert S.srftq_dequantize(sh, a, None, None, None, a, stream=0) == S.SRFTQ_ERR_NULL
    assert S.srftq_rotate(sh, a, None, None, stream=0) == S.SRFTQ_ERR_NULL
    assert S.srftq_unrotate(sh, None, None, a, stream=0) == S.SRFTQ_ERR_NULL
    assert S.srftq_calibrate_lambda(sh, a, None, None, stream=0) == S.SRFTQ_ERR_NULL
    # misaligned data pointers
    assert S.srftq_quantize(sh, mis, None, None, a, a, stream=0) == S.SRFTQ_ERR_ALIGN
    assert S.srftq_quantize(sh, a, None, None, mis, a, stream=0) == S.SRFTQ_ERR_ALIGN
    assert S.srftq_dequantize(sh, a, mis, None, None, a, stream=0) == S.SRFTQ_ERR_ALIGN
    assert S.srftq_quantize(sh, a, _Fake(0x10001), None, a, a, stream=0) == S.SRFTQ_ERR_ALIGN
    assert S.srftq_quantize(sh, a, None, _Fake(0x10002), a, a, stream=0) == S.SRFTQ_ERR_ALIGN
    # bad shape wins over everything
    bad = S.make_shape(1, 64, 8, 100, 16, 4)
    assert S.srftq_quantize(bad, a, None, None, a, a, stream=0) == S.SRFTQ_ERR_UNSUPPORTED


def test_cache_argument_errors_return_before_launch():
    sh = S.make_shape(2, 5, 8, 128, 16, 4)
    a = _Fake(0x10000)
    # capacity: negative, or fewer rows than a read asks for
    assert S.srftq_cache_append(sh, -1, None, a, None, None, a, a, stream=0) == S.SRFTQ_ERR_SHAPE
    assert S.srftq_cache_read(sh, -1, a, a, None, None, a, stream=0) == S.SRFTQ_ERR_SHAPE
    assert S.srftq_cache_read(sh, 4, a, a, None, None, a, stream=0) == S.SRFTQ_ERR_SHAPE
    assert S.srftq_cache_append(sh, 1 << 45, None, a, None, None, a, a, stream=0) == S.SRFTQ_ERR_SHAPE
    # NULL and misaligned pointers
    assert S.srftq_cache_append(sh, 16, None, None, None, None, a, a, stream=0) == S.SRFTQ_ERR_NULL
    assert S.srftq_cache_append(sh, 16, None, a, None, None, a, None, stream=0) == S.SRFTQ_ERR_NULL
    assert S.srftq_cache_read(sh, 16, a, a, None, None, None, stream=0) == S.SRFTQ_ERR_NULL
    assert S.srftq_cache_append(sh, 16, _Fake(0x10002), a, None, None, a, a, stream=0) == S.SRFTQ_ERR_ALIGN
    assert S.srftq_cache_append(sh, 16, None, a, None, None, _Fake(0x10008), a, stream=0) == S.SRFTQ_ERR_ALIGN
    assert S.srftq_cache_read(sh, 16, a, a, None, None, _Fake(0x10004), stream=0) == S.SRFTQ_ERR_ALIGN
    # shape errors first, as for every other call
    bad = S.make_shape(2, 5, 8, 112, 16, 4)
    assert S.srftq_cache_append(bad, 16, None, a, None, None, a, a, stream=0) == S.SRFTQ_ERR_UNSUPPORTED
    # nothing to do: no tokens, or no rows to write into
    assert S.srftq_cache_append(sh, 0, None, None, None, None, None, None, stream=0) == S.SRFTQ_OK
    empty = S.make_shape(2, 0, 8, 128, 16, 4)
    assert S.srftq_cache_append(empty, 16, None, None, None, None, None, None, stream=0) == S.SRFTQ_OK
    assert S.srftq_cache_read(empty, 16, None, None, None, None, None, stream=0) == S.SRFTQ_OK


def test_attention_workspace_and_argument_errors():
    sh = S.make_shape(2, 1000, 2, 128, 16, 4)
    need = S.srftq_attention_workspace_bytes(sh, 6)
    # rotated queries + per-query-head exponents + per-chunk (max, sum) and accumulators
    assert need >= 2 * 2 * 6 * 128 * 4 + 2 * 2 * 6 * (2 + 128) * 4
    assert S.srftq_attention_workspace_bytes(sh, 0) == 0
    assert S.srftq_attention_workspace_bytes(sh, 17) == 0
    assert S.srftq_attention_workspace_bytes(S.make_shape(2, 1000, 2, 128, 8, 4), 6) == 0
    a, mis = _Fake(0x10000), _Fake(0x10008)
    kv = S.CacheView(0x10000, 0x10000, None, None)
    call = lambda shape=sh, t_cap=1000, R=6, q=a, k=kv, v=kv, lengths=None, scale=0.1, out=a, ws=a, nbytes=need: \
        S.srftq_decode_attention(shape, t_cap, R, q, k, v, lengths, scale, out, ws, nbytes, stream=0)
    assert call(R=0) == S.SRFTQ_ERR_SHAPE
    assert call(R=17) == S.SRFTQ_ERR_SHAPE
    assert call(shape=S.make_shape(2, 1000, 2, 128, 8, 4)) == S.SRFTQ_ERR_UNSUPPORTED
    # d = 96 is supported with the SRFT; the Walsh-Hadamard rotation needs a power of two
    assert S.srftq_attention_workspace_bytes(S.make_shape(2, 1000, 2, 96, 32, 4), 6) > 0
    assert call(shape=S.make_shape(2, 1000, 2, 96, 16, 4, rot="srht")) == S.SRFTQ_ERR_UNSUPPORTED
    assert call(t_cap=999) == S.SRFTQ_ERR_SHAPE
    assert call(scale=float("nan")) == S.SRFTQ_ERR_SHAPE
    assert call(scale=float("inf")) == S.SRFTQ_ERR_SHAPE
    assert call(q=None) == S.SRFTQ_ERR_NULL
    assert call(ws=None) == S.SRFTQ_ERR_NULL
    assert call(k=S.CacheView(0x10000, None, None, None)) == S.SRFTQ_ERR_NULL
    assert call(out=mis) == S.SRFTQ_ERR_ALIGN
    assert call(v=S.CacheView(0x10008, 0x10000, None, None)) == S.SRFTQ_ERR_ALIGN
    assert call(lengths=_Fake(0x10002)) == S.SRFTQ_ERR_ALIGN
    assert call(k=S.CacheView(0x10000, 0x10000, 0x10001, None)) == S.SRFTQ_ERR_ALIGN
    assert call(nbytes=need - 1) == S.SRFTQ_ERR_SHAPE
    # no tensors or no heads: nothing to do
    assert call(shape=S.make_shape(0, 1000, 2, 128, 16, 4), q=None, out=None, ws=None) == S.SRFTQ_OK


def test_noalloc_attention_argument_errors_return_before_launch():
    """srftq_decode_attention_noalloc checks everything srftq_decode_attention
    does, and a problem larger than the static scratch, before it touches a
    device."""
    sh = S.make_shape(2, 1000, 2, 128, 16, 4)
    a, mis = _Fake(0x10000), _Fake(0x10008)
    kv = S.CacheView(0x10000, 0x10000, None, None)
    call = lambda shape=sh, t_cap=1000, R=6, q=a, k=kv, v=kv, lengths=None, scale=0.1, out=a: \
        S.srftq_decode_attention_noalloc(shape, t_cap, R, q, k, v, lengths, scale, out, stream=0)
    assert call(R=0) == S.SRFTQ_ERR_SHAPE
    assert call(shape=S.make_shape(2, 1000, 2, 128, 8, 4)) == S.SRFTQ_ERR_UNSUPPORTED
    assert call(t_cap=999) == S.SRFTQ_ERR_SHAPE
    assert call(q=None) == S.SRFTQ_ERR_NULL
    assert call(out=mis) == S.SRFTQ_ERR_ALIGN
    assert call(shape=S.make_shape(0, 1000, 2, 128, 16, 4), q=None, out=None) == S.SRFTQ_OK
    # a workspace beyond the static array: 1,200 (tensor, head) pairs of 16 query heads at d = 256
    big = S.make_shape(600, 20000, 2, 256, 16, 4)
    assert S.srftq_attention_workspace_bytes(big, 16) > S.ATTENTION_SCRATCH_BYTES
    assert call(shape=big, t_cap=20000, R=16) == S.SRFTQ_ERR_CAPACITY
    hdr = open(os.path.join(ROOT, "include", "srftq.h")).read()
    m = re.search(r"#define SRFTQ_ATTENTION_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == S.ATTENTION_SCRATCH_BYTES
    # the benchmark's decode step fits
    bench = S.make_shape(28, 32768, 2, 128, 16, 4)
    assert 0 < S.srftq_attention_workspace_bytes(bench, 6) <= S.ATTENTION_SCRATCH_BYTES


def test_dense_attention_argument_errors_return_before_launch():
    sh = S.make_shape(2, 1000, 2, 128, 16, 4)
    need = S.srftq_attention_workspace_bytes(sh, 6)
    a, mis = _Fake(0x10000), _Fake(0x10008)
    kv = S.CacheView(0x10000, 0x10000, None, None)
    call = lambda shape=sh, Qk=a, Qv=a, qs=0, t_cap=1000, R=6, q=a, k=kv, v=kv, scale=0.1, out=a, ws=a, \
        nbytes=need: S.srftq_decode_attention_dense(shape, t_cap, R, Qk, Qv, qs, q, k, v, None, scale, out, ws,
                                                    nbytes, stream=0)
    # the sizes of the rotation-matrix quantizer with group >= 16
    assert call(shape=S.make_shape(2, 1000, 2, 96, 16, 4)) == S.SRFTQ_ERR_UNSUPPORTED
    assert call(shape=S.make_shape(2, 1000, 2, 128, 8, 4)) == S.SRFTQ_ERR_UNSUPPORTED
    assert call(shape=S.make_shape(2, 1000, 2, 128, 64, 4)) == S.SRFTQ_ERR_UNSUPPORTED
    assert call(qs=-1) == S.SRFTQ_ERR_SHAPE
    assert call(qs=128 * 128 - 4) == S.SRFTQ_ERR_SHAPE
    assert call(qs=128 * 128 + 2) == S.SRFTQ_ERR_SHAPE
    assert call(R=17) == S.SRFTQ_ERR_SHAPE
    assert call(Qk=None) == S.SRFTQ_ERR_NULL
    assert call(Qv=None) == S.SRFTQ_ERR_NULL
    assert call(Qv=mis) == S.SRFTQ_ERR_ALIGN
    assert call(q=None) == S.SRFTQ_ERR_NULL
    assert call(out=mis) == S.SRFTQ_ERR_ALIGN
    assert call(nbytes=need - 1) == S.SRFTQ_ERR_SHAPE
    assert call(shape=S.make_shape(0, 1000, 2, 128, 16, 4), Qk=None, Qv=None, q=None, out=None,
                ws=None) == S.SRFTQ_OK


def test_dense_argument_errors_return_before_launch():
    a, mis = _Fake(0x10000), _Fake(0x10008)
    sh = S.make_shape(2, 64, 4, 256, 16, 4)
    q = lambda shape=sh, Q=a, qs=0, x=a, signs=None, lam=None, codes=a, scales=a: \
        S.srftq_quantize_dense(shape, Q, qs, x, signs, lam, codes, scales, stream=0)
    dq = lambda shape=sh, Q=a, qs=0, codes=a, scales=a, signs=None, lam=None, out=a: \
        S.srftq_dequantize_dense(shape, Q, qs, codes, scales, signs, lam, out, stream=0)
    # supported sizes: d 64 / 128 / 256, groups 8 / 16 / 32; rot and variant unused
    assert q(shape=S.make_shape(2, 64, 4, 96, 16, 4)) == S.SRFTQ_ERR_UNSUPPORTED
    assert q(shape=S.make_shape(2, 64, 4, 256, 64, 4)) == S.SRFTQ_ERR_UNSUPPORTED
    assert dq(shape=S.make_shape(2, 64, 4, 128, 128, 8)) == S.SRFTQ_ERR_UNSUPPORTED
    assert q(shape=S.make_shape(2, 64, 4, 128, 16, 3)) == S.SRFTQ_ERR_UNSUPPORTED
    assert q(shape=S.make_shape(-1, 64, 4, 128, 16, 4)) == S.SRFTQ_ERR_SHAPE
    # matrix stride: 0, or at least d*d and a multiple of 4
    assert q(qs=-1) == S.SRFTQ_ERR_SHAPE
    assert q(qs=256 * 256 - 4) == S.SRFTQ_ERR_SHAPE
    assert dq(qs=256 * 256 + 2) == S.SRFTQ_ERR_SHAPE
    # NULL and misaligned pointers
    assert q(Q=None) == S.SRFTQ_ERR_NULL
    assert q(x=None) == S.SRFTQ_ERR_NULL
    assert dq(out=None) == S.SRFTQ_ERR_NULL
    assert q(Q=mis) == S.SRFTQ_ERR_ALIGN
    assert q(codes=mis) == S.SRFTQ_ERR_ALIGN
    assert dq(scales=mis) == S.SRFTQ_ERR_ALIGN
    assert q(signs=_Fake(0x10001)) == S.SRFTQ_ERR_ALIGN
    assert dq(lam=_Fake(0x10002)) == S.SRFTQ_ERR_ALIGN
    # empty problem
    empty = S.make_shape(2, 0, 4, 256, 16, 4)
    assert q(shape=empty, Q=None, x=None, codes=None, scales=None) == S.SRFTQ_OK
    assert dq(shape=empty, Q=None, codes=None, scales=None, out=None) == S.SRFTQ_OK
    # Householder products: d 1..256, k 0..1024, n 0..65535
    hh = lambda d=256, k=128, n=3, V=a, Q=a: S.srftq_householder_matrix(d, k, n, V, Q, stream=0)
    assert hh(d=0) == S.SRFTQ_ERR_SHAPE
    assert hh(d=257) == S.SRFTQ_ERR_SHAPE
    assert hh(k=-1) == S.SRFTQ_ERR_SHAPE
    assert hh(k=1025) == S.SRFTQ_ERR_SHAPE
    assert hh(n=-1) == S.SRFTQ_ERR_SHAPE
    assert hh(n=65536) == S.SRFTQ_ERR_SHAPE
    assert hh(V=None) == S.SRFTQ_ERR_NULL
    assert hh(Q=None) == S.SRFTQ_ERR_NULL
    assert hh(Q=_Fake(0x10002)) == S.SRFTQ_ERR_ALIGN
    assert hh(n=0, V=None, Q=None) == S.SRFTQ_OK


def test_empty_problem_is_a_no_op():
    sh = S.make_shape(1, 0, 8, 128, 16, 4)
    assert S.srftq_quantize(sh, None, None, None, None, None, stream=0) == S.SRFTQ_OK
    assert S.srftq_dequantize(sh, None, None, None, None, None, stream=0) == S.SRFTQ_OK
    assert S.srftq_rotate(sh, None, None, None, stream=0) == S.SRFTQ_OK
    assert S.srftq_unrotate(sh, None, None, None, stream=0) == S.SRFTQ_OK


def test_device_calls_without_a_device_report_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present; this checks the GPU-less failure path only")
    sh = S.make_shape(1, 64, 8, 128, 16, 4)
    a = _Fake(0x10000)
    assert S.srftq_quantize(sh, a, None, None, a, a, stream=0) == S.SRFTQ_ERR_HIP
    kv = S.CacheView(0x10000, 0x10000, None, None)
    need = S.srftq_attention_workspace_bytes(sh, 2)
    assert S.srftq_decode_attention(sh, 64, 2, a, kv, kv, None, 0.1, a, a, need, stream=0) == S.SRFTQ_ERR_HIP


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(S, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(S, "_lib", None)
    with pytest.raises(RuntimeError):
        S.lib()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus 2 exits with a message before any GPU work."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


# --------------------------------------------------------------------------
# The Python binding rejects misshaped or misplaced side tensors before any
# launch (the kernels index signs and lambda as [B, H, d] and lengths as [B]).
# --------------------------------------------------------------------------

def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros((2, 4, 3, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="CUDA"):
        S.quantize(x)
    with pytest.raises(ValueError, match="CUDA"):
        S.cache_append(x, torch.zeros((2, 3, 8, 32), dtype=torch.uint8),
                       torch.zeros((2, 3, 8, 4), dtype=torch.float16))


def test_head_rows_shapes():
    import torch
    B, H, d = 2, 3, 64
    ok = torch.ones((B, H, d), dtype=torch.int8)
    assert S._head_rows(ok, B, H, d, "signs") is ok
    assert S._head_rows(None, B, H, d, "signs") is None
    with pytest.raises(ValueError, match="signs must have shape"):
        S._head_rows(torch.ones((H, d), dtype=torch.int8), B, H, d, "signs", flat_ok=True)
    with pytest.raises(ValueError, match="lambda must have shape"):
        S._head_rows(torch.ones((B, H, d // 2)), B, H, d, "lambda")
    with pytest.raises(ValueError, match="lambda must have shape"):
        S._head_rows(torch.ones((B + 1, H, d)), B, H, d, "lambda")
    # one tensor, 3-D data: [H, d] and [1, H, d] both hold one row per head
    assert S._head_rows(torch.ones((H, d)), 1, H, d, "lambda", flat_ok=True) is not None
    assert S._head_rows(torch.ones((1, H, d)), 1, H, d, "lambda", flat_ok=True) is not None
    with pytest.raises(ValueError, match="is on"):
        S._same_device(torch.device("cuda", 0), pos=torch.zeros(2, dtype=torch.int32))


def test_cache_appender_rejects_cpu_tokens():
    """CacheAppender checks the new tokens' device on every call: a CPU
    tensor of the right shape and dtype raises before its host pointer could
    reach the kernel."""
    import torch
    app = object.__new__(S.CacheAppender)          # the fields __call__ reads, no device needed
    app.x_shape = (2, 1, 3, 64)
    app._f16 = torch.float16
    app._device = torch.device("cuda", 0)
    app._fn = None                                  # never reached
    with pytest.raises(ValueError, match="on cuda:0"):
        app(torch.zeros(app.x_shape, dtype=torch.float16))
    with pytest.raises(ValueError, match="shape"):
        app(torch.zeros((2, 2, 3, 64), dtype=torch.float16))


def test_quantizer_and_dequantizer_reject_bad_inputs():
    """Quantizer / Dequantizer check every call's inputs (shape, dtype,
    contiguity, device) before a pointer reaches the library, and refuse CPU
    outputs at construction."""
    import torch
    q = object.__new__(S.Quantizer)                 # the fields __call__ reads, no device needed
    q.x_shape = (2, 64, 3, 128)
    q._f16 = torch.float16
    q._device = torch.device("cuda", 0)
    q._fn = None                                    # never reached
    with pytest.raises(ValueError, match="on cuda:0"):
        q(torch.zeros(q.x_shape, dtype=torch.float16))
    with pytest.raises(ValueError, match="shape"):
        q(torch.zeros((2, 65, 3, 128), dtype=torch.float16))
    dq = object.__new__(S.Dequantizer)
    dq.codes_shape, dq.scales_shape = (2, 3, 64, 64), (2, 3, 64, 8)
    dq._u8, dq._f16 = torch.uint8, torch.float16
    dq._device = torch.device("cuda", 0)
    dq._fn = None
    with pytest.raises(ValueError, match="codes"):
        dq(torch.zeros(dq.codes_shape, dtype=torch.uint8), torch.zeros(dq.scales_shape, dtype=torch.float16))
    with pytest.raises(ValueError, match="codes"):
        dq(torch.zeros((2, 3, 64, 32), dtype=torch.uint8), torch.zeros(dq.scales_shape, dtype=torch.float16))
    with pytest.raises(ValueError, match="CUDA"):
        S.Quantizer((2, 64, 3, 128), torch.zeros((2, 3, 64, 64), dtype=torch.uint8),
                    torch.zeros((2, 3, 64, 8), dtype=torch.float16))
    with pytest.raises(ValueError, match="CUDA"):
        S.Dequantizer(torch.zeros((2, 64, 3, 128), dtype=torch.float16))


def test_cache_save_load_roundtrip(tmp_path):
    """QuantizedKVCache.save / load on the host: the rows written so far, the
    positions, signs, lambda and parameters come back unchanged, into a
    larger capacity if asked; a smaller capacity or a foreign file is refused.
    (No kernel runs: the buffers are filled directly.)"""
    import torch

    from kv_cache_quantization_srft_amd import kvcache
    L, B, H, d, cap, g, bits = 2, 3, 2, 64, 40, 16, 4
    r = np.random.default_rng(7100)
    signs = torch.from_numpy((1 - 2 * r.integers(0, 2, (L, 2, B, H, d))).astype(np.int8))
    lam = torch.from_numpy(r.uniform(0.5, 2.0, (L, 2, B, H, d)).astype(np.float32))
    c = kvcache.QuantizedKVCache(L, B, H, d, cap, g, bits, "srht", signs, lam, device="cpu")
    c.codes.copy_(torch.from_numpy(r.integers(0, 256, c.codes.shape).astype(np.uint8)))
    c.scales.copy_(torch.from_numpy(r.standard_normal(c.scales.shape).astype(np.float16)))
    c.pos.copy_(torch.tensor([7, 23, 11], dtype=torch.int32))
    c.length = 23
    f = tmp_path / "cache.safetensors"
    c.save(f)
    for capacity in (None, 64):
        c2 = kvcache.QuantizedKVCache.load(f, device="cpu", capacity=capacity)
        assert (c2.n_layers, c2.B, c2.H, c2.d, c2.group, c2.bits, c2.rot, c2.length) == \
            (L, B, H, d, g, bits, "srht", 23)
        assert c2.capacity == (cap if capacity is None else capacity)
        assert torch.equal(c2.pos, c.pos)
        assert torch.equal(c2.signs, signs) and torch.equal(c2.lam, lam)
        assert torch.equal(c2.codes[..., :23, :], c.codes[..., :23, :])
        assert torch.equal(c2.scales[..., :23, :].view(torch.int16), c.scales[..., :23, :].view(torch.int16))
        assert int(c2.codes[..., 23:, :].abs().sum()) == 0   # rows past the saved ones start empty
    with pytest.raises(ValueError):
        kvcache.QuantizedKVCache.load(f, device="cpu", capacity=20)
    from safetensors.torch import save_file
    g2 = tmp_path / "other.safetensors"
    save_file({"codes": torch.zeros(1, dtype=torch.uint8)}, str(g2), metadata={"format": "x"})
    with pytest.raises(ValueError):
        kvcache.QuantizedKVCache.load(g2, device="cpu")


def test_memfloor_library_rejects_bad_arguments_before_launch():
    """The benchmark's memory-floor library loads, exports its one call and
    turns a bad mix, size, grid or pointer into hipErrorInvalidValue (1)
    before any launch."""
    path = os.path.join(ROOT, "kv_cache_quantization_srft_amd", "libsrftq_memfloor.so")
    L = ctypes.CDLL(path)
    f = L.srftq_memfloor
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_int, ctypes.c_void_p]
    a, b = 0x10000, 0x20000
    assert f(3, 1, a, b, 64, 64, None) == 1           # unknown mix
    assert f(0, 1, a, b, 0, 1, None) == 1             # no tiles
    assert f(0, 1, a, b, 64, 65, None) == 1           # grid beyond the tiles
    assert f(0, 1, a, b, 64, 0, None) == 1            # empty grid
    assert f(1, 0, None, b, 64, 64, None) == 1        # NULL input
    assert f(1, 0, a + 8, b, 64, 64, None) == 1       # misaligned


def test_decode_attention_prepared_rejects_host_tensors():
    """DecodeAttention checks every argument at construction: host tensors
    raise before anything reaches the library."""
    import torch
    q = torch.zeros((1, 2, 128), dtype=torch.float16)
    kc = torch.zeros((1, 1, 64, 64), dtype=torch.uint8)
    ks = torch.zeros((1, 1, 64, 8), dtype=torch.float16)
    with pytest.raises(ValueError):
        S.DecodeAttention(q, kc, ks, kc, ks)
