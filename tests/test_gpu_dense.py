"""GPU parity of the rotation-matrix path (learned / Householder rotations,
"When Quantization Is Free", Metodologia 3) against the oracle.

Inputs: the rotation matrices are the oracle's fp64 Householder products of
seeded reflector vectors, rounded to fp32, and are given to both sides; the
GPU's own Householder builder is checked separately against the oracle's.
Bars (oracle/compare.py): codes bit-exact except +-1 at rounding ties or in a
group whose fp16 scale sits on a rounding boundary; scales within one fp16
step; dequantized values within one fp16 ulp plus the fp32 budget
2^-18 ||x||.  The GPU product splits Q into two fp16 parts (about 2^-22
relative) with fp32 sums, well inside both bars; dequantize takes the codes
themselves as the exact second operand (1/lambda inside Q's parts, each
group's sigma applied to its fp32 partial) for groups of 16 and 32, and
splits yhat = q sigma / lambda into two parts as well for groups of 8.
"""
import numpy as np
import pytest
import torch

from kv_cache_quantization_srft_amd import srftq as S
from kv_cache_quantization_srft_amd import workloads as W
from oracle import compare, oracle

pytestmark = pytest.mark.gpu


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def householder_q(seed, lead, d, k):
    """fp32 reflectors [*lead, k, d] and the oracle's fp32 Q [*lead, d, d]."""
    r = np.random.default_rng(seed)
    V = r.standard_normal(tuple(lead) + (k, d)).astype(np.float32)
    return V, oracle.householder_matrix(V.astype(np.float64)).astype(np.float32)


def rand_x(seed, B, T, H, d, scale=1.0, lam=False, signs=True):
    r = np.random.default_rng(seed)
    g = np.exp(r.standard_normal((B, 1, H, d))).astype(np.float32)      # lognormal channel gains
    x = (r.standard_normal((B, T, H, d)) * g * scale).astype(np.float16)
    s = (1 - 2 * r.integers(0, 2, (B, H, d))).astype(np.int8) if signs else None
    l = r.uniform(0.25, 4.0, (B, H, d)).astype(np.float32) if lam else None
    return x, s, l


def run_and_check(x, Q, s, l, group, bits, dequant=True):
    d = x.shape[-1]
    xd, Qd, sd, ld = dev(x), dev(Q), dev(s), dev(l)
    codes_g, scales_g = S.quantize_dense(xd, Qd, sd, ld, group, bits)
    torch.cuda.synchronize()
    codes_o, scales_o, z_o = oracle.quantize_dense(x, Q, s, l, group, bits, return_z=True)
    cg, sg = host(codes_g), host(scales_g).view(np.uint16)
    st = compare.check_quantize(cg, sg, codes_o, scales_o, z_o, bits, group, d)
    if dequant:
        xg = S.dequantize_dense(codes_g, scales_g, Qd, sd, ld, group, bits, d=d)
        torch.cuda.synchronize()
        xo = oracle.dequantize_dense(cg, sg, Q, s, l, group, bits, d=d)
        st.update(compare.check_dequantize(host(xg), xo))
    return st


@pytest.mark.parametrize("d", [64, 128, 256, 100, 7])
@pytest.mark.parametrize("kind", ["half", "one", "none"])
def test_householder_matrix_matches_oracle(d, kind):
    """Q = H_1 ... H_k built on the GPU in fp64 against the oracle's fp64
    product, both rounded to fp32: at most one fp32 rounding step apart."""
    k = {"half": max(d // 2, 1), "one": 1, "none": 0}[kind]
    V, Q = householder_q(9000 + d + k, (3,), d, max(k, 1))
    V = V[:, :k]
    Q = oracle.householder_matrix(V.astype(np.float64)) if k else np.broadcast_to(np.eye(d), (3, d, d))
    Vd = dev(V) if k else torch.empty((3, 0, d), dtype=torch.float32, device="cuda")
    Qg = host(S.householder_matrix(Vd))
    err = np.abs(Qg.astype(np.float64) - Q)
    assert err.max() <= 2.0 ** -24, err.max()
    if k == 0:
        assert np.array_equal(Qg, np.broadcast_to(np.eye(d, dtype=np.float32), Qg.shape))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("group,bits", [(8, 4), (16, 4), (32, 4), (8, 8), (16, 8), (32, 8)])
def test_dense_matrix(d, group, bits):
    """Several tiles and a ragged tail, several tensors and heads; lambda on
    for half the cases; one shared matrix or one per head."""
    lam = (group + bits) % 3 != 0
    per_head = group != 16
    B, T, H = 2, 150, 3
    x, s, l = rand_x(9100 + d + group + bits, B, T, H, d, lam=lam)
    _, Q = householder_q(9200 + d, (B, H) if per_head else (), d, d // 2)
    print(f"[dense d={d} g={group} b={bits} lam={lam} per_head={per_head}]", flush=True)
    print(run_and_check(x, Q, s, l, group, bits))


@pytest.mark.parametrize("T", [1, 15, 16, 63, 64, 65, 200])
def test_dense_token_counts(T):
    x, s, _ = rand_x(9300 + T, 2, T, 2, 128)
    _, Q = householder_q(9301, (), 128, 64)
    print(run_and_check(x, Q, s, None, 16, 4))


def test_dense_heads_switch_inside_blocks():
    """More tiles than resident blocks, so a block walks across heads and
    rebuilds its matrix rows (per-head matrices, signs and lambda)."""
    B, T, H, d = 40, 130, 4, 256
    x, s, l = rand_x(9400, B, T, H, d, lam=True)
    _, Q = householder_q(9401, (B, H), d, d // 2)
    print(run_and_check(x, Q, s, l, 16, 4))


def test_dense_identity_and_srft_matrices():
    """Q = I and Q = the packed SRFT matrix (the oracle's FFT applied to the
    unit vectors): the GPU dense path reproduces the oracle's rot none / srft
    decisions."""
    d, g, bits = 128, 16, 4
    x, s, l = rand_x(9500, 2, 100, 2, d, lam=True)
    M = oracle.rotate(np.eye(d, dtype=np.float16).reshape(d, 1, d), None, "srft")[:, 0, :].T
    for rot, Q in (("none", np.eye(d, dtype=np.float32)), ("srft", M.astype(np.float32))):
        codes_g, scales_g = S.quantize_dense(dev(x), dev(Q), dev(s), dev(l), g, bits)
        torch.cuda.synchronize()
        co, so, zo = oracle.quantize(x, s, l, g, bits, rot, return_z=True)
        print(rot, compare.check_quantize(host(codes_g), host(scales_g).view(np.uint16), co, so, zo, bits, g, d))


def test_dense_zero_subnormal_and_saturated_groups():
    """Zero vectors, fp16-subnormal scales (the clamp path) and saturated
    scales (lambda = 1000 on head 1), through Q = I (values reach the
    quantizer as built) and through a Householder rotation.  The large rows
    are smaller for the rotation: it spreads a row of 60000s over every
    coordinate, and an int4 reconstruction of such a row leaves the fp16
    range on both sides."""
    d, g = 128, 16
    _, Qh = householder_q(9600, (), d, d // 2)
    for Q, big in ((np.eye(d, dtype=np.float32), 60000.0), (Qh, 20000.0)):
        x = np.zeros((1, 66, 2, d), dtype=np.float16)
        x[0, :, 0, 16] = np.float16(7 * 1.4 * 2.0 ** -24)
        x[0, :, 0, 33] = np.float16(3e-5)
        x[0, 3, 1, :] = big
        x[0, 4, 1, ::3] = -big / 2
        lam = np.ones((1, 2, d), dtype=np.float32)
        lam[0, 1] = 1000.0
        for bits in (4, 8):
            print(f"[dense edge big={big} bits={bits}]", flush=True)
            run_and_check(x, Q, None, lam, g, bits)
            run_and_check(x, Q, None, None, g, bits)


def test_dense_determinism_and_no_signs():
    d = 64
    x, s, _ = rand_x(9700, 1, 90, 2, d)
    _, Q = householder_q(9701, (), d, 32)
    a = S.quantize_dense(dev(x), dev(Q), None, None, 16, 4)
    b = S.quantize_dense(dev(x), dev(Q), torch.ones((1, 2, d), dtype=torch.int8, device="cuda"), None, 16, 4)
    c = S.quantize_dense(dev(x), dev(Q), None, None, 16, 4)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    for u, v in zip(a, c):
        assert torch.equal(u, v)
    print(run_and_check(x, Q, None, None, 16, 4))


def test_householder_workload_full_size_sampled():
    """The benchmark's workload (52 tensors x [T=32768, H=1, d=256], group 16,
    int4, k = 128 reflectors per tensor): GPU-built matrices against the
    oracle's, then quantize + dequantize at full size with the oracle's
    matrices, checked by the oracle on sampled tokens of several tensors."""
    w = W.WORKLOADS["householder"]
    x, s = W.generate(w)
    V = W.reflectors(w)
    print(f"[householder full] {x.shape} reflectors {V.shape}", flush=True)
    Q = oracle.householder_matrix(V.astype(np.float64))               # [B, H, d, d] fp64
    Qg = host(S.householder_matrix(dev(V)))
    assert np.abs(Qg.astype(np.float64) - Q).max() <= 2.0 ** -24
    Q = Q.astype(np.float32)
    xd, sd, Qd = dev(x), dev(s), dev(Q)
    codes, scales = S.quantize_dense(xd, Qd, sd, None, w.group, w.bits)
    xhat = S.dequantize_dense(codes, scales, Qd, sd, None, w.group, w.bits)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    for b in (0, 17, 34, w.B - 1):
        ts = np.sort(np.concatenate([[0, w.T - 1], rng.choice(w.T, 94, replace=False)]))
        xs = np.ascontiguousarray(x[b:b + 1, ts])                     # [1, n, H, d]
        co, so, zo = oracle.quantize_dense(xs, Q[b, 0], s[b:b + 1], None, w.group, w.bits, return_z=True)
        cg = host(codes[b:b + 1, :, ts])
        sg = host(scales[b:b + 1, :, ts]).view(np.uint16)
        st = compare.check_quantize(cg, sg, co, so, zo, w.bits, w.group, w.d)
        xo = oracle.dequantize_dense(cg, sg, Q[b, 0], s[b:b + 1], None, w.group, w.bits, d=w.d)
        st.update(compare.check_dequantize(host(xhat[b:b + 1, ts]), xo))
        print(f"[householder tensor {b}]", st, flush=True)
    rel = (torch.linalg.vector_norm(xhat.float() - xd.float()) / torch.linalg.vector_norm(xd.float())).item()
    print("roundtrip rel L2", rel)
    assert rel < 0.15
