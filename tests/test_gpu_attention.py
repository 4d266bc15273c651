"""GPU parity of srftq_decode_attention (attention of one new query token per
tensor over quantized K/V caches) against the oracle's fp64 definition.

Tolerance, per output vector o (fp32) against the oracle's o_ref (fp64),
derived from the arithmetic of the GPU path:
  * the P.V product rounds p * 2^14 and c_v * sigma_v to fp16, two relative
    errors of at most 2^-11 per term, so |sum_t p_t e_t y^_t| <= 2^-10
    max_t ||v^_t|| (the unrotation is orthonormal);
  * a score error eps (query split into fp16 hi + lo parts, residual
    2^-22 relative; fp32 accumulation) changes each p_t by a relative
    2 ln2 eps at most; with eps <= 2^-19 * Smax, Smax the largest
    sum_j |scale u_j y^_j| (the largest score magnitude before cancellation),
    that adds 2^-17 * Smax * max ||v^||;
  * fp32 exponentials, sums and the inverse transform are far below both.
So ||o - o_ref|| <= max_t ||v^_t|| * (2^-9 + 2^-17 * Smax), with a factor 2 of
margin on the first term; in addition the relative L2 error over all
outputs must stay within 1e-3 (the rotation tolerance of the path).
"""
import numpy as np
import pytest
import torch

from kv_cache_quantization_srft_amd import kvcache
from kv_cache_quantization_srft_amd import srftq as S
from oracle import oracle
from oracle.compare import decode_codes

pytestmark = pytest.mark.gpu


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def make_case(seed, B, T, H, R, d, g, bits, rot, lam=True, scale_k=1.0, scale_v=2.0, cap=None):
    r = np.random.default_rng(seed)
    cap = T if cap is None else cap
    k = (r.standard_normal((B, T, H, d)) * scale_k).astype(np.float16)
    v = (r.standard_normal((B, T, H, d)) * scale_v).astype(np.float16)
    sk = (1 - 2 * r.integers(0, 2, (B, H, d))).astype(np.int8)
    sv = (1 - 2 * r.integers(0, 2, (B, H, d))).astype(np.int8)
    lk = r.uniform(0.5, 2.0, (B, H, d)).astype(np.float32) if lam else None
    lv = r.uniform(0.5, 2.0, (B, H, d)).astype(np.float32) if lam else None
    q = (r.standard_normal((B, H * R, d)) * 1.5).astype(np.float16)
    kc, ks = oracle.quantize(k, sk, lk, g, bits, rot)
    vc, vs = oracle.quantize(v, sv, lv, g, bits, rot)
    if cap > T:   # cache with spare rows past T (filled with junk that must not be read as valid)
        pad = lambda a, fill: np.concatenate([a, np.full(a.shape[:2] + (cap - T,) + a.shape[3:], fill, a.dtype)], 2)
        kc, vc = pad(kc, 0x77), pad(vc, 0x77)
        ks, vs = pad(ks, 0x7BFF), pad(vs, 0x7BFF)
    return dict(q=q, K=(kc, ks, sk, lk), V=(vc, vs, sv, lv), g=g, bits=bits, rot=rot, T=T)


def make_case_dense(seed, B, T, H, R, d, g, bits, Qk, Qv, lam=True):
    """Caches written by the oracle's rotation-matrix quantizer: Qk, Qv fp32
    [d, d] or [B, H, d, d]."""
    r = np.random.default_rng(seed)
    k = r.standard_normal((B, T, H, d)).astype(np.float16)
    v = (r.standard_normal((B, T, H, d)) * 2.0).astype(np.float16)
    sk = (1 - 2 * r.integers(0, 2, (B, H, d))).astype(np.int8)
    sv = (1 - 2 * r.integers(0, 2, (B, H, d))).astype(np.int8)
    lk = r.uniform(0.5, 2.0, (B, H, d)).astype(np.float32) if lam else None
    lv = r.uniform(0.5, 2.0, (B, H, d)).astype(np.float32) if lam else None
    q = (r.standard_normal((B, H * R, d)) * 1.5).astype(np.float16)
    kc, ks = oracle.quantize_dense(k, Qk, sk, lk, g, bits)
    vc, vs = oracle.quantize_dense(v, Qv, sv, lv, g, bits)
    return dict(q=q, K=(kc, ks, sk, lk), V=(vc, vs, sv, lv), g=g, bits=bits, rot="dense", T=T, Qk=Qk, Qv=Qv)


def run_gpu(c, lengths=None, scale=None):
    K, V = c["K"], c["V"]
    args = (dev(c["q"]), dev(K[0]), dev(K[1].view(np.float16)), dev(V[0]), dev(V[1].view(np.float16)))
    kw = dict(k_signs=dev(K[2]), k_lam=dev(K[3]), v_signs=dev(V[2]), v_lam=dev(V[3]), lengths=dev(lengths),
              T=c["T"], scale=scale, group=c["g"], bits=c["bits"])
    if c["rot"] == "dense":
        out = S.decode_attention_dense(*args, dev(c["Qk"]), dev(c["Qv"]), **kw)
    else:
        out = S.decode_attention(*args, rot=c["rot"], **kw)
    torch.cuda.synchronize()
    return host(out)


def check(c, got, lengths=None, scale=None):
    K, V, q = c["K"], c["V"], c["q"]
    B, HR, d = q.shape
    H = K[0].shape[1]
    R, T, g, bits, rot = HR // H, c["T"], c["g"], c["bits"], c["rot"]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    kw = dict(T=T, lengths=lengths, signs_k=K[2], lam_k=K[3], signs_v=V[2], lam_v=V[3], group=g, bits=bits,
              scale=scale)
    if rot == "dense":
        ref = oracle.decode_attention_dense(q, K[0], K[1], V[0], V[1], c["Qk"], c["Qv"], **kw)
        _, vh = oracle.dequantize_dense(V[0][:, :, :T], V[1][:, :, :T], c["Qv"], V[2], V[3], g, bits, d=d,
                                        return_f64=True)
    else:
        ref = oracle.decode_attention(q, K[0], K[1], V[0], V[1], rot=rot, **kw)
        _, vh = oracle.dequantize(V[0][:, :, :T], V[1][:, :, :T], V[2], V[3], g, bits, rot, d=d,
                                  return_f64=True)
    assert np.all(np.isfinite(got))
    # per-vector bound
    vnorm = np.linalg.norm(vh, axis=-1)                                   # [B, T, H]
    ck = decode_codes(K[0][:, :, :T], bits, d).astype(np.float64)         # [B, H, T, d]
    sk = np.repeat(K[1][:, :, :T].view(np.float16).astype(np.float64), g, axis=-1)
    yk = ck * sk / (1.0 if K[3] is None else K[3][:, :, None].astype(np.float64))
    if rot == "dense":                                                    # u = Qk (s_k . q) * scale
        Qk = np.broadcast_to(np.asarray(c["Qk"], np.float64), (B, H, d, d))
        xs = q.astype(np.float64).reshape(B, H, R, d) * (1.0 if K[2] is None else K[2][:, :, None])
        u = np.einsum("bhjm,bhrm->bhrj", Qk, xs).reshape(B, HR, d) * scale
    else:
        u = oracle.rotate(q.reshape(B, 1, HR, d), np.repeat(K[2], R, axis=1) if K[2] is not None else None,
                          rot)[:, 0] * scale                              # [B, HR, d]
    worst = 0.0
    for b in range(B):
        L = T if lengths is None else min(max(int(lengths[b]), 0), T)
        for r in range(HR):
            h = r // R
            err = np.linalg.norm(got[b, r] - ref[b, r])
            if L == 0:
                assert err == 0.0, (b, r)
                continue
            smax = np.max(np.abs(yk[b, h, :L]) @ np.abs(u[b, r]))
            tol = vnorm[b, :L, h].max() * (2.0 ** -9 + 2.0 ** -17 * smax)
            assert err <= tol, f"b={b} r={r} err={err:.3g} tol={tol:.3g}"
            worst = max(worst, err / tol)
    den = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / den if den > 0 else np.linalg.norm(got)
    assert rel <= 1e-3, f"relative L2 {rel:.3g}"
    return {"rel_l2": float(rel), "worst_err_over_tol": float(worst)}


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("g,bits", [(16, 4), (32, 8), (64, 4)])
@pytest.mark.parametrize("rot", ["srft", "srht", "none"])
def test_attention_matrix(d, g, bits, rot):
    """Several chunks per head (1100 tokens: 4 chunks of 4 waves), a ragged
    tail, two tensors of different lengths, grouped query heads; lambda on
    for half the cases."""
    R = {64: 1, 128: 6, 256: 16}[d]
    lam = (d + g) % 2 == 0 and rot != "none"
    c = make_case(7000 + d + g + bits, 2, 1100, 2, R, d, g, bits, rot, lam=lam)
    lengths = np.array([1100, 681], dtype=np.int32)
    print(f"[attention d={d} g={g} b={bits} {rot} R={R} lam={lam}]", flush=True)
    print(check(c, run_gpu(c, lengths), lengths))


@pytest.mark.parametrize("d,g", [(64, 32), (64, 64), (128, 32), (128, 128), (256, 32), (256, 128), (256, 256)])
def test_attention_int4_group_sizes(d, g):
    """int4 V codes unpack in blocks of 32 coordinates, each lane taking both
    nibbles of one byte, with the lane's group scale chosen per lane at
    group 16 and per block otherwise: groups of 32 (one per block), 64 and
    more (one per several blocks), up to the whole vector."""
    R = {64: 2, 128: 6, 256: 8}[d]
    c = make_case(7080 + d + g, 2, 1100, 2, R, d, g, 4, "srft", lam=True)
    lengths = np.array([1100, 681], dtype=np.int32)
    print(f"[attention int4 d={d} g={g}]", flush=True)
    print(check(c, run_gpu(c, lengths), lengths))


@pytest.mark.parametrize("g,bits", [(16, 4), (32, 4), (16, 8), (32, 8)])
@pytest.mark.parametrize("rot", ["srft", "none"])
def test_attention_d96(g, bits, rot):
    """d = 96 (the SRFT with its radix-3 step): the direct-DFT query rotation
    and unrotation at a head size that is not a power of two, and 6-byte
    scale rows at group 32; four chunks, ragged lengths."""
    lam = bits == 4 and rot == "srft"
    c = make_case(7050 + g + bits, 2, 1100, 2, 6, 96, g, bits, rot, lam=lam)
    lengths = np.array([1100, 681], dtype=np.int32)
    print(f"[attention d=96 g={g} b={bits} {rot} lam={lam}]", flush=True)
    print(check(c, run_gpu(c, lengths), lengths))


def test_attention_d96_lengths():
    """Odd token counts in the last block (2-byte scale pieces, clamped to the
    last valid row), zero and one token, lengths past T."""
    c = make_case(7060, 8, 80, 1, 4, 96, 32, 4, "srft", cap=96)
    lengths = np.array([0, 1, 15, 16, 17, 63, 80, 500], dtype=np.int32)
    print(check(c, run_gpu(c, lengths), lengths))


def _householder(seed, lead, d):
    r = np.random.default_rng(seed)
    return oracle.householder_matrix(r.standard_normal(tuple(lead) + (d // 2, d))).astype(np.float32)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("g,bits", [(16, 4), (32, 8)])
def test_attention_dense(d, g, bits):
    """Caches written with Householder rotations (one per head for K, one
    shared matrix for V), four chunks, ragged lengths, lambda on for int4."""
    B, T, H, R = 2, 1100, 2, {64: 2, 128: 6, 256: 8}[d]
    Qk = _householder(7400 + d, (B, H), d)
    Qv = _householder(7401 + d, (), d)
    Qv = np.ascontiguousarray(np.broadcast_to(Qv, (B, H, d, d)))
    c = make_case_dense(7402 + d + g, B, T, H, R, d, g, bits, Qk, Qv, lam=bits == 4)
    lengths = np.array([1100, 681], dtype=np.int32)
    print(f"[attention dense d={d} g={g} b={bits}]", flush=True)
    print(check(c, run_gpu(c, lengths), lengths))


def test_attention_dense_shared_matrix_and_identity():
    """One matrix for every head (q_stride 0); the identity matrix gives the
    rot = none attention of the same caches."""
    B, T, H, R, d, g, bits = 2, 300, 2, 3, 128, 16, 4
    Q = _householder(7410, (), d)
    c = make_case_dense(7411, B, T, H, R, d, g, bits, Q, Q)
    lengths = np.array([300, 17], dtype=np.int32)
    print(check(c, run_gpu(c, lengths), lengths))
    I = np.eye(d, dtype=np.float32)
    c = make_case(7412, B, T, H, R, d, g, bits, "none")
    got_none = run_gpu(c, lengths)
    c.update(rot="dense", Qk=I, Qv=I)
    got_eye = run_gpu(c, lengths)
    print(check(c, got_eye, lengths))
    assert np.allclose(got_eye, got_none, rtol=1e-5, atol=1e-5 * np.abs(got_none).max())


def test_attention_lengths():
    """Zero, one, and block-boundary lengths, lengths past T (clamped), and a
    cache with spare rows past T holding junk."""
    c = make_case(7100, 8, 80, 1, 4, 128, 16, 4, "srft", cap=96)
    lengths = np.array([0, 1, 15, 16, 17, 64, 80, 500], dtype=np.int32)
    print(check(c, run_gpu(c, lengths), lengths))
    print(check(c, run_gpu(c, None), None))     # every tensor attends T tokens


def test_attention_more_heads_than_resident_blocks():
    """1,200 (tensor, KV head) pairs: one chunk each, a grid of more blocks
    than the chip holds at once, short ragged lengths."""
    c = make_case(7150, 300, 40, 4, 2, 64, 16, 4, "srft")
    lengths = (np.arange(300, dtype=np.int32) * 7) % 45
    print(check(c, run_gpu(c, lengths), lengths))


def test_attention_scale_and_large_scores():
    """A large softmax scale (peaked attention) and a tiny one (near uniform)."""
    c = make_case(7200, 2, 200, 2, 2, 64, 32, 4, "srft", scale_k=4.0)
    for scale in (2.0, 1e-4):
        print(check(c, run_gpu(c, scale=scale), scale=scale))


def test_attention_long_context():
    """20,000 tokens per head (many chunks of many blocks per wave): the P.V
    terms are tiny individually and must not lose precision."""
    c = make_case(7300, 2, 20000, 2, 6, 128, 16, 4, "srft")
    lengths = np.array([20000, 12345], dtype=np.int32)
    print(check(c, run_gpu(c, lengths), lengths))


def test_attention_more_chunks_than_threads():
    """One (tensor, KV head) pair with 70,000 tokens: 273 chunks, more than
    the combine kernel's 256 threads, so its loops over the chunk maxima and
    sums take more than one pass."""
    c = make_case(7310, 1, 70000, 1, 2, 64, 16, 4, "srft")
    lengths = np.array([69999], dtype=np.int32)
    print(check(c, run_gpu(c, lengths), lengths))


def test_attention_with_the_append_cache():
    """The container's caches, grown by a prefill and decode steps, read by
    decode attention at the container's lengths."""
    L, B, H, R, d, cap, g, bits = 1, 3, 2, 3, 128, 120, 16, 4
    r = np.random.default_rng(7400)
    signs = (1 - 2 * r.integers(0, 2, (L, 2, B, H, d))).astype(np.int8)
    cache = kvcache.QuantizedKVCache(L, B, H, d, cap, g, bits, "srft", dev(signs), None)
    k = r.standard_normal((B, 70, H, d)).astype(np.float16)
    v = r.standard_normal((B, 70, H, d)).astype(np.float16)
    cache.update(0, dev(k[:, :68]), dev(v[:, :68]))
    cache.update(0, dev(k[:, 68:69]), dev(v[:, 68:69]))
    cache.update(0, dev(k[:, 69:70]), dev(v[:, 69:70]))
    q = (r.standard_normal((B, H * R, d))).astype(np.float16)
    out = S.decode_attention(dev(q), cache.codes[0, 0], cache.scales[0, 0], cache.codes[0, 1],
                             cache.scales[0, 1], cache.signs[0, 0], None, cache.signs[0, 1], None,
                             lengths=cache.pos, T=cap)
    torch.cuda.synchronize()
    c = dict(q=q, K=(host(cache.codes[0, 0]), host(cache.scales[0, 0]).view(np.uint16), signs[0, 0], None),
             V=(host(cache.codes[0, 1]), host(cache.scales[0, 1]).view(np.uint16), signs[0, 1], None),
             g=g, bits=bits, rot="srft", T=cap)
    print(check(c, host(out), host(cache.pos)))


def test_attention_bench_workload_sampled():
    """The benchmark's decode step: 28 layers' caches of [T=32768, H=2,
    d=128] (group 16, int4, calibrated lambda), 6 query heads per KV head,
    in one launch; the oracle checks two of the layers."""
    from kv_cache_quantization_srft_amd import workloads as W
    w = W.WORKLOADS["outlier"]
    x, s = W.generate(w)
    lam = oracle.calibrate_lambda(np.ascontiguousarray(x[:, :512]), s, "srft")
    xd, sd, ld = dev(x), dev(s), dev(lam)
    codes, scales = S.quantize(xd, sd, ld, w.group, w.bits)
    kc, vc = codes[0::2].contiguous(), codes[1::2].contiguous()
    ks, vs = scales[0::2].contiguous(), scales[1::2].contiguous()
    q = W.attention_queries(w, R=6)
    out = S.decode_attention(dev(q), kc, ks, vc, vs, sd[0::2].contiguous(), ld[0::2].contiguous(),
                             sd[1::2].contiguous(), ld[1::2].contiguous(), group=w.group, bits=w.bits)
    torch.cuda.synchronize()
    out = host(out)
    for b in (0, w.B // 2 - 1):
        c = dict(q=q[b:b + 1], K=(host(kc[b:b + 1]), host(ks[b:b + 1]).view(np.uint16), s[2 * b:2 * b + 1],
                                  lam[2 * b:2 * b + 1]),
                 V=(host(vc[b:b + 1]), host(vs[b:b + 1]).view(np.uint16), s[2 * b + 1:2 * b + 2],
                    lam[2 * b + 1:2 * b + 2]),
                 g=w.group, bits=w.bits, rot="srft", T=w.T)
        print(f"[bench workload layer {b}]", check(c, out[b:b + 1]), flush=True)


@pytest.mark.parametrize("kind", ["srft", "dense"])
def test_attention_in_graph_replays(kind):
    """One decode-attention call captured in a HIP graph (fixed workspace and
    output) and replayed three times with new queries, eager work and
    synchronisations in between: every replay equals the eager call bit for
    bit (the launches hold no memsets and the plan depends on the shape only)."""
    B, T, H, R, d, g, bits = 2, 600, 2, 6, 128, 16, 4
    if kind == "dense":
        Q = _householder(7500, (), d)
        c = make_case_dense(7501, B, T, H, R, d, g, bits, Q, Q)
    else:
        c = make_case(7502, B, T, H, R, d, g, bits, "srft")
    K, V = c["K"], c["V"]
    lengths = dev(np.array([600, 333], dtype=np.int32))
    caches = (dev(K[0]), dev(K[1].view(np.float16)), dev(V[0]), dev(V[1].view(np.float16)))
    side = dict(k_signs=dev(K[2]), k_lam=dev(K[3]), v_signs=dev(V[2]), v_lam=dev(V[3]), lengths=lengths,
                group=g, bits=bits)
    if kind == "dense":
        Qd = dev(Q)
        call = lambda qq, **kw: S.decode_attention_dense(qq, *caches, Qd, Qd, **side, **kw)
    else:
        call = lambda qq, **kw: S.decode_attention(qq, *caches, rot="srft", **side, **kw)
    r = np.random.default_rng(7503)
    qs = [dev(r.standard_normal((B, H * R, d)).astype(np.float16)) for _ in range(3)]
    eager = [call(qq).clone() for qq in qs]
    torch.cuda.synchronize()

    q_buf = qs[0].clone()
    ws = torch.empty((S.srftq_attention_workspace_bytes(S.make_shape(B, T, H, d, g, bits), R),),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((B, H * R, d), dtype=torch.float32, device="cuda")
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):            # warm-up outside the capture
        call(q_buf, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(q_buf, workspace=ws, out=out)
    for i in range(3):
        q_buf.copy_(qs[i])
        out.fill_(float("nan"))
        call(qs[(i + 1) % 3])              # eager work on the same buffers' neighbours in between
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[i]), f"replay {i}"


def test_prepared_decode_attention_equals_plain_calls():
    """DecodeAttention (arguments checked once, one library call per step)
    gives the plain call's output bit for bit over two steps, with the query
    refilled and the lengths changed on the device in between, and matches
    the oracle."""
    c = make_case(7090, 2, 700, 2, 6, 128, 16, 4, "srft", lam=True)
    K, V = c["K"], c["V"]
    q = dev(c["q"])
    caches = (dev(K[0]), dev(K[1].view(np.float16)), dev(V[0]), dev(V[1].view(np.float16)))
    side = dict(k_signs=dev(K[2]), k_lam=dev(K[3]), v_signs=dev(V[2]), v_lam=dev(V[3]))
    lengths = dev(np.array([700, 333], dtype=np.int32))
    att = S.DecodeAttention(q, *caches, lengths=lengths, group=16, bits=4, **side)
    for step, (q_new, lens) in enumerate([(c["q"], [700, 333]), (c["q"][:, ::-1] * 0.5, [17, 700])]):
        q.copy_(dev(np.ascontiguousarray(q_new)))
        lengths.copy_(dev(np.array(lens, dtype=np.int32)))
        got = host(att()).copy()
        ref = host(S.decode_attention(q, *caches, lengths=lengths, group=16, bits=4, **side))
        torch.cuda.synchronize()
        assert np.array_equal(got, ref), f"step {step}"
        cc = dict(c, q=np.ascontiguousarray(q_new).astype(np.float16))
        print(step, check(cc, got, np.array(lens, dtype=np.int32)))
