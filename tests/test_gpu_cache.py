"""GPU parity of the growing quantized cache (srftq_cache_append /
srftq_cache_read and the QuantizedKVCache container) against the oracle.

Written rows are compared with the oracle's quantization of the same tokens
(oracle/compare.py tolerances: codes exact except at rounding ties); rows
that no append reaches must keep the sentinel they were filled with.
"""
import numpy as np
import pytest
import torch

from kv_cache_quantization_srft_amd import kvcache
from kv_cache_quantization_srft_amd import srftq as S
from kv_cache_quantization_srft_amd import workloads as W
from oracle import compare, oracle

pytestmark = pytest.mark.gpu

SENT_C, SENT_S = 0xA5, 0x5A5A


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def sentinel_cache(B, H, cap, d, g, bits):
    c = torch.full((B, H, cap, d * bits // 8), SENT_C, dtype=torch.uint8, device="cuda")
    s = torch.full((B, H, cap, d // g), SENT_S, dtype=torch.int16, device="cuda").view(torch.float16)
    return c, s


def check_placed(cc, cs, x, s, l, pos, g, bits, rot):
    """One append of x [B,n,H,d] at pos into a sentinel cache: placed rows
    match the oracle, every other row is untouched."""
    B, n, H, d = x.shape
    cap = cc.shape[2]
    cg, sg = host(cc), host(cs).view(np.uint16)
    co, so, zo = oracle.quantize(x, s, l, g, bits, rot, return_z=True)      # [B, H, n, .]
    written = np.zeros((B, cap), dtype=bool)
    for b in range(B):
        p = 0 if pos is None else int(pos[b])
        lo, hi = max(0, -p), min(n, cap - p)
        if lo >= hi:
            continue
        written[b, p + lo:p + hi] = True
        sl = (slice(b, b + 1), slice(None))
        compare.check_quantize(cg[sl + (slice(p + lo, p + hi),)], sg[sl + (slice(p + lo, p + hi),)],
                               co[sl + (slice(lo, hi),)], so[sl + (slice(lo, hi),)],
                               zo[sl + (slice(lo, hi),)], bits, g, d)
    keep = ~written
    assert np.all(cg.transpose(0, 2, 1, 3)[keep] == SENT_C)
    assert np.all(sg.transpose(0, 2, 1, 3)[keep] == SENT_S)
    return written


@pytest.mark.parametrize("d,g,bits,rot,lam", [
    (128, 16, 4, "srft", True), (64, 32, 8, "srht", False), (256, 16, 4, "srft", True),
    (128, 8, 4, "none", False), (96, 16, 4, "srft", True), (96, 32, 8, "srft", False)])
def test_append_ragged_positions(d, g, bits, rot, lam):
    """Several tiles and a ragged tail per head, positions that spill past
    both ends of the capacity."""
    B, n, H, cap = 5, 70, 3, 100
    r = np.random.default_rng(5000 + d + g)
    x = (r.standard_normal((B, n, H, d)) * 2).astype(np.float16)
    s = (1 - 2 * r.integers(0, 2, (B, H, d))).astype(np.int8)
    l = r.uniform(0.25, 4.0, (B, H, d)).astype(np.float32) if lam else None
    pos = np.array([0, 30, 95, -10, 100], dtype=np.int32)
    print(f"[append d={d} g={g} b={bits} {rot} lam={lam}] pos={pos.tolist()}", flush=True)
    cc, cs = sentinel_cache(B, H, cap, d, g, bits)
    S.cache_append(dev(x), cc, cs, dev(pos), dev(s), dev(l), g, bits, rot)
    torch.cuda.synchronize()
    written = check_placed(cc, cs, x, s, l, pos, g, bits, rot)
    assert written.sum() == 70 + 70 + 5 + 60 + 0


def test_append_without_positions_is_quantize():
    """pos = NULL writes token t to row t: with t_cap = T the cache equals
    srftq_quantize's output."""
    r = np.random.default_rng(5100)
    x = r.standard_normal((2, 130, 4, 128)).astype(np.float16)
    s = (1 - 2 * r.integers(0, 2, (2, 4, 128))).astype(np.int8)
    xd, sd = dev(x), dev(s)
    c1, s1 = S.quantize(xd, sd, None, 16, 4)
    c2, s2 = sentinel_cache(2, 4, 130, 128, 16, 4)
    S.cache_append(xd, c2, s2, None, sd, None, 16, 4)
    assert torch.equal(c1, c2) and torch.equal(s1.view(torch.int16), s2.view(torch.int16))


def test_decode_append_steps():
    """The decode-append shape: 256 sequences each appending one token per
    step ([256, 1, H=8, d=64], int8, group 32), positions advanced on the
    device between steps; after the steps, rows [0, steps) of every head are
    the oracle's codes of the whole sequence, the rest untouched."""
    w = W.WORKLOADS["decode"]
    steps, cap = 12, 16
    vals = W.values(w, B=steps)                           # [steps, 256, H, d]
    s = W.signs(w, B=w.T)                                 # one row per (sequence, head)
    x_all = np.ascontiguousarray(vals.transpose(1, 0, 2, 3))   # [256, steps, H, d]
    B, H, d = w.T, w.H, w.d
    print(f"[decode append] {steps} steps of {(B, 1, H, d)}", flush=True)
    cc, cs = sentinel_cache(B, H, cap, d, w.group, w.bits)
    sd = dev(s)
    pos = torch.zeros((B,), dtype=torch.int32, device="cuda")
    for t in range(steps):
        S.cache_append(dev(x_all[:, t:t + 1]), cc, cs, pos, sd, None, w.group, w.bits)
        pos += 1
    torch.cuda.synchronize()
    co, so, zo = oracle.quantize(x_all, s, None, w.group, w.bits, "srft", return_z=True)
    cg, sg = host(cc), host(cs).view(np.uint16)
    print(compare.check_quantize(cg[:, :, :steps], sg[:, :, :steps], co, so, zo, w.bits, w.group, d))
    assert np.all(cg[:, :, steps:] == SENT_C) and np.all(sg[:, :, steps:] == SENT_S)


@pytest.mark.parametrize("rot,lam", [("srft", True), ("srht", False)])
def test_cache_read_prefix(rot, lam):
    """Reading rows [0, T) of a cache with more rows than T (several tiles
    and a ragged tail) matches the oracle's dequantize of those codes."""
    B, T, H, d, cap, g, bits = 3, 77, 2, 128, 150, 16, 4
    r = np.random.default_rng(5200)
    x = r.standard_normal((B, 140, H, d)).astype(np.float16)
    s = (1 - 2 * r.integers(0, 2, (B, H, d))).astype(np.int8)
    l = r.uniform(0.5, 2.0, (B, H, d)).astype(np.float32) if lam else None
    cc, cs = sentinel_cache(B, H, cap, d, g, bits)
    S.cache_append(dev(x), cc, cs, None, dev(s), dev(l), g, bits, rot)
    xg = S.cache_read(cc, cs, T, dev(s), dev(l), g, bits, rot)
    torch.cuda.synchronize()
    cg, sg = host(cc), host(cs).view(np.uint16)
    xo = oracle.cache_read(cg, sg, T, s, l, g, bits, rot, d=d)
    print(compare.check_dequantize(host(xg), xo))
    assert S.cache_read(cc, cs, 0, dev(s), dev(l), g, bits, rot).shape == (B, 0, H, d)
    with pytest.raises(S.SrftqError):
        S.cache_read(cc, cs, cap + 1, dev(s), dev(l), g, bits, rot)


def test_container_prefill_then_decode():
    """QuantizedKVCache over two layers: a 70-token prefill, then two decode
    steps; each update returns K, V of every token so far, equal to the
    oracle's dequantization of the cache's codes, which equal the oracle's
    quantization of the tokens."""
    L, B, H, d, cap, g, bits = 2, 3, 2, 128, 80, 16, 4
    r = np.random.default_rng(5300)
    signs = (1 - 2 * r.integers(0, 2, (L, 2, B, H, d))).astype(np.int8)
    lam = r.uniform(0.5, 2.0, (L, 2, B, H, d)).astype(np.float32)
    cache = kvcache.QuantizedKVCache(L, B, H, d, cap, g, bits, "srft", dev(signs), dev(lam))
    chunks = [70, 1, 1]
    xs = {(l, k): (r.standard_normal((B, sum(chunks), H, d)) * 1.5).astype(np.float16)
          for l in range(L) for k in range(2)}
    t0 = 0
    for n in chunks:
        for l in range(L):
            K, V = cache.update(l, dev(xs[(l, 0)][:, t0:t0 + n]), dev(xs[(l, 1)][:, t0:t0 + n]))
            assert K.shape == (B, t0 + n, H, d) and V.shape == K.shape
            torch.cuda.synchronize()
            for kind, got in ((0, K), (1, V)):
                cg = host(cache.codes[l, kind])
                sg = host(cache.scales[l, kind]).view(np.uint16)
                xk = xs[(l, kind)][:, :t0 + n]
                co, so, zo = oracle.quantize(xk, signs[l, kind], lam[l, kind], g, bits, "srft",
                                             return_z=True)
                compare.check_quantize(cg[:, :, :t0 + n], sg[:, :, :t0 + n], co, so, zo, bits, g, d)
                xo = oracle.cache_read(cg, sg, t0 + n, signs[l, kind], lam[l, kind], g, bits, "srft", d=d)
                compare.check_dequantize(host(got), xo)
        t0 += n
    assert cache.length == sum(chunks)
    assert torch.equal(cache.pos, torch.full((B,), sum(chunks), dtype=torch.int32, device="cuda"))


def test_append_in_graph_replays():
    """Decode steps captured in a HIP graph (append, then the positions
    advanced by a torch kernel) and replayed three times, with eager work and
    synchronisations in between: every replay writes what eager calls write."""
    B, H, d, g, bits, steps, cap = 8, 2, 64, 32, 8, 3, 16
    r = np.random.default_rng(5400)
    xs = [dev(r.standard_normal((B, 1, H, d)).astype(np.float16)) for _ in range(steps)]
    s = dev((1 - 2 * r.integers(0, 2, (B, H, d))).astype(np.int8))
    ce, se = sentinel_cache(B, H, cap, d, g, bits)
    pos = torch.zeros((B,), dtype=torch.int32, device="cuda")
    for i in range(steps):
        S.cache_append(xs[i], ce, se, pos, s, None, g, bits)
        pos += 1
    torch.cuda.synchronize()

    cc, cs = sentinel_cache(B, H, cap, d, g, bits)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up outside the capture
        S.cache_append(xs[0], cc, cs, pos, s, None, g, bits)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            S.cache_append(xs[i], cc, cs, pos, s, None, g, bits)
            pos += 1
    for rep in range(3):
        cc.fill_(SENT_C)
        cs.view(torch.int16).fill_(SENT_S)
        pos.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(cc, ce), f"replay {rep}: codes differ from eager"
        assert torch.equal(cs.view(torch.int16), se.view(torch.int16)), f"replay {rep}: scales differ"
        assert torch.equal(pos, torch.full((B,), steps, dtype=torch.int32, device="cuda"))
        S.quantize(xs[0], s, None, g, bits)   # eager work between replays
        torch.cuda.synchronize()


def test_prepared_appender_matches_cache_append():
    """CacheAppender (arguments checked once, positions advanced on the device
    between calls) writes exactly what cache_append writes, with lambda, and
    rejects an input of another shape or type."""
    B, H, d, g, bits, steps, cap = 16, 4, 128, 16, 4, 5, 8
    r = np.random.default_rng(5500)
    xs = [dev(r.standard_normal((B, 1, H, d)).astype(np.float16)) for _ in range(steps)]
    s = dev((1 - 2 * r.integers(0, 2, (B, H, d))).astype(np.int8))
    lam = dev(r.uniform(0.5, 2.0, (B, H, d)).astype(np.float32))
    start = torch.from_numpy(r.integers(0, 3, B).astype(np.int32)).cuda()
    ce, se = sentinel_cache(B, H, cap, d, g, bits)
    pos = start.clone()
    for i in range(steps):
        S.cache_append(xs[i], ce, se, pos, s, lam, g, bits)
        pos += 1
    cp, sp = sentinel_cache(B, H, cap, d, g, bits)
    pos = start.clone()
    app = S.CacheAppender(cp, sp, pos, s, lam, g, bits)
    for i in range(steps):
        app(xs[i])
        pos += 1
    torch.cuda.synchronize()
    assert torch.equal(cp, ce)
    assert torch.equal(sp.view(torch.int16), se.view(torch.int16))
    with pytest.raises(ValueError):
        app(xs[0].float())
    with pytest.raises(ValueError):
        app(torch.cat([xs[0], xs[1]], dim=1))


def test_container_saved_and_loaded_reads_the_same(tmp_path):
    """A cache filled on the GPU, saved and loaded back (into a larger
    capacity), reads back bit for bit what the original reads, and goes on
    appending from the saved positions."""
    L, B, H, d, cap, g, bits = 2, 2, 2, 128, 48, 16, 4
    r = np.random.default_rng(5500)
    signs = (1 - 2 * r.integers(0, 2, (L, 2, B, H, d))).astype(np.int8)
    lam = r.uniform(0.5, 2.0, (L, 2, B, H, d)).astype(np.float32)
    cache = kvcache.QuantizedKVCache(L, B, H, d, cap, g, bits, "srft", dev(signs), dev(lam))
    for l in range(L):
        cache.update(l, dev(r.standard_normal((B, 33, H, d)).astype(np.float16)),
                     dev(r.standard_normal((B, 33, H, d)).astype(np.float16)))
    torch.cuda.synchronize()
    f = tmp_path / "c.safetensors"
    cache.save(f)
    back = kvcache.QuantizedKVCache.load(f, device="cuda", capacity=64)
    for l in range(L):
        for a, b in zip(cache.read(l), back.read(l)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    k = dev(r.standard_normal((B, 1, H, d)).astype(np.float16))
    for c in (cache, back):
        for l in range(L):
            c.update(l, k, k)
    torch.cuda.synchronize()
    for l in range(L):
        for a, b in zip(cache.read(l), back.read(l)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
