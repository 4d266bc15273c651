"""Benchmark of the SRFT rotate-then-quantize hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload outlier]

One step = the whole hot path over one batch of synthetic KV tensors:
srftq_quantize (sign, SRFT, lambda, group absmax, int4 rounding and packing)
then srftq_dequantize (unpack, inverse SRFT, sign, fp16) of every vector,
one launch each.  The default workload is the 28-layer K+V outlier case:
56 tensors of fp16 [T=32768, H=2, d=128], lambda calibrated per rotated
coordinate, group 16, int4.

Prints one JSON line: throughput in KV vectors per second (each vector
quantized and dequantized), the per-kernel HBM roofline of the dominant
kernel (algorithmic bytes / measured kernel time vs 8 TB/s), the memory
floor of the same traffic (kernels that move a launch's bytes with no
arithmetic), and the CPU oracle timed on a bounded sample of the same
workload; then the other workloads' sections (the 128K-token roundtrip, the
d = 256 wide head with SRFT and SRHT, tiny launches, decode appends, decode
attention, d = 96 and rotation matrices).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCES = ["dev_common.h", "xform.h", "quant.h", "kernels.h", "dispatch.inc"]


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and whitespace removed, so a
    traffic record stays valid across edits that change no code."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "kv_cache_quantization_srft_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update("".join(src.split()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes_per_vector(d: int, group: int, bits: int) -> int:
    """fp16 vector + packed codes + fp16 group scales (one direction)."""
    return 2 * d + d * bits // 8 + 2 * (d // group)


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when missing or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def _kernel_family(name: str, w) -> str | None:
    """'quantize' / 'dequantize' for the workload's own kernel instance
    (template arguments d, group, bits), 'copy' for the copy probe."""
    import re
    inst = rf"<\s*{w.d},\s*{w.group},\s*{w.bits},"
    if re.search(r"dequantize_kernel" + inst, name):
        return "dequantize"
    if re.search(r"(?<!de)quantize_kernel" + inst, name):
        return "quantize"
    return "copy" if "neg" in name else None


def _counter_means(csv_path: str, counter: str, w) -> dict:
    """Mean counter value per dispatch, by kernel family, from a rocprofv3
    counter_collection.csv (values summed over the counter's instances)."""
    import csv
    per = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            fam = _kernel_family(row.get("Kernel_Name", ""), w)
            if fam is None:
                continue
            key = (fam, row.get("Dispatch_Id"))
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (fam, _), v in per.items():
        out.setdefault(fam, []).append(v)
    return {k: sum(v) / len(v) for k, v in out.items()}


def write_traffic(fetch_csv: str, write_csv: str, workload: str) -> None:
    """HBM bytes per launch of each streaming kernel from two rocprofv3 runs
    of this benchmark (--pmc FETCH_SIZE, --pmc WRITE_SIZE).  Each counter is
    scaled by what it reads for the copy kernel of known size (torch.neg over
    the quantize input: reads and writes exactly 2*d bytes per vector)."""
    from kv_cache_quantization_srft_amd import workloads as W
    w = W.WORKLOADS[workload]
    copy_bytes = 2 * w.d * w.nvec
    fetch = _counter_means(fetch_csv, "FETCH_SIZE", w)
    write = _counter_means(write_csv, "WRITE_SIZE", w)
    f_scale = copy_bytes / (fetch["copy"] * 1024.0)
    w_scale = copy_bytes / (write["copy"] * 1024.0)
    bpv = algorithmic_bytes_per_vector(w.d, w.group, w.bits)
    for k in ("quantize", "dequantize"):
        rd = fetch[k] * 1024.0 * f_scale
        wr = write[k] * 1024.0 * w_scale
        rec = {"kernel": k, "workload": workload, "kernel_source_hash": kernel_source_hash(),
               "fetch_kib_per_launch": fetch[k], "write_kib_per_launch": write[k],
               "fetch_scale": f_scale, "write_scale": w_scale,
               "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
               "hbm_bytes_per_launch": rd + wr,
               "algorithmic_bytes_per_launch": bpv * w.nvec,
               "traffic_over_algorithmic": (rd + wr) / (bpv * w.nvec)}
        path = os.path.join(ROOT, "profiles", f"traffic_{k}_{workload}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))


def _oracle_sample(w, x, s, lam, target_s: float):
    """The oracle, as it stands, on the first tokens of every tensor (quantize
    then dequantize), sized by a pilot run to about target_s seconds."""
    import numpy as np
    from oracle import oracle

    tp = 16
    xs = np.ascontiguousarray(x[:, :tp])
    t0 = time.perf_counter()
    c, sc = oracle.quantize(xs, s, lam, w.group, w.bits, "srft")
    oracle.dequantize(c, sc, s, lam, w.group, w.bits, "srft", d=w.d)
    pilot = time.perf_counter() - t0
    tn = int(min(w.T, max(tp, tp * target_s / max(pilot, 1e-6))))
    xs = np.ascontiguousarray(x[:, :tn])
    t0 = time.perf_counter()
    c, sc = oracle.quantize(xs, s, lam, w.group, w.bits, "srft")
    oracle.dequantize(c, sc, s, lam, w.group, w.bits, "srft", d=w.d)
    dt = time.perf_counter() - t0
    nv = w.B * tn * w.H
    return nv / dt, (f"first {tn} tokens of each of the {w.B} tensors ({nv} vectors), "
                     f"quantize + dequantize, fp64 direct DFT, {dt:.1f} s")


def cpu_baseline(w, x, s, lam, target_s: float = 12.0):
    """The oracle on all its threads (OpenMP over vectors), then on one core."""
    from oracle import oracle

    threads = oracle.num_threads()
    v, sample = _oracle_sample(w, x, s, lam, target_s)
    oracle.set_num_threads(1)
    try:
        v1, sample1 = _oracle_sample(w, x, s, lam, target_s / 2)
    finally:
        oracle.set_num_threads(threads)
    return {"value": v, "unit": "KV vectors/s", "cores": threads, "kind": "oracle", "sample": sample,
            "host_cpu_count": os.cpu_count(),
            "one_core": {"value": v1, "unit": "KV vectors/s", "cores": 1, "sample": sample1}}


SECTION_SETTLE_S = 0.3


def _settle(fn, seconds: float = SECTION_SETTLE_S) -> int:
    """Untimed calls of fn for `seconds` of sustained load before a section's
    timed launches: after a light phase (single-token appends, host work)
    the GPU's clocks need a sustained load to return to their working level,
    and a section timed straight away can run several times slower for its
    first tens of milliseconds.  Returns the number of calls."""
    import torch

    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def decode_append_latency(steps: int = 1000, graph_steps: int = 100) -> dict:
    """The decode-append shape: 256 sequences each append one token per step
    ([256, 1, H=8, d=64], int8, group 32) into a per-head cache of
    `steps` rows through srftq_cache_append, write positions advanced on the
    device.  Reported: the per-step time of eager calls through the Python
    binding (host-bound at this size), and of the same steps replayed from
    a HIP graph of `graph_steps` steps (GPU time per step)."""
    import numpy as np
    import torch

    from kv_cache_quantization_srft_amd import srftq as S
    from kv_cache_quantization_srft_amd import workloads as W

    w = W.WORKLOADS["decode"]
    B, H, d = w.T, w.H, w.d
    dev = torch.device("cuda:0")
    vals = torch.from_numpy(W.values(w, B=graph_steps)).to(dev)          # [steps, 256, H, d]
    xs = [vals[i].unsqueeze(1).contiguous() for i in range(graph_steps)]   # [256, 1, H, d] each
    sd = torch.from_numpy(W.signs(w, B=B)).to(dev)
    codes = torch.zeros((B, H, steps, d * w.bits // 8), dtype=torch.uint8, device=dev)
    scales = torch.zeros((B, H, steps, d // w.group), dtype=torch.float16, device=dev)
    pos = torch.zeros((B,), dtype=torch.int32, device=dev)

    def one(i):
        S.cache_append(xs[i % graph_steps], codes, scales, pos, sd, None, w.group, w.bits)
        pos.add_(1)

    for i in range(20):
        one(i)
    torch.cuda.synchronize()
    pos.zero_()
    wall = []
    torch.cuda.synchronize()
    for i in range(steps):
        t = time.perf_counter()
        one(i)
        torch.cuda.synchronize()
        wall.append((time.perf_counter() - t) * 1e6)
    wall = np.array(wall)
    eager_codes, eager_scales = codes.clone(), scales.clone()

    # the same eager steps through a CacheAppender (arguments checked once),
    # into a cleared cache, so that matching rows show the appender wrote them
    app = S.CacheAppender(codes, scales, pos, sd, None, w.group, w.bits)
    pos.zero_()
    codes.zero_()
    scales.zero_()
    for i in range(20):
        app(xs[i % graph_steps])
        pos.add_(1)
    pos.zero_()
    codes.zero_()
    scales.zero_()
    torch.cuda.synchronize()
    wall_p = []
    for i in range(steps):
        t = time.perf_counter()
        app(xs[i % graph_steps])
        pos.add_(1)
        torch.cuda.synchronize()
        wall_p.append((time.perf_counter() - t) * 1e6)
    wall_p = np.array(wall_p)
    prepared_same = bool(torch.equal(codes, eager_codes)
                         and torch.equal(scales.view(torch.int16), eager_scales.view(torch.int16)))

    # the same steps captured once and replayed (positions keep advancing on
    # the device; rows past the capacity would be dropped, none are reached)
    pos.zero_()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(graph_steps):
            one(i)
    reps = max(1, (steps - 1) // graph_steps)
    codes.zero_()
    scales.zero_()
    pos.zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    pos.zero_()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / (reps * graph_steps)
    # every replayed step wrote the rows an eager step wrote from the same input
    n = reps * graph_steps
    same = bool(torch.equal(codes[:, :, :n], eager_codes[:, :, :n])
                and torch.equal(scales[:, :, :n].view(torch.int16), eager_scales[:, :, :n].view(torch.int16)))
    return {"workload": f"decode-append: {B} sequences x 1 token, H={H}, d={d}, "
                        f"SRFT, group {w.group}, int{w.bits}, {steps} steps",
            "vectors_per_step": B * H,
            "eager_us_per_step": {"mean": float(wall.mean()), "p50": float(np.percentile(wall, 50)),
                                  "p99": float(np.percentile(wall, 99))},
            "eager_prepared_us_per_step": {"mean": float(wall_p.mean()), "p50": float(np.percentile(wall_p, 50)),
                                           "p99": float(np.percentile(wall_p, 99)),
                                           "rows_match_eager": prepared_same},
            "graph_us_per_step": graph_us,
            "graph_ns_per_vector": graph_us * 1e3 / (B * H),
            "graph_rows_match_eager": same,
            "step": "srftq_cache_append of the new tokens, then the positions advanced (+1)"}


def decode_attention_timing(w, codes, scales, sd, lam, steps: int, R: int = 6) -> dict:
    """One decode step of attention over the workload's caches read as 28
    layers' K (even tensors) and V (odd tensors): srftq_decode_attention of
    one new query token per layer, R query heads per KV head, all layers in
    one call.  Algorithmic bytes: every cached code and scale of K and V once
    (queries and outputs are under 0.1 %)."""
    import numpy as np
    import torch

    from kv_cache_quantization_srft_amd import srftq as S
    from kv_cache_quantization_srft_amd import workloads as W

    dev = codes.device
    kc, vc = codes[0::2].contiguous(), codes[1::2].contiguous()
    ks, vs = scales[0::2].contiguous(), scales[1::2].contiguous()
    sk, sv = sd[0::2].contiguous(), sd[1::2].contiguous()
    lk = None if lam is None else lam[0::2].contiguous()
    lv = None if lam is None else lam[1::2].contiguous()
    q = torch.from_numpy(W.attention_queries(w, R)).to(dev)
    L = w.B // 2
    sh = S.make_shape(L, w.T, w.H, w.d, w.group, w.bits)
    ws = torch.empty((S.srftq_attention_workspace_bytes(sh, R),), dtype=torch.uint8, device=dev)
    out = torch.empty((L, w.H * R, w.d), dtype=torch.float32, device=dev)

    def call():
        S.decode_attention(q, kc, ks, vc, vs, sk, lk, sv, lv, group=w.group, bits=w.bits,
                           workspace=ws, out=out)

    _settle(call)
    # calls back to back (a decode loop's pattern), one event pair around
    # them, and the host's enqueue time of the same calls: the GPU time per
    # call is the kernels' own only while the host enqueues faster
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    b0.record()
    for _ in range(steps):
        call()
    b1.record()
    host_us = (time.perf_counter() - h0) / steps * 1e6
    torch.cuda.synchronize()
    ms = b0.elapsed_time(b1) / steps
    # the same calls through srftq.DecodeAttention (arguments checked once)
    att = S.DecodeAttention(q, kc, ks, vc, vs, sk, lk, sv, lv, group=w.group, bits=w.bits, workspace=ws, out=out)
    att()
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    b0.record()
    for _ in range(steps):
        att()
    b1.record()
    host_prep_us = (time.perf_counter() - h0) / steps * 1e6
    torch.cuda.synchronize()
    prep_ms = b0.elapsed_time(b1) / steps
    # and with an event pair around each call (which also drains the queue
    # between calls)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    per_call = _dist([e0.elapsed_time(e1) for e0, e1 in evs])
    bpv = w.d * w.bits // 8 + 2 * (w.d // w.group)
    nbytes = 2 * L * w.H * w.T * bpv
    fp16_bytes = 2 * L * w.H * w.T * 2 * w.d
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"decode attention: {L} layers x K+V caches [T={w.T}, H={w.H}, d={w.d}], "
                        f"group {w.group}, int{w.bits}, {R} query heads per KV head, one query token",
            "ms": ms, "calls_back_to_back": steps, "host_enqueue_us_per_call": host_us,
            "prepared": {"ms": prep_ms, "host_enqueue_us_per_call": host_prep_us,
                         "call": "srftq.DecodeAttention (arguments checked once)"},
            "per_call_events": per_call,
            "algorithmic_bytes": nbytes, "GBps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS,
            "cached_tokens_per_s": L * w.H * w.T / (ms * 1e-3),
            "fp16_cache_bytes": fp16_bytes,
            "fp16_cache_read_ms_at_same_GBps": fp16_bytes / (gbps * 1e9) * 1e3,
            "step": "srftq_decode_attention (query rotation, partial attention over token chunks, "
                    "chunk merge + unrotation: three launches)"}


def non_pow2_timing(steps: int) -> dict:
    """Quantize + dequantize at d = 96 (the SRFT with a radix-3 step, per-lane
    kernels): 8 tensors of fp16 [T=32768, H=8, d=96], N(0,1) drawn on the
    device from a fixed seed, group 16, int4."""
    import torch

    from kv_cache_quantization_srft_amd import srftq as S

    B, T, H, d, g, bits = 8, 32768, 8, 96, 16, 4
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260508)
    x = torch.randn((B, T, H, d), device=dev, generator=gen).half()
    s = (torch.randint(0, 2, (B, H, d), device=dev, generator=gen) * 2 - 1).to(torch.int8)
    codes = torch.empty((B, H, T, d * bits // 8), dtype=torch.uint8, device=dev)
    scales = torch.empty((B, H, T, d // g), dtype=torch.float16, device=dev)
    xhat = torch.empty_like(x)
    def pair():
        S.quantize(x, s, None, g, bits, codes=codes, scales=scales)
        S.dequantize(codes, scales, s, None, g, bits, out=xhat)
    _settle(pair)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tq = tdq = 0.0
    for _ in range(steps):
        ev[0].record()
        S.quantize(x, s, None, g, bits, codes=codes, scales=scales)
        ev[1].record()
        S.dequantize(codes, scales, s, None, g, bits, out=xhat)
        ev[2].record()
        torch.cuda.synchronize()
        tq += ev[0].elapsed_time(ev[1])
        tdq += ev[1].elapsed_time(ev[2])
    n = B * T * H
    bpv = algorithmic_bytes_per_vector(d, g, bits)
    q_ms, dq_ms = tq / steps, tdq / steps
    return {"workload": f"{B} x fp16 [T={T}, H={H}, d={d}], SRFT (radix-3 step), group {g}, int{bits}",
            "quantize_ms": q_ms, "dequantize_ms": dq_ms, "bytes_per_vector": bpv,
            "quantize_hbm_frac": bpv * n / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "dequantize_hbm_frac": bpv * n / (dq_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "vectors_per_s_step": n / ((q_ms + dq_ms) * 1e-3)}


def memory_floor_timing(nvec: int, pairs: int, q_ms: float, dq_ms: float) -> dict | None:
    """HBM floor of the headline's two traffic mixes, measured in the same
    run: libsrftq_memfloor.so's kernels move exactly a quantize launch's
    bytes (16 KiB read, 5 KiB written per 64-vector tile) and a dequantize
    launch's (5 KiB read, 16 KiB written), with no arithmetic, alternating
    as the benchmark step does (the second reads what the first wrote).
    Each launch shape (one tile per block; persistent grids of 2048 and
    4096 waves) and store policy is timed over `pairs` pairs; the fastest
    median per mix is the floor."""
    import ctypes

    import torch

    path = os.path.join(ROOT, "kv_cache_quantization_srft_amd", "libsrftq_memfloor.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.srftq_memfloor.restype = ctypes.c_int
    lib.srftq_memfloor.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    assert nvec % 64 == 0
    n_tiles = nvec // 64
    big = torch.empty(n_tiles * 16384, dtype=torch.uint8, device="cuda")
    small = torch.empty(n_tiles * 5120, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    small.fill_(2)
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)

    def launch(mix, nt, grid):
        src, dst = (big, small) if mix == 0 else (small, big)
        rc = lib.srftq_memfloor(mix, nt, src.data_ptr(), dst.data_ptr(), n_tiles, grid, sh)
        if rc != 0:
            raise RuntimeError(f"srftq_memfloor failed: {rc}")

    configs = []
    for grid in (n_tiles, 2048, 4096):
        for nt in (1, 0):
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(pairs)]
            for _ in range(5):
                launch(0, nt, grid)
                launch(1, nt, grid)
            for e in ev:
                e[0].record(stream)
                launch(0, nt, grid)
                e[1].record(stream)
                launch(1, nt, grid)
                e[2].record(stream)
            torch.cuda.synchronize()
            configs.append({"grid": "one tile per block" if grid == n_tiles else f"persistent {grid}",
                            "nontemporal_stores": bool(nt),
                            "quantize_mix": _dist([e[0].elapsed_time(e[1]) for e in ev]),
                            "dequantize_mix": _dist([e[1].elapsed_time(e[2]) for e in ev])})
    del big, small
    bq = min(configs, key=lambda c: c["quantize_mix"]["p50_ms"])
    bd = min(configs, key=lambda c: c["dequantize_mix"]["p50_ms"])
    fq, fd = bq["quantize_mix"]["p50_ms"], bd["dequantize_mix"]["p50_ms"]
    tile_bytes = 21504
    return {
        "what": "kernels that move a launch's bytes (contiguous 64-vector tiles, 16 KiB + 5 KiB) with no "
                "arithmetic, alternating like the benchmark step; fastest launch shape and store policy",
        "quantize_mix_ms": fq, "dequantize_mix_ms": fd,
        "quantize_mix_hbm_frac": tile_bytes * n_tiles / (fq * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "dequantize_mix_hbm_frac": tile_bytes * n_tiles / (fd * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "quantize_frac_of_floor": fq / q_ms, "dequantize_frac_of_floor": fd / dq_ms,
        "best_quantize_mix_shape": {"grid": bq["grid"], "nontemporal_stores": bq["nontemporal_stores"]},
        "best_dequantize_mix_shape": {"grid": bd["grid"], "nontemporal_stores": bd["nontemporal_stores"]},
        "configs": configs,
    }


def _dist(ms_list) -> dict:
    """Per-launch times (ms): mean, median and the 10th / 90th percentiles."""
    import numpy as np
    a = np.asarray(ms_list, dtype=np.float64)
    return {"launches": int(a.size), "mean_ms": float(a.mean()), "p50_ms": float(np.percentile(a, 50)),
            "p10_ms": float(np.percentile(a, 10)), "p90_ms": float(np.percentile(a, 90))}


def _direction(ms_list, nvec, d, bpv) -> dict:
    """Rates of one direction from its per-launch times (median launch)."""
    t = _dist(ms_list)
    sec = t["p50_ms"] * 1e-3
    t.update({"vectors_per_s": nvec / sec, "fp16_GBps": 2 * d * nvec / sec / 1e9,
              "algo_GBps": bpv * nvec / sec / 1e9, "hbm_frac": bpv * nvec / sec / 1e9 / HBM_PEAK_GBPS})
    return t


def rotating_roundtrip(x, s, lam, group, bits, rot, launches: int, sets: int = 4, settle_s: float = 0.5):
    """Quantize and dequantize of x fp16 [B,T,H,d] (device) timed per launch
    with HIP events on the launch stream, over `sets` input / output buffer
    sets used in turn (every launch reads buffers last touched more than a
    last-level cache's worth of traffic earlier): step i quantizes set i %
    sets and dequantizes set (i + sets/2) % sets, written two steps before.
    Returns (quantize ms list, dequantize ms list, reconstruction rel L2)."""
    import torch

    from kv_cache_quantization_srft_amd import srftq as S

    B, T, H, d = x.shape
    xs = [x] + [x.clone() for _ in range(sets - 1)]
    cs = [torch.empty((B, H, T, d * bits // 8), dtype=torch.uint8, device=x.device) for _ in range(sets)]
    ss = [torch.empty((B, H, T, d // group), dtype=torch.float16, device=x.device) for _ in range(sets)]
    os_ = [torch.empty_like(x) for _ in range(sets)]
    q = lambda k: S.quantize(xs[k], s, lam, group, bits, rot, codes=cs[k], scales=ss[k])
    dq = lambda k: S.dequantize(cs[k], ss[k], s, lam, group, bits, rot, out=os_[k])
    for k in range(sets):
        q(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < settle_s or i < 4:
        q(i % sets)
        dq((i + sets // 2) % sets)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(launches)]
    for i in range(launches):
        ev[i][0].record()
        q(i % sets)
        ev[i][1].record()
        dq((i + sets // 2) % sets)
        ev[i][2].record()
    torch.cuda.synchronize()
    tq = [e[0].elapsed_time(e[1]) for e in ev]
    tdq = [e[1].elapsed_time(e[2]) for e in ev]
    xf = x.float()
    rel = (torch.linalg.vector_norm(os_[0].float() - xf) / torch.linalg.vector_norm(xf)).item()
    del xs, cs, ss, os_
    return tq, tdq, rel


def roundtrip_timing(launches: int) -> dict:
    """The round trip at the 128K-token shape: fp16 [T=131072, H=8, d=128],
    Student-t(3) values, SRFT, lambda 1, group 16, int4; each direction
    timed per launch over four rotating buffer sets (1 GiB of inputs)."""
    import torch

    from kv_cache_quantization_srft_amd import workloads as W

    w = W.WORKLOADS["roundtrip"]
    x, s = W.generate(w)
    xd = torch.from_numpy(x).to("cuda:0")              # [1, T, H, d]
    sd = torch.from_numpy(s).to("cuda:0")
    del x
    tq, tdq, rel = rotating_roundtrip(xd, sd, None, w.group, w.bits, "srft", launches)
    bpv = algorithmic_bytes_per_vector(w.d, w.group, w.bits)
    return {"workload": f"roundtrip: fp16 [T={w.T}, H={w.H}, d={w.d}], Student-t(3), SRFT, lambda 1, "
                        f"group {w.group}, int{w.bits}; 4 rotating buffer sets",
            "vectors": w.nvec, "bytes_per_vector": bpv,
            "quantize": _direction(tq, w.nvec, w.d, bpv), "dequantize": _direction(tdq, w.nvec, w.d, bpv),
            "reconstruction_rel_l2": rel}


def wide_timing(launches: int) -> dict:
    """The wide head: fp16 [T=131072, H=4, d=256], lognormal channels with
    sparse x30 outliers, lambda calibrated per rotation, group 16, int4;
    SRFT and SRHT each timed per direction (four rotating buffer sets), with
    the reconstruction error of each (the pages call the two equivalent in
    quality)."""
    import torch

    from kv_cache_quantization_srft_amd import srftq as S
    from kv_cache_quantization_srft_amd import workloads as W

    w = W.WORKLOADS["wide"]
    x, s = W.generate(w)
    xd = torch.from_numpy(x).to("cuda:0")
    sd = torch.from_numpy(s).to("cuda:0")
    del x
    bpv = algorithmic_bytes_per_vector(w.d, w.group, w.bits)
    out = {"workload": f"wide: fp16 [T={w.T}, H={w.H}, d={w.d}], lognormal channels, "
                       f"lambda calibrated, group {w.group}, int{w.bits}; 4 rotating buffer sets",
           "vectors": w.nvec, "bytes_per_vector": bpv}
    for rot in ("srft", "srht"):
        lam = S.calibrate_lambda(xd, sd, rot)
        tq, tdq, rel = rotating_roundtrip(xd, sd, lam, w.group, w.bits, rot, launches)
        out[rot] = {"quantize": _direction(tq, w.nvec, w.d, bpv), "dequantize": _direction(tdq, w.nvec, w.d, bpv),
                    "reconstruction_rel_l2": rel}
    return out


def tiny_timing(launches: int) -> dict:
    """The tiny workload, fp16 [T=1024, H=8, d=128] (8,192 vectors, 2 MiB):
    launch-bound, so microseconds per launch (HIP events), no roofline: the
    plain calls, the prepared ones (Quantizer / Dequantizer) and HIP-graph
    replays."""
    import torch

    from kv_cache_quantization_srft_amd import srftq as S
    from kv_cache_quantization_srft_amd import workloads as W

    w = W.WORKLOADS["tiny"]
    x, s = W.generate(w)
    xd = torch.from_numpy(x).to("cuda:0")
    sd = torch.from_numpy(s).to("cuda:0")
    codes, scales = S.quantize(xd, sd, None, w.group, w.bits)
    xhat = S.dequantize(codes, scales, sd, None, w.group, w.bits)
    for _ in range(50):
        S.quantize(xd, sd, None, w.group, w.bits, codes=codes, scales=scales)
        S.dequantize(codes, scales, sd, None, w.group, w.bits, out=xhat)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(launches)]
    for i in range(launches):
        ev[i][0].record()
        S.quantize(xd, sd, None, w.group, w.bits, codes=codes, scales=scales)
        ev[i][1].record()
        S.dequantize(codes, scales, sd, None, w.group, w.bits, out=xhat)
        ev[i][2].record()
    torch.cuda.synchronize()
    us = lambda a: {k.replace("_ms", "_us"): (v * 1e3 if k.endswith("_ms") else v) for k, v in _dist(a).items()}

    # The prepared calls (arguments checked once, one library call per launch)
    qz = S.Quantizer(xd.shape, codes, scales, sd, None, w.group, w.bits)
    dqz = S.Dequantizer(xhat, sd, None, w.group, w.bits)
    for _ in range(20):
        qz(xd)
        dqz(codes, scales)
    torch.cuda.synchronize()
    evp = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(launches)]
    for i in range(launches):
        evp[i][0].record()
        qz(xd)
        evp[i][1].record()
        dqz(codes, scales)
        evp[i][2].record()
    torch.cuda.synchronize()

    # The same launches captured in HIP graphs (50 of one direction each) and
    # replayed: the device time per launch without the host's per-call work
    # (argument checks, ctypes), which the events above include.
    n_g, reps = 50, max(1, launches // 50)
    codes_g, scales_g, xhat_g = torch.zeros_like(codes), torch.zeros_like(scales), torch.zeros_like(xhat)
    q = lambda: S.quantize(xd, sd, None, w.group, w.bits, codes=codes_g, scales=scales_g)
    dq = lambda: S.dequantize(codes_g, scales_g, sd, None, w.group, w.bits, out=xhat_g)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q()
        dq()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = {}
    for name, f in (("quantize", q), ("dequantize", dq)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n_g):
                f()
        graphs[name] = g
    codes_g.zero_()
    scales_g.zero_()
    xhat_g.zero_()
    torch.cuda.synchronize()
    graph_us = {}
    for name in ("quantize", "dequantize"):
        graphs[name].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graphs[name].replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us[name] = e0.elapsed_time(e1) * 1e3 / (reps * n_g)
    same = bool(torch.equal(codes_g, codes) and torch.equal(scales_g, scales) and torch.equal(xhat_g, xhat))
    return {"workload": f"tiny: fp16 [T={w.T}, H={w.H}, d={w.d}], SRFT, lambda 1, group {w.group}, int{w.bits}",
            "vectors": w.nvec,
            "quantize": us([e[0].elapsed_time(e[1]) for e in ev]),
            "dequantize": us([e[1].elapsed_time(e[2]) for e in ev]),
            "prepared_quantize": us([e[0].elapsed_time(e[1]) for e in evp]),
            "prepared_dequantize": us([e[1].elapsed_time(e[2]) for e in evp]),
            "graph_us_per_launch": graph_us, "graph_launches": reps * n_g,
            "graph_outputs_match_eager": same}


MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix-core peak


def householder_timing(steps: int) -> dict:
    """Quantize + dequantize with a Householder rotation (k = d/2 reflectors
    at d = 256): the 'householder' workload, 52 tensors of fp16 [T=32768,
    H=1, d=256], group 16, int4, one matrix per tensor built on the device
    from the workload's seeded reflectors.  The product is a dense
    contraction on the matrix cores: algorithmic 2 d^2 flops per vector (the
    kernels execute it as 2 (quantize) / 3 (dequantize) fp16 passes)."""
    import torch

    from kv_cache_quantization_srft_amd import srftq as S
    from kv_cache_quantization_srft_amd import workloads as W

    w = W.WORKLOADS["householder"]
    x, s = W.generate(w)
    V = W.reflectors(w)
    dev = torch.device("cuda:0")
    xd = torch.from_numpy(x).to(dev)
    sd = torch.from_numpy(s).to(dev)
    Vd = torch.from_numpy(V).to(dev)
    del x
    Q = S.householder_matrix(Vd)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    S.householder_matrix(Vd, out=Q)
    e1.record()
    torch.cuda.synchronize()
    build_ms = e0.elapsed_time(e1)
    codes, scales = S.quantize_dense(xd, Q, sd, None, w.group, w.bits)
    xhat = S.dequantize_dense(codes, scales, Q, sd, None, w.group, w.bits)
    def pair():
        S.quantize_dense(xd, Q, sd, None, w.group, w.bits, codes=codes, scales=scales)
        S.dequantize_dense(codes, scales, Q, sd, None, w.group, w.bits, out=xhat)
    _settle(pair)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tq = tdq = 0.0
    for _ in range(steps):
        ev[0].record()
        S.quantize_dense(xd, Q, sd, None, w.group, w.bits, codes=codes, scales=scales)
        ev[1].record()
        S.dequantize_dense(codes, scales, Q, sd, None, w.group, w.bits, out=xhat)
        ev[2].record()
        torch.cuda.synchronize()
        tq += ev[0].elapsed_time(ev[1])
        tdq += ev[1].elapsed_time(ev[2])
    rel = (torch.linalg.vector_norm(xhat.float() - xd.float()) / torch.linalg.vector_norm(xd.float())).item()
    del xhat
    # decode attention over these caches read as 26 layers' K (even tensors)
    # and V (odd tensors), each with its own matrix, 8 query heads per KV head
    R = 8
    L = w.B // 2
    kc, vc = codes[0::2].contiguous(), codes[1::2].contiguous()
    ks, vs = scales[0::2].contiguous(), scales[1::2].contiguous()
    sk, sv = sd[0::2].contiguous(), sd[1::2].contiguous()
    Qk, Qv = Q[0::2].contiguous(), Q[1::2].contiguous()
    qa = torch.from_numpy(W.attention_queries(w, R)).to(dev)
    ws = torch.empty((S.srftq_attention_workspace_bytes(S.make_shape(L, w.T, w.H, w.d, w.group, w.bits), R),),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((L, w.H * R, w.d), dtype=torch.float32, device=dev)
    attend = lambda: S.decode_attention_dense(qa, kc, ks, vc, vs, Qk, Qv, sk, None, sv, None, group=w.group,
                                              bits=w.bits, workspace=ws, out=out)
    _settle(attend)
    ta = 0.0
    for _ in range(steps):
        ev[0].record()
        attend()
        ev[1].record()
        torch.cuda.synchronize()
        ta += ev[0].elapsed_time(ev[1])
    attn_ms = ta / steps
    attn_bytes = 2 * L * w.H * w.T * (w.d * w.bits // 8 + 2 * (w.d // w.group))
    n = w.nvec
    q_ms, dq_ms = tq / steps, tdq / steps
    flops = 2.0 * w.d * w.d * n
    bpv = algorithmic_bytes_per_vector(w.d, w.group, w.bits)
    tq_tf, tdq_tf = flops / (q_ms * 1e-3) / 1e12, flops / (dq_ms * 1e-3) / 1e12
    return {"workload": f"householder: {w.B} x fp16 [T={w.T}, H={w.H}, d={w.d}], k={w.reflectors} "
                        f"reflectors per tensor, group {w.group}, int{w.bits}",
            "householder_build_ms": build_ms,
            "quantize_ms": q_ms, "dequantize_ms": dq_ms,
            "vectors_per_s_step": n / ((q_ms + dq_ms) * 1e-3),
            "algorithmic_flops_per_vector": 2 * w.d * w.d,
            "quantize_TFLOPs": tq_tf, "dequantize_TFLOPs": tdq_tf,
            "quantize_mfma_frac": tq_tf / MFMA_F16_PEAK_TFLOPS,
            "dequantize_mfma_frac": tdq_tf / MFMA_F16_PEAK_TFLOPS,
            # fp16 MFMA passes over the product (hi/lo operand parts): groups
            # of 16 and 32 dequantize in two, groups of 8 in three
            "executed_fp16_passes": {"quantize": 2, "dequantize": 2 if w.group >= 16 else 3},
            "quantize_hbm_frac": bpv * n / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "dequantize_hbm_frac": bpv * n / (dq_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "reconstruction_rel_l2": rel,
            "decode_attention": {"step": f"srftq_decode_attention_dense: {L} layers x K+V caches, {R} query "
                                         "heads per KV head, one query token, each cache with its own matrix",
                                 "ms": attn_ms, "algorithmic_bytes": attn_bytes,
                                 "GBps": attn_bytes / (attn_ms * 1e-3) / 1e9,
                                 "hbm_frac": attn_bytes / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="untimed steps for this long before the warmup steps, so the timed "
                         "steps run at the clocks a sustained load settles to")
    ap.add_argument("--workload", default="outlier")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--section-launches", type=int, default=None,
                    help="launches per direction in the roundtrip, wide-head and tiny sections "
                         "(default: max(100, steps)); fewer for profiler passes")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-append, decode-attention and d = 96 figures")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<kernel>_<workload>.json from two rocprofv3 "
                         "counter_collection.csv files of this benchmark, then exit")
    args = ap.parse_args()
    if args.traffic:
        write_traffic(args.traffic[0], args.traffic[1], args.workload)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (every KV vector is "
              "independent, so the path shards by heads or tokens with no exchange)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from kv_cache_quantization_srft_amd import srftq as S
    from kv_cache_quantization_srft_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    t0 = time.perf_counter()
    x, s = W.generate(w)
    gen_s = time.perf_counter() - t0
    dev = torch.device("cuda:0")
    xd = torch.from_numpy(x).to(dev)
    sd = torch.from_numpy(s).to(dev)
    lam = S.calibrate_lambda(xd, sd) if w.calibrated_lambda else None
    torch.cuda.synchronize()
    lam_h = lam.cpu().numpy() if lam is not None else None

    # head-major quantized cache [B, H, T, .], two sets used in turn: step i
    # quantizes the batch into set i % 2 and dequantizes set (i + 1) % 2,
    # which the previous step wrote (2.5 GB of traffic ago, so dequantize
    # reads its codes from HBM, as from a cache written earlier)
    codes2 = [torch.empty((w.B, w.H, w.T, w.d * w.bits // 8), dtype=torch.uint8, device=dev) for _ in range(2)]
    scales2 = [torch.empty((w.B, w.H, w.T, w.d // w.group), dtype=torch.float16, device=dev) for _ in range(2)]
    codes, scales = codes2[0], scales2[0]
    xhat = torch.empty_like(xd)

    def step(i, ev=None, rot="srft"):
        if ev is not None:
            ev[0].record()
        S.quantize(xd, sd, lam, w.group, w.bits, rot, codes=codes2[i % 2], scales=scales2[i % 2])
        if ev is not None:
            ev[1].record()
        S.dequantize(codes2[(i + 1) % 2], scales2[(i + 1) % 2], sd, lam, w.group, w.bits, rot, out=xhat)
        if ev is not None:
            ev[2].record()

    S.quantize(xd, sd, lam, w.group, w.bits, codes=codes2[1], scales=scales2[1])
    # the GPU's clocks need a sustained load to settle (the first ~100 calls of
    # a kernel run up to 15 % slower): untimed steps for settle_s seconds
    t_settle = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(10):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(n_settle + i)
    torch.cuda.synchronize()
    i0 = n_settle + args.warmup
    # the timed steps: one event pair around all of them (events between the
    # launches would add their own records to the step time)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(i0 + i)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    # then the same number of steps with an event pair around each launch,
    # for the per-kernel times and the roofline
    i0 += args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i0 + i, evs[i])
    torch.cuda.synchronize()
    tq = [e[0].elapsed_time(e[1]) for e in evs]
    tdq = [e[1].elapsed_time(e[2]) for e in evs]
    q_ms = sum(tq) / args.steps
    dq_ms = sum(tdq) / args.steps
    ms_step = total_ms / args.steps
    # the last step dequantized the set quantized the step before, from the same x
    rel = (torch.linalg.vector_norm(xhat.float() - xd.float()) / torch.linalg.vector_norm(xd.float())).item()

    nvec = w.nvec
    bpv = algorithmic_bytes_per_vector(w.d, w.group, w.bits)
    per_kernel = {
        "quantize": {"ms": q_ms, "vectors_per_s": nvec / (q_ms * 1e-3),
                     "fp16_GBps": 2 * w.d * nvec / (q_ms * 1e-3) / 1e9,
                     "algo_GBps": bpv * nvec / (q_ms * 1e-3) / 1e9, **_dist(tq)},
        "dequantize": {"ms": dq_ms, "vectors_per_s": nvec / (dq_ms * 1e-3),
                       "fp16_GBps": 2 * w.d * nvec / (dq_ms * 1e-3) / 1e9,
                       "algo_GBps": bpv * nvec / (dq_ms * 1e-3) / 1e9, **_dist(tdq)},
    }
    for k in per_kernel.values():
        k["hbm_frac"] = k["algo_GBps"] / HBM_PEAK_GBPS
    dom = "quantize" if q_ms >= dq_ms else "dequantize"
    traffic = load_traffic(dom, w.name)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": per_kernel[dom]["algo_GBps"],
                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": per_kernel[dom]["algo_GBps"] / HBM_PEAK_GBPS,
                "traffic": traffic,
                "bytes_per_vector": bpv, "vectors_per_launch": nvec}

    # the same kernels with no rotation (rot none: loads, quantizer, stores):
    # the memory path's own floor at this shape, for comparison
    floor = None
    if not args.no_decode:
        fl = max(20, args.steps // 4)
        for i in range(4):
            step(i, rot="none")
        torch.cuda.synchronize()
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(fl)]
        for i in range(fl):
            step(i, fev[i], rot="none")
        torch.cuda.synchronize()
        fq = _dist([e[0].elapsed_time(e[1]) for e in fev])
        fdq = _dist([e[1].elapsed_time(e[2]) for e in fev])
        floor = {"what": "the same workload with rot none: tile loads, lambda, quantizer and stores, "
                         "no transform", "quantize": fq, "dequantize": fdq,
                 "quantize_hbm_frac": bpv * nvec / (fq["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                 "dequantize_hbm_frac": bpv * nvec / (fdq["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        step(0)            # leave set 0 holding the SRFT codes (decode attention reads it)
        torch.cuda.synchronize()

    # the floor kernels move 16 KiB + 5 KiB per 64-vector tile: d = 128, int4, group 16
    mfloor = None
    if not args.no_decode and bpv == 336 and w.d == 128:
        mfloor = memory_floor_timing(nvec, max(50, args.steps // 4), per_kernel["quantize"]["p50_ms"],
                                     per_kernel["dequantize"]["p50_ms"])

    # plain copy kernel of the quantize input's size (fp16 negate: reads and
    # writes 2*d bytes per vector): achievable-bandwidth reference, and the
    # known-size kernel the HBM byte counters are scaled against
    src = xd.view(-1)
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record()
    for _ in range(args.steps):
        torch.neg(src, out=dst)
    c1.record()
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / args.steps
    copy_probe = {"bytes_read": src.numel() * 2, "bytes_written": dst.numel() * 2, "ms": copy_ms,
                  "GBps": 2 * src.numel() * 2 / (copy_ms * 1e-3) / 1e9}
    del dst, src

    del codes2[1], scales2[1]
    dec = None if args.no_decode else decode_append_latency()
    attn = None if args.no_decode else decode_attention_timing(w, codes, scales, sd, lam, args.steps)
    d96 = None if args.no_decode else non_pow2_timing(min(args.steps, 50))
    del xhat
    hh = None if args.no_decode else householder_timing(min(args.steps, 20))
    del xd, codes, scales, codes2, scales2
    torch.cuda.empty_cache()
    launches = args.section_launches or max(100, args.steps)
    c5 = None if args.no_decode else roundtrip_timing(launches)
    c4 = None if args.no_decode else wide_timing(launches)
    tiny = None if args.no_decode else tiny_timing(launches)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, x, s, lam_h)

    out = {
        "metric": "KV vectors/s + fp16-in GB/s (% of HBM peak), SRFT\u2192int4 pack, d=128",
        "value": nvec / (ms_step * 1e-3),
        "unit": "KV vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": n_settle,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded numpy; stands in for LLM KV caches)",
        "config": {"workload": f"{w.name}: {w.B} x fp16 [T={w.T}, H={w.H}, d={w.d}], "
                               f"SRFT, lambda {'calibrated' if w.calibrated_lambda else '1'}, "
                               f"group {w.group}, int{w.bits}",
                   "B": w.B, "T": w.T, "H": w.H, "d": w.d, "group": w.group, "bits": w.bits,
                   "rot": "srft", "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_kernel": per_kernel,
        "copy_probe": copy_probe,
        "fp16_in_GBps_quantize": per_kernel["quantize"]["fp16_GBps"],
        "hbm_peak_frac_quantize": per_kernel["quantize"]["hbm_frac"],
        "hbm_peak_frac_dequantize": per_kernel["dequantize"]["hbm_frac"],
        "step": "srftq_quantize of the batch into one of two code sets, then srftq_dequantize of "
                "the set the previous step wrote (one launch each)",
        "reconstruction_rel_l2": rel,
        "rot_none_floor": floor,
        "memory_floor": mfloor,
        "roundtrip_128k": c5,
        "wide_d256": c4,
        "tiny_launch": tiny,
        "decode_append": dec,
        "decode_attention": attn,
        "non_pow2_d96": d96,
        "householder_d256": hh,
        "device": torch.cuda.get_device_name(0),
        "input_generation_s": gen_s,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
