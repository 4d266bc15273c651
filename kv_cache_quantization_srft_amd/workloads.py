"""Seeded synthetic KV-cache workloads.

This module only draws random numbers: it holds none of the quantizer's
arithmetic, and both the GPU path and the CPU oracle take their inputs from
it.  The five workloads mirror the shapes and value statistics of the
workloads the "When Quantization Is Free" pages run on (KV caches of small
LLMs with outlier channels, decode-time appends, 128K-token contexts); the
real model tensors are not available, so these seeded draws stand in for them.

Recipe (numpy PCG64, master seed 20260508 + workload index, one independent
sub-stream per quantity):

  tiny        [T=1024, H=8, d=128]; x ~ N(0,1); per head 4 channels picked
              without replacement are multiplied by 20 for every token;
              lambda = 1; group 16; int4.
  outlier     28 layers x {K, V} = B=56 tensors of [T=32768, H=2, d=128];
              x = N(0,1) * sigma[b,h,c], sigma ~ LogNormal(0, 1) per channel,
              then max(1, round(0.01*H*d)) = 3 (h, c) channels per tensor are
              multiplied by 50; lambda calibrated per rotated coordinate;
              group 16; int4.
  decode      256 sequences x 1 new token per step: [T=256, H=8, d=64] per
              step, 1000 steps (B=1000 when drawn at once);
              x = N(0,1) * sigma[h,c], sigma ~ LogNormal(0,1) fixed over
              steps; lambda = 1; group 32; int8.
  wide        [T=131072, H=4, d=256]; x = N(0,1) * sigma[h,c],
              sigma ~ LogNormal(0,1); round(0.01*H*d) = 10 channels x 30;
              lambda calibrated per rotated coordinate; group 16; int4.
  roundtrip   [T=131072, H=8, d=128]; x ~ Student-t(nu=3); lambda = 1;
              group 16; int4.
  householder the Householder rotation at d = 256 ("When Quantization Is
              Free", Metodologia 3: k = d/2 reflectors at d = 256, the head
              size of Gemma-3 1B, one of the pages' models): 26 layers x
              {K, V} = B=52 tensors of [T=32768, H=1, d=256];
              x = N(0,1) * sigma[b,h,c], sigma ~ LogNormal(0,1),
              round(0.01*H*d) = 3 channels x 30; lambda = 1; group 16;
              int4; per (tensor, head) k = 128 reflector vectors ~ N(0, I)
              in fp32 (``reflectors``), standing in for learned ones.

Signs: one +-1 vector per (tensor, head), int8, drawn uniformly.

Decode-attention queries (``attention_queries``): for a workload whose
tensors are the K and V caches of B/2 layers, one N(0,1) fp16 query token per
layer and query head ([B/2, H*R, d]), from their own sub-stream.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

MASTER_SEED = 20260508

_STREAM = {"x": 1, "signs": 2, "sigma": 3, "outlier": 4, "query": 5, "reflectors": 6}


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    T: int
    H: int
    d: int
    group: int
    bits: int
    values: str                # "normal", "lognormal", "student_t3"
    outlier_per_head: int = 0  # tiny: fixed channels per head
    outlier_frac: float = 0.0  # outlier / wide: fraction of (h, c) channels
    outlier_gain: float = 1.0
    calibrated_lambda: bool = False
    rots: tuple = field(default=("srft",))
    steps: int = 1
    reflectors: int = 0        # householder: reflector vectors per (tensor, head)

    @property
    def seed(self) -> int:
        return MASTER_SEED + self.index

    @property
    def nvec(self) -> int:
        return self.B * self.T * self.H

    def scaled(self, T=None, B=None) -> "Workload":
        """The same recipe at a smaller size (for parity checks)."""
        return replace(self, T=self.T if T is None else T, B=self.B if B is None else B)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 1024, 8, 128, 16, 4, "normal",
                     outlier_per_head=4, outlier_gain=20.0),
    "outlier": Workload("outlier", 1, 56, 32768, 2, 128, 16, 4, "lognormal",
                        outlier_frac=0.01, outlier_gain=50.0, calibrated_lambda=True),
    "decode": Workload("decode", 2, 1, 256, 8, 64, 32, 8, "lognormal", steps=1000),
    "wide": Workload("wide", 3, 1, 131072, 4, 256, 16, 4, "lognormal",
                     outlier_frac=0.01, outlier_gain=30.0, calibrated_lambda=True,
                     rots=("srft", "srht")),
    "roundtrip": Workload("roundtrip", 4, 1, 131072, 8, 128, 16, 4, "student_t3"),
    "householder": Workload("householder", 5, 52, 32768, 1, 256, 16, 4, "lognormal",
                            outlier_frac=0.01, outlier_gain=30.0, rots=(), reflectors=128),
}


def _rng(seed: int, stream: str) -> np.random.Generator:
    return np.random.default_rng([seed, _STREAM[stream]])


def signs(w: Workload, B: int | None = None) -> np.ndarray:
    """int8 +-1 of shape [B, H, d]."""
    B = w.B if B is None else B
    r = _rng(w.seed, "signs")
    bits = r.integers(0, 2, size=(B, w.H, w.d), dtype=np.int8)
    return (1 - 2 * bits).astype(np.int8)


def channel_gain(w: Workload, B: int | None = None) -> np.ndarray:
    """float32 per-(tensor, head, channel) multiplier [B, H, d]."""
    B = w.B if B is None else B
    g = np.ones((B, w.H, w.d), dtype=np.float32)
    if w.values == "lognormal":
        r = _rng(w.seed, "sigma")
        # decode: one sigma per (h, c) shared by every step
        if w.steps > 1:
            g[:] = r.lognormal(0.0, 1.0, size=(1, w.H, w.d)).astype(np.float32)
        else:
            g[:] = r.lognormal(0.0, 1.0, size=(B, w.H, w.d)).astype(np.float32)
    ro = _rng(w.seed, "outlier")
    if w.outlier_per_head:
        for b in range(B):
            for h in range(w.H):
                ch = ro.choice(w.d, size=w.outlier_per_head, replace=False)
                g[b, h, ch] *= w.outlier_gain
    elif w.outlier_frac > 0:
        n = max(1, int(round(w.outlier_frac * w.H * w.d)))
        for b in range(B):
            flat = ro.choice(w.H * w.d, size=n, replace=False)
            g[b].reshape(-1)[flat] *= w.outlier_gain
    return g


def values(w: Workload, B: int | None = None, T: int | None = None,
           chunk: int = 1 << 22) -> np.ndarray:
    """fp16 KV tensor [B, T, H, d], drawn in chunks of tokens."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    r = _rng(w.seed, "x")
    g = channel_gain(w, B)
    out = np.empty((B, T, w.H, w.d), dtype=np.float16)
    per_tok = w.H * w.d
    tstep = max(1, chunk // per_tok)
    for b in range(B):
        for t0 in range(0, T, tstep):
            t1 = min(T, t0 + tstep)
            shape = (t1 - t0, w.H, w.d)
            if w.values == "student_t3":
                v = r.standard_t(3.0, size=shape).astype(np.float32)
            else:
                v = r.standard_normal(size=shape, dtype=np.float32)
            v *= g[b][None]
            out[b, t0:t1] = v.astype(np.float16)
    return out


def reflectors(w: Workload, B: int | None = None) -> np.ndarray:
    """Householder reflector vectors, fp32 [B, H, k, d] ~ N(0, I)."""
    B = w.B if B is None else B
    r = _rng(w.seed, "reflectors")
    return r.standard_normal((B, w.H, w.reflectors, w.d), dtype=np.float32)


def attention_queries(w: Workload, R: int) -> np.ndarray:
    """Decode-step queries for a workload whose B tensors are the K and V
    caches of B/2 layers (K = even tensors, V = odd): fp16 [B/2, H*R, d],
    N(0, 1), one new token per layer and R query heads per KV head."""
    r = _rng(w.seed, "query")
    return r.standard_normal((w.B // 2, w.H * R, w.d)).astype(np.float16)


def generate(w: Workload):
    """(x fp16 [B,T,H,d], signs int8 [B,H,d]) for the workload as sized."""
    return values(w), signs(w)
