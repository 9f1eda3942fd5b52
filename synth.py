"""Seeded synthetic inputs for the outlier-aware quantized linear layer.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic (no quantization, no transform, no scale rule), so both the
CPU oracle and the HIP library can be fed from it without sharing any of the
computation under test.

Every array is drawn from ``numpy.random.default_rng(seed)`` (PCG64) in float32
and rounded once to float16 (round-to-nearest-even) where the layer takes fp16.
The recipes follow the five workloads the layer is measured on:

* tiny W8A8: a few channels scaled x100 (activation outliers about 100x the
  typical channel, as the Quaff notes describe in "research background");
* Quaff q_proj: a fixed 5% outlier channel set whose magnitudes are U[50,150]
  and drift by 5% per step (outlier positions stay fixed, the Quaff notes'
  "Outlier Spatial Stability Hypothesis" in "key design");
* QQQ decode / prefill: N(0,1) tokens with 1% outlier channels x100 and
  N(0, 0.02^2) weights at LLaMA-7B FFN shapes;
* OffQ: after the PCA step the outlier energy sits on the first channel of each
  128-channel group (OffQ "methodology"), modelled as N(200, 20^2) on channel
  128*b and N(0,1) elsewhere; the random signs of the partially random Hadamard
  matrix are drawn here and passed in as data.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

W_STD = 0.02


def _normal16(rng: np.random.Generator, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a.astype(np.float16)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


@dataclass
class Linear:
    """One linear-layer workload: activations X [M x K] and weights W [K x N] (fp16)."""
    x: np.ndarray
    w: np.ndarray
    seed: int
    outliers: np.ndarray | None = None          # sorted int32 channel indices, when planted
    extra: dict = field(default_factory=dict)

    @property
    def shape(self):
        return self.x.shape[0], self.x.shape[1], self.w.shape[1]


def plain_linear(M: int, K: int, N: int, seed: int, n_outliers: int = 0, factor: float = 100.0) -> Linear:
    """X ~ N(0,1) with ``n_outliers`` channels multiplied by ``factor``; W ~ N(0, 0.02^2)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=(M, K), dtype=np.float32)
    o = None
    if n_outliers:
        o = np.sort(rng.choice(K, n_outliers, replace=False)).astype(np.int32)
        x[:, o] *= np.float32(factor)
    w = _normal16(rng, (K, N), W_STD)
    return Linear(x.astype(np.float16), w, seed, o)


def tiny_w8a8(seed: int = 0) -> Linear:
    """X fp16 [16x256] with 8 seeded channels x100; W fp16 [256x128] ~ N(0, 0.02^2)."""
    return plain_linear(16, 256, 128, seed, n_outliers=8)


@dataclass
class QuaffSteps:
    xs: list                 # list of fp16 [M x K] activations, one per fine-tuning step
    w: np.ndarray            # fp16 [K x N]
    outliers: np.ndarray     # sorted int32 [nO]
    magnitudes: list         # fp32 [nO] per step (the drifted outlier magnitudes)
    seed: int


def quaff_steps(M: int = 2048, K: int = 4096, N: int = 4096, n_outliers: int = 205,
                steps: int = 10, drift: float = 0.05, seed: int = 1) -> QuaffSteps:
    """Activations for ``steps`` consecutive steps over a fixed outlier set O.

    Each step draws a fresh N(0,1) base; the outlier columns are scaled by a
    per-channel magnitude that starts at U[50,150] and is multiplied by
    (1 + drift) or (1 - drift), sign drawn per channel per step.
    """
    rng = np.random.default_rng(seed)
    o = np.sort(rng.choice(K, n_outliers, replace=False)).astype(np.int32)
    mag = rng.uniform(50.0, 150.0, size=n_outliers).astype(np.float32)
    w = _normal16(rng, (K, N), W_STD)
    xs, mags = [], []
    for t in range(steps):
        if t > 0:
            sign = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=n_outliers)
            mag = (mag * (np.float32(1.0) + np.float32(drift) * sign)).astype(np.float32)
        base = rng.standard_normal(size=(M, K), dtype=np.float32)
        base[:, o] *= mag
        xs.append(base.astype(np.float16))
        mags.append(mag.copy())
    return QuaffSteps(xs, w, o, mags, seed)


def grad_output(M: int, N: int, seed: int, std: float = 1.0) -> np.ndarray:
    """Upstream gradient dL/dY for a backward pass: N(0, std^2), fp16 [M x N]."""
    rng = np.random.default_rng(seed)
    return _normal16(rng, (M, N), std)


def pca_calibration(S: int = 128, T: int = 512, K: int = 4096, seed: int = 6, planted: int = 2,
                    amp_lo: float = 500.0, amp_hi: float = 1500.0):
    """Calibration sequences with a planted outlier direction: tokens N(0,1)
    fp16 [S x T x K]; in every sequence ``planted`` random tokens get a * u
    added, u one dense random unit direction shared by all sequences and
    a ~ U(amp_lo, amp_hi) per token.  Returns (x, u float64 [K])."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(K)
    u /= np.linalg.norm(u)
    x = rng.standard_normal(size=(S, T, K), dtype=np.float32)
    for s_ in range(S):
        ts = rng.choice(T, planted, replace=False)
        amps = rng.uniform(amp_lo, amp_hi, planted)
        x[s_, ts, :] += (amps[:, None] * u[None, :]).astype(np.float32)
    return x.astype(np.float16), u


def qqq_decode(M: int, K: int = 4096, N: int = 11008, seed: int = 2) -> Linear:
    """Decode / small-batch tokens: N(0,1) with 1% outlier channels x100."""
    return plain_linear(M, K, N, seed, n_outliers=max(1, round(0.01 * K)))


def qqq_prefill(M: int = 4096, K: int = 11008, N: int = 4096, seed: int = 3) -> Linear:
    """Prefill tokens at down_proj shape: N(0,1), no planted outliers."""
    return plain_linear(M, K, N, seed)


def offq_inputs(M: int = 2048, K: int = 4096, N: int = 14336, seed: int = 4, block: int = 128,
                offset_mean: float = 200.0, offset_std: float = 20.0, offset_spread: float = 0.0) -> Linear:
    """OffQ-style activations: channel ``block*b`` ~ N(200, 20^2), others N(0,1).

    With ``offset_spread`` > 0 the mean of channel ``block*b`` is drawn per
    block from U(-offset_spread, offset_spread) instead (one outlier level per
    group, the case of group-wise offsets).
    ``extra['signs']`` holds the int8 +-1 row signs of the partially random
    Hadamard matrix (one per channel; the sign of each block's first row is +1).
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=(M, K), dtype=np.float32)
    heads = np.arange(0, K, block)
    mean = np.float32(offset_mean)
    if offset_spread > 0:
        mean = rng.uniform(-offset_spread, offset_spread, size=heads.size).astype(np.float32)
    x[:, heads] = rng.standard_normal(size=(M, heads.size), dtype=np.float32) * np.float32(offset_std) + mean
    signs = rng.choice(np.array([-1, 1], dtype=np.int8), size=K)
    signs[heads] = 1
    w = _normal16(rng, (K, N), W_STD)
    return Linear(x.astype(np.float16), w, seed, heads.astype(np.int32), {"signs": signs})


# Workload table: the five layer configurations the path is measured on.
WORKLOADS = {
    "tiny_w8a8": dict(M=16, K=256, N=128),
    "quaff_q_proj": dict(M=2048, K=4096, N=4096, n_outliers=205, steps=10, gamma=0.9),
    "qqq_decode": dict(Ms=(1, 16, 64), K=4096, N=11008),
    "qqq_prefill_g128": dict(M=4096, K=11008, N=4096, group=128),
    "offq_w4a4": dict(M=2048, K=4096, N=14336, block=128),
}
