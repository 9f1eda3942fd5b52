"""OffQ's concentration step, Top-1 PCA (test infrastructure only).

OffQ ("OffQ: Taming Structured Outliers in LLM Quantization by Offsetting",
methodology, "concentration via Top-1 PCA"): from a calibration set, take per
sequence only the token with the largest L-infinity norm, form the covariance
of these extreme tokens, take its leading eigenvector, and rotate the
activations so that the dominant outlier direction lands in the first channel;
the weights take the inverse rotation, so X W is unchanged.

Readings used here (the page names the steps, not their arithmetic):
* the extreme token of a sequence is argmax_t max_k |x_tk| (fp32 of the fp16
  values), the first such t on ties;
* the covariance is the sample covariance of the S extreme tokens, centred on
  their mean, C = Zc^T Zc / (S - 1), in float64;
* the leading eigenvector v (unit norm) is taken with v_0 <= 0;
* the rotation is the Householder reflection H = I - beta w w^T with
  w = v - e_0, beta = 2 / (w^T w), the plainest orthogonal matrix with H v = e_0:
  x H puts x . v into channel 0.  H is symmetric and its own inverse, so the
  weights become H W;
* rotated activations and weights are rounded once to fp16 from float64.
"""
from __future__ import annotations

import numpy as np


def select_extreme_tokens(x: np.ndarray):
    """x fp16 [S x T x K] -> (idx int32 [S], z fp16 [S x K]): per sequence the
    token with the largest max_k |x| (the first on ties)."""
    x = np.asarray(x)
    S, T, K = x.shape
    linf = np.abs(x.astype(np.float32)).max(axis=2) if K else np.zeros((S, T), np.float32)
    idx = np.argmax(linf, axis=1).astype(np.int32)  # argmax returns the first maximum
    z = x[np.arange(S), idx, :]
    return idx, z


def covariance(z: np.ndarray) -> np.ndarray:
    """Sample covariance of the rows of z (float64, centred, divided by S - 1)."""
    zf = np.asarray(z, np.float64)
    zc = zf - zf.mean(axis=0, keepdims=True)
    return zc.T @ zc / max(1, zf.shape[0] - 1)


def leading_eigvec(z: np.ndarray):
    """Leading eigenvector of covariance(z) with v_0 <= 0, and its eigenvalue."""
    c = covariance(z)
    lam, vecs = np.linalg.eigh(c)
    v = vecs[:, -1].copy()
    if v[0] > 0:
        v = -v
    return v, float(lam[-1])


def householder(v: np.ndarray):
    """w = v - e_0 and beta = 2 / (w^T w) of the reflection with H v = e_0 (v unit, v_0 <= 0)."""
    w = np.asarray(v, np.float64).copy()
    w[0] -= 1.0
    return w, 2.0 / float(w @ w)


def rotate_acts(x: np.ndarray, v: np.ndarray) -> np.ndarray:
    """fp16(x H) for tokens x [M x K]: x - beta (x . w) w^T in float64."""
    w, beta = householder(v)
    xf = np.asarray(x, np.float64)
    return (xf - beta * np.outer(xf @ w, w)).astype(np.float16)


def fold_weight(wt: np.ndarray, v: np.ndarray) -> np.ndarray:
    """fp16(H W) for weights W [K x N]: W - beta w (w^T W) in float64."""
    w, beta = householder(v)
    wf = np.asarray(wt, np.float64)
    return (wf - beta * np.outer(w, w @ wf)).astype(np.float16)
