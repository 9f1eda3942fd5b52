"""Hadamard matrices for OffQ's offsetting step (test infrastructure only).

OffQ ("OffQ: Taming Structured Outliers in LLM Quantization by Offsetting",
methodology, "absorption via offsetting"): a partially random Hadamard matrix H
whose first row is all ones is applied to each group of channels after the
outliers have been concentrated into the group's first channel.  The outlier's
magnitude then becomes the same constant added to every channel of the group.

Reading used here (the page does not spell out the construction): start from
the natural-order Sylvester matrix H_n (H_1 = [1], H_2n = [[H, H], [H, -H]]),
whose row 0 is all ones, and multiply rows 1..n-1 by seeded signs d_i; row 0
keeps d_0 = +1.  So H' = diag(d) H_n, and a row vector x of one group maps to
t = x H' = (x * d) H_n.  H' H'^T = n I, hence the inverse that the weights take
is H'^{-1} = H_n diag(d) / n.
"""
from __future__ import annotations

import numpy as np


def sylvester(n: int) -> np.ndarray:
    """Natural-order Sylvester Hadamard matrix H_n (int64 entries +-1); n a power of two."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def partial_random(signs_block: np.ndarray) -> np.ndarray:
    """H' = diag(d) H_n for one group: row i of H_n times d_i (d_0 must be +1)."""
    d = np.asarray(signs_block, dtype=np.int64)
    if d[0] != 1:
        raise ValueError("the first row must stay all ones (d_0 = +1)")
    return d[:, None] * sylvester(d.size)


def transform_blocks(x: np.ndarray, signs: np.ndarray, block: int = 128) -> np.ndarray:
    """Per token and per group of ``block`` channels: t = x_b H'_b, evaluated exactly.

    x is fp16 [M x K]; the products and sums are done in float64, which is exact
    here (inputs are fp16, so every partial sum is a multiple of 2**-24 below
    128 * 65504 < 2**23 in magnitude, i.e. it needs at most 47 significant
    bits).  Returns float64 [M x K]; the caller rounds once.
    """
    M, K = x.shape
    if K % block:
        raise ValueError("K must be a multiple of the block size")
    xf = x.astype(np.float64)
    out = np.empty((M, K), dtype=np.float64)
    for b in range(K // block):
        sl = slice(b * block, (b + 1) * block)
        hp = partial_random(signs[sl]).astype(np.float64)
        out[:, sl] = xf[:, sl] @ hp
    return out


def inverse_transform_weight(w: np.ndarray, signs: np.ndarray, block: int = 128) -> np.ndarray:
    """W'' = blockdiag(H'_b^{-1}) W with H'^{-1} = H_n diag(d) / n, exactly in float64.

    Then (x H') (H'^{-1} W) = x W, so the layer output is unchanged when the
    activations are transformed and the weights take the inverse.
    """
    K, N = w.shape
    wf = w.astype(np.float64)
    out = np.empty((K, N), dtype=np.float64)
    for b in range(K // block):
        sl = slice(b * block, (b + 1) * block)
        hp = partial_random(signs[sl]).astype(np.float64)
        out[sl, :] = (hp.T @ wf[sl, :]) / block
    return out
