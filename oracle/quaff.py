"""Quaff: sparse outlier compensation and targeted momentum scaling
(test infrastructure only).

Source: "Quaff: Quantized Parameter-Efficient Fine-Tuning under Outlier Spatial
Stability Hypothesis" (paper notes), "key design".
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def weight_row_absmax(w_o: np.ndarray) -> np.ndarray:
    """max_n |W_O[o, n]| per outlier row o (fp32; W is frozen, so once per layer)."""
    w = np.asarray(w_o).astype(F32)
    if w.shape[1] == 0:
        return np.zeros(w.shape[0], F32)
    return np.max(np.abs(w), axis=1)


def momentum_update(x: np.ndarray, outliers: np.ndarray, wmax_o: np.ndarray,
                    gamma: float, s: np.ndarray):
    """One step of targeted momentum scaling on the fixed outlier set O.

    Quaff notes ("key design", targeted momentum scaling):
    s_t = gamma * s_{t-1} + (1 - gamma) * beta, where for an outlier channel i
    beta_i = max(1, sqrt(max|X[:, i]| / max|W_i|)) and beta_i = 1 otherwise.

    Readings: s starts at 1 everywhere and is only ever changed on O, so s = 1
    off O; the column maximum is over the current batch's unscaled tokens; a
    zero weight row (or an empty batch) gives beta = 1.  fp32, one rounding per
    operation: c = max_m |x_mo|; rho = c / wmax; beta = max(1, sqrt(rho));
    s_o = (gamma * s_o) + ((1 - gamma) * beta);  r = 1 / s for every channel.

    Returns (s_new fp32 [K], r fp32 [K]).
    """
    xf = np.asarray(x).astype(F32)
    o = np.asarray(outliers, np.int64)
    g = F32(gamma)
    s_new = np.array(s, dtype=F32, copy=True)
    if o.size:
        cols = xf[:, o]
        c = np.max(np.abs(cols), axis=0) if cols.shape[0] else np.zeros(o.size, F32)
        wmax = np.asarray(wmax_o, F32)
        rho = np.zeros(o.size, F32)
        np.divide(c, wmax, out=rho, where=wmax != 0)
        beta = np.where(wmax != 0, np.maximum(F32(1), np.sqrt(rho)), F32(1)).astype(F32)
        g1 = F32(F32(1) - g)
        s_new[o] = (g * s_new[o]) + (g1 * beta)
    r = (F32(1) / s_new).astype(F32)
    return s_new, r


def compensation(q_o: np.ndarray, step_a: np.ndarray, s_o: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """The sparse compensation term X-hat_{:,O} (s_O - 1) W_O in float64.

    Quaff notes ("key design", decoupled WAQ): Y = X-hat (sW) splits into
    X-hat W + X-hat_{:,O} (s_O - 1) W_O; (s - 1) vanishes off O, so only the
    outlier columns contribute.  X-hat is the quantized activation, so
    X-hat_{m,o} = q_mo * step_a[m]; W_O are the full-precision (fp16) rows of W
    for the channels in O.
    comp_mn = sum_o (q_mo * step_a[m]) * (s_o - 1) * W_O[o, n].
    """
    xo = np.asarray(q_o, np.float64) * np.asarray(step_a, np.float64)[:, None]
    so = np.asarray(s_o, np.float64) - 1.0
    return xo @ (so[:, None] * np.asarray(w_o, np.float64))
