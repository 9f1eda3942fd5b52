"""Quaff: sparse outlier compensation and targeted momentum scaling
(test infrastructure only).

Source: "Quaff: Quantized Parameter-Efficient Fine-Tuning under Outlier Spatial
Stability Hypothesis" (paper notes), "key design".
"""
from __future__ import annotations

import numpy as np

from . import gemm, quant

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


def ste_backward_exact(dy: np.ndarray, qw: np.ndarray, sw: np.ndarray, s: np.ndarray, r: np.ndarray,
                       outliers: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """Input gradient of the layer under the straight-through estimator, in
    float64 (Quaff notes, "loss function / training strategy": standard STE
    for backpropagation; the forward is the decoupled form of "key design").

    The forward is Y = X-hat W-hat + X-hat_{:,O} (s_O - 1) W_O with
    X-hat = Q(X * r), W-hat = W_int * sw (per output channel n).  STE passes the
    gradient through Q unchanged, so dX-hat/dX = diag(r) and
      dX = (dY W-hat^T + scatter_O(dY W_O^T * (s_O - 1))) * r.
    dy [M x N], qw int8 [K x N], sw fp16 [N], s, r fp32 [K], w_o fp16 [nO x N].
    """
    d = np.asarray(dy, np.float64)
    what = np.asarray(qw, np.float64) * np.asarray(sw, np.float64)[None, :]
    g = d @ what.T
    o = np.asarray(outliers, np.int64)
    if o.size:
        g[:, o] += (d @ np.asarray(w_o, np.float64).T) * (np.asarray(s, np.float64)[o] - 1.0)[None, :]
    return g * np.asarray(r, np.float64)[None, :]


def ste_backward(dy: np.ndarray, qw: np.ndarray, sw: np.ndarray, s: np.ndarray, r: np.ndarray,
                 outliers: np.ndarray, w_o: np.ndarray):
    """The STE input gradient with the main product on int8 codes.

    The weight step sw[n] lies along the reduction of dY W-hat^T, so it moves
    to the gradient: G = dY * sw (fp32, one rounding), quantized per token by
    the rule of the forward activations (symmetric int8, step gs[m]).  Then
      acc[m, k] = sum_n gq[m, n] * W_int[k, n]                (exact int32)
      cb[m, j]  = sum_n dY[m, n] * W_O[j, n]                   (float64)
      dX[m, k]  = r_k * (gs[m] * acc[m, k] + [k = O_j] (s_k - 1) * cb[m, j])
    Returns dict(gq, gs, acc, cb, dx) with dx in float64.
    """
    gq, gs = quant.quant_act_sym_int8(dy, np.asarray(sw).astype(F32))
    acc = gemm.exact_int_matmul(gq, np.asarray(qw).T)
    if acc.size and np.max(np.abs(acc)) >= 2 ** 31:
        raise ValueError("backward accumulator exceeds int32")
    o = np.asarray(outliers, np.int64)
    d = np.asarray(dy, np.float64)
    cb = d @ np.asarray(w_o, np.float64).T if o.size else np.zeros((d.shape[0], 0))
    main = acc.astype(np.float64) * np.asarray(gs, np.float64)[:, None]
    if o.size:
        main[:, o] += cb * (np.asarray(s, np.float64)[o] - 1.0)[None, :]
    dx = main * np.asarray(r, np.float64)[None, :]
    return dict(gq=gq, gs=gs, acc=acc.astype(np.int32), cb=cb, dx=dx)
