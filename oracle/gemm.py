"""Integer accumulators and dequantized outputs (test infrastructure only).

Each accumulator is the plain definition acc_mn = sum_k a_mk * b_kn of integer
codes.  It is evaluated as a float64 matrix product of integer-valued arrays,
which is exact because every partial sum is an integer below 2**53 in magnitude
(checked before the product).  Outputs are computed in float64.
"""
from __future__ import annotations

import numpy as np


def exact_int_matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """sum_k a[m,k] * b[k,n] for integer arrays, returned as int64 (exact)."""
    a = np.asarray(a)
    b = np.asarray(b)
    K = a.shape[1]
    if K != b.shape[0]:
        raise ValueError("inner dimensions differ")
    amax = int(np.max(np.abs(a.astype(np.int64)))) if a.size else 0
    bmax = int(np.max(np.abs(b.astype(np.int64)))) if b.size else 0
    if K * amax * bmax >= 2 ** 53:
        raise ValueError("float64 product would not be exact")
    return (a.astype(np.float64) @ b.astype(np.float64)).astype(np.int64)


def w8a8(q: np.ndarray, step_a: np.ndarray, qw: np.ndarray, step_w: np.ndarray):
    """W8A8 (Quaff notes, "key design": INT8 x INT8 with integer accumulation).

    acc = q @ qw (int32);  y = acc * step_a[m] * step_w[n] in float64.
    Returns (acc int32 [M x N], y float64 [M x N]).
    """
    acc = exact_int_matmul(q, qw)
    y = acc.astype(np.float64) * np.asarray(step_a, np.float64)[:, None] \
        * np.asarray(step_w, np.float64)[None, :]
    return acc.astype(np.int32), y


def w4a8_channel(q: np.ndarray, step_a: np.ndarray, q4: np.ndarray, step_w: np.ndarray):
    """QQQ per-channel W4A8 ("technical architecture", per-channel W4A8 GEMM):
    INT4 -> INT8, INT8 GEMM, INT32 -> FP16.  The INT4 -> INT8 step (a left shift
    by 4) multiplies every weight by 16, so the kernel's sum is 16 * acc exactly;
    the accumulator reported here is acc = sum_k q * q4, and y = acc * step_a * step_w.
    """
    return w8a8(q, step_a, q4, step_w)


def w4a8_group(q: np.ndarray, step_a: np.ndarray, w8: np.ndarray, s_c: np.ndarray):
    """QQQ per-group W4A8: after the fused dequant-quant the weight is int8 w8
    with per-channel scale s_c; acc = q @ w8, y = acc * step_a * s_c."""
    return w8a8(q, step_a, w8, s_c)


def w4a4(qa: np.ndarray, step_a: np.ndarray, za: np.ndarray,
         qw: np.ndarray, step_w: np.ndarray, zw: np.ndarray):
    """Asymmetric W4A4 on unsigned codes (OffQ uses uniform 4-bit weights and
    activations with zero points; methodology and "core contributions").

    acc_mn = sum_k (qa_mk - za_m)(qw_kn - zw_n), computed here directly from the
    centred codes; y = acc * step_a[m] * step_w[n] in float64.
    Returns (acc int32, y float64); raises if acc leaves the int32 range.
    """
    ca = qa.astype(np.int64) - np.asarray(za, np.int64)[:, None]
    cw = qw.astype(np.int64) - np.asarray(zw, np.int64)[None, :]
    acc = exact_int_matmul(ca, cw)
    if acc.size and np.max(np.abs(acc)) >= 2 ** 31:
        raise ValueError("W4A4 accumulator exceeds int32")
    y = acc.astype(np.float64) * np.asarray(step_a, np.float64)[:, None] \
        * np.asarray(step_w, np.float64)[None, :]
    return acc.astype(np.int32), y


def w4a4_group(qa: np.ndarray, step_a: np.ndarray, za: np.ndarray,
               qw: np.ndarray, step_w: np.ndarray, zw: np.ndarray, group: int = 128,
               return_acc: bool = False):
    """W4A4 with per-token, per-group activation steps and zero points (OffQ,
    methodology, "grouped implementation"): each group of ``group`` k has its
    own activation step step_a[m, g] and zero za[m, g]; the weights keep one
    step and zero per output channel.

    acc_g[m, n] = sum_{k in g} (qa_mk - za_mg)(qw_kn - zw_n)   (exact integers)
    y[m, n]     = step_w[n] * sum_g step_a[m, g] * acc_g[m, n]  (float64)
    Returns y, or (y, acc int32 [G x M x N]) with ``return_acc``; raises if an
    acc_g leaves the int32 range.
    """
    qa = np.asarray(qa)
    M, K = qa.shape
    N = np.asarray(qw).shape[1]
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    cw = np.asarray(qw, np.int64) - np.asarray(zw, np.int64)[None, :]
    y = np.zeros((M, N), np.float64)
    accs = []
    for g in range(K // group):
        ks = slice(g * group, (g + 1) * group)
        ca = qa[:, ks].astype(np.int64) - np.asarray(za, np.int64)[:, g][:, None]
        acc = exact_int_matmul(ca, cw[ks])
        if acc.size and np.max(np.abs(acc)) >= 2 ** 31:
            raise ValueError("W4A4 group accumulator exceeds int32")
        if return_acc:
            accs.append(acc.astype(np.int32))
        y += acc.astype(np.float64) * np.asarray(step_a, np.float64)[:, g][:, None]
    y = y * np.asarray(step_w, np.float64)[None, :]
    if return_acc:
        return y, np.stack(accs) if accs else np.zeros((0, M, N), np.int32)
    return y


def w4a4_raw(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """raw_mn = sum_k qa_mk * qw_kn on the unsigned codes (int64)."""
    return exact_int_matmul(qa, qw)


def fp16_out(y: np.ndarray) -> np.ndarray:
    """The layer's fp16 output: one round-to-nearest-even of the float64 value."""
    return np.asarray(y, np.float64).astype(np.float16)


def max_abs_rel(y: np.ndarray, y_ref: np.ndarray) -> float:
    """Normwise error max|y - y_ref| / max|y_ref| (0 when both are empty/zero)."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    if y_ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(y_ref)))
    num = float(np.max(np.abs(y - y_ref)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
