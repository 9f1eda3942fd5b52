"""Whole-layer forward passes composed from the oracle's steps (test
infrastructure only).  Each returns every intermediate the GPU path exposes, so
tests can compare codes, scales and accumulators bit-exactly and the fp16
output within tolerance.
"""
from __future__ import annotations

import numpy as np

from . import gemm, quant, quaff, hadamard  # noqa: F401


def w8a8_forward(x, w):
    """Per-token int8 activations x per-channel int8 weights."""
    q, sa = quant.quant_act_sym_int8(x)
    qw, sw = quant.quant_weight_sym(w, 8)
    acc, y = gemm.w8a8(q, sa, qw, sw.astype(np.float32))
    return dict(q=q, sa=sa, qw=qw, sw=sw, acc=acc, y=y)


def quaff_prepare(w, outliers):
    """Offline: W_int (int8 per channel) of all rows, W_O = fp16 rows of W on O,
    and their row absmax (Quaff notes, "overall framework")."""
    qw, sw = quant.quant_weight_sym(w, 8)
    w_o = np.asarray(w)[np.asarray(outliers, np.int64), :]
    return dict(qw=qw, sw=sw, w_o=w_o, wmax=quaff.weight_row_absmax(w_o))


def quaff_step(x, prep, outliers, s, gamma=0.9):
    """One fine-tuning-step forward: update s from this batch, then quantize
    X * (1/s), run the int8 GEMM and add the sparse compensation term
    (Quaff notes, "overall framework": momentum scaling of the outlier channels,
    then the INT8 forward)."""
    o = np.asarray(outliers, np.int64)
    s_new, r = quaff.momentum_update(x, o, prep["wmax"], gamma, s)
    q, sa = quant.quant_act_sym_int8(x, r)
    acc, y_main = gemm.w8a8(q, sa, prep["qw"], prep["sw"].astype(np.float32))
    comp = quaff.compensation(q[:, o], sa, s_new[o], prep["w_o"])
    return dict(s=s_new, r=r, q=q, sa=sa, acc=acc, y=y_main + comp, comp=comp)


def w4a8_channel_forward(x, w):
    q, sa = quant.quant_act_sym_int8(x)
    q4, sw = quant.quant_weight_sym(w, 4)
    acc, y = gemm.w4a8_channel(q, sa, q4, sw.astype(np.float32))
    return dict(q=q, sa=sa, q4=q4, sw=sw, acc=acc, y=y)


def w4a8_group_forward(x, w, group=128):
    q, sa = quant.quant_act_sym_int8(x)
    q4, sg, sc, rg = quant.quant_weight_group(w, group)
    w8 = quant.requant_group(q4, rg, group)
    acc, y = gemm.w4a8_group(q, sa, w8, sc.astype(np.float32))
    return dict(q=q, sa=sa, q4=q4, sg=sg, sc=sc, rg=rg, w8=w8, acc=acc, y=y)


def offq_forward(x, w, signs, block=128):
    qa, sa, za, rowsum, t = quant.hadamard_offset_int4(x, signs, block)
    qw, sw, zw, colsum = quant.offq_weight(w, signs, block)
    acc, y = gemm.w4a4(qa, sa, za, qw, sw, zw)
    return dict(qa=qa, sa=sa, za=za, rowsum=rowsum, t=t, qw=qw, sw=sw, zw=zw,
                colsum=colsum, acc=acc, y=y)


def offq_group_forward(x, w, signs, block=128):
    """OffQ with group-wise offsets: per-token per-block activation steps and
    zero points, per-channel asymmetric int4 weights."""
    qa, sa, za, rowsum, t = quant.hadamard_offset_int4_group(x, signs, block)
    qw, sw, zw, colsum = quant.offq_weight(w, signs, block)
    y = gemm.w4a4_group(qa, sa, za, qw, sw, zw, block)
    return dict(qa=qa, sa=sa, za=za, rowsum=rowsum, t=t, qw=qw, sw=sw, zw=zw,
                colsum_g=quant.weight_colsum_group(qw, block), y=y)
