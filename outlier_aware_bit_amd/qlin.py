"""Thin PyTorch binding of libqlin: one function per C entry point, same names.

Each function checks dtypes, devices and contiguity, allocates outputs with
torch when the caller does not pass them, and calls the C ABI with raw device
pointers and the current HIP stream.  Every step of the layer runs in the HIP
kernels; nothing here computes.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import QLIN_LAYOUT_W4S, QLIN_LAYOUT_W4U, QLIN_LAYOUT_W8, QLIN_LAYOUT_W8T, QLIN_LAYOUT_WO, QlinError  # noqa: F401


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _req(t, name, dtype, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _opt(t, name, dtype, shape=None):
    return None if t is None else _req(t, name, dtype, shape)


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def qlin_abi_version() -> int:
    return _lib.load().qlin_abi_version()


def qlin_outlier_ld(nO) -> int:
    return int(_lib.load().qlin_outlier_ld(nO))


def qlin_quant_act(x, r=None, O=None, s=None, q=None, scale=None, qO=None, xO=None, want_qO=True,
                   want_xO=None):
    """Per-token symmetric int8 of x (optionally x * r).  With O, also the
    outlier columns qO = q[:, O] and, with s, xO = fp16(q[:, O] * (s[O] - 1)),
    both [M, qlin_outlier_ld(nO)].  Returns (q, scale, qO, xO)."""
    lib = _lib.load()
    _req(x, "x", torch.float16)
    M, K = x.shape
    _opt(r, "r", torch.float32, (K,))
    q = _req(q, "q", torch.int8, (M, K)) if q is not None else _empty((M, K), torch.int8, x)
    scale = _req(scale, "scale", torch.float32, (M,)) if scale is not None else _empty((M,), torch.float32, x)
    nO = 0
    if O is not None:
        _req(O, "O", torch.int32)
        nO = O.numel()
    if nO == 0:
        _lib.check("qlin_quant_act", lib.qlin_quant_act(x.data_ptr(), M, K, _ptr(r), q.data_ptr(),
                                                        scale.data_ptr(), None, 0, None, None, None, _stream()))
        return q, scale, None, None
    ld = qlin_outlier_ld(nO)
    if want_xO is None:
        want_xO = s is not None
    if want_qO or qO is not None:
        qO = _req(qO, "qO", torch.int8, (M, ld)) if qO is not None else _empty((M, ld), torch.int8, x)
    if want_xO or xO is not None:
        _req(s, "s", torch.float32, (K,))
        xO = _req(xO, "xO", torch.float16, (M, ld)) if xO is not None else _empty((M, ld), torch.float16, x)
    _lib.check("qlin_quant_act", lib.qlin_quant_act(x.data_ptr(), M, K, _ptr(r), q.data_ptr(), scale.data_ptr(),
                                                    O.data_ptr(), nO, _ptr(s) if xO is not None else None,
                                                    _ptr(qO), _ptr(xO), _stream()))
    return q, scale, qO, xO


def qlin_hadamard_offset(x, signs, block=128, want_t=False, q4=None, scale=None, zero=None, rowsum=None):
    """OffQ block Hadamard + per-token asymmetric int4.
    Returns (q4 uint8 [M, K/2], scale, zero, rowsum, t or None)."""
    lib = _lib.load()
    _req(x, "x", torch.float16)
    M, K = x.shape
    _req(signs, "signs", torch.int8, (K,))
    q4 = _req(q4, "q4", torch.uint8, (M, K // 2)) if q4 is not None else _empty((M, K // 2), torch.uint8, x)
    scale = _req(scale, "scale", torch.float32, (M,)) if scale is not None else _empty((M,), torch.float32, x)
    zero = _req(zero, "zero", torch.int32, (M,)) if zero is not None else _empty((M,), torch.int32, x)
    rowsum = _req(rowsum, "rowsum", torch.int32, (M,)) if rowsum is not None else _empty((M,), torch.int32, x)
    t = _empty((M, K), torch.float32, x) if want_t else None
    _lib.check("qlin_hadamard_offset", lib.qlin_hadamard_offset(
        x.data_ptr(), M, K, signs.data_ptr(), block, q4.data_ptr(), scale.data_ptr(), zero.data_ptr(),
        rowsum.data_ptr(), _ptr(t), _stream()))
    return q4, scale, zero, rowsum, t


def qlin_hadamard_offset_group(x, signs, block=128, want_t=False, q4=None, scale=None, zero=None, rowsum=None):
    """OffQ block Hadamard + asymmetric int4 with a step and zero point per
    token and group of ``block`` channels.
    Returns (q4 uint8 [M, K/2], scale [M, G], zero [M, G], rowsum [M, G], t or None)."""
    lib = _lib.load()
    _req(x, "x", torch.float16)
    M, K = x.shape
    G = K // block if block else 0
    _req(signs, "signs", torch.int8, (K,))
    q4 = _req(q4, "q4", torch.uint8, (M, K // 2)) if q4 is not None else _empty((M, K // 2), torch.uint8, x)
    scale = _req(scale, "scale", torch.float32, (M, G)) if scale is not None else _empty((M, G), torch.float32, x)
    zero = _req(zero, "zero", torch.int32, (M, G)) if zero is not None else _empty((M, G), torch.int32, x)
    rowsum = _req(rowsum, "rowsum", torch.int32, (M, G)) if rowsum is not None else _empty((M, G), torch.int32, x)
    t = _empty((M, K), torch.float32, x) if want_t else None
    _lib.check("qlin_hadamard_offset_group", lib.qlin_hadamard_offset_group(
        x.data_ptr(), M, K, signs.data_ptr(), block, q4.data_ptr(), scale.data_ptr(), zero.data_ptr(),
        rowsum.data_ptr(), _ptr(t), _stream()))
    return q4, scale, zero, rowsum, t


def qlin_momentum_work_bytes(M, nO) -> int:
    return int(_lib.load().qlin_momentum_work_bytes(M, nO))


def qlin_momentum_update(x, O, wmax_O, gamma, s, r, work=None):
    """One step of Quaff's momentum scaling; updates s in place and writes r.
    work: a device workspace (float32) of at least qlin_momentum_work_bytes(M, nO)
    bytes for the two-launch form, or None for the single-launch form."""
    lib = _lib.load()
    _req(x, "x", torch.float16)
    M, K = x.shape
    _req(O, "O", torch.int32)
    nO = O.numel()
    _req(wmax_O, "wmax_O", torch.float32, (nO,))
    _req(s, "s", torch.float32, (K,))
    _req(r, "r", torch.float32, (K,))
    if work is not None:
        _req(work, "work", torch.float32)
        need = qlin_momentum_work_bytes(M, nO)
        if work.numel() * 4 < need:
            raise ValueError(f"work holds {work.numel() * 4} bytes, {need} needed")
    _lib.check("qlin_momentum_update", lib.qlin_momentum_update(
        x.data_ptr(), M, K, O.data_ptr() if nO else None, nO, wmax_O.data_ptr() if nO else None,
        float(gamma), s.data_ptr(), r.data_ptr(), _ptr(work), _stream()))
    return s, r


def qlin_quaff_momentum_quant_work_bytes(M, nO) -> int:
    return int(_lib.load().qlin_quaff_momentum_quant_work_bytes(M, nO))


def qlin_quaff_momentum_quant(x, O, wmax_O, gamma, s, r, work=None, q=None, scale=None, xO=None):
    """Quaff's momentum update (s in place, r written), then the per-token
    int8 of x * r and xO = fp16(q[:, O] * (s[O] - 1)) with the new s and r.
    work: a float32 device workspace of at least
    qlin_quaff_momentum_quant_work_bytes(M, nO) bytes, or None.
    Returns (q, scale, xO)."""
    lib = _lib.load()
    _req(x, "x", torch.float16)
    M, K = x.shape
    _req(O, "O", torch.int32)
    nO = O.numel()
    _req(wmax_O, "wmax_O", torch.float32, (nO,))
    _req(s, "s", torch.float32, (K,))
    _req(r, "r", torch.float32, (K,))
    q = _req(q, "q", torch.int8, (M, K)) if q is not None else _empty((M, K), torch.int8, x)
    scale = _req(scale, "scale", torch.float32, (M,)) if scale is not None else _empty((M,), torch.float32, x)
    if nO:
        ld = qlin_outlier_ld(nO)
        xO = _req(xO, "xO", torch.float16, (M, ld)) if xO is not None else _empty((M, ld), torch.float16, x)
    else:
        xO = None
    if work is not None:
        _req(work, "work", torch.float32)
        need = qlin_quaff_momentum_quant_work_bytes(M, nO)
        if work.numel() * 4 < need:
            raise ValueError(f"work holds {work.numel() * 4} bytes, {need} needed")
    _lib.check("qlin_quaff_momentum_quant", lib.qlin_quaff_momentum_quant(
        x.data_ptr(), M, K, O.data_ptr() if nO else None, nO, wmax_O.data_ptr() if nO else None, float(gamma),
        s.data_ptr(), r.data_ptr(), _ptr(work), q.data_ptr(), scale.data_ptr(), _ptr(xO), _stream()))
    return q, scale, xO


def qlin_weight_row_absmax(w_rows, out=None):
    lib = _lib.load()
    _req(w_rows, "w_rows", torch.float16)
    R, N = w_rows.shape
    out = out if out is not None else _empty((R,), torch.float32, w_rows)
    _req(out, "out", torch.float32, (R,))
    _lib.check("qlin_weight_row_absmax", lib.qlin_weight_row_absmax(
        w_rows.data_ptr() if R else None, R, N, out.data_ptr() if R else None, _stream()))
    return out


def qlin_quant_weight_sym(w, bits):
    lib = _lib.load()
    _req(w, "w", torch.float16)
    K, N = w.shape
    codes = _empty((K, N), torch.int8, w)
    scale = _empty((N,), torch.float16, w)
    _lib.check("qlin_quant_weight_sym", lib.qlin_quant_weight_sym(
        w.data_ptr(), K, N, bits, codes.data_ptr(), scale.data_ptr(), _stream()))
    return codes, scale


def qlin_quant_weight_group(w, group=128):
    lib = _lib.load()
    _req(w, "w", torch.float16)
    K, N = w.shape
    codes = _empty((K, N), torch.int8, w)
    gs = _empty((K // group, N), torch.float16, w)
    cs = _empty((N,), torch.float16, w)
    ratio = _empty((K // group, N), torch.float16, w)
    _lib.check("qlin_quant_weight_group", lib.qlin_quant_weight_group(
        w.data_ptr(), K, N, group, codes.data_ptr(), gs.data_ptr(), cs.data_ptr(), ratio.data_ptr(), _stream()))
    return codes, gs, cs, ratio


def qlin_quant_weight_offq(w, signs, block=128):
    lib = _lib.load()
    _req(w, "w", torch.float16)
    K, N = w.shape
    _req(signs, "signs", torch.int8, (K,))
    codes = _empty((K, N), torch.uint8, w)
    scale = _empty((N,), torch.float32, w)
    zero = _empty((N,), torch.int32, w)
    colsum = _empty((N,), torch.int32, w)
    _lib.check("qlin_quant_weight_offq", lib.qlin_quant_weight_offq(
        w.data_ptr(), K, N, signs.data_ptr(), block, codes.data_ptr(), scale.data_ptr(), zero.data_ptr(),
        colsum.data_ptr(), _stream()))
    return codes, scale, zero, colsum


def qlin_weight_colsum_group(codes, group=128):
    """Column sums of uint8 weight codes [K, N] over each group of ``group`` k: int32 [K/group, N]."""
    lib = _lib.load()
    _req(codes, "codes", torch.uint8)
    K, N = codes.shape
    out = _empty((K // group if group else 0, N), torch.int32, codes)
    _lib.check("qlin_weight_colsum_group", lib.qlin_weight_colsum_group(
        codes.data_ptr(), K, N, group, out.data_ptr(), _stream()))
    return out


def qlin_packed_bytes(layout, K, N) -> int:
    return int(_lib.load().qlin_packed_bytes(layout, K, N))


def qlin_pack_weight(layout, codes, out=None):
    """Pack weights (int8 codes for W8/W4S/W8T, uint8 for W4U, fp16 rows for WO)."""
    lib = _lib.load()
    dt = {QLIN_LAYOUT_W4U: torch.uint8, QLIN_LAYOUT_WO: torch.float16}.get(layout, torch.int8)
    _req(codes, "codes", dt)
    K, N = codes.shape
    nbytes = qlin_packed_bytes(layout, K, N)
    out = out if out is not None else _empty((nbytes,), torch.uint8, codes)
    _req(out, "packed", torch.uint8, (nbytes,))
    _lib.check("qlin_pack_weight", lib.qlin_pack_weight(layout, codes.data_ptr(), K, N, out.data_ptr(), _stream()))
    return out


def qlin_gemm_w8a8(qa, sa, w8, sw, N, xO=None, nO=0, WO=None, want_acc=False, y=None):
    """y = fp16(sa * (acc * sw + xO @ W_O)); returns (y, acc or None).
    WO is the packed W_O (qlin_pack_weight(QLIN_LAYOUT_WO, ...)) of nO rows."""
    lib = _lib.load()
    _req(qa, "qa", torch.int8)
    M, K = qa.shape
    _req(sa, "sa", torch.float32, (M,))
    _req(w8, "w8", torch.uint8, (qlin_packed_bytes(QLIN_LAYOUT_W8, K, N),))
    _req(sw, "sw", torch.float16, (N,))
    if nO:
        _req(xO, "xO", torch.float16, (M, qlin_outlier_ld(nO)))
        _req(WO, "WO", torch.uint8, (qlin_packed_bytes(QLIN_LAYOUT_WO, nO, N),))
    else:
        xO = WO = None
    y = y if y is not None else _empty((M, N), torch.float16, qa)
    _req(y, "y", torch.float16, (M, N))
    acc = _empty((M, N), torch.int32, qa) if want_acc else None
    _lib.check("qlin_gemm_w8a8", lib.qlin_gemm_w8a8(
        qa.data_ptr(), sa.data_ptr(), w8.data_ptr(), sw.data_ptr(), M, N, K, _ptr(xO), nO, _ptr(WO),
        y.data_ptr(), _ptr(acc), _stream()))
    return y, acc


def qlin_gemm_w4a8_work_bytes(M, N, K, group) -> int:
    return int(_lib.load().qlin_gemm_w4a8_work_bytes(M, N, K, group))


def qlin_gemm_w4a8(qa, sa, w4, sw, N, ratio=None, group=0, want_acc=False, y=None, work=None):
    """W4A8 per channel (group=0) or per group of 128 (group=128); returns (y, acc or None).
    work: an optional device workspace (uint8) of at least
    qlin_gemm_w4a8_work_bytes(M, N, K, group) bytes; with it, the per-group
    form requantizes the weights once per call instead of in every tile."""
    lib = _lib.load()
    _req(qa, "qa", torch.int8)
    M, K = qa.shape
    _req(sa, "sa", torch.float32, (M,))
    _req(w4, "w4", torch.uint8, (qlin_packed_bytes(QLIN_LAYOUT_W4S, K, N),))
    _req(sw, "sw", torch.float16, (N,))
    if group:
        _req(ratio, "ratio", torch.float16, (K // group, N))
    y = y if y is not None else _empty((M, N), torch.float16, qa)
    _req(y, "y", torch.float16, (M, N))
    acc = _empty((M, N), torch.int32, qa) if want_acc else None
    need = qlin_gemm_w4a8_work_bytes(M, N, K, group)
    if work is not None and need:
        _req(work, "work", torch.uint8)
        if work.numel() < need:
            raise ValueError(f"work: {work.numel()} bytes, needs {need}")
    else:
        work = None
    _lib.check("qlin_gemm_w4a8", lib.qlin_gemm_w4a8(
        qa.data_ptr(), sa.data_ptr(), w4.data_ptr(), sw.data_ptr(), _ptr(ratio) if group else None, group, M, N, K,
        y.data_ptr(), _ptr(acc), _ptr(work), _stream()))
    return y, acc


def qlin_gemm_w4a4(qa4, sa, za, rowsum, w4, sw, zw, colsum, N, want_acc=False, y=None):
    lib = _lib.load()
    _req(qa4, "qa4", torch.uint8)
    M, K2 = qa4.shape
    K = 2 * K2
    for t, n, d, sh in [(sa, "sa", torch.float32, (M,)), (za, "za", torch.int32, (M,)),
                        (rowsum, "rowsum", torch.int32, (M,)), (sw, "sw", torch.float32, (N,)),
                        (zw, "zw", torch.int32, (N,)), (colsum, "colsum", torch.int32, (N,))]:
        _req(t, n, d, sh)
    _req(w4, "w4", torch.uint8, (qlin_packed_bytes(QLIN_LAYOUT_W4U, K, N),))
    y = y if y is not None else _empty((M, N), torch.float16, qa4)
    _req(y, "y", torch.float16, (M, N))
    acc = _empty((M, N), torch.int32, qa4) if want_acc else None
    _lib.check("qlin_gemm_w4a4", lib.qlin_gemm_w4a4(
        qa4.data_ptr(), sa.data_ptr(), za.data_ptr(), rowsum.data_ptr(), w4.data_ptr(), sw.data_ptr(), zw.data_ptr(),
        colsum.data_ptr(), M, N, K, y.data_ptr(), _ptr(acc), _stream()))
    return y, acc


def qlin_gemm_w4a4_group(qa4, sa, za, rowsum, w4, sw, zw, colsum_g, N, want_acc=False, y=None):
    """W4A4 with a step, zero point and code sum per token and 128-k group
    (sa, za, rowsum [M, K/128]) and per-channel weights (colsum_g [K/128, N]).
    Returns (y, acc); acc is the int32 raw sums of every group [K/128, M, N]
    when want_acc, else None."""
    lib = _lib.load()
    _req(qa4, "qa4", torch.uint8)
    M, K2 = qa4.shape
    K = 2 * K2
    G = K // 128
    for t, n, d, sh in [(sa, "sa", torch.float32, (M, G)), (za, "za", torch.int32, (M, G)),
                        (rowsum, "rowsum", torch.int32, (M, G)), (sw, "sw", torch.float32, (N,)),
                        (zw, "zw", torch.int32, (N,)), (colsum_g, "colsum_g", torch.int32, (G, N))]:
        _req(t, n, d, sh)
    _req(w4, "w4", torch.uint8, (qlin_packed_bytes(QLIN_LAYOUT_W4U, K, N),))
    y = y if y is not None else _empty((M, N), torch.float16, qa4)
    _req(y, "y", torch.float16, (M, N))
    acc = _empty((G, M, N), torch.int32, qa4) if want_acc else None
    _lib.check("qlin_gemm_w4a4_group", lib.qlin_gemm_w4a4_group(
        qa4.data_ptr(), sa.data_ptr(), za.data_ptr(), rowsum.data_ptr(), w4.data_ptr(), sw.data_ptr(), zw.data_ptr(),
        colsum_g.data_ptr(), M, N, K, y.data_ptr(), _ptr(acc), _stream()))
    return y, acc


def qlin_quaff_backward(dy, sw, w8t, s, r, K, O=None, w_o=None, want_acc=False, dx=None, gq=None, gs=None, cb=None):
    """STE input gradient of the Quaff layer: dX [M, K] (fp16).  w8t is the
    int8 weight packed with QLIN_LAYOUT_W8T, w_o the fp16 rows W[O].
    Returns (dx, gq, gs, cb or None, acc or None); cb = dY W_O^T [M, qlin_outlier_ld(nO)]."""
    lib = _lib.load()
    _req(dy, "dy", torch.float16)
    M, N = dy.shape
    _req(sw, "sw", torch.float16, (N,))
    _req(w8t, "w8t", torch.uint8, (qlin_packed_bytes(QLIN_LAYOUT_W8T, K, N),))
    _req(s, "s", torch.float32, (K,))
    _req(r, "r", torch.float32, (K,))
    nO = 0 if O is None else O.numel()
    if nO:
        _req(O, "O", torch.int32, (nO,))
        _req(w_o, "w_o", torch.float16, (nO, N))
        ld = qlin_outlier_ld(nO)
        cb = _req(cb, "cb", torch.float32, (M, ld)) if cb is not None else _empty((M, ld), torch.float32, dy)
    else:
        O = w_o = cb = None
    gq = _req(gq, "gq", torch.int8, (M, N)) if gq is not None else _empty((M, N), torch.int8, dy)
    gs = _req(gs, "gs", torch.float32, (M,)) if gs is not None else _empty((M,), torch.float32, dy)
    dx = _req(dx, "dx", torch.float16, (M, K)) if dx is not None else _empty((M, K), torch.float16, dy)
    acc = _empty((M, K), torch.int32, dy) if want_acc else None
    _lib.check("qlin_quaff_backward", lib.qlin_quaff_backward(
        dy.data_ptr(), M, N, K, sw.data_ptr(), w8t.data_ptr(), s.data_ptr(), r.data_ptr(), _ptr(O), nO, _ptr(w_o),
        gq.data_ptr(), gs.data_ptr(), _ptr(cb), dx.data_ptr(), _ptr(acc), _stream()))
    return dx, gq, gs, cb, acc


def qlin_outlier_comp(xO, sa, nO, WO, y):
    """y += sa * (xO @ W_O), in place (WO packed, nO rows)."""
    lib = _lib.load()
    _req(y, "y", torch.float16)
    M, N = y.shape
    if nO:
        _req(xO, "xO", torch.float16, (M, qlin_outlier_ld(nO)))
        _req(sa, "sa", torch.float32, (M,))
        _req(WO, "WO", torch.uint8, (qlin_packed_bytes(QLIN_LAYOUT_WO, nO, N),))
    _lib.check("qlin_outlier_comp", lib.qlin_outlier_comp(
        _ptr(xO) if nO else None, _ptr(sa) if nO else None, nO, _ptr(WO) if nO else None, M, N,
        y.data_ptr(), _stream()))
    return y


# ---------------------------------------------------------------- OffQ Top-1 PCA (offline)
def qlin_pca_select(x):
    """x fp16 [S, T, K] -> (idx int32 [S], z fp16 [S, K]): each sequence's most extreme token."""
    lib = _lib.load()
    _req(x, "x", torch.float16)
    S, T, K = x.shape
    idx = _empty((S,), torch.int32, x)
    z = _empty((S, K), torch.float16, x)
    _lib.check("qlin_pca_select", lib.qlin_pca_select(x.data_ptr(), S, T, K, idx.data_ptr(), z.data_ptr(),
                                                      _stream()))
    return idx, z


def qlin_pca_leading_eigvec(z, max_iter=200, tol=1e-12):
    """Leading eigenvector of the extreme tokens' covariance: (v float64 [K], lambda, iterations)."""
    lib = _lib.load()
    _req(z, "z", torch.float16)
    S, K = z.shape
    v = _empty((K,), torch.float64, z)
    lam = _empty((1,), torch.float64, z)
    its = _empty((1,), torch.int32, z)
    ws = _empty((S * S + K + S + 1,), torch.float64, z)
    _lib.check("qlin_pca_leading_eigvec", lib.qlin_pca_leading_eigvec(
        z.data_ptr(), S, K, max_iter, tol, v.data_ptr(), lam.data_ptr(), its.data_ptr(), ws.data_ptr(), _stream()))
    return v, lam, its


def qlin_pca_fold_weight(w, v):
    """fp16(H W) for the Householder reflection with H v = e_0."""
    lib = _lib.load()
    _req(w, "w", torch.float16)
    K, N = w.shape
    _req(v, "v", torch.float64, (K,))
    out = _empty((K, N), torch.float16, w)
    ws = _empty((N,), torch.float64, w)
    _lib.check("qlin_pca_fold_weight", lib.qlin_pca_fold_weight(w.data_ptr(), K, N, v.data_ptr(), out.data_ptr(),
                                                                ws.data_ptr(), _stream()))
    return out


def qlin_pca_rotate(x, v):
    """fp16(x H) for tokens x [M, K]."""
    lib = _lib.load()
    _req(x, "x", torch.float16)
    M, K = x.shape
    _req(v, "v", torch.float64, (K,))
    out = _empty((M, K), torch.float16, x)
    _lib.check("qlin_pca_rotate", lib.qlin_pca_rotate(x.data_ptr(), M, K, v.data_ptr(), out.data_ptr(), _stream()))
    return out
