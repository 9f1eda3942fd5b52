"""Quantizers of the outlier-aware linear layer (test infrastructure only).

All code decisions are taken in IEEE float32, one rounding per operation, no
fused multiply-add; ``np.rint`` is round-half-to-even.  Conventions where the
pages are silent (each listed in the design notes as a reading):

* symmetric codes use [-127, 127] for int8 and [-8, 7] for int4;
* a per-token (or per-channel) scale divides once: inv = qmax / a, and every
  element is quantized as rint(v * inv); the stored step is a / qmax;
* an all-zero token or channel has step 0 and codes 0;
* activation steps are fp32; symmetric weight steps are rounded to fp16
  (fp16(fp32(a / qmax))); asymmetric weight steps are fp32.
"""
from __future__ import annotations

import numpy as np

from . import hadamard

F32 = np.float32


def _safe_div(num, den):
    """float32 num / den where den != 0, else 0 (no warnings)."""
    num = np.asarray(num, dtype=F32)
    den = np.asarray(den, dtype=F32)
    out = np.zeros(np.broadcast(num, den).shape, dtype=F32)
    nz = np.broadcast_to(den != 0, out.shape)
    np.divide(np.broadcast_to(num, out.shape), np.broadcast_to(den, out.shape), out=out, where=nz)
    return out


# --------------------------------------------------------------------------
# Activations
# --------------------------------------------------------------------------

def quant_act_sym_int8(x: np.ndarray, r: np.ndarray | None = None):
    """Per-token symmetric int8 activation quantization, optionally of X * r.

    Quaff notes ("key design", decoupled WAQ): the activations are quantized to
    INT8 so the product runs in integer arithmetic; with momentum scaling the
    quantized operand is X-hat = Q(X / s), i.e. X times r = 1/s per channel.
    QQQ ("technical architecture", W4A8 GEMM kernels) quantizes activations to
    8 bits per token.

    For token m: v_k = fp32(x_mk) * r_k; a = max_k |v_k|;
    inv = 127 / a, step = a / 127 (both 0 when a == 0);
    q_mk = clamp(rint(v_k * inv), -127, 127).
    Returns (q int8 [M x K], step fp32 [M]).
    """
    v = np.asarray(x).astype(F32)
    if r is not None:
        v = v * np.asarray(r, dtype=F32)[None, :]
    M = v.shape[0]
    a = np.max(np.abs(v), axis=1) if v.shape[1] else np.zeros(M, F32)
    inv = _safe_div(F32(127), a)
    step = _safe_div(a, F32(127))
    q = np.clip(np.rint(v * inv[:, None]), -127, 127).astype(np.int8)
    return q, step


def quant_act_asym_int4(t: np.ndarray):
    """Per-token asymmetric int4 quantization with an integer zero point.

    OffQ (methodology, "absorption via offsetting"): after the Hadamard step the
    outlier has become a constant offset shared by the group's channels, and the
    offset is absorbed into the zero point z of asymmetric uniform
    quantization.  Range per token is [min, max] of the values themselves (not
    widened to include 0, so the offset lands in z rather than in the step).

    t is fp32 [M x K].  rng = max - min;  inv = 15 / rng, step = rng / 15
    (inv = step = 1 when rng == 0);  z = rint(-min * inv) as int32;
    q = clamp(rint(t * inv) + z, 0, 15);  rowsum = sum_k q.
    Returns (q uint8 [M x K], step fp32 [M], z int32 [M], rowsum int32 [M]).
    """
    t = np.asarray(t, dtype=F32)
    M, K = t.shape
    if K == 0:
        z0 = np.zeros(M, np.int32)
        return np.zeros((M, 0), np.uint8), np.ones(M, F32), z0, z0.copy()
    mn = t.min(axis=1)
    mx = t.max(axis=1)
    rng = (mx - mn).astype(F32)
    zero_rng = rng == 0
    inv = np.where(zero_rng, F32(1), _safe_div(F32(15), rng)).astype(F32)
    step = np.where(zero_rng, F32(1), _safe_div(rng, F32(15))).astype(F32)
    z = np.rint((-mn) * inv).astype(np.int64)
    q = np.rint(t * inv[:, None]).astype(np.int64) + z[:, None]
    q = np.clip(q, 0, 15)
    rowsum = q.sum(axis=1)
    return q.astype(np.uint8), step, z.astype(np.int32), rowsum.astype(np.int32)


def hadamard_offset_int4(x: np.ndarray, signs: np.ndarray, block: int = 128):
    """OffQ activation path: t = x H' per group (exact), rounded once to fp32,
    then per-token asymmetric int4 (see ``quant_act_asym_int4``).

    Returns (q, step, z, rowsum, t32).
    """
    t = hadamard.transform_blocks(x, signs, block).astype(F32)
    q, step, z, rowsum = quant_act_asym_int4(t)
    return q, step, z, rowsum, t


def quant_act_asym_int4_group(t: np.ndarray, group: int = 128):
    """Per-token, per-group asymmetric int4: every group of ``group``
    consecutive channels of a token gets its own step and zero point.

    OffQ (methodology, "grouped implementation"; ablations: group size 128):
    several outlier channels are handled by splitting the channels into groups,
    each group's top outlier is turned into an offset of that group alone, and
    each group's own scale and zero point absorb it.  Within a group the rule is
    the per-token rule of ``quant_act_asym_int4`` (range of the group's own
    values, not widened to 0).

    t fp32 [M x K], K a multiple of ``group``; G = K / group.
    Returns (q uint8 [M x K], step fp32 [M x G], z int32 [M x G],
    rowsum int32 [M x G]) with rowsum[m, g] = sum of the codes of group g.
    """
    t = np.asarray(t, dtype=F32)
    M, K = t.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    q = np.zeros((M, K), np.uint8)
    step = np.zeros((M, G), F32)
    z = np.zeros((M, G), np.int32)
    rowsum = np.zeros((M, G), np.int32)
    for g in range(G):
        cols = slice(g * group, (g + 1) * group)
        q[:, cols], step[:, g], z[:, g], rowsum[:, g] = quant_act_asym_int4(t[:, cols])
    return q, step, z, rowsum


def hadamard_offset_int4_group(x: np.ndarray, signs: np.ndarray, block: int = 128):
    """OffQ's group-wise activation path: the block transform of
    ``hadamard_offset_int4`` (groups = Hadamard blocks), then per-token
    per-group asymmetric int4 (``quant_act_asym_int4_group``).

    Returns (q, step [M x G], z [M x G], rowsum [M x G], t32).
    """
    t = hadamard.transform_blocks(x, signs, block).astype(F32)
    q, step, z, rowsum = quant_act_asym_int4_group(t, block)
    return q, step, z, rowsum, t


# --------------------------------------------------------------------------
# Weights (offline preparation; W is [K x N], channel = output column n)
# --------------------------------------------------------------------------

def _sym_codes(wf: np.ndarray, step16: np.ndarray, lo: int, hi: int) -> np.ndarray:
    s = step16.astype(F32)
    q = np.rint(_safe_div(wf, s))
    q = np.where(s == 0, 0, q)
    return np.clip(q, lo, hi).astype(np.int8)


def quant_weight_sym(w: np.ndarray, bits: int):
    """Symmetric per-output-channel weight quantization (QQQ is symmetric:
    "technical architecture", per-channel W4A8 GEMM; Quaff quantizes the frozen
    weight once to W_int, "overall framework").

    a_n = max_k |W_kn|;  step_n = fp16(fp32(a_n / qmax));
    q = clamp(rint(W / step_n), -qmax-1 (int4) or -127 (int8), qmax)
    with qmax = 127 (8 bits) or 7 (4 bits).  Returns (q int8 [K x N], step fp16 [N]).
    """
    wf = np.asarray(w).astype(F32)
    qmax = {8: 127, 4: 7}[bits]
    lo = -127 if bits == 8 else -8
    a = np.max(np.abs(wf), axis=0)
    step = (a / F32(qmax)).astype(F32).astype(np.float16)
    return _sym_codes(wf, step[None, :], lo, qmax), step


def quant_weight_group(w: np.ndarray, group: int = 128):
    """QQQ per-group int4 weights plus the folded requantization ratio.

    QQQ ("technical architecture", per-group W4A8 GEMM and FusedDequantQuant):
    the group scale divided by the channel scale becomes one factor, so the
    int4 weight is dequantized and requantized to int8 in one multiply.

    s_g = fp16(fp32(max_{k in g} |W_kn|) / 7);  q4 = clamp(rint(W / s_g), -8, 7);
    s_c = fp16(fp32(max_k |W_kn|) / 127);      r_g = fp16(fp32(s_g) / fp32(s_c))
    (r_g = 0 where s_c = 0).  Returns (q4 int8 [K x N], s_g fp16 [K/g x N],
    s_c fp16 [N], r_g fp16 [K/g x N]).
    """
    wf = np.asarray(w).astype(F32)
    K, N = wf.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    wg = wf.reshape(K // group, group, N)
    ag = np.max(np.abs(wg), axis=1)
    sg = (ag / F32(7)).astype(F32).astype(np.float16)
    q4 = _sym_codes(wg, sg[:, None, :], -8, 7).reshape(K, N)
    a = np.max(np.abs(wf), axis=0)
    sc = (a / F32(127)).astype(F32).astype(np.float16)
    rg = _safe_div(sg.astype(F32), sc.astype(F32)[None, :]).astype(np.float16)
    return q4, sg, sc, rg


def requant_group(q4: np.ndarray, rg: np.ndarray, group: int = 128) -> np.ndarray:
    """The fused dequant-quant of one int4 weight, in the fp16 path QQQ uses
    ("technical architecture": INT4 -> FP16, FusedDequantQuant, FP16 -> INT8).

    w8 = clamp(rint(fp16(q4 * r_g)), -127, 127): the product of a 4-bit integer
    and an fp16 ratio is exact in fp32, so this is one fp16 rounding of the
    exact product, then one round-half-even to an integer.
    q4 int8 [K x N], rg fp16 [K/g x N] -> w8 int8 [K x N].
    """
    K, N = q4.shape
    r = np.repeat(np.asarray(rg), group, axis=0).astype(F32)
    with np.errstate(over="ignore"):  # an fp16 overflow gives +-inf, clamped below
        prod16 = (q4.astype(F32) * r).astype(np.float16)
    return np.clip(np.rint(prod16.astype(F32)), -127, 127).astype(np.int8)


def quant_weight_asym(w_transformed: np.ndarray):
    """Per-output-channel asymmetric int4 of already-transformed weights W''.

    The same rules as ``quant_act_asym_int4`` applied over k for each column n:
    values rounded once to fp32, rng = max - min, inv = 15 / rng, step = rng / 15
    (both 1 when rng == 0), zw = rint(-min * inv), qw = clamp(rint(W'' * inv) + zw, 0, 15),
    colsum = sum_k qw.  Returns (qw uint8 [K x N], step fp32 [N], zw int32 [N],
    colsum int32 [N]).
    """
    t = np.asarray(w_transformed).astype(F32)
    q, step, z, s = quant_act_asym_int4(t.T)
    return np.ascontiguousarray(q.T), step, z, s


def offq_weight(w: np.ndarray, signs: np.ndarray, block: int = 128):
    """OffQ weight side: W'' = blockdiag(H'^{-1}) W exactly, then asymmetric int4
    per output channel.  Returns (qw, step, zw, colsum)."""
    return quant_weight_asym(hadamard.inverse_transform_weight(w, signs, block).astype(F32))


def weight_colsum_group(qw: np.ndarray, group: int = 128) -> np.ndarray:
    """Column sums of the weight codes over each group of k:
    colsum_g[g, n] = sum_{k in group g} qw[k, n] (int32 [K/group x N]).  The
    group-wise zero-point correction needs them, since the activation zero
    point changes from one group to the next."""
    qw = np.asarray(qw)
    K, N = qw.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    return qw.astype(np.int64).reshape(K // group, group, N).sum(axis=1).astype(np.int32)
