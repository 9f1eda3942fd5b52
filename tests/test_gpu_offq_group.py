"""GPU parity of OffQ's group-wise offsets (a step and zero point per token
and 128-channel group) against the CPU oracle, through the C ABI.

Activation codes, steps, zero points, group code sums, the transformed values
and the weight column sums per group must match bit for bit; fp16 outputs of
the group-wise W4A4 GEMM must be within the normwise relative tolerance 1e-3
of the oracle's float64 value computed from the same codes.
"""
import numpy as np
import pytest

import synth
from oracle import gemm, layer, quant
from tests.gpu_helpers import assert_close, assert_equal, dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    assert torch.cuda.is_available()
    from outlier_aware_bit_amd import qlin
    return qlin


def _codes(packed, M, K):
    codes = np.empty((M, K), np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    return codes


# K = 8320 is 65 groups: 260 chunks of 32 channels, so the last pass over the
# row has only one live quad of lanes.
@pytest.mark.parametrize("M,K", [(1, 128), (37, 512), (300, 4096), (6, 11008 - 11008 % 128), (3, 8320)])
def test_hadamard_offset_group(q, M, K):
    log(f"hadamard_offset_group M={M} K={K}")
    lin = synth.offq_inputs(M=M, K=K, N=64, seed=70 + M, offset_spread=400.0)
    signs = lin.extra["signs"]
    x = lin.x
    want_q, want_s, want_z, want_rs, want_t = quant.hadamard_offset_int4_group(x, signs)
    q4, ss, zz, rs, t = q.qlin_hadamard_offset_group(dev(x), dev(signs), want_t=True)
    assert_equal(host(t), want_t, "t")
    assert_equal(_codes(host(q4), M, K), want_q, "codes")
    assert_equal(host(ss), want_s, "scale")
    assert_equal(host(zz), want_z, "zero")
    assert_equal(host(rs), want_rs, "rowsum")


def test_hadamard_offset_group_degenerate_groups(q):
    # Zero rows, a token whose every group holds only its first channel (each
    # group constant after the transform: range 0), and a token with one
    # constant group among ordinary ones.
    rng = np.random.default_rng(80)
    K = 512
    x = np.zeros((4, K), np.float16)
    x[1, ::128] = [5.0, -2.5, 300.0, 0.0]
    x[2] = rng.standard_normal(K).astype(np.float16)
    x[2, 128:256] = 0
    x[2, 128] = 7.0
    x[3] = rng.standard_normal(K).astype(np.float16)
    signs = rng.choice(np.array([-1, 1], np.int8), K)
    signs[::128] = 1
    want = quant.hadamard_offset_int4_group(x, signs)
    q4, ss, zz, rs, t = q.qlin_hadamard_offset_group(dev(x), dev(signs), want_t=True)
    assert_equal(_codes(host(q4), 4, K), want[0], "codes")
    assert_equal(host(ss), want[1], "scale")
    assert_equal(host(zz), want[2], "zero")
    assert_equal(host(rs), want[3], "rowsum")
    assert_equal(host(t), want[4], "t")


def test_hadamard_offset_group_empty_and_errors(q):
    import torch
    from outlier_aware_bit_amd import _lib
    x = torch.zeros((0, 256), dtype=torch.float16, device="cuda")
    s = torch.ones(256, dtype=torch.int8, device="cuda")
    q4, ss, zz, rs, _ = q.qlin_hadamard_offset_group(x, s)
    assert q4.shape == (0, 128) and ss.shape == (0, 2)
    with pytest.raises(_lib.QlinError):
        q.qlin_hadamard_offset_group(torch.zeros((2, 256), dtype=torch.float16, device="cuda"), s, block=64)


@pytest.mark.parametrize("K,N", [(256, 64), (1024, 320), (11008 - 11008 % 128, 128)])
def test_weight_colsum_group(q, K, N):
    rng = np.random.default_rng(K + N)
    codes = rng.integers(0, 16, (K, N)).astype(np.uint8)
    got = q.qlin_weight_colsum_group(dev(codes))
    assert_equal(host(got), quant.weight_colsum_group(codes), "colsum_g")


def check_group_sums(got, ref, group=128):
    """The GEMM's int32 sums of every group, got [G, M, N], bit for bit against
    the oracle's raw sums of each group, and -- expanded with the documented
    zero-point terms -- against the oracle's centred sums of each group."""
    qa, qw = ref["qa"], ref["qw"]
    G = qa.shape[1] // group
    assert got.shape == (G, qa.shape[0], qw.shape[1]), got.shape
    _, want_c = gemm.w4a4_group(qa, ref["sa"], ref["za"], qw, ref["sw"], ref["zw"], group, return_acc=True)
    za = ref["za"].astype(np.int64)
    zw = np.asarray(ref["zw"], np.int64)
    for g in range(G):
        ks = slice(g * group, (g + 1) * group)
        assert_equal(got[g], gemm.w4a4_raw(qa[:, ks], qw[ks]).astype(np.int32), f"raw sums of group {g}")
        centred = (got[g].astype(np.int64) - za[:, g][:, None] * ref["colsum_g"][g].astype(np.int64)[None, :]
                   - zw[None, :] * (ref["rowsum"][:, g].astype(np.int64) - group * za[:, g])[:, None])
        assert_equal(centred, want_c[g].astype(np.int64), f"centred sums of group {g}")


GROUP_SHAPES = [(1, 128, 64), (7, 384, 192), (33, 512, 64), (65, 256, 320), (130, 1664, 320),
                (200, 1024, 256), (300, 768, 128), (1000, 512, 1024)]


@pytest.mark.parametrize("M,K,N", GROUP_SHAPES)
def test_gemm_w4a4_group(q, M, K, N):
    # The oracle's own codes go to the GPU GEMM, and the GPU's whole path
    # (transform, group codes, weight codes, GEMM) is checked end to end.
    log(f"w4a4 group M={M} K={K} N={N}")
    lin = synth.offq_inputs(M=M, K=K, N=N, seed=M * 19 + K, offset_spread=400.0)
    signs = lin.extra["signs"]
    x = lin.x
    ref = layer.offq_group_forward(x, lin.w, signs)
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4U, dev(ref["qw"]))
    packed = (ref["qa"][:, 0::2] | (ref["qa"][:, 1::2] << 4)).astype(np.uint8)
    y, acc = q.qlin_gemm_w4a4_group(dev(packed), dev(ref["sa"]), dev(ref["za"]), dev(ref["rowsum"]), w4,
                                    dev(ref["sw"]), dev(ref["zw"]), dev(ref["colsum_g"]), N, want_acc=True)
    assert_close(host(y), ref["y"], "y from oracle codes")
    check_group_sums(host(acc), ref)
    y0, _ = q.qlin_gemm_w4a4_group(dev(packed), dev(ref["sa"]), dev(ref["za"]), dev(ref["rowsum"]), w4,
                                   dev(ref["sw"]), dev(ref["zw"]), dev(ref["colsum_g"]), N)
    assert_equal(host(y0).view(np.uint16), host(y).view(np.uint16), "y with and without the group sums")
    qa4, sa, za, rs, _ = q.qlin_hadamard_offset_group(dev(x), dev(signs))
    cw, sw, zw, _ = q.qlin_quant_weight_offq(dev(lin.w), dev(signs))
    csg = q.qlin_weight_colsum_group(cw)
    y2, _ = q.qlin_gemm_w4a4_group(qa4, sa, za, rs, q.qlin_pack_weight(q.QLIN_LAYOUT_W4U, cw), sw, zw, csg, N)
    assert_close(host(y2), ref["y"], "y end to end")


# 65 groups: three chunks of the zero-point term (the last with one group)
# and two of the staged group constants.  100 groups: three chunks of the
# group constants, the third loaded ahead of the K loop's last, partial
# rotation of stages.
@pytest.mark.parametrize("M,K,N", [(70, 8320, 128), (130, 12800, 192)])
def test_gemm_w4a4_group_many_groups_and_scales(q, M, K, N):
    # Zero points up to 2000 in magnitude and activation steps that jump by
    # 10^3 from one 32-group chunk to the next and fall again, from codes
    # drawn directly, against the oracle's group-wise product.
    G = K // 128
    log(f"w4a4 group from codes M={M} K={K} N={N}")
    rng = np.random.default_rng(2024 + K)
    qa = rng.integers(0, 16, (M, K)).astype(np.uint8)
    qw = rng.integers(0, 16, (K, N)).astype(np.uint8)
    chunk_scale = np.array([1.0, 1e3, 1e-2])[(np.arange(G) // 32) % 3]
    sa = (rng.uniform(0.5, 2.0, (M, G)) * chunk_scale[None, :]).astype(np.float32)
    za = rng.integers(-2000, 2001, (M, G)).astype(np.int32)
    zw = rng.integers(0, 16, N).astype(np.int32)
    rowsum = qa.reshape(M, G, 128).astype(np.int32).sum(axis=2).astype(np.int32)
    colsum = quant.weight_colsum_group(qw)
    y1 = gemm.w4a4_group(qa, sa, za, qw, np.ones(N), zw)
    sw = (1000.0 / np.maximum(np.abs(y1).max(axis=0), 1e-30)).astype(np.float32)
    ref = gemm.w4a4_group(qa, sa, za, qw, sw, zw)
    packed = (qa[:, 0::2] | (qa[:, 1::2] << 4)).astype(np.uint8)
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4U, dev(qw))
    y, acc = q.qlin_gemm_w4a4_group(dev(packed), dev(sa), dev(za), dev(rowsum), w4, dev(sw), dev(zw), dev(colsum), N,
                                    want_acc=True)
    assert_close(host(y), ref, "y")
    y0, _ = q.qlin_gemm_w4a4_group(dev(packed), dev(sa), dev(za), dev(rowsum), w4, dev(sw), dev(zw), dev(colsum), N)
    assert_close(host(y0), ref, "y without the group sums")
    got = host(acc)
    for g in range(G):
        ks = slice(g * 128, (g + 1) * 128)
        assert_equal(got[g], gemm.w4a4_raw(qa[:, ks], qw[ks]).astype(np.int32), f"raw sums of group {g}")


def test_gemm_w4a4_group_one_group_matches_per_token(q):
    # K = 128: one group, so the group-wise GEMM must give the per-token
    # GEMM's output for the same codes (both against the oracle).
    M, K, N = 77, 128, 192
    lin = synth.offq_inputs(M=M, K=K, N=N, seed=90)
    signs = lin.extra["signs"]
    ref = layer.offq_forward(lin.x, lin.w, signs)
    qa4, sa, za, rs, _ = q.qlin_hadamard_offset(dev(lin.x), dev(signs))
    cw, sw, zw, cs = q.qlin_quant_weight_offq(dev(lin.w), dev(signs))
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4U, cw)
    y, _ = q.qlin_gemm_w4a4_group(qa4, sa.reshape(M, 1).contiguous(), za.reshape(M, 1).contiguous(),
                                  rs.reshape(M, 1).contiguous(), w4, sw, zw, cs.reshape(1, N).contiguous(), N)
    assert_close(host(y), ref["y"], "y")


# Code patterns at the ends of the range: every group sum at its largest
# (all codes 15: 128 * 225 = 28800), all zero, and alternating 0 / 15 rows
# against 15 / 0 columns (sums of 0 and of 28800 / 2 side by side).  The
# group-wise product forms each group sum on the fp8 matrix cores (codes read
# as e4m3 values c * 2^-9), exact only if every such sum is; the per-group
# sums are compared bit-exactly.
@pytest.mark.parametrize("pattern", ["all15", "zeros", "alternate"])
def test_gemm_w4a4_group_code_extremes(q, pattern):
    M, K, N = 70, 384, 128
    G = K // 128
    log(f"w4a4 group code extremes {pattern} M={M} K={K} N={N}")
    if pattern == "all15":
        qa = np.full((M, K), 15, np.uint8)
        qw = np.full((K, N), 15, np.uint8)
    elif pattern == "zeros":
        qa = np.zeros((M, K), np.uint8)
        qw = np.zeros((K, N), np.uint8)
    else:
        qa = np.where((np.arange(M)[:, None] + np.arange(K)[None, :] // 128) % 2 == 0, 15, 0).astype(np.uint8)
        qw = np.where((np.arange(N)[None, :] + np.arange(K)[:, None] // 128) % 2 == 0, 0, 15).astype(np.uint8)
    rng = np.random.default_rng(77)
    sa = (rng.uniform(0.5, 2.0, (M, G)) * 1e-3).astype(np.float32)  # |y| well inside fp16
    za = rng.integers(-20, 21, (M, G)).astype(np.int32)
    zw = rng.integers(0, 16, N).astype(np.int32)
    sw = (rng.uniform(0.5, 2.0, N) * 1e-3).astype(np.float32)
    rowsum = qa.reshape(M, G, 128).astype(np.int32).sum(axis=2).astype(np.int32)
    colsum = quant.weight_colsum_group(qw)
    ref = gemm.w4a4_group(qa, sa, za, qw, sw, zw)
    packed = (qa[:, 0::2] | (qa[:, 1::2] << 4)).astype(np.uint8)
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4U, dev(qw))
    y, acc = q.qlin_gemm_w4a4_group(dev(packed), dev(sa), dev(za), dev(rowsum), w4, dev(sw), dev(zw), dev(colsum), N,
                                    want_acc=True)
    got = host(acc)
    for g in range(G):
        ks = slice(g * 128, (g + 1) * 128)
        assert_equal(got[g], gemm.w4a4_raw(qa[:, ks], qw[ks]).astype(np.int32), f"raw sums of group {g}")
    y0, _ = q.qlin_gemm_w4a4_group(dev(packed), dev(sa), dev(za), dev(rowsum), w4, dev(sw), dev(zw), dev(colsum), N)
    assert_equal(host(y0).view(np.uint16), host(y).view(np.uint16), "y with and without the group sums")
    assert_close(host(y), ref, "y")


def test_gemm_w4a4_group_errors(q):
    import torch
    from outlier_aware_bit_amd import _lib
    lib = _lib.load()
    # A misaligned pointer is rejected before any launch.
    buf = torch.zeros(1024, dtype=torch.int32, device="cuda")
    st = _lib.load().qlin_gemm_w4a4_group(buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), buf.data_ptr(),
                                          buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), buf.data_ptr() + 4,
                                          1, 64, 128, buf.data_ptr(), None, None)
    assert st == _lib.QLIN_ERR_ALIGN
    st = lib.qlin_gemm_w4a4_group(buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), buf.data_ptr(),
                                  buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), 1, 64, 100, buf.data_ptr(), None,
                                  None)
    assert st == _lib.QLIN_ERR_SHAPE
    assert lib.qlin_gemm_w4a4_group(None, None, None, None, None, None, None, None, 0, 64, 128, None, None,
                                    None) == 0
