"""GPU parity of every libqlin entry point against the CPU oracle, called through
the C ABI (via the thin binding) on seeded synthetic inputs.

Integer results (codes, zero points, row/column sums, int32 accumulators) and
the fp32 scales, s and r must match bit for bit; fp16 outputs must be within a
normwise relative error of 1e-3 of the oracle's float64 value computed from
the same codes.  Shapes span several tiles with ragged tails (M not a multiple
of the tile, N a multiple of 64 but not of 128, K a multiple of 128 only).
"""
import numpy as np
import pytest

import synth
from oracle import gemm, hadamard, layer, quant, quaff
from tests.gpu_helpers import assert_close, assert_equal, dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    assert torch.cuda.is_available()
    from outlier_aware_bit_amd import qlin
    return qlin


# ------------------------------------------------------------ activations
@pytest.mark.parametrize("M,K,n_out,use_r", [
    (16, 256, 8, False), (1, 4096, 41, False), (37, 384, 3, True), (300, 1024, 10, True),
    (5, 11008, 110, False), (3, 16384 + 2048, 5, True),
])
def test_quant_act(q, M, K, n_out, use_r):
    log(f"quant_act M={M} K={K} r={use_r}")
    lin = synth.plain_linear(M, K, 64, seed=100 + M, n_outliers=n_out)
    r = None
    if use_r:
        r = np.random.default_rng(M).uniform(0.01, 1.5, K).astype(np.float32)
    want_q, want_s = quant.quant_act_sym_int8(lin.x, r)
    O = lin.outliers
    s = np.random.default_rng(K).uniform(1.0, 60.0, K).astype(np.float32)
    qq, ss, qO, xO = q.qlin_quant_act(dev(lin.x), None if r is None else dev(r), dev(O), s=dev(s))
    assert_equal(host(qq), want_q, "q")
    assert_equal(host(ss), want_s, "scale")
    ld = q.qlin_outlier_ld(O.size)
    assert qO.shape == (M, ld) and xO.shape == (M, ld)
    assert_equal(host(qO)[:, :O.size], want_q[:, O], "qO")
    assert np.all(host(qO)[:, O.size:] == 0) and np.all(host(xO)[:, O.size:] == 0)
    # xO is the compensation operand fp16(q * (s - 1)) in fp32 arithmetic.
    want_x = (want_q[:, O].astype(np.float32) * (s[O] - np.float32(1))).astype(np.float16)
    assert_equal(host(xO)[:, :O.size].view(np.uint16), want_x.view(np.uint16), "xO")


def test_quant_act_zero_rows_and_empty(q):
    x = np.zeros((4, 256), np.float16)
    x[2, 7] = -3.0
    qq, ss, _, _ = q.qlin_quant_act(dev(x))
    want_q, want_s = quant.quant_act_sym_int8(x)
    assert_equal(host(qq), want_q, "q")
    assert_equal(host(ss), want_s, "scale")
    import torch
    qq, ss, _, _ = q.qlin_quant_act(torch.zeros((0, 256), dtype=torch.float16, device="cuda"))
    assert qq.shape == (0, 256)


@pytest.mark.parametrize("M,K", [(1, 128), (37, 512), (300, 4096), (6, 11008)])
def test_hadamard_offset(q, M, K):
    log(f"hadamard_offset M={M} K={K}")
    lin = synth.offq_inputs(M=M, K=K, N=64, seed=7 + M)
    signs = lin.extra["signs"]
    want_q, want_s, want_z, want_rs, want_t = quant.hadamard_offset_int4(lin.x, signs)
    q4, ss, zz, rs, t = q.qlin_hadamard_offset(dev(lin.x), dev(signs), want_t=True)
    assert_equal(host(t), want_t, "t")
    packed = host(q4)
    codes = np.empty((M, K), np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    assert_equal(codes, want_q, "codes")
    assert_equal(host(ss), want_s, "scale")
    assert_equal(host(zz), want_z, "zero")
    assert_equal(host(rs), want_rs, "rowsum")


def test_hadamard_offset_constant_tokens(q):
    # Only channel 0 of a single group set: the token is constant after the
    # transform (range 0), the degenerate branch of the quantizer.
    x = np.zeros((3, 128), np.float16)
    x[:, 0] = [5.0, -2.5, 0.0]
    signs = np.ones(128, np.int8)
    want = quant.hadamard_offset_int4(x, signs)
    q4, ss, zz, rs, t = q.qlin_hadamard_offset(dev(x), dev(signs), want_t=True)
    assert_equal(host(t), want[4], "t")
    assert_equal(host(ss), want[1], "scale")
    assert_equal(host(zz), want[2], "zero")
    assert_equal(host(rs), want[3], "rowsum")


# ------------------------------------------------------------ Quaff
# Up to 8300 tokens: one and several passes of a strip's 2048-row loads
# (single launch); with a workspace, from 4096 tokens, the two-launch form:
# 16 row blocks of 256 rows (4096), of ragged ones (5000) and of several
# passes each (8300).  Below 4096 tokens a workspace is not used.
@pytest.mark.parametrize("work", [False, True])
@pytest.mark.parametrize("M,nO", [(300, 51), (1, 1), (0, 4), (64, 0), (513, 7), (2048, 51), (4096, 33),
                                  (5000, 205), (8300, 60)])
def test_momentum_ten_steps(q, M, nO, work):
    import torch
    log(f"momentum M={M} nO={nO} work={work}")
    K = 1024
    d = synth.quaff_steps(M=max(M, 1), K=K, N=64, n_outliers=max(nO, 1), steps=10, seed=3)
    O = d.outliers[:nO]
    wmax = (np.random.default_rng(1).uniform(0.0, 0.1, nO)).astype(np.float32)
    if nO > 1:
        wmax[0] = 0.0
    s_ref = np.ones(K, np.float32)
    s = torch.ones(K, dtype=torch.float32, device="cuda")
    r = torch.empty(K, dtype=torch.float32, device="cuda")
    Od, wd = dev(O.astype(np.int32)), dev(wmax)
    wk = None
    if work:
        nb = q.qlin_momentum_work_bytes(M, nO)
        assert nb == min(16, max(1, -(-M // 128))) * nO * 4
        wk = torch.full((max(nb // 4, 1),), float("nan"), dtype=torch.float32, device="cuda")
    for t in range(10):
        x = d.xs[t][:M]
        s_ref, r_ref = quaff.momentum_update(x, O, wmax, 0.9, s_ref)
        q.qlin_momentum_update(dev(x), Od, wd, 0.9, s, r, work=wk)
        assert_equal(host(s), s_ref, f"s step {t}")
        assert_equal(host(r), r_ref, f"r step {t}")


def test_weight_row_absmax(q):
    w = (np.random.default_rng(2).standard_normal((37, 192)) * 0.02).astype(np.float16)
    w[5] = 0
    assert_equal(host(q.qlin_weight_row_absmax(dev(w))), quaff.weight_row_absmax(w), "wmax")


# ------------------------------------------------------------ weights
@pytest.mark.parametrize("K,N", [(256, 128), (384, 192), (1024, 64)])
def test_weight_quantizers(q, K, N):
    log(f"weights K={K} N={N}")
    rng = np.random.default_rng(K + N)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    w[:, 3] = 0
    w[:128, 5] *= 50
    for bits in (8, 4):
        want_c, want_s = quant.quant_weight_sym(w, bits)
        c, s = q.qlin_quant_weight_sym(dev(w), bits)
        assert_equal(host(c), want_c, f"codes{bits}")
        assert_equal(host(s).view(np.uint16), want_s.view(np.uint16), f"scale{bits}")
    want = quant.quant_weight_group(w, 128)
    got = q.qlin_quant_weight_group(dev(w), 128)
    for g, wv, name in zip(got, want, ["codes", "group_scale", "channel_scale", "ratio"]):
        if wv.dtype == np.float16:
            assert_equal(host(g).view(np.uint16), wv.view(np.uint16), name)
        else:
            assert_equal(host(g), wv, name)
    signs = rng.choice(np.array([-1, 1], np.int8), K)
    signs[::128] = 1
    want = quant.offq_weight(w, signs)
    got = q.qlin_quant_weight_offq(dev(w), dev(signs))
    for g, wv, name in zip(got, want, ["codes", "scale", "zero", "colsum"]):
        assert_equal(host(g), wv, name)


# ------------------------------------------------------------ GEMMs
GEMM_SHAPES = [(1, 256, 128), (7, 384, 192), (16, 256, 128), (33, 512, 64), (64, 1024, 256),
               (65, 256, 192), (100, 384, 320), (128, 512, 128), (129, 256, 64), (200, 384, 320),
               (256, 512, 128), (1000, 512, 1024)]


@pytest.mark.parametrize("M,K,N", GEMM_SHAPES)
def test_gemm_w8a8(q, M, K, N):
    log(f"w8a8 M={M} K={K} N={N}")
    lin = synth.plain_linear(M, K, N, seed=M * 7 + K, n_outliers=3)
    ref = layer.w8a8_forward(lin.x, lin.w)
    codes, sw = q.qlin_quant_weight_sym(dev(lin.w), 8)
    w8 = q.qlin_pack_weight(q.QLIN_LAYOUT_W8, codes)
    qa, sa, _, _ = q.qlin_quant_act(dev(lin.x))
    y, acc = q.qlin_gemm_w8a8(qa, sa, w8, sw, N, want_acc=True)
    assert_equal(host(acc), ref["acc"], "acc")
    assert_close(host(y), ref["y"], "y")


@pytest.mark.parametrize("M,K,N", GEMM_SHAPES)
def test_gemm_w4a8_channel(q, M, K, N):
    log(f"w4a8 channel M={M} K={K} N={N}")
    lin = synth.plain_linear(M, K, N, seed=M * 11 + K, n_outliers=2)
    ref = layer.w4a8_channel_forward(lin.x, lin.w)
    codes, sw = q.qlin_quant_weight_sym(dev(lin.w), 4)
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, codes)
    qa, sa, _, _ = q.qlin_quant_act(dev(lin.x))
    y, acc = q.qlin_gemm_w4a8(qa, sa, w4, sw, N, want_acc=True)
    assert_equal(host(acc), ref["acc"], "acc")
    assert_close(host(y), ref["y"], "y")


def _requant_work(q, M, N, K):
    # A workspace of the size the library asks for, filled with a pattern:
    # its contents on entry must not matter.
    import torch
    nbytes = q.qlin_gemm_w4a8_work_bytes(M, N, K, 128)
    return torch.full((max(nbytes, 16),), 0xA5, dtype=torch.uint8, device="cuda"), nbytes


@pytest.mark.parametrize("work", [False, True])
@pytest.mark.parametrize("M,K,N", GEMM_SHAPES)
def test_gemm_w4a8_group(q, M, K, N, work):
    # With a workspace, above 128 tokens the weights are requantized once per
    # call and the int8 tile runs on them; the result is the same to the bit.
    log(f"w4a8 group M={M} K={K} N={N} work={work}")
    lin = synth.plain_linear(M, K, N, seed=M * 13 + K)
    ref = layer.w4a8_group_forward(lin.x, lin.w)
    codes, gs, cs, ratio = q.qlin_quant_weight_group(dev(lin.w), 128)
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, codes)
    qa, sa, _, _ = q.qlin_quant_act(dev(lin.x))
    buf = None
    if work:
        buf, nbytes = _requant_work(q, M, N, K)
        assert nbytes == (K * N if M > 128 else 0)
    y, acc = q.qlin_gemm_w4a8(qa, sa, w4, cs, N, ratio=ratio, group=128, want_acc=True, work=buf)
    assert_equal(host(acc), ref["acc"], "acc")
    assert_close(host(y), ref["y"], "y")
    if work:
        y0, _ = q.qlin_gemm_w4a8(qa, sa, w4, cs, N, ratio=ratio, group=128)
        assert_equal(host(y), host(y0), "y with and without the workspace")


# The skinny kernels with LDS-staged activations (33..128 tokens) around their
# dispatch edges: 32/33, 64/65, 96/97 and 128 tokens, with K from one
# partial round (K = 128: 2 of a round's 8 or 16 units) to several rounds
# with a partial last one (K = 640: 10 units).
SKINNY_EDGE = [(M, K, N) for M in (32, 33, 64, 65, 96, 97, 128) for K, N in ((128, 64), (640, 192))]


@pytest.mark.parametrize("M,K,N", SKINNY_EDGE)
def test_skinny_dispatch_edges(q, M, K, N):
    log(f"skinny edges M={M} K={K} N={N}")
    lin = synth.plain_linear(M, K, N, seed=M * 19 + K, n_outliers=2)
    qa, sa, _, _ = q.qlin_quant_act(dev(lin.x))
    ref8 = layer.w8a8_forward(lin.x, lin.w)
    codes, sw = q.qlin_quant_weight_sym(dev(lin.w), 8)
    y, acc = q.qlin_gemm_w8a8(qa, sa, q.qlin_pack_weight(q.QLIN_LAYOUT_W8, codes), sw, N, want_acc=True)
    assert_equal(host(acc), ref8["acc"], "w8a8 acc")
    assert_close(host(y), ref8["y"], "w8a8 y")
    ref4 = layer.w4a8_channel_forward(lin.x, lin.w)
    codes, sw = q.qlin_quant_weight_sym(dev(lin.w), 4)
    y, acc = q.qlin_gemm_w4a8(qa, sa, q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, codes), sw, N, want_acc=True)
    assert_equal(host(acc), ref4["acc"], "w4a8 channel acc")
    assert_close(host(y), ref4["y"], "w4a8 channel y")
    refg = layer.w4a8_group_forward(lin.x, lin.w)
    codes, gs, cs, ratio = q.qlin_quant_weight_group(dev(lin.w), 128)
    y, acc = q.qlin_gemm_w4a8(qa, sa, q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, codes), cs, N, ratio=ratio, group=128,
                              want_acc=True)
    assert_equal(host(acc), refg["acc"], "w4a8 group acc")
    assert_close(host(y), refg["y"], "w4a8 group y")


@pytest.mark.parametrize("M,K,N", [(129, 128, 64), (300, 128, 192), (130, 1152, 64)])
def test_gemm_w4a8_group_workspace_small_k(q, M, K, N):
    # The once-per-call requantization at one group (K = 128) and at an odd
    # number of groups, against the oracle and the in-loop form.
    import torch
    log(f"w4a8 group workspace M={M} K={K} N={N}")
    lin = synth.plain_linear(M, K, N, seed=M * 23 + K)
    ref = layer.w4a8_group_forward(lin.x, lin.w)
    codes, gs, cs, ratio = q.qlin_quant_weight_group(dev(lin.w), 128)
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, codes)
    qa, sa, _, _ = q.qlin_quant_act(dev(lin.x))
    work = torch.full((q.qlin_gemm_w4a8_work_bytes(M, N, K, 128),), 0x5A, dtype=torch.uint8, device="cuda")
    assert work.numel() == K * N
    y, acc = q.qlin_gemm_w4a8(qa, sa, w4, cs, N, ratio=ratio, group=128, want_acc=True, work=work)
    assert_equal(host(acc), ref["acc"], "acc")
    assert_close(host(y), ref["y"], "y")
    y0, acc0 = q.qlin_gemm_w4a8(qa, sa, w4, cs, N, ratio=ratio, group=128, want_acc=True)
    assert_equal(host(acc0), host(acc), "acc in the K loop vs once per call")
    assert_equal(host(y0), host(y), "y in the K loop vs once per call")


def test_gemm_w4a8_group_requant_edge_ratios(q):
    # Hand-picked ratios (ties, clamping, fp16 rounding that changes the integer)
    # and every int4 code, including -8, checked through the GEMM accumulator
    # with one-hot activations: acc[m, n] is exactly the requantized weight.
    K, N = 128, 64
    rng = np.random.default_rng(0)
    codes = np.tile(np.arange(-8, 8, dtype=np.int8), K // 16)[:, None].repeat(N, 1)
    rg = np.zeros((1, N), np.float16)
    rg[0, :8] = [0.2142333984375, 16.5, 18.5, 16.0, 3.0, 0.0, 18.140625, 1e-7]
    rg[0, 8:] = rng.uniform(0, 18.2, N - 8).astype(np.float16)
    want_w8 = quant.requant_group(codes, rg, 128)
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, dev(codes))
    qa = np.eye(K, dtype=np.int8)
    y, acc = q.qlin_gemm_w4a8(dev(qa), dev(np.ones(K, np.float32)), w4, dev(np.ones(N, np.float16)), N,
                              ratio=dev(rg), group=128, want_acc=True)
    assert_equal(host(acc), want_w8.astype(np.int32), "requantized weights")


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("M,work", [(128, False), (256, False), (256, True)])
def test_gemm_w4a8_group_requant_exhaustive(q, sign, M, work):
    # QQQ's fused dequant-quant on the device, exhaustively: one column per
    # finite fp16 ratio of the given sign (31,744 of each, bit patterns
    # 0x0000..0x7bff or 0x8000..0xfbff, N = 496 * 64), every int4 code -8..7
    # down K = 128, one-hot int8 activations, unit scales, so that
    # acc[m, n] = w8[m mod 128, n] = clamp(rint(fp16(q4 * r)), -127, 127).
    # M = 128 runs the skinny kernel, M = 256 the 128-row tiles (requantizing
    # in the K loop) or, with a workspace, the once-per-call requantization
    # followed by the int8 tile.
    import torch
    K = 128
    bits = np.arange(0x7C00, dtype=np.uint32)
    if sign < 0:
        bits |= 0x8000
    rg = bits.astype(np.uint16).view(np.float16)[None, :]
    N = rg.shape[1]
    assert N % 64 == 0
    log(f"requant exhaustive sign={sign} M={M} N={N} work={work}")
    codes = np.tile(np.arange(-8, 8, dtype=np.int8), K // 16)[:, None].repeat(N, 1)
    want_w8 = quant.requant_group(codes, rg, 128).astype(np.int32)
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, dev(codes))
    qa = np.tile(np.eye(K, dtype=np.int8), (M // K, 1))
    buf = _requant_work(q, M, N, K)[0] if work else None
    y, acc = q.qlin_gemm_w4a8(dev(qa), dev(np.ones(M, np.float32)), w4, dev(np.ones(N, np.float16)), N,
                              ratio=dev(rg), group=128, want_acc=True, work=buf)
    torch.cuda.synchronize()
    got = host(acc)
    for r0 in range(0, M, K):
        assert_equal(got[r0:r0 + K], want_w8, f"requantized weights, rows {r0}..{r0 + K - 1}")
    assert_equal(host(y).astype(np.float64), np.tile(want_w8, (M // K, 1)).astype(np.float64), "y = w8")


@pytest.mark.parametrize("M,K,N", GEMM_SHAPES)
def test_gemm_w4a4(q, M, K, N):
    log(f"w4a4 M={M} K={K} N={N}")
    lin = synth.offq_inputs(M=M, K=K, N=N, seed=M * 17 + K)
    signs = lin.extra["signs"]
    ref = layer.offq_forward(lin.x, lin.w, signs)
    qa4, sa, za, rs, _ = q.qlin_hadamard_offset(dev(lin.x), dev(signs))
    codes, sw, zw, cs = q.qlin_quant_weight_offq(dev(lin.w), dev(signs))
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4U, codes)
    y, acc = q.qlin_gemm_w4a4(qa4, sa, za, rs, w4, sw, zw, cs, N, want_acc=True)
    assert_equal(host(acc), ref["acc"], "acc")
    assert_close(host(y), ref["y"], "y")


# The tiled kernels unroll their K loop by 6 stages of 128 k with register
# and buffer rotations: every stage count from 1 to 13 (no full unrolled
# period, one, two, with every remainder) on a ragged tile grid (M = 130: a
# partial second tile row; N = 320: a second tile column with one live
# column group).
@pytest.mark.parametrize("stages", list(range(1, 14)))
def test_gemm_tiled_k_depths(q, stages):
    M, N, K = 130, 320, 128 * stages
    log(f"tiled K depth: M={M} K={K} N={N}")
    lin = synth.plain_linear(M, K, N, seed=500 + stages, n_outliers=2)
    qa, sa, _, _ = q.qlin_quant_act(dev(lin.x))
    ref = layer.w8a8_forward(lin.x, lin.w)
    codes, sw = q.qlin_quant_weight_sym(dev(lin.w), 8)
    y, acc = q.qlin_gemm_w8a8(qa, sa, q.qlin_pack_weight(q.QLIN_LAYOUT_W8, codes), sw, N, want_acc=True)
    assert_equal(host(acc), ref["acc"], "w8a8 acc")
    assert_close(host(y), ref["y"], "w8a8 y")
    ref = layer.w4a8_channel_forward(lin.x, lin.w)
    codes, sw = q.qlin_quant_weight_sym(dev(lin.w), 4)
    y, acc = q.qlin_gemm_w4a8(qa, sa, q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, codes), sw, N, want_acc=True)
    assert_equal(host(acc), ref["acc"], "w4a8 channel acc")
    assert_close(host(y), ref["y"], "w4a8 channel y")
    ref = layer.w4a8_group_forward(lin.x, lin.w)
    codes, gs, cs, ratio = q.qlin_quant_weight_group(dev(lin.w), 128)
    y, acc = q.qlin_gemm_w4a8(qa, sa, q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, codes), cs, N, ratio=ratio, group=128,
                              want_acc=True)
    assert_equal(host(acc), ref["acc"], "w4a8 group acc")
    assert_close(host(y), ref["y"], "w4a8 group y")
    lin = synth.offq_inputs(M=M, K=K, N=N, seed=600 + stages)
    signs = lin.extra["signs"]
    ref = layer.offq_forward(lin.x, lin.w, signs)
    qa4, sa4, za, rs, _ = q.qlin_hadamard_offset(dev(lin.x), dev(signs))
    codes, sw, zw, csum = q.qlin_quant_weight_offq(dev(lin.w), dev(signs))
    y, acc = q.qlin_gemm_w4a4(qa4, sa4, za, rs, q.qlin_pack_weight(q.QLIN_LAYOUT_W4U, codes), sw, zw, csum, N,
                              want_acc=True)
    assert_equal(host(acc), ref["acc"], "w4a4 acc")
    assert_close(host(y), ref["y"], "w4a4 y")


# The fused compensation has three forms by the padded outlier count ldO:
# ldO <= 208, xO rows and W_O tiles both staged in LDS before the K loop;
# ldO <= 384, xO rows staged, W_O read from memory; above, after the K loop.
@pytest.mark.parametrize("M,K,N,nO", [(16, 256, 128, 13), (200, 512, 192, 64), (130, 384, 64, 33),
                                       (300, 256, 320, 16), (257, 1024, 256, 205), (200, 1024, 192, 209),
                                       (150, 1024, 128, 400)])
def test_quaff_fused_and_standalone_compensation(q, M, K, N, nO):
    import torch
    log(f"quaff comp M={M} K={K} N={N} nO={nO}")
    d = synth.quaff_steps(M=M, K=K, N=N, n_outliers=nO, steps=3, seed=M + nO)
    prep = layer.quaff_prepare(d.w, d.outliers)
    s_ref = np.ones(K, np.float32)
    O = dev(d.outliers)
    codes, sw = q.qlin_quant_weight_sym(dev(d.w), 8)
    w8 = q.qlin_pack_weight(q.QLIN_LAYOUT_W8, codes)
    WO = dev(np.ascontiguousarray(d.w[d.outliers]))
    WOp = q.qlin_pack_weight(q.QLIN_LAYOUT_WO, WO)
    wmax = q.qlin_weight_row_absmax(WO)
    assert_equal(host(wmax), prep["wmax"], "wmax")
    s = torch.ones(K, dtype=torch.float32, device="cuda")
    r = torch.empty(K, dtype=torch.float32, device="cuda")
    for t, x in enumerate(d.xs):
        ref = layer.quaff_step(x, prep, d.outliers, s_ref)
        s_ref = ref["s"]
        xd = dev(x)
        q.qlin_momentum_update(xd, O, wmax, 0.9, s, r)
        qa, sa, qO, xO = q.qlin_quant_act(xd, r, O, s=s)
        assert_equal(host(s), ref["s"], "s")
        assert_equal(host(qa), ref["q"], "q")
        assert_equal(host(qO)[:, :nO], ref["q"][:, d.outliers], "qO")
        y, acc = q.qlin_gemm_w8a8(qa, sa, w8, sw, N, xO=xO, nO=nO, WO=WOp, want_acc=True)
        assert_equal(host(acc), ref["acc"], "acc")
        assert_close(host(y), ref["y"], f"fused y step {t}")
        y2, _ = q.qlin_gemm_w8a8(qa, sa, w8, sw, N)
        q.qlin_outlier_comp(xO, sa, nO, WOp, y2)
        assert_close(host(y2), ref["y"], f"standalone y step {t}")


def test_gemm_w8a8_single_tile_identity(q):
    # acc[m, n] = sum_k qa[m, k] * w[k, n] with qa = identity rows: the output
    # reproduces W's codes, which pins the fragment row/column layout.
    K, N, M = 256, 128, 128
    rng = np.random.default_rng(5)
    codes = rng.integers(-127, 128, (K, N)).astype(np.int8)
    w8 = q.qlin_pack_weight(q.QLIN_LAYOUT_W8, dev(codes))
    qa = np.zeros((M, K), np.int8)
    qa[np.arange(M), np.arange(M)] = 1
    y, acc = q.qlin_gemm_w8a8(dev(qa), dev(np.ones(M, np.float32)), w8, dev(np.ones(N, np.float16)), N,
                              want_acc=True)
    assert_equal(host(acc), codes[:M].astype(np.int32), "acc")
