"""GPU parity at the full sizes of the five layer workloads (plus the
group-wise form of the OffQ one and the token-count sweep), in the launch
configurations bench.py times.

Everything is compared in full, on every row: integer stages (codes, zero
points, sums, the momentum state s and r, int32 accumulators) bit for bit,
fp16 outputs within the normwise relative tolerance 1e-3.  The oracle's exact
integer products run as float64 BLAS (a few seconds per full-size product on
a 16-core host).
"""
import numpy as np
import pytest

import synth
from oracle import gemm, layer, quant, quaff
from tests.gpu_helpers import assert_close, assert_equal, dev, host, log
from tests.test_gpu_offq_group import check_group_sums

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    assert torch.cuda.is_available()
    from outlier_aware_bit_amd import qlin
    return qlin


def test_tiny_w8a8_full(q):
    lin = synth.tiny_w8a8(seed=0)
    log("tiny W8A8 16x256x128")
    ref = layer.w8a8_forward(lin.x, lin.w)
    codes, sw = q.qlin_quant_weight_sym(dev(lin.w), 8)
    assert_equal(host(codes), ref["qw"], "weight codes")
    w8 = q.qlin_pack_weight(q.QLIN_LAYOUT_W8, codes)
    qa, sa, _, _ = q.qlin_quant_act(dev(lin.x))
    assert_equal(host(qa), ref["q"], "activation codes")
    assert_equal(host(sa), ref["sa"], "activation steps")
    y, acc = q.qlin_gemm_w8a8(qa, sa, w8, sw, 128, want_acc=True)
    assert_equal(host(acc), ref["acc"], "acc")
    assert_close(host(y), ref["y"], "y")


def test_quaff_q_proj_ten_steps(q):
    import torch
    M, K, N, nO = 2048, 4096, 4096, 205
    log(f"Quaff q_proj {M}x{K}x{N} |O|={nO}, 10 steps")
    d = synth.quaff_steps(M=M, K=K, N=N, n_outliers=nO, steps=10, seed=1)
    prep = layer.quaff_prepare(d.w, d.outliers)
    codes, sw = q.qlin_quant_weight_sym(dev(d.w), 8)
    assert_equal(host(codes), prep["qw"], "weight codes")
    assert_equal(host(sw).view(np.uint16), prep["sw"].view(np.uint16), "weight steps")
    w8 = q.qlin_pack_weight(q.QLIN_LAYOUT_W8, codes)
    O = dev(d.outliers)
    WO = dev(np.ascontiguousarray(d.w[d.outliers]))
    WOp = q.qlin_pack_weight(q.QLIN_LAYOUT_WO, WO)
    wmax = q.qlin_weight_row_absmax(WO)
    s = torch.ones(K, dtype=torch.float32, device="cuda")
    r = torch.empty_like(s)
    work = torch.empty((q.qlin_momentum_work_bytes(M, nO) // 4,), dtype=torch.float32, device="cuda")
    s_ref = np.ones(K, np.float32)
    o = d.outliers.astype(np.int64)
    for t, x in enumerate(d.xs):
        log(f"  step {t}")
        s_ref, r_ref = quaff.momentum_update(x, o, prep["wmax"], 0.9, s_ref)
        xd = dev(x)
        q.qlin_momentum_update(xd, O, wmax, 0.9, s, r, work=work)
        qa, sa, _, xO = q.qlin_quant_act(xd, r, O, s=s, want_qO=False)
        y, acc = q.qlin_gemm_w8a8(qa, sa, w8, sw, N, xO=xO, nO=nO, WO=WOp, want_acc=True)
        assert_equal(host(s), s_ref, f"s step {t}")
        assert_equal(host(r), r_ref, f"r step {t}")
        q_ref, sa_ref = quant.quant_act_sym_int8(x, r_ref)
        assert_equal(host(qa), q_ref, f"codes step {t}")
        assert_equal(host(sa), sa_ref, f"steps step {t}")
        acc_ref, y_main = gemm.w8a8(q_ref, sa_ref, prep["qw"], prep["sw"].astype(np.float32))
        y_ref = y_main + quaff.compensation(q_ref[:, o], sa_ref, s_ref[o], prep["w_o"])
        assert_equal(host(acc), acc_ref, f"acc step {t}")
        assert_close(host(y), y_ref, f"y step {t}")


@pytest.mark.parametrize("M", [1, 16, 64])
def test_qqq_decode_w4a8_channel_full(q, M):
    K, N = 4096, 11008
    log(f"QQQ decode W4A8 per channel M={M} K={K} N={N}")
    lin = synth.qqq_decode(M=M, K=K, N=N, seed=2)
    ref = layer.w4a8_channel_forward(lin.x, lin.w)
    codes, sw = q.qlin_quant_weight_sym(dev(lin.w), 4)
    assert_equal(host(codes), ref["q4"], "weight codes")
    assert_equal(host(sw).view(np.uint16), ref["sw"].view(np.uint16), "weight steps")
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, codes)
    qa, sa, _, _ = q.qlin_quant_act(dev(lin.x))
    assert_equal(host(qa), ref["q"], "activation codes")
    y, acc = q.qlin_gemm_w4a8(qa, sa, w4, sw, N, want_acc=True)
    assert_equal(host(acc), ref["acc"], "acc")
    assert_close(host(y), ref["y"], "y")


def test_qqq_prefill_w4a8_group_full(q):
    M, K, N = 4096, 11008, 4096
    log(f"QQQ prefill W4A8 g128 {M}x{K}x{N}")
    lin = synth.qqq_prefill(M=M, K=K, N=N, seed=3)
    q4, sg, sc, rg = quant.quant_weight_group(lin.w, 128)
    codes, gs, cs, ratio = q.qlin_quant_weight_group(dev(lin.w), 128)
    assert_equal(host(codes), q4, "weight codes")
    assert_equal(host(gs).view(np.uint16), sg.view(np.uint16), "group scales")
    assert_equal(host(cs).view(np.uint16), sc.view(np.uint16), "channel scales")
    assert_equal(host(ratio).view(np.uint16), rg.view(np.uint16), "ratios")
    w8 = quant.requant_group(q4, rg, 128)
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, codes)
    qa, sa, _, _ = q.qlin_quant_act(dev(lin.x))
    q_ref, sa_ref = quant.quant_act_sym_int8(lin.x)
    assert_equal(host(qa), q_ref, "activation codes")
    assert_equal(host(sa), sa_ref, "activation steps")
    # As timed: requantized once per call into a workspace, then the int8
    # tile; the in-loop requantization must give the same bits.
    import torch
    work = torch.empty(q.qlin_gemm_w4a8_work_bytes(M, N, K, 128), dtype=torch.uint8, device="cuda")
    y, acc = q.qlin_gemm_w4a8(qa, sa, w4, cs, N, ratio=ratio, group=128, want_acc=True, work=work)
    y0, acc0 = q.qlin_gemm_w4a8(qa, sa, w4, cs, N, ratio=ratio, group=128, want_acc=True)
    assert_equal(host(acc0), host(acc), "acc, requantized in the K loop vs once per call")
    assert_equal(host(y0), host(y), "y, requantized in the K loop vs once per call")
    log("  oracle product")
    acc_ref, y_ref = gemm.w4a8_group(q_ref, sa_ref, w8, sc.astype(np.float32))
    assert_equal(host(acc), acc_ref, "acc")
    assert_close(host(y), y_ref, "y")


def test_offq_w4a4_full(q):
    M, K, N = 2048, 4096, 14336
    log(f"OffQ W4A4 {M}x{K}x{N}")
    lin = synth.offq_inputs(M=M, K=K, N=N, seed=4)
    signs = lin.extra["signs"]
    qa_ref, sa_ref, za_ref, rs_ref, t_ref = quant.hadamard_offset_int4(lin.x, signs)
    qw_ref, sw_ref, zw_ref, cs_ref = quant.offq_weight(lin.w, signs)
    sd = dev(signs)
    qa4, sa, za, rs, t = q.qlin_hadamard_offset(dev(lin.x), sd, want_t=True)
    assert_equal(host(t), t_ref, "transformed activations")
    packed = host(qa4)
    codes = np.empty((M, K), np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    assert_equal(codes, qa_ref, "activation codes")
    assert_equal(host(sa), sa_ref, "activation steps")
    assert_equal(host(za), za_ref, "activation zero points")
    assert_equal(host(rs), rs_ref, "row sums")
    cw, sw, zw, cs = q.qlin_quant_weight_offq(dev(lin.w), sd)
    assert_equal(host(cw), qw_ref, "weight codes")
    assert_equal(host(sw), sw_ref, "weight steps")
    assert_equal(host(zw), zw_ref, "weight zero points")
    assert_equal(host(cs), cs_ref, "column sums")
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4U, cw)
    y, acc = q.qlin_gemm_w4a4(qa4, sa, za, rs, w4, sw, zw, cs, N, want_acc=True)
    log("  oracle product")
    acc_ref, y_ref = gemm.w4a4(qa_ref, sa_ref, za_ref, qw_ref, sw_ref, zw_ref)
    assert_equal(host(acc), acc_ref, "acc")
    assert_close(host(y), y_ref, "y")


def test_offq_w4a4_group_full(q):
    # Group-wise offsets at the OffQ shape, one outlier level per group.
    M, K, N = 2048, 4096, 14336
    log(f"OffQ W4A4 group-wise {M}x{K}x{N}")
    lin = synth.offq_inputs(M=M, K=K, N=N, seed=4, offset_spread=400.0)
    signs = lin.extra["signs"]
    qa_ref, sa_ref, za_ref, rs_ref, t_ref = quant.hadamard_offset_int4_group(lin.x, signs)
    qw_ref, sw_ref, zw_ref, _ = quant.offq_weight(lin.w, signs)
    sd = dev(signs)
    qa4, sa, za, rs, t = q.qlin_hadamard_offset_group(dev(lin.x), sd, want_t=True)
    assert_equal(host(t), t_ref, "transformed activations")
    packed = host(qa4)
    codes = np.empty((M, K), np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    assert_equal(codes, qa_ref, "activation codes")
    assert_equal(host(sa), sa_ref, "activation steps")
    assert_equal(host(za), za_ref, "activation zero points")
    assert_equal(host(rs), rs_ref, "group code sums")
    cw, sw, zw, _ = q.qlin_quant_weight_offq(dev(lin.w), sd)
    assert_equal(host(cw), qw_ref, "weight codes")
    csg = q.qlin_weight_colsum_group(cw)
    assert_equal(host(csg), quant.weight_colsum_group(qw_ref), "column sums per group")
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4U, cw)
    y, _ = q.qlin_gemm_w4a4_group(qa4, sa, za, rs, w4, sw, zw, csg, N)
    log("  oracle product")
    y_ref = gemm.w4a4_group(qa_ref, sa_ref, za_ref, qw_ref, sw_ref, zw_ref)
    assert_close(host(y), y_ref, "y")
    del y_ref
    # Every group's int32 sums (G x M x N), from the variant that writes them.
    y2, acc = q.qlin_gemm_w4a4_group(qa4, sa, za, rs, w4, sw, zw, csg, N, want_acc=True)
    assert_equal(host(y2).view(np.uint16), host(y).view(np.uint16), "y with and without the group sums")
    log("  group sums")
    got = host(acc)
    del acc, y2
    check_group_sums(got, dict(qa=qa_ref, qw=qw_ref, sa=sa_ref, za=za_ref, sw=sw_ref, zw=zw_ref, rowsum=rs_ref,
                               colsum_g=quant.weight_colsum_group(qw_ref)))


SWEEP_MS = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096]


def test_token_sweep_llama7b(q):
    # The token-count sweep of the three W*A8 GEMMs at K = 4096, N = 11008:
    # every M goes through the library's own dispatch (skinny kernels up to
    # 128 tokens, 128- or 256-row tiles above).  Output rows do not depend on
    # M, so the oracle runs once at the largest M and every M is compared on
    # all of its rows: accumulators exact, outputs within 1e-3.
    K, N = 4096, 11008
    Mx = max(SWEEP_MS)
    lin = synth.qqq_decode(M=Mx, K=K, N=N, seed=2)
    q_ref, sa_ref = quant.quant_act_sym_int8(lin.x)
    w8_ref, s8_ref = quant.quant_weight_sym(lin.w, 8)
    w4_ref, s4_ref = quant.quant_weight_sym(lin.w, 4)
    wg_ref, _, sc_ref, rg_ref = quant.quant_weight_group(lin.w, 128)
    w8g_ref = quant.requant_group(wg_ref, rg_ref)
    wd = dev(lin.w)
    qa, sa, _, _ = q.qlin_quant_act(dev(lin.x))
    assert_equal(host(qa), q_ref, "activation codes")
    c8, s8 = q.qlin_quant_weight_sym(wd, 8)
    c4, s4 = q.qlin_quant_weight_sym(wd, 4)
    cg, _, sc, ratio = q.qlin_quant_weight_group(wd, 128)
    assert_equal(host(c8), w8_ref, "int8 weight codes")
    assert_equal(host(c4), w4_ref, "int4 weight codes")
    assert_equal(host(cg), wg_ref, "group weight codes")
    p8 = q.qlin_pack_weight(q.QLIN_LAYOUT_W8, c8)
    p4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, c4)
    pg = q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, cg)
    import torch
    work = torch.empty(q.qlin_gemm_w4a8_work_bytes(Mx, N, K, 128), dtype=torch.uint8, device="cuda")
    cases = {
        "w8a8": (lambda a, s_: q.qlin_gemm_w8a8(a, s_, p8, s8, N, want_acc=True), w8_ref, s8_ref),
        "w4a8 channel": (lambda a, s_: q.qlin_gemm_w4a8(a, s_, p4, s4, N, want_acc=True), w4_ref, s4_ref),
        "w4a8 group": (lambda a, s_: q.qlin_gemm_w4a8(a, s_, pg, sc, N, ratio=ratio, group=128, want_acc=True),
                       w8g_ref, sc_ref),
        "w4a8 group, workspace": (lambda a, s_: q.qlin_gemm_w4a8(a, s_, pg, sc, N, ratio=ratio, group=128,
                                                                 want_acc=True, work=work), w8g_ref, sc_ref),
    }
    for name, (fn, wq, ws) in cases.items():
        log(f"token sweep {name}: oracle product at M={Mx}")
        acc_ref, y_ref = gemm.w8a8(q_ref, sa_ref, wq, ws.astype(np.float32))
        for M in SWEEP_MS:
            log(f"token sweep {name} M={M}")
            y, acc = fn(qa[:M], sa[:M])
            assert_equal(host(acc), acc_ref[:M], f"{name} acc M={M}")
            assert_close(host(y), y_ref[:M], f"{name} y M={M}")
        del acc_ref, y_ref


def test_quaff_q_proj_backward(q):
    # The STE backward at the q_proj shape with the momentum state of one
    # forward step: every row of the gradient codes and steps, acc, cb and dX.
    M, K, N, nO = 2048, 4096, 4096, 205
    log(f"Quaff q_proj backward {M}x{N}x{K} |O|={nO}")
    d = synth.quaff_steps(M=M, K=K, N=N, n_outliers=nO, steps=1, seed=1)
    prep = layer.quaff_prepare(d.w, d.outliers)
    o = d.outliers.astype(np.int64)
    s_ref, r_ref = quaff.momentum_update(d.xs[0], o, prep["wmax"], 0.9, np.ones(K, np.float32))
    dy = synth.grad_output(M, N, seed=5)
    codes, sw = q.qlin_quant_weight_sym(dev(d.w), 8)
    w8t = q.qlin_pack_weight(q.QLIN_LAYOUT_W8T, codes)
    dx, gq, gs, cb, acc = q.qlin_quaff_backward(dev(dy), sw, w8t, dev(s_ref), dev(r_ref), K, O=dev(d.outliers),
                                                w_o=dev(np.ascontiguousarray(prep["w_o"])), want_acc=True)
    gq_ref, gs_ref = quant.quant_act_sym_int8(dy, prep["sw"].astype(np.float32))
    assert_equal(host(gq), gq_ref, "gradient codes")
    assert_equal(host(gs), gs_ref, "gradient steps")
    log("  oracle product")
    ref = quaff.ste_backward(dy, prep["qw"], prep["sw"], s_ref, r_ref, o, prep["w_o"])
    assert_equal(host(acc), ref["acc"], "acc")
    assert_close(host(cb)[:, :nO], ref["cb"], "cb", tol=1e-5)
    assert_close(host(dx), ref["dx"], "dx")
