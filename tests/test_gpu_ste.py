"""GPU parity of the Quaff straight-through-estimator backward
(qlin_quaff_backward) against the CPU oracle, through the C ABI.

The quantized gradient (codes and steps) and the int32 accumulators must
match bit for bit; the fp32 compensation product cb within a normwise 1e-5
(fp32 accumulation of exact fp16 products); the fp16 input gradient within the
normwise 1e-3 of the oracle's float64 value from the same codes.
"""
import numpy as np
import pytest

import synth
from oracle import gemm, layer, quant, quaff
from tests.gpu_helpers import assert_close, assert_equal, dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    assert torch.cuda.is_available()
    from outlier_aware_bit_amd import qlin
    return qlin


def _state(K, nO, seed):
    rng = np.random.default_rng(seed)
    o = np.sort(rng.choice(K, nO, replace=False)).astype(np.int32)
    s = np.ones(K, np.float32)
    s[o] = rng.uniform(1.0, 6.0, nO).astype(np.float32)
    r = (np.float32(1) / s).astype(np.float32)
    return o, s, r


def _run(q, dy, w, o, s, r):
    codes, sw = q.qlin_quant_weight_sym(dev(w), 8)
    w8t = q.qlin_pack_weight(q.QLIN_LAYOUT_W8T, codes)
    K = w.shape[0]
    kw = {}
    if o.size:
        kw = dict(O=dev(o), w_o=dev(np.ascontiguousarray(w[o.astype(np.int64)])))
    return q.qlin_quaff_backward(dev(dy), sw, w8t, dev(s), dev(r), K, want_acc=True, **kw)


@pytest.mark.parametrize("M,N,K,nO", [(1, 128, 128, 0), (7, 256, 384, 5), (33, 384, 256, 13), (130, 512, 384, 33),
                                       (300, 256, 640, 64), (64, 1280, 512, 205), (1000, 384, 1024, 40)])
def test_quaff_backward(q, M, N, K, nO):
    log(f"quaff backward M={M} N={N} K={K} nO={nO}")
    rng_seed = M * 31 + N + K
    lin = synth.plain_linear(M, K, N, seed=rng_seed)
    dy = synth.grad_output(M, N, seed=rng_seed + 1)
    o, s, r = _state(K, nO, rng_seed + 2)
    prep = layer.quaff_prepare(lin.w, o)
    ref = quaff.ste_backward(dy, prep["qw"], prep["sw"], s, r, o, prep["w_o"])
    dx, gq, gs, cb, acc = _run(q, dy, lin.w, o, s, r)
    assert_equal(host(gq), ref["gq"], "gradient codes")
    assert_equal(host(gs), ref["gs"], "gradient steps")
    assert_equal(host(acc), ref["acc"], "acc")
    if nO:
        ld = q.qlin_outlier_ld(nO)
        got = host(cb)
        assert np.all(got[:, nO:ld] == 0)
        assert_close(got[:, :nO], ref["cb"], "cb", tol=1e-5)
    assert_close(host(dx), ref["dx"], "dx")


def test_quaff_backward_no_outliers_unit_scale(q):
    # s = r = 1 and no outliers: dX = fp16(gs * acc), the transposed product.
    M, N, K = 70, 256, 384
    lin = synth.plain_linear(M, K, N, seed=40)
    dy = synth.grad_output(M, N, seed=41)
    ones = np.ones(K, np.float32)
    none = np.zeros(0, np.int32)
    dx, gq, gs, cb, acc = _run(q, dy, lin.w, none, ones, ones)
    qw, sw = quant.quant_weight_sym(lin.w, 8)
    gq_ref, gs_ref = quant.quant_act_sym_int8(dy, sw.astype(np.float32))
    acc_ref = gemm.exact_int_matmul(gq_ref, qw.T)
    assert_equal(host(acc), acc_ref.astype(np.int32), "acc")
    assert_close(host(dx), acc_ref * gs_ref.astype(np.float64)[:, None], "dx")
    assert cb is None


def test_quaff_backward_empty_batch(q):
    import torch
    K, N = 256, 128
    lin = synth.plain_linear(1, K, N, seed=42)
    codes, sw = q.qlin_quant_weight_sym(dev(lin.w), 8)
    w8t = q.qlin_pack_weight(q.QLIN_LAYOUT_W8T, codes)
    ones = torch.ones(K, dtype=torch.float32, device="cuda")
    dx, gq, gs, cb, acc = q.qlin_quaff_backward(torch.zeros((0, N), dtype=torch.float16, device="cuda"), sw, w8t,
                                                ones, ones, K)
    assert dx.shape == (0, K)
