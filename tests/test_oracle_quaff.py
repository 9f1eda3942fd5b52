"""Pins of the oracle's Quaff compensation term and momentum update (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np

import synth
from oracle import gemm, layer, quant, quaff
from tests.exact import f32

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _lossless_weights(rng, K, N):
    """W = code * 2^-j exactly, with a +-127 code in each column, so per-channel
    int8 quantization reproduces W exactly (step = 2^-j)."""
    codes = rng.integers(-127, 128, (K, N))
    codes[0, :] = 127
    j = 9
    return (codes / 2.0 ** j).astype(np.float16), codes


def test_quaff_identity_exact_rationals():
    # X-hat (sW) == X-hat W + X-hat_{:,O} (s_O - 1) W_O with s = 1 off O, where
    # X-hat is the dequantized int8 activation; checked against exact rationals.
    rng = np.random.default_rng(0)
    M, K, N = 3, 8, 5
    o = np.array([1, 6])
    x = rng.standard_normal((M, K)).astype(np.float16)
    w, codes = _lossless_weights(rng, K, N)
    s = np.ones(K, np.float32)
    s[o] = np.array([7.375, 12.5], np.float32)
    r = (np.float32(1) / s).astype(np.float32)
    q, sa = quant.quant_act_sym_int8(x, r)
    qw, sw = quant.quant_weight_sym(w, 8)
    assert np.array_equal(qw, codes)
    acc, y_main = gemm.w8a8(q, sa, qw, sw.astype(np.float32))
    y = y_main + quaff.compensation(q[:, o], sa, s[o], w[o, :])
    for m in range(M):
        xhat = [Fraction(int(q[m, k])) * Fraction(float(sa[m])) for k in range(K)]
        for n in range(N):
            want = sum(xhat[k] * Fraction(float(s[k])) * Fraction(float(w[k, n])) for k in range(K))
            assert abs(Fraction(y[m, n]) - want) <= abs(want) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


def test_compensation_vanishes_when_s_is_one():
    d = synth.quaff_steps(M=16, K=256, N=64, n_outliers=13, steps=1)
    prep = layer.quaff_prepare(d.w, d.outliers)
    q, sa = quant.quant_act_sym_int8(d.xs[0])
    comp = quaff.compensation(q[:, d.outliers], sa, np.ones(13, np.float32), prep["w_o"])
    assert np.all(comp == 0)
    ref = layer.w8a8_forward(d.xs[0], d.w)
    acc, y = gemm.w8a8(q, sa, prep["qw"], prep["sw"].astype(np.float32))
    assert np.array_equal(acc, ref["acc"]) and np.array_equal(y, ref["y"])


def test_momentum_worked_example():
    g = GOLD["momentum_step"]
    x = np.zeros((5, 4), np.float16)
    x[2, 1] = -g["colmax"]
    x[4, 1] = 3.0
    s = np.ones(4, np.float32)
    s1, r1 = quaff.momentum_update(x, np.array([1]), np.array([g["wmax"]], np.float32), g["gamma"], s)
    assert Fraction(float(s1[1])) == Fraction(g["s1_num"], 2 ** g["s1_den_log2"])
    assert Fraction(float(r1[1])) == Fraction(g["r1_num"], 2 ** g["r1_den_log2"])
    assert np.all(s1[[0, 2, 3]] == 1) and np.all(r1[[0, 2, 3]] == 1)
    # The second step re-done in exact rationals with an fp32 rounding per op.
    gam = f32(Fraction(9, 10))
    g1 = f32(1 - gam)
    s2_want = f32(f32(gam * Fraction(float(s1[1]))) + f32(g1 * 2))
    s2, r2 = quaff.momentum_update(x, np.array([1]), np.array([g["wmax"]], np.float32), g["gamma"], s1)
    assert Fraction(float(s2[1])) == s2_want
    assert Fraction(float(r2[1])) == f32(1 / s2_want)


def test_momentum_closed_form_constant_beta():
    # With the same batch every step, beta is constant and
    # s_t = beta + gamma^t (s_0 - beta).
    rng = np.random.default_rng(1)
    K = 64
    o = np.array([3, 17, 40])
    x = rng.standard_normal((32, K)).astype(np.float16)
    x[:, o] *= np.array([80, 120, 0.01], np.float16)
    wmax = np.array([0.05, 0.08, 0.5], np.float32)
    beta = np.maximum(1.0, np.sqrt(np.abs(x[:, o].astype(np.float64)).max(0) / wmax.astype(np.float64)))
    s = np.ones(K, np.float32)
    for t in range(1, 21):
        s, r = quaff.momentum_update(x, o, wmax, 0.9, s)
        want = beta + 0.9 ** t * (1 - beta)
        assert np.allclose(s[o], want, rtol=2e-6 * t, atol=0)
        assert np.all(s >= 1)
        mask = np.ones(K, bool)
        mask[o] = False
        assert np.all(s[mask] == 1) and np.all(r[mask] == 1)
    assert s[40] == 1  # the 0.01-scaled channel has beta = 1


def test_momentum_special_cases():
    x = np.full((4, 8), 2.0, np.float16)
    o = np.array([0, 5])
    # gamma = 0: s is beta itself.
    s, _ = quaff.momentum_update(x, o, np.array([0.5, 0.0], np.float32), 0.0, np.ones(8, np.float32))
    assert s[0] == 2.0  # sqrt(2 / 0.5)
    assert s[5] == 1.0  # zero weight row: beta = 1
    # Empty batch: beta = 1, s decays toward 1.
    s0 = np.full(8, 3.0, np.float32)
    s1, _ = quaff.momentum_update(np.zeros((0, 8), np.float16), o, np.array([1.0, 1.0], np.float32), 0.5, s0)
    assert s1[0] == 2.0 and s1[3] == 3.0


def test_momentum_checkpoint_resume_bit_exact():
    d = synth.quaff_steps(M=64, K=256, N=8, n_outliers=13, steps=10)
    wmax = quaff.weight_row_absmax(d.w[d.outliers])
    s = np.ones(256, np.float32)
    hist = []
    for x in d.xs:
        s, r = quaff.momentum_update(x, d.outliers, wmax, 0.9, s)
        hist.append(s.copy())
    s2 = hist[4].copy()
    for x in d.xs[5:]:
        s2, _ = quaff.momentum_update(x, d.outliers, wmax, 0.9, s2)
    assert np.array_equal(s2, hist[-1])


def test_quaff_error_bound_and_gain_over_plain_w8a8():
    d = synth.quaff_steps(M=64, K=512, N=96, n_outliers=26, steps=10)
    prep = layer.quaff_prepare(d.w, d.outliers)
    s = np.ones(512, np.float32)
    for x in d.xs:
        out = layer.quaff_step(x, prep, d.outliers, s)
        s = out["s"]
    x = d.xs[-1]
    xf, wf = x.astype(np.float64), d.w.astype(np.float64)
    truth = xf @ wf
    # Error bound from the two quantization steps (weights: step_w/2, activations:
    # step_a/2 on X/s, plus fp32 rounding of X * r), per output element.
    v = np.abs(xf / out["s"].astype(np.float64)[None, :])
    da = out["sa"].astype(np.float64)[:, None]
    dw = prep["sw"].astype(np.float64)[None, :]
    e = da / 2 * 1.001 + v.max(1, keepdims=True) * 2.0 ** -21
    sm1 = (out["s"].astype(np.float64) - 1.0)
    bound = (v @ np.ones_like(wf)) * dw / 2 + e * (np.ones_like(xf) @ np.abs(wf)) + 512 * e * dw / 2 \
        + e * (np.ones((64, 1)) @ (sm1[None, :] @ np.abs(wf)))
    assert np.all(np.abs(out["y"] - truth) <= bound)
    plain = layer.w8a8_forward(x, d.w)
    assert np.abs(out["y"] - truth).max() < 0.5 * np.abs(plain["y"] - truth).max()


def test_weight_row_absmax_worked_example():
    g = GOLD["weight_row_absmax_rows"]
    got = quaff.weight_row_absmax(np.asarray(g["w_rows"], np.float16))
    assert got.dtype == np.float32
    assert np.array_equal(got, np.asarray(g["absmax"], np.float32))
