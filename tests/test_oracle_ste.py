"""Pins of the oracle's straight-through-estimator backward of the Quaff layer
(CPU only): the closed form against torch autograd of the forward definition,
the int8 gradient product against brute force and its error bound, and a
hand-worked example."""
import json
import os

import numpy as np
import pytest

from oracle import gemm, quant, quaff
from tests.exact import f32

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _case(seed, M=6, K=256, N=128, nO=5):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)) * 2).astype(np.float16)
    w = (rng.standard_normal((K, N)) * 0.05).astype(np.float16)
    dy = rng.standard_normal((M, N)).astype(np.float16)
    o = np.sort(rng.choice(K, nO, replace=False)).astype(np.int64)
    s = np.ones(K, np.float32)
    s[o] = rng.uniform(1.0, 4.0, nO).astype(np.float32)
    r = (np.float32(1) / s).astype(np.float32)
    qw, sw = quant.quant_weight_sym(w, 8)
    return x, w, dy, o, s, r, qw, sw


def test_ste_closed_form_matches_autograd():
    # Autograd of the forward definition with a straight-through quantizer:
    # the quantized values enter through a detached difference.
    torch = pytest.importorskip("torch")
    x16, w, dy, o, s, r, qw, sw = _case(1)
    q, sa = quant.quant_act_sym_int8(x16, r)
    x = torch.tensor(x16.astype(np.float64), requires_grad=True)
    xr = x * torch.tensor(r.astype(np.float64))
    deq = torch.tensor(q.astype(np.float64) * sa.astype(np.float64)[:, None])
    xq = xr + (deq - xr).detach()
    what = torch.tensor(qw.astype(np.float64) * sw.astype(np.float64)[None, :])
    w_o = torch.tensor(w[o].astype(np.float64))
    y = xq @ what + xq[:, torch.tensor(o)] @ (torch.tensor(s[o].astype(np.float64) - 1.0)[:, None] * w_o)
    (y * torch.tensor(dy.astype(np.float64))).sum().backward()
    got = quaff.ste_backward_exact(dy, qw, sw, s, r, o, w[o])
    want = x.grad.numpy()
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_ste_worked_example():
    g = GOLD["ste_backward_tiny"]
    dy = np.array(g["dy"], np.float16)
    qw = np.array(g["qw"], np.int8)
    sw = np.array(g["sw"], np.float16)
    s = np.array(g["s"], np.float32)
    r = (np.float32(1) / s).astype(np.float32)
    o = np.array(g["outliers"])
    w_o = np.array(g["w_o"], np.float16)
    out = quaff.ste_backward(dy, qw, sw, s, r, o, w_o)
    assert out["gq"].tolist() == g["gq"]
    assert out["acc"].tolist() == g["acc"]
    assert out["cb"].tolist() == g["cb"]
    assert np.allclose(out["dx"], g["dx_approx"], rtol=1e-6)
    assert np.allclose(quaff.ste_backward_exact(dy, qw, sw, s, r, o, w_o), g["dx_exact"], rtol=1e-6)
    assert float(out["gs"][0]) == float(f32(np.float64(0.5) / 127))


def test_ste_int8_product_brute_force():
    rng = np.random.default_rng(2)
    M, K, N = 3, 8, 6
    dy = rng.standard_normal((M, N)).astype(np.float16)
    qw = rng.integers(-127, 128, (K, N)).astype(np.int8)
    sw = rng.uniform(0.001, 0.01, N).astype(np.float16)
    s = np.ones(K, np.float32)
    out = quaff.ste_backward(dy, qw, sw, s, s, np.zeros(0, np.int64), np.zeros((0, N), np.float16))
    for m in range(M):
        for k in range(K):
            assert out["acc"][m, k] == sum(int(out["gq"][m, n]) * int(qw[k, n]) for n in range(N))
            assert out["dx"][m, k] == pytest.approx(float(out["gs"][m]) * int(out["acc"][m, k]), rel=1e-15)


def test_ste_int8_within_gradient_quantization_bound():
    # The only difference from the closed form is rounding G = dY * sw to the
    # per-token int8 grid: |gs * gq - G| <= gs / 2 per element (plus the fp32
    # rounding of G), so |dX_int8 - dX| <= r_k * (gs / 2) * sum_n |W_int[k, n]|.
    x16, w, dy, o, s, r, qw, sw = _case(3, M=20, K=384, N=256, nO=9)
    out = quaff.ste_backward(dy, qw, sw, s, r, o, w[o])
    exact = quaff.ste_backward_exact(dy, qw, sw, s, r, o, w[o])
    bound = (r.astype(np.float64)[None, :] * (out["gs"].astype(np.float64)[:, None] / 2)
             * np.abs(qw.astype(np.float64)).sum(axis=1)[None, :])
    err = np.abs(out["dx"] - exact)
    assert np.all(err <= bound * (1 + 1e-5) + 1e-9 * np.abs(exact).max())
    assert err.max() > 0  # the bound is not vacuous: G is off the grid here


def test_ste_without_outliers_is_the_transposed_product():
    x16, w, dy, o, s, r, qw, sw = _case(4)
    ones = np.ones_like(s)
    none = np.zeros(0, np.int64)
    got = quaff.ste_backward_exact(dy, qw, sw, ones, ones, none, np.zeros((0, w.shape[1]), np.float16))
    what = qw.astype(np.float64) * sw.astype(np.float64)[None, :]
    ref = np.einsum("mn,kn->mk", dy.astype(np.float64), what)
    assert np.allclose(got, ref, rtol=1e-13, atol=0)
