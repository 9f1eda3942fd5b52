"""Pins of the oracle's Top-1 PCA concentration (CPU only): the extreme-token
choice by brute force, the covariance against numpy's, the leading
eigenvector in a closed-form rank-one case and by its eigen-equation, the
Householder rotation's defining identities, and the concentration the pages
claim on planted-direction data."""
import numpy as np
import pytest

import synth
from oracle import pca, quant


def test_select_extreme_tokens_brute_force():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 9, 16)).astype(np.float16)
    x[2, 3, 7] = 40.0
    x[2, 6, 1] = -40.0  # a tie in |x|: the first token wins
    idx, z = pca.select_extreme_tokens(x)
    for s in range(5):
        best, bt = -1.0, -1
        for t in range(9):
            v = max(abs(float(e)) for e in x[s, t])
            if v > best:
                best, bt = v, t
        assert idx[s] == bt
        assert np.array_equal(z[s], x[s, bt])
    assert idx[2] == 3


def test_covariance_matches_numpy():
    rng = np.random.default_rng(1)
    z = (rng.standard_normal((40, 12)) * 3 + 7).astype(np.float16)
    assert np.allclose(pca.covariance(z), np.cov(z.astype(np.float64), rowvar=False), rtol=1e-12, atol=1e-12)


def test_leading_eigvec_rank_one_closed_form():
    # Extreme tokens a_s * u with no noise: C = var(a) u u^T, so v = +-u and
    # lambda = var(a) |u|^2.
    rng = np.random.default_rng(2)
    u = rng.standard_normal(32)
    u /= np.linalg.norm(u)
    a = rng.uniform(1, 5, 50)
    z = np.outer(a, u)
    v, lam = pca.leading_eigvec(z)
    assert v[0] <= 0
    assert abs(abs(v @ u) - 1) < 1e-12
    assert lam == pytest.approx(np.var(a, ddof=1), rel=1e-10)


def test_leading_eigvec_eigen_equation():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((30, 20)).astype(np.float16)
    v, lam = pca.leading_eigvec(z)
    c = pca.covariance(z)
    assert np.linalg.norm(c @ v - lam * v) < 1e-10 * lam
    assert abs(np.linalg.norm(v) - 1) < 1e-12
    # the largest: no unit vector has a larger Rayleigh quotient
    for _ in range(20):
        y = rng.standard_normal(20)
        y /= np.linalg.norm(y)
        assert y @ c @ y <= lam * (1 + 1e-12)


def test_householder_identities():
    rng = np.random.default_rng(4)
    v = rng.standard_normal(24)
    v /= np.linalg.norm(v)
    if v[0] > 0:
        v = -v
    w, beta = pca.householder(v)
    h = np.eye(24) - beta * np.outer(w, w)
    e0 = np.zeros(24)
    e0[0] = 1
    assert np.allclose(h @ v, e0, atol=1e-15)
    assert np.allclose(h, h.T) and np.allclose(h @ h, np.eye(24), atol=1e-15)
    # v = -e0 (the largest cancellation-free case) maps to e0 too
    w, beta = pca.householder(-e0)
    assert np.allclose((np.eye(24) - beta * np.outer(w, w)) @ -e0, e0)


def test_rotation_preserves_xw_and_concentrates_outliers():
    x, u = synth.pca_calibration(S=32, T=64, K=512, seed=5)
    idx, z = pca.select_extreme_tokens(x)
    v, _ = pca.leading_eigvec(z)
    assert abs(abs(v @ u) - 1) < 1e-3  # the planted direction is found
    xr = pca.rotate_acts(z, v).astype(np.float64)
    # channel 0 carries x . v: at least 99% of each extreme token's energy along u
    proj = z.astype(np.float64) @ v
    assert np.allclose(xr[:, 0], proj, rtol=1e-3, atol=0.05)
    assert np.all(xr[:, 0] ** 2 >= 0.99 * (z.astype(np.float64) @ u) ** 2 * 0.98)
    rest = np.abs(xr[:, 1:]).max()
    assert rest < 0.2 * np.abs(xr[:, 0]).min()
    # (x H)(H W) = x W up to the fp16 rounding of both factors
    rng = np.random.default_rng(6)
    wt = (rng.standard_normal((512, 64)) * 0.02).astype(np.float16)
    wf = pca.fold_weight(wt, v).astype(np.float64)
    ref = z.astype(np.float64) @ wt.astype(np.float64)
    got = xr @ wf
    assert np.abs(got - ref).max() <= 2e-3 * np.abs(ref).max()


def test_concentration_helps_offq():
    # OffQ's pipeline on the extreme tokens of planted-direction data: with the
    # Top-1 PCA rotation the outlier becomes one channel, the Hadamard turns it
    # into the group-0 offset and the zero point absorbs it; without it, the
    # dense outlier direction sets every range.  Relative error of the
    # dequantized int4 activations against the transformed values.
    x, u = synth.pca_calibration(S=16, T=32, K=512, seed=7)
    _, z = pca.select_extreme_tokens(x)
    v, _ = pca.leading_eigvec(z)
    rng = np.random.default_rng(8)
    signs = rng.choice(np.array([-1, 1], np.int8), 512)
    signs[::128] = 1

    def rel_err(toks):
        q, st, zz, _, t = quant.hadamard_offset_int4(toks, signs)
        deq = (q.astype(np.float64) - zz[:, None]) * st[:, None]
        return np.mean((deq - t) ** 2) / np.mean(t.astype(np.float64) ** 2)

    assert rel_err(pca.rotate_acts(z, v)) < 0.1 * rel_err(z)
