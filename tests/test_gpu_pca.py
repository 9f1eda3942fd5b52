"""GPU parity of OffQ's Top-1 PCA concentration (offline calibration kernels)
against the CPU oracle, through the C ABI.

The extreme-token choice and the copied tokens must match bit for bit.  The
leading eigenvector comes from a float64 power iteration on the GPU and from
numpy's eigh in the oracle: on planted-direction data (a large eigengap) they
must agree to 1e-9 in direction and 1e-9 relative in the eigenvalue.  The
rotated fp16 weights and activations are float64 values rounded once: a
different summation order may move a value across a rounding boundary, so at
most one fp16 ulp of difference is allowed, on at most 1e-3 of the elements.
"""
import numpy as np
import pytest

import synth
from oracle import pca, quant
from tests.gpu_helpers import assert_equal, dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    assert torch.cuda.is_available()
    from outlier_aware_bit_amd import qlin
    return qlin


def _ulps(a, b):
    ai = np.asarray(a, np.float16).view(np.int16).astype(np.int32)
    bi = np.asarray(b, np.float16).view(np.int16).astype(np.int32)
    ai = np.where(ai < 0, -32768 - ai, ai)
    bi = np.where(bi < 0, -32768 - bi, bi)
    return np.abs(ai - bi)


@pytest.mark.parametrize("S,T,K", [(3, 5, 8), (2, 3, 64), (8, 64, 512), (17, 130, 1000), (64, 128, 4096)])
def test_pca_select(q, S, T, K):
    log(f"pca select S={S} T={T} K={K}")
    x, _ = synth.pca_calibration(S=S, T=T, K=K, seed=S + T, planted=min(2, T))
    x[0, T - 1] = x[0, 0]  # a tie: the first token must win
    x[0, 0, 0] = 3000.0
    x[0, T - 1, 0] = 3000.0
    idx_ref, z_ref = pca.select_extreme_tokens(x)
    idx, z = q.qlin_pca_select(dev(x))
    assert_equal(host(idx), idx_ref, "extreme token index")
    assert_equal(host(z), z_ref, "extreme tokens")
    assert int(host(idx)[0]) == 0


# S <= 128 keeps the Gram matrix in LDS; 200 (ragged 16-row tiles) and 2048
# (the largest S) read it from memory; S = 2 is the smallest.
@pytest.mark.parametrize("S,K", [(2, 64), (16, 128), (64, 1000), (128, 4096), (200, 512), (2048, 256)])
def test_pca_leading_eigvec(q, S, K):
    log(f"pca eigvec S={S} K={K}")
    x, u = synth.pca_calibration(S=S, T=8, K=K, seed=K + S)
    _, z = pca.select_extreme_tokens(x)
    v_ref, lam_ref = pca.leading_eigvec(z)
    v, lam, its = q.qlin_pca_leading_eigvec(dev(z))
    vg = host(v)
    assert int(host(its)[0]) < 200
    assert vg[0] <= 0
    assert abs(abs(float(vg @ v_ref)) - 1.0) < 1e-9
    assert np.max(np.abs(vg - v_ref)) < 1e-6
    assert float(host(lam)[0]) == pytest.approx(lam_ref, rel=1e-9)


@pytest.mark.parametrize("K,N", [(8, 64), (40, 64), (128, 64), (1000, 192), (4096, 4096), (8192, 128)])
def test_pca_fold_and_rotate(q, K, N):
    log(f"pca fold/rotate K={K} N={N}")
    rng = np.random.default_rng(K + N)
    v = rng.standard_normal(K)
    v /= np.linalg.norm(v)
    if v[0] > 0:
        v = -v
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    x = (rng.standard_normal((300, K)) * 4).astype(np.float16)
    wf = host(q.qlin_pca_fold_weight(dev(w), dev(v)))
    xr = host(q.qlin_pca_rotate(dev(x), dev(v)))
    for got, want, what in [(wf, pca.fold_weight(w, v), "folded weights"), (xr, pca.rotate_acts(x, v), "rotated tokens")]:
        d = _ulps(got, want)
        assert d.max() <= 1, what
        assert np.mean(d > 0) <= 1e-3, what


def test_pca_end_to_end_concentrates(q):
    # GPU pipeline on planted data: the rotated extreme tokens carry the
    # planted direction in channel 0, and OffQ's int4 activations of them lose
    # far less than without the rotation.
    x, u = synth.pca_calibration(S=32, T=64, K=1024, seed=9)
    _, z = q.qlin_pca_select(dev(x))
    v, _, _ = q.qlin_pca_leading_eigvec(z)
    assert abs(abs(float(host(v) @ u)) - 1) < 1e-3
    zr = q.qlin_pca_rotate(z, v)
    rng = np.random.default_rng(10)
    signs = rng.choice(np.array([-1, 1], np.int8), 1024)
    signs[::128] = 1

    def rel_err(toks):
        q4, st, zz, _, t = q.qlin_hadamard_offset(toks, dev(signs), want_t=True)
        p = host(q4)
        codes = np.empty((toks.shape[0], 1024), np.int64)
        codes[:, 0::2] = p & 0xF
        codes[:, 1::2] = p >> 4
        deq = (codes - host(zz)[:, None]) * host(st).astype(np.float64)[:, None]
        tt = host(t).astype(np.float64)
        return np.mean((deq - tt) ** 2) / np.mean(tt ** 2)

    assert rel_err(zr) < 0.1 * rel_err(z)
