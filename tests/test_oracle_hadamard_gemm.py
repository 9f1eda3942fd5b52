"""Pins of the oracle's Hadamard transform and integer GEMMs (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle import gemm, hadamard, quant
from tests.exact import sylvester_entry

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_sylvester_matches_scipy_and_popcount_formula(n):
    h = hadamard.sylvester(n)
    assert np.array_equal(h, scipy.linalg.hadamard(n))
    assert all(h[i, j] == sylvester_entry(i, j) for i in range(n) for j in range(n))
    assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))


def test_partial_random_first_row_all_ones_and_orthogonal():
    rng = np.random.default_rng(0)
    d = rng.choice(np.array([-1, 1], np.int8), 128)
    d[0] = 1
    hp = hadamard.partial_random(d)
    assert np.all(hp[0] == 1)
    assert np.array_equal(hp @ hp.T, 128 * np.eye(128, dtype=np.int64))
    with pytest.raises(ValueError):
        d[0] = -1
        hadamard.partial_random(d)


def test_block_transform_worked_example():
    g = GOLD["hadamard_offset_block4"]
    x = np.array([g["x"]], np.float16)
    t = hadamard.transform_blocks(x, np.array(g["signs"], np.int8), block=g["block"])
    assert t[0].tolist() == g["t"]
    q, step, z, rs, _ = quant.hadamard_offset_int4(x, np.array(g["signs"], np.int8), block=g["block"])
    assert q[0].tolist() == g["q"] and int(z[0]) == g["z"] and int(rs[0]) == g["rowsum"]


def test_outlier_channel_becomes_constant_offset():
    # Only the first channel of each group is non-zero: the transform spreads it
    # as the same constant over every channel of the group (row 0 is all ones).
    rng = np.random.default_rng(1)
    K = 512
    d = rng.choice(np.array([-1, 1], np.int8), K)
    d[::128] = 1
    x = np.zeros((3, K), np.float16)
    x[:, ::128] = np.array([[200.0, -3.5, 17.25, 0.5]] * 3, np.float16)
    t = hadamard.transform_blocks(x, d)
    for b in range(4):
        blk = t[:, b * 128:(b + 1) * 128]
        assert np.all(blk == blk[:, :1])
        assert blk[0, 0] == float(x[0, b * 128])
    # A token that is one group with only channel 0 set is constant after the
    # transform, so its range is 0 and the degenerate quantizer branch applies.
    q, step, z, rs, _ = quant.hadamard_offset_int4(x[:, :128], d[:128])
    assert np.all(q == 0) and np.all(step == 1)


def test_block_transform_brute_force_exact():
    # Python-integer brute force with the popcount formula, on fp16 inputs that
    # are small dyadic rationals (so Fraction arithmetic is exact).
    rng = np.random.default_rng(2)
    K, block = 64, 16
    x = (rng.integers(-2000, 2000, (2, K)) / 64).astype(np.float16)
    d = rng.choice(np.array([-1, 1], np.int8), K)
    d[::block] = 1
    t = hadamard.transform_blocks(x, d, block)
    for m in range(2):
        for b in range(K // block):
            for j in range(block):
                want = sum(Fraction(float(x[m, b * block + i])) * int(d[b * block + i]) * sylvester_entry(i, j)
                           for i in range(block))
                assert Fraction(t[m, b * block + j]) == want


def test_block_transform_exact_at_fp16_extremes():
    # Largest and smallest fp16 magnitudes in one group: float64 keeps every
    # partial sum exact (47 significant bits at most).
    x = np.zeros((1, 128), np.float16)
    x[0, 0] = 65504
    x[0, 1] = np.float16(2.0 ** -24)
    x[0, 2] = -65504
    x[0, 3] = np.float16(2.0 ** -14)
    d = np.ones(128, np.int8)
    t = hadamard.transform_blocks(x, d)
    for j in range(128):
        want = (Fraction(65504) * sylvester_entry(0, j) + Fraction(1, 2 ** 24) * sylvester_entry(1, j)
                - Fraction(65504) * sylvester_entry(2, j) + Fraction(1, 2 ** 14) * sylvester_entry(3, j))
        assert Fraction(t[0, j]) == want


def test_parseval_and_weight_inverse_restore_xw():
    rng = np.random.default_rng(3)
    M, K, N = 4, 256, 6
    x = (rng.integers(-64, 64, (M, K)) / 8).astype(np.float16)
    w = (rng.integers(-64, 64, (K, N)) / 1024).astype(np.float16)
    d = rng.choice(np.array([-1, 1], np.int8), K)
    d[::128] = 1
    t = hadamard.transform_blocks(x, d)
    xf = x.astype(np.float64)
    assert np.array_equal((t * t).sum(1), 128 * (xf * xf).sum(1))
    w2 = hadamard.inverse_transform_weight(w, d)
    assert np.array_equal(t @ w2, xf @ w.astype(np.float64))


def test_exact_int_matmul_brute_force():
    rng = np.random.default_rng(4)
    a = rng.integers(-127, 128, (5, 37))
    b = rng.integers(-127, 128, (37, 3))
    got = gemm.exact_int_matmul(a, b)
    for m in range(5):
        for n in range(3):
            assert got[m, n] == sum(int(a[m, k]) * int(b[k, n]) for k in range(37))
    with pytest.raises(ValueError):
        gemm.exact_int_matmul(np.full((1, 2 ** 20), 2 ** 20), np.full((2 ** 20, 1), 2 ** 14))


def test_w4a4_worked_example():
    g = GOLD["w4a4_zero_point"]
    acc, y = gemm.w4a4(np.array(g["qa"]), np.ones(2), np.array(g["za"]),
                       np.array(g["qw"]), np.ones(2), np.array(g["zw"]))
    assert acc.tolist() == g["acc"]


def test_w4a4_zero_point_expansion_brute_force():
    # sum_k (qa - za)(qw - zw) == raw - zw*rowsum - za*colsum + K*za*zw.
    rng = np.random.default_rng(5)
    M, K, N = 6, 40, 5
    qa = rng.integers(0, 16, (M, K))
    qw = rng.integers(0, 16, (K, N))
    za = rng.integers(-20, 20, M)
    zw = rng.integers(-3, 19, N)
    acc, _ = gemm.w4a4(qa, np.ones(M), za, qw, np.ones(N), zw)
    raw = gemm.w4a4_raw(qa, qw)
    for m in range(M):
        rowsum = sum(int(v) for v in qa[m])
        for n in range(N):
            colsum = sum(int(v) for v in qw[:, n])
            direct = sum((int(qa[m, k]) - int(za[m])) * (int(qw[k, n]) - int(zw[n])) for k in range(K))
            expanded = int(raw[m, n]) - int(zw[n]) * rowsum - int(za[m]) * colsum + K * int(za[m]) * int(zw[n])
            assert acc[m, n] == direct == expanded


def test_shift_by_four_is_times_sixteen():
    # QQQ's INT4 -> INT8 conversion: a nibble moved to the high half of a byte
    # reads, as a signed byte, as 16 times its two's-complement value.
    for n in range(16):
        signed = n - 16 if n >= 8 else n
        byte = np.array([n << 4], np.uint8).view(np.int8)[0]
        assert int(byte) == 16 * signed


def test_w8a8_dequant_and_error_bound():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((32, 256)).astype(np.float32)
    x[:, [7, 99]] *= 100
    x = x.astype(np.float16)
    w = (rng.standard_normal((256, 64)) * 0.02).astype(np.float16)
    q, sa = quant.quant_act_sym_int8(x)
    qw, sw = quant.quant_weight_sym(w, 8)
    acc, y = gemm.w8a8(q, sa, qw, sw.astype(np.float32))
    xf, wf = x.astype(np.float64), w.astype(np.float64)
    da, dw = sa.astype(np.float64)[:, None], sw.astype(np.float64)[None, :]
    bound = (np.abs(xf) @ np.ones_like(wf)) * dw / 2 + (np.ones_like(xf) @ np.abs(wf)) * da / 2 + 256 * da * dw / 4
    assert np.all(np.abs(y - xf @ wf) <= bound * 1.001)
    assert gemm.max_abs_rel(y, y) == 0.0


def test_max_abs_rel_worked_examples():
    # The parity measure itself, against hand-worked values: the denominator
    # is max|y_ref| (not max|y|), the numerator the largest signed difference.
    for c in GOLD["max_abs_rel_cases"]["cases"]:
        y = np.asarray(c["y"], np.float64)
        y_ref = np.asarray(c["y_ref"], np.float64)
        got = gemm.max_abs_rel(y, y_ref)
        if c.get("inf"):
            assert got == float("inf"), c["derivation"]
        else:
            assert Fraction(got).limit_denominator(1000) == Fraction(c["num"], c["den"]), c["derivation"]


def test_max_abs_rel_flags_a_planted_error():
    # One element off by 2e-3 of the reference's largest magnitude must fail
    # the 1e-3 bar, whatever the other elements hold.
    rng = np.random.default_rng(3)
    y_ref = rng.standard_normal((64, 64))
    y = y_ref.copy()
    y[17, 5] += 2e-3 * np.max(np.abs(y_ref))
    assert 1.99e-3 < gemm.max_abs_rel(y, y_ref) < 2.01e-3


def test_offq_weight_worked_example():
    g = GOLD["offq_weight_block4"]
    w = np.asarray(g["w"], np.float16)
    signs = np.asarray(g["signs"], np.int64)
    wt = hadamard.inverse_transform_weight(w, signs, g["block"])
    assert np.array_equal(wt, np.asarray(g["w_transformed"], np.float64))
    qw, step, zw, colsum = quant.offq_weight(w, signs, g["block"])
    assert np.array_equal(qw, np.asarray(g["q"], np.uint8))
    want_step = [np.float32(n) / np.float32(d) for n, d in zip(g["step_num"], g["step_den"])]
    assert np.array_equal(step, np.asarray(want_step, np.float32))
    assert np.array_equal(zw, np.asarray(g["z"], np.int32))
    assert np.array_equal(colsum, np.asarray(g["colsum"], np.int32))
