"""Pins of the oracle's group-wise OffQ path: per-token, per-group
asymmetric int4 activations and the W4A4 product with a step and zero point
per group of k (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import gemm, hadamard, quant
from tests.exact import f32, rint_half_even

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))
FIFTH = float(np.float32(3.0) / np.float32(15.0))


def test_group_quant_worked_example():
    g = GOLD["asym_int4_group_block4"]
    q, step, z, rs = quant.quant_act_asym_int4_group(np.array(g["t"], np.float32), group=g["group"])
    assert q.tolist() == g["q"]
    assert z.tolist() == g["z"] and rs.tolist() == g["rowsum"]
    want_step = [[FIFTH if f else 1.0 for f in row] for row in g["step_is_fifth"]]
    assert step.tolist() == want_step


def test_group_gemm_worked_example():
    g = GOLD["w4a4_group_block4"]
    a = GOLD["asym_int4_group_block4"]
    qa = np.array(a["q"])
    za = np.array(a["z"])
    sa = np.array([[FIFTH if f else 1.0 for f in row] for row in a["step_is_fifth"]])
    y, acc = gemm.w4a4_group(qa, sa, za, np.array(g["qw"]), np.array(g["sw"]), np.array(g["zw"]),
                             group=a["group"], return_acc=True)
    assert acc.tolist() == g["acc"]
    for m, (cs, c0) in enumerate(g["y_over_s"]):
        assert y[m, 0] == pytest.approx(cs * FIFTH + c0, rel=1e-14)


def test_group_quant_matches_exact_rational_rules():
    # Every decision re-derived with exact rationals rounded to fp32 where the
    # rule rounds, group by group, element by element.
    rng = np.random.default_rng(11)
    M, group, G = 3, 32, 4
    t = (rng.standard_normal((M, group * G)) * rng.uniform(0.1, 50, (M, 1))
         + rng.uniform(-300, 300, (M, G)).repeat(group, axis=1)).astype(np.float32)
    t[1, group:2 * group] = 7.25  # a constant group
    q, step, z, rs = quant.quant_act_asym_int4_group(t, group)
    for m in range(M):
        for g in range(G):
            vals = [Fraction(float(v)) for v in t[m, g * group:(g + 1) * group]]
            mn, mx = min(vals), max(vals)
            rngv = f32(mx - mn)
            inv = Fraction(1) if rngv == 0 else f32(Fraction(15) / rngv)
            stp = Fraction(1) if rngv == 0 else f32(rngv / 15)
            zz = rint_half_even(f32(-mn * inv))
            codes = [min(15, max(0, rint_half_even(f32(v * inv)) + zz)) for v in vals]
            assert Fraction(float(step[m, g])) == stp
            assert int(z[m, g]) == zz
            assert q[m, g * group:(g + 1) * group].tolist() == codes
            assert int(rs[m, g]) == sum(codes)


def test_group_quant_invariants():
    rng = np.random.default_rng(12)
    M, K = 50, 512
    t = (rng.standard_normal((M, K)) * 3 + rng.uniform(-500, 500, (M, K // 128)).repeat(128, axis=1)).astype(np.float32)
    q, step, z, rs = quant.quant_act_asym_int4_group(t)
    assert q.min() >= 0 and q.max() <= 15
    tg = t.reshape(M, 4, 128)
    qg = q.reshape(M, 4, 128).astype(np.int64)
    for g in range(4):
        assert np.all(qg[np.arange(M), g, np.argmin(tg[:, g], axis=1)] == 0)
        assert np.all(np.isin(qg[np.arange(M), g, np.argmax(tg[:, g], axis=1)], [14, 15]))
    deq = (qg - z[:, :, None]) * step.astype(np.float64)[:, :, None]
    assert np.all(np.abs(deq - tg) <= step[:, :, None] * 0.5 * (1 + 1e-3) + np.abs(tg) * 2e-7)
    assert np.array_equal(rs, qg.sum(axis=2))


def test_group_offsets_land_in_the_zero_points():
    # Integer values 0..15 in every group (min 0 and max 15 present), plus a
    # different integer offset per group: each group's step stays 1, its codes
    # are the values themselves and its zero point is minus the offset, so the
    # group-wise dequantization is exact.  One step per token cannot do that.
    rng = np.random.default_rng(13)
    M, G = 4, 4
    base = rng.integers(0, 16, (M, G, 128))
    base[:, :, 0] = 0
    base[:, :, 1] = 15
    offs = np.array([0, 200, -50, 1000])
    t = (base + offs[None, :, None]).reshape(M, G * 128).astype(np.float32)
    q, step, z, rs = quant.quant_act_asym_int4_group(t)
    assert np.all(step == 1)
    assert np.array_equal(q.reshape(M, G, 128), base)
    assert np.array_equal(z, np.broadcast_to(-offs, (M, G)))
    deq = (q.reshape(M, G, 128).astype(np.int64) - z[:, :, None]) * step[:, :, None]
    assert np.array_equal(deq.reshape(M, -1), t)
    qt, st, zt, _ = quant.quant_act_asym_int4(t)
    err_token = np.abs((qt.astype(np.int64) - zt[:, None]) * st[:, None].astype(np.float64) - t).max()
    assert err_token > 10


def test_group_wise_error_beats_per_token_on_offq_data():
    # OffQ-style activations: a different large outlier in the first channel
    # of every block; after the transform each block carries its own offset.
    rng = np.random.default_rng(14)
    M, K = 64, 1024
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, ::128] = rng.uniform(-300, 300, (1, K // 128))
    x = x.astype(np.float16)
    d = rng.choice(np.array([-1, 1], np.int8), K)
    d[::128] = 1
    qg, sg, zg, _, t = quant.hadamard_offset_int4_group(x, d)
    qt, st, zt, _, _ = quant.hadamard_offset_int4(x, d)
    deq_g = ((qg.reshape(M, -1, 128).astype(np.int64) - zg[:, :, None]) * sg[:, :, None]).reshape(M, K)
    deq_t = (qt.astype(np.int64) - zt[:, None]) * st[:, None]
    mse_g = np.mean((deq_g - t) ** 2)
    mse_t = np.mean((deq_t - t) ** 2)
    assert mse_g * 10 < mse_t


def test_group_gemm_equals_dequantized_product():
    # The per-group integer route against a float64 product of the
    # dequantized operands (different arithmetic, same value).
    rng = np.random.default_rng(15)
    M, K, N = 7, 384, 9
    qa = rng.integers(0, 16, (M, K))
    qw = rng.integers(0, 16, (K, N))
    za = rng.integers(-600, 20, (M, K // 128))
    zw = rng.integers(-3, 19, N)
    sa = rng.uniform(0.01, 2, (M, K // 128))
    sw = rng.uniform(0.001, 0.1, N)
    y = gemm.w4a4_group(qa, sa, za, qw, sw, zw)
    xa = (qa - np.repeat(za, 128, axis=1)) * np.repeat(sa, 128, axis=1)
    xw = (qw - zw[None, :]) * sw[None, :]
    ref = xa @ xw
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_group_gemm_brute_force_acc():
    rng = np.random.default_rng(16)
    M, K, N, group = 3, 24, 2, 8
    qa = rng.integers(0, 16, (M, K))
    qw = rng.integers(0, 16, (K, N))
    za = rng.integers(-40, 20, (M, K // group))
    zw = rng.integers(0, 16, N)
    _, acc = gemm.w4a4_group(qa, np.ones((M, K // group)), za, qw, np.ones(N), zw, group=group, return_acc=True)
    for g in range(K // group):
        for m in range(M):
            for n in range(N):
                want = sum((int(qa[m, k]) - int(za[m, g])) * (int(qw[k, n]) - int(zw[n]))
                           for k in range(g * group, (g + 1) * group))
                assert acc[g, m, n] == want


def test_group_gemm_one_group_is_the_per_token_gemm():
    # With K = one group the two forms are the same product.
    rng = np.random.default_rng(17)
    qa = rng.integers(0, 16, (5, 128))
    qw = rng.integers(0, 16, (128, 4))
    za = rng.integers(-100, 20, 5)
    zw = rng.integers(0, 16, 4)
    sa = rng.uniform(0.1, 1, 5)
    sw = rng.uniform(0.1, 1, 4)
    acc, y_tok = gemm.w4a4(qa, sa, za, qw, sw, zw)
    y_grp = gemm.w4a4_group(qa, sa[:, None], za[:, None], qw, sw, zw)
    assert np.allclose(y_grp, y_tok, rtol=1e-14, atol=0)


def test_weight_colsum_group_brute_force():
    rng = np.random.default_rng(18)
    qw = rng.integers(0, 16, (256, 5)).astype(np.uint8)
    cs = quant.weight_colsum_group(qw)
    assert cs.shape == (2, 5) and cs.dtype == np.int32
    for g in range(2):
        for n in range(5):
            assert cs[g, n] == sum(int(qw[k, n]) for k in range(128 * g, 128 * g + 128))
    with pytest.raises(ValueError):
        quant.weight_colsum_group(qw[:100])


def test_group_layer_preserves_xw():
    # End to end: the group-wise layer output approximates x W in float64.
    rng = np.random.default_rng(19)
    M, K, N = 16, 512, 32
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, ::128] = rng.uniform(-200, 200, (1, K // 128))
    x = x.astype(np.float16)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    d = rng.choice(np.array([-1, 1], np.int8), K)
    d[::128] = 1
    from oracle import layer
    out = layer.offq_group_forward(x, w, d)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    tok = layer.offq_forward(x, w, d)
    err_g = np.abs(out["y"] - ref).max() / np.abs(ref).max()
    err_t = np.abs(tok["y"] - ref).max() / np.abs(ref).max()
    assert err_g < 0.1 and err_g < err_t
