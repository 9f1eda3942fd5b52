"""Pins of the oracle's quantizers (CPU only).

Each test fixes the oracle against something other than itself: hand-worked
examples (tests/golden/worked_examples.json), exact rational arithmetic,
closed-form invariants, or degenerate cases with a known answer.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant
from tests.exact import f16, f32, rint_half_even

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def test_sym_int8_worked_example():
    g = GOLD["sym_int8_token"]
    q, step = quant.quant_act_sym_int8(np.array([g["x"]], np.float16))
    assert q[0].tolist() == g["q"]
    assert float(step[0]) == g["step"]
    assert Fraction(float(step[0])) == f32(Fraction(2, 127))


def test_sym_int8_zero_token():
    g = GOLD["sym_int8_zero_token"]
    q, step = quant.quant_act_sym_int8(np.array([g["x"]], np.float16))
    assert q[0].tolist() == g["q"] and float(step[0]) == 0.0


def test_sym_int8_matches_exact_rational_rules():
    # Every fp32 operation re-done in exact rationals with one rounding each.
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((4, 37)) * 3).astype(np.float16)
    r = rng.uniform(0.01, 2.0, 37).astype(np.float32)
    q, step = quant.quant_act_sym_int8(x, r)
    for m in range(4):
        v = [f32(Fraction(float(x[m, k])) * Fraction(float(r[k]))) for k in range(37)]
        a = max(abs(t) for t in v)
        inv = f32(Fraction(127) / a)
        assert Fraction(float(step[m])) == f32(a / 127)
        want = [max(-127, min(127, rint_half_even(f32(t * inv)))) for t in v]
        assert q[m].tolist() == want


def test_sym_int8_invariants_outlier_data():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[:, [3, 100, 400]] *= 100
    x = x.astype(np.float16)
    q, step = quant.quant_act_sym_int8(x)
    v = x.astype(np.float64)
    assert q.min() >= -127 and q.max() <= 127
    am = np.argmax(np.abs(v), axis=1)
    assert np.all(np.abs(q[np.arange(64), am]) == 127)
    err = np.abs(q * step[:, None].astype(np.float64) - v)
    assert np.all(err <= step[:, None] * 0.5 * (1 + 1e-4) + 1e-30)


def test_sym_int8_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 128)).astype(np.float16)
    q1, s1 = quant.quant_act_sym_int8(x)
    q2, s2 = quant.quant_act_sym_int8(x, np.full(128, 0.25, np.float32))
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2 * 4, s1)


def test_sym_int8_empty():
    q, s = quant.quant_act_sym_int8(np.zeros((0, 256), np.float16))
    assert q.shape == (0, 256) and s.shape == (0,)


@pytest.mark.parametrize("name", ["asym_int4_token", "asym_int4_tie"])
def test_asym_int4_worked_examples(name):
    g = GOLD[name]
    q, step, z, rs = quant.quant_act_asym_int4(np.array([g["t"]], np.float32))
    assert q[0].tolist() == g["q"]
    assert int(z[0]) == g["z"] and int(rs[0]) == g["rowsum"]
    if "step" in g:
        assert float(step[0]) == g["step"]


def test_asym_int4_invariants():
    rng = np.random.default_rng(7)
    t = (rng.standard_normal((200, 256)) * 10 + rng.uniform(-300, 300, (200, 1))).astype(np.float32)
    q, step, z, rs = quant.quant_act_asym_int4(t)
    assert q.min() >= 0 and q.max() <= 15
    mn = np.argmin(t, axis=1)
    mx = np.argmax(t, axis=1)
    assert np.all(q[np.arange(200), mn] == 0)
    assert np.all(np.isin(q[np.arange(200), mx], [14, 15]))
    deq = (q.astype(np.float64) - z[:, None]) * step[:, None]
    assert np.all(np.abs(deq - t) <= step[:, None] * 0.5 * (1 + 1e-3) + np.abs(t) * 2e-7)
    assert np.array_equal(rs, q.astype(np.int64).sum(axis=1))


def test_asym_int4_constant_token():
    # rng == 0: inv = step = 1, every code equals rint(c) + rint(-c) = 0.
    t = np.full((3, 16), 7.25, np.float32)
    q, step, z, rs = quant.quant_act_asym_int4(t)
    assert np.all(q == 0) and np.all(step == 1) and np.all(z == -7) and np.all(rs == 0)


def test_weight_sym_int8_worked_example():
    g = GOLD["weight_sym_int8_column"]
    w = np.array(g["w"], np.float16)[:, None]
    q, s = quant.quant_weight_sym(w, 8)
    assert float(s[0]) == g["step_fp16"]
    assert Fraction(float(s[0])) == f16(f32(Fraction(1, 127)))
    assert q[:, 0].tolist() == g["q"]


@pytest.mark.parametrize("bits", [8, 4])
def test_weight_sym_invariants(bits):
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((256, 48)) * 0.02).astype(np.float16)
    w[:, 5] = 0
    q, s = quant.quant_weight_sym(w, bits)
    qmax = 127 if bits == 8 else 7
    assert q.min() >= -qmax and q.max() <= qmax
    assert s[5] == 0 and np.all(q[:, 5] == 0)
    wf = w.astype(np.float64)
    sf = s.astype(np.float64)
    am = np.argmax(np.abs(wf), axis=0)
    live = sf > 0
    assert np.all(np.abs(q[am, np.arange(48)][live]) == qmax)
    err = np.abs(q * sf[None, :] - wf)
    assert np.all(err <= sf[None, :] * 0.5 * (1 + 1e-3) + 1e-30)


def test_weight_sym_matches_exact_rational_rules():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((40, 3)) * 0.02).astype(np.float16)
    for bits, qmax, lo in [(8, 127, -127), (4, 7, -8)]:
        q, s = quant.quant_weight_sym(w, bits)
        for n in range(3):
            col = [Fraction(float(v)) for v in w[:, n]]
            a = max(abs(v) for v in col)
            step = f16(f32(a / qmax))
            assert Fraction(float(s[n])) == step
            want = [max(lo, min(qmax, rint_half_even(f32(v / step)))) for v in col]
            assert q[:, n].tolist() == want


def test_group_requant_worked_examples():
    for c in GOLD["group_requant"]["cases"]:
        q4 = np.array([[c["q4"]]], np.int8)
        rg = np.array([[c["r"]]], np.float16)
        assert float(rg[0, 0]) == c["r"]
        assert int(quant.requant_group(q4, rg, group=1)[0, 0]) == c["w8"], c


def test_group_requant_exhaustive_against_exact_rationals():
    # All int4 codes x every finite non-negative fp16 ratio (and their negatives):
    # one fp16 rounding of the exact product, then round half to even, clamp.
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    r = bits.view(np.float16)
    r = np.concatenate([r, -r[1:]])
    q4 = np.arange(-8, 8, dtype=np.int8)
    got = quant.requant_group(np.repeat(q4[:, None], r.size, axis=1),
                              np.tile(r[None, :], (1, 1)).reshape(1, -1), group=16)
    # Independent evaluation: the exact product is a float64 (exact: 4 x 11 bits),
    # rounded once to fp16 by numpy's float64 -> float16 conversion, then Python's
    # round() (half to even).
    prod = q4.astype(np.float64)[:, None] * r.astype(np.float64)[None, :]
    with np.errstate(over="ignore"):
        p16 = prod.astype(np.float16).astype(np.float64)  # products past 65504 become +-inf
    want = np.vectorize(round)(np.clip(p16, -200, 200)).clip(-127, 127)
    assert np.array_equal(got.astype(np.int64), want.astype(np.int64))
    # Spot-check a few entries fully in exact rationals.
    for i, j in [(0, 100), (1, 0x3C00), (15, 0x5A00), (3, 12345)]:
        exact = Fraction(int(q4[i])) * Fraction(float(r[j]))
        assert int(got[i, j]) == max(-127, min(127, rint_half_even(f16(exact))))


def test_group_weights_rules():
    rng = np.random.default_rng(10)
    w = (rng.standard_normal((256, 8)) * 0.02).astype(np.float16)
    w[:128, 2] *= 10  # one group of one column much larger
    q4, sg, sc, rg = quant.quant_weight_group(w, 128)
    assert q4.min() >= -8 and q4.max() <= 7
    for n in range(8):
        col = [Fraction(float(v)) for v in w[:, n]]
        sc_want = f16(f32(max(abs(v) for v in col) / 127))
        assert Fraction(float(sc[n])) == sc_want
        for g in range(2):
            grp = col[g * 128:(g + 1) * 128]
            sg_want = f16(f32(max(abs(v) for v in grp) / 7))
            assert Fraction(float(sg[g, n])) == sg_want
            assert Fraction(float(rg[g, n])) == f16(f32(sg_want / sc_want))
            want = [max(-8, min(7, rint_half_even(f32(v / sg_want)))) for v in grp]
            assert q4[g * 128:(g + 1) * 128, n].tolist() == want
    # Requantized weights stay within int8 and approximate W / s_c.
    w8 = quant.requant_group(q4, rg)
    assert np.abs(w8).max() <= 127
    approx = w8 * sc.astype(np.float64)[None, :]
    bound = (sg.astype(np.float64).repeat(128, 0) * 0.5 + sc.astype(np.float64)[None, :]) * 1.01
    assert np.all(np.abs(approx - w.astype(np.float64)) <= bound)


def test_requant_reduces_to_shift_by_four_when_ratio_is_16():
    # r_g == 16 makes every requantized weight 16 * q4: the per-group path
    # reduces to the per-channel shift-by-4 path.
    q4 = np.arange(-7, 8, dtype=np.int8)[:, None].repeat(4, 1)
    rg = np.full((1, 4), 16.0, np.float16)
    w8 = quant.requant_group(q4, rg, group=15)
    assert np.array_equal(w8.astype(np.int64), 16 * q4.astype(np.int64))
