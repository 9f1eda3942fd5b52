"""GPU parity of qlin_quaff_momentum_quant: one Quaff step's activation side
(Quaff notes, "key design": the targeted momentum update of s on the fixed
outlier set O, then the per-token INT8 quantization of X * r and the
compensation operand fp16(q[:, O] * (s[O] - 1)) with the new s and r).

Checked bit for bit over ten steps against the oracle (quaff.momentum_update,
quant.quant_act_sym_int8), and against the two library calls it stands for.
The cases cover the folded form (a workspace, 1 <= nO <= 256, K <= 8192) at
both register widths of the quantizer, ragged token counts, fewer tokens than
row blocks, and each condition that selects the two-call form instead.
"""
import numpy as np
import pytest

import synth
from oracle import quant, quaff
from tests.gpu_helpers import assert_equal, dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    assert torch.cuda.is_available()
    from outlier_aware_bit_amd import qlin
    return qlin


def _steps(M, K, nO, seed):
    d = synth.quaff_steps(M=max(M, 1), K=K, N=64, n_outliers=max(nO, 1), steps=10, seed=seed)
    O = d.outliers[:nO].astype(np.int32)
    wmax = np.random.default_rng(seed).uniform(0.0, 0.1, nO).astype(np.float32)
    if nO > 1:
        wmax[1] = 0.0  # beta = 1 for that channel
    return [x[:M] for x in d.xs], O, wmax


@pytest.mark.parametrize("M,K,nO,work", [
    (1, 256, 3, True),        # fewer tokens than row blocks
    (5, 128, 7, True),        # the shortest rows (two 64-channel strips)
    (2, 384, 1, True),        # one outlier channel
    (3, 1024, 16, True),
    (70, 1024, 13, True),
    (513, 4096, 205, True),   # ragged, the q_proj channel count
    (300, 8192, 256, True),   # eight register chunks, the largest slot count
    (130, 2048, 64, False),   # no workspace: the two calls
    (200, 1024, 300, True),   # nO > 256: the two calls
    (64, 8320, 40, True),     # K > 8192: the two calls
    (50, 1024, 0, True),      # no outliers
    (0, 1024, 10, True),      # no tokens: the momentum update alone
])
def test_momentum_quant_ten_steps(q, M, K, nO, work):
    import torch
    log(f"momentum+quant M={M} K={K} nO={nO} work={work}")
    xs, O, wmax = _steps(M, K, nO, seed=M + K + nO)
    s_ref = np.ones(K, np.float32)
    s = torch.ones(K, dtype=torch.float32, device="cuda")
    r = torch.full((K,), float("nan"), dtype=torch.float32, device="cuda")
    Od, wd = dev(O), dev(wmax)
    wk = None
    if work:
        nb = q.qlin_quaff_momentum_quant_work_bytes(M, nO)
        wk = torch.full((max(nb // 4, 1),), float("nan"), dtype=torch.float32, device="cuda")
    ld = q.qlin_outlier_ld(nO)
    for t, x in enumerate(xs):
        s_ref, r_ref = quaff.momentum_update(x, O, wmax, 0.9, s_ref)
        qq, sa, xO = q.qlin_quaff_momentum_quant(dev(x), Od, wd, 0.9, s, r, work=wk)
        assert_equal(host(s), s_ref, f"s step {t}")
        assert_equal(host(r), r_ref, f"r step {t}")
        if M == 0:
            continue
        q_ref, sa_ref = quant.quant_act_sym_int8(x, r_ref)
        assert_equal(host(qq), q_ref, f"codes step {t}")
        assert_equal(host(sa), sa_ref, f"steps step {t}")
        if nO:
            want_x = (q_ref[:, O].astype(np.float32) * (s_ref[O] - np.float32(1))).astype(np.float16)
            got = host(xO)
            assert got.shape == (M, ld)
            assert_equal(got[:, :nO].view(np.uint16), want_x.view(np.uint16), f"xO step {t}")
            assert np.all(got[:, nO:] == 0), f"xO padding step {t}"
        else:
            assert xO is None


def test_momentum_quant_q_proj_matches_separate_calls(q):
    """The q_proj workload (2048 x 4096, |O| = 205): the folded call and the
    momentum update followed by the quantizer give the same bits at every one
    of ten steps; the first three steps are also checked against the oracle."""
    import torch
    M, K, nO = 2048, 4096, 205
    log(f"momentum+quant q_proj {M}x{K} |O|={nO}, 10 steps")
    xs, O, wmax = _steps(M, K, nO, seed=11)
    Od, wd = dev(O), dev(wmax)
    s1 = torch.ones(K, dtype=torch.float32, device="cuda")
    r1 = torch.empty_like(s1)
    s2, r2 = s1.clone(), r1.clone()
    wk = torch.full((q.qlin_quaff_momentum_quant_work_bytes(M, nO) // 4,), float("nan"), dtype=torch.float32,
                    device="cuda")
    s_ref = np.ones(K, np.float32)
    for t, x in enumerate(xs):
        xd = dev(x)
        qa, sa, xO = q.qlin_quaff_momentum_quant(xd, Od, wd, 0.9, s1, r1, work=wk)
        q.qlin_momentum_update(xd, Od, wd, 0.9, s2, r2)
        qb, sb, _, xOb = q.qlin_quant_act(xd, r2, Od, s=s2, want_qO=False)
        assert_equal(host(s1), host(s2), f"s step {t}")
        assert_equal(host(r1), host(r2), f"r step {t}")
        assert_equal(host(qa), host(qb), f"codes step {t}")
        assert_equal(host(sa), host(sb), f"steps step {t}")
        assert_equal(host(xO).view(np.uint16), host(xOb).view(np.uint16), f"xO step {t}")
        if t < 3:
            s_ref, r_ref = quaff.momentum_update(x, O, wmax, 0.9, s_ref)
            q_ref, sa_ref = quant.quant_act_sym_int8(x, r_ref)
            assert_equal(host(s1), s_ref, f"s oracle step {t}")
            assert_equal(host(qa), q_ref, f"codes oracle step {t}")
            assert_equal(host(sa), sa_ref, f"steps oracle step {t}")
