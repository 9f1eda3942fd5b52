"""The allocation-free momentum update, qlin_momentum_update_noalloc (for
callers that cannot allocate device memory), called through the C ABI and
checked bit for bit against the entry point that takes a workspace, and
against the oracle: two calls in a row on the library's static scratch, the
second with a smaller batch and fewer outlier channels, so that it runs on
the partial maxima the first call left behind."""
import numpy as np
import pytest

import synth
from oracle import quaff
from tests.gpu_helpers import assert_equal, dev, host, log

pytestmark = pytest.mark.gpu


def test_momentum_noalloc_matches_workspace_entry_point():
    import torch
    from outlier_aware_bit_amd import _lib
    from outlier_aware_bit_amd import qlin as q
    lib = _lib.load()
    # (M, K, nO): batches long enough for the two-launch form that uses the
    # scratch (M >= 4096): 8192 tokens at the q_proj width, then a smaller one.
    for M, K, nO, seed in [(8192, 4096, 205, 31), (4500, 1024, 51, 32)]:
        log(f"momentum noalloc M={M} K={K} nO={nO}")
        d = synth.quaff_steps(M=M, K=K, N=64, n_outliers=nO, steps=3, seed=seed)
        wmax = np.random.default_rng(seed).uniform(0.01, 0.1, nO).astype(np.float32)
        O, wd = dev(d.outliers.astype(np.int32)), dev(wmax)
        s1 = torch.ones(K, dtype=torch.float32, device="cuda")
        r1 = torch.empty_like(s1)
        s2 = torch.ones(K, dtype=torch.float32, device="cuda")
        r2 = torch.full_like(s2, float("nan"))
        work = torch.empty((q.qlin_momentum_work_bytes(M, nO) // 4,), dtype=torch.float32, device="cuda")
        s_ref = np.ones(K, np.float32)
        for t, x in enumerate(d.xs):
            xd = dev(x)
            s_ref, r_ref = quaff.momentum_update(x, d.outliers, wmax, 0.9, s_ref)
            q.qlin_momentum_update(xd, O, wd, 0.9, s1, r1, work=work)
            st = lib.qlin_momentum_update_noalloc(xd.data_ptr(), M, K, O.data_ptr(), nO, wd.data_ptr(), 0.9,
                                                  s2.data_ptr(), r2.data_ptr(),
                                                  torch.cuda.current_stream().cuda_stream)
            assert st == _lib.QLIN_OK, lib.qlin_last_error().decode()
            torch.cuda.synchronize()
            assert_equal(host(s2), host(s1), f"s, step {t}")
            assert_equal(host(r2), host(r1), f"r, step {t}")
            assert_equal(host(s2), s_ref, f"s vs oracle, step {t}")
            assert_equal(host(r2), r_ref, f"r vs oracle, step {t}")


def test_momentum_noalloc_rejects_more_outliers_than_the_scratch_holds():
    from outlier_aware_bit_amd import _lib
    lib = _lib.load()
    A = 0x10000
    assert lib.qlin_momentum_update_noalloc(A, 8, 16384, A, 8193, A, 0.9, A, A, None) == _lib.QLIN_ERR_SHAPE
    assert lib.qlin_momentum_update_noalloc(A, 8, 256, A, 4, A, 1.5, A, A, None) == _lib.QLIN_ERR_INVALID_ARG
