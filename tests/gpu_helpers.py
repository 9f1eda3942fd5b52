"""Host-side helpers shared by the GPU parity tests (no method arithmetic)."""
import sys

import numpy as np

TOL = 1e-3  # normwise max|y - y_ref| / max|y_ref| on fp16 outputs


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def assert_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {got[i]!r} want {want[i]!r}")


def assert_close(y, y_ref, what, tol=TOL):
    from oracle.gemm import max_abs_rel
    err = max_abs_rel(np.asarray(y, np.float64), y_ref)
    assert np.all(np.isfinite(np.asarray(y, np.float64))), what
    assert err <= tol, f"{what}: normwise error {err:.3e} > {tol}"
    return err
