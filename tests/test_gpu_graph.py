"""The Quaff layer step (momentum update -> quantization with the compensation
operand -> fused W8A8 GEMM) captured into HIP graphs and replayed, checked
bit for bit against the same step launched eagerly from the same state; the
first two as separate calls, or as one qlin_quaff_momentum_quant call with a
workspace (its maxima kernel leaves markers in r that the quantizer reads).

The momentum state s is updated in place by every step, so the eager and the
graph paths each own a copy of it.  Replays alternate between two activation
batches, with unrelated eager work and host synchronisations between them,
and every replay is compared (s, r, codes, steps, compensation operand, y).
"""
import numpy as np
import pytest

import synth
from tests.gpu_helpers import assert_equal, dev, host, log

pytestmark = pytest.mark.gpu


class _Step:
    def __init__(self, q, d, w8, sw, WOp, wmax, O, nO, fold):
        import torch
        M, K = d.xs[0].shape
        N = d.w.shape[1]
        self.q, self.w8, self.sw, self.WOp, self.wmax, self.O, self.nO, self.N = q, w8, sw, WOp, wmax, O, nO, N
        self.s = torch.ones(K, dtype=torch.float32, device="cuda")
        self.r = torch.empty_like(self.s)
        self.qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
        self.sa = torch.empty((M,), dtype=torch.float32, device="cuda")
        self.xO = torch.empty((M, q.qlin_outlier_ld(nO)), dtype=torch.float16, device="cuda")
        self.y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        self.work = (torch.empty((q.qlin_quaff_momentum_quant_work_bytes(M, nO) // 4,), dtype=torch.float32,
                                 device="cuda") if fold else None)

    def run(self, x):
        q = self.q
        if self.work is not None:
            q.qlin_quaff_momentum_quant(x, self.O, self.wmax, 0.9, self.s, self.r, work=self.work, q=self.qa,
                                        scale=self.sa, xO=self.xO)
        else:
            q.qlin_momentum_update(x, self.O, self.wmax, 0.9, self.s, self.r)
            q.qlin_quant_act(x, self.r, self.O, s=self.s, q=self.qa, scale=self.sa, xO=self.xO, want_qO=False)
        q.qlin_gemm_w8a8(self.qa, self.sa, self.w8, self.sw, self.N, xO=self.xO, nO=self.nO, WO=self.WOp, y=self.y)

    def state(self):
        return [host(t) for t in (self.s, self.r, self.qa, self.sa, self.xO, self.y)]


@pytest.mark.parametrize("fold", [False, True], ids=["two_calls", "folded"])
def test_quaff_step_graph_replays_match_eager(fold):
    import torch
    from outlier_aware_bit_amd import qlin as q
    M, K, N, nO = 1024, 1024, 512, 51
    log(f"graph replay of the Quaff step M={M} K={K} N={N} |O|={nO} fold={fold}")
    d = synth.quaff_steps(M=M, K=K, N=N, n_outliers=nO, steps=2, seed=11)
    codes, sw = q.qlin_quant_weight_sym(dev(d.w), 8)
    w8 = q.qlin_pack_weight(q.QLIN_LAYOUT_W8, codes)
    WO = dev(np.ascontiguousarray(d.w[d.outliers]))
    WOp = q.qlin_pack_weight(q.QLIN_LAYOUT_WO, WO)
    wmax = q.qlin_weight_row_absmax(WO)
    O = dev(d.outliers)
    xs = [dev(x) for x in d.xs]
    eager = _Step(q, d, w8, sw, WOp, wmax, O, nO, fold)
    graphed = _Step(q, d, w8, sw, WOp, wmax, O, nO, fold)
    torch.cuda.synchronize()

    graphs = []
    for x in xs:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            graphed.run(x)
        graphs.append(g)
    torch.cuda.synchronize()
    # Capture launches nothing: the graph path's state is still the initial one.
    assert_equal(host(graphed.s), np.ones(K, np.float32), "s after capture")

    scratch = torch.randn(1 << 20, device="cuda")
    for t in range(6):
        b = t % 2
        eager.run(xs[b])
        scratch.mul_(1.0001).add_(0.5)  # unrelated eager work between replays
        torch.cuda.synchronize()
        graphs[b].replay()
        torch.cuda.synchronize()
        names = ("s", "r", "codes", "steps", "xO", "y")
        for name, a, g in zip(names, eager.state(), graphed.state()):
            assert_equal(g.view(np.uint8), a.view(np.uint8), f"replay {t}: {name}")
        log(f"  replay {t} matches")
