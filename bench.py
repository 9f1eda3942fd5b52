"""Benchmark of the outlier-aware quantized linear layer on one MI355X.

The headline workload is the Quaff W8A8 layer at LLaMA-7B q_proj shape:
X [2048 x 4096] fp16 with a fixed 5% outlier channel set (205 channels at
50-150x, drifting 5% per step over 10 activation batches), W [4096 x 4096]
pre-quantized to int8 per output channel, fp16 rows W_O on the outlier set,
momentum gamma = 0.9.  One step is one forward of the layer on one batch:
  momentum update of s on O  ->  per-token int8 quantization of X / s
  ->  W8A8 int8-MFMA GEMM with the fused compensation term  ->  Y fp16.
The first two run as one qlin_quaff_momentum_quant call (the momentum
maxima over row blocks, folded by the quantizer; bit-identical to the
momentum update followed by the quantizer).

Printed: one JSON line with the step throughput (TOPS of the layer's
algorithmic work), the roofline of the dominant kernel (the fused GEMM) timed
with HIP events on its own stream, the CPU oracle timed on the host on a
bounded sample, and per-kernel measurements of the other steps of the path at
their own workload shapes ("rows").

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-rows]
                       [--copy-calibration]

--copy-calibration first runs a plain device-to-device copy of a known size
(256 MiB read, 256 MiB written, three times) so that a counter run
(rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE) can scale the GEMM's counter
readings to bytes.  The scaled per-launch traffic is kept in
profiles/gemm_w8a8_comp_q_proj_traffic.md together with a SHA-256 of the GEMM
kernel's sources; roofline.traffic reports it only while the sources still
hash to that value, and null otherwise.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized-linear TOPS and HBM GB/s at LLaMA-7B layer shapes; % of roofline"
PEAK_INT8_TOPS = 5000.0   # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_FP16_TFLOPS = 2500.0  # dense fp16 MFMA
PEAK_HBM_GBS = 8000.0      # HBM3E, 8 TB/s
MALL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w8a8_comp_q_proj_traffic.md")
# Sources that make up the fused W8A8 GEMM kernel.
GEMM_SOURCES = ["gemm.hip", "comp.hpp", "layout.hpp", "common.hpp"]
COPY_CALIB_BYTES = 256 << 20
GEMM_KERNEL = "gemm_tile<W8,I8,comp>"


def gemm_sources_sha256():
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "outlier_aware_bit_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """Per-launch HBM bytes of the fused GEMM from the committed counter
    summary, or None when it is absent or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    kv = dict(re.findall(r"^- (\w+): `([^`]*)`", text, flags=re.M))
    if kv.get("kernel_sources_sha256") != gemm_sources_sha256():
        return None
    try:
        return {"read": int(kv["read_bytes_per_launch"]), "write": int(kv["write_bytes_per_launch"])}
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain copy of COPY_CALIB_BYTES, three times, for counter scaling."""
    import torch
    src = torch.ones(COPY_CALIB_BYTES // 2, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


class FenceFreeEvent:
    """A HIP timing event created with hipEventDisableSystemFence, through the
    HIP runtime torch has loaded.  Recording a default event releases and
    acquires at system scope, which writes back and invalidates the caches:
    about 2 us per record on the GPU timeline, and a cold L2 for the kernel
    that follows.  These events only timestamp the stream; they are read
    after a device synchronisation."""
    _lib = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    @classmethod
    def _hip(cls):
        if cls._lib is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64.so" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded")
            lib = ctypes.CDLL(path)
            v, i = ctypes.c_void_p, ctypes.c_int
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(v), ctypes.c_uint]
            lib.hipEventCreateWithFlags.restype = i
            lib.hipEventRecord.argtypes = [v, v]
            lib.hipEventRecord.restype = i
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), v, v]
            lib.hipEventElapsedTime.restype = i
            lib.hipEventDestroy.argtypes = [v]
            lib.hipEventDestroy.restype = i
            cls._lib = lib
        return cls._lib

    def __init__(self):
        import ctypes
        self.ev = ctypes.c_void_p()
        rc = self._hip().hipEventCreateWithFlags(ctypes.byref(self.ev), self.FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags: {rc}")

    def record(self):
        import torch
        rc = self._hip().hipEventRecord(self.ev, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord: {rc}")

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        rc = self._hip().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime: {rc}")
        return ms.value

    def __del__(self):
        if self._lib is not None and self.ev:
            self._lib.hipEventDestroy(self.ev)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


PROFILE_LAUNCHES = 0  # > 0: rows launch eagerly this many times each, untimed (counter runs)


def time_launches(fn, reps, trials=5, warm=3, graph_len=24):
    """Median over trials of the mean per-launch time (ms) of `reps`
    back-to-back calls, timed with HIP events on the current stream.

    The calls are captured once into a HIP graph of `graph_len` launches
    (call i uses fn(i)), which is replayed: the time is the device's, not that
    of the Python argument checks of each call, which for a kernel of a few
    microseconds would otherwise set the pace."""
    import torch
    if PROFILE_LAUNCHES:
        for i in range(PROFILE_LAUNCHES):
            fn(i)
        torch.cuda.synchronize()
        return float("nan")
    for _ in range(warm):
        fn(0)
    torch.cuda.synchronize()
    n = max(1, min(graph_len, reps))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    replays = max(1, reps // n)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    res = []
    for t in range(trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        e1.synchronize()
        res.append(e0.elapsed_time(e1) / (replays * n))
    del g
    return statistics.median(res)


# ------------------------------------------------------------------ headline
class QuaffLayer:
    def __init__(self, q, M=2048, K=4096, N=4096, n_outliers=205, batches=10, gamma=0.9, seed=1):
        import torch
        self.q = q
        self.M, self.K, self.N, self.gamma = M, K, N, gamma
        log(f"generating Quaff q_proj inputs M={M} K={K} N={N} |O|={n_outliers} batches={batches}")
        import synth
        d = self.data = synth.quaff_steps(M=M, K=K, N=N, n_outliers=n_outliers, steps=batches, seed=seed)
        self.xs = [dev(x) for x in d.xs]
        self.O = dev(d.outliers)
        self.nO = int(d.outliers.size)
        w = dev(d.w)
        codes, self.sw = q.qlin_quant_weight_sym(w, 8)
        self.w8 = q.qlin_pack_weight(q.QLIN_LAYOUT_W8, codes)
        self.w8t = q.qlin_pack_weight(q.QLIN_LAYOUT_W8T, codes)  # for the STE backward
        WO = self.WO = dev(np.ascontiguousarray(d.w[d.outliers]))
        self.WOp = q.qlin_pack_weight(q.QLIN_LAYOUT_WO, WO)
        self.wmax = q.qlin_weight_row_absmax(WO)
        self.s = torch.ones(K, dtype=torch.float32, device="cuda")
        self.r = torch.empty_like(self.s)
        self.mq_work = torch.empty((max(1, q.qlin_quaff_momentum_quant_work_bytes(M, self.nO) // 4),),
                                   dtype=torch.float32, device="cuda")
        self.work = torch.empty((max(1, q.qlin_momentum_work_bytes(M, self.nO) // 4),), dtype=torch.float32,
                                device="cuda")
        self.qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
        self.sa = torch.empty((M,), dtype=torch.float32, device="cuda")
        self.xO = torch.empty((M, q.qlin_outlier_ld(self.nO)), dtype=torch.float16, device="cuda")
        self.y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        del w, codes, WO
        torch.cuda.synchronize()

    def momentum(self, x):
        self.q.qlin_momentum_update(x, self.O, self.wmax, self.gamma, self.s, self.r)

    def momentum_quant(self, x):
        self.q.qlin_quaff_momentum_quant(x, self.O, self.wmax, self.gamma, self.s, self.r, work=self.mq_work,
                                         q=self.qa, scale=self.sa, xO=self.xO)

    def quant(self, x):
        self.q.qlin_quant_act(x, self.r, self.O, s=self.s, q=self.qa, scale=self.sa, xO=self.xO, want_qO=False)

    def gemm(self):
        self.q.qlin_gemm_w8a8(self.qa, self.sa, self.w8, self.sw, self.N, xO=self.xO, nO=self.nO, WO=self.WOp,
                              y=self.y)

    def step(self, t, ev=None):
        x = self.xs[t % len(self.xs)]
        self.momentum_quant(x)
        if ev is not None:
            ev[0].record()
        self.gemm()
        if ev is not None:
            ev[1].record()

    def capture(self):
        """HIP graphs of the step: per activation batch one graph of the
        momentum update and the quantization, and one graph of the GEMM (the
        same buffers for every batch), so the GEMM can still be timed with
        events recorded between graph launches."""
        import torch
        self.g_pre = []
        for x in self.xs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.momentum_quant(x)
            self.g_pre.append(g)
        self.g_gemm = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g_gemm):
            self.gemm()
        torch.cuda.synchronize()

    def graph_step(self, t, ev=None):
        self.g_pre[t % len(self.g_pre)].replay()
        if ev is not None:
            ev[0].record()
        self.g_gemm.replay()
        if ev is not None:
            ev[1].record()

    def int8_ops(self):
        return 2 * self.M * self.K * self.N

    def fp16_flops(self):
        return 2 * self.M * self.nO * self.N

    def gemm_bytes(self):
        """Operands of the fused GEMM, each counted once: codes, packed int8
        weights, token and column steps, the compensation operand xO and the
        packed fp16 W_O (both padded to ldO rows), and the fp16 output."""
        M, K, N = self.M, self.K, self.N
        ldO = self.q.qlin_outlier_ld(self.nO)
        return M * K + K * N + 4 * M + 2 * N + 2 * M * ldO + 2 * ldO * N + 2 * M * N


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(layer, budget_s=12.0, rows=128):
    """The oracle as it stands, on the host: the momentum update over the full
    batch, then quantization, the exact int8 GEMM (float64 BLAS) and the
    compensation term on a sample of `rows` tokens; repeated until `budget_s`.
    Each stage is also timed on its own (median of 3)."""
    from oracle import layer as ol
    from threadpoolctl import threadpool_info
    d = layer.data
    prep = ol.quaff_prepare(d.w, d.outliers)
    s = np.ones(layer.K, np.float32)
    x_full = d.xs[0]
    from oracle import quaff, quant, gemm
    sw32 = prep["sw"].astype(np.float32)
    o = d.outliers

    def med3(fn):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    x = x_full[:rows]
    s1, r1 = quaff.momentum_update(x_full, o, prep["wmax"], layer.gamma, s)
    qa1, sa1 = quant.quant_act_sym_int8(x, r1)
    stages = {
        "momentum_ms": med3(lambda: quaff.momentum_update(x_full, o, prep["wmax"], layer.gamma, s)),
        "quant_ms": med3(lambda: quant.quant_act_sym_int8(x, r1)),
        "gemm_ms": med3(lambda: gemm.w8a8(qa1, sa1, prep["qw"], sw32)),
        "compensation_ms": med3(lambda: quaff.compensation(qa1[:, o], sa1, s1[o], prep["w_o"])),
    }
    stages = {k: round(v * 1e3, 3) for k, v in stages.items()}
    t0 = time.perf_counter()
    n = 0
    while True:
        s, r = quaff.momentum_update(x_full, o, prep["wmax"], layer.gamma, s)
        qa, sa = quant.quant_act_sym_int8(x, r)
        acc, y = gemm.w8a8(qa, sa, prep["qw"], sw32)
        y = y + quaff.compensation(qa[:, o], sa, s[o], prep["w_o"])
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    ops = n * (2 * rows * layer.K * layer.N + 2 * rows * layer.nO * layer.N)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": ops / el / 1e12, "unit": "TOPS", "cores": int(threads), "kind": "oracle",
        "sample": f"{n} oracle layer steps on {rows} of {layer.M} tokens (momentum over all {layer.M}); "
                  f"{el:.1f} s; ops counted for the sampled rows only",
        "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
        "stages": dict(stages, sample_rows=rows, momentum_rows=layer.M),
    }


# ------------------------------------------------------------------ rows
def rows_measurements(q, layer):
    import torch
    out = {}
    M, K, N, nO = layer.M, layer.K, layer.N, layer.nO

    x = layer.xs[0]
    t = time_launches(lambda i: layer.momentum(layer.xs[i % len(layer.xs)]), 200)
    b = 2 * M * nO + 4 * nO * 3 + 4 * K * 2
    out["A1_momentum_update"] = dict(workload=f"quaff M={M} K={K} |O|={nO}", ms=t, bytes=b, gbs=b / t / 1e6,
                                     frac=b / t / 1e6 / PEAK_HBM_GBS, bound="hbm")
    t = time_launches(lambda i: layer.quant(layer.xs[i % len(layer.xs)]), 200)
    b = 2 * M * K + M * K + 4 * M + 4 * K + 2 * M * nO
    out["A2_quant_act"] = dict(workload=f"quaff M={M} K={K} with r and xO", ms=t, bytes=b, gbs=b / t / 1e6,
                               frac=b / t / 1e6 / PEAK_HBM_GBS, bound="hbm")
    # The step's form of A1 + A2: the momentum maxima over row blocks, folded
    # by the quantizer (two launches); the algorithmic bytes of the two rows.
    t = time_launches(lambda i: layer.momentum_quant(layer.xs[i % len(layer.xs)]), 200)
    b = (2 * M * nO + 4 * nO * 3 + 4 * K * 2) + (2 * M * K + M * K + 4 * M + 4 * K + 2 * M * nO)
    out["A1A2_momentum_quant"] = dict(workload=f"quaff M={M} K={K} |O|={nO}, one call", ms=t, bytes=b,
                                      gbs=b / t / 1e6, frac=b / t / 1e6 / PEAK_HBM_GBS, bound="hbm")
    t = time_launches(lambda i: layer.gemm(), 100)
    ops = layer.int8_ops() + 2 * layer.fp16_flops()
    out["A4A5_gemm_w8a8_fused_comp"] = dict(workload=f"{M}x{K}x{N} + |O|={nO}", ms=t, int8_equiv_ops=ops,
                                            tops=ops / t / 1e9, frac=ops / t / 1e9 / PEAK_INT8_TOPS, bound="mfma")
    t = time_launches(lambda i: q.qlin_gemm_w8a8(layer.qa, layer.sa, layer.w8, layer.sw, N, y=layer.y), 100)
    ops = layer.int8_ops()
    out["A4_gemm_w8a8"] = dict(workload=f"{M}x{K}x{N}", ms=t, ops=ops, tops=ops / t / 1e9,
                               frac=ops / t / 1e9 / PEAK_INT8_TOPS, bound="mfma")
    y2 = layer.y.clone()
    t = time_launches(lambda i: q.qlin_outlier_comp(layer.xO, layer.sa, nO, layer.WOp, y2), 100)
    fl = layer.fp16_flops()
    # Bound by the read-modify-write of y (the products are 3.4 GFLOP): bytes
    # of xO, the packed W_O, sa and y read and written.
    ldO = q.qlin_outlier_ld(nO)
    b = 2 * M * ldO + 2 * ldO * N + 4 * M + 2 * 2 * M * N
    out["A5_outlier_comp_standalone"] = dict(workload=f"{M}x{nO}x{N}", ms=t, bytes=b, gbs=b / t / 1e6,
                                             frac=b / t / 1e6 / PEAK_HBM_GBS, bound="hbm", flops=fl,
                                             tflops=fl / t / 1e9)
    del y2

    # Quaff STE backward at the same shape: quantized gradient, the outlier
    # product dY W_O^T and the int8 product against the transposed weights.
    w8t = layer.w8t
    import synth as _synth
    dy = dev(_synth.grad_output(M, N, seed=5))
    dx, gq, gs, cbuf, _ = q.qlin_quaff_backward(dy, layer.sw, w8t, layer.s, layer.r, K, O=layer.O, w_o=layer.WO)
    t = time_launches(lambda i: q.qlin_quaff_backward(dy, layer.sw, w8t, layer.s, layer.r, K, O=layer.O,
                                                      w_o=layer.WO, dx=dx, gq=gq, gs=gs, cb=cbuf), 100)
    ops = 2 * M * N * K + 2 * (2 * M * nO * N)
    out["NEXT3_quaff_ste_backward"] = dict(workload=f"dX {M}x{K} from dY {M}x{N}, |O|={nO}", ms=t,
                                           int8_equiv_ops=ops, tops=ops / t / 1e9,
                                           frac=ops / t / 1e9 / PEAK_INT8_TOPS, bound="mfma",
                                           launches="quantize dY*sw, dY W_O^T, int8 GEMM with the fix-up epilogue")
    del dy, dx, gq, gs, cbuf

    # QQQ W4A8 per-channel decode, weights rotated through >= 2x the MALL.
    import synth
    K3, N3 = 4096, 11008
    lin = synth.qqq_decode(M=64, K=K3, N=N3, seed=2)
    w = dev(lin.w)
    codes, sw = q.qlin_quant_weight_sym(w, 4)
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, codes)
    copies = max(2, (2 * MALL_BYTES) // w4.numel() + 1)
    bufs = [w4.clone() for _ in range(copies)]
    del w, codes
    for m in (1, 16, 64):
        qa, sa, _, _ = q.qlin_quant_act(dev(lin.x[:m]))
        y = torch.empty((m, N3), dtype=torch.float16, device="cuda")
        t = time_launches(lambda i: q.qlin_gemm_w4a8(qa, sa, bufs[i % copies], sw, N3, y=y), 240)
        b = K3 * N3 // 2 + m * K3 + 2 * N3 + 4 * m + 2 * m * N3
        out[f"A6_gemm_w4a8_channel_M{m}"] = dict(workload=f"{m}x{K3}x{N3} ({copies} rotating weight copies)",
                                                 ms=t, bytes=b, gbs=b / t / 1e6, frac=b / t / 1e6 / PEAK_HBM_GBS,
                                                 tops=2 * m * K3 * N3 / t / 1e9, bound="hbm")
    del bufs, w4

    # QQQ W4A8 per-group prefill at down_proj shape.
    M4, K4, N4 = 4096, 11008, 4096
    lin = synth.qqq_prefill(M=M4, K=K4, N=N4, seed=3)
    codes, gs, cs, ratio = q.qlin_quant_weight_group(dev(lin.w), 128)
    w4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, codes)
    xq = dev(lin.x)
    qa, sa, _, _ = q.qlin_quant_act(xq)
    t = time_launches(lambda i: q.qlin_quant_act(xq, q=qa, scale=sa), 50)
    b = 3 * M4 * K4 + 4 * M4
    out["A2_quant_act_prefill"] = dict(workload=f"{M4}x{K4}", ms=t, bytes=b, gbs=b / t / 1e6,
                                       frac=b / t / 1e6 / PEAK_HBM_GBS, bound="hbm")
    y = torch.empty((M4, N4), dtype=torch.float16, device="cuda")
    work = torch.empty(q.qlin_gemm_w4a8_work_bytes(M4, N4, K4, 128), dtype=torch.uint8, device="cuda")
    t = time_launches(lambda i: q.qlin_gemm_w4a8(qa, sa, w4, cs, N4, ratio=ratio, group=128, y=y, work=work), 20)
    ops = 2 * M4 * K4 * N4
    out["A7_gemm_w4a8_group128"] = dict(workload=f"{M4}x{K4}x{N4}", ms=t, ops=ops, tops=ops / t / 1e9,
                                        frac=ops / t / 1e9 / PEAK_INT8_TOPS, bound="mfma",
                                        launches="requantization once per call into a workspace, then the int8 tile")
    t = time_launches(lambda i: q.qlin_gemm_w4a8(qa, sa, w4, cs, N4, ratio=ratio, group=128, y=y), 20)
    out["A7_gemm_w4a8_group128_in_loop"] = dict(workload=f"{M4}x{K4}x{N4}", ms=t, ops=ops, tops=ops / t / 1e9,
                                                frac=ops / t / 1e9 / PEAK_INT8_TOPS, bound="mfma",
                                                launches="one tile kernel requantizing in its K loop (no workspace)")
    del codes, w4, xq, qa, y, work

    # OffQ W4A4 at LLaMA-3-8B up_proj shape.
    M5, K5, N5 = 2048, 4096, 14336
    lin = synth.offq_inputs(M=M5, K=K5, N=N5, seed=4)
    signs = dev(lin.extra["signs"])
    xo = dev(lin.x)
    qa4, sa, za, rs, _ = q.qlin_hadamard_offset(xo, signs)
    t = time_launches(lambda i: q.qlin_hadamard_offset(xo, signs, q4=qa4, scale=sa, zero=za, rowsum=rs), 50)
    b = 2 * M5 * K5 + M5 * K5 // 2 + 12 * M5 + K5
    out["A3_hadamard_offset"] = dict(workload=f"{M5}x{K5}", ms=t, bytes=b, gbs=b / t / 1e6,
                                     frac=b / t / 1e6 / PEAK_HBM_GBS, bound="hbm")
    cw, swf, zw, cs = q.qlin_quant_weight_offq(dev(lin.w), signs)
    w4u = q.qlin_pack_weight(q.QLIN_LAYOUT_W4U, cw)
    y = torch.empty((M5, N5), dtype=torch.float16, device="cuda")
    t = time_launches(lambda i: q.qlin_gemm_w4a4(qa4, sa, za, rs, w4u, swf, zw, cs, N5, y=y), 20)
    ops = 2 * M5 * K5 * N5
    out["A8_gemm_w4a4"] = dict(workload=f"{M5}x{K5}x{N5}", ms=t, ops=ops, tops=ops / t / 1e9,
                               frac=ops / t / 1e9 / PEAK_INT8_TOPS, bound="mfma")
    if PROFILE_LAUNCHES:
        # Counter runs only: the W4A4 tile at K = 256 beside the row above, and
        # the int8 tile of the same 256-row configuration at K = 256 and 4096,
        # so that a counter's share per 128-deep stage can be told from its
        # fixed share (prologue and epilogue).
        Kd = 256
        lin_d = synth.offq_inputs(M=M5, K=Kd, N=N5, seed=4)
        signs_d = dev(lin_d.extra["signs"])
        qd4, sad, zad, rsd, _ = q.qlin_hadamard_offset(dev(lin_d.x), signs_d)
        cwd, swd, zwd, csd = q.qlin_quant_weight_offq(dev(lin_d.w), signs_d)
        wd4 = q.qlin_pack_weight(q.QLIN_LAYOUT_W4U, cwd)
        time_launches(lambda i: q.qlin_gemm_w4a4(qd4, sad, zad, rsd, wd4, swd, zwd, csd, N5, y=y), 0)
        for Kw in (Kd, K5):
            lin_w = synth.plain_linear(M5, Kw, N5, seed=8)
            c8, s8 = q.qlin_quant_weight_sym(dev(lin_w.w), 8)
            w8d = q.qlin_pack_weight(q.QLIN_LAYOUT_W8, c8)
            qa8, sa8, _, _ = q.qlin_quant_act(dev(lin_w.x))
            time_launches(lambda i: q.qlin_gemm_w8a8(qa8, sa8, w8d, s8, N5, y=y), 0)
        del lin_d, qd4, cwd, wd4, c8, w8d, qa8

    # OffQ group-wise offsets (a step and zero point per token and 128-channel
    # group), same shape, one outlier level per group.
    lin = synth.offq_inputs(M=M5, K=K5, N=N5, seed=4, offset_spread=400.0)
    xo = dev(lin.x)
    G5 = K5 // 128
    qg4, sag, zag, rsg, _ = q.qlin_hadamard_offset_group(xo, signs)
    t = time_launches(lambda i: q.qlin_hadamard_offset_group(xo, signs, q4=qg4, scale=sag, zero=zag, rowsum=rsg), 50)
    b = 2 * M5 * K5 + M5 * K5 // 2 + 12 * M5 * G5 + K5
    out["A3g_hadamard_offset_group"] = dict(workload=f"{M5}x{K5}, groups of 128", ms=t, bytes=b, gbs=b / t / 1e6,
                                            frac=b / t / 1e6 / PEAK_HBM_GBS, bound="hbm")
    csg = q.qlin_weight_colsum_group(cw)
    t = time_launches(lambda i: q.qlin_gemm_w4a4_group(qg4, sag, zag, rsg, w4u, swf, zw, csg, N5, y=y), 20)
    out["A8g_gemm_w4a4_group"] = dict(workload=f"{M5}x{K5}x{N5}, groups of 128", ms=t, ops=ops, tops=ops / t / 1e9,
                                      frac=ops / t / 1e9 / PEAK_INT8_TOPS, bound="mfma")
    del cw, w4u, y, xo, qg4, csg

    # OffQ Top-1 PCA calibration (offline, once per layer): 128 sequences of
    # 512 tokens at K = 4096, then the fold of a 4096 x 4096 weight and the
    # rotation of 2048 tokens.
    S6, T6, K6 = 128, 512, 4096
    xc, _ = _synth.pca_calibration(S=S6, T=T6, K=K6, seed=6)
    xcd = dev(xc)
    del xc
    t_sel = time_launches(lambda i: q.qlin_pca_select(xcd), 10, graph_len=4)
    _, zc = q.qlin_pca_select(xcd)
    t_eig = time_launches(lambda i: q.qlin_pca_leading_eigvec(zc), 4, graph_len=2)
    v6, _, its6 = q.qlin_pca_leading_eigvec(zc)
    wf16 = (torch.randn(K6, K6, device="cuda") * 0.02).half()
    t_fold = time_launches(lambda i: q.qlin_pca_fold_weight(wf16, v6), 4, graph_len=2)
    xt = layer.xs[0]
    t_rot = time_launches(lambda i: q.qlin_pca_rotate(xt, v6), 50)
    b = S6 * T6 * K6 * 2
    out["NEXT4_pca_select"] = dict(workload=f"{S6} sequences x {T6} tokens x {K6}", ms=t_sel, bytes=b,
                                   gbs=b / t_sel / 1e6, frac=b / t_sel / 1e6 / PEAK_HBM_GBS, bound="hbm")
    out["NEXT4_pca_leading_eigvec"] = dict(workload=f"{S6} extreme tokens x {K6}", ms=t_eig,
                                           iterations=int(its6.item()), bound="latency (mean, fp64-MFMA Gram matrix, one-workgroup iteration, projection)")
    b = 2 * 2 * K6 * K6
    out["NEXT4_pca_fold_weight"] = dict(workload=f"{K6}x{K6}", ms=t_fold, bytes=b, gbs=b / t_fold / 1e6,
                                        frac=b / t_fold / 1e6 / PEAK_HBM_GBS, bound="hbm")
    b = 2 * 2 * M * K6
    out["NEXT4_pca_rotate"] = dict(workload=f"{M}x{K6}", ms=t_rot, bytes=b, gbs=b / t_rot / 1e6,
                                   frac=b / t_rot / 1e6 / PEAK_HBM_GBS, bound="hbm")
    del xcd, zc, wf16

    # Tiny W8A8 (latency only).
    lin = synth.tiny_w8a8(seed=0)
    codes, sw = q.qlin_quant_weight_sym(dev(lin.w), 8)
    w8 = q.qlin_pack_weight(q.QLIN_LAYOUT_W8, codes)
    xt = dev(lin.x)
    qa, sa, _, _ = q.qlin_quant_act(xt)
    yt = torch.empty((16, 128), dtype=torch.float16, device="cuda")
    t = time_launches(lambda i: (q.qlin_quant_act(xt, q=qa, scale=sa), q.qlin_gemm_w8a8(qa, sa, w8, sw, 128, y=yt)), 200)
    out["tiny_w8a8_quant_plus_gemm"] = dict(workload="16x256x128", ms=t, bound="launch")
    torch.cuda.synchronize()
    for v in out.values():
        for k in list(v):
            if isinstance(v[k], float):
                v[k] = round(v[k], 6)
    return out


SWEEP_MS = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096]


def token_sweep(q):
    """W8A8, W4A8 per channel and W4A8 per group of 128 over token counts
    M = 1 .. 4096 at a LLaMA-7B up_proj shape (K = 4096, N = 11008), each
    through the library's own M-dependent dispatch.  Weight copies rotate
    through at least twice the Infinity Cache, so small-M runs stream weights
    from HBM.  An fp16 torch GEMM of the same shape is timed beside them as
    context (eager, so its small-M figures include launch cost)."""
    import torch
    import synth
    K, N = 4096, 11008
    lin = synth.qqq_decode(M=max(SWEEP_MS), K=K, N=N, seed=2)
    w = dev(lin.w)
    x16 = dev(lin.x)
    qa, sa, _, _ = q.qlin_quant_act(x16)
    c8, s8 = q.qlin_quant_weight_sym(w, 8)
    c4, s4 = q.qlin_quant_weight_sym(w, 4)
    cg, _, sc, ratio = q.qlin_quant_weight_group(w, 128)

    def copies_of(t):
        n = max(2, (2 * MALL_BYTES) // t.numel() + 1)
        return [t.clone() for _ in range(n)]

    w8s = copies_of(q.qlin_pack_weight(q.QLIN_LAYOUT_W8, c8))
    w4s = copies_of(q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, c4))
    wgs = copies_of(q.qlin_pack_weight(q.QLIN_LAYOUT_W4S, cg))
    w16s = copies_of(w)
    del c8, c4, cg
    y = torch.empty((max(SWEEP_MS), N), dtype=torch.float16, device="cuda")
    work = torch.empty(q.qlin_gemm_w4a8_work_bytes(max(SWEEP_MS), N, K, 128), dtype=torch.uint8, device="cuda")
    res = {"workload": f"M x {K} x {N}", "M": SWEEP_MS, "w8a8_us": [], "w4a8_channel_us": [], "w4a8_group_us": [],
           "w4a8_group_work_us": [], "fp16_torch_us": []}
    for m in SWEEP_MS:
        a, s_, yy = qa[:m], sa[:m], y[:m]
        reps = 240 if m <= 64 else (48 if m <= 1024 else 24)
        res["w8a8_us"].append(1e3 * time_launches(
            lambda i: q.qlin_gemm_w8a8(a, s_, w8s[i % len(w8s)], s8, N, y=yy), reps))
        res["w4a8_channel_us"].append(1e3 * time_launches(
            lambda i: q.qlin_gemm_w4a8(a, s_, w4s[i % len(w4s)], s4, N, y=yy), reps))
        res["w4a8_group_us"].append(1e3 * time_launches(
            lambda i: q.qlin_gemm_w4a8(a, s_, wgs[i % len(wgs)], sc, N, ratio=ratio, group=128, y=yy), reps))
        res["w4a8_group_work_us"].append(1e3 * time_launches(
            lambda i: q.qlin_gemm_w4a8(a, s_, wgs[i % len(wgs)], sc, N, ratio=ratio, group=128, y=yy, work=work),
            reps))
        xm = x16[:m]
        for i in range(3):
            torch.matmul(xm, w16s[i % len(w16s)])
        torch.cuda.synchronize()
        n16 = 4 * len(w16s)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n16):
            torch.matmul(xm, w16s[i % len(w16s)])
        e1.record()
        e1.synchronize()
        res["fp16_torch_us"].append(1e3 * e0.elapsed_time(e1) / n16)
    for k in ("w8a8_us", "w4a8_channel_us", "w4a8_group_us", "w4a8_group_work_us", "fp16_torch_us"):
        res[k] = [round(v, 2) for v in res[k]]
    res["w4a8_channel_speedup_vs_w8a8"] = [round(a / b, 3) for a, b in zip(res["w8a8_us"], res["w4a8_channel_us"])]
    res["w4a8_group_speedup_vs_w8a8"] = [round(a / b, 3) for a, b in zip(res["w8a8_us"], res["w4a8_group_us"])]
    res["w4a8_group_work_speedup_vs_w8a8"] = [round(a / b, 3)
                                              for a, b in zip(res["w8a8_us"], res["w4a8_group_work_us"])]
    del w8s, w4s, wgs, w16s
    torch.cuda.synchronize()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-rows", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--profile", type=int, default=0, metavar="N",
                    help="counter runs: after the headline steps, launch every row's kernels N times eagerly "
                         "(untimed, no graphs, no token sweep)")
    ap.add_argument("--graphs", action="store_true",
                    help="launch the step as HIP graphs (slower than eager launches on ROCm 7)")
    ap.add_argument("--event-every", type=int, default=0,
                    help="record the GEMM's timing events on every n-th timed step (default 0: every "
                         "max(1, steps // 20)-th, so at least 20 samples, or every step below 40 steps)")
    ap.add_argument("--torch-events", action="store_true",
                    help="time the GEMM with torch's default events (with a system-scope fence on each record)")
    a = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE={world}); "
              "the layer is data-parallel over tokens with no communication, so N GPUs would run N "
              "independent copies of this single-GPU measurement.", file=sys.stderr)
        sys.exit(2)

    import torch
    from outlier_aware_bit_amd import qlin as q
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if a.copy_calibration:
        copy_calibration()
    layer = QuaffLayer(q)
    # The per-row measurements and the token sweep run before the layer step
    # is timed: their seconds of GPU work also bring the GPU from idle to its
    # steady clock, which the 20 warm-up steps (about a millisecond) do not.
    # Timed straight after the inputs are generated on the host, the same
    # 200 steps read up to 58.6 us each; once the GPU has been busy, 51-53 us
    # on the same box.
    rows = sweep = None
    if not a.no_rows and not a.profile:
        rows = rows_measurements(q, layer)
        sweep = token_sweep(q)
    run = layer.step
    if a.graphs:
        layer.capture()
        run = layer.graph_step

    for t in range(a.warmup):
        run(t)
    torch.cuda.synchronize()
    # Each event record costs the GPU about a microsecond beside a 60-us step,
    # so the events sample the GEMM (at least 20 samples) rather than
    # bracket every launch.
    every = a.event_every if a.event_every > 0 else max(1, a.steps // 20)
    if a.torch_events:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range((a.steps + every - 1) // every)]
    else:
        evs = [(FenceFreeEvent(), FenceFreeEvent()) for _ in range((a.steps + every - 1) // every)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(a.steps):
        run(a.warmup + t, evs[t // every] if t % every == 0 else None)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el * 1e3 / a.steps
    gemm_samples = [e0.elapsed_time(e1) for e0, e1 in evs]
    gemm_ms = statistics.mean(gemm_samples)
    ops_step = layer.int8_ops() + layer.fp16_flops()
    eq_ops = layer.int8_ops() + 2 * layer.fp16_flops()
    achieved = eq_ops / (gemm_ms * 1e-3) / 1e12
    log(f"step {ms_step:.4f} ms, fused GEMM {gemm_ms:.4f} ms ({achieved:.1f} int8-equivalent TOPS)")
    tr = recorded_traffic()

    rec = {
        "metric": METRIC,
        "value": round(ops_step / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "quaff_w8a8_outlier_comp_q_proj", "M_tokens": layer.M, "K": layer.K,
                   "N": layer.N, "n_outliers": layer.nO, "gamma": layer.gamma, "activation_batches": 10,
                   "step": "quaff_momentum_quant (momentum update + quant_act) + gemm_w8a8(fused compensation)",
                   "launch": "hip_graphs" if a.graphs else "eager"},
        "roofline": {"bound": "mfma", "kernel": GEMM_KERNEL, "achieved": round(achieved, 2),
                     "peak": PEAK_INT8_TOPS, "unit": "TOPS", "frac": round(achieved / PEAK_INT8_TOPS, 4),
                     "traffic": (tr["read"] + tr["write"]) if tr else None,
                     "traffic_read_write": [tr["read"], tr["write"]] if tr else None,
                     "algorithmic_bytes": layer.gemm_bytes(), "launch_ms": round(gemm_ms, 5),
                     "launch_ms_median": round(statistics.median(gemm_samples), 5),
                     "event_samples": len(gemm_samples),
                     "timing": ("HIP events (hipEventDisableSystemFence unless --torch-events) around the GEMM "
                                f"launch on its stream, every {every}. timed step"),
                     "work": "int8 MACs x2 plus fp16 compensation flops x2 (fp16 peak is half the int8 peak)"},
    }
    if a.profile:
        global PROFILE_LAUNCHES
        PROFILE_LAUNCHES = a.profile
        rows_measurements(q, layer)
        log(f"profile run: every row launched {a.profile} times")
        a.no_rows = True
        a.no_cpu = True
    if rows is not None:
        rec["rows"] = rows
        # The same kernel replayed back to back from a HIP graph (no event
        # packets beside each launch), for comparison with the live figure.
        rec["roofline"]["launch_ms_graph"] = rec["rows"]["A4A5_gemm_w8a8_fused_comp"]["ms"]
        rec["token_sweep"] = sweep
    if not a.no_cpu:
        log("timing the CPU oracle")
        rec["cpu_baseline"] = cpu_baseline(layer, budget_s=a.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
