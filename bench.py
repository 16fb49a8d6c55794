"""Benchmark of the conv2d training layer on one MI355X.

A step is one pass of the layer's hot path over one batch of seeded synthetic input, on
the wide bf16 layer N=64, 56x56x128 -> 128, 3x3 s1 p1, bias + tanh (fp32 accumulate):
conv2d_forward (conv + bias + activation; only the output y is stored, since the tanh
derivative is a function of y) and conv2d_backward_full (activation derivative from y,
dX, dW + db).  Layers with a normalisation run forward, activation_backward, dX and dW
as four calls.  The headline value
is (forward + dX + dW flops) / step time in TFLOP/s.  Batch-norm statistics GB/s are
measured on the conv + batch-norm layer (fp32, N=128, 32x32x64 -> 64) in the same run.

Per-call durations come from HIP events recorded on the stream the library launches on
(torch's current stream) around every call of the timed steps.  The fp64 oracle is
timed on a bounded sample of the same layer on the host cores (cpu_baseline).

HBM traffic and MFMA utilisation of the dominant call come from rocprofv3 counter runs
of this script: FETCH_SIZE and WRITE_SIZE (scaled by what the same counters read for a
plain device copy of known size), and SQ_VALU_MFMA_BUSY_CYCLES over the kernel's GPU
cycles (GRBM_GUI_ACTIVE of one XCD: the reported sum over the 8 XCDs / 8) times the 1024
SIMDs -- the fraction of SIMD cycles the matrix pipe is busy, rocprofv3's MfmaUtil, i.e.
the MFMA rate as a fraction of the peak at the clock the kernel actually ran at -- with
SQ_INSTS_VALU_MFMA_MOPS_* x 512 (the flops the matrix pipe executed).  The
figures live in profiles/traffic.json, per workload, with a hash of the kernel sources
they were taken on, and are reported as null once the sources change.  Modes for
producing them:
  python bench.py --workload W --steps 3 --warmup 1 --no-cpu-baseline --no-bn  (counter runs)
  python bench.py --calibrate-copy                                              (copy kernel)
  python bench.py --summarize DIR --workload W   (rocprofv3 CSVs -> summary text, traffic.json)

Prints ONE JSON line.  Only one GPU is used: --gpus above 1 exits with a message.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as WL  # noqa: E402

PEAK_TFLOPS = {WL.BF16: 2516.6, WL.F32: 157.3}  # MI355X dense MFMA peaks
PEAK_HBM_GBS = 8000.0
SIMD_NUM = 1024  # 256 CUs x 4 SIMDs
XCD_NUM = 8  # rocprofv3's per-dispatch GRBM_GUI_ACTIVE is the sum over the 8 XCDs
METRIC = "conv2d fwd+dX+dW TFLOP/s and % MFMA peak; BN-stats GB/s (1 MI355X)"
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read + 1 GiB written
CONV_CALLS = ("forward", "backward_data", "backward_weight")
PRODUCTS = {"forward": 1, "backward_data": 1, "backward_weight": 1, "backward_full": 2}  # conv products per call


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the library's kernel and host sources (traffic figures are tied to it)."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "convolution_layer_amd", "csrc", "*"))):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Layer:
    """Device buffers and the four library calls of one training step."""

    def __init__(self, wl: WL.Workload, x=None, evaluation=False, norm=None):
        """norm: None, or (normalization, groups, activation) replacing the workload's
        (layer / group norm variants on the workload's shape)."""
        import torch

        import convolution_layer_amd as cm
        from tests import gpu_harness as G
        self.cm, self.G, self.wl = cm, G, wl
        s, dt = wl.shape, wl.dtype
        d = WL.make_inputs(wl)
        self.desc = G.desc_for(wl)
        if evaluation:
            self.desc.mode = cm.MODE_EVAL
        if norm is not None:
            self.desc.normalization, self.desc.groups, self.desc.activation = norm
            r = np.random.default_rng(97)
            d.setdefault("gamma", WL.round_to(WL.F32, r.uniform(0.5, 1.5, s.OC)))
            d.setdefault("beta", WL.round_to(WL.F32, r.normal(0.0, 0.1, s.OC)))
        dev = lambda a, t=None: G.dev(a, t)
        self.x = x if x is not None else dev(d["x"], dt)  # a chained layer takes the previous y
        self.w = dev(d["w"], dt)
        self.b = dev(d.get("b"))
        self.dy = dev(d["dy"], dt)
        self.bn = wl.norm == WL.NORM_BATCH
        self.gamma, self.beta = dev(d.get("gamma")), dev(d.get("beta"))
        self.rm, self.rv = dev(d.get("running_mean")), dev(d.get("running_var"))
        if norm is not None:  # layer / group norm keep no running statistics
            self.rm = self.rv = None
        tdt = G.tdtype(dt)
        self.z = torch.empty(s.y_shape, dtype=tdt, device="cuda")
        self.y = torch.empty(s.y_shape, dtype=tdt, device="cuda")
        self.dz = torch.empty(s.y_shape, dtype=tdt, device="cuda")
        self.dx = torch.empty(s.x_shape, dtype=tdt, device="cuda")
        self.dw = torch.empty(s.w_shape, dtype=torch.float32, device="cuda")
        self.db = torch.empty(s.OC, dtype=torch.float32, device="cuda")
        f32 = lambda n=s.OC: torch.empty(n, dtype=torch.float32, device="cuda")
        normed = self.desc.normalization != cm.NORM_NONE
        self.sm, self.si = (f32(cm.stat_count(self.desc)), f32(cm.stat_count(self.desc))) if normed else (None, None)
        self.dg, self.dbt = (f32(), f32()) if normed else (None, None)
        n = max(cm.workspace_size(self.desc, op) for op in range(6))
        self.ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")

    def forward(self):
        self.cm.conv2d_forward(self.desc, self.x, self.w, self.b, self.gamma, self.beta, self.rm, self.rv,
                               self.sm, self.si, self.z, self.y, self.ws)

    def forward_y(self):
        """Forward storing only y (no normalisation: the backward reads y)."""
        self.cm.conv2d_forward(self.desc, self.x, self.w, self.b, None, None, None, None, None, None, None, self.y,
                               self.ws)

    def bwd_full(self):
        self.cm.conv2d_backward_full(self.desc, self.x, self.w, self.y, 1, self.dy, self.dx, self.dw, self.db, 0,
                                     self.ws)

    def act_bwd(self):
        self.cm.activation_backward(self.desc, self.z, self.dy, self.gamma, self.beta, self.sm, self.si, self.dz,
                                    self.dg, self.dbt, 0, self.ws)

    def bwd_data(self):
        self.cm.conv2d_backward_data(self.desc, self.dz, self.w, self.dx, self.ws)

    def bwd_weight(self):
        self.cm.conv2d_backward_weight(self.desc, self.x, self.dz, self.dw, self.db, 0, self.ws)

    def bn_stats(self):
        self.cm.bn_stats_training(self.desc, self.z, self.sm, self.si, None, None, self.ws)

    def calls(self):
        """The calls of one training step."""
        if not self.bn and self.wl.norm == WL.NORM_NONE and self.wl.act != WL.ACT_GELU:
            return [("forward", self.forward_y), ("backward_full", self.bwd_full)]
        return self.unit_calls()

    @staticmethod
    def calls_of(wl):
        fused = wl.norm == WL.NORM_NONE and wl.act != WL.ACT_GELU
        return [("forward", None), ("backward_full", None)] if fused else \
            [("forward", None), ("activation_backward", None), ("backward_data", None), ("backward_weight", None)]

    def unit_calls(self):
        return [("forward", self.forward), ("activation_backward", self.act_bwd),
                ("backward_data", self.bwd_data), ("backward_weight", self.bwd_weight)]


def chain_input(wl: WL.Workload):
    """x of a chained layer (the RL stack's second and third): the stored output y of the
    layers before it, each run forward by the library on its own inputs.  None otherwise."""
    if wl.x_dist[0] != "chain":
        return None
    import torch
    prev = WL.WORKLOADS[wl.x_dist[1]]
    layer = Layer(prev, x=chain_input(prev))
    layer.forward()
    torch.cuda.synchronize()
    y = layer.y.clone()
    del layer
    return y


def timed_steps(layer, steps, warmup, only=None):
    """Run warmup + timed steps; returns (total seconds, {call: mean ms})."""
    import torch
    calls = [(n, f) for n, f in layer.calls() if only is None or n == only]
    for _ in range(warmup):
        for _, f in calls:
            f()
    torch.cuda.synchronize()
    ev = {name: [] for name, _ in calls}
    t0 = time.perf_counter()
    for _ in range(steps):
        for name, f in calls:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            ev[name].append((a, b))
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    ms = {name: float(np.mean([a.elapsed_time(b) for a, b in v])) for name, v in ev.items()}
    return total, ms


def graph_steps(layer, steps, warmup):
    """Seconds for `steps` training steps launched as one captured HIP graph of the step's
    calls (the same kernels in the same order; the graph removes the host's per-launch
    gaps between them).  The replayed step must reproduce the eager step bit for bit."""
    import torch
    calls = [f for _, f in layer.calls()]
    for _ in range(warmup):
        for f in calls:
            f()
    torch.cuda.synchronize()
    eager = (layer.dx.clone(), layer.dw.clone(), layer.y.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in calls:
            f()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    if not (torch.equal(eager[0], layer.dx) and torch.equal(eager[1], layer.dw) and torch.equal(eager[2], layer.y)):
        raise RuntimeError("graph replay of the training step differs from the eager step")
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    del g
    return total


def time_call(f, reps):
    import torch
    f()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        f()
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in pairs]))


def time_graph(f, calls=20, replays=10):
    """Per-call device time of a short call: `calls` calls captured in one HIP graph,
    replayed `replays` times between two events (per-call events would also time the
    host's launch work, which is longer than such a call)."""
    import torch
    f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            f()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (calls * replays), g


REPORT_ORDER = ("c1", "c2a", "c2b", "c2c", "c3", "c4", "c5")


def call_bytes(wl: WL.Workload, call: str, evaluation: bool = False, norm: bool = False) -> int:
    """Algorithmic HBM bytes of one call: what the operation itself must read and write.
    norm: a layer / group norm variant of the workload (statistics pass over z)."""
    s = wl.shape
    e = 2 if wl.dtype == WL.BF16 else 4
    x, w, y = s.N * s.H * s.W * s.IC, s.OC * s.KH * s.KW * s.IC, s.P * s.OC
    if call == "norm_stats":
        return y * e
    if call == "forward":  # x, w, bias, z and y (training batch norm: + the statistics pass over z)
        stats = (wl.norm == WL.NORM_BATCH and not evaluation) or norm
        return (x + w + 2 * y) * e + 4 * s.OC + (y * e if stats else 0)
    if call == "forward_y":  # x, w, bias -> y
        return (x + w + y) * e + 4 * s.OC
    if call == "backward_full":  # x, w, y, dy -> dx, dw (fp32), db
        return (2 * x + w + 2 * y) * e + 4 * w + 4 * s.OC
    if call == "bn_stats":
        return y * e
    if call == "activation_backward":  # z, dy -> dz
        return 3 * y * e
    if call == "backward_data":  # dz, w -> dx
        return (y + w + x) * e
    if call == "backward_weight":  # x, dz -> dw (fp32), db
        return (x + y) * e + 4 * w + 4 * s.OC
    raise ValueError(call)


def graph_ms(fs, k, replays):
    """Per-replay device times (ms) of a HIP graph holding k rounds of the calls fs."""
    import torch
    for f in fs:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(k):
            for f in fs:
                f()
    g.replay()
    torch.cuda.synchronize()
    evs = []
    for _ in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    del g
    return np.array([a.elapsed_time(b) for a, b in evs])


def cold_warm_ms(f, replays=10):
    """Device time of one call, warm and cold.  Warm: K calls in one HIP graph, per-call
    time = replay time / K.  Cold: K rounds of (read 512 MB, call) minus K rounds of the
    read alone, / K; the read (row sums of a 512 MB buffer) evicts L2 and the 256 MB MALL
    with clean lines, so the call reads HBM without also paying for write-backs of
    someone else's dirty lines (a 512 MB write as the eviction leaves the MALL dirty and
    charged the call ~10 us of those write-backs on a 150 MB pass).
    Returns (warm per-replay array, cold per-replay array, K), all per call in ms."""
    import torch
    flush = torch.ones((1 << 17, 1 << 10), dtype=torch.float32, device="cuda")  # 512 MB
    sums = torch.empty(1 << 17, dtype=torch.float32, device="cuda")

    def evict():
        torch.sum(flush, dim=1, out=sums)

    est = time_call(f, 3)  # ms, host gaps included: only sizes the graphs
    k = int(max(1, min(50, round(0.5 / max(est, 1e-3)))))
    warm = graph_ms([f], k, replays) / k
    both = graph_ms([evict, f], k, replays)
    alone = graph_ms([evict], k, replays)
    cold = (both - np.median(alone)) / k
    del flush, sums
    return warm, cold, k


def report(replays=10):
    """Every configuration, every call: device time warm and cold (see cold_warm_ms),
    median / p10 / p90 over the replays."""
    import torch
    prev_y, out = None, []
    for name in REPORT_ORDER:
        wl = WL.WORKLOADS[name]
        layer = Layer(wl, x=prev_y if wl.x_dist[0] == "chain" else None)
        layer.forward()
        torch.cuda.synchronize()
        prev_y = layer.y.clone() if name in ("c2a", "c2b") else None
        calls = [("forward", layer.forward)]
        if layer.bn:
            calls.append(("bn_stats", layer.bn_stats))
        calls += [("activation_backward", layer.act_bwd), ("backward_data", layer.bwd_data),
                  ("backward_weight", layer.bwd_weight)]
        if wl.norm == WL.NORM_NONE:  # the fused step: forward storing y only, then backward_full from y
            calls += [("forward_y", layer.forward_y), ("backward_full", layer.bwd_full)]
        if layer.bn:  # evaluation-mode batch norm: running statistics, constant in the backward
            ev = Layer(wl, x=layer.x, evaluation=True)
            ev.forward()
            calls += [("forward[eval]", ev.forward), ("activation_backward[eval]", ev.act_bwd)]
        if name in ("c3", "c4"):  # layer norm and group norm (8 groups) with GELU on the same shape
            import convolution_layer_amd as cm
            for tag, norm in (("layer", (cm.NORM_LAYER, 1, cm.ACT_GELU)), ("group8", (cm.NORM_GROUP, 8, cm.ACT_GELU))):
                v = Layer(wl, x=layer.x, norm=norm)
                v.forward()
                calls += [(f"forward[{tag}]", v.forward), (f"norm_stats[{tag}]", v.bn_stats),
                          (f"activation_backward[{tag}]", v.act_bwd)]
        for cname, f in calls:
            warm, cold, k = cold_warm_ms(f, replays)
            row = {"config": name, "call": cname, "dtype": wl.dtype, "graph_calls": k,
                   "warm_ms": {q: round(float(np.percentile(warm, p)), 5) for q, p in (("p10", 10), ("median", 50), ("p90", 90))},
                   "cold_ms": {q: round(float(np.percentile(cold, p)), 5) for q, p in (("p10", 10), ("median", 50), ("p90", 90))}}
            med = row["warm_ms"]["median"]
            by = call_bytes(wl, cname.split("[")[0], evaluation=cname.endswith("[eval]"),
                            norm=cname.endswith("[layer]") or cname.endswith("[group8]"))
            row["GB/s"] = round(by / (med * 1e-3) / 1e9, 1)
            row["hbm_frac"] = round(row["GB/s"] / PEAK_HBM_GBS, 4)
            row["cold_GB/s"] = round(by / (row["cold_ms"]["median"] * 1e-3) / 1e9, 1)
            row["cold_hbm_frac"] = round(row["cold_GB/s"] / PEAK_HBM_GBS, 4)
            if cname.startswith("forward") or cname in ("backward_data", "backward_weight", "backward_full"):
                tf = (2 if cname == "backward_full" else 1) * wl.shape.flops() / (med * 1e-3) / 1e12
                row["TFLOP/s"] = round(tf, 3)
                row["mfma_frac"] = round(tf / PEAK_TFLOPS[wl.dtype], 4)
            out.append(row)
            print(json.dumps(row), flush=True)
        del layer
        torch.cuda.empty_cache()
    print()
    print("warm: K calls per HIP graph replay (inputs may sit in the 256 MB MALL); cold: after a 512 MB read")
    print("TFLOP/s and %MFMA from the warm median; GB/s = algorithmic bytes / median time")
    print(f"{'cfg':5} {'call':20} {'dtype':5} {'warm us':>9} {'p10':>8} {'p90':>8} {'cold us':>9} {'p10':>8} "
          f"{'p90':>8} {'TFLOP/s':>9} {'%MFMA':>7} {'warm GB/s':>10} {'cold GB/s':>10} {'%HBM cold':>9}")
    for r in out:
        w, c = r["warm_ms"], r["cold_ms"]
        tf = f"{r['TFLOP/s']:9.2f} {100 * r['mfma_frac']:6.1f}%" if "TFLOP/s" in r else f"{'':9} {'':7}"
        print(f"{r['config']:5} {r['call']:20} {r['dtype']:5} {1e3 * w['median']:9.2f} {1e3 * w['p10']:8.2f} "
              f"{1e3 * w['p90']:8.2f} {1e3 * c['median']:9.2f} {1e3 * c['p10']:8.2f} {1e3 * c['p90']:8.2f} {tf} "
              f"{r['GB/s']:10.1f} {r['cold_GB/s']:10.1f} {100 * r['cold_hbm_frac']:8.1f}%")


def cpu_baseline(wl: WL.Workload, n_images: int):
    """The fp64 oracle, untuned, on n_images of the workload's batch: forward,
    activation backward, dX and dW.  Returns (TFLOP/s, seconds, threads)."""
    import oracle as O
    sub = wl.with_batch(n_images)
    s = sub.shape
    d = WL.make_inputs(sub)
    if "x" not in d:  # a chained layer's input is the previous layer's ReLU output: a stand-in of that form
        d["x"] = WL.round_to(wl.dtype, np.maximum(np.random.default_rng(wl.seed).standard_normal(s.x_shape), 0.0))
    st, pd = (s.sh, s.sw), (s.ph, s.pw)
    t0 = time.perf_counter()
    z = O.conv2d_forward(d["x"], d["w"], d.get("b"), st, pd)
    O.apply_activation(z, wl.act)
    dz, _, _ = O.activation_backward(z, d["dy"], wl.act)
    O.conv2d_backward_data(dz, d["w"], s.x_shape, st, pd)
    O.conv2d_backward_weight(d["x"], dz, s.w_shape, st, pd)
    sec = time.perf_counter() - t0
    return 3 * s.flops() / sec / 1e12, sec, O.num_threads()


def calibrate_copy(reps=5):
    """A plain device-to-device copy of COPY_BYTES, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": COPY_BYTES, "reps": reps}), flush=True)


# ------------------------------------------------------------------ rocprofv3 summaries
KERNEL_OF_CALL = {  # kernel-name fragments each library call launches
    "forward": ("halo_rb_kernel<", "halo_kernel<", "frag_weights", "igemm2_kernel<", "igemm_kernel<",
                "conv_fwd_direct"),
    "backward_data": ("halo_rb_kernel<", "halo_kernel<", "frag_weights", "dx_weights", "igemm2_kernel<",
                      "igemm_kernel<", "conv_dx_direct"),
    "backward_weight": ("dw3_kernel", "dw2_kernel", "dw_kernel", "dw_reduce4", "conv_dw_direct"),
    "backward_full": ("act_bwd<", "halo_rb_kernel<", "halo_kernel<", "frag_weights", "dx_weights", "igemm2_kernel<",
                      "igemm_kernel<", "conv_dx_direct", "dw3_kernel", "dw2_kernel", "dw_kernel", "dw_reduce4",
                      "conv_dw_direct"),
}


def _read_counters(d):
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            key = (r["Kernel_Name"], r["Counter_Name"])
            out.setdefault(key, []).append(float(r["Counter_Value"]))
    return out


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F32")


def summarize(d, workload):
    """Summarise rocprofv3 output of one workload under d/<workload>/ (kt/, fetch/, write/,
    mfma/) with the copy calibration in d/copy_fetch/, d/copy_write/: kernel durations,
    FETCH_SIZE / WRITE_SIZE per dispatch scaled by the copy calibration, and per kernel
    the matrix pipe's busy fraction and executed flops.  Updates the workload's entry of
    d/traffic.json and prints the text summary."""
    lines = [f"rocprofv3 summary of {d}, workload {workload} (library sources {source_hash()})", ""]
    wd = os.path.join(d, workload)
    stats = glob.glob(os.path.join(wd, "kt", "**", "*kernel_stats.csv"), recursive=True)
    avg_us = {}
    if stats:
        lines.append(f"{'kernel':90s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s}")
        for r in csv.DictReader(open(stats[0])):
            avg_us[r["Name"]] = float(r["AverageNs"]) / 1e3
            lines.append(f"{r['Name'][:90]:90s} {r['Calls']:>6s} {float(r['AverageNs']) / 1e3:9.2f} "
                         f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}")
        lines.append("")
    scale = {}
    for cnt, sub in (("FETCH_SIZE", "copy_fetch"), ("WRITE_SIZE", "copy_write")):
        c = _read_counters(os.path.join(d, sub))
        vals = [v for (k, n), vs in c.items() if n == cnt and "copy" in k.lower() for v in vs]
        if vals:
            kib = float(np.median(vals))
            scale[cnt] = (COPY_BYTES / 1024.0) / kib
            lines.append(f"copy calibration {cnt}: {kib:.0f} KiB per {COPY_BYTES >> 20} MiB copy -> factor "
                         f"{scale[cnt]:.4f}")
    path = os.path.join(d, "traffic.json")
    try:
        traffic = json.load(open(path))
    except (OSError, ValueError):
        traffic = {}
    if traffic.get("sources") != source_hash():
        traffic = {"sources": source_hash(), "workloads": {}}
    if scale:
        traffic["scale"] = scale
    per_kernel = {}
    for cnt, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        c = _read_counters(os.path.join(wd, sub))
        for (k, n), vs in c.items():
            if n == cnt:
                per_kernel.setdefault(k, {})[cnt] = float(np.median(vs))
    if per_kernel:
        lines.append("")
        lines.append(f"{'kernel':90s} {'FETCH KiB':>12s} {'WRITE KiB':>12s} (per dispatch, raw)")
        for k, v in sorted(per_kernel.items()):
            lines.append(f"{k[:90]:90s} {v.get('FETCH_SIZE', float('nan')):12.0f} "
                         f"{v.get('WRITE_SIZE', float('nan')):12.0f}")
    c = _read_counters(os.path.join(wd, "mfma"))
    mf = {}
    for (k, n), vs in c.items():
        if n in MFMA_COUNTERS:
            mf.setdefault(k, {})[n] = float(np.median(vs))
    mfma = {}
    for k, v in sorted(mf.items()):
        if v.get("GRBM_GUI_ACTIVE") and "SQ_VALU_MFMA_BUSY_CYCLES" in v:
            mops = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + v.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0)
            if mops == 0:
                continue
            cycles = v["GRBM_GUI_ACTIVE"] / XCD_NUM
            mfma[k] = {"busy": v["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * SIMD_NUM), "mfma_flops": mops * 512.0,
                       "gpu_cycles": cycles, **v}
    if mfma:
        lines.append("")
        lines.append(f"{'kernel':90s} {'MFMA busy':>10s} {'MFMA GFLOP':>11s} {'TFLOP/s':>9s} {'GHz':>6s} (per "
                     f"dispatch; busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCD_NUM} x {SIMD_NUM} SIMDs); "
                     "TFLOP/s from the trace's average duration; GHz = cycles / duration)")
        for k, v in mfma.items():
            t = avg_us.get(k)
            rate = f"{v['mfma_flops'] / (t * 1e-6) / 1e12:9.1f}" if t else f"{'':9s}"
            ghz = f"{v['gpu_cycles'] / (t * 1e3):6.2f}" if t else f"{'':6s}"
            lines.append(f"{k[:90]:90s} {100 * v['busy']:9.1f}% {v['mfma_flops'] / 1e9:11.2f} {rate} {ghz}")
    traffic.setdefault("workloads", {})[workload] = {"kernels": per_kernel, "mfma": mfma, "avg_us": avg_us}
    with open(path, "w") as f:
        json.dump(traffic, f, indent=1)
    print("\n".join(lines))


def _counters(workload: str):
    """The workload's entry of profiles/traffic.json and the copy scale, or None when
    absent or taken on different sources."""
    try:
        t = json.load(open(TRAFFIC_JSON))
    except (OSError, ValueError):
        return None, None
    if t.get("sources") != source_hash() or len(t.get("scale", {})) != 2:
        return None, None
    return t.get("workloads", {}).get(workload), t["scale"]


def _of_call(k: str, call: str) -> bool:
    shared = "igemm" in k or "halo" in k  # one template for both directions: FwdOut / DxOut
    return any(f in k for f in KERNEL_OF_CALL[call]) and (not shared or ("FwdOut" in k) == (call == "forward"))


def call_traffic(call: str, workload: str):
    """HBM bytes per launch of one library call (all its kernels), or None."""
    w, scale = _counters(workload)
    if not w or not w.get("kernels"):
        return None
    total, seen = 0.0, False
    for k, v in w["kernels"].items():
        if _of_call(k, call):
            total += v.get("FETCH_SIZE", 0) * scale["FETCH_SIZE"] + v.get("WRITE_SIZE", 0) * scale["WRITE_SIZE"]
            seen = True
    return total * 1024.0 if seen else None


def call_mfma(call: str, workload: str):
    """Matrix-pipe busy fraction and flops of the call's longest kernel, or None."""
    w, _ = _counters(workload)
    if not w or not w.get("mfma"):
        return None
    ks = [k for k in w["mfma"] if _of_call(k, call)]
    if not ks:
        return None
    k = max(ks, key=lambda k_: w.get("avg_us", {}).get(k_, 0.0))
    v = w["mfma"][k]
    t = w.get("avg_us", {}).get(k)
    name = k.replace("(anonymous namespace)::", "").replace("void ", "")
    return {"kernel": name.split("(")[0][:100], "busy": round(v["busy"], 4), "mfma_gflop": round(v["mfma_flops"] / 1e9, 3),
            "kernel_us": None if t is None else round(t, 2)}


def vendor(names=("c3", "c4", "c5"), reps=20):
    """Context, not part of the bench line: the vendor libraries on the same GPU and the same
    shapes -- torch's conv2d and its convolution_backward (MIOpen on ROCm; channels-last, so
    NHWC like ours) and torch.matmul (hipBLASLt) on the implicit-GEMM shape [P, KH*KW*IC] x
    [KH*KW*IC, OC] -- beside this library's forward (convolution + bias, no normalisation or
    activation), input-gradient and weight-gradient calls, all timed the same way: eager
    calls between HIP events, median of `reps` after warm-up, inputs resident."""
    import torch
    import torch.nn.functional as F
    import convolution_layer_amd as cm
    torch.backends.cudnn.benchmark = True

    def med_us(f):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        return float(np.median(ts))

    for name in names:
        wl = WL.WORKLOADS[name]
        s = wl.shape
        tdt = torch.bfloat16 if wl.dtype == WL.BF16 else torch.float32
        cl = torch.channels_last
        g = torch.Generator(device="cuda").manual_seed(1)
        x = torch.randn(s.N, s.IC, s.H, s.W, device="cuda", generator=g).to(tdt).contiguous(memory_format=cl)
        w = (0.05 * torch.randn(s.OC, s.IC, s.KH, s.KW, device="cuda", generator=g)).to(tdt).contiguous(memory_format=cl)
        b = torch.randn(s.OC, device="cuda", generator=g).to(tdt) if wl.b_dist is not None else None
        dy = torch.randn(s.N, s.OC, s.OH, s.OW, device="cuda", generator=g).to(tdt).contiguous(memory_format=cl)
        st, pd = [s.sh, s.sw], [s.ph, s.pw]
        bwd = lambda mask: torch.ops.aten.convolution_backward(dy, x, w, [s.OC], st, pd, [1, 1], False, [0, 0], 1, mask)
        K = s.KH * s.KW * s.IC
        A = torch.randn(s.P, K, device="cuda", generator=g).to(tdt)
        B = torch.randn(K, s.OC, device="cuda", generator=g).to(tdt)
        ven = {"forward": med_us(lambda: F.conv2d(x, w, b, stride=st, padding=pd)),
               "backward_data": med_us(lambda: bwd([True, False, False])),
               "backward_weight": med_us(lambda: bwd([False, True, True])),
               "gemm": med_us(lambda: A @ B)}
        del x, w, b, dy, A, B
        torch.cuda.empty_cache()
        layer = Layer(wl, norm=(cm.NORM_NONE, 1, cm.ACT_IDENTITY))
        layer.forward_y()
        layer.dz.copy_(layer.dy)  # identity activation: dz = dy
        torch.cuda.synchronize()
        ours = {"forward": med_us(layer.forward_y), "backward_data": med_us(layer.bwd_data),
                "backward_weight": med_us(layer.bwd_weight)}
        del layer
        torch.cuda.empty_cache()
        tf = lambda us: round(s.flops() / (us * 1e-6) / 1e12, 1)
        print(json.dumps({"workload": name, "dtype": wl.dtype, "timing": f"eager, HIP events, median of {reps}",
                          "vendor_us": {k: round(v, 2) for k, v in ven.items()},
                          "vendor_TFLOP/s": {k: tf(v) for k, v in ven.items()},
                          "convmi_us": {k: round(v, 2) for k, v in ours.items()},
                          "convmi_TFLOP/s": {k: tf(v) for k, v in ours.items()},
                          "speedup": {k: round(ven[k] / ours[k], 2) for k in ours}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4", choices=sorted(WL.WORKLOADS))
    ap.add_argument("--cpu-images", type=int, default=64, help="images of the batch the oracle baseline runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bn", action="store_true", help="skip the batch-norm statistics measurement")
    ap.add_argument("--only", choices=("forward", "activation_backward", "backward_data", "backward_weight",
                                       "backward_full"))
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize", metavar="DIR")
    ap.add_argument("--report", action="store_true",
                    help="time every call of every configuration (warm and cold) instead of the bench step")
    ap.add_argument("--vendor", action="store_true",
                    help="time MIOpen (torch conv2d) and hipBLASLt (torch.matmul) beside this library on c3-c5")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.workload)
        return
    if args.report:
        report()
        return
    if args.vendor:
        vendor()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); multi-GPU sharding is not built.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench needs a GPU"
    if args.calibrate_copy:
        calibrate_copy()
        return
    wl = WL.WORKLOADS[args.workload]
    s = wl.shape
    log(f"bench: workload {wl.name} ({wl.note}); building inputs")
    layer = Layer(wl, x=chain_input(wl))
    log("bench: timing steps")
    eager_total, ms = timed_steps(layer, args.steps, args.warmup, args.only)
    if args.only:
        print(json.dumps({"only": args.only, "ms": ms}), flush=True)
        return
    total = graph_steps(layer, args.steps, args.warmup)
    step_ms = total / args.steps * 1e3
    flops = 3 * s.flops()
    value = flops / (total / args.steps) / 1e12
    log(f"bench: step {step_ms:.3f} ms (graph), {eager_total / args.steps * 1e3:.3f} ms (eager); per call ms {ms}")

    # dominant kernel: the single-product convolution call with the longest mean duration
    # (in the fused step, the forward; backward_full holds two products and three launches)
    conv_calls = {k: v for k, v in ms.items() if k in PRODUCTS}
    single = {k: v for k, v in conv_calls.items() if PRODUCTS[k] == 1}
    dom = max(single, key=single.get)
    # the dominant call's device time: 8 calls back to back in one HIP graph, replayed 10
    # times between events on the library's stream (median); unlike the eager per-call
    # events this leaves out the host's launch gaps between the call's kernels
    dom_fn = dict(layer.calls())[dom]
    dom_ms = float(np.median(graph_ms([dom_fn], 8, 10))) / 8
    achieved = s.flops() / (dom_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]
    tr = call_traffic(dom, wl.name)
    mf = call_mfma(dom, wl.name)
    roofline = {"bound": "mfma", "kernel": f"conv2d_{dom}", "call_ms": round(dom_ms, 5),
                "call_timing": "8 calls per HIP graph replay, median of 10 replays",
                "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None if tr is None else round(tr),
                "mfma_busy": None if mf is None else mf["busy"], "mfma_counters": mf,
                "per_call_ms_eager": {k: round(v, 4) for k, v in ms.items()},
                "per_call_tflops": {k: round(PRODUCTS[k] * s.flops() / (v * 1e-3) / 1e12, 2)
                                    for k, v in conv_calls.items()},
                "per_call_hbm_bytes": {k: call_traffic(k, wl.name) for k in conv_calls},
                "per_call_mfma_busy": {k: (lambda m: None if m is None else m["busy"])(call_mfma(k, wl.name))
                                       for k in conv_calls}}

    bn = None
    if not args.no_bn:
        del layer
        torch.cuda.empty_cache()
        bn_wl = WL.WORKLOADS["c3"]
        bn_layer = Layer(bn_wl)
        bn_layer.forward()
        bn_layer.bn_stats()
        torch.cuda.synchronize()
        ref = (bn_layer.sm.clone(), bn_layer.si.clone())
        eager_ms = time_call(bn_layer.bn_stats, 50)
        warm, cold, k = cold_warm_ms(bn_layer.bn_stats)
        # every replay recomputes the same statistics (the call is deterministic)
        if not (torch.equal(ref[0], bn_layer.sm) and torch.equal(ref[1], bn_layer.si)):
            raise RuntimeError("graph replay of bn_stats_training differs from the eager call")
        bn_ms, cold_ms = float(np.median(warm)), float(np.median(cold))
        zbytes = bn_wl.shape.P * bn_wl.shape.OC * 4
        bn_gbs = zbytes / (bn_ms * 1e-3) / 1e9
        cold_gbs = zbytes / (cold_ms * 1e-3) / 1e9
        bn = {"workload": "c3", "bytes": zbytes, "ms": round(bn_ms, 5), "GB/s": round(bn_gbs, 1),
              "frac": round(bn_gbs / PEAK_HBM_GBS, 4), "cold_ms": round(cold_ms, 5),
              "cold_GB/s": round(cold_gbs, 1), "cold_frac": round(cold_gbs / PEAK_HBM_GBS, 4),
              "timing": f"HIP graph of {k} calls, median of 10 replays; cold = after a 512 MB read that "
                        "evicts L2 and MALL (read time subtracted)",
              "eager_ms_per_call": round(eager_ms, 5)}
        log(f"bench: bn_stats {bn}")
        del bn_layer
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log(f"bench: cpu baseline (oracle, {args.cpu_images} images)")
        tf, sec, thr = cpu_baseline(wl, min(args.cpu_images, s.N))
        cpu = {"value": round(tf, 6), "unit": "TFLOP/s", "cores": thr, "kind": "oracle",
               "sample": f"{wl.name} with N={min(args.cpu_images, s.N)} of {s.N} images: fwd + act bwd + dX + dW, "
                         f"fp64, {sec:.1f} s"}

    line = {"metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.dtype == WL.BF16 else "f32",
            "data": "synthetic",
            "config": {"workload": f"{wl.name}: {wl.note}", "N": s.N, "H": s.H, "W": s.W, "IC": s.IC,
                       "OC": s.OC, "kernel": f"{s.KH}x{s.KW}", "stride": s.sh, "pad": s.ph,
                       "step": " + ".join(n for n, _ in Layer.calls_of(wl)),
                       "launch": "the step's calls captured once in a HIP graph and replayed",
                       "eager_ms_per_step": round(eager_total / args.steps * 1e3, 4),
                       "flops_per_step": flops},
            "mfma_peak_frac": round(value / peak, 4),
            "roofline": roofline, "bn_stats": bn, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
