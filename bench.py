"""Benchmark of the FNO spectral-convolution layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config c2] [--dtype f16]

A step is one whole layer (every launch of the path) over one batch of
synthetic input already resident in HBM. Buffer sets are rotated so that the
whole working set exceeds 1 GiB and the 256 MB Infinity Cache cannot serve
it. Before the W warm-up steps of every timed loop the same calls run untimed
for --settle-ms (default 300 ms): after an idle period the device's power
management first runs kernels fast for about a millisecond and then slows
every kernel in steps by up to ~25 % for a few milliseconds before settling,
so a short timed region that starts from idle measures that transient instead
of the sustained rate. Prints one JSON line:

* value: layers/s on the headline workload (default: the 256x256 fp16 layer,
  B=32, Cin=Cout=64, modes 32x32), GB/s and the fraction of the 8 TB/s HBM
  peak from the layer's minimal bytes (read x + read w + write y once);
* roofline: the layer's dominant kernel, its algorithmic bytes per launch
  (the compulsory bytes of its own step: x for the forward planes, w for the
  contraction, y for the inverse planes) over its average launch time (HIP
  events on the stream it runs on), the spectra-inclusive rate beside it, and
  the measured HBM traffic per launch from the committed counter summary;
* cpu_baseline: the float64 oracle timed on this host's cores on a bounded
  sample of the headline workload (whole batch elements), scaled to layers/s;
* metric_configs: the same three objects (layer rate, roofline,
  cpu_baseline) for every workload the metric is quoted on: 128x128 fp32 and
  fp16, 256x256 fp16 and bf16, 64^3 fp32. The headline times exactly K
  layers; every other workload at least 200 (its `steps`), since 20 layers
  of the 128x128 layer last ~0.5 ms, too short to read stably;
* per_layer_us / hot_single_set_layers_per_s: the distribution of single
  layers inside the rotating back-to-back loop, and the same loop on one
  buffer set (which the Infinity Cache may serve; never the headline);
* configs: the 16x16 fp32 layer (launch-bound);
* latency: per-call latency of the 128^2 fp32 layer shape at batch 1, 2, 4, 8,
  launched eagerly and replayed from a captured HIP graph;
* model: the full FNO2d forward (B=20, 256^2, width 64, modes 24x24, fp16);
* backward: the layer's backward pass on the 128^2 fp32, 256^2 fp16 and 64^3
  fp32 layers, from its minimal bytes (read x, w, dL/dy, write grad_x, grad_w).
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused spectral-conv layers/sec + GB/s (% HBM peak) at 128², 256², 64³"
HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 1 << 30
MAX_SETS = 64


SETTLE_MS = 300.0


def _kernel_bytes(cfg, dtype, name, half_exchange=False):
    """Bytes of one launch of kernel `name`: (algorithmic, exchange).

    Algorithmic bytes are the compulsory bytes of the kernel's own step of
    the layer: x for the forward planes, w for the contraction, y for the
    inverse planes, nothing for the 3D outer-axis passes. Exchange bytes are
    the spectra (and 3D slab transforms) it also writes or reads: complex
    fp32 (8 bytes a mode), or with the half exchange fp16 pairs (4 bytes a
    mode) plus an int32 exponent per forward plane and an int8 one per four
    contracted modes."""
    s = 4 if dtype == "f32" else 2
    pts = int(np.prod(cfg.grid))
    x = cfg.batch * cfg.c_in * pts * s
    y = cfg.batch * cfg.c_out * pts * s
    w = cfg.n_modes * cfg.c_in * cfg.c_out * 2 * s
    if half_exchange:
        xh = cfg.batch * cfg.c_in * (cfg.n_modes * 4 + 4)
        yh = cfg.batch * cfg.c_out * (cfg.n_modes * 4 + (cfg.n_modes + 3) // 4)
    else:
        xh = cfg.batch * cfg.c_in * cfg.n_modes * 8
        yh = cfg.batch * cfg.c_out * cfg.n_modes * 8
    if cfg.ndim == 2:
        ti = to = None
    else:
        C = 2 * cfg.modes[1] * cfg.modes[2]
        ti = cfg.batch * cfg.c_in * cfg.grid[0] * C * 8
        to = cfg.batch * cfg.c_out * cfg.grid[0] * C * 8
    if name.startswith("fno_fwd_plane"):
        return x, (xh if ti is None else ti)
    if name.startswith("fno_fwd_axis"):
        return 0, ti + xh
    if name.startswith("fno_contract"):
        return w, xh + yh
    if name.startswith("fno_inv_axis"):
        return 0, yh + to
    if name.startswith("fno_inv_plane"):
        return y, (yh if to is None else to)
    if name.startswith("fno_layer_fused"):
        return x + w + y, 2 * (xh + yh)
    raise KeyError(name)


def to_device(arr, dtype, device="cuda:0"):
    import torch
    a = np.ascontiguousarray(arr)
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" \
        else torch.from_numpy(a)
    return t.to(device)


class Layer:
    """Plan plus rotating device buffer sets for one workload."""

    def __init__(self, cfg, dtype):
        import torch
        import spectral_convolution_amd as fno
        import workloads as wl
        self.fno, self.cfg, self.dtype = fno, cfg, dtype
        inp = wl.layer_inputs(cfg, dtype)
        self.plan = fno.fno_plan_create(cfg.ndim, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid,
                                        cfg.modes, dtype, 0)
        x0, w0 = to_device(inp["x"], dtype), to_device(inp["w"], dtype)
        per_set = cfg.minimal_bytes(dtype)
        # enough sets to exceed the Infinity Cache; tiny layers stay cache-resident
        # whatever the count, so their rotation is capped
        self.nsets = min(MAX_SETS, max(1, math.ceil(ROTATE_BYTES / per_set)))
        self.sets = []
        for i in range(self.nsets):
            x = x0 if i == 0 else x0.clone()
            w = w0 if i == 0 else w0.clone()
            y = torch.empty(self.plan.y_shape(), dtype=x0.dtype, device=x0.device)
            self.sets.append((x, w, y))
        self.call = fno.fno_spectral_conv2d if cfg.ndim == 2 else fno.fno_spectral_conv3d
        self.stream = torch.cuda.current_stream()
        self.names = [fno.fno_plan_launch_name(self.plan, i)
                      for i in range(fno.fno_plan_num_launches(self.plan))]

    def step(self, i):
        x, w, y = self.sets[i % self.nsets]
        self.call(self.plan, x, w, y, self.stream)

    def launch(self, idx, i):
        x, w, y = self.sets[i % self.nsets]
        self.fno.fno_plan_run_launch(self.plan, idx, x, w, y, self.stream)

    def set_shape(self, shape):
        """Select a launch shape; False when the plan has no such shape."""
        try:
            self.fno.fno_plan_set_launch_shape(self.plan, shape)
        except self.fno.FnoError:
            return False
        self.names = [self.fno.fno_plan_launch_name(self.plan, i)
                      for i in range(self.fno.fno_plan_num_launches(self.plan))]
        return True

    def close(self):
        self.fno.fno_plan_destroy(self.plan)
        self.sets = []


class Backward:
    """Plan plus rotating device buffer sets for the backward pass of one
    workload."""

    def __init__(self, cfg, dtype):
        import torch
        import spectral_convolution_amd as fno
        import workloads as wl
        self.fno, self.cfg, self.dtype = fno, cfg, dtype
        inp = wl.layer_inputs(cfg, dtype)
        gout = wl.layer_grad_output(cfg, dtype)
        self.plan = fno.fno_plan_create(cfg.ndim, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid,
                                        cfg.modes, dtype, 0)
        x0, w0, g0 = (to_device(inp["x"], dtype), to_device(inp["w"], dtype),
                      to_device(gout["g"], dtype))
        self.nsets = min(MAX_SETS, max(1, math.ceil(ROTATE_BYTES / backward_minimal_bytes(cfg, dtype))))
        self.sets = []
        for i in range(self.nsets):
            x, w, g = (x0, w0, g0) if i == 0 else (x0.clone(), w0.clone(), g0.clone())
            self.sets.append((x, w, g, torch.empty_like(x), torch.empty_like(w)))
        self.call = (fno.fno_spectral_conv2d_backward if cfg.ndim == 2
                     else fno.fno_spectral_conv3d_backward)
        self.stream = torch.cuda.current_stream()
        # the training-step form: the forward leaves the spectra of x in a
        # saved buffer (written once here, outside any timing) and the
        # backward reads them instead of x
        self.saved = []
        self.saved_bytes = fno.fno_plan_saved_bytes(self.plan)
        self.y = torch.empty(self.plan.y_shape(), dtype=x0.dtype, device=x0.device)
        if self.saved_bytes is not None:
            for x, w, _, _, _ in self.sets:
                buf = fno.fno_saved_empty(self.plan)
                fno.fno_spectral_conv_forward_save(self.plan, x, w, self.y, buf, self.stream)
                self.saved.append(buf)
            torch.cuda.synchronize()

    def step(self, i):
        x, w, g, gx, gw = self.sets[i % self.nsets]
        self.call(self.plan, x, w, g, gx, gw, self.stream)

    def step_saved(self, i):
        _, w, g, gx, gw = self.sets[i % self.nsets]
        self.fno.fno_spectral_conv_backward_saved(self.plan, self.saved[i % self.nsets], w, g, gx, gw,
                                                  self.stream)

    def train_step(self, i):
        """One layer's share of a training step: the forward that saves the
        spectra of x, then the backward from them."""
        x, w, _, _, _ = self.sets[i % self.nsets]
        self.fno.fno_spectral_conv_forward_save(self.plan, x, w, self.y, self.saved[i % self.nsets], self.stream)
        self.step_saved(i)

    def close(self):
        self.fno.fno_plan_destroy(self.plan)
        self.sets = []
        self.saved = []


def backward_minimal_bytes(cfg, dtype):
    """Read x, w and dL/dy once; write grad_x and grad_w once."""
    s = 4 if dtype == "f32" else 2
    pts = int(np.prod(cfg.grid))
    w = cfg.n_modes * cfg.c_in * cfg.c_out * 2 * s
    return 2 * cfg.batch * cfg.c_in * pts * s + cfg.batch * cfg.c_out * pts * s + 2 * w


def backward_saved_minimal_bytes(cfg, dtype, saved_bytes):
    """Read the saved spectra of x, w and dL/dy once; write grad_x and grad_w
    once."""
    s = 4 if dtype == "f32" else 2
    pts = int(np.prod(cfg.grid))
    w = cfg.n_modes * cfg.c_in * cfg.c_out * 2 * s
    return saved_bytes + cfg.batch * cfg.c_in * pts * s + cfg.batch * cfg.c_out * pts * s + 2 * w


def measure_backward(cfg, dtype, steps, warmup, settle_ms=SETTLE_MS):
    """The backward from x, and (where the plan has a saved format) from the
    spectra of x that the forward saved."""
    bw = Backward(cfg, dtype)
    try:
        ms = _time_loop(bw.step, steps, warmup, bw.stream, settle_ms)
        gbps = backward_minimal_bytes(cfg, dtype) / (ms * 1e-3) / 1e9
        out = {"workload": cfg.name, "dtype": dtype, "ms_per_backward": ms,
               "backward_per_s": 1000.0 / ms, "minimal_bytes": backward_minimal_bytes(cfg, dtype),
               "gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS}
        if bw.saved:
            ms_s = _time_loop(bw.step_saved, steps, warmup, bw.stream, settle_ms)
            nb = backward_saved_minimal_bytes(cfg, dtype, bw.saved_bytes)
            ms_t = _time_loop(bw.train_step, steps, warmup, bw.stream, settle_ms)
            out.update({"ms_per_backward_saved": ms_s, "backward_saved_per_s": 1000.0 / ms_s,
                        "saved_bytes": bw.saved_bytes, "minimal_bytes_saved": nb,
                        "gbps_saved": nb / (ms_s * 1e-3) / 1e9,
                        "ms_per_train_step": ms_t, "train_steps_per_s": 1000.0 / ms_t})
        return out
    finally:
        bw.close()


def _latencies(fn, n, warmup, stream):
    """Per-call latency in µs: each call between its own pair of events,
    synchronised before the next."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        fn(i)
        b.record(stream)
        b.synchronize()
    t = np.array([a.elapsed_time(b) * 1000.0 for a, b in ev])
    return {"mean": float(t.mean()), "std": float(t.std()), "min": float(t.min()),
            "p50": float(np.median(t)), "p99": float(np.percentile(t, 99))}


def latency_sweep(n=200, warmup=20):
    """The 128^2 fp32 layer (Ci=Co=32, modes 16x16) at batch 1..8: eager
    calls in the plan's default launch shape (three kernels) and as one
    cooperative launch, and replays of a captured graph of one call (the
    three kernels: a captured call never takes the cooperative launch)."""
    import torch
    import spectral_convolution_amd as fno
    import workloads as wl
    base = wl.CONFIGS["c1"]
    out = []
    for B in (1, 2, 4, 8):
        inp = wl.layer_inputs(base, "f32", batch=B)
        plan = fno.fno_plan_create(2, B, base.c_in, base.c_out, base.grid, base.modes, "f32", 0)
        try:
            x, w = to_device(inp["x"], "f32"), to_device(inp["w"], "f32")
            y = torch.empty(plan.y_shape(), dtype=x.dtype, device=x.device)
            stream = torch.cuda.current_stream()
            shape = fno.fno_plan_get_launch_shape(plan)
            fno.fno_plan_set_launch_shape(plan, "fused")
            eager_fused = _latencies(lambda i: fno.fno_spectral_conv2d(plan, x, w, y, stream), n, warmup, stream)
            fno.fno_plan_set_launch_shape(plan, shape)
            eager = _latencies(lambda i: fno.fno_spectral_conv2d(plan, x, w, y, stream), n, warmup, stream)
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                fno.fno_spectral_conv2d(plan, x, w, y)
            stream.wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fno.fno_spectral_conv2d(plan, x, w, y)
            torch.cuda.synchronize()
            replay = _latencies(lambda i: graph.replay(), n, warmup, torch.cuda.current_stream())
            del graph
            out.append({"batch": B, "launch_shape": shape, "eager_us": eager, "eager_fused_us": eager_fused,
                        "graph_us": replay,
                        "samples_per_s_eager": B / (eager["mean"] * 1e-6),
                        "samples_per_s_graph": B / (replay["mean"] * 1e-6)})
        finally:
            torch.cuda.synchronize()
            fno.fno_plan_destroy(plan)
    return {"workload": "FNO2d spectral-conv layer, fp32, Cin=Cout=32, 128x128, modes 16x16",
            "calls_per_batch": n, "sweep": out,
            "throughput_gain_b1_to_b8_eager": out[-1]["samples_per_s_eager"] / out[0]["samples_per_s_eager"],
            "throughput_gain_b1_to_b8_graph": out[-1]["samples_per_s_graph"] / out[0]["samples_per_s_graph"]}


class Model:
    """FNO2d model plan with random-init parameters on the device."""

    def __init__(self, cfg, batch=None):
        import torch
        import spectral_convolution_amd as fno
        import workloads as wl
        inp = wl.model_inputs(cfg, batch=batch)
        dt = inp["dtype"]
        self.fno, self.B = fno, inp["batch"]
        H, W = inp["grid"]
        self.model = fno.fno_model2d_create(self.B, (H, W), cfg.in_channels, cfg.width, cfg.n_layers,
                                            cfg.modes, cfg.proj_hidden, cfg.out_channels, dt, 0)
        self.params = [to_device(inp["P"], dt), to_device(inp["p"], dt)]
        for L in inp["layers"]:
            self.params += [to_device(L["spectral"], dt), to_device(L["W"], dt), to_device(L["b"], dt)]
        self.params += [to_device(inp[k], dt) for k in ("Q1", "q1", "Q2", "q2")]
        self.f = to_device(inp["features"], dt)
        self.out = torch.empty((self.B, cfg.out_channels, H, W), dtype=self.f.dtype, device=self.f.device)
        self.stream = torch.cuda.current_stream()

    def step(self, i):
        self.fno.fno_model2d_forward(self.model, self.f, self.params, self.out, self.stream)

    def set_graph(self, on):
        self.fno.fno_model2d_set_graph(self.model, on)

    def close(self):
        self.fno.fno_model2d_destroy(self.model)


def measure_model(steps, warmup, settle_ms=SETTLE_MS):
    """The B=20 forward (eager kernels, and replayed from the model's captured
    HIP graph) and its batch-1 latency both ways."""
    import workloads as wl
    cfg = wl.CONFIGS["c4"]
    m = Model(cfg)
    try:
        ms = _time_loop(m.step, steps, warmup, m.stream, settle_ms)
        res = {"workload": "FNO2d forward, B=20, 256x256, lift 3->64, 4 x (spectral conv 64->64 modes "
                           "24x24 + 1x1 conv + GELU), projection 64->128->1, fp16 storage",
               "ms_per_forward": ms, "samples_per_s": m.B / (ms * 1e-3)}
        m.set_graph(True)
        msg = _time_loop(m.step, steps, warmup, m.stream, settle_ms)
        res["ms_per_forward_graph"] = msg
        res["samples_per_s_graph"] = m.B / (msg * 1e-3)
    finally:
        m.close()
    m1 = Model(cfg, batch=1)
    try:
        res["latency_b1_us"] = _latencies(m1.step, 100, 10, m1.stream)
        m1.set_graph(True)
        res["latency_b1_graph_us"] = _latencies(m1.step, 100, 10, m1.stream)
    finally:
        m1.close()
    return res


def _settle(fn, ms, stream):
    """Run fn(i) untimed for `ms` milliseconds of wall time, keeping about
    eight calls queued on the device (waits on an event recorded eight calls
    earlier), so the device never idles while the host loops."""
    import torch
    if ms <= 0:
        return 0
    pending = []
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1000.0 < ms:
        fn(n)
        n += 1
        ev = torch.cuda.Event()
        ev.record(stream)
        pending.append(ev)
        if len(pending) > 8:
            pending.pop(0).synchronize()
    return n


def _time_loop(fn, steps, warmup, stream, settle_ms=0.0):
    """ms per call of `steps` back-to-back calls between two HIP events on
    `stream`, after `settle_ms` of untimed calls and `warmup` warm-up calls."""
    import torch
    _settle(fn, settle_ms, stream)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per call


def _per_call(fn, n, stream, settle_ms=0.0):
    """Per-call times in µs inside a back-to-back stream of calls: one event
    between consecutive calls, no synchronisation until the end."""
    import torch
    _settle(fn, settle_ms, stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for i in range(n):
        fn(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t = np.array([ev[i].elapsed_time(ev[i + 1]) * 1000.0 for i in range(n)])
    return {"mean": float(t.mean()), "std": float(t.std()), "min": float(t.min()),
            "p50": float(np.median(t)), "n": n}


def _kernel_times(lay, steps, warmup, settle_ms):
    """Average duration of each launch of the layer: max(steps, 200)
    back-to-back launches of that kernel alone (rotating buffer sets) between
    two HIP events recorded on the plan's stream, the stream the kernel runs
    on (at least 200, so one stalled launch cannot dominate the average)."""
    n = max(steps, 200)
    return [_time_loop(lambda i, idx=idx: lay.launch(idx, i), n, warmup, lay.stream, settle_ms)
            for idx in range(len(lay.names))]


def _roofline(cfg, dtype, kernels):
    """Roofline object of the layer's dominant (longest) kernel."""
    dom = max(kernels, key=lambda k: k["ms"])
    return {"bound": "hbm", "kernel": dom["kernel"], "achieved": dom["gbps"], "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": dom["gbps"] / HBM_PEAK_GBPS,
            "traffic": measured_traffic(dom["kernel"], cfg.name, dtype),
            "algorithmic_bytes": dom["algorithmic_bytes"], "exchange_bytes": dom["exchange_bytes"],
            "ms_per_launch": dom["ms"], "achieved_with_exchange": dom["gbps_with_exchange"]}


def measure(cfg, dtype, steps, warmup, settle_ms=SETTLE_MS, per_kernel=True, shapes=("fused", "separate")):
    lay = Layer(cfg, dtype)
    try:
        ms = _time_loop(lay.step, steps, warmup, lay.stream, settle_ms)
        res = {"workload": cfg.name, "description": cfg.description, "dtype": dtype, "ms_per_layer": ms,
               "layers_per_s": 1000.0 / ms, "minimal_bytes": cfg.minimal_bytes(dtype),
               "gbps": cfg.minimal_bytes(dtype) / (ms * 1e-3) / 1e9}
        res["hbm_frac"] = res["gbps"] / HBM_PEAK_GBPS
        # distribution of single layers inside the rotating back-to-back loop
        res["per_layer_us"] = _per_call(lay.step, min(steps, 500), lay.stream, settle_ms)
        # one buffer set reused: x, w and y may then be served from the
        # Infinity Cache, so this is not the HBM-bound figure
        hot = _time_loop(lambda i: lay.step(0), steps, max(2, warmup // 4), lay.stream, settle_ms)
        res["hot_single_set_layers_per_s"] = 1000.0 / hot
        shape = lay.fno.fno_plan_get_launch_shape(lay.plan)
        res["launch_shape"] = shape
        res["half_exchange"] = lay.fno.fno_plan_spectra_format(lay.plan) == 1
        res["arithmetic"] = arithmetic(dtype, res["half_exchange"])
        # ablation: the layer in each launch shape the plan has (one
        # cooperative launch, or the three stand-alone kernels)
        res["launch_shapes"] = {}
        for sh in shapes:
            if not lay.set_shape(sh):
                continue
            t = _time_loop(lay.step, steps, warmup, lay.stream, settle_ms)
            res["launch_shapes"][sh] = {"ms_per_layer": t, "layers_per_s": 1000.0 / t,
                                        "launches_per_layer": len(lay.names)}
        if per_kernel:
            # every kernel of both shapes alone; the roofline takes the
            # dominant kernel of the shape the layer runs in
            res["kernels"] = []
            for sh in [x for x in ("separate", "fused") if x in shapes]:
                if not lay.set_shape(sh):
                    continue
                kms = _kernel_times(lay, steps, max(2, warmup // 4), settle_ms)
                half = sh == "separate" and lay.fno.fno_plan_spectra_format(lay.plan) == 1
                for name, t in zip(lay.names, kms):
                    alg, exch = _kernel_bytes(cfg, dtype, name, half)
                    g = alg / (t * 1e-3) / 1e9
                    res["kernels"].append({"kernel": name, "launch_shape": sh, "ms": t, "algorithmic_bytes": alg,
                                           "exchange_bytes": exch, "gbps": g, "frac": g / HBM_PEAK_GBPS,
                                           "gbps_with_exchange": (alg + exch) / (t * 1e-3) / 1e9})
            res["roofline"] = _roofline(cfg, dtype, [k for k in res["kernels"] if k["launch_shape"] == shape])
        lay.set_shape(shape)
        return res
    finally:
        lay.close()


# layers (or backward passes) timed per workload other than the headline
EXTRA_STEPS = 200


def measured_traffic(kernel, cfg_name, dtype):
    """HBM bytes per launch of `kernel` on this workload from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by
    what the counter reads for a plain copy of known size), or None when no
    summary exists or the kernel source changed since it was taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"{kernel}_{cfg_name}_{dtype}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    srcs = re.findall(r"^source:\s*(\S+)\s+sha256\s+([0-9a-f]{64})", text, re.M)
    if not (m_b and srcs):
        return None
    # every source the kernel is compiled from must be unchanged
    for rel, digest in srcs:
        src = os.path.join(ROOT, rel)
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != digest:
            return None
    return int(m_b.group(1))


def copy_bandwidth(nbytes, steps=20, warmup=3):
    """Device-to-device copy of nbytes (read + write counted): the achievable
    HBM rate on this machine, and a plain copy kernel of known size for scaling
    hardware byte counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    ms = _time_loop(lambda i: dst.copy_(src), steps, warmup, torch.cuda.current_stream())
    return {"bytes_copied": nbytes, "ms": ms, "gbps": 2 * nbytes / (ms * 1e-3) / 1e9}


def cache_probe(cfg, dtype, n=100):
    """Where the exchanged spectra are read from. Each launch of the layer
    is timed alone (events around it) when it runs right after its producer,
    against runs with a read-only sweep of 1 GiB (a sum, no dirty lines)
    in between, which evicts the 256 MB Infinity Cache:
      as_layer:        forward, contraction, inverse
      weights_evicted: sweep, forward, contraction, inverse
      spectra_evicted: forward, sweep, contraction, sweep, inverse
    Medians over n iterations, in us."""
    import torch
    lay = Layer(cfg, dtype)
    try:
        big = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        acc = torch.zeros(1, device="cuda:0")
        s = lay.stream
        out = {}
        for mode in ("as_layer", "weights_evicted", "spectra_evicted"):
            t = {k: [] for k in lay.names}
            for it in range(n + 10):
                if mode == "weights_evicted":
                    acc.add_(big.sum())
                ev = []
                for idx in range(len(lay.names)):
                    if mode == "spectra_evicted" and idx > 0:
                        acc.add_(big.sum())
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(s)
                    lay.launch(idx, 0)
                    e1.record(s)
                    ev.append((e0, e1))
                torch.cuda.synchronize()
                if it >= 10:
                    for idx, (e0, e1) in enumerate(ev):
                        t[lay.names[idx]].append(e0.elapsed_time(e1) * 1000.0)
            out[mode] = {k: float(np.median(v)) for k, v in t.items()}
        return out
    finally:
        lay.close()


def cpu_baseline(cfg, dtype, budget_s=8.0):
    """The float64 oracle, as it stands, on this host's cores. Batch elements
    of the layer are independent, so it runs on one batch element of the
    workload (same grid, channels, modes and weights shape) for about
    budget_s seconds after one warm-up, and the rate is scaled to layers/s of
    the full batch."""
    import oracle
    import workloads as wl
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))
    nb = 1
    inp = wl.layer_inputs(cfg, dtype, batch=nb)
    f = oracle.spectral_conv2d if cfg.ndim == 2 else oracle.spectral_conv3d
    with threadpool_limits(limits=cores):
        pools = threadpool_info()
        used = max([p.get("num_threads", 1) for p in pools] + [1])
        blas = ", ".join(sorted({f"{p.get('internal_api', '?')} {p.get('version') or ''}".strip()
                                 for p in pools if p.get("user_api") == "blas"})) or "unknown"
        f(inp["x64"], inp["w64"], *cfg.modes)  # warm-up
        n, t0 = 0, time.perf_counter()
        while True:
            f(inp["x64"], inp["w64"], *cfg.modes)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    rate = n * nb / cfg.batch / el
    return {"value": rate, "unit": "layers/s", "cores": int(used), "kind": "oracle",
            "sample": f"{cfg.name} layer ({cfg.description}) on {nb} of its {cfg.batch} batch elements, "
                      f"{n} runs in {el:.1f} s after one warm-up, scaled by {nb}/{cfg.batch} to layers/s; "
                      f"float64 numpy (BLAS: {blas}), host affinity {cores} cores",
            "gbps_minimal_bytes": cfg.minimal_bytes(dtype) * rate / 1e9}


def arithmetic(dtype, half_exchange):
    """What the layer multiplies in, by storage dtype and spectra exchange
    format (fp16 / bf16 plans from batch 16 exchange fp16 spectra and run the
    matrix-core contraction; smaller batches keep complex fp32 spectra and
    the fp32 contraction)."""
    if dtype == "f32":
        return ("f32 storage; transforms on f16 hi+lo split MFMA operands (about 22 significant bits), "
                "contraction on f32 MFMA, f32 accumulation throughout")
    head = (f"{dtype} storage; transforms on f16 MFMA operands scaled by powers of two, ")
    if not half_exchange:
        return head + "spectra exchanged as complex f32, contraction on f32 MFMA, f32 accumulation throughout"
    if dtype == "f16":
        return head + ("spectra exchanged as f16 pairs with power-of-two exponents, contraction on f16 MFMA "
                       "operands (spectra at one power-of-two scale per batch row, weights as stored), "
                       "f32 accumulation throughout")
    return head + ("spectra exchanged as f16 pairs with power-of-two exponents, contraction on bf16 hi+lo split "
                   "MFMA operands (exact for f16 spectra and bf16 weights), f32 accumulation throughout")


DTYPE_LABEL = {"f32": "f32 (f16 hi+lo MFMA, f32 acc)", "f16": "f16 (MFMA, f32 acc)",
               "bf16": "bf16 storage (f16 MFMA, f32 acc)"}

# every workload the metric is quoted on: 128^2, 256^2 and 64^3 layers
METRIC_CONFIGS = [("c2", "f16"), ("c2", "bf16"), ("c1", "f32"), ("c1", "f16"), ("c3", "f32")]


def _summary(r):
    d = r["per_layer_us"]
    rf = r["roofline"]
    shp = ", ".join(f"{k} {v['layers_per_s']:.0f}/s" for k, v in r.get("launch_shapes", {}).items())
    return (f"{r['workload']} {r['dtype']} [{r.get('launch_shape')}; {shp}]: {r['layers_per_s']:.1f} layers/s, "
            f"{r['gbps']:.0f} GB/s "
            f"({100 * r['hbm_frac']:.1f} % of 8 TB/s); per layer p50 {d['p50']:.1f} us (mean {d['mean']:.1f}, "
            f"std {d['std']:.1f}, min {d['min']:.1f}); dominant {rf['kernel']} {1000 * rf['ms_per_launch']:.1f} us "
            f"= {rf['achieved']:.0f} GB/s algorithmic ({100 * rf['frac']:.1f} %)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 100 warm-up and 1000 timed launches per workload (the timed region
    # of the 256^2 layers is then ~0.15 s)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed calls before every warm-up (device power-state settle)")
    ap.add_argument("--config", default="c2")
    ap.add_argument("--dtype", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="only the headline workload")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-latency", action="store_true")
    ap.add_argument("--no-model", action="store_true")
    ap.add_argument("--model-only", action="store_true", help="only time the full FNO2d forward (profiling runs)")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time the backward pass of --config/--dtype (profiling runs)")
    ap.add_argument("--separate-only", action="store_true",
                    help="time only the three-launch shape (profiling runs: no cooperative launch)")
    ap.add_argument("--cache-probe", action="store_true",
                    help="only time each launch of --config/--dtype right after its producer and with the "
                         "Infinity Cache evicted in between (where the exchanged spectra are read from)")
    ap.add_argument("--copy-only", type=int, default=0, metavar="BYTES",
                    help="only time a device-to-device copy of BYTES (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported (the layer "
              "shards over the batch with no communication, so one GPU's throughput at its "
              "per-GPU shape is the measurement)", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py: no GPU available", file=sys.stderr)
        sys.exit(1)
    if args.copy_only:
        print(json.dumps({"copy": copy_bandwidth(args.copy_only, args.steps, args.warmup)}))
        return
    cfg = wl.CONFIGS[args.config]
    dtype = args.dtype or cfg.dtypes[0]
    settle = args.settle_ms
    if args.model_only:
        print(json.dumps({"model": measure_model(args.steps, args.warmup, settle)}))
        return
    if args.cache_probe:
        print(json.dumps({"cache_probe": cache_probe(cfg, dtype)}))
        return
    if args.backward_only:
        print(json.dumps({"backward": [measure_backward(cfg, dtype, args.steps, args.warmup, settle)]}))
        return
    shapes = ("separate",) if args.separate_only else ("fused", "separate")
    main_res = measure(cfg, dtype, args.steps, args.warmup, settle, shapes=shapes)
    print("[bench] " + _summary(main_res), file=sys.stderr, flush=True)
    out = {
        "metric": METRIC, "value": main_res["layers_per_s"], "unit": "layers/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_layer"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE_LABEL[dtype], "arithmetic": main_res["arithmetic"],
        "data": "synthetic (seeded Gaussian random fields; random weights)",
        "config": {"workload": cfg.description, "name": cfg.name, "batch": cfg.batch,
                   "c_in": cfg.c_in, "c_out": cfg.c_out, "grid": list(cfg.grid),
                   "modes": list(cfg.modes), "storage": dtype,
                   "minimal_bytes": cfg.minimal_bytes(dtype)},
        "gbps": main_res["gbps"], "hbm_frac": main_res["hbm_frac"],
        "roofline": main_res["roofline"],
        "kernels": main_res["kernels"],
        "per_layer_us": main_res["per_layer_us"],
        "hot_single_set_layers_per_s": main_res["hot_single_set_layers_per_s"],
        "settle_ms": settle,
    }
    results = {(cfg.name, dtype): main_res}
    if not args.no_extra:
        for name, dt in METRIC_CONFIGS + [("c0", "f32")]:
            if (name, dt) in results:
                continue
            # the other workloads time at least EXTRA_STEPS layers: a 20-layer
            # loop of the 128x128 layer is ~0.5 ms, too short to read stably
            r = measure(wl.CONFIGS[name], dt, max(args.steps, EXTRA_STEPS), max(args.warmup, EXTRA_STEPS // 10),
                        settle, shapes=shapes)
            r["steps"] = max(args.steps, EXTRA_STEPS)
            results[(name, dt)] = r
            print("[bench] " + _summary(r), file=sys.stderr, flush=True)
    cpu = {}
    if not args.no_cpu_baseline:
        for name, dt in [(cfg.name, dtype)] + METRIC_CONFIGS:
            if name in cpu or (name, dt) not in results:
                continue
            cpu[name] = cpu_baseline(wl.CONFIGS[name], dt)
            print(f"[bench] oracle {name}: {cpu[name]['value']:.3f} layers/s on {cpu[name]['cores']} cores",
                  file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu.get(cfg.name)
    out["metric_configs"] = []
    for key in METRIC_CONFIGS:
        if key in results:
            r = dict(results[key])
            r["cpu_baseline"] = cpu.get(key[0])
            r["dtype_label"] = DTYPE_LABEL[key[1]]
            out["metric_configs"].append(r)
    out["configs"] = [results[k] for k in results if k not in METRIC_CONFIGS and k != (cfg.name, dtype)]
    if not args.no_backward:
        bwd = []
        for name, dt in (("c1", "f32"), ("c2", "f16"), ("c3", "f32")):
            r = measure_backward(wl.CONFIGS[name], dt, max(EXTRA_STEPS, args.steps // 2), max(5, args.warmup // 2),
                                 settle)
            bwd.append(r)
            sv = (f"; from saved spectra {r['backward_saved_per_s']:.1f} /s, {r['gbps_saved']:.0f} GB/s; "
                  f"forward (saving) + backward {r['train_steps_per_s']:.1f} /s"
                  if "backward_saved_per_s" in r else "")
            print(f"[bench] backward {name} {dt}: {r['backward_per_s']:.1f} /s, {r['gbps']:.0f} GB/s{sv}",
                  file=sys.stderr, flush=True)
        out["backward"] = bwd
    if not args.no_model:
        out["model"] = measure_model(max(10, args.steps // 10), max(3, args.warmup // 4), settle)
        mo = out["model"]
        print(f"[bench] model: {mo['ms_per_forward']:.3f} ms per B=20 forward ({mo['ms_per_forward_graph']:.3f} "
              f"graph), B=1 latency {mo['latency_b1_us']['mean']:.1f} us ({mo['latency_b1_graph_us']['mean']:.1f} "
              f"graph)", file=sys.stderr, flush=True)
    if not args.no_latency:
        out["latency"] = latency_sweep()
        print("[bench] latency " + ", ".join(
            f"B={r['batch']}: eager ({r['launch_shape']}) {r['eager_us']['mean']:.1f}±{r['eager_us']['std']:.1f} us, "
            f"eager (fused) {r['eager_fused_us']['mean']:.1f} us, "
            f"graph {r['graph_us']['mean']:.1f}±{r['graph_us']['std']:.1f} us"
            for r in out["latency"]["sweep"]), file=sys.stderr, flush=True)
    out["copy_1gib"] = copy_bandwidth(1 << 30)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
