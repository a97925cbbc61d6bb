"""Benchmark of the fused-path FNO spectral-convolution layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config c1] [--dtype f32]

A step is one whole layer (every launch of the path) over one batch of
synthetic input already resident in HBM. Buffer sets are rotated so that the
whole working set exceeds 1 GiB and the 256 MB Infinity Cache cannot serve
it. Prints one JSON line:

* value: layers/s on the main workload (default: the 128x128 fp32 layer,
  B=16, Cin=Cout=32, modes 16x16), plus GB/s and the fraction of the 8 TB/s
  HBM peak from the minimal bytes (read x + read w + write y once);
* roofline: the dominant kernel's algorithmic bytes per launch over its
  average launch time (HIP events on the stream it runs on);
* cpu_baseline: the float64 oracle timed on this host's cores on the same
  workload;
* per_layer_us: the distribution (p50, mean, std, min) of single layers
  inside the rotating back-to-back loop, and hot_single_set_layers_per_s:
  the same loop on one buffer set (which the Infinity Cache may serve;
  labelled, never the headline);
* configs: the same figures for the 128^2 fp16, 256^2 fp16 / bf16, 64^3
  fp32 and 16^2 fp32 layers;
* latency: per-call latency (mean, std, min over individually timed calls)
  of the 128^2 fp32 layer shape at batch 1, 2, 4, 8, launched eagerly and
  replayed from a captured HIP graph, with the throughput gain from batch 1
  to 8;
* model: the full FNO2d forward (lift, four spectral blocks with the 1x1
  bypass and GELU, projection; B=20, 256^2, width 64, modes 24x24, fp16
  storage) as forwards/s and samples/s, and its per-call latency at batch 1;
* backward: the layer's backward pass (grad_x and grad_w from dL/dy) on the
  128^2 fp32, 256^2 fp16 and 64^3 fp32 layers, as backward passes/s and GB/s
  from its minimal bytes (read x, w, dL/dy once, write grad_x, grad_w once).
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


def _bytes_per_launch(cfg, dtype):
    """Algorithmic bytes of each launch: its compulsory input and output."""
    s = 4 if dtype == "f32" else 2
    pts = int(np.prod(cfg.grid))
    x = cfg.batch * cfg.c_in * pts * s
    y = cfg.batch * cfg.c_out * pts * s
    w = cfg.n_modes * cfg.c_in * cfg.c_out * 2 * s
    xh = cfg.batch * cfg.c_in * cfg.n_modes * 8
    yh = cfg.batch * cfg.c_out * cfg.n_modes * 8
    if cfg.ndim == 2:
        return {"fno_fwd_plane": x + xh, "fno_fwd_plane_mx": x + xh, "fno_contract": xh + w + yh,
                "fno_inv_plane": yh + y, "fno_inv_plane_mx": yh + y}
    C = 2 * cfg.modes[1] * cfg.modes[2]
    ti = cfg.batch * cfg.c_in * cfg.grid[0] * C * 8
    to = cfg.batch * cfg.c_out * cfg.grid[0] * C * 8
    return {"fno_fwd_plane": x + ti, "fno_fwd_plane_mx": x + ti, "fno_fwd_axis": ti + xh,
            "fno_contract": xh + w + yh, "fno_inv_axis": yh + to, "fno_inv_plane": to + y,
            "fno_inv_plane_mx": to + y}


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

    def step(self, i):
        x, w, g, gx, gw = self.sets[i % self.nsets]
        self.call(self.plan, x, w, g, gx, gw, self.stream)

    def close(self):
        self.fno.fno_plan_destroy(self.plan)
        self.sets = []


def backward_minimal_bytes(cfg, dtype):
    """Read x, w and dL/dy once; write grad_x and grad_w once."""
    s = 4 if dtype == "f32" else 2
    pts = int(np.prod(cfg.grid))
    w = cfg.n_modes * cfg.c_in * cfg.c_out * 2 * s
    return 2 * cfg.batch * cfg.c_in * pts * s + cfg.batch * cfg.c_out * pts * s + 2 * w


def measure_backward(cfg, dtype, steps, warmup):
    bw = Backward(cfg, dtype)
    try:
        ms = _time_loop(bw.step, steps, warmup, bw.stream)
        gbps = backward_minimal_bytes(cfg, dtype) / (ms * 1e-3) / 1e9
        return {"workload": cfg.name, "dtype": dtype, "ms_per_backward": ms,
                "backward_per_s": 1000.0 / ms, "minimal_bytes": backward_minimal_bytes(cfg, dtype),
                "gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS}
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
    calls and replays of a captured graph of one call."""
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
            out.append({"batch": B, "eager_us": eager, "graph_us": replay,
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

    def close(self):
        self.fno.fno_model2d_destroy(self.model)


def measure_model(steps, warmup):
    import workloads as wl
    cfg = wl.CONFIGS["c4"]
    m = Model(cfg)
    try:
        ms = _time_loop(m.step, steps, warmup, m.stream)
        res = {"workload": "FNO2d forward, B=20, 256x256, lift 3->64, 4 x (spectral conv 64->64 modes "
                           "24x24 + 1x1 conv + GELU), projection 64->128->1, fp16 storage",
               "ms_per_forward": ms, "samples_per_s": m.B / (ms * 1e-3)}
    finally:
        m.close()
    m1 = Model(cfg, batch=1)
    try:
        res["latency_b1_us"] = _latencies(m1.step, 100, 10, m1.stream)
    finally:
        m1.close()
    return res


def _time_loop(fn, steps, warmup, stream):
    import torch
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


def _per_call(fn, n, stream):
    """Per-call times in µs inside a back-to-back stream of calls: one event
    between consecutive calls, no synchronisation until the end."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for i in range(n):
        fn(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t = np.array([ev[i].elapsed_time(ev[i + 1]) * 1000.0 for i in range(n)])
    return {"mean": float(t.mean()), "std": float(t.std()), "min": float(t.min()),
            "p50": float(np.median(t)), "n": n}


def _kernel_times(lay, steps, warmup):
    """Average duration of each launch of the layer: `steps` back-to-back
    launches of that kernel alone (rotating buffer sets) between two HIP
    events recorded on the plan's stream."""
    return [_time_loop(lambda i, idx=idx: lay.launch(idx, i), steps, warmup, lay.stream)
            for idx in range(len(lay.names))]


def measure(cfg, dtype, steps, warmup, per_kernel=True):
    lay = Layer(cfg, dtype)
    try:
        ms = _time_loop(lay.step, steps, warmup, lay.stream)
        res = {"workload": cfg.name, "dtype": dtype, "ms_per_layer": ms,
               "layers_per_s": 1000.0 / ms,
               "gbps": cfg.minimal_bytes(dtype) / (ms * 1e-3) / 1e9}
        res["hbm_frac"] = res["gbps"] / HBM_PEAK_GBPS
        # distribution of single layers inside the rotating back-to-back loop
        res["per_layer_us"] = _per_call(lay.step, min(steps, 500), lay.stream)
        # one buffer set reused: x, w and y may then be served from the
        # Infinity Cache, so this is not the HBM-bound figure
        hot = _time_loop(lambda i: lay.step(0), steps, max(2, warmup // 4), lay.stream)
        res["hot_single_set_layers_per_s"] = 1000.0 / hot
        if per_kernel:
            bpl = _bytes_per_launch(cfg, dtype)
            kms = _kernel_times(lay, steps, max(2, warmup // 4))
            res["kernels"] = [{"kernel": name, "ms": t, "bytes": bpl[name], "gbps": bpl[name] / (t * 1e-3) / 1e9}
                              for name, t in zip(lay.names, kms)]
        return res
    finally:
        lay.close()


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
    m_s = re.search(r"^source:\s*(\S+)\s+sha256\s+([0-9a-f]{64})", text, re.M)
    if not (m_b and m_s):
        return None
    src = os.path.join(ROOT, m_s.group(1))
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != m_s.group(2):
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


def cpu_baseline(cfg, dtype, min_seconds=10.0):
    """The float64 oracle on this host's cores, repeated for ~min_seconds."""
    import oracle
    import workloads as wl
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))
    inp = wl.layer_inputs(cfg, dtype)
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
            if el >= min_seconds:
                break
    return {"value": n / el, "unit": "layers/s", "cores": int(used), "kind": "oracle",
            "sample": f"whole {cfg.name} {dtype} layer (B={cfg.batch}), {n} runs in {el:.1f} s "
                      f"after one warm-up, float64 numpy (BLAS: {blas}), host affinity {cores} cores"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 100 warm-up and 1000 timed launches per workload (the timed region
    # of the 128^2 layer is then ~30 ms, of the 256^2 layers ~0.16 s)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="c1")
    ap.add_argument("--dtype", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-latency", action="store_true")
    ap.add_argument("--no-model", action="store_true")
    ap.add_argument("--model-only", action="store_true", help="only time the full FNO2d forward (profiling runs)")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time the backward pass of --config/--dtype (profiling runs)")
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
    if args.model_only:
        print(json.dumps({"model": measure_model(args.steps, args.warmup)}))
        return
    if args.backward_only:
        print(json.dumps({"backward": [measure_backward(cfg, dtype, args.steps, args.warmup)]}))
        return
    main_res = measure(cfg, dtype, args.steps, args.warmup)
    dom = max(main_res["kernels"], key=lambda k: k["ms"])
    out = {
        "metric": METRIC, "value": main_res["layers_per_s"], "unit": "layers/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_layer"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if dtype == "f32" else f"{dtype} storage, f32 compute",
        "data": "synthetic (seeded Gaussian random fields; random weights)",
        "config": {"workload": cfg.description, "name": cfg.name, "batch": cfg.batch,
                   "c_in": cfg.c_in, "c_out": cfg.c_out, "grid": list(cfg.grid),
                   "modes": list(cfg.modes), "storage": dtype,
                   "minimal_bytes": cfg.minimal_bytes(dtype)},
        "gbps": main_res["gbps"], "hbm_frac": main_res["hbm_frac"],
        "roofline": {"bound": "hbm", "kernel": dom["kernel"], "achieved": dom["gbps"],
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": dom["gbps"] / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(dom["kernel"], cfg.name, dtype),
                     "bytes_per_launch": dom["bytes"], "ms_per_launch": dom["ms"]},
        "kernels": main_res["kernels"],
        "per_layer_us": main_res["per_layer_us"],
        "hot_single_set_layers_per_s": main_res["hot_single_set_layers_per_s"],
    }
    if not args.no_extra:
        extra = []
        for name, dt in (("c1", "f16"), ("c2", "f16"), ("c2", "bf16"), ("c3", "f32"), ("c0", "f32")):
            if name == cfg.name and dt == dtype:
                continue
            r = measure(wl.CONFIGS[name], dt, args.steps, args.warmup)
            extra.append(r)
            d = r["per_layer_us"]
            print(f"[bench] {name} {dt}: {r['layers_per_s']:.1f} layers/s, {r['gbps']:.0f} GB/s; "
                  f"per layer p50 {d['p50']:.1f} us (mean {d['mean']:.1f}, std {d['std']:.1f}, "
                  f"min {d['min']:.1f}); one buffer set {r['hot_single_set_layers_per_s']:.0f} layers/s",
                  file=sys.stderr, flush=True)
        out["configs"] = extra
    if not args.no_backward:
        bwd = []
        for name, dt in (("c1", "f32"), ("c2", "f16"), ("c3", "f32")):
            r = measure_backward(wl.CONFIGS[name], dt, max(20, args.steps // 2), max(5, args.warmup // 2))
            bwd.append(r)
            print(f"[bench] backward {name} {dt}: {r['backward_per_s']:.1f} /s, {r['gbps']:.0f} GB/s",
                  file=sys.stderr, flush=True)
        out["backward"] = bwd
    if not args.no_model:
        out["model"] = measure_model(max(10, args.steps // 10), max(3, args.warmup // 4))
        print(f"[bench] model: {out['model']['ms_per_forward']:.3f} ms per B=20 forward, "
              f"B=1 latency {out['model']['latency_b1_us']['mean']:.1f} us", file=sys.stderr, flush=True)
    if not args.no_latency:
        out["latency"] = latency_sweep()
        print("[bench] latency " + ", ".join(
            f"B={r['batch']}: eager {r['eager_us']['mean']:.1f}±{r['eager_us']['std']:.1f} us, "
            f"graph {r['graph_us']['mean']:.1f}±{r['graph_us']['std']:.1f} us"
            for r in out["latency"]["sweep"]), file=sys.stderr, flush=True)
    out["copy_1gib"] = copy_bandwidth(1 << 30)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, dtype)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
