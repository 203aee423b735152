#!/usr/bin/env python3
"""Throughput of convolution lowered to GEMM on one MI355X.

One step = the whole hot path over one batch of seeded synthetic input, for
every conv layer of the workload: forward (im2col -> GEMM NN with the
conv_reshape + bias epilogue), data gradient (by default the implicit GEMM
over dy, no dcol; --dgrad explicit: GEMM to dcol, col2im) and filter + bias
gradients (reshape dy, split-K GEMM NT on the saved col, reduction, bias
row sum).  Inputs are resident in HBM before timing starts.

Default workload: the AlexNet conv3-5 stack (batch 64, 256x13x13 -> 384 ->
384 -> 256 filters 3x3 pad 1) in fp32, the largest GEMM-dominated
configuration; ``--workload`` / ``--dtype`` select the others.

Printed: one JSON line.  ``value`` = algorithmic TFLOP/s of the step
(3 GEMMs x 2*O*Kc*N per layer, padding zeros included, divided by the step
time).  ``roofline`` describes the kernel with the largest share of the
step, timed with HIP events the library records on its own launch stream.
``cpu_baseline`` times the CPU oracle (direct convolution, float64) on a
bounded batch sample on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# AMD's published MI355X dense peaks (TFLOP/s) and HBM3E bandwidth (GB/s).
MFMA_PEAK = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}
HBM_PEAK_GBPS = 8000.0
METRIC = "conv fwd+bwd TFLOP/s and % of MFMA peak; im2col/col2im GB/s vs HBM peak"


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4",
                    help="c1..c5, or lenet / alexnet: one whole LeNet-5 / AlexNet training step "
                         "(conv, ReLU, pooling, linear layers, softmax-CE, SGD) at --batch")
    ap.add_argument("--batch", type=int, default=64, help="batch of the lenet / alexnet workload")
    ap.add_argument("--dtype", default=None, help="f32 | f16 | bf16 (default: workload's first)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--detail", default=None, help="write per-kernel detail JSON here")
    ap.add_argument("--forward", choices=("auto", "explicit", "implicit"), default="auto",
                    help="explicit: im2col + GEMM (col saved for the filter gradient); "
                         "implicit: implicit-GEMM forward, im2col redone in the filter gradient; "
                         "auto: implicit for the 1x1 layers (x read in place, no im2col) and for the "
                         "16-bit layers whose forward reads x as NHWC on the direct-to-LDS kernel, "
                         "explicit elsewhere")
    ap.add_argument("--dgrad", choices=("explicit", "implicit"), default="implicit",
                    help="implicit: implicit-GEMM data gradient, no dcol (stride-1 square-kernel "
                         "layers; others run explicit); explicit: the page's GEMM to dcol + col2im")
    ap.add_argument("--backward", choices=("combined", "separate"), default="combined",
                    help="combined: one d4r_conv_backward call per layer (dy prepared once for both "
                         "gradients where the layer allows); separate: the data-gradient call, then "
                         "the filter-gradient call (always with --streams 2 or --dgrad explicit)")
    ap.add_argument("--streams", type=int, choices=(1, 2), default=1,
                    help="2: the forwards and filter gradients on one stream, the data gradients "
                         "(own workspace) on a second one after the forwards, joined at the step's "
                         "end -- the two gradients of a layer only share dy, so they may overlap")
    ap.add_argument("--rotate", type=int, default=1,
                    help="cycle through this many independent copies of every input, output and "
                         "workspace, so that a step's operands are not left in the 256 MB MALL by "
                         "the previous step (cold-cache timing)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step as a HIP graph (stream capture) and time its replays; "
                         "per-kernel event timing is then unavailable")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before warmup (counter "
                         "calibration for rocprofv3 --pmc runs; untimed)")
    ap.add_argument("--no-configs", action="store_true",
                    help="headline only: skip the other GEMM-dominated configurations (AlexNet conv1 "
                         "fp32, conv3-5 bf16, the 46x80 feature-map convs f16) the default run reports")
    ap.add_argument("--gemm", default=None, metavar="M,K,N,FLAGS",
                    help="time one standalone d4r_gemm of this shape and transpose flags instead of "
                         "a convolution workload (seeded N(0,1) operands in --dtype)")
    return ap.parse_args()


def library_digest() -> str:
    """sha256 over every library source and the C header (file names and
    contents, in sorted order): any change to a kernel, the planner or the
    launch sequence changes it."""
    import glob
    import hashlib
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "gemm_scratch_nn_amd", "csrc", "*")) +
                   [os.path.join(ROOT, "include", "d4r_conv.h")])
    for path in files:
        h.update(os.path.relpath(path, ROOT).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summaries
    (profiles/traffic_*.txt), or None when none matches or the library
    (kernels, planner, launch sequence) changed since the counters were
    taken."""
    import glob
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.txt"))):
        fields = {}
        with open(path) as f:
            for line in f:
                if line.startswith("traffic_") and ":" in line:
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("traffic_kernel") != kernel:
            continue
        if fields.get("traffic_library_sha256") != library_digest():
            continue
        return float(fields["traffic_bytes_per_launch"]), os.path.relpath(path, ROOT)
    return None


def layer_flops(sh) -> float:
    return 3.0 * sh.gemm_flops()


def forward_label(t: dict) -> str:
    """How the step ran a layer's forward (the library's form for the implicit call)."""
    if not t["implicit"]:
        return "explicit (im2col + GEMM)"
    return {"nhwc": "implicit (NHWC)", "pointwise": "pointwise (1x1: x read in place)",
            "gathered": "implicit (gathered)"}.get(t["fwd_form"], "implicit")


def cpu_baseline(wl, dtype: str, target_s: float) -> dict:
    """The oracle as it stands, on a prefix of the batch, timed on this host."""
    import oracle
    import workloads as W

    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()

    def run(bs: int) -> float:
        total = 0.0
        for li, layer in enumerate(wl.layers):
            sh = layer.shape
            b = min(bs, sh.batch)
            ops = W.conv_inputs(wl, li, dtype, batch=b)
            x, w, g, bias = ops["x"].exact, ops["w"].exact, ops["g"].exact, ops["bias"].exact
            t0 = time.perf_counter()
            oracle.conv_forward(x, w, bias, sh.stride, sh.padding)
            oracle.conv_backward_data(g, w, x.shape, sh.stride, sh.padding)
            oracle.conv_backward_filter(x, g, w.shape, sh.stride, sh.padding)
            oracle.conv_backward_bias(g)
            total += time.perf_counter() - t0
        return total

    t1 = run(1)
    full = max(l.shape.batch for l in wl.layers)
    bs = int(max(1, min(full, target_s / max(t1, 1e-6))))
    t = t1 if bs == 1 else run(bs)
    flops = sum(layer_flops(l.shape.with_batch(min(bs, l.shape.batch))) for l in wl.layers)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{wl.key} {dtype}: all layers, forward + data/filter/bias gradients, "
                      f"first {bs} of {full} images (float64 direct loops); {t:.2f} s",
            "seconds": t}


def kernel_table(stats, peak_tf):
    """Per kernel symbol: launches, average time, share, TFLOP/s or GB/s."""
    by_kernel = {}
    for s in stats:
        k = s["name"].split(":")[0]
        a = by_kernel.setdefault(k, {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
        for f in ("launches", "ms", "flops", "bytes"):
            a[f] += s[f]
    total = max(1e-12, sum(v["ms"] for v in by_kernel.values()))
    kernels = {}
    for k, a in by_kernel.items():
        e = {"launches": a["launches"], "avg_us": 1e3 * a["ms"] / a["launches"], "share": a["ms"] / total}
        if a["flops"] > 0:
            e["TFLOPs"] = a["flops"] / (a["ms"] * 1e-3) / 1e12
            e["frac_mfma"] = e["TFLOPs"] / peak_tf
            # roofline of the launch class: min(peak, intensity * HBM bandwidth)
            e["attainable_TFLOPs"] = attainable_tf(a["flops"], a["bytes"], peak_tf)
            e["frac_attainable"] = e["TFLOPs"] / e["attainable_TFLOPs"]
        else:
            e["GBps"] = a["bytes"] / (a["ms"] * 1e-3) / 1e9
            e["frac_hbm"] = e["GBps"] / HBM_PEAK_GBPS
        kernels[k] = e
    return by_kernel, kernels


def roofline_of(by_kernel, dom, peak_tf):
    d = by_kernel[dom]
    if d["flops"] > 0:
        achieved = d["flops"] / (d["ms"] * 1e-3) / 1e12
        return {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": peak_tf, "unit": "TFLOP/s",
                "frac": achieved / peak_tf, "traffic": None,
                "avg_launch_us": 1e3 * d["ms"] / d["launches"], "launches": d["launches"]}
    achieved = d["bytes"] / (d["ms"] * 1e-3) / 1e9
    return {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
            "avg_launch_us": 1e3 * d["ms"] / d["launches"], "launches": d["launches"]}


def bench_lenet(args) -> int:
    """Whole LeNet-5 or AlexNet training steps (forward, backward, SGD) at --batch, fp32."""
    import torch

    import workloads as W

    B = args.batch
    alex = args.workload == "alexnet"
    if alex:
        from gemm_scratch_nn_amd.alexnet import AlexNetStep as Net
        lr, clip = 0.01, 0.002
        inp, params = W.alexnet_step_inputs(B, 0), W.ALEXNET_PARAMS
    else:
        from gemm_scratch_nn_amd.lenet import LeNetStep as Net
        lr, clip = 0.01, 0.05
        inp, params = W.lenet_step_inputs(B, 0), W.LENET_PARAMS
    net = Net(B)
    net.load({n: torch.from_numpy(inp[n]).cuda() for n, _ in params})
    x = torch.from_numpy(inp["x"]).cuda()
    lab = torch.from_numpy(inp["labels"]).cuda()

    def step():
        net.step(x, lab, lr, clip)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is None:
            step()
        else:
            graph.replay()
    t_enqueued = time.perf_counter()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    host_ms = (t_enqueued - t0) * 1e3 / args.steps
    import gemm_scratch_nn_amd as d4r
    d4r.d4r_profile_reset()
    d4r.d4r_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    d4r.d4r_profile_enable(False)
    by_kernel, kernels = kernel_table(d4r.d4r_profile_read(), MFMA_PEAK["f32"])
    dom = max(by_kernel, key=lambda k: by_kernel[k]["ms"])
    ms = elapsed * 1e3 / args.steps
    busy_ms = sum(v["ms"] for v in by_kernel.values()) / args.steps
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        if not os.path.exists(oracle.LIB_PATH):
            oracle.build()
        n, t = 0, 0.0
        if alex:
            # a bounded sample: the first two images of the batch
            sample = {k: (v[:2] if k in ("x", "labels") else v) for k, v in inp.items()}
            nb = 2
        else:
            sample, nb = inp, B
        step_fn = oracle.alexnet_step if alex else oracle.lenet_step
        while t < args.cpu_seconds and n < 1000:
            t1 = time.perf_counter()
            step_fn(sample, lr, clip)
            t += time.perf_counter() - t1
            n += 1
        cpu = {"value": n * nb / t, "unit": "images/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{n} whole {'AlexNet' if alex else 'LeNet-5'} steps at batch {nb} (float64); {t:.2f} s"}
    net_name = "AlexNet" if alex else "LeNet-5"
    desc = ("AlexNet 3x224x224: conv 11x11/4 3->96, pool 3/2, conv 5x5 96->256, pool, conv 3x3 256->384->"
            "384->256, pool, linear 9216->4096->4096->2" if alex else
            "LeNet-5 1x28x28: conv 5x5 1->6, pool 2, conv 5x5 6->16, pool 2, linear 256->120->84->10")
    line = {
        "metric": f"{net_name} training throughput (images/s): forward, backward and SGD update",
        "value": B / (ms * 1e-3),
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": ("synthetic (seeded U[0,1) images, Kaiming weights, uniform labels)" if alex else
                 "synthetic (seeded dyadic images and conv weights, Kaiming linear weights, uniform labels)"),
        "config": {"workload": f"{desc}, softmax-CE, SGD lr {lr} clip {clip}",
                   "batch": B, "hip_graph": bool(args.graph)},
        "kernel_busy_ms_per_step": busy_ms,
        "host_enqueue_ms_per_step": host_ms,
        "launches_per_step": sum(v["launches"] for v in by_kernel.values()) / args.steps,
        "roofline": roofline_of(by_kernel, dom, MFMA_PEAK["f32"]),
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_gemm(args) -> int:
    """One standalone d4r_gemm (C = op(A) op(B)) of the --gemm shape, timed like a step."""
    import numpy as np
    import torch

    import gemm_scratch_nn_amd as d4r
    import workloads as W

    M, K, N, flags = (int(v) for v in args.gemm.split(","))
    dtype = args.dtype or "bf16"
    code = {"f32": d4r.D4R_F32, "f16": d4r.D4R_F16, "bf16": d4r.D4R_BF16}[dtype]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    dev = torch.device("cuda:0")

    def operand(shape, tid):
        op = W.quantize(W.draw(("normal", 1.0), shape, (77, 0, tid)), dtype)
        if dtype == "f32":
            return torch.from_numpy(op.stored).to(dev)
        return torch.from_numpy(op.stored.view(np.int16)).to(dev).view(tdt)

    A = operand((K, M) if flags & 1 else (M, K), W.TID_A)
    B = operand((N, K) if flags & 2 else (K, N), W.TID_BM)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    wsb = d4r.d4r_gemm_workspace_size(M, K, N, flags, code)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)

    def step():
        d4r.d4r_gemm(M, K, N, flags, code, A, B, C, ws, wsb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    d4r.d4r_profile_reset()
    d4r.d4r_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    d4r.d4r_profile_enable(False)
    by_kernel, kernels = kernel_table(d4r.d4r_profile_read(), MFMA_PEAK[dtype])
    dom = max(by_kernel, key=lambda k: by_kernel[k]["ms"])
    ms = elapsed * 1e3 / args.steps
    flops = 2.0 * M * N * K
    value = flops / (ms * 1e-3) / 1e12
    line = {
        "metric": "standalone GEMM TFLOP/s and % of MFMA peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic (seeded N(0,1) operands)",
        "config": {"workload": f"GEMM M={M} K={K} N={N} flags={flags}", "M": M, "K": K, "N": N,
                   "flags": flags},
        "pct_mfma_peak": value / MFMA_PEAK[dtype],
        "roofline": roofline_of(by_kernel, dom, MFMA_PEAK[dtype]),
        "cpu_baseline": None,
        "kernels": kernels,
    }
    print(json.dumps(line), flush=True)
    return 0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# The GEMM-dominated configurations reported beside the headline (each
# convolution layer also separately): AlexNet conv1 (fp32), AlexNet conv3-5
# (bf16) and the 46x80 feature-map convolutions (f16).
SECONDARY = (("c3", "f32"), ("c4", "bf16"), ("c5", "f16"))


def bench_conv(args, key: str, dtype: str, steps: int, warmup: int, rotate: int, graph_mode: bool,
               streams: int, with_cpu: bool, per_layer: bool):
    """Times `steps` steps of one convolution workload; returns (line, stats)."""
    import numpy as np
    import torch

    import gemm_scratch_nn_amd as d4r
    import workloads as W

    wl = W.WORKLOADS[key]
    code = {"f32": d4r.D4R_F32, "f16": d4r.D4R_F16, "bf16": d4r.D4R_BF16}[dtype]
    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    peak = MFMA_PEAK[dtype]

    def to_dev(op):
        if op.dtype == "f32":
            return torch.from_numpy(op.stored).to(dev)
        return torch.from_numpy(op.stored.view(np.int16)).to(dev).view(tdt)

    def build_layers():
        out = []
        for li, layer in enumerate(wl.layers):
            sh = layer.shape
            ops = W.conv_inputs(wl, li, dtype)
            pl = d4r.ConvPlan(sh.batch, sh.inC, sh.inH, sh.inW, sh.kH, sh.kW, sh.stride, sh.padding,
                              sh.outC, code, device=dev)
            t = {k: to_dev(ops[k]) for k in ("x", "w", "g")}
            t["bias"] = torch.from_numpy(ops["bias"].stored).to(dev)
            t["y"] = torch.empty(sh.y_shape(), dtype=torch.float32, device=dev)
            t["dx"] = torch.empty(sh.x_shape(), dtype=torch.float32, device=dev)
            t["dw"] = torch.empty(sh.w_shape(), dtype=torch.float32, device=dev)
            t["db"] = torch.empty((sh.outC,), dtype=torch.float32, device=dev)
            t["fwd_form"] = d4r.d4r_conv_describe(pl.h)["fwd_implicit"]
            if args.forward == "auto":
                # 1x1 layers read x in place (no im2col anywhere in the step)
                t["implicit"] = t["fwd_form"] == "pointwise" or (dtype != "f32" and t["fwd_form"] == "nhwc")
            else:
                t["implicit"] = args.forward == "implicit"
            out.append((layer, pl, t))
        return out

    sets = [build_layers() for _ in range(rotate)]
    layers = sets[0]
    n_step = [0]
    stream = torch.cuda.current_stream().cuda_stream

    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    dgrad_fn = (d4r.d4r_conv_backward_data_implicit if args.dgrad == "implicit"
                else d4r.d4r_conv_backward_data)

    def forward(layer, pl, t, stream):
        if t["implicit"]:
            d4r.d4r_conv_forward_implicit(pl.h, t["x"], t["w"], t["bias"], t["y"], pl.ws, pl.ws_bytes, stream)
        else:
            d4r.d4r_conv_forward(pl.h, t["x"], t["w"], t["bias"], t["y"], pl.ws, pl.ws_bytes, stream)

    def wgrad(layer, pl, t, stream):
        # the implicit forward leaves no col: the filter gradient redoes im2col
        implicit = t["implicit"]
        d4r.d4r_conv_backward_filter(pl.h, t["x"] if implicit else None, t["g"], t["dw"], t["db"],
                                     0 if implicit else 1, pl.ws, pl.ws_bytes, stream)

    if streams == 2:
        aux = torch.cuda.Stream()  # default priority
        for st in sets:
            for _, pl, t in st:
                t["ws2"] = torch.empty(pl.ws_bytes, dtype=torch.uint8, device=dev)

    combined = args.backward == "combined" and args.dgrad == "implicit"

    def layer_step(layer, pl, t, stream):
        forward(layer, pl, t, stream)
        if combined:
            implicit = t["implicit"]
            d4r.d4r_conv_backward(pl.h, t["x"] if implicit else None, t["w"], t["g"], t["dx"], t["dw"],
                                  t["db"], 0 if implicit else 1, pl.ws, pl.ws_bytes, stream)
        else:
            dgrad_fn(pl.h, t["w"], t["g"], t["dx"], pl.ws, pl.ws_bytes, stream)
            wgrad(layer, pl, t, stream)

    def step(stream=stream, streams=streams):
        layers = sets[n_step[0] % len(sets)]
        n_step[0] += 1
        if streams == 1:
            for layer, pl, t in layers:
                layer_step(layer, pl, t, stream)
            return
        # forwards, then per layer (last first, as a backward pass runs) the
        # filter gradient on this stream and the data gradient on the other
        cur = torch.cuda.ExternalStream(stream) if isinstance(stream, int) else stream
        for layer, pl, t in layers:
            forward(layer, pl, t, stream)
        aux.wait_stream(cur)
        for layer, pl, t in reversed(layers):
            dgrad_fn(pl.h, t["w"], t["g"], t["dx"], t["ws2"], pl.ws_bytes, aux.cuda_stream)
            wgrad(layer, pl, t, stream)
        cur.wait_stream(aux)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    graph = None
    if graph_mode:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(torch.cuda.current_stream().cuda_stream)
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()

    # Timed region: K steps with no event recording (a recorded event pair per
    # launch adds GPU-side gaps between kernels).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        if graph is None:
            step()
        else:
            graph.replay()
    t_enqueued = time.perf_counter()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # host time to enqueue the K steps (launches or graph replays): when it
    # is close to the step time, the host, not the GPU, sets the pace
    host_ms = (t_enqueued - t0) * 1e3 / steps

    # Kernel timing: the same K steps again, eager and on one stream (so no
    # kernel shares the GPU with another), with the library's HIP event pair
    # around every launch on its stream.
    def profiled(fn, reps):
        d4r.d4r_profile_reset()
        d4r.d4r_profile_enable(True)
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        d4r.d4r_profile_enable(False)
        out = d4r.d4r_profile_read()
        d4r.d4r_profile_reset()
        return out

    stats = profiled(lambda: step(streams=1), steps)

    ms_per_step = elapsed * 1e3 / steps
    step_flops = sum(layer_flops(l.shape) for l, _, _ in layers)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    # per kernel symbol (the part before ':' is one template instantiation)
    by_kernel, kernels = kernel_table(stats, peak)
    dom = max(by_kernel, key=lambda k: by_kernel[k]["ms"])
    d = by_kernel[dom]
    roof = roofline_of(by_kernel, dom, peak)
    tr = recorded_traffic(dom)
    if tr is not None:
        roof["traffic"] = tr[0]
        roof["traffic_source"] = tr[1]
        roof["algorithmic_bytes_per_launch"] = d["bytes"] / d["launches"]

    def col2im_alone(layer, pl):
        """col2im timed through d4r_conv_col2im (the page's data gradient runs it;
        the default implicit data gradient does not)."""
        sh = layer.shape
        dcol = torch.zeros((sh.Kc, sh.N), dtype=torch.float32, device=dev)
        dx = torch.empty(sh.x_shape(), dtype=torch.float32, device=dev)
        for _ in range(2):
            d4r.d4r_conv_col2im(pl.h, dcol, dx)
        st = profiled(lambda: d4r.d4r_conv_col2im(pl.h, dcol, dx), max(5, steps // 2))
        del dcol, dx
        return stage_of(kernel_table(st, peak)[0], "col2im")

    col2im_standalone = {}
    per = []
    if per_layer:
        for layer, pl, t in layers:
            sh = layer.shape
            for _ in range(2):
                layer_step(layer, pl, t, stream)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for _ in range(steps):
                layer_step(layer, pl, t, stream)
            torch.cuda.synchronize()
            lms = (time.perf_counter() - t1) * 1e3 / steps
            lst = profiled(lambda: layer_step(layer, pl, t, stream), steps)
            lbk, _ = kernel_table(lst, peak)
            ltf = layer_flops(sh) / (lms * 1e-3) / 1e12
            entry = {"layer": layer.name,
                     "shape": f"{sh.batch}x{sh.inC}x{sh.inH}x{sh.inW} -> {sh.outC} {sh.kH}x{sh.kW} "
                              f"s{sh.stride} p{sh.padding}",
                     "ms": lms, "TFLOPs": ltf, "frac_mfma": ltf / peak,
                     "forward": forward_label(t)}
            entry.update(gemm_summary(lbk, peak))
            entry["im2col"] = stage_of(lbk, "im2col")
            c2 = stage_of(lbk, "col2im")
            if c2 is None:
                c2 = col2im_alone(layer, pl)
                if c2 is not None:
                    c2["timed"] = "standalone d4r_conv_col2im (the step's data gradient has no col2im)"
            entry["col2im"] = c2
            per.append(entry)
    else:
        c2 = stage_of(by_kernel, "col2im")
        if c2 is None:
            parts = [col2im_alone(layer, pl) for layer, pl, _ in layers]
            parts = [p for p in parts if p]
            if parts:
                col2im_standalone = {"GBps": sum(p["GBps"] for p in parts) / len(parts),
                                     "timed": "standalone d4r_conv_col2im per layer (mean)"}

    cpu = None
    if with_cpu:
        cpu = cpu_baseline(wl, dtype, args.cpu_seconds)
        cpu.pop("seconds", None)
        cpu["cpu_model"] = cpu_model()

    desc = "; ".join(f"{l.name} {l.shape.inC}x{l.shape.inH}x{l.shape.inW}->{l.shape.outC} "
                     f"{l.shape.kH}x{l.shape.kW} s{l.shape.stride} p{l.shape.padding}"
                     for l in wl.layers)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; shapes and distributions of the pages' workloads)",
        "config": {"workload": f"{wl.title}: {desc}", "batch": wl.layers[0].shape.batch,
                   "dtype": dtype, "forward": args.forward,
                   "implicit_forward_layers": [l.name for l, _, t in layers if t["implicit"]],
                   "dgrad": args.dgrad,
                   "backward": "combined" if combined and streams == 1 else "separate",
                   "streams": streams,
                   "rotate": rotate, "hip_graph": bool(graph_mode),
                   "step_gflop": step_flops / 1e9},
        "pct_mfma_peak": value / peak,
        "host_enqueue_ms_per_step": host_ms,
    }
    line.update(gemm_summary(by_kernel, peak))
    line["im2col"] = stage_of(by_kernel, "im2col")
    line["col2im"] = stage_of(by_kernel, "col2im") or (col2im_standalone or None)
    line["roofline"] = roof
    if per:
        line["layers"] = per
    line["kernel_timing"] = ("HIP event pair per launch, recorded by the library on its launch stream "
                             "during a second, single-stream pass of the same steps (step time from an "
                             "event-free pass)")
    line["cpu_baseline"] = cpu
    line["kernels"] = kernels
    return line, stats


def stage_of(by_kernel, prefix):
    sel = [v for k, v in by_kernel.items() if k.startswith(prefix)]
    if not sel:
        return None
    ms = sum(v["ms"] for v in sel)
    gbps = sum(v["bytes"] for v in sel) / (ms * 1e-3) / 1e9
    return {"GBps": gbps, "frac_hbm": gbps / HBM_PEAK_GBPS}


def gemm_summary(by_kernel, peak):
    """The GEMMs of a step together: TFLOP/s, fraction of the MFMA peak and of
    the attainable rate min(peak, I * HBM bandwidth), I = algorithmic flops per
    algorithmic byte of each launch class (time-weighted)."""
    g = {k: v for k, v in by_kernel.items() if k.startswith("gemm") and v["flops"] > 0}
    if not g:
        return {}
    ms = sum(v["ms"] for v in g.values())
    tf = sum(v["flops"] for v in g.values()) / (ms * 1e-3) / 1e12
    # time at the attainable rate of each class, summed
    t_att = sum(v["flops"] / (attainable_tf(v["flops"], v["bytes"], peak) * 1e12) for v in g.values())
    return {"gemm_TFLOPs": tf, "gemm_frac_mfma": tf / peak,
            "gemm_frac_attainable": (t_att * 1e3) / ms}


def attainable_tf(flops, bytes_, peak):
    if bytes_ <= 0:
        return peak
    return min(peak, flops / bytes_ * HBM_PEAK_GBPS / 1e3)


def hbm_reference(reps: int = 10) -> dict:
    """The attainable HBM rates of the library's own streaming kernels on 1 GiB
    buffers: d4r_stream_copy (read + write) and d4r_stream_fill (write)."""
    import torch

    import gemm_scratch_nn_amd as d4r
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    d4r.d4r_stream_fill(src, 0x3F800000, n)
    out = {"bytes": n, "kernels": "d4r_stream_copy (read + write), d4r_stream_fill (write only)"}
    for name, fn in (("copy", lambda: d4r.d4r_stream_copy(dst, src, n)),
                     ("fill", lambda: d4r.d4r_stream_fill(dst, 0, n))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        d4r.d4r_profile_reset()
        d4r.d4r_profile_enable(True)
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        d4r.d4r_profile_enable(False)
        st = d4r.d4r_profile_read()
        d4r.d4r_profile_reset()
        ms = sum(r["ms"] for r in st)
        out[f"{name}_GBps"] = sum(r["bytes"] for r in st) / (ms * 1e-3) / 1e9
    del src, dst
    return out


def mfma_reference(reps: int = 5) -> dict:
    """The MFMA rate of the library's ceiling kernel (d4r_mfma_ceiling: MFMAs
    on register-resident random operands, no loads) for each dtype, in
    TFLOP/s: what the GPU sustains at the clock it holds under a full MFMA
    load, the reference beside the GEMM rates (the roofline keeps the
    published peak).  Each launch runs several milliseconds, after two
    warm-up launches: shorter ones (1-2 ms) read 10-15% low for fp32, the
    clock still ramping."""
    import torch

    import gemm_scratch_nn_amd as d4r
    g = torch.Generator(device="cpu").manual_seed(7)
    out = {"kernel": "d4r_mfma_ceiling: 1024 workgroups x 8 wavefronts, 4 x 2 accumulators of 32 x 32 each, "
                     "random operands (N(0,1)) read once"}
    blocks = 1024
    for dt, code, tdt, per_lane, iters in (("f32", d4r.D4R_F32, torch.float32, 1, 4000),
                                           ("bf16", d4r.D4R_BF16, torch.bfloat16, 8, 6000),
                                           ("f16", d4r.D4R_F16, torch.float16, 8, 6000)):
        src = torch.randn(6 * 64 * per_lane, generator=g).to(tdt).cuda()
        res = torch.empty(blocks * 8, dtype=torch.float32, device="cuda")
        for _ in range(2):
            d4r.d4r_mfma_ceiling(code, src, res, blocks, iters)
        torch.cuda.synchronize()
        d4r.d4r_profile_reset()
        d4r.d4r_profile_enable(True)
        for _ in range(reps):
            d4r.d4r_mfma_ceiling(code, src, res, blocks, iters)
        torch.cuda.synchronize()
        d4r.d4r_profile_enable(False)
        st = d4r.d4r_profile_read()
        d4r.d4r_profile_reset()
        ms = sum(r["ms"] for r in st)
        out[f"{dt}_TFLOPs"] = sum(r["flops"] for r in st) / (ms * 1e-3) / 1e12
        out[f"{dt}_frac_of_peak"] = out[f"{dt}_TFLOPs"] / MFMA_PEAK[dt]
    return out


def main() -> int:
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build runs on one GPU; "
              "multi-GPU batch sharding is a design note only", file=sys.stderr)
        return 2

    if args.gemm:
        return bench_gemm(args)
    if args.workload in ("lenet", "alexnet"):
        return bench_lenet(args)
    if args.rotate < 1 or (args.rotate > 1 and args.graph):
        print("bench.py: --rotate must be >= 1 and cannot be combined with --graph", file=sys.stderr)
        return 2

    import workloads as W
    wl = W.WORKLOADS[args.workload]
    dtype = args.dtype or wl.dtypes[0]
    line, stats = bench_conv(args, args.workload, dtype, args.steps, args.warmup, args.rotate, args.graph,
                             args.streams, not args.no_cpu_baseline, per_layer=True)
    if not args.no_configs and args.workload == "c4" and dtype == "f32" and not args.graph and args.rotate == 1:
        # cold caches: three independent copies of every buffer in rotation,
        # so a step's operands come from HBM, not from the 256 MB MALL
        cl, _ = bench_conv(args, "c4", "f32", max(5, min(args.steps, 20)), min(args.warmup, 3), 3, False, 1,
                           False, per_layer=False)
        line["cold"] = {"rotate": 3, "ms_per_step": cl["ms_per_step"], "value": cl["value"],
                        "pct_mfma_peak": cl["pct_mfma_peak"], "im2col": cl["im2col"]}
        ref = hbm_reference()
        line["hbm_reference"] = ref
        mref = mfma_reference()
        line["mfma_reference"] = mref
        line["gemm_frac_of_mfma_ceiling"] = line["gemm_TFLOPs"] / mref[f"{dtype}_TFLOPs"]

        def rel(stage):
            if stage and "GBps" in stage:
                stage["frac_of_stream_copy"] = stage["GBps"] / ref["copy_GBps"]
                stage["frac_of_stream_fill"] = stage["GBps"] / ref["fill_GBps"]
        rel(line["im2col"])
        rel(line["col2im"])
        for l in line.get("layers", []):
            rel(l["im2col"])
            rel(l["col2im"])
    if not args.no_configs and args.workload == "c4" and dtype == "f32":
        # the other GEMM-dominated configurations, each with its layers
        sec_steps = max(5, min(args.steps, 20))
        configs = []
        for key, dt in SECONDARY:
            sl, _ = bench_conv(args, key, dt, sec_steps, min(args.warmup, 3), 1, False, 1, False,
                               per_layer=True)
            keep = ("value", "unit", "ms_per_step", "dtype", "pct_mfma_peak", "gemm_TFLOPs",
                    "gemm_frac_mfma", "gemm_frac_attainable", "im2col", "col2im", "layers", "roofline")
            entry = {"workload": sl["config"]["workload"], "steps": sec_steps}
            entry.update({k: sl[k] for k in keep if k in sl})
            mref = line.get("mfma_reference")
            if mref and entry.get("gemm_TFLOPs"):
                entry["gemm_frac_of_mfma_ceiling"] = entry["gemm_TFLOPs"] / mref[f"{dt}_TFLOPs"]
            ref = line.get("hbm_reference")
            if ref:
                for st in [entry.get("im2col"), entry.get("col2im")] + \
                          [x for l in entry.get("layers", []) for x in (l["im2col"], l["col2im"])]:
                    if st and "GBps" in st:
                        st["frac_of_stream_copy"] = st["GBps"] / ref["copy_GBps"]
                        st["frac_of_stream_fill"] = st["GBps"] / ref["fill_GBps"]
            configs.append(entry)
        line["configs"] = configs
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump({"line": line, "stats": stats}, f, indent=1)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
