"""Benchmark of one per-GPU K-FAC step on an MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one pass of the whole hot path over one batch of synthetic input:
A factors and G factors of every layer with their running average, pack and
unpack of all factors through the fused buffer, the damped inverse of every
factor, and the preconditioned gradient of every layer.  Inputs are seeded
synthetic tensors of the workload's shapes, resident in GPU memory before the
timed region.  Prints one JSON line.

Workloads (--config): 1 single FC layer, 2 four-layer MLP, 3 ResNet-50
shapes, 4 twelve-layer encoder with bf16 inputs, 5 large-factor stress
(16 layers, 25,088 rows, gamma = 1e-2; the default: the largest workload,
the one the headline figure is quoted on).
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

# MI355X published peaks
PEAK_FP64_MFMA = 78.6e12
PEAK_FP32_MFMA = 157.3e12   # the float32 matrix cores, for comparison with the split products
PEAK_BF16_MFMA = 2.5e15
# float32 operands run on the bf16 matrix cores as six bf16 products per
# float32 product (exact three-way splits of each value), so their products'
# ceiling is the bf16 peak over six
SPLIT_PRODUCTS = 6
PEAK_F32_SPLIT = PEAK_BF16_MFMA / SPLIT_PRODUCTS
# the inverse: potrf and V = U^-1 (two thirds of its d^3 flops) on the fp64
# matrix cores, the last product V V^T (one third) as float32 split products
PEAK_INVERSE = 1.0 / ((2.0 / 3.0) / PEAK_FP64_MFMA + (1.0 / 3.0) / PEAK_F32_SPLIT)
PEAK_HBM = 8.0e12


def algorithmic_work(cfg):
    """Algorithmic flops and bytes of one step (upper-triangle factor work,
    d^3 per inverse, 2 dg da (dg + da) per preconditioned layer)."""
    dims = [l.d_a for l in cfg.layers] + [l.d_g for l in cfg.layers]
    rows = [l.rows for l in cfg.layers] * 2
    f_factor = sum(r * d * (d + 1) for r, d in zip(rows, dims))
    f_inverse = sum(d ** 3 for d in dims)
    f_precond = sum(2 * l.d_g * l.d_a * (l.d_g + l.d_a) for l in cfg.layers)
    packed = sum(d * (d + 1) // 2 for d in dims)
    b_pack = 8 * packed
    b_unpack = 4 * (packed + sum(d * d for d in dims))
    return dict(factor=f_factor, inverse=f_inverse, precondition=f_precond,
                pack_bytes=b_pack, unpack_bytes=b_unpack, packed=packed)


def matrix_core_rates(dev, runs=3):
    """FLOP/s that kfac_matrix_rate's register-only product loops sustain on
    this part (bf16 32x32x16, fp64 16x16x4, fp32 32x32x2; about 25 ms per
    run, mean of `runs` after one warm-up): the measured counterpart of the
    published peaks, taken under the part's own clock and power limits."""
    import torch
    import linear_algebra_amd as la
    blocks = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(4 * blocks, device=dev)
    out = {}
    for name, kind, iters in (("bf16", la.KFAC_RATE_BF16, 200000), ("fp64", la.KFAC_RATE_F64, 100000),
                              ("fp32", la.KFAC_RATE_F32, 100000)):
        la.kfac_matrix_rate(kind, iters // 10, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        flops = 0.0
        e0.record()
        for _ in range(runs):
            flops += la.kfac_matrix_rate(kind, iters, sink)
        e1.record()
        torch.cuda.synchronize()
        out[name] = flops / (e0.elapsed_time(e1) * 1e-3)
    return out


def measured_ceiling(stage, cfg, rates):
    """A stage's ceiling from the measured matrix-core rates, in the same
    composition as its published ceiling."""
    split = rates["bf16"] / SPLIT_PRODUCTS
    if stage in ("factors_A", "factors_G"):
        return rates["bf16"] if cfg.in_dtype == "bf16" else split
    if stage == "inverse":
        return 1.0 / ((2.0 / 3.0) / rates["fp64"] + (1.0 / 3.0) / split)
    return split


def kernel_source_sha256():
    """Hash of the sources of the step's stage kernels, the key of stored
    counter data.  Comments and blank lines are left out, so that the key
    changes only with the code."""
    import glob
    import hashlib
    import re
    h = hashlib.sha256()
    # the files that hold no kernel of the step's stages: the matrix-core
    # reference loops and the layer row (im2col, gradient rows)
    skip = {"rates.hip", "layers.hip"}
    for p in sorted(glob.glob(os.path.join(ROOT, "linear_algebra_amd", "csrc", "*"))):
        if p.endswith((".hip", ".h", ".cpp")) and os.path.basename(p) not in skip:
            h.update(os.path.basename(p).encode())
            with open(p, encoding="utf-8") as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
            lines = [ln.rstrip() for ln in text.splitlines()]
            h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()


def measured_traffic(workload, stage):
    """HBM bytes per call (FETCH_SIZE + WRITE_SIZE, calibrated) of a stage,
    from profiles/hbm_traffic.json, or None when none was taken for this
    workload and stage or the kernels have changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    sha = kernel_source_sha256()
    for e in doc.get("entries", []):
        if e.get("workload") == workload and e.get("stage") == stage and e.get("kernel_source_sha256") == sha:
            return int(e["fetch_bytes"]) + int(e["write_bytes"])
    return None


def cpu_baseline(cfg, data, budget_s=25.0, min_s=10.0):
    """The fp64 oracle on the host cores, over a bounded sample of the step:
    whole layers (A and G factors, running average, pack/unpack, both
    inverses, the preconditioned gradient) are added in order, wrapping
    round to the first layer when a step is done early, until `min_s` is
    reached or the budget is spent; the rate is the sample's algorithmic
    flops over its time."""
    import numpy as np
    import oracle

    eps, gamma = np.float32(cfg.eps), np.float32(cfg.gammas[0])
    flops, spent, done = 0, 0.0, 0
    order = list(range(cfg.n_layers))
    while True:
        li = order[done % len(order)]
        layer = cfg.layers[li]
        a, g, grad = data[li]
        t0 = time.perf_counter()
        fa = oracle.factor(oracle.upcast(a, cfg.in_dtype))
        fg = oracle.factor(oracle.upcast(g, cfg.in_dtype))
        ma = oracle.running_average(None, fa, eps, True)
        mg = oracle.running_average(None, fg, eps, True)
        dims = [layer.d_a, layer.d_g]
        p = oracle.pack([ma.astype(np.float32), mg.astype(np.float32)], dims)
        oracle.unpack(p, dims)
        za, _ = oracle.damped_inverse(ma, gamma)
        zg, _ = oracle.damped_inverse(mg, gamma)
        oracle.precondition(zg, grad, za)
        spent += time.perf_counter() - t0
        done += 1
        for d in dims:
            flops += layer.rows * d * (d + 1) + d ** 3
        flops += 2 * layer.d_g * layer.d_a * (layer.d_g + layer.d_a)
        if spent >= min(min_s, budget_s):
            break
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": min(cores, threads),
        "kind": "oracle",
        "sample": f"{done} layer passes over the {cfg.n_layers} layers of one step (factors, running average, "
                  f"pack/unpack, both damped inverses, preconditioned gradient), fp64, {spent:.1f} s",
    }


def sweep_inverse(dims=(64, 128, 256, 512, 768, 1024, 1536, 2048, 3072, 4096, 6144, 8192), gamma=1e-3):
    """Inverse time of one damped factor against its dimension: the
    computation performance model of "Accelerating Distributed K-FAC with
    Smart Parallelism of Computing and Communication Tasks" (Eq. 26 and
    Fig. 8: d in [64, 8192], mean of 100 runs after 10 warm-ups; fewer runs
    above d = 2048 to keep the sweep short).  Inputs are factors
    (1/rows) a^T a of ReLU(N(0,1)) draws with rows = 2d.  Eq. 26 itself did
    not survive on the page; it is read as t = alpha exp(beta d), fitted by
    least squares on log t, and set against the cubic law t = a + b d^3."""
    import numpy as np
    import torch

    import linear_algebra_amd as la

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    rows_out = []
    for d in dims:
        x = torch.randn(2 * d, d, device=dev, generator=gen).clamp_(min=0.0)
        m = torch.zeros(d, d, device=dev)
        la.kfac_factors([x], [m], 0.0, True)
        z = torch.empty_like(m)
        info = torch.zeros(1, dtype=torch.int32, device=dev)
        runs = 100 if d <= 2048 else (30 if d <= 4096 else 10)
        for _ in range(10):
            la.kfac_damped_inverse([m], gamma, [z], info)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(runs):
            la.kfac_damped_inverse([m], gamma, [z], info)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / runs
        if int(info.item()) != 0:
            raise RuntimeError(f"inverse failed at d={d}")
        rows_out.append({"d": d, "ms": round(ms, 4), "runs": runs,
                         "tflops_alg": round(d ** 3 / (ms * 1e-3) / 1e12, 3)})
        print(f"sweep: d={d} {ms:.3f} ms", file=sys.stderr, flush=True)
        del x, m, z
    d = np.array([r["d"] for r in rows_out], dtype=np.float64)
    t = np.array([r["ms"] for r in rows_out], dtype=np.float64)
    # cubic: least squares on t = a + b d^3
    A = np.stack([np.ones_like(d), d ** 3], axis=1)
    (a3, b3), *_ = np.linalg.lstsq(A, t, rcond=None)
    # exponential: least squares on log t = log a + b d
    B = np.stack([np.ones_like(d), d], axis=1)
    (la_, be), *_ = np.linalg.lstsq(B, np.log(t), rcond=None)
    # chain + bulk: t = a d + b d^3 (a sequential pass over d/64 diagonal
    # blocks plus cubic block-product work), relative least squares
    C = np.stack([d / t, d ** 3 / t], axis=1)
    (ac, bc), *_ = np.linalg.lstsq(C, np.ones_like(t), rcond=None)

    def rel_rms(pred):
        return float(np.sqrt(np.mean(((pred - t) / t) ** 2)))
    return {
        "metric": "damped inverse time vs dimension (computation performance model)",
        "gamma": gamma, "points": rows_out,
        "fit_cubic": {"a_ms": float(a3), "b_ms_per_d3": float(b3), "rel_rms": rel_rms(a3 + b3 * d ** 3)},
        "fit_exponential": {"a_ms": float(np.exp(la_)), "b_per_d": float(be), "rel_rms": rel_rms(np.exp(la_ + be * d))},
        "fit_chain_cubic": {"a_ms_per_d": float(ac), "b_ms_per_d3": float(bc), "rel_rms": rel_rms(ac * d + bc * d ** 3)},
    }


def resnet50_conv_geometry(batch=32):
    """Input shape, kernel, stride and padding of each ResNet-50 convolution,
    read back from the factor workload's layer list (d_A = c_in k^2,
    rows = batch H_out W_out; stride 2 on the stem and on the 3x3 and
    shortcut convolutions of each down-sampling block)."""
    import math
    from workloads import CONFIGS
    out = []
    for l in CONFIGS[3].layers:
        if l.name == "fc":
            continue
        k = 7 if l.name == "conv1" else (3 if l.name.endswith("conv2") else 1)
        parts = l.name.split(".")
        s = 2 if l.name == "conv1" or (parts[0] in ("layer2", "layer3", "layer4") and parts[1] == "0"
                                       and parts[2] in ("conv2", "downsample")) else 1
        ho = int(round(math.sqrt(l.rows / batch)))
        out.append(dict(name=l.name, c_in=l.d_a // (k * k), c_out=l.d_g, h_in=ho * s, h_out=ho, k=k, s=s, p=k // 2,
                        rows=l.rows, d_a=l.d_a))
    return out


def bench_layers(steps=10, warmup=3):
    """Factor inputs of real layers: kfac_im2col over the 53 ResNet-50
    convolution inputs and kfac_grad_rows over their output gradients (batch
    32, one call each, HBM-bound: bytes = the input elements the patches
    touch, read once, + the output written once),
    and one KFACPreconditioner step on the four-layer MLP built from
    torch.nn.Linear layers (batch 128, inverses every step)."""
    import numpy as np
    import torch

    import linear_algebra_amd as la
    from linear_algebra_amd.kfac_preconditioner import KFACPreconditioner

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    geo = resnet50_conv_geometry()
    xs, shapes, outs, gys, gouts = [], [], [], [], []
    bytes_im2col = bytes_rows = 0
    for g in geo:
        x = torch.randn(32, g["c_in"], g["h_in"], g["h_in"], device=dev, generator=gen)
        sh = dict(kernel=(g["k"], g["k"]), stride=(g["s"], g["s"]), padding=(g["p"], g["p"]), dilation=(1, 1),
                  ones=False)
        assert la.conv_out_hw(g["h_in"], g["h_in"], g["k"], g["k"], sh["stride"], sh["padding"]) == (g["h_out"], g["h_out"])
        xs.append(x)
        shapes.append(sh)
        outs.append(torch.empty(g["rows"], g["d_a"], device=dev))
        gy = torch.randn(32, g["c_out"], g["h_out"], g["h_out"], device=dev, generator=gen)
        gys.append(gy)
        gouts.append(torch.empty(g["rows"], g["c_out"], device=dev))
        # input elements some patch reads (all of them, except the skipped
        # rows and columns of a 1x1 stride-2 shortcut), read once, + a written
        ref = len({y * g["s"] - g["p"] + i for y in range(g["h_out"]) for i in range(g["k"])} & set(range(g["h_in"])))
        bytes_im2col += 4 * (32 * g["c_in"] * ref * ref + g["rows"] * g["d_a"])
        bytes_rows += 8 * gy.numel()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_im2col = timed(lambda: la.kfac_im2col(xs, shapes, outs))
    ms_rows = timed(lambda: la.kfac_grad_rows(gys, 32.0, gouts))
    del xs, outs, gys, gouts
    torch.cuda.empty_cache()

    torch.manual_seed(1)
    model = torch.nn.Sequential(torch.nn.Linear(1024, 2048), torch.nn.ReLU(), torch.nn.Linear(2048, 2048),
                                torch.nn.ReLU(), torch.nn.Linear(2048, 1024), torch.nn.ReLU(),
                                torch.nn.Linear(1024, 10)).to(dev)
    pre = KFACPreconditioner(model, damping=1e-3, factor_decay=0.95, inv_update_freq=1)
    x = torch.randn(128, 1024, device=dev, generator=gen)
    y = torch.randint(0, 10, (128,), device=dev, generator=gen)
    torch.nn.functional.cross_entropy(model(x), y).backward()
    ms_pre = timed(pre.step)
    return {
        "metric": "factor inputs of real layers and one preconditioner step",
        "im2col": {"workload": "ResNet-50, 53 convolutions, batch 32, fp32", "ms": round(ms_im2col, 4),
                   "bytes": bytes_im2col, "achieved_GBps": round(bytes_im2col / ms_im2col / 1e6, 1),
                   "peak_GBps": PEAK_HBM / 1e9, "frac": round(bytes_im2col / (ms_im2col * 1e-3) / PEAK_HBM, 4)},
        "grad_rows": {"workload": "ResNet-50 output gradients, batch 32, fp32", "ms": round(ms_rows, 4),
                      "bytes": bytes_rows, "achieved_GBps": round(bytes_rows / ms_rows / 1e6, 1),
                      "frac": round(bytes_rows / (ms_rows * 1e-3) / PEAK_HBM, 4)},
        "preconditioner_step": {"workload": "MLP 1024-2048-2048-1024-10 as nn.Linear, batch 128, inverses every step",
                                "ms": round(ms_pre, 4)},
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=25.0)
    ap.add_argument("--layers", action="store_true",
                    help="time the layer factor inputs (im2col, gradient rows) and a preconditioner step")
    ap.add_argument("--sweep-inverse", action="store_true",
                    help="time kfac_damped_inverse on single matrices of d in [64, 8192] and fit time models")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for {args.gpus}); "
              "the multi-GPU exchange of the fused factor buffer is not part of it.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import linear_algebra_amd as la
    from workloads import CONFIGS, gen_layer_step

    la.load_library()
    if args.sweep_inverse:
        print(json.dumps(sweep_inverse()), flush=True)
        return 0
    if args.layers:
        print(json.dumps(bench_layers()), flush=True)
        return 0
    dev = torch.device("cuda:0")
    cfg = CONFIGS[args.config]
    L = cfg.layers
    n = len(L)
    eps, gamma = float(np.float32(cfg.eps)), float(np.float32(cfg.gammas[0]))

    print(f"bench: generating config {cfg.cid} ({cfg.name}) inputs", file=sys.stderr, flush=True)
    data = gen_layer_step(cfg, 0, threads=16)

    def dev_tensor(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    a_d = [dev_tensor(t[0]) for t in data]
    g_d = [dev_tensor(t[1]) for t in data]
    w_d = [dev_tensor(t[2]) for t in data]
    ma = [torch.zeros(l.d_a, l.d_a, device=dev) for l in L]
    mg = [torch.zeros(l.d_g, l.d_g, device=dev) for l in L]
    za = [torch.zeros(l.d_a, l.d_a, device=dev) for l in L]
    zg = [torch.zeros(l.d_g, l.d_g, device=dev) for l in L]
    out = [torch.zeros(l.d_g, l.d_a, device=dev) for l in L]
    facs = ma + mg[::-1]                      # A's forward, G's backward
    zs = za + zg[::-1]
    dims = [l.d_a for l in L] + [l.d_g for l in reversed(L)]
    packed = torch.zeros(la.kfac_packed_size(dims), device=dev)
    info = torch.zeros(len(facs), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    stages = ["factors_A", "factors_G", "pack", "unpack", "inverse", "precondition"]

    def step(first, ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        la.kfac_factors(a_d, ma, eps, first)
        mark(1)
        la.kfac_factors(g_d, mg, eps, first)
        mark(2)
        la.kfac_pack_sym(facs, packed, la.KFAC_PACK)
        mark(3)
        la.kfac_pack_sym(facs, packed, la.KFAC_UNPACK)
        mark(4)
        la.kfac_damped_inverse(facs, gamma, zs, info)
        mark(5)
        la.kfac_precondition(zg, w_d, za, out)
        mark(6)

    print(f"bench: warmup {args.warmup}", file=sys.stderr, flush=True)
    for w in range(args.warmup):
        step(w == 0)
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(args.warmup == 0 and s == 0, events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"bench: {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    stage_ms = {name: 0.0 for name in stages}
    for ev in events:
        for i, name in enumerate(stages):
            stage_ms[name] += ev[i].elapsed_time(ev[i + 1])
    stage_ms = {k: v / args.steps for k, v in stage_ms.items()}
    ms = wall * 1e3 / args.steps
    # spread of the step over the timed steps (HIP events around each step)
    per_step = np.array([ev[0].elapsed_time(ev[-1]) for ev in events])
    step_stats = {"median": round(float(np.median(per_step)), 4), "mean": round(float(per_step.mean()), 4),
                  "std": round(float(per_step.std()), 4), "min": round(float(per_step.min()), 4),
                  "max": round(float(per_step.max()), 4)}

    # the factor stages in their first-step form (M <- F: the running
    # average is not read), after the timed region
    fs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(5)]
    for ev in fs:
        ev[0].record()
        la.kfac_factors(a_d, ma, eps, True)
        ev[1].record()
        la.kfac_factors(g_d, mg, eps, True)
        ev[2].record()
    torch.cuda.synchronize()
    first_step = {"factors_A": round(sum(ev[0].elapsed_time(ev[1]) for ev in fs) / len(fs), 4),
                  "factors_G": round(sum(ev[1].elapsed_time(ev[2]) for ev in fs) / len(fs), 4)}

    # streaming reference for the HBM-bound stages: the library's plain copy
    # of a buffer as large as the fused one (same bytes as pack moves)
    # (whole 16-byte units of it)
    n4 = packed.numel() // 4 * 4
    copy_src, copy_dst = packed[:n4], torch.empty(n4, device=dev)
    for _ in range(3):
        la.kfac_stream_copy(copy_src, copy_dst)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(20):
        la.kfac_stream_copy(copy_src, copy_dst)
    c1.record()
    torch.cuda.synchronize()
    copy_rate = 2 * n4 * 4 / (c0.elapsed_time(c1) / 20 * 1e-3)
    del copy_src, copy_dst

    # measured reference for the matrix-core-bound stages: register-only
    # product loops of the library on every CU (two workgroups per CU)
    rates = matrix_core_rates(dev)

    bad = [i for i, v in enumerate(info.cpu().tolist()) if v != 0]
    finite = all(bool(torch.isfinite(o).all()) for o in out)
    if bad or not finite:
        print(f"bench: numerical failure (info nonzero at {bad}, finite outputs {finite})", file=sys.stderr)
        return 1

    work = algorithmic_work(cfg)
    flops = work["factor"] + work["inverse"] + work["precondition"]
    value = flops / (ms * 1e-3) / 1e12
    factor_peak = PEAK_BF16_MFMA if cfg.in_dtype == "bf16" else PEAK_F32_SPLIT
    split_basis = "bf16 MFMA 2.5 PFLOP/s / 6 bf16 products per float32 product"
    basis = {"factors_A": "bf16 MFMA" if cfg.in_dtype == "bf16" else split_basis,
             "factors_G": "bf16 MFMA" if cfg.in_dtype == "bf16" else split_basis,
             "pack": "HBM", "unpack": "HBM",
             "inverse": "fp64 MFMA 78.6 TFLOP/s for potrf and U^-1 (2/3 of the flops), " + split_basis + " for V V^T (1/3)",
             "precondition": split_basis}
    fa_flops = sum(l.rows * l.d_a * (l.d_a + 1) for l in L)
    fg_flops = sum(l.rows * l.d_g * (l.d_g + 1) for l in L)
    stage_rate = {
        "factors_A": ("mfma", fa_flops / (stage_ms["factors_A"] * 1e-3), factor_peak, "TFLOP/s"),
        "factors_G": ("mfma", fg_flops / (stage_ms["factors_G"] * 1e-3), factor_peak, "TFLOP/s"),
        "pack": ("hbm", work["pack_bytes"] / (stage_ms["pack"] * 1e-3), PEAK_HBM, "GB/s"),
        "unpack": ("hbm", work["unpack_bytes"] / (stage_ms["unpack"] * 1e-3), PEAK_HBM, "GB/s"),
        "inverse": ("mfma", work["inverse"] / (stage_ms["inverse"] * 1e-3), PEAK_INVERSE, "TFLOP/s"),
        "precondition": ("mfma", work["precondition"] / (stage_ms["precondition"] * 1e-3), PEAK_F32_SPLIT, "TFLOP/s"),
    }
    scale = {"TFLOP/s": 1e12, "GB/s": 1e9}
    stages_out = {}
    for k in stages:
        bound, rate, peak, unit = stage_rate[k]
        stages_out[k] = {"ms": round(stage_ms[k], 4), "achieved": round(rate / scale[unit], 3), "unit": unit,
                         "peak": round(peak / scale[unit], 1), "peak_basis": basis[k], "frac": round(rate / peak, 4),
                         "traffic": measured_traffic(cfg.name, k)}
        if bound == "hbm":
            stages_out[k]["frac_of_copy"] = round(rate / copy_rate, 4)
        if basis[k] == split_basis:
            stages_out[k]["rate_over_fp32_mfma_peak"] = round(rate / PEAK_FP32_MFMA, 4)
        if bound == "mfma":
            stages_out[k]["frac_of_measured_rate"] = round(rate / measured_ceiling(k, cfg, rates), 4)
    dom = max(stages, key=lambda k: stage_ms[k])
    bound, rate, peak, unit = stage_rate[dom]
    roofline = {"bound": bound, "stage": dom, "achieved": round(rate / scale[unit], 3),
                "peak": round(peak / scale[unit], 1), "peak_basis": basis[dom],
                "unit": unit, "frac": round(rate / peak, 4), "traffic": measured_traffic(cfg.name, dom)}

    result = {
        "metric": "K-FAC step ms (factors+inverse+precondition) & TFLOP/s vs MFMA peak, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms_events": step_stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16-in/f32-accumulate" if cfg.in_dtype == "bf16" else "f32") + " factors, f32 precondition, "
                 "f64 inverse (float32 products as six bf16 products of exact three-way splits)",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.note}", "layers": n, "factors": len(dims),
                   "gamma": gamma, "eps": eps, "flops_per_step": flops, "parallelism": "single GPU"},
        "roofline": roofline,
        "stages": stages_out,
        "first_step_factors_ms": first_step,
        "matrix_core_rate": {k: {"TFLOPs": round(v / 1e12, 1), "frac_of_peak": round(v / p, 4)}
                             for (k, v), p in zip(rates.items(), (PEAK_BF16_MFMA, PEAK_FP64_MFMA, PEAK_FP32_MFMA))},
        "stream_copy": {"GBps": round(copy_rate / 1e9, 1), "bytes": 2 * n4 * 4,
                        "frac_of_peak": round(copy_rate / PEAK_HBM, 4),
                        "note": "kfac_stream_copy of a buffer the size of the fused one: the achievable "
                                "streaming rate beside the 8 TB/s peak"},
    }
    if not args.no_cpu_baseline:
        print("bench: timing the oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, data, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
