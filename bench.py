#!/usr/bin/env python3
"""Benchmark of the 2-D convolution forward on one MI355X.

A step is one forward pass of the headline workload: the ResNet-style
bottleneck 3x3 layer, fp16 operands with fp32 accumulation, N=32, 256->256
channels, 14x14, stride 1, pad 1, bias + residual + ReLU, with every operand
resident in HBM before the timed region starts.  The operand sets rotate over
>= 1 GiB of device memory so that no call finds its inputs in the 256 MB
Infinity Cache.  Every other workload layer is timed the same way and reported
in "layers" (TFLOP/s, GB/s of algorithmic bytes, fraction of its roofline).

Each layer's figure is the median of --loops event-timed loops of --steps
back-to-back calls.  The fp64 oracle is timed on the host cores beside it, per
layer (cpu_baseline, and layers[].oracle), and per-config sums of both are
reported in "configs".

Prints one JSON line.  Options: --gpus N (only 1 is supported: the build runs on
one GPU), --steps K, --warmup W, --loops L, --no-cpu-baseline, --oracle-budget S,
--layers a,b,..., --headline-only, --copy-calib BYTES (runs only a plain device
copy of that size, for calibrating the HBM byte counters).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HEADLINE = "w2_bottleneck3x3_f16"
METRIC = "conv fwd TFLOP/s (2*MACs/s) and HBM GB/s per layer config, % of roofline"
PEAK = {  # MI355X published peaks
    "f16_mfma_tflops": 2500.0,
    "f32_tflops": 157.3,
    "hbm_gbs": 8000.0,
    "i8_mfma_tops": 5000.0,
}
ROTATE_BYTES = 1 << 30


def esize(dt):
    return 4 if dt == "f32" else 2


def layer_stats(layer):
    """MACs (as 'Convolutions' section 2.3 counts them; ConvT: x*w products)
    and algorithmic bytes (x, w, bias, residual and y once each)."""
    N, C, H, W = layer.out_shape
    if layer.transpose:
        macs = layer.n * layer.c_in * layer.h * layer.w * (layer.c_out // layer.groups) * \
            layer.kh * layer.kw
    else:
        macs = N * layer.c_out * H * W * (layer.c_in // layer.groups) * layer.kh * layer.kw
    es = esize(layer.dtype)
    nbytes = (math.prod(layer.x_shape) + math.prod(layer.w_shape) + N * C * H * W) * es
    if layer.bias:
        nbytes += layer.c_out * es
    if layer.residual:
        nbytes += N * C * H * W * es
    return macs, nbytes


def roof(layer, macs, nbytes):
    """Binding roof: min(compute peak, AI * HBM peak)."""
    flops = 2 * macs
    # bf16 and fp16 dense MFMA share the 2.5 PFLOP/s peak
    peak_c = PEAK["f32_tflops"] if layer.dtype == "f32" else PEAK["f16_mfma_tflops"]
    t_c = flops / (peak_c * 1e12)
    t_m = nbytes / (PEAK["hbm_gbs"] * 1e9)
    if layer.groups == layer.c_in and layer.groups > 1 and not layer.transpose:
        bound = "hbm"  # depthwise runs on the VALU without MFMA; bandwidth binds
        t_c = 0.0
    else:
        bound = "mfma" if t_c >= t_m else "hbm"
    return bound, max(t_c, t_m)


def build_problem(cf, layer):
    return cf.make_problem(layer.n, layer.c_in, layer.h, layer.w, layer.c_out, layer.kh,
                           layer.kw, groups=layer.groups, stride=layer.stride,
                           dilation=layer.dilation, pads=layer.pads, out_pad=layer.out_pad,
                           transpose=layer.transpose, act=layer.act, bias=layer.bias,
                           residual=layer.residual, variant=layer.variant)


def time_layer(cf, torch, layer, steps, warmup, loops):
    """Event-timed loops of `steps` back-to-back calls on one stream; the
    figure is the median loop.  Operand sets rotate over >= 1 GiB and the
    rotation index runs on across the warmup, host-timing and device loops, so
    a set is reused only after every other set (over 1 GiB of other operands)
    has been touched: no call finds its inputs in the 256 MB Infinity Cache."""
    p = build_problem(cf, layer)
    variant = cf.conv_describe_variant(p, layer.dtype)
    inp = workloads.make_inputs(layer)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[layer.dtype]
    # bfloat16 inputs are bfloat16-exact float32 values: the conversion is exact
    dev = lambda a: None if a is None else \
        torch.from_numpy(np.ascontiguousarray(a)).cuda().to(tdt)
    base = [dev(inp.x), dev(inp.w), dev(inp.b), dev(inp.r)]
    ydt = tdt
    macs, nbytes = layer_stats(layer)
    nsets = max(1, min(256, math.ceil(ROTATE_BYTES / nbytes)))
    sets = []
    for i in range(nsets):
        cl = [None if t is None else (t if i == 0 else t.clone()) for t in base]
        y = torch.empty(layer.out_shape, dtype=ydt, device="cuda")
        sets.append(cl + [y])
    whole, _ = cf.conv_scratch_size(p, layer.dtype)
    scratch = torch.empty(max(whole // 4, 4), dtype=torch.float32, device="cuda") if whole else None
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    fn = cf.lib().conv_transpose_forward if layer.transpose else cf.lib().conv_forward
    pref = ctypes.byref(p)
    dt = cf.DTYPES[layer.dtype]
    sp = None if scratch is None else scratch.data_ptr()
    args = [[None if t is None else t.data_ptr() for t in st] for st in sets]
    counter = [0]

    def call():
        x, w, b, r, y = args[counter[0] % nsets]
        counter[0] += 1
        st = fn(pref, dt, x, w, b, r, y, sp, whole, sh)
        if st:
            raise cf.ConvError(st, "conv_forward")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    # Host submission (ctypes + validation + launch) is timed on its own; for
    # the device timing a GPU-side delay first holds the stream while all K
    # calls are enqueued, so the events measure the kernels back to back, not
    # the host's launch rate.
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    host_us = (time.perf_counter() - t0) / steps * 1e6
    torch.cuda.synchronize()
    loop_s = []
    wall = 0.0
    for _ in range(loops):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(sleep_cycles(torch, host_us * steps * 1.5 + 2000.0))
        ev0.record(stream)
        t0 = time.perf_counter()
        for _ in range(steps):
            call()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall += time.perf_counter() - t0
        loop_s.append(ev0.elapsed_time(ev1) * 1e-3)
    del sets
    torch.cuda.empty_cache()
    bound, t_roof = roof(layer, macs, nbytes)
    total = float(np.median(loop_s))
    avg = total / steps
    return {
        "name": layer.name, "variant": variant, "dtype": layer.dtype,
        "rotating_sets": nsets, "rotation_bytes": nsets * nbytes,
        "us_avg": avg * 1e6, "us_loops": [round(t / steps * 1e6, 3) for t in loop_s],
        "host_us_per_call": host_us, "wall_s": wall,
        "tflops": 2 * macs / avg / 1e12, "gbs": nbytes / avg / 1e9,
        "macs": macs, "alg_bytes": nbytes, "bound": bound,
        "roof_us": t_roof * 1e6, "roof_frac": t_roof / avg, "total_s": total,
    }


def time_pool(cf, torch, layer, steps, warmup, loops):
    """The pooling layers, timed like the convolutions (rotating operand sets,
    median of event-timed loops); bound by HBM: bytes = x + y once each."""
    p = cf.make_pool_problem(layer.n, layer.c, layer.h, layer.w, layer.kind,
                             kernel=layer.kernel, stride=layer.stride, dilation=layer.dilation,
                             pads=layer.pads, ceil_mode=layer.ceil_mode,
                             count_include_pad=layer.count_include_pad)
    variant = cf.pool_describe_variant(p, layer.dtype)
    ho, wo = cf.pool_output_extent(p)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[layer.dtype]
    x0 = torch.from_numpy(np.ascontiguousarray(workloads.make_pool_input(layer))).cuda().to(tdt)
    es = esize(layer.dtype)
    nbytes = (x0.numel() + layer.n * layer.c * ho * wo) * es
    nsets = max(1, min(256, math.ceil(ROTATE_BYTES / nbytes)))
    sets = [(x0 if i == 0 else x0.clone(),
             torch.empty((layer.n, layer.c, ho, wo), dtype=tdt, device="cuda"))
            for i in range(nsets)]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    fn = cf.lib().pool_forward
    pref = ctypes.byref(p)
    dt = cf.DTYPES[layer.dtype]
    args = [(x.data_ptr(), y.data_ptr()) for x, y in sets]
    counter = [0]

    def call():
        x, y = args[counter[0] % nsets]
        counter[0] += 1
        st = fn(pref, dt, x, y, sh)
        if st:
            raise cf.ConvError(st, "pool_forward")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    host_us = (time.perf_counter() - t0) / steps * 1e6
    torch.cuda.synchronize()
    loop_s = []
    for _ in range(loops):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(sleep_cycles(torch, host_us * steps * 1.5 + 2000.0))
        ev0.record(stream)
        for _ in range(steps):
            call()
        ev1.record(stream)
        torch.cuda.synchronize()
        loop_s.append(ev0.elapsed_time(ev1) * 1e-3)
    del sets
    torch.cuda.empty_cache()
    avg = float(np.median(loop_s)) / steps
    roof_s = nbytes / (PEAK["hbm_gbs"] * 1e9)
    return {"name": layer.name, "variant": variant, "dtype": layer.dtype, "rotating_sets": nsets,
            "us_avg": avg * 1e6, "us_loops": [round(t / steps * 1e6, 3) for t in loop_s],
            "gbs": nbytes / avg / 1e9, "alg_bytes": nbytes, "bound": "hbm",
            "roof_us": roof_s * 1e6, "roof_frac": roof_s / avg}


def time_int(cf, torch, layer, steps, warmup, loops):
    """The quantized layers (ConvInteger): int8 operands, int32 output; bound by
    the int8 MFMA peak or HBM (bytes = x + w + y once each)."""
    p = cf.make_problem(layer.n, layer.c_in, layer.h, layer.w, layer.c_out, layer.kh, layer.kw,
                        groups=layer.groups, stride=layer.stride, dilation=layer.dilation,
                        pads=layer.pads)
    variant = cf.conv_integer_describe_variant(p, layer.x_type, layer.w_type)
    x, w, xz, wz = workloads.make_int_inputs(layer)
    npt = {"u8": np.uint8, "i8": np.int8}
    x0 = torch.from_numpy(np.ascontiguousarray(x.astype(npt[layer.x_type]).view(np.uint8))).cuda()
    w0 = torch.from_numpy(np.ascontiguousarray(w.astype(npt[layer.w_type]).view(np.uint8))).cuda()
    xzd = torch.from_numpy(np.array([xz]).astype(npt[layer.x_type]).view(np.uint8)).cuda()
    wzd = torch.from_numpy(wz.astype(npt[layer.w_type]).view(np.uint8)).cuda()
    N, C, H, W = layer.out_shape
    macs = N * C * H * W * (layer.c_in // layer.groups) * layer.kh * layer.kw
    nbytes = x0.numel() + w0.numel() + N * C * H * W * 4
    nsets = max(1, min(256, math.ceil(ROTATE_BYTES / nbytes)))
    sets = [(x0 if i == 0 else x0.clone(), w0 if i == 0 else w0.clone(),
             torch.empty(layer.out_shape, dtype=torch.int32, device="cuda")) for i in range(nsets)]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    fn = cf.lib().conv_integer_forward
    pref = ctypes.byref(p)
    xt, wt = cf.CONVI_TYPES[layer.x_type], cf.CONVI_TYPES[layer.w_type]
    args = [(a.data_ptr(), b.data_ptr(), c.data_ptr()) for a, b, c in sets]
    counter = [0]

    def call():
        xa, wa, ya = args[counter[0] % nsets]
        counter[0] += 1
        st = fn(pref, xt, wt, xa, wa, xzd.data_ptr(), wzd.data_ptr(), 1, ya, sh)
        if st:
            raise cf.ConvError(st, "conv_integer_forward")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    host_us = (time.perf_counter() - t0) / steps * 1e6
    torch.cuda.synchronize()
    loop_s = []
    for _ in range(loops):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(sleep_cycles(torch, host_us * steps * 1.5 + 2000.0))
        ev0.record(stream)
        for _ in range(steps):
            call()
        ev1.record(stream)
        torch.cuda.synchronize()
        loop_s.append(ev0.elapsed_time(ev1) * 1e-3)
    del sets
    torch.cuda.empty_cache()
    avg = float(np.median(loop_s)) / steps
    t_c = 2 * macs / (PEAK["i8_mfma_tops"] * 1e12)
    t_m = nbytes / (PEAK["hbm_gbs"] * 1e9)
    return {"name": layer.name, "variant": variant, "dtype": f"{layer.x_type}{layer.w_type}->i32",
            "rotating_sets": nsets, "us_avg": avg * 1e6,
            "us_loops": [round(t / steps * 1e6, 3) for t in loop_s],
            "tops": 2 * macs / avg / 1e12, "gbs": nbytes / avg / 1e9, "macs": macs,
            "alg_bytes": nbytes, "bound": "mfma" if t_c >= t_m else "hbm",
            "roof_us": max(t_c, t_m) * 1e6, "roof_frac": max(t_c, t_m) / avg}


def oracle_int(layer, budget_s):
    import oracle

    x, w, xz, wz = workloads.make_int_inputs(layer)
    g = oracle.Geom(layer.n, layer.c_in, layer.h, layer.w, layer.c_out, layer.kh, layer.kw,
                    groups=layer.groups, sh=layer.stride[0], sw=layer.stride[1],
                    dh=layer.dilation[0], dw=layer.dilation[1], pt=layer.pads[0],
                    pl=layer.pads[1], pb=layer.pads[2], pr=layer.pads[3])
    runs, spent = 0, 0.0
    while runs == 0 or (spent < budget_s and runs < 50):
        t0 = time.perf_counter()
        oracle.conv_integer(g, x, w, xz, wz)
        spent += time.perf_counter() - t0
        runs += 1
    N, C, H, W = layer.out_shape
    macs = N * C * H * W * (layer.c_in // layer.groups) * layer.kh * layer.kw
    return {"s_per_run": spent / runs, "runs": runs, "gops": 2 * macs * runs / spent / 1e9}


def oracle_pool(layer, budget_s):
    """The pooling oracle on the host cores over the whole layer (single thread:
    the pooling definitions are plain loops)."""
    import oracle

    x = workloads.make_pool_input(layer)
    runs, spent = 0, 0.0
    while runs == 0 or (spent < budget_s and runs < 50):
        t0 = time.perf_counter()
        if layer.kind.startswith("global"):
            oracle.global_pool(layer.kind.split("_")[1], x)
        else:
            g = oracle.PoolGeom(layer.n, layer.c, layer.h, layer.w, *layer.kernel, *layer.stride,
                                *layer.dilation, *layer.pads, kind=layer.kind,
                                ceil_mode=layer.ceil_mode,
                                count_include_pad=layer.count_include_pad)
            oracle.pool2d(g, x, dtype=layer.dtype)
        spent += time.perf_counter() - t0
        runs += 1
    return {"s_per_run": spent / runs, "runs": runs, "threads": 1}


_SLEEP_RATE = None


def sleep_cycles(torch, us):
    """Argument of torch.cuda._sleep that holds the stream for about `us`."""
    global _SLEEP_RATE
    if _SLEEP_RATE is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        a.record()
        torch.cuda._sleep(2_000_000)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_RATE = 2_000_000 / max(a.elapsed_time(b) * 1e3, 1.0)  # cycles per us
    return int(_SLEEP_RATE * us)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_layer(layer, budget_s):
    """The fp64 oracle (plain C loops, OpenMP over output planes) on the host
    cores over the whole layer, repeated until about budget_s of work (at least
    one run); the time covers y and the |w*x| scale together."""
    import oracle  # CPU baseline leg only

    inp = workloads.make_inputs(layer)
    t, l, b, r = layer.pads
    g = oracle.Geom(layer.n, layer.c_in, layer.h, layer.w, layer.c_out, layer.kh, layer.kw,
                    groups=layer.groups, sh=layer.stride[0], sw=layer.stride[1],
                    dh=layer.dilation[0], dw=layer.dilation[1], pt=t, pl=l, pb=b, pr=r,
                    oph=layer.out_pad[0], opw=layer.out_pad[1], act=layer.act)
    f = oracle.conv_transpose2d if layer.transpose else oracle.conv2d
    macs, _ = layer_stats(layer)
    runs, spent = 0, 0.0
    while runs == 0 or (spent < budget_s and runs < 500):
        t0 = time.perf_counter()
        f(g, inp.x, inp.w, inp.b, inp.r)
        spent += time.perf_counter() - t0
        runs += 1
    return {"s_per_run": spent / runs, "runs": runs, "gflops": 2 * macs * runs / spent / 1e9}


def cpu_baseline(results, budget_s):
    """The oracle timed per layer on the host cores (rank 0, one GPU): whole
    layers, each repeated for about budget_s.  Returns the headline entry and
    attaches each layer's figures to its result."""
    import oracle

    for r in results.values():
        r["oracle"] = oracle_layer(workloads.BY_NAME[r["name"]], budget_s)
        print(f"# oracle {r['name']}: {r['oracle']['s_per_run']:.3f} s per run, "
              f"{r['oracle']['gflops']:.1f} GFLOP/s", file=sys.stderr, flush=True)
    h = results[HEADLINE]["oracle"]
    return {
        "value": round(h["gflops"] / 1e3, 6), "unit": "TFLOP/s",
        "cores": oracle.max_threads(), "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"whole headline layer (N={workloads.BY_NAME[HEADLINE].n}), fp64 direct "
                  f"loops with the |w*x| scale, {h['runs']} run(s) of {h['s_per_run']:.3f} s; "
                  f"every other layer likewise in layers[].oracle",
    }


CONFIGS = {  # the five workloads as their layers
    1: ["w1_conv3x3_f32"], 2: ["w2_bottleneck3x3_f16"],
    3: ["w3a_stem7x7s2_f16", "w3b_pointwise_f16"],
    4: ["w4a_depthwise5x5_f32", "w4b_depthwise3x3s2_f32", "w4c_pointwise_f32"],
    5: ["w5a_dilated_grouped_f16", "w5b_convtranspose2x2s2_f16"],
}


def config_sums(results):
    out = []
    for cfg, names in CONFIGS.items():
        if not all(n in results for n in names):
            continue
        rs = [results[n] for n in names]
        t = sum(r["us_avg"] for r in rs)
        flops = sum(2 * r["macs"] for r in rs)
        nbytes = sum(r["alg_bytes"] for r in rs)
        roof = sum(r["roof_us"] for r in rs)
        e = {"config": cfg, "layers": names, "us": round(t, 3),
             "tflops": round(flops / (t * 1e-6) / 1e12, 3),
             "gbs": round(nbytes / (t * 1e-6) / 1e9, 1), "roof_us": round(roof, 3),
             "roof_frac": round(roof / t, 4)}
        if all("oracle" in r for r in rs):
            os_ = sum(r["oracle"]["s_per_run"] for r in rs)
            e["oracle_s"] = round(os_, 4)
            e["oracle_gflops"] = round(flops / os_ / 1e9, 2)
        out.append(e)
    return out


def traffic_from_profiles(kernel_src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"^traffic: (.*)$", txt, re.M)
    if not m:
        return None
    # only the two fields used; the kernel name that follows may hold spaces
    sha = re.search(r"\bsource_sha=(\S+)", m.group(1))
    nbytes = re.search(r"\bbytes_per_launch=([0-9.]+)", m.group(1))
    if not sha or not nbytes or sha.group(1) != kernel_src_hash:
        return None
    return float(nbytes.group(1))


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "convolution_forward_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def ceilings(torch):
    """Measured ceilings of this GPU: a streaming copy (1 GiB read + 1 GiB written,
    16-byte vectors) and register-only MFMA loops, from libconvprobe.so."""
    path = os.path.join(ROOT, "convolution_forward_amd", "libconvprobe.so")
    L = ctypes.CDLL(path)
    L.probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                             ctypes.c_void_p]
    L.probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                             ctypes.c_void_p]
    L.probe_l2read.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e-3 / reps

    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    best_copy = 0.0
    for per_cu in (4, 8, 16):
        t = timed(lambda: L.probe_copy(src.data_ptr(), dst.data_ptr(), nbytes // 16, cus * per_cu, sh), 5)
        best_copy = max(best_copy, 2 * nbytes / t / 1e9)
    del src, dst
    # L2 -> CU reads: a 2 MiB buffer (resident in every XCD's 4 MiB L2), each
    # workgroup reading 2 MiB of it, 2 to 8 workgroups per CU
    l2buf = torch.ones((2 << 20) // 4, dtype=torch.float32, device="cuda")
    l2out = torch.empty(cus * 8 * 256, dtype=torch.int32, device="cuda")
    per_wg = 512
    best_l2 = 0.0
    for per_cu in (2, 4, 8):
        blocks = cus * per_cu
        t = timed(lambda: L.probe_l2read(l2buf.data_ptr(), (2 << 20) // 16, per_wg, blocks,
                                         l2out.data_ptr(), sh), 5)
        best_l2 = max(best_l2, blocks * per_wg * 4096 / t / 1e9)
    del l2buf, l2out
    out = torch.empty(cus * 4 * 256, dtype=torch.float32, device="cuda")
    macs_per_iter = {0: 4 * 32 * 32 * 16, 1: 8 * 16 * 16 * 32, 2: 8 * 16 * 16 * 64}
    names = {0: "mfma_f32_32x32x16_f16_tflops", 1: "mfma_f32_16x16x32_f16_tflops",
             2: "mfma_i32_16x16x64_i8_tops"}
    res = {"copy_gbs": round(best_copy, 1), "copy_bytes": 2 * nbytes,
           "l2_read_gbs": round(best_l2, 1), "l2_read_gbs_per_cu": round(best_l2 / cus, 2)}
    iters = 4000
    for kind in (0, 1, 2):
        best = 0.0
        for per_cu in (1, 2, 4):
            blocks = cus * per_cu
            t = timed(lambda: L.probe_mfma(kind, iters, blocks, out.data_ptr(), sh), 3)
            best = max(best, 2 * blocks * 4 * iters * macs_per_iter[kind] / t / 1e12)
        res[names[kind]] = round(best, 1)
    res["compute_units"] = cus
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--loops", type=int, default=5)
    ap.add_argument("--oracle-budget", type=float, default=1.5,
                    help="seconds of oracle work per layer for cpu_baseline")
    ap.add_argument("--layers", default="")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib", type=int, default=0)
    ap.add_argument("--ceilings", action="store_true",
                    help="also measure the streaming-copy and register-only MFMA ceilings")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the path would shard by batch or output channel; no multi-GPU run is provided)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import convolution_forward_amd as cf

    if args.copy_calib:
        n = args.copy_calib // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n * 4}))
        return

    cf.lib()  # fail loudly if the native library is missing
    ceil = ceilings(torch) if args.ceilings else None
    default = [l.name for l in workloads.LAYERS] + [l.name for l in workloads.EXTRA_LAYERS]
    names = [HEADLINE] if args.headline_only else (
        args.layers.split(",") if args.layers else default)
    if HEADLINE not in names:
        names.insert(0, HEADLINE)
    results = {}
    for nm in names:
        results[nm] = time_layer(cf, torch, workloads.BY_NAME[nm], args.steps, args.warmup,
                                 args.loops)
        print(f"# {nm}: {results[nm]['variant']} {results[nm]['us_avg']:.2f} us "
              f"{results[nm]['tflops']:.1f} TFLOP/s {results[nm]['gbs']:.0f} GB/s "
              f"{100 * results[nm]['roof_frac']:.1f}% of {results[nm]['bound']} roof "
              f"(loops {results[nm]['us_loops']})", file=sys.stderr, flush=True)
    h = results[HEADLINE]
    layer = workloads.BY_NAME[HEADLINE]
    macs, nbytes = layer_stats(layer)
    value = 2 * macs / (h["total_s"] / args.steps) / 1e12
    traffic = traffic_from_profiles(kernel_source_hash())
    pools = []
    if not args.headline_only and not args.layers:
        for pl in workloads.POOL_LAYERS:
            r = time_pool(cf, torch, pl, args.steps, args.warmup, args.loops)
            print(f"# {pl.name}: {r['variant']} {r['us_avg']:.2f} us {r['gbs']:.0f} GB/s "
                  f"{100 * r['roof_frac']:.1f}% of hbm roof", file=sys.stderr, flush=True)
            pools.append(r)
    ints = []
    if not args.headline_only and not args.layers:
        for il in workloads.INT_LAYERS:
            r = time_int(cf, torch, il, args.steps, args.warmup, args.loops)
            print(f"# {il.name}: {r['variant']} {r['us_avg']:.2f} us {r['tops']:.1f} TOP/s "
                  f"{100 * r['roof_frac']:.1f}% of {r['bound']} roof", file=sys.stderr, flush=True)
            ints.append(r)
    cpu = None if args.no_cpu_baseline else cpu_baseline(results, args.oracle_budget)
    if cpu is not None:
        for r in pools:
            r["oracle"] = oracle_pool(workloads.POOL_BY_NAME[r["name"]], args.oracle_budget)
        for r in ints:
            r["oracle"] = oracle_int(workloads.INT_BY_NAME[r["name"]], args.oracle_budget)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["total_s"] / args.steps * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded U[-1,1] inputs, He-normal weights, U[-0.1,0.1] bias, "
                "U[-1,1] residual)",
        "config": {"workload": "ResNet-style bottleneck 3x3 fp16 (fp32 accumulate), N=32, "
                               "Cin=Cout=256, 14x14, stride 1, pad 1, bias + residual + ReLU",
                   "variant": h["variant"], "rotating_sets": h["rotating_sets"],
                   "rotation_bytes": h["rotation_bytes"], "loops": args.loops,
                   "timing": f"median of {args.loops} event-timed loops of {args.steps} calls",
                   "hbm_gbs_alg": round(h["gbs"], 1)},
        "roofline": {
            "bound": "mfma",
            "achieved": round(2 * macs / (h["us_avg"] * 1e-6) / 1e12, 3),
            "peak": PEAK["f16_mfma_tflops"],
            "unit": "TFLOP/s",
            "frac": round(2 * macs / (h["us_avg"] * 1e-6) / 1e12 / PEAK["f16_mfma_tflops"], 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "configs": config_sums(results),
        "ceilings": ceil,
        "pools": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                  for r in pools],
        "conv_integer": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                         for r in ints],
        "layers": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()
                    if k not in ("total_s", "wall_s")} for r in results.values()],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
