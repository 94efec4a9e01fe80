"""Benchmark of the 2:4 + rank-r linear hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: for every layer of the
workload, the 2:4 projection + pack of the residual R = W - U V (splr_prune24_pack), then the layer
product Y = X S^T + (X V^T) U^T with the freshly packed S (splr_linear, issued as its two stages:
splr_linear_stage1 computes T = X V^T, splr_linear_stage2 the sparse product and the low-rank
epilogue). Inputs are resident in HBM before timing starts. Each step reads a different copy of the
weights and activations when one step's footprint is small, so repeated steps are not served from
the 256 MB Infinity Cache.

Timed region (value): exactly K steps issued on one stream between two events. A spin kernel queued
before the start event keeps the GPU busy while the host enqueues all K steps, so the region
measures back-to-back GPU execution of the steps, not host launch gaps (measured here, replaying
HIP graphs of the steps was slower than plain stream launches; --graph times that variant).
Per-kernel region: the same K steps again, every library call issued 8 times back to back with an
event after each group (the calls are idempotent), so a call's average duration carries 1/8 of
the cost of an event.

Prints one JSON line. `value` is dense-equivalent TFLOP/s (2 M n_out n_in per layer) of the whole
step for the prefill workloads, or GB/s of the weight-side bytes (packed values, metadata, U, V)
for the decode workload. `roofline` describes the kernel with the largest share of the step;
`context` holds reference points from the same run (a dense GEMM of the first layer's shape through
torch, a plain device copy moving as many bytes as its weight side).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C2] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "2:4+rank-r linear: dense-equiv TFLOP/s & HBM GB/s vs roofline, Llama3-8B shapes"
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3     # MI355X fp32 (vector / MFMA)
# fp32 fused multiply-add on the vector ALUs without packed (two-wide) instructions, which this
# library does not use: 256 CUs x 4 SIMDs x 16 lanes per clock x 2 FLOP x 2.4 GHz = 78.6 TFLOP/s (the
# vendor's 157.3 TFLOP/s fp32 vector figure counts two-wide packed fused multiply-adds)
PEAK_FP32_VALU_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E
MALL_DEFEAT_BYTES = 640 << 20  # > 2 x (256 MB Infinity Cache + 8 x 4 MB L2)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
REPEAT = 8                    # back-to-back launches per timed group in the per-kernel region

# library call -> source file of the kernel it launches (the traffic figures are tied to it)
KERNEL_SOURCE = {"pack": "pack.hip", "stage2": "linear_bf16.hip"}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="C2", help="C1..C5 (default: C2, the prefill q_proj layer)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    p.add_argument("--no-next", action="store_true", help="skip the measurements of the parts beyond the hot path")
    p.add_argument("--cpu-rows", type=int, default=0, help="token rows of the oracle sample (0 = auto)")
    p.add_argument("--graph", action="store_true", help="replay the steps from HIP graphs (for comparison)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device-to-device copy 5 times (scale for HBM counters) and exit")
    return p.parse_args()


def layer_bytes(n_in, n_out, r, itemsize):
    """Weight-side bytes one splr_linear call must read: packed values, metadata, U, V."""
    return n_out * n_in // 2 * itemsize + n_out * n_in // 8 + (n_out * r + r * n_in) * itemsize


def pack_bytes(n_in, n_out, itemsize):
    """Bytes splr_prune24_pack must move: read R, write values and metadata."""
    return n_out * n_in * itemsize + n_out * n_in // 2 * itemsize + n_out * n_in // 8


def stage2_work(L, itemsize, decode):
    """Algorithmic work of splr_linear_stage2: the kept products (M n_out n_in / 2 multiply-adds)
    plus the rank-r epilogue (M n_out r multiply-adds), in FLOP; or, for decode, the bytes it must
    move: packed values, metadata, U, X, T (as the bfloat16 pair) and the float32 Y."""
    if decode:
        return (L.n_out * L.n_in // 2 * itemsize + L.n_out * L.n_in // 8 + L.n_out * L.r * itemsize
                + L.M * L.n_in * itemsize + L.M * L.r * 4 + L.M * L.n_out * 4)
    return L.M * L.n_out * L.n_in + 2 * L.M * L.n_out * L.r


def source_sha(name):
    path = os.path.join(ROOT, "sparse_rank_linear_prune24_amd", "csrc", name)
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter summary, or None
    when there is none or the kernel source changed since the counters were taken."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    pat = re.compile(r"^\|\s*(\w+)\s*\|\s*(\w+)\s*\|\s*([0-9a-f]{16})\s*\|.*\|\s*([0-9.]+)\s*\|$")
    want = source_sha(KERNEL_SOURCE[kernel])
    with open(COUNTERS_FILE) as fh:
        for line in fh:
            m = pat.match(line.strip())
            if m and m.group(1) == kernel and m.group(2) == workload:
                return float(m.group(4)) if m.group(3) == want else None
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the layer shards by output rows or input columns; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps(dict(copy_bytes=src.numel(), calls=5)), flush=True)
        return

    from sparse_rank_linear_prune24_amd import binding, configs, inputs

    cfg = configs.get(args.workload)
    dtype = cfg.dtype
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    isz = inputs.itemsize(dtype)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.lib()
    decode = cfg.M <= 64

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    # ---------------------------------------------------------------- inputs (host, then HBM)
    t0 = time.perf_counter()
    layers = [inputs.make_layer(cfg.name, li) for li in range(len(cfg.layers))]
    gen_s = time.perf_counter() - t0

    step_bytes = 0
    for L in layers:
        step_bytes += (L.R.nbytes + L.n_out * L.n_in // 2 * isz + L.n_out * L.n_in // 8 + L.U.nbytes + L.V.nbytes
                       + L.X.nbytes + L.M * L.n_out * 4)
    copies = max(1, math.ceil(MALL_DEFEAT_BYTES / step_bytes))

    sets = []
    for c in range(copies):
        s = []
        for L in layers:
            ws_n = binding.workspace_bytes(L.M, L.n_out, L.n_in, L.r, tdt)
            s.append(dict(
                R=to_dev(L.R), W=to_dev(L.W), X=to_dev(L.X), U=to_dev(L.U), V=to_dev(L.V),
                values=torch.empty((*binding.tiles(L.n_out, L.n_in), 64, 8), dtype=tdt, device=dev),
                meta=torch.empty((*binding.tiles(L.n_out, L.n_in), 2, 16), dtype=torch.int32, device=dev),
                Y=torch.empty((L.M, L.n_out), dtype=torch.float32, device=dev),
                ws=torch.zeros(max(ws_n, 256), dtype=torch.uint8, device=dev)))
        sets.append(s)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    n_layers = len(layers)
    calls = ("pack", "stage1", "stage2")

    def step(i, ev=None, repeat=1):
        """One step on `stream`. With `ev`, every library call is issued `repeat` times back to back
        and ev[c][li] is recorded after the repeats of call c of layer li (the calls are idempotent)."""
        s = sets[i % copies]
        for li, d in enumerate(s):
            for _ in range(repeat):
                binding.prune24_pack(d["R"], d["values"], d["meta"], stream=stream)
            if ev is not None:
                ev[0][li].record(stream)
        for li, d in enumerate(s):
            for _ in range(repeat):
                binding.linear_stage1(d["X"], d["V"], d["ws"], stream=stream)
            if ev is not None:
                ev[1][li].record(stream)
            for _ in range(repeat):
                binding.linear_stage2(d["X"], d["values"], d["meta"], d["U"], d["ws"], n_out=d["Y"].shape[1],
                                      out=d["Y"], stream=stream)
            if ev is not None:
                ev[2][li].record(stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()

        # optional: one graph per weight copy, each holding exactly one step
        graphs = []
        if args.graph:
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    step(c)
                graphs.append(g)
            for g in graphs:
                g.replay()
            torch.cuda.synchronize()
        spin_cycles = int(4e4 * args.steps * 3 * n_layers)  # ~60 us of GPU time per library call issued

        # timed region: exactly K steps
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(spin_cycles)
        start.record(stream)
        for i in range(args.steps):
            if graphs:
                graphs[i % copies].replay()
            else:
                step(i)
        end.record(stream)
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(end)

        # per-kernel region: the same K steps with every library call issued REPEAT times back to back
        # and an event after each group, so the cost of an event is spread over REPEAT launches
        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(n_layers)] for _ in calls]
               for _ in range(args.steps)]
        first = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(spin_cycles * REPEAT)
        first.record(stream)
        for i in range(args.steps):
            step(i, evs[i], repeat=REPEAT)
        torch.cuda.synchronize()

    # per-call durations (ms), averaged over the steps: the interval since the previous event
    call_ms = {c: np.zeros(n_layers) for c in calls}
    order = [(0, li) for li in range(n_layers)] + [(c, li) for li in range(n_layers) for c in (1, 2)]
    for i, ev in enumerate(evs):
        prev = first if i == 0 else evs[i - 1][2][n_layers - 1]
        for c, li in order:
            call_ms[calls[c]][li] += prev.elapsed_time(ev[c][li])
            prev = ev[c][li]
    for c in calls:
        call_ms[c] = call_ms[c] / (args.steps * REPEAT)

    ms_per_step = total_ms / args.steps
    flop_step = sum(2 * L.M * L.n_out * L.n_in for L in layers)
    wbytes_step = sum(layer_bytes(L.n_in, L.n_out, L.r, isz) for L in layers)
    pbytes_step = sum(pack_bytes(L.n_in, L.n_out, isz) for L in layers)
    s2_work = sum(stage2_work(L, isz, decode) for L in layers)

    per_layer = []
    for li, L in enumerate(layers):
        pb = pack_bytes(L.n_in, L.n_out, isz)
        lin = call_ms["stage1"][li] + call_ms["stage2"][li]
        per_layer.append(dict(
            layer=L.name, pack_us=round(call_ms["pack"][li] * 1e3, 2),
            pack_GBps=round(pb / (call_ms["pack"][li] * 1e-3) / 1e9, 1),
            stage1_us=round(call_ms["stage1"][li] * 1e3, 2), stage2_us=round(call_ms["stage2"][li] * 1e3, 2),
            linear_dense_equiv_TFLOPs=round(2 * L.M * L.n_out * L.n_in / (lin * 1e-3) / 1e12, 1),
            linear_weight_GBps=round(layer_bytes(L.n_in, L.n_out, L.r, isz) / (lin * 1e-3) / 1e9, 1)))

    # roofline of the kernel with the largest share of the step
    pack_s, s2_s = call_ms["pack"].sum() * 1e-3, call_ms["stage2"].sum() * 1e-3
    wl = cfg.name
    if pack_s >= s2_s:
        ach = pbytes_step / pack_s / 1e9
        roofline = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                        frac=round(ach / PEAK_HBM_GBPS, 4), traffic=recorded_traffic("pack", wl),
                        kernel="prune24_pack_kernel", work="bytes read + written: R, packed values, metadata")
    elif decode:
        ach = s2_work / s2_s / 1e9
        roofline = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                        frac=round(ach / PEAK_HBM_GBPS, 4), traffic=recorded_traffic("stage2", wl),
                        kernel="linear_decode_kernel", work="bytes: packed values, metadata, U, X, T, Y")
    else:
        peak = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_TFLOPS
        ach = s2_work / s2_s / 1e12
        roofline = dict(bound="mfma", achieved=round(ach, 1), peak=peak, unit="TFLOP/s",
                        frac=round(ach / peak, 4), traffic=recorded_traffic("stage2", wl),
                        kernel="linear_prefill_kernel",
                        work="algorithmic FLOP: kept 2:4 products (M n_out n_in) + rank-r epilogue (2 M n_out r)",
                        dense_equiv_TFLOPs=round(flop_step / s2_s / 1e12, 1))

    if decode:
        value, unit = wbytes_step / (ms_per_step * 1e-3) / 1e9, "GB/s"
    else:
        value, unit = flop_step / (ms_per_step * 1e-3) / 1e12, "TFLOP/s"

    out = dict(
        metric=METRIC, value=round(value, 2), unit=unit, n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms_per_step, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype=dtype, data="synthetic",
        config=dict(workload=f"{cfg.name}: {cfg.description}", tokens=cfg.M, rank=cfg.r,
                    layers=[f"{n}:{k}->{o}" for n, k, o in cfg.layers],
                    step="prune24_pack on every layer's residual, then splr_linear (stage 1 + stage 2) on every "
                         "layer", launch="graph replay" if graphs else "stream, queue pre-filled", parallelism="single GPU",
                    copies_rotated=copies),
        roofline=roofline,
        kernels=dict(per_layer=per_layer,
                     pack_GBps=round(pbytes_step / pack_s / 1e9, 1),
                     linear_dense_equiv_TFLOPs=round(
                         flop_step / ((call_ms["stage1"].sum() + call_ms["stage2"].sum()) * 1e-3) / 1e12, 1)),
        input_generation_s=round(gen_s, 1),
    )

    out["context"] = measure_context(layers, decode, tdt, stream, dev, args)

    if not args.no_next:
        out["next"] = measure_next(binding, inputs, layers, sets, copies, stream, dev, args)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, layers, dtype, flop_step, wbytes_step, decode, args.cpu_rows)
    print(json.dumps(out), flush=True)


def time_per_call(issue, n, stream, spin_cycles):
    """Average GPU time (ms) of one call: `issue(i)` enqueues call i on `stream`; n calls, each
    issued REPEAT times back to back, between two events behind a queue-filling spin."""
    import torch
    for i in range(3):
        issue(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(spin_cycles)
        e0.record(stream)
        for i in range(n):
            for _ in range(REPEAT):
                issue(i)
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (n * REPEAT)


def measure_context(layers, decode, tdt, stream, dev, args):
    """Reference points measured in the same run (context for the fractions of peak, not targets),
    on the first layer: a dense GEMM of the layer's shape (torch.mm in the storage type: X
    [M x n_in] times a dense [n_in x n_out], hipBLASLt; prefill workloads), and a plain read stream
    of the same size as the layer's weight-side bytes (packed values, metadata, U, V): a device copy
    reading half of them and writing the other half, rotated over enough buffers to miss the 256 MB
    Infinity Cache."""
    import torch
    L = layers[0]
    isz = 2 if tdt == torch.bfloat16 else 4
    n = max(8, args.steps // 2)
    spin = int(4e4 * n * REPEAT)
    res = {}
    if not decode:
        g = torch.Generator(device=dev)
        g.manual_seed(0)
        X = torch.randn(L.M, L.n_in, device=dev, generator=g).to(tdt)
        Ws = [torch.randn(L.n_in, L.n_out, device=dev, generator=g).to(tdt) for _ in range(4)]
        ms = time_per_call(lambda i: torch.mm(X, Ws[i % len(Ws)]), n, stream, spin)
        flop = 2 * L.M * L.n_out * L.n_in
        peak = PEAK_BF16_TFLOPS if isz == 2 else PEAK_FP32_TFLOPS
        res["dense_gemm"] = dict(layer=L.name, op="torch.mm (hipBLASLt), dense weight of the same shape",
                                 us=round(ms * 1e3, 2), TFLOPs=round(flop / (ms * 1e-3) / 1e12, 1),
                                 frac_of_peak=round(flop / (ms * 1e-3) / 1e12 / peak, 4))
        del X, Ws
    wbytes = L.n_out * L.n_in // 2 * isz + L.n_out * L.n_in // 8 + (L.n_out + L.n_in) * L.r * isz
    half = wbytes // 2 // 16 * 16
    nbuf = max(2, math.ceil(MALL_DEFEAT_BYTES / wbytes))
    srcs = [torch.ones(half, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    dsts = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    ms = time_per_call(lambda i: dsts[i % nbuf].copy_(srcs[i % nbuf]), n, stream, spin)
    res["stream"] = dict(layer=L.name, op="device copy moving the weight-side bytes (half read, half written)",
                         bytes=2 * half, us=round(ms * 1e3, 2), GBps=round(2 * half / (ms * 1e-3) / 1e9, 1),
                         frac_hbm=round(2 * half / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4))
    del srcs, dsts
    torch.cuda.synchronize()
    return res


def measure_next(binding, inputs, layers, sets, copies, stream, dev, args):
    """The parts built beyond the hot path, each timed per call on every layer of the workload
    (outside the timed step): the activation-aware pack (keys |R| |d|, d = column norms of the
    layer's activations), the 2:8 projection stored in the 2:4 layout, the fused residual + pack
    (R = W - U V formed in the kernel), the layer
    product with a bfloat16 Y (splr_linear_ex) and steps of the data-free alternating minimisation."""
    import torch
    n = max(8, args.steps // 2)
    spin = int(4e4 * n * REPEAT)
    res = {}
    per_layer = []
    for li, L in enumerate(layers):
        d = torch.from_numpy(inputs.column_scales(L.X, L.dtype)).to(dev)
        isz = inputs.itemsize(L.dtype)
        nbytes = pack_bytes(L.n_in, L.n_out, isz) + L.n_in * 4

        def issue(i, li=li, d=d):
            s = sets[i % copies][li]
            binding.prune24_pack_scaled(s["R"], d, s["values"], s["meta"], stream=stream)

        ms = time_per_call(issue, n, stream, spin)
        per_layer.append(dict(layer=L.name, us=round(ms * 1e3, 2), GBps=round(nbytes / (ms * 1e-3) / 1e9, 1),
                              frac_hbm=round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)))
    res["pack_scaled"] = dict(entry="splr_prune24_pack_scaled", bound="hbm",
                              work="bytes: R + d + packed values + metadata", per_layer=per_layer)

    # N:M projection (2:8, the pages' post-fine-tuning pattern) stored in the 2:4 layout: HBM bound,
    # the same bytes as the 2:4 pack
    per_layer = []
    for li, L in enumerate(layers):
        nbytes = pack_bytes(L.n_in, L.n_out, inputs.itemsize(L.dtype))

        def issue(i, li=li):
            s = sets[i % copies][li]
            binding.prune_nm_pack(s["R"], 2, 8, s["values"], s["meta"], stream=stream)

        ms = time_per_call(issue, n, stream, spin)
        per_layer.append(dict(layer=L.name, us=round(ms * 1e3, 2), GBps=round(nbytes / (ms * 1e-3) / 1e9, 1),
                              frac_hbm=round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)))
    res["pack_2_8"] = dict(entry="splr_prune_nm_pack (n = 2, m = 8)", bound="hbm",
                           work="bytes: R + packed values + metadata", per_layer=per_layer)

    # fused residual + pack: vector-ALU bound (r fused multiply-adds per weight, binary32, not packed)
    per_layer = []
    for li, L in enumerate(layers):
        isz = inputs.itemsize(L.dtype)
        nbytes = pack_bytes(L.n_in, L.n_out, isz) + (L.n_out + L.n_in) * L.r * isz
        fmas = L.n_out * L.n_in * L.r

        def issue(i, li=li):
            s = sets[i % copies][li]
            binding.prune24_pack_residual(s["W"], s["U"], s["V"], s["values"], s["meta"], stream=stream)

        ms = time_per_call(issue, n, stream, spin)
        tflops = 2 * fmas / (ms * 1e-3) / 1e12
        per_layer.append(dict(layer=L.name, us=round(ms * 1e3, 2), fp32_TFLOPs=round(tflops, 1),
                              frac_alu=round(tflops / PEAK_FP32_VALU_TFLOPS, 4),
                              GBps=round(nbytes / (ms * 1e-3) / 1e9, 1)))
    res["pack_residual"] = dict(entry="splr_prune24_pack_residual", bound="alu",
                                peak_TFLOPs=PEAK_FP32_VALU_TFLOPS,
                                work="2 n_out n_in r FLOP (the residual's fused multiply-adds); bytes W + U + V + "
                                     "packed values + metadata", per_layer=per_layer)

    # bfloat16 Y: the same layer product with the output rounded to bfloat16 (half the Y bytes)
    per_layer = []
    for li, L in enumerate(layers):
        if L.dtype != "bf16":
            continue
        y16 = torch.empty((L.M, L.n_out), dtype=torch.bfloat16, device=dev)

        def issue(i, li=li, y16=y16):
            s = sets[i % copies][li]
            binding.linear_ex(s["X"], s["values"], s["meta"], s["U"], s["V"], y_dtype=torch.bfloat16,
                              n_out=L.n_out, out=y16, workspace=s["ws"], stream=stream)

        ms = time_per_call(issue, n, stream, spin)
        per_layer.append(dict(layer=L.name, us=round(ms * 1e3, 2),
                              dense_equiv_TFLOPs=round(2 * L.M * L.n_out * L.n_in / (ms * 1e-3) / 1e12, 1)))
    res["linear_bf16_y"] = dict(entry="splr_linear_ex (y_dtype bfloat16)", bound="mfma",
                                work="dense-equivalent FLOP 2 M n_out n_in", per_layer=per_layer)

    # data-free alternating minimisation on the first layer: per-step time (untracked) and the
    # objective / layer error over a few steps (tracked)
    from sparse_rank_linear_prune24_amd import am
    L = layers[0]
    s0 = sets[0][0]
    if L.r > 0:
        steps = 6
        am.alternating_minimization(s0["W"], L.r, 1, track=False)  # warm-up (library initialisation)
        t = am.alternating_minimization(s0["W"], L.r, steps, track=False)
        tracked = am.alternating_minimization(s0["W"], L.r, steps, X=s0["X"])
        wnorm = float(torch.linalg.norm(s0["W"].float()))
        res["am_loop"] = dict(layer=L.name, steps=steps, ms_per_step=round(t["seconds"] / steps * 1e3, 3),
                              est_80_steps_s=round(t["seconds"] / steps * 80, 3),
                              rel_objective=[round(o / wnorm, 5) for o in tracked["objective"]],
                              layer_rel_error=[round(e, 5) for e in tracked["layer_rel_error"]],
                              step="splr_prune24_pack_residual + dense reconstruct of S + rank-r subspace "
                                   "iteration (torch matmul / QR / small SVD)")
    return res


def cpu_baseline(cfg, layers, dtype, flop_step, wbytes_step, decode, rows_arg):
    """The oracle, untuned, on this host's cores: the full pack of every layer plus the layer product
    on a sample of token rows, scaled to one step."""
    import oracle

    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    oracle.build(force=False)
    t_pack = 0.0
    t_lin = 0.0
    frac_rows = []
    for L in layers:
        t0 = time.perf_counter()
        v, m = oracle.prune24_pack(L.R, dtype)
        t_pack += time.perf_counter() - t0
        rows = rows_arg or max(1, min(L.M, int(4e9 / (L.n_out * L.n_in / 2) // 1)))
        rows = min(rows, L.M)
        sel = np.linspace(0, L.M - 1, rows).astype(np.int64)
        t0 = time.perf_counter()
        oracle.linear(L.X, v, m, L.n_out, L.U, L.V, dtype, rows=sel)
        dt = time.perf_counter() - t0
        t_lin += dt * (L.M / rows)
        frac_rows.append(f"{L.name}: {rows}/{L.M} rows")
    t_step = t_pack + t_lin
    if decode:
        value, unit = wbytes_step / t_step / 1e9, "GB/s"
    else:
        value, unit = flop_step / t_step / 1e12, "TFLOP/s"
    cpu = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(value=round(value, 6), unit=unit, cores=int(os.environ["OMP_NUM_THREADS"]), kind="oracle",
                sample=f"full pack of every layer; layer product on evenly spaced token rows ({'; '.join(frac_rows)}), "
                       f"time scaled to all rows; float64, OpenMP",
                step_s_equiv=round(t_step, 3), pack_s=round(t_pack, 3), cpu=cpu)


if __name__ == "__main__":
    main()
