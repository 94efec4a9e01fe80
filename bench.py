"""Benchmark of the 2:4 + rank-r linear hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input. For the prefill workloads
(C1, C2, C4, C5; C5 by default) it is, for every layer, the 2:4 projection + pack of the residual
R = W - U V (splr_prune24_pack), then the layer product Y = X S^T + (X V^T) U^T with the freshly
packed S (splr_linear, issued as its two stages: splr_linear_stage1 computes T = X V^T,
splr_linear_stage2 the sparse product and the low-rank epilogue). For the decode workload (C3),
whose figure is the layer product's HBM rate on the packed S, metadata, U and V, the step is the
layer product alone; the pack of its layer is timed beside it and reported in `kernels`. Inputs
are resident in HBM before timing starts. Steps rotate over enough copies of the weights and
activations that no step finds its data in the 256 MB Infinity Cache.

Timed region (value): exactly K steps issued on one stream between two events. A spin kernel queued
before the start event keeps the GPU busy while the host enqueues all K steps, so the region
measures back-to-back GPU execution of the steps, not host launch gaps (measured here, replaying
HIP graphs of the steps was slower than plain stream launches; --graph times that variant).

Per-kernel region: the same K steps again with events between the library calls, for the
per-kernel durations and the roofline. Where one step moves less than twice the Infinity Cache
plus L2, every call is issued REPEAT = 8 times back to back on 8 different copies between two
events (so a call carries 1/8 of an event's cost and never re-reads a copy that is still cached);
larger steps issue every call once, between events.

Prints one JSON line. `value` is dense-equivalent TFLOP/s (2 M n_out n_in per layer) of the whole
step for the prefill workloads, or GB/s of the weight-side bytes (packed values, metadata, U, V)
for the decode workload. `roofline` describes the kernel with the largest share of the step;
`context` holds reference points from the same run (a dense GEMM of the first layer's shape through
torch, a plain device copy moving as many bytes as its weight side).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
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
REPEAT_SMALL = 8              # back-to-back launches per timed group when a step is small

# kernel -> the source files it is built from (the traffic figures are tied to their hash)
KERNEL_SOURCE = {"pack": ("pack.hip", "common.hpp"),
                 "stage2": ("linear_bf16.hip", "tile_common.hpp", "common.hpp"),
                 "decode": ("decode.hip", "tile_common.hpp", "common.hpp")}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="C5",
                   help="C1..C5 (default: C5, the Llama-3-8B block linear set, 8192 tokens, rank 128)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    p.add_argument("--no-group", action="store_true",
                   help="one stage-2 launch per layer (no grouped launch of equal-shape layers)")
    p.add_argument("--no-next", action="store_true", help="skip the measurements of the parts beyond the hot path")
    p.add_argument("--no-context", action="store_true", help="skip the same-run reference points (profiling runs)")
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


def wide_tile(L, count=1):
    """The library's tile rule: 512-row tiles when the launch's layers together give every CU
    (256) a tile of 512 rows x 128 tokens, else 256 rows."""
    return count * -(-L.n_out // 512) * -(-L.M // 128) >= 256


def tile_rounds(L, count=1):
    """Rounds of 256 CUs the stage-2 tiles of `count` layers shaped like L take in one launch."""
    rows = 512 if wide_tile(L, count) else 256
    return -(-count * -(-L.n_out // rows) * -(-L.M // 128) // 256)


def stage2_units(layers, decode):
    """The step's stage-2 launches: adjacent layers of one shape go into one grouped launch
    (splr_linear_stage2_group, up to 4 layers) when that needs fewer rounds of tiles than launching
    them one by one -- k_proj and v_proj of the block (alone 256-row tiles, together 512-row ones),
    or layers whose tile count leaves a part-filled last round (gate and up at 4096 tokens: 3.5
    rounds each, 7 together); every other layer is a launch of its own."""
    runs = []
    for li, L in enumerate(layers):
        prev = runs[-1] if runs else None
        if (not decode and prev is not None and len(prev) < 4
                and (layers[prev[0]].M, layers[prev[0]].n_in, layers[prev[0]].n_out, layers[prev[0]].r)
                == (L.M, L.n_in, L.n_out, L.r)):
            prev.append(li)
        else:
            runs.append([li])
    units = []
    for u in runs:
        L = layers[u[0]]
        if len(u) > 1 and tile_rounds(L, len(u)) < len(u) * tile_rounds(L):
            units.append(u)
        else:
            units.extend([j] for j in u)
    return units


def prefill_kernels(layers, units):
    """Which stage-2 tile each launch takes (both are linear_prefill_wide_kernel)."""
    names = {}
    for u in units:
        L = layers[u[0]]
        key = "512-row tile" if wide_tile(L, len(u)) else "256-row tile"
        names.setdefault(key, []).append("+".join(layers[j].name for j in u) + (" grouped" if len(u) > 1 else ""))
    return "linear_prefill_wide_kernel: " + "; ".join(f"{k} ({', '.join(v)})" for k, v in names.items())


def source_sha(names):
    """First 16 hex digits of the SHA-256 over the files (name, NUL, contents, NUL, in order)."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "sparse_rank_linear_prune24_amd", "csrc", name), "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read() + b"\0")
    return h.hexdigest()[:16]


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

    # bytes one step moves per copy (pack: R, values, metadata; layer product: values, metadata, U,
    # V, X, T partials, Y)
    step_bytes = 0
    for L in layers:
        lin = layer_bytes(L.n_in, L.n_out, L.r, isz) + L.X.nbytes + L.M * L.n_out * 4 + 2 * L.M * L.r * 4
        step_bytes += lin + (0 if decode else pack_bytes(L.n_in, L.n_out, isz))
    repeat = REPEAT_SMALL if step_bytes < MALL_DEFEAT_BYTES else 1
    # between two uses of one copy, every other copy's step passes through the caches
    copies = 1 if repeat == 1 else max(2 * repeat, math.ceil(MALL_DEFEAT_BYTES / step_bytes) + 1)

    sets = []
    for c in range(copies):
        s = []
        for L in layers:
            ws_n = binding.workspace_bytes(L.M, L.n_out, L.n_in, L.r, tdt)
            s.append(dict(
                R=to_dev(L.R), X=to_dev(L.X), U=to_dev(L.U), V=to_dev(L.V),
                values=torch.empty((*binding.tiles(L.n_out, L.n_in), 64, 8), dtype=tdt, device=dev),
                meta=torch.empty(binding.meta_shape(L.n_out, L.n_in), dtype=torch.int32, device=dev),
                Y=torch.empty((L.M, L.n_out), dtype=torch.float32, device=dev),
                ws=torch.empty(max(ws_n, 256), dtype=torch.uint8, device=dev)))
        sets.append(s)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    n_layers = len(layers)
    calls = ("stage1", "stage2") if decode else ("pack", "stage1", "stage2")

    def pack(d):
        binding.prune24_pack(d["R"], d["values"], d["meta"], stream=stream)

    def stage1(d):
        binding.linear_stage1(d["X"], d["V"], d["ws"], stream=stream)

    units = [[li] for li in range(n_layers)] if args.no_group else stage2_units(layers, decode)

    def stage2(s, unit):
        """Stage 2 of the layers in `unit` (indices into the copy s): one launch either way."""
        if len(unit) == 1:
            d = s[unit[0]]
            binding.linear_stage2(d["X"], d["values"], d["meta"], d["U"], d["ws"], n_out=d["Y"].shape[1],
                                  out=d["Y"], stream=stream)
        else:
            ds = [s[j] for j in unit]
            binding.linear_stage2_group([d["X"] for d in ds], [d["values"] for d in ds], [d["meta"] for d in ds],
                                        [d["U"] for d in ds], [d["ws"] for d in ds], n_out=ds[0]["Y"].shape[1],
                                        outs=[d["Y"] for d in ds], stream=stream)

    def call(c, s, unit):
        if c == "stage2":
            stage2(s, unit)
        else:
            (pack if c == "pack" else stage1)(s[unit[0]])

    def step(i):
        """Step i on `stream`, on copy i % copies: for each stage-2 launch, the pack of its layers
        (prefill workloads), their first stage, then the launch -- each layer's packed S and X are
        then still in the Infinity Cache when its stage 2 reads them (measured: C5 2.531-2.537
        against 2.555-2.564 ms per step with every pack first; C4 unchanged)."""
        s = sets[i % copies]
        for unit in units:
            if not decode:
                for li in unit:
                    pack(s[li])
            for li in unit:
                stage1(s[li])
            stage2(s, unit)

    def step_timed(i, ev):
        """Step i of the per-kernel region: each call issued `repeat` times on `repeat` consecutive
        copies (starting at copy i * repeat), ev[c][li] recorded after the group of call c whose
        (first) layer is li. The stages of one layer read the workspace of their own copy."""
        base = i * repeat
        order = [(c, u) for unit in units
                 for c, u in ([("pack", [li]) for li in unit] if not decode else [])
                 + [("stage1", [li]) for li in unit] + [("stage2", unit)]]
        for c, unit in order:
            for j in range(repeat):
                call(c, sets[(base + j) % copies], unit)
            ev[calls.index(c)][unit[0]].record(stream)
        return order

    with torch.cuda.stream(stream):
        for i in range(max(args.warmup, copies)):   # every copy's workspace written once
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
        spin_cycles = int(1e5 * args.steps * len(calls) * n_layers)  # covers the host enqueue of every call

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

        # per-kernel region: the same K steps with events between the library calls (groups of
        # `repeat` calls on distinct copies)
        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(n_layers)] for _ in calls]
               for _ in range(args.steps)]
        first = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(spin_cycles * repeat)
        first.record(stream)
        orders = [step_timed(i, evs[i]) for i in range(args.steps)]
        torch.cuda.synchronize()

    # per-call durations (ms), averaged over the steps: the interval since the previous event
    call_ms = {c: np.zeros(n_layers) for c in ("pack", "stage1", "stage2")}
    prev = first
    for i, ev in enumerate(evs):
        for c, unit in orders[i]:
            e = ev[calls.index(c)][unit[0]]
            call_ms[c][unit[0]] += prev.elapsed_time(e)
            prev = e
    for c in calls:
        call_ms[c] = call_ms[c] / (args.steps * repeat)

    # decode: the pack of the layer is not part of the step; timed beside it, on rotating copies
    if decode:
        spin = int(1e5 * max(8, args.steps) * REPEAT_SMALL)
        for li in range(n_layers):
            call_ms["pack"][li] = time_per_call(lambda i, li=li: pack(sets[i % copies][li]), max(8, args.steps),
                                                stream, spin, repeat)

    ms_per_step = total_ms / args.steps
    flop_step = sum(2 * L.M * L.n_out * L.n_in for L in layers)
    wbytes_step = sum(layer_bytes(L.n_in, L.n_out, L.r, isz) for L in layers)
    pbytes_step = sum(pack_bytes(L.n_in, L.n_out, isz) for L in layers)
    s2_work = sum(stage2_work(L, isz, decode) for L in layers)

    # a grouped stage-2 launch is timed once; each of its layers is shown with an equal share
    s2_share = np.zeros(n_layers)
    groups = []
    for unit in units:
        s2_share[unit] = call_ms["stage2"][unit[0]] / len(unit)
        if len(unit) > 1:
            groups.append(dict(layers=[layers[j].name for j in unit], entry="splr_linear_stage2_group",
                               stage2_us=round(call_ms["stage2"][unit[0]] * 1e3, 2)))
    per_layer = []
    for li, L in enumerate(layers):
        pb = pack_bytes(L.n_in, L.n_out, isz)
        lin = call_ms["stage1"][li] + s2_share[li]
        per_layer.append(dict(
            layer=L.name, pack_us=round(call_ms["pack"][li] * 1e3, 2),
            pack_GBps=round(pb / (call_ms["pack"][li] * 1e-3) / 1e9, 1),
            stage1_us=round(call_ms["stage1"][li] * 1e3, 2), stage2_us=round(s2_share[li] * 1e3, 2),
            linear_dense_equiv_TFLOPs=round(2 * L.M * L.n_out * L.n_in / (lin * 1e-3) / 1e12, 1),
            linear_weight_GBps=round(layer_bytes(L.n_in, L.n_out, L.r, isz) / (lin * 1e-3) / 1e9, 1)))

    # roofline of the kernel with the largest share of the step
    pack_s = call_ms["pack"].sum() * 1e-3 if not decode else 0.0
    s2_s = call_ms["stage2"].sum() * 1e-3
    wl = cfg.name
    if pack_s >= s2_s:
        ach = pbytes_step / pack_s / 1e9
        roofline = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                        frac=round(ach / PEAK_HBM_GBPS, 4), traffic=recorded_traffic("pack", wl),
                        kernel="prune24_pack_kernel", work="bytes read + written: R, packed values, metadata")
    elif decode:
        ach = s2_work / s2_s / 1e9
        roofline = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                        frac=round(ach / PEAK_HBM_GBPS, 4), traffic=recorded_traffic("decode", wl),
                        kernel="linear_decode_kernel" if dtype == "bf16" else "linear_f32_kernel",
                        work="bytes: packed values, metadata, U, X, T, Y")
    else:
        peak = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_TFLOPS
        ach = s2_work / s2_s / 1e12
        roofline = dict(bound="mfma", achieved=round(ach, 1), peak=peak, unit="TFLOP/s",
                        frac=round(ach / peak, 4), traffic=recorded_traffic("stage2", wl),
                        kernel=prefill_kernels(layers, units) if dtype == "bf16" else "linear_f32_kernel",
                        work="algorithmic FLOP: kept 2:4 products (M n_out n_in) + rank-r epilogue (2 M n_out r)",
                        dense_equiv_TFLOPs=round(flop_step / s2_s / 1e12, 1))

    if decode:
        value, unit = wbytes_step / (ms_per_step * 1e-3) / 1e9, "GB/s"
    else:
        value, unit = flop_step / (ms_per_step * 1e-3) / 1e12, "TFLOP/s"

    step_desc = ("splr_linear (stage 1 + stage 2) on every layer; the layer's prune24_pack is timed beside the "
                 "step (kernels.per_layer.pack_us)" if decode else
                 "for every layer: prune24_pack of its residual, then splr_linear (stage 1 + stage 2)"
                 + ("; stage 2 of " + ", ".join("+".join(g["layers"]) for g in groups)
                    + " as one grouped launch (splr_linear_stage2_group)" if groups else ""))
    out = dict(
        metric=METRIC, value=round(value, 2), unit=unit, n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms_per_step, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype=dtype, data="synthetic",
        config=dict(workload=f"{cfg.name}: {cfg.description}", tokens=cfg.M, rank=cfg.r,
                    layers=[f"{n}:{k}->{o}" for n, k, o in cfg.layers], step=step_desc,
                    launch="graph replay" if graphs else "stream, queue pre-filled", parallelism="single GPU",
                    copies_rotated=copies, per_kernel_repeat=repeat),
        roofline=roofline,
        kernels=dict(per_layer=per_layer, stage2_groups=groups,
                     pack_GBps=round(pbytes_step / (call_ms["pack"].sum() * 1e-3) / 1e9, 1),
                     linear_dense_equiv_TFLOPs=round(
                         flop_step / ((call_ms["stage1"].sum() + call_ms["stage2"].sum()) * 1e-3) / 1e12, 1),
                     linear_weight_GBps=round(
                         wbytes_step / ((call_ms["stage1"].sum() + call_ms["stage2"].sum()) * 1e-3) / 1e9, 1)),
        input_generation_s=round(gen_s, 1),
    )

    if not args.no_context:
        out["context"] = measure_context(layers, decode, tdt, stream, dev, args)

    if not args.no_next:
        out["next"] = measure_next(binding, inputs, layers, stream, dev, args, to_dev)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, layers, dtype, flop_step, wbytes_step, decode, args.cpu_rows)
    print(json.dumps(out), flush=True)


def time_per_call(issue, n, stream, spin_cycles, repeat=REPEAT_SMALL):
    """Average GPU time (ms) of one call: `issue(i)` enqueues call i on `stream` (the caller maps i to
    a rotating copy of its data); n groups of `repeat` calls, i = 0, 1, 2, ... in issue order,
    between two events behind a queue-filling spin."""
    import torch
    for i in range(3):
        issue(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(spin_cycles)
        e0.record(stream)
        for i in range(n * repeat):
            issue(i)
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (n * repeat)


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
    spin = int(1e5 * n * REPEAT_SMALL)
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


def measure_next(binding, inputs, layers, stream, dev, args, to_dev):
    """The parts built beyond the hot path, each timed per call on the first layer of the workload
    (outside the timed step), rotating over enough copies of that layer that no call finds its data
    in the Infinity Cache: the activation-aware pack (keys |R| |d|, d = column norms of the layer's
    activations), the 2:8 projection stored in the 2:4 layout, the fused residual + pack (R = W - U V
    formed in the kernel), the layer product with a bfloat16 Y (splr_linear_ex), stage 2 with S
    decompressed on chip and dense MFMA against the structured-sparse stage 2, and steps of the
    data-free alternating minimisation."""
    import torch
    n = max(8, args.steps // 2)
    spin = int(1e5 * n * REPEAT_SMALL)
    res = {}
    L = layers[0]
    isz = inputs.itemsize(L.dtype)
    tdt = torch.bfloat16 if L.dtype == "bf16" else torch.float32
    nc = max(2 * REPEAT_SMALL, math.ceil(MALL_DEFEAT_BYTES / pack_bytes(L.n_in, L.n_out, isz)) + 1)
    TR, TK = binding.tiles(L.n_out, L.n_in)
    R0, W0, X0, U0, V0 = to_dev(L.R), to_dev(L.W), to_dev(L.X), to_dev(L.U), to_dev(L.V)
    cp = [dict(R=R0.clone(), W=W0.clone(), X=X0.clone(), U=U0.clone(), V=V0.clone(),
               values=torch.empty((TR, TK, 64, 8), dtype=tdt, device=dev),
               meta=torch.empty(binding.meta_shape(L.n_out, L.n_in), dtype=torch.int32, device=dev),
               ws=binding.new_workspace(L.M, L.n_out, L.n_in, L.r, tdt, dev, stream)) for _ in range(nc)]
    d = torch.from_numpy(inputs.column_scales(L.X, L.dtype)).to(dev)

    def entry(name, bound, work, **kw):
        return dict(entry=name, bound=bound, work=work, layer=L.name, copies_rotated=nc, **kw)

    ms = time_per_call(lambda i: binding.prune24_pack_scaled(cp[i % nc]["R"], d, cp[i % nc]["values"],
                                                             cp[i % nc]["meta"], stream=stream), n, stream, spin)
    nbytes = pack_bytes(L.n_in, L.n_out, isz) + L.n_in * 4
    res["pack_scaled"] = entry("splr_prune24_pack_scaled", "hbm", "bytes: R + d + packed values + metadata",
                               us=round(ms * 1e3, 2), GBps=round(nbytes / (ms * 1e-3) / 1e9, 1),
                               frac_hbm=round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4))

    # N:M projection (2:8, the pages' post-fine-tuning pattern) stored in the 2:4 layout: HBM bound,
    # the same bytes as the 2:4 pack
    ms = time_per_call(lambda i: binding.prune_nm_pack(cp[i % nc]["R"], 2, 8, cp[i % nc]["values"],
                                                       cp[i % nc]["meta"], stream=stream), n, stream, spin)
    nbytes = pack_bytes(L.n_in, L.n_out, isz)
    res["pack_2_8"] = entry("splr_prune_nm_pack (n = 2, m = 8)", "hbm", "bytes: R + packed values + metadata",
                            us=round(ms * 1e3, 2), GBps=round(nbytes / (ms * 1e-3) / 1e9, 1),
                            frac_hbm=round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4))

    # fused residual + pack: vector-ALU bound (r fused multiply-adds per weight, binary32, not packed)
    ms = time_per_call(lambda i: binding.prune24_pack_residual(cp[i % nc]["W"], cp[i % nc]["U"], cp[i % nc]["V"],
                                                               cp[i % nc]["values"], cp[i % nc]["meta"],
                                                               stream=stream), n, stream, spin)
    nbytes = pack_bytes(L.n_in, L.n_out, isz) + (L.n_out + L.n_in) * L.r * isz
    tflops = 2 * L.n_out * L.n_in * L.r / (ms * 1e-3) / 1e12
    res["pack_residual"] = entry("splr_prune24_pack_residual", "alu",
                                 "2 n_out n_in r FLOP (the residual's fused multiply-adds); bytes W + U + V + "
                                 "packed values + metadata", peak_TFLOPs=PEAK_FP32_VALU_TFLOPS,
                                 us=round(ms * 1e3, 2), fp32_TFLOPs=round(tflops, 1),
                                 frac_alu=round(tflops / PEAK_FP32_VALU_TFLOPS, 4),
                                 GBps=round(nbytes / (ms * 1e-3) / 1e9, 1))

    # bfloat16 Y: the same layer product with the output rounded to bfloat16 (half the Y bytes)
    if L.dtype == "bf16":
        y16 = [torch.empty((L.M, L.n_out), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        ms = time_per_call(lambda i: binding.linear_ex(cp[i % nc]["X"], cp[i % nc]["values"], cp[i % nc]["meta"],
                                                       cp[i % nc]["U"], cp[i % nc]["V"], y_dtype=torch.bfloat16,
                                                       n_out=L.n_out, out=y16[i % 2], workspace=cp[i % nc]["ws"],
                                                       stream=stream), n, stream, spin)
        res["linear_bf16_y"] = entry("splr_linear_ex (y_dtype bfloat16)", "mfma",
                                     "dense-equivalent FLOP 2 M n_out n_in", us=round(ms * 1e3, 2),
                                     dense_equiv_TFLOPs=round(2 * L.M * L.n_out * L.n_in / (ms * 1e-3) / 1e12, 1))

        # the measured choice for the sparse product: stage 2 with the structured-sparse MFMA (what
        # splr_linear runs) against S decompressed to dense bfloat16 on chip + dense MFMA, on the same
        # first-stage output (stage 1 run once per copy beforehand)
        for c in cp:
            binding.linear_stage1(c["X"], c["V"], c["ws"], stream=stream)
        y32 = [torch.empty((L.M, L.n_out), dtype=torch.float32, device=dev) for _ in range(2)]
        choice = {}
        for kind, fn in (("smfmac", binding.linear_stage2), ("dense", binding.linear_stage2_dense)):
            ms = time_per_call(lambda i: fn(cp[i % nc]["X"], cp[i % nc]["values"], cp[i % nc]["meta"], cp[i % nc]["U"],
                                            cp[i % nc]["ws"], n_out=L.n_out, out=y32[i % 2], stream=stream),
                               n, stream, spin)
            choice[kind + "_us"] = round(ms * 1e3, 2)
            choice[kind + "_dense_equiv_TFLOPs"] = round(2 * L.M * L.n_out * L.n_in / (ms * 1e-3) / 1e12, 1)
        res["stage2_smfmac_vs_dense"] = entry(
            "splr_linear_stage2 against splr_linear_stage2_dense", "mfma",
            "dense-equivalent FLOP 2 M n_out n_in; the dense path issues twice the matrix-core instructions",
            **choice, dense_over_smfmac=round(choice["dense_us"] / choice["smfmac_us"], 3))
        del y32
    s0 = cp[0]

    # data-free alternating minimisation on the first layer: per-step time (untracked) and the
    # objective / layer error over a few steps (tracked)
    from sparse_rank_linear_prune24_amd import am
    if L.r > 0:
        steps = 10
        am.alternating_minimization(s0["W"], L.r, 2, track=False)  # warm-up (library initialisation)
        t = am.alternating_minimization(s0["W"], L.r, steps, track=False)
        steady = float(np.median(t["step_seconds"][2:]))  # steps 0 and 1: initial C_r(W), graph capture
        tracked = am.alternating_minimization(s0["W"], L.r, steps, X=s0["X"])
        wnorm = float(torch.linalg.norm(s0["W"].float()))
        res["am_loop"] = dict(layer=L.name, steps=steps, ms_per_step=round(steady * 1e3, 3),
                              ms_per_step_note="median host time of steps 2..9 (each step waits for the "
                                               "device once); steps 0-1 hold the initial C_r(W) and the "
                                               "graph capture",
                              first_steps_ms=[round(x * 1e3, 2) for x in t["step_seconds"][:2]],
                              est_80_steps_s=round(sum(t["step_seconds"][:2]) + steady * 78, 3),
                              rel_objective=[round(o / wnorm, 5) for o in tracked["objective"]],
                              layer_rel_error=[round(e, 5) for e in tracked["layer_rel_error"]],
                              step="splr_prune24_pack_residual + dense reconstruct of S + rank-r subspace "
                                   "iteration (torch matmul, splr_gram_f64 + splr_chol_rinv Cholesky QR, one "
                                   "host k x k eigen-solve), replayed as two HIP graphs per step")
    return res


def cpu_baseline(cfg, layers, dtype, flop_step, wbytes_step, decode, rows_arg):
    """The oracle, untuned, on this host's cores: the full pack of every layer plus the layer product
    on a sample of token rows, scaled to one step."""
    import oracle

    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    oracle.build(force=False)

    def run(row_div):
        """Pack of every layer, layer product on evenly spaced rows; seconds scaled to one step."""
        t_pack = t_lin = 0.0
        frac_rows = []
        for L in layers:
            t0 = time.perf_counter()
            v, m = oracle.prune24_pack(L.R, dtype)
            t_pack += time.perf_counter() - t0
            rows = rows_arg or max(1, min(L.M, int(4e9 / (L.n_out * L.n_in / 2) // 1)))
            rows = max(1, min(rows, L.M) // row_div)
            sel = np.linspace(0, L.M - 1, rows).astype(np.int64)
            t0 = time.perf_counter()
            oracle.linear(L.X, v, m, L.n_out, L.U, L.V, dtype, rows=sel)
            t_lin += (time.perf_counter() - t0) * (L.M / rows)
            frac_rows.append(f"{L.name}: {rows}/{L.M} rows")
        return t_pack, t_lin, frac_rows

    def rate(t_step):
        return (wbytes_step / t_step / 1e9, "GB/s") if decode else (flop_step / t_step / 1e12, "TFLOP/s")

    t_pack, t_lin, frac_rows = run(1)
    t_step = t_pack + t_lin
    value, unit = rate(t_step)
    # the small workloads also on one thread (the same OpenMP runtime as the oracle's), with a
    # sixteenth of the rows
    one_thread = None
    if cfg.name in ("C1", "C2", "C3"):
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        try:
            p1, l1, rows1 = run(16)
        finally:
            gomp.omp_set_num_threads(int(os.environ["OMP_NUM_THREADS"]))
        v1, _ = rate(p1 + l1)
        one_thread = dict(value=round(v1, 6), unit=unit, cores=1, step_s_equiv=round(p1 + l1, 3),
                          sample=f"full pack of every layer; layer product on {'; '.join(rows1)}")
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
                step_s_equiv=round(t_step, 3), pack_s=round(t_pack, 3), cpu=cpu,
                **({"one_thread": one_thread} if one_thread else {}))


if __name__ == "__main__":
    main()
