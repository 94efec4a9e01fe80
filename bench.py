"""Benchmark of the 2:4 + rank-r linear hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: for every layer of the
workload, the 2:4 projection + pack of the residual R = W - U V (splr_prune24_pack), then the layer
product Y = X S^T + (X V^T) U^T with the freshly packed S (splr_linear). Inputs are resident in
HBM before timing starts. Each step reads a different copy of the weights and activations when
one step's footprint is small, so repeated steps are not served from the 256 MB Infinity Cache.

Prints one JSON line. `value` is dense-equivalent TFLOP/s (2 M n_out n_in per layer) of the whole
step for the prefill workloads, or GB/s of the weight-side bytes (packed values, metadata, U, V)
for the decode workload. Per-call durations come from HIP events recorded on the benchmark stream
around every library call inside the timed loop.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C2] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "2:4+rank-r linear: dense-equiv TFLOP/s & HBM GB/s vs roofline, Llama3-8B shapes"
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3     # MI355X fp32 (vector / MFMA)
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E
MALL_DEFEAT_BYTES = 640 << 20  # > 2 x (256 MB Infinity Cache + 8 x 4 MB L2)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="C2", help="C1..C5 (default: C2, the prefill q_proj layer)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    p.add_argument("--cpu-rows", type=int, default=0, help="token rows of the oracle sample (0 = auto)")
    return p.parse_args()


def layer_bytes(n_in, n_out, r, itemsize):
    """Weight-side bytes one splr_linear call must read: packed values, metadata, U, V."""
    return n_out * n_in // 2 * itemsize + n_out * n_in // 8 + (n_out * r + r * n_in) * itemsize


def pack_bytes(n_in, n_out, itemsize):
    """Bytes splr_prune24_pack must move: read R, write values and metadata."""
    return n_out * n_in * itemsize + n_out * n_in // 2 * itemsize + n_out * n_in // 8


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the layer shards by output rows or input columns; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_rank_linear_prune24_amd import binding, configs, inputs

    cfg = configs.get(args.workload)
    dtype = cfg.dtype
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    isz = inputs.itemsize(dtype)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.lib()

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
            R = to_dev(L.R)
            ws_n = binding.workspace_bytes(L.M, L.n_out, L.n_in, L.r, tdt)
            s.append(dict(
                R=R, X=to_dev(L.X), U=to_dev(L.U), V=to_dev(L.V),
                values=torch.empty((*binding.tiles(L.n_out, L.n_in), 64, 8), dtype=tdt, device=dev),
                meta=torch.empty((*binding.tiles(L.n_out, L.n_in), 2, 16), dtype=torch.int32, device=dev),
                Y=torch.empty((L.M, L.n_out), dtype=torch.float32, device=dev),
                ws=torch.empty(max(ws_n, 256), dtype=torch.uint8, device=dev)))
        sets.append(s)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    n_layers = len(layers)

    def step(i, ev=None):
        s = sets[i % copies]
        if ev is not None:
            ev[0].record(stream)
        for li, d in enumerate(s):
            binding.prune24_pack(d["R"], d["values"], d["meta"], stream=stream)
            if ev is not None:
                ev[1 + li].record(stream)
        for li, d in enumerate(s):
            binding.linear(d["X"], d["values"], d["meta"], d["U"], d["V"], n_out=d["Y"].shape[1], out=d["Y"],
                           workspace=d["ws"], stream=stream)
            if ev is not None:
                ev[1 + n_layers + li].record(stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()

        # timed region 1: the steps alone
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(args.steps):
            step(i)
        end.record(stream)
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(end)

        # timed region 2: the same steps with an event after every library call
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(1 + 2 * n_layers)] for _ in range(args.steps)]
        for i in range(args.steps):
            step(i, evs[i])
        torch.cuda.synchronize()

    pack_ms = np.zeros(n_layers)
    lin_ms = np.zeros(n_layers)
    for ev in evs:
        for li in range(n_layers):
            pack_ms[li] += ev[li].elapsed_time(ev[1 + li]) if li == 0 else ev[li].elapsed_time(ev[1 + li])
            prev = ev[n_layers] if li == 0 else ev[n_layers + li]
            lin_ms[li] += prev.elapsed_time(ev[1 + n_layers + li])
    pack_ms /= args.steps
    lin_ms /= args.steps

    ms_per_step = total_ms / args.steps
    flop_step = sum(2 * L.M * L.n_out * L.n_in for L in layers)
    wbytes_step = sum(layer_bytes(L.n_in, L.n_out, L.r, isz) for L in layers)
    pbytes_step = sum(pack_bytes(L.n_in, L.n_out, isz) for L in layers)
    decode = cfg.M <= 64

    per_layer = []
    for li, L in enumerate(layers):
        fl = 2 * L.M * L.n_out * L.n_in
        wb = layer_bytes(L.n_in, L.n_out, L.r, isz)
        pb = pack_bytes(L.n_in, L.n_out, isz)
        per_layer.append(dict(
            layer=L.name, pack_us=round(pack_ms[li] * 1e3, 2), pack_GBps=round(pb / (pack_ms[li] * 1e-3) / 1e9, 1),
            linear_us=round(lin_ms[li] * 1e3, 2), linear_TFLOPs=round(fl / (lin_ms[li] * 1e-3) / 1e12, 1),
            linear_weight_GBps=round(wb / (lin_ms[li] * 1e-3) / 1e9, 1)))

    peak_mfma = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_TFLOPS
    lin_total_s = lin_ms.sum() * 1e-3
    if decode:
        value = wbytes_step / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        ach = wbytes_step / lin_total_s / 1e9
        roofline = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                        frac=round(ach / PEAK_HBM_GBPS, 4), traffic=None, kernel="splr_linear (decode)")
    else:
        value = flop_step / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        ach = flop_step / lin_total_s / 1e12
        roofline = dict(bound="mfma", achieved=round(ach, 1), peak=peak_mfma, unit="TFLOP/s",
                        frac=round(ach / peak_mfma, 4), traffic=None, kernel="splr_linear (prefill)")

    out = dict(
        metric=METRIC, value=round(value, 2), unit=unit, n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms_per_step, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype=dtype, data="synthetic",
        config=dict(workload=f"{cfg.name}: {cfg.description}", tokens=cfg.M, rank=cfg.r,
                    layers=[f"{n}:{k}->{o}" for n, k, o in cfg.layers], step="prune24_pack on every layer's "
                    "residual, then splr_linear on every layer", parallelism="single GPU", copies_rotated=copies),
        roofline=roofline,
        kernels=dict(per_layer=per_layer,
                     pack_GBps=round(pbytes_step / (pack_ms.sum() * 1e-3) / 1e9, 1),
                     pack_frac_hbm=round(pbytes_step / (pack_ms.sum() * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                     linear_TFLOPs=round(flop_step / lin_total_s / 1e12, 1),
                     linear_weight_GBps=round(wbytes_step / lin_total_s / 1e9, 1)),
        input_generation_s=round(gen_s, 1),
    )

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, layers, dtype, flop_step, wbytes_step, decode, args.cpu_rows)
    print(json.dumps(out), flush=True)


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
