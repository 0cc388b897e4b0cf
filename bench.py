"""Benchmark: effective TOPS of the fused W4A4 + low-rank linear on FLUX shapes.

One step = the FLUX-shaped MLP pair in MXFP4, every launch of the hot path:
  fc1: svdq_quantize_act + svdq_gemm (M=4608, K=3072 -> N=12288, r=32, GELU fused)
  fc2: svdq_quantize_act + svdq_gemm (M=4608, K=12288 -> N=3072, r=32)
on synthetic seeded inputs already resident in HBM (weights packed once before
timing, as at load time).  value = (2 M N K of fc1 + of fc2) per step / time.

Prints one JSON line.  `roofline` is the fc1 GEMM kernel (the dominant launch),
timed with HIP events around each of its launches inside the timed region.
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same workload.
With --workload mod_w4a16 the step is one W4A16 launch (svdq_gemm_w4a16: bf16
activations times INT4 weights, the memory-bound modulation projection) and
`roofline` is HBM-bound: algorithmic bytes (codes, scales, X, Y, bias) per
launch over its event-timed duration.
For the MXFP4 pair, `fused_mlp` times the same pair with fc1's GEMM quantizing
its output for fc2 in its epilogue (svdq_gemm_quant: three launches plus the
down-projection sum instead of four), same inputs, same step count.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TOPS of fused W4A4+low-rank linear, FLUX shapes; % of FP4 MFMA peak"
# MI355X dense MFMA peaks of the instruction each format runs on: FP4 (MXFP4),
# INT8 (INT4 codes), fp16 (NVFP4-style codes, dequantized in registers)
PEAK_TFLOPS = {"mxfp4": 10100.0, "int4": 5000.0, "nvfp4": 2500.0}
PAIRS = {
    "mlp_mxfp4": ("fc1_mxfp4", "fc2_mxfp4"),
    "mlp_int4": ("fc1_int4", "fc2_int4"),
    "mlp_nvfp4": ("fc1_nvfp4", "fc2_nvfp4"),
}
SINGLE = ("qkv", "lowm", "lora", "single")
W4A16 = ("mod_w4a16",)
HBM_PEAK_GBPS = 8000.0                                      # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="mlp_mxfp4", choices=list(PAIRS) + list(SINGLE) + list(W4A16))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="before the timed region, copy MIB mebibytes device to device once (a plain copy of "
                        "known size, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def layers_of(workload):
    import synth
    names = PAIRS.get(workload, (workload,))
    return [synth.CONFIGS[n] for n in names]


def gemm_source_hash() -> str:
    """Hash of the sources the GEMM kernels are compiled from."""
    h = hashlib.sha256()
    for name in ("gemm.hip", "common.h", "layout.h"):
        with open(os.path.join(ROOT, "w4a4_quantized_linear_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current GEMM source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        e = d.get(f"{workload}:{kernel}")
        if e and e.get("gemm_source_sha256_16") == gemm_source_hash():
            return e.get("bytes_per_launch")
    except (ValueError, OSError):
        return None
    return None


def gpu_leg(args):
    import numpy as np
    import torch

    import synth
    import w4a4_quantized_linear_amd as sq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    specs = layers_of(args.workload)
    layers, weights, inputs = [], [], []
    for i, spec in enumerate(specs):
        L = synth.draw_layer(spec)
        r = spec.rank + spec.lora_rank
        layer = sq.Layer(spec.fmt, spec.K, spec.N, r)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).to(dev)
        w = sq.pack_weight(layer, t(L["R"]), t(L["L1"]), t(L["L2"]), t(L["lam"]), t(L["b"]))
        layers.append(layer)
        weights.append(w)
        inputs.append(t(L["X"]) if i == 0 else None)
        del L
    M = specs[0].M
    ws = [torch.empty(sq.act_bytes(l, M), dtype=torch.uint8, device=dev) for l in layers]
    outs = [torch.empty((M, l.N), dtype=torch.bfloat16, device=dev) for l in layers]
    epis = [sq.EPI_LOWRANK | sq.EPI_BIAS | (sq.EPI_GELU if s.gelu else 0) for s in specs]
    torch.cuda.synchronize()

    n = len(layers)

    def step(ev=None):
        x = inputs[0]
        for i in range(n):
            if ev is not None:
                ev[i][0].record()
            sq.quantize_act(layers[i], weights[i], x, out=ws[i])
            if ev is not None:
                ev[i][1].record()
            sq.gemm(layers[i], weights[i], ws[i], M, epis[i], out=outs[i])
            if ev is not None:
                ev[i][2].record()
            x = outs[i].view(torch.int16)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(args.steps):
        step(evs[k])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(stop)

    quant_us = [sum(evs[k][i][0].elapsed_time(evs[k][i][1]) for k in range(args.steps)) * 1e3 / args.steps
                for i in range(n)]
    gemm_us = [sum(evs[k][i][1].elapsed_time(evs[k][i][2]) for k in range(args.steps)) * 1e3 / args.steps
               for i in range(n)]
    flops = [2.0 * M * s.N * s.K for s in specs]
    ms_per_step = wall * 1e3 / args.steps
    value = sum(flops) / (ms_per_step * 1e-3) / 1e12

    # dominant kernel: the GEMM with the most work (fc1 for the MLP pair)
    i_dom = max(range(n), key=lambda i: gemm_us[i])
    fmt = specs[i_dom].fmt
    achieved = flops[i_dom] / (gemm_us[i_dom] * 1e-6) / 1e12
    peak = PEAK_TFLOPS[fmt]
    kname = f"gemm_{fmt}_{specs[i_dom].name}"
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_for(kname, args.workload),
                "kernel": kname, "flops_per_launch": flops[i_dom], "avg_launch_us": round(gemm_us[i_dom], 2)}
    breakdown = {}
    for i, s in enumerate(specs):
        hbm_q = 2 * M * s.K + M * s.K // 2 + M * s.K // 32 + 4 * M * layers[i].rank + 2 * s.K * layers[i].rank
        breakdown[s.name] = {
            "quantize_us": round(quant_us[i], 2),
            "quantize_GBps": round(hbm_q / (quant_us[i] * 1e-6) / 1e9, 1),
            "gemm_us": round(gemm_us[i], 2),
            "gemm_TFLOPs": round(flops[i] / (gemm_us[i] * 1e-6) / 1e12, 1),
            "linear_TOPS": round(flops[i] / ((gemm_us[i] + quant_us[i]) * 1e-6) / 1e12, 1),
        }
    fused = None
    if args.workload == "mlp_mxfp4":
        fused = fused_pair(args, sq, torch, layers, weights, inputs[0], ws, outs, epis, M, sum(flops))
    elif args.workload == "qkv":
        fused = fused_qkv(args, sq, synth, torch, np, layers[0], weights[0], inputs[0], ws[0], outs[0], epis[0], M,
                          flops[0])
    return dict(value=value, ms_per_step=ms_per_step, gpu_ms_per_step=gpu_ms / args.steps, roofline=roofline,
                breakdown=breakdown, specs=specs, fmt=specs[0].fmt, fused=fused)


def w4a16_bytes(M, K, N):
    """Algorithmic HBM bytes of one W4A16 launch: INT4 codes and fp16 group
    scales of W, bf16 X, bf16 Y and bf16 bias, each read or written once."""
    return N * K // 2 + N * (K // 64) * 2 + M * K * 2 + M * N * 2 + N * 2


def gpu_leg_w4a16(args):
    import numpy as np
    import torch

    import synth
    import w4a4_quantized_linear_amd as sq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = synth.CONFIGS[args.workload]
    d = synth.draw_w4a16(spec)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).to(dev)
    layer = sq.Layer("int4", spec.K, spec.N, 0)
    w0 = sq.pack_weight(layer, t(d["W"]), None, None, t(np.ones(spec.K, np.float32)), t(d["b"]))
    # The layer's weights are a few tens of MB, well inside the 256 MB last-level
    # cache; consecutive launches rotate over copies spanning 1 GiB, so every
    # launch streams its weights from HBM as a model's successive layers would.
    copies = max(1, -(-(1 << 30) // w0.numel()))
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    x = t(d["X"])
    out = torch.empty((spec.M, spec.N), dtype=torch.bfloat16, device=dev)
    del d
    M = spec.M
    it = [0]

    def step():
        w = ws[it[0] % copies]
        it[0] += 1
        sq.gemm_w4a16(layer, w, x, sq.EPI_BIAS, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # one launch per step, back to back on the current stream: the kernel is a
    # few microseconds long, so events around each launch would time mostly
    # themselves; the events bracket the whole run instead
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    launch_us = start.elapsed_time(stop) * 1e3 / args.steps
    flops = 2.0 * M * spec.N * spec.K
    nbytes = w4a16_bytes(M, spec.K, spec.N)
    achieved = nbytes / (launch_us * 1e-6) / 1e9
    kname = f"gemm_w4a16_{spec.name}"
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_for(kname, args.workload),
                "kernel": kname, "bytes_per_launch": nbytes, "avg_launch_us": round(launch_us, 2),
                "weight_copies": copies}
    breakdown = {spec.name: {"gemm_us": round(launch_us, 2), "GBps": round(achieved, 1),
                             "gemm_TFLOPs": round(flops / (launch_us * 1e-6) / 1e12, 3)}}
    return dict(value=flops / (ms_per_step * 1e-3) / 1e12, ms_per_step=ms_per_step, gpu_ms_per_step=None,
                roofline=roofline, breakdown=breakdown, specs=[spec], fmt="bf16", fused=None)


def cpu_baseline_w4a16(spec):
    """The W4A16 oracle, as it stands, on the whole workload (quantize W, fp64
    product): about 10 s of host time."""
    import synth
    from oracle import w4a16 as W

    d = synth.draw_w4a16(spec)
    threads = _blas_threads()
    t0 = time.perf_counter()
    W.forward(d["X"], d["W"], d["b"])
    secs = time.perf_counter() - t0
    return {"value": round(2.0 * spec.M * spec.N * spec.K / secs / 1e12, 6), "unit": "TOPS", "cores": threads,
            "kind": "oracle",
            "sample": f"{spec.name}: all {spec.M} tokens x {spec.N} outputs (K={spec.K}); {secs:.1f} s of oracle "
                      "time (INT4 weight quantization, fp64 product, bias); quantization is single-threaded "
                      f"numpy, the product uses {threads} BLAS threads"}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover - optional dependency
        return 1


def fused_qkv(args, sq, synth, torch, np, layer, w, x, ws, out, epi, M, flops):
    """The QKV layer with the Q/K RMS normalization and rotary embedding in the
    GEMM epilogue (svdq_gemm_qkv), same inputs and step count."""
    E = synth.draw_qkv_extras(M)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
    wq, wk, cs, sn = t(E["norm_q"]), t(E["norm_k"]), t(E["cos"]), t(E["sin"])

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        sq.quantize_act(layer, w, x, out=ws)
        if ev is not None:
            ev[1].record()
        sq.gemm_qkv(layer, w, ws, M, epi, wq, wk, E["eps"], cs, sn, out=out)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    seg = [sum(evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)) * 1e3 / args.steps
           for i in range(2)]
    return {"value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TOPS", "ms_per_step": round(ms, 4),
            "quantize_us": round(seg[0], 2), "gemm_qkv_us": round(seg[1], 2),
            "launches": "quantize_act; gemm_qkv (GEMM with Q/K RMS norm and rotary embedding in the epilogue)"}


def fused_pair(args, sq, torch, layers, weights, x, ws, outs, epis, M, flops):
    """The MLP pair with fc1's output quantized for fc2 inside fc1's GEMM."""
    def step(ev=None):
        if ev is not None:
            ev[0].record()
        sq.quantize_act(layers[0], weights[0], x, out=ws[0])
        if ev is not None:
            ev[1].record()
        sq.gemm_quant(layers[0], weights[0], ws[0], M, epis[0], layers[1], weights[1], out=ws[1])
        if ev is not None:
            ev[2].record()
        sq.gemm(layers[1], weights[1], ws[1], M, epis[1], out=outs[1])
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    seg = [sum(evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)) * 1e3 / args.steps
           for i in range(3)]
    return {"value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TOPS", "ms_per_step": round(ms, 4),
            "fc1_quantize_us": round(seg[0], 2), "fc1_gemm_quant_us": round(seg[1], 2),
            "fc2_gemm_us": round(seg[2], 2),
            "launches": "fc1 quantize_act; fc1 gemm_quant (GEMM + fc2 quantize in the epilogue, then the "
                        "down-projection sum); fc2 gemm"}


def cpu_baseline(specs, budget_rows=2048):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    `budget_rows` tokens of each layer against 1/2 (K <= 4096) or 1/8 of the
    output columns (about 10 s of host time), scaled to effective TOPS of the
    sampled work."""
    import numpy as np

    import synth
    from oracle import layer as Ly

    threads = _blas_threads()
    work, secs, parts = 0.0, 0.0, []
    for spec in specs:
        L = synth.draw_layer(spec)
        r = spec.rank + spec.lora_rank
        rows = np.arange(min(budget_rows, spec.M))
        ncols = max(16, spec.N // (2 if spec.K <= 4096 else 8))
        cols = np.arange(ncols)
        t0 = time.perf_counter()
        Ly.forward_rows(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], spec.fmt, rows, cols,
                        gelu_act=spec.gelu)
        secs += time.perf_counter() - t0
        work += 2.0 * rows.size * ncols * spec.K
        parts.append(f"{spec.name}: {rows.size} tokens x {ncols} outputs (K={spec.K}, r={r})")
        del L
    return {"value": round(work / secs / 1e12, 6), "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "sample": "; ".join(parts) + f"; {secs:.1f} s of oracle time (quantize both operands, fp64 product, "
                      "low-rank branch, bias, GELU); quantization is single-threaded numpy, the product uses "
                      f"{threads} BLAS threads"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the layer runs on "
              "a single GPU (token-parallel sharding needs no collective, so N GPUs are N copies of "
              "this measurement).", file=sys.stderr)
        sys.exit(2)
    w4a16 = args.workload in W4A16
    r = gpu_leg_w4a16(args) if w4a16 else gpu_leg(args)
    specs = r["specs"]
    cfg = {"workload": args.workload, "layers": [
        {"name": s.name, "M": s.M, "K": s.K, "N": s.N, "rank": s.rank + s.lora_rank, "fmt": s.fmt,
         "epilogue": "bias" if w4a16 else "lowrank+bias" + ("+gelu" if s.gelu else "")} for s in specs],
        "output": "bf16", "weights": "packed once before timing"}
    if w4a16:
        cfg["activations"] = "bf16 (W4A16)"
    line = {
        "metric": METRIC, "value": round(r["value"], 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": r["fmt"], "data": "synthetic",
        "config": cfg, "roofline": r["roofline"], "breakdown": r["breakdown"],
    }
    if r["gpu_ms_per_step"] is not None:
        line["gpu_ms_per_step"] = round(r["gpu_ms_per_step"], 4)
    if r["fused"] is not None:
        line["fused_mlp" if args.workload == "mlp_mxfp4" else "fused_qkv"] = r["fused"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_w4a16(specs[0]) if w4a16 else cpu_baseline(specs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
