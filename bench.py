"""Benchmark: effective TOPS of the fused W4A4 + low-rank linear on FLUX shapes.

One step = the FLUX-shaped MLP pair in MXFP4, every launch of the hot path:
  fc1: svdq_quantize_act + svdq_gemm (M=4608, K=3072 -> N=12288, r=32, GELU fused)
  fc2: svdq_quantize_act + svdq_gemm (M=4608, K=12288 -> N=3072, r=32)
on synthetic seeded inputs already resident in HBM (weights packed once before
timing, as at load time).  value = (2 M N K of fc1 + of fc2) per step / time.

Prints one JSON line.  `roofline` is the fc1 GEMM kernel (the dominant launch),
timed with HIP events around its launches in every --roofline-every-th step of
the timed region (the only markers there; each marker adds a small gap to the
stream); `breakdown` times every launch with events in a second, untimed pass.  Before the warmup steps the same steps run untimed for
--settle-ms so that the shader clock has left its idle level.
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same workload.
With --workload mod_w4a16 the step is one W4A16 launch (svdq_gemm_w4a16: bf16
activations times INT4 weights, the memory-bound modulation projection) and
`roofline` is HBM-bound: algorithmic bytes (codes, scales, X, Y, bias) per
launch over its event-timed duration.
For the MXFP4 and INT4 pairs, `fused_mlp` times the same pair with fc1's GEMM quantizing
its output for fc2 in its epilogue (svdq_gemm_quant: three calls instead of four), same
inputs and step count, with no event inside its timed steps either (its per-launch
times come from a second pass); `fused_qkv` likewise for svdq_gemm_qkv.  With
--workload qkv, `lowrank_ablation` times the layer's 4-bit branch alone, that
branch with the low-rank branch as separate bf16 library GEMMs, and the fused
layer (the comparison of the SVDQuant notes page, section 4.3, Fig. 6(a)).

Operands (--operands): "calibrated" (default) converts each workload's dense
seeded draw the way the SVDQuant notes page, section 4.2, makes a layer
(smoothing factors from the data, SVD of the smoothed weight, residual), with
w4a4_quantized_linear_amd.convert on the host before timing; the MLP pair's
second layer is calibrated on the dense MLP's hidden activation
GELU(X W1 + b1).  "drawn" takes synth.draw_layer's look-alike operands.

`cold` repeats the timed loop over three or more copies of every operand,
workspace and output (more bytes than the 256 MB last-level cache), so each
step reads its operands from HBM; `repeats` gives the median of five more hot
runs of the same loop; `clock` is the shader clock level the driver's sysfs file
(pp_dpm_sclk) marks as current before and after.
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
    p.add_argument("--fmt", choices=["mxfp4", "int4", "nvfp4"], default=None,
                   help="4-bit format of every layer of the workload (default: the workload's own)")
    p.add_argument("--operands", default="calibrated", choices=["calibrated", "drawn"],
                   help="layer operands: converted from the dense draw (default) or drawn look-alikes")
    p.add_argument("--no-cold", action="store_true", help="skip the cold (operand-rotating) timing")
    p.add_argument("--no-ablation", action="store_true",
                   help="qkv: skip the fused / unfused low-rank branch timing")
    p.add_argument("--roofline-every", type=int, default=5, metavar="N",
                   help="events around the roofline GEMM in every N-th timed step (default 5)")
    p.add_argument("--settle-ms", type=float, default=300.0,
                   help="run untimed steps for this long before the warmup, so the shader clock has ramped up")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="before the timed region, copy MIB mebibytes device to device once (a plain copy of "
                        "known size, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    p.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                   help="no benchmark: summarize rocprofv3 --pmc output directories of this script's runs "
                        "(a markdown table per kernel role on stdout)")
    p.add_argument("--summarize-trace", metavar="DIR",
                   help="no benchmark: launch durations per kernel role from a rocprofv3 --kernel-trace output "
                        "directory of this script's runs (markdown on stdout)")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no benchmark: HBM bytes per launch from a FETCH_SIZE and a WRITE_SIZE run made with "
                        "--copy-calibration; prints the table and rewrites profiles/traffic.json")
    return p.parse_args()


# ---- rocprofv3 counter summaries (host only) ----

def _counter_rows(d):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "*counter_collection.csv"))):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _short(name):
    name = name.replace("void ", "").replace("svdq::", "")
    return name[:name.index("(")] if "(" in name else name


def _dispatch_roles(rows):
    """{dispatch id: role}.  GEMM launches are named by their kernel; an
    activation quantize or down-projection sum belongs to the next GEMM
    launched after it (bench.py runs each layer's launches back to back),
    except a sum launched right after a GEMM, which finishes that GEMM's
    fused quantization of the next layer's input."""
    order = {}
    for r in rows:
        order.setdefault(int(r["Dispatch_Id"]), _short(r["Kernel_Name"]))
    roles, pending, prev = {}, [], ""
    for did in sorted(order):
        k = order[did]
        if k.startswith("gemm_"):
            roles[did] = k
            for p, pk in pending:
                roles[p] = f"{pk} -> {k}"
            pending = []
        elif k.startswith("reduce_down_kernel") and prev.startswith("gemm_"):
            roles[did] = f"{k} <- {prev}"
        elif k.startswith(("quantize_act_kernel", "reduce_down_kernel")):
            pending.append((did, k))
        prev = k
    return roles


def _per_role(rows, counters):
    import collections
    roles = _dispatch_roles(rows)
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    n = collections.defaultdict(set)
    for r in rows:
        did = int(r["Dispatch_Id"])
        if did not in roles or r["Counter_Name"] not in counters:
            continue
        acc[roles[did]][r["Counter_Name"]] += float(r["Counter_Value"])
        n[roles[did]].add(did)
    return {k: {c: v / len(n[k]) for c, v in cs.items()} for k, cs in acc.items()}, {k: len(v) for k, v in n.items()}


def summarize_counters(dirs):
    """Mean per launch of every counter, and the derived figures: cycles =
    GRBM_GUI_ACTIVE / 8 (the counter sums the 8 XCDs); MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / cycles; VALU issue = SQ_INSTS_VALU /
    256 CUs / cycles (a CU issues at most one wave64 VALU instruction per
    cycle); LDS conflicts = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; waiting =
    SQ_WAIT_ANY / SQ_WAVE_CYCLES."""
    merged, counts = {}, {}
    for d in dirs:
        rows = _counter_rows(d)
        names = {r["Counter_Name"] for r in rows}
        per, cnt = _per_role(rows, names)
        for k, cs in per.items():
            merged.setdefault(k, {}).update(cs)
            counts[k] = max(counts.get(k, 0), cnt[k])
    print("| kernel (launches) | cycles | MFMA busy | VALU issue | VALU / MFMA instr | LDS conflict | waiting |")
    print("|---|---|---|---|---|---|---|")
    for k in sorted(merged):
        c = merged[k]
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / 8
        f = lambda v: "-" if v is None else f"{v:.1%}"
        mb = c["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / cyc if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in c else None
        vi = c["SQ_INSTS_VALU"] / 256 / cyc if cyc and "SQ_INSTS_VALU" in c else None
        vpm = (f"{c['SQ_INSTS_VALU'] / c['SQ_INSTS_MFMA']:.1f}" if c.get("SQ_INSTS_MFMA") else "-")
        lc = (c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"] if c.get("SQ_LDS_IDX_ACTIVE") else None)
        wt = (c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"] if c.get("SQ_WAVE_CYCLES") else None)
        print(f"| `{k}` ({counts[k]}) | {cyc:.0f} | {f(mb)} | {f(vi)} | {vpm} | {f(lc)} | {f(wt)} |")
    print()
    print("Raw means per launch:")
    for k in sorted(merged):
        print(f"- `{k}`: " + ", ".join(f"{c} {v:.0f}" for c, v in sorted(merged[k].items())))


def summarize_trace(d):
    """Mean, min and max duration per kernel role over every launch of a
    kernel-trace run (settle, warmup, timed and breakdown passes alike)."""
    import csv
    import glob
    import statistics
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "*kernel_trace.csv"))):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    roles = _dispatch_roles(rows)
    dur = {}
    for r in rows:
        did = int(r["Dispatch_Id"])
        if did in roles:
            dur.setdefault(roles[did], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("| kernel role | launches | mean us | median us | min us | max us |")
    print("|---|---|---|---|---|---|")
    for k in sorted(dur):
        v = dur[k]
        print(f"| `{k}` | {len(v)} | {statistics.mean(v):.1f} | {statistics.median(v):.1f} | {min(v):.1f} | "
              f"{max(v):.1f} |")


def traffic_from(fetch_dir, write_dir):
    """Read and written HBM bytes per launch of the pair's kernels, scaled by
    what the same counters read for the 256 MiB calibration copy (the largest
    __amd_rocclr_copyBuffer launch)."""
    res = {}
    for which, d in (("fetch", fetch_dir), ("write", write_dir)):
        rows = _counter_rows(d)
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]
                  and int(r["Grid_Size"]) == max(int(x["Grid_Size"]) for x in rows if "copyBuffer" in x["Kernel_Name"])]
        scale = (256 * 1024) / copies[-1]
        per, cnt = _per_role(rows, {"FETCH_SIZE", "WRITE_SIZE"})
        for k, cs in per.items():
            v = next(iter(cs.values()))
            res.setdefault(k, {})[which] = (v, scale, cnt[k])
    print("| kernel (launches) | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB | written MB | total MB |")
    print("|---|---|---|---|---|---|")
    out = {}
    for k in sorted(res):
        (fv, fs, n), (wv, ws, _) = res[k]["fetch"], res[k]["write"]
        rb, wb = fv * fs * 1024, wv * ws * 1024
        print(f"| `{k}` ({n}) | {fv:.0f} | {wv:.0f} | {rb / 1e6:.1f} | {wb / 1e6:.1f} | {(rb + wb) / 1e6:.1f} |")
        out[k] = {"fetch_kib_counter": round(fv, 1), "write_kib_counter": round(wv, 1), "fetch_scale": round(fs, 4),
                  "write_scale": round(ws, 4), "read_bytes": int(rb), "write_bytes": int(wb),
                  "bytes_per_launch": int(rb + wb), "launches": n}
    print(f"\nscales: FETCH_SIZE x{res[next(iter(res))]['fetch'][1]:.4f}, WRITE_SIZE x{res[next(iter(res))]['write'][1]:.4f}")
    return out


def layers_of(workload, fmt=None):
    import dataclasses
    import synth
    names = PAIRS.get(workload, (workload,))
    specs = [synth.CONFIGS[n] for n in names]
    return [dataclasses.replace(s, fmt=fmt) for s in specs] if fmt else specs


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


def _bits(t):
    """uint16 numpy view of a bf16 CPU tensor."""
    import numpy as np
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _bf16(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def calibrated_operands(spec):
    """The layer converted from its dense seeded draw (host, float64): smoothing
    factors from the activations it is calibrated on, SVD of the smoothed
    weight, bf16 factors, fp32 residual.  The second layer of the MLP pair is
    calibrated on GELU(X W1 + b1) of the dense first layer (bf16), which is also
    its input in the CPU baseline.  Cached under $TMPDIR by workload and seed."""
    import tempfile

    import numpy as np
    import torch

    import synth
    from w4a4_quantized_linear_amd import convert

    base = spec.name.split("_")[0] if spec.name.startswith(("fc1_", "fc2_")) else spec.name
    cdir = os.path.join(tempfile.gettempdir(), "svdq_bench_calib")
    path = os.path.join(cdir, f"{base}_M{spec.M}_K{spec.K}_N{spec.N}_r{spec.rank}_l{spec.lora_rank}.npz")
    if os.path.exists(path):
        try:
            with np.load(path) as z:
                return {k: z[k] for k in z.files}
        except (OSError, ValueError):
            pass
    raw = synth.draw_raw(spec)
    if spec.name.startswith("fc2_"):
        raw1 = synth.draw_raw(synth.CONFIGS[spec.name.replace("fc2_", "fc1_")])
        y = _bf16(raw1["X"]).double() @ _bf16(raw1["W"]).double() + _bf16(raw1["b"]).double()
        X = _bits((0.5 * y * (1.0 + torch.erf(y * 0.7071067811865476))).to(torch.bfloat16))
        del raw1, y
    else:
        X = raw["X"]
    adapter = (_bf16(raw["A"]), _bf16(raw["B"])) if spec.lora_rank else None
    c = convert.convert_linear(_bf16(X), _bf16(raw["W"]).t(), spec.rank, _bf16(raw["b"]), adapter)
    out = {"X": X, "lam": c["lam"].numpy(), "L1": _bits(c["L1"]), "L2": _bits(c["L2"]), "R": c["R"].numpy(),
           "b": _bits(c["b"])}
    try:
        os.makedirs(cdir, exist_ok=True)
        np.savez(path + ".tmp.npz", **out)
        os.replace(path + ".tmp.npz", path)
    except OSError:
        pass
    return out


def layer_operands(specs, kind):
    import synth
    return [calibrated_operands(s) if kind == "calibrated" else synth.draw_layer(s) for s in specs]


def gpu_leg(args, ops):
    import numpy as np
    import torch

    import synth
    import w4a4_quantized_linear_amd as sq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    specs = layers_of(args.workload, args.fmt)
    layers, weights, inputs = [], [], []
    for i, spec in enumerate(specs):
        L = ops[i]
        r = spec.rank + spec.lora_rank
        layer = sq.Layer(spec.fmt, spec.K, spec.N, r)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).to(dev)
        w = sq.pack_weight(layer, t(L["R"]), t(L["L1"]), t(L["L2"]), t(L["lam"]), t(L["b"]))
        layers.append(layer)
        weights.append(w)
        inputs.append(t(L["X"]) if i == 0 else None)
    M = specs[0].M
    ws = [torch.empty(sq.act_bytes(l, M), dtype=torch.uint8, device=dev) for l in layers]
    outs = [torch.empty((M, l.N), dtype=torch.bfloat16, device=dev) for l in layers]
    epis = [sq.EPI_LOWRANK | sq.EPI_BIAS | (sq.EPI_GELU if s.gelu else 0) for s in specs]
    torch.cuda.synchronize()

    n = len(layers)

    # The roofline kernel: the first layer's GEMM (fc1 of the MLP pair, whose
    # GELU epilogue makes it the longest launch).
    i_dom = 0

    def step(ev=None, opset=None, dom_ev=None):
        """One pass of the hot path.  ev: events around every launch; dom_ev: a
        pair of events around the roofline GEMM only (fewer markers in the
        timed region)."""
        wts, x, wss, ots = opset if opset is not None else (weights, inputs[0], ws, outs)
        for i in range(n):
            if ev is not None:
                ev[i][0].record()
            sq.quantize_act(layers[i], wts[i], x, out=wss[i])
            if ev is not None:
                ev[i][1].record()
            if dom_ev is not None and i == i_dom:
                dom_ev[0].record()
            sq.gemm(layers[i], wts[i], wss[i], M, epis[i], out=ots[i])
            if dom_ev is not None and i == i_dom:
                dom_ev[1].record()
            if ev is not None:
                ev[i][2].record()
            x = ots[i].view(torch.int16)

    # Clock settling: the shader clock ramps up over the first ~0.1 s of load,
    # so the same steps run untimed for at least `settle_ms` before the warmup.
    settle_steps, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms and settle_steps < 5000:
        step()
        settle_steps += 1
        if settle_steps % 16 == 0:
            torch.cuda.synchronize()
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

    # Timed region: exactly `steps` steps; the only markers are a pair of events
    # around the roofline GEMM in every `roofline_every`-th step (each marker
    # adds a gap to the stream, so fewer of them keep the step time clean).
    every = max(1, args.roofline_every)
    sampled = list(range(0, args.steps, every))
    dom = {k: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for k in sampled}
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(args.steps):
        step(dom_ev=dom.get(k))
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(stop)
    dom_us = sum(dom[k][0].elapsed_time(dom[k][1]) for k in sampled) * 1e3 / len(sampled)
    flops = [2.0 * M * s.N * s.K for s in specs]
    ms_per_step = wall * 1e3 / args.steps
    value = sum(flops) / (ms_per_step * 1e-3) / 1e12

    # Per-launch breakdown: the same steps again after the timed region, with
    # events around every launch.
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    quant_us = [sum(evs[k][i][0].elapsed_time(evs[k][i][1]) for k in range(args.steps)) * 1e3 / args.steps
                for i in range(n)]
    gemm_us = [sum(evs[k][i][1].elapsed_time(evs[k][i][2]) for k in range(args.steps)) * 1e3 / args.steps
               for i in range(n)]
    fmt = specs[i_dom].fmt
    achieved = flops[i_dom] / (dom_us * 1e-6) / 1e12
    peak = PEAK_TFLOPS[fmt]
    kname = f"gemm_{fmt}_{specs[i_dom].name}"
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_for(kname, args.workload),
                "kernel": kname, "flops_per_launch": flops[i_dom], "avg_launch_us": round(dom_us, 2),
                "launches_timed": len(sampled)}
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
    repeats = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for k in range(args.steps):
            step()
        b.record()
        torch.cuda.synchronize()
        repeats.append(a.elapsed_time(b) / args.steps)
    rep = sorted(repeats)
    repeat_info = {"ms_per_step": [round(x, 4) for x in repeats], "median_ms_per_step": round(rep[2], 4),
                   "median_value": round(sum(flops) / (rep[2] * 1e-3) / 1e12, 2)}
    cold = None if args.no_cold else cold_pair(args, torch, step, layers, weights, inputs[0], ws, outs,
                                                sum(flops), gemm_us, i_dom)
    fused = None
    if len(layers) == 2 and layers[0].fmt == layers[1].fmt and layers[0].fmt in ("mxfp4", "int4"):
        fused = fused_pair(args, sq, torch, layers, weights, inputs[0], ws, outs, epis, M, sum(flops))
    elif args.workload == "qkv":
        fused = fused_qkv(args, sq, synth, torch, np, layers[0], weights[0], inputs[0], ws[0], outs[0], epis[0], M,
                          flops[0])
    ablation = None
    if args.workload == "qkv" and not args.no_ablation:
        ablation = lowrank_ablation(sq, torch, np, ops[0], layers[0], weights[0], inputs[0], ws[0], outs[0],
                                    epis[0], M)
    return dict(value=value, ms_per_step=ms_per_step, gpu_ms_per_step=gpu_ms / args.steps, roofline=roofline,
                breakdown=breakdown, specs=specs, fmt=specs[0].fmt, fused=fused, repeats=repeat_info, cold=cold,
                settle_steps=settle_steps, ablation=ablation)


def lowrank_ablation(sq, torch, np, L, layer, w, x, ws, out, epi, M):
    """What the low-rank branch costs fused, as the layer runs (the down
    projection inside the activation quantize, the up projection in the GEMM's
    accumulators), against run as separate kernels after the 4-bit branch: the
    comparison of the SVDQuant notes page, section 4.3 (Fig. 6(a)), on the QKV
    projection.  Three timings of the same layer: the 4-bit branch alone (a
    rank-0 pack of the same residual: no D, no low-rank MFMAs); that branch
    followed by a bf16 down projection D = X (Lambda^-1 L1) and an up projection
    Y += D L2 as library GEMMs (torch.matmul and addmm_), which read X again and
    Y twice; and the fused layer.  A timing ablation: the library never runs the
    unfused branch."""
    dev = x.device
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).to(dev)
    layer0 = sq.Layer(layer.fmt, layer.K, layer.N, 0)
    w0 = sq.pack_weight(layer0, t(L["R"]), None, None, t(L["lam"]), t(L["b"]))
    ws0 = torch.empty(sq.act_bytes(layer0, M), dtype=torch.uint8, device=dev)
    l1 = torch.from_numpy((L["L1"].astype(np.uint32) << 16).view(np.float32)).to(dev)
    l1s = (l1 / t(L["lam"])[:, None]).to(torch.bfloat16).contiguous()      # Lambda^-1 L1, K x r
    l2 = t(L["L2"]).view(torch.bfloat16).contiguous()                        # r x N
    xb = x.view(torch.bfloat16)
    d = torch.empty((M, layer.rank), dtype=torch.bfloat16, device=dev)
    y0 = torch.empty_like(out)
    epi0 = epi & ~sq.EPI_LOWRANK

    def fourbit():
        sq.quantize_act(layer0, w0, x, out=ws0)
        sq.gemm(layer0, w0, ws0, M, epi0, out=y0)

    def unfused():
        fourbit()
        torch.matmul(xb, l1s, out=d)
        y0.addmm_(d, l2)

    def fused():
        sq.quantize_act(layer, w, x, out=ws)
        sq.gemm(layer, w, ws, M, epi, out=out)

    variants = {"fourbit": fourbit, "unfused": unfused, "fused": fused}
    for f in variants.values():
        for _ in range(10):
            f()
    torch.cuda.synchronize()
    res = {k: [] for k in variants}
    for _ in range(3):
        for k, f in variants.items():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(20):
                f()
            b.record()
            torch.cuda.synchronize()
            res[k].append(a.elapsed_time(b) * 1e3 / 20)
    us = {k: sorted(v)[1] for k, v in res.items()}
    unfused()
    fused()
    torch.cuda.synchronize()
    yf, yu = out.float(), y0.float()
    rel = float((yu - yf).abs().max() / yf.pow(2).mean().sqrt())
    return {"fourbit_us": round(us["fourbit"], 2), "unfused_us": round(us["unfused"], 2),
            "fused_us": round(us["fused"], 2),
            "unfused_lowrank_overhead": round(us["unfused"] / us["fourbit"] - 1.0, 3),
            "fused_lowrank_overhead": round(us["fused"] / us["fourbit"] - 1.0, 3),
            "max_diff_unfused_vs_fused_over_rms": round(rel, 4),
            "unfused_branch": "bf16 down projection X (Lambda^-1 L1) and up projection Y += D L2 as torch "
                              "matmul / addmm_ after the rank-0 4-bit layer; medians of 3 x 20 launches each"}


def cold_pair(args, torch, step, layers, weights, x0, ws, outs, flops, gemm_us_hot, i_dom):
    """The same steps rotating over copies of every weight blob, input, workspace
    and output, enough that the copies exceed the 256 MB last-level cache three
    times over: a step's operands were last touched two or more steps earlier and
    have been evicted by the others, so they come from HBM."""
    per_set = sum(t.numel() * t.element_size() for t in list(weights) + [x0] + list(ws) + list(outs))
    nsets = max(3, -(-(3 * (256 << 20)) // per_set))
    sets = [(list(weights), x0, list(ws), list(outs))]
    for _ in range(nsets - 1):
        sets.append(([w.clone() for w in weights], x0.clone(), [torch.empty_like(t) for t in ws],
                     [torch.empty_like(t) for t in outs]))
    n = len(layers)
    for k in range(nsets):
        step(opset=sets[k])
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)] for _ in range(args.steps)]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for k in range(args.steps):
        step(evs[k], opset=sets[k % nsets])
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    g_us = [sum(evs[k][i][1].elapsed_time(evs[k][i][2]) for k in range(args.steps)) * 1e3 / args.steps
            for i in range(n)]
    q_us = [sum(evs[k][i][0].elapsed_time(evs[k][i][1]) for k in range(args.steps)) * 1e3 / args.steps
            for i in range(n)]
    del sets
    return {"value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TOPS", "ms_per_step": round(ms, 4),
            "operand_sets": nsets, "bytes_per_set": per_set, "gemm_us": [round(x, 2) for x in g_us],
            "quantize_us": [round(x, 2) for x in q_us], "dominant_gemm_us": round(g_us[i_dom], 2),
            "dominant_gemm_us_hot": round(gemm_us_hot[i_dom], 2)}


def shader_clock():
    """The GPU's current shader clock from the amdgpu driver's sysfs files
    (the starred pp_dpm_sclk level), or None.  Read in-process: a child
    program started after the GPU is initialised is not wanted here."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                cur = [l.strip() for l in f if l.rstrip().endswith("*")]
        except OSError:
            continue
        if cur:
            return [f"{path.split('/')[4]}: {c}" for c in cur]
    return None


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

    settle_steps, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms and settle_steps < 20000:
        step()
        settle_steps += 1
        if settle_steps % 64 == 0:
            torch.cuda.synchronize()
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
                roofline=roofline, breakdown=breakdown, specs=[spec], fmt="bf16", fused=None,
                settle_steps=settle_steps)


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
            "kind": "oracle", "host_cpus": len(os.sched_getaffinity(0)), "blas_threads": int(threads),
            "sample": f"{spec.name}: all {spec.M} tokens x {spec.N} outputs (K={spec.K}); {secs:.1f} s of oracle "
                      "time (INT4 weight quantization, fp64 product, bias); quantization is single-threaded "
                      f"numpy, the product uses {threads} BLAS threads"}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover - optional dependency
        return 1


def _timed_then_breakdown(args, torch, step, n_launch):
    """Warmup, then `steps` steps timed by the host clock with no event inside
    the loop (as the main timed region), then the same steps again with events
    around every launch for the per-launch breakdown (microseconds)."""
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_launch + 1)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    seg = [sum(evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)) * 1e3 / args.steps
           for i in range(n_launch)]
    return ms, seg


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

    ms, seg = _timed_then_breakdown(args, torch, step, 2)
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

    ms, seg = _timed_then_breakdown(args, torch, step, 3)
    return {"value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TOPS", "ms_per_step": round(ms, 4),
            "fc1_quantize_us": round(seg[0], 2), "fc1_gemm_quant_us": round(seg[1], 2),
            "fc2_gemm_us": round(seg[2], 2),
            "launches": "fc1 quantize_act; fc1 gemm_quant (GEMM + fc2 quantize in the epilogue, then the "
                        "down-projection sum); fc2 gemm"}


def cpu_baseline(specs, ops, budget_rows=2048):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    `budget_rows` tokens of each layer against 1/2 (K <= 4096) or 1/8 of the
    output columns (about 10 s of host time), scaled to effective TOPS of the
    sampled work."""
    import numpy as np

    import synth
    from oracle import layer as Ly

    threads = _blas_threads()
    work, secs, parts = 0.0, 0.0, []
    for spec, L in zip(specs, ops):
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
    return {"value": round(work / secs / 1e12, 6), "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "host_cpus": len(os.sched_getaffinity(0)), "blas_threads": int(threads),
            "sample": "; ".join(parts) + f"; {secs:.1f} s of oracle time (quantize both operands, fp64 product, "
                      "low-rank branch, bias, GELU); quantization is single-threaded numpy, the product uses "
                      f"{threads} BLAS threads on a host with {len(os.sched_getaffinity(0))} CPUs"}


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.traffic_from:
        t = traffic_from(*args.traffic_from)
        names = {"gemm_mxfp4_kernel<4, 4, false, true, -1, false, 4, 3>": "mlp_mxfp4:gemm_mxfp4_fc1_mxfp4",
                 "gemm_mxfp4_kernel<8, 8, false, false, -1, false, 7, 4>": "mlp_mxfp4:gemm_mxfp4_fc2_mxfp4"}
        d = {names[k]: dict(v, gemm_source_sha256_16=gemm_source_hash()) for k, v in t.items() if k in names}
        with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
            json.dump(d, f, indent=1)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the layer runs on "
              "a single GPU (token-parallel sharding needs no collective, so N GPUs are N copies of "
              "this measurement).", file=sys.stderr)
        sys.exit(2)
    w4a16 = args.workload in W4A16
    clock_before = shader_clock()
    if w4a16:
        r = gpu_leg_w4a16(args)
        ops = None
    else:
        ops = layer_operands(layers_of(args.workload, args.fmt), args.operands)
        r = gpu_leg(args, ops)
    clock_after = shader_clock()
    specs = r["specs"]
    cfg = {"workload": args.workload, "layers": [
        {"name": s.name, "M": s.M, "K": s.K, "N": s.N, "rank": s.rank + s.lora_rank, "fmt": s.fmt,
         "epilogue": "bias" if w4a16 else "lowrank+bias" + ("+gelu" if s.gelu else "")} for s in specs],
        "output": "bf16", "weights": "packed once before timing"}
    if not w4a16:
        cfg["operands"] = args.operands
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
        line["fused_mlp" if len(specs) == 2 else "fused_qkv"] = r["fused"]
    if r.get("ablation") is not None:
        line["lowrank_ablation"] = r["ablation"]
    if r.get("repeats") is not None:
        line["repeats"] = r["repeats"]
    if r.get("cold") is not None:
        line["cold"] = r["cold"]
    if r.get("settle_steps") is not None:
        line["clock_settle"] = {"ms": args.settle_ms, "untimed_steps": r["settle_steps"]}
    line["clock"] = {"before": clock_before, "after": clock_after}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_w4a16(specs[0]) if w4a16 else cpu_baseline(specs, ops)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
