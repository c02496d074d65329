"""Benchmark of the W4A16 hot path on one MI355X.

One step = one decode pass of the Qwen-2.5-7B projection shapes (18944x3584
gate/up, 3584x18944 down, 3584x3584 qkv-o) at M = 1 through ``fp4w.linear``
with NVFP4 weights and a rank-16 LoRA, on weights rotated over more than 1 GiB
of distinct copies so that every call streams its weights from HBM.  ``value``
is the step's algorithmic bytes over its time (GB/s).  The JSON line also holds
the roofline of the decode kernel (HIP events around a graph of back-to-back
launches of it), the CPU oracle timed on a bounded sample, and the other
hot-path rows (M = 8, MXFP4, the 16384-row prefill GEMM, its backward dX
through the frozen base, its Scale-QLoRA delta gradient and its W4A4 MXFP4
form, quantize, merge, dequantize, grouped MoE).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-rows]
       python bench.py --only TARGET     (one kernel's launches and a plain copy of known
                                          size, for profiler runs; TARGET is one of
                                          decode_m1_lora, decode_m1, decode_m8_lora,
                                          quantize_nvfp4, gemm)
       --roofline-only = --only decode_m1_lora;  --gemm-only = --only gemm
Progress goes to stderr; stdout is exactly one JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense fp4 MFMA, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
ROTATE_BYTES = 1 << 30         # rotate each weight over at least 1 GiB (4x the 256 MB MALL)
METRIC = "W4A16 NVFP4 linear: effective HBM GB/s (% peak) at M=1/8; TFLOP/s at M=16K"
PROFILE_TARGETS = ("decode_m1_lora", "decode_m1", "decode_m8_lora", "quantize_nvfp4", "gemm")
# kernel sources behind each profiled target: a committed counter summary whose
# recorded hash differs from these files' hash no longer describes the kernel
TARGET_SOURCES = {
    "decode_m1_lora": ("decode.hip", "xenc.hpp", "lora_handover.hpp", "sync.hpp", "fp4w_device.hpp",
                       "fp4w_internal.hpp"),
    "decode_m1": ("decode.hip", "xenc.hpp", "sync.hpp", "fp4w_device.hpp", "fp4w_internal.hpp"),
    "decode_m8_lora": ("decode_xs.hip", "lora_handover.hpp", "sync.hpp", "fp4w_device.hpp", "fp4w_internal.hpp"),
    "quantize_nvfp4": ("quantize.hip", "codec.hpp", "fp4w_device.hpp", "fp4w_internal.hpp"),
    "gemm": ("gemm.hip", "gemm_common.hpp", "linear.hip", "fp4w_device.hpp", "fp4w_internal.hpp"),
}
PROFILE_FILES = {
    "decode_m1_lora": "decode_gate_up_m1_nvfp4_lora_pmc.txt",
    "decode_m1": "decode_gate_up_m1_nvfp4_pmc.txt",
    "decode_m8_lora": "decode_gate_up_m8_nvfp4_lora_pmc.txt",
    "quantize_nvfp4": "quantize_gate_up_nvfp4_pmc.txt",
    "gemm": "prefill_gemm_16384x18944x3584_pmc.txt",
}
# the kernels one call of each profiled target launches (name prefixes in the traces)
TARGET_KERNELS = {
    "decode_m1_lora": ("decode_f8f4_kernel",),
    "decode_m1": ("decode_f8f4_kernel",),
    "decode_m8_lora": ("decode_xs_kernel",),
    "quantize_nvfp4": ("nvfp4_amax_kernel", "nvfp4_encode_kernel"),
    "gemm": ("gemm_w4_kernel<0", "lora_down_kernel"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--skip-rows", action="store_true", help="only the headline step and its roofline")
    p.add_argument("--gemm-only", action="store_true",
                   help="only the prefill GEMM rows (both formats), for profiler runs")
    p.add_argument("--roofline-only", action="store_true",
                   help="only the roofline launches of the decode kernel and a copy kernel of known size")
    p.add_argument("--only", choices=PROFILE_TARGETS, default=None,
                   help="only one kernel's launches (and a copy of known size), for profiler runs")
    p.add_argument("--cpu-seconds", type=float, default=8.0, help="budget of the CPU-oracle headline sample")
    p.add_argument("--summarize", choices=PROFILE_TARGETS, default=None,
                   help="write profiles/<target> from rocprofv3 csv output (no GPU): --trace, --fetch, --write dirs")
    p.add_argument("--trace", default=None, help="rocprofv3 --kernel-trace --stats output directory")
    p.add_argument("--fetch", default=None, help="rocprofv3 --pmc FETCH_SIZE output directory")
    p.add_argument("--write", default=None, help="rocprofv3 --pmc WRITE_SIZE output directory")
    p.add_argument("--sq", default=None, help="rocprofv3 --pmc output directory with SQ counters (gemm)")
    p.add_argument("--commands", default=None, help="file holding the commands that made the directories")
    p.add_argument("--bench-json", default=None, help="the --only run's JSON line (HIP-event timing), for comparison")
    a = p.parse_args()
    if a.roofline_only:
        a.only = "decode_m1_lora"
    if a.gemm_only:
        a.only = "gemm"
    return a


# ---- algorithmic work ---------------------------------------------------------------

def linear_bytes(fmt, m, n, k, r):
    blk = 16 if fmt == 0 else 32
    w = n * k // 2 + n * k // blk + (4 if fmt == 0 else 0)
    return w + 2 * r * (k + n) + 2 * m * (k + n)


def linear_flops(m, n, k, r):
    return 2 * m * n * k + 2 * m * r * (k + n)


def quant_bytes(fmt, count):
    blk = 16 if fmt == 0 else 32
    return 2 * count + count // 2 + count // blk + (4 if fmt == 0 else 0)


# ---- device helpers -------------------------------------------------------------------

def main():
    args = parse()
    if args.summarize:
        summarize_profile(args)
        return
    if args.gpus != 1:
        log(f"bench.py measures one GPU only: every box here has a single MI355X, so --gpus {args.gpus} "
            "is not supported (the multi-GPU sharding of this path is described in DESIGN.md).")
        sys.exit(2)
    import torch
    from mxfp4_bit_weight_amd import fp4w
    from mxfp4_bit_weight_amd import workloads as W

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def sync():
        torch.cuda.synchronize(dev)

    def copies_for(nbytes):
        return max(2, -(-ROTATE_BYTES // nbytes))

    def time_loop(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        sync()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            fn(warmup + i)
        e1.record()
        sync()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall

    def time_graph(fn, steps, warmup, replays=1):
        """Capture `warmup` and `steps` calls of fn into two HIP graphs and time the
        replay of the second (launch overhead off the critical path); with
        replays > 1 the second is replayed that many times and the median kept."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)
        torch.cuda.current_stream().wait_stream(s)
        sync()
        gw, gt = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw):
            for i in range(warmup):
                fn(i)
        with torch.cuda.graph(gt):
            for i in range(steps):
                fn(warmup + i)
        gw.replay()
        sync()
        times = []
        t0 = time.perf_counter()
        for _ in range(replays):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            gt.replay()
            e1.record()
            sync()
            times.append(e0.elapsed_time(e1) / steps)
        wall = time.perf_counter() - t0
        if replays > 1:
            log(f"[bench]   replays (ms per call): {', '.join(f'{t:.5f}' for t in times)}")
        return sorted(times)[len(times) // 2], wall

    if args.only == "gemm":
        rank = W.LORA_RANK
        n, k = W.QWEN7B_SHAPES["gate_up"]
        weights = {}
        for fmt in (0, 1):
            w, _, a, b = W.linear_inputs(100, n, k, 1, rank=rank, wkind="outlier" if fmt == 0 else "student_t")
            weights[fmt] = (fp4w.quantize(bf16(w), fmt), bf16(a), bf16(b), n, k)
        calibration_copy(torch, dev, sync)
        rows = gemm_rows(torch, fp4w, W, dev, bf16, time_loop, rank, weights, prefill_only=True)
        print(json.dumps({"target": "gemm", "rows": rows, "kernel_sources_sha256": kernel_sources_sha256("gemm")}),
              flush=True)
        return

    # ---- decode weights: quantize once on the device, then clone for rotation ----------
    rank = W.LORA_RANK
    shapes = W.QWEN7B_SHAPES
    decode = {}
    t_gen = time.time()
    for fmt in (0, 1):
        if args.only and fmt == 1:
            break
        for si, (name, (n, k)) in enumerate(shapes.items()):
            if args.only and name != "gate_up":
                continue
            wkind = "outlier" if fmt == 0 else "student_t"
            w, x1, a, b = W.linear_inputs(100 + si, n, k, 1, rank=rank, wkind=wkind)
            x8 = W.normal_bf16(100 + si, W.TID_X + 50, (8, k), 1.0)
            q0 = fp4w.quantize(bf16(w), fmt)
            nb = linear_bytes(fmt, 1, n, k, rank)
            reps = copies_for(nb)
            qs = []
            ad, bd = bf16(a), bf16(b)
            for _ in range(reps):
                qs.append((fp4w.QWeight(fmt, q0.codes.clone(), q0.scales.clone(),
                                        q0.tensor_scale.clone() if q0.tensor_scale is not None else None, n, k),
                           ad.clone(), bd.clone()))
            decode[(fmt, name)] = dict(n=n, k=k, x1=bf16(x1), x8=bf16(x8), qs=qs, host=(w, x1, a, b))
            log(f"[bench] prepared fmt={fmt} {name} ({n},{k}) x{reps} copies")
    sync()
    log(f"[bench] inputs ready in {time.time() - t_gen:.1f}s")

    ys = {name: torch.empty((8, d["n"]), dtype=torch.bfloat16, device=dev)
          for (fmt, name), d in decode.items() if fmt == 0}
    ws_bytes = max(fp4w.linear_workspace_bytes(m, n, k, rank) for (n, k) in shapes.values() for m in (1, 8))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)      # zero-filled once, reused by every call

    # ---- the decode kernel on W (18944, 3584): with the LoRA (the headline's kernel) and without
    dg = decode[(0, "gate_up")]
    n, k = dg["n"], dg["k"]

    def gemv(m, lora):
        x = dg["x1"] if m == 1 else dg["x8"]

        def f(i):
            q, a, b = dg["qs"][i % len(dg["qs"])]
            if lora:
                fp4w.linear(x, q, a, b, out=ys["gate_up"][:m], workspace=ws)
            else:
                fp4w.linear(x, q, out=ys["gate_up"][:m], workspace=ws)
        return f

    launches = max(args.steps, 100)
    if args.only:
        copy_bytes = calibration_copy(torch, dev, sync)
        if args.only == "quantize_nvfp4":
            w = bf16(dg["host"][0])
            outs = [fp4w.empty_qweight(0, n, k, dev) for _ in range(4)]
            per, _ = time_loop(lambda i: fp4w.quantize(w, 0, out=outs[i % 4]), launches, args.warmup)
            what = "quantize"
        else:
            m, lora = {"decode_m1_lora": (1, True), "decode_m1": (1, False), "decode_m8_lora": (8, True)}[args.only]
            per, _ = time_graph(gemv(m, lora), launches, args.warmup)
            what = "linear"
        print(json.dumps({"target": args.only, "launches": launches, "per_launch_us": round(per * 1e3, 3),
                          "calls": what, "copy_kernel_bytes": copy_bytes,
                          "kernel_sources_sha256": kernel_sources_sha256(args.only)}), flush=True)
        return

    # ---- headline step: NVFP4, M = 1, three shapes, LoRA r = 16 ------------------------
    def step(i):
        for name in shapes:
            d = decode[(0, name)]
            q, a, b = d["qs"][i % len(d["qs"])]
            fp4w.linear(d["x1"], q, a, b, out=ys[name][:1], workspace=ws)

    step_bytes = sum(linear_bytes(0, 1, n_, k_, rank) for n_, k_ in shapes.values())
    ms_step, wall = time_graph(step, args.steps, args.warmup)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"[bench] step (graph replay): {ms_step * 1e3:.2f} us, {value:.1f} GB/s ({100 * value / HBM_PEAK_GBS:.1f}% of peak)")
    ms_eager, _ = time_loop(step, args.steps, args.warmup)
    log(f"[bench] step (eager launches): {ms_eager * 1e3:.2f} us")

    # ---- roofline: the headline's dominant kernel, one launch per call -------------------
    per_lora, _ = time_graph(gemv(1, True), launches, args.warmup)
    per_plain, _ = time_graph(gemv(1, False), launches, args.warmup)
    clock = sclk_mhz(torch, dev, sync)
    bytes_lora = linear_bytes(0, 1, n, k, rank)
    bytes_plain = linear_bytes(0, 1, n, k, 0)
    achieved = bytes_lora / (per_lora * 1e-3) / 1e9
    ach_plain = bytes_plain / (per_plain * 1e-3) / 1e9
    ceiling = read_ceiling(torch, dev, sync, time_graph, bytes_lora, launches, args.warmup)
    roofline = {"kernel": "decode_f8f4_kernel<NVFP4, 1 row, LoRA r=16 formed inside the launch> on W (18944, 3584), M=1",
                "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": pmc_traffic("decode_m1_lora"),
                "avg_launch_us": round(per_lora * 1e3, 3), "launches_timed": launches,
                "timing": "HIP events around a graph of back-to-back launches on their stream "
                          "(weights rotated over >1 GiB)",
                "algorithmic_bytes_per_launch": bytes_lora,
                "variants": {"no_lora": {"achieved": round(ach_plain, 1), "frac": round(ach_plain / HBM_PEAK_GBS, 4),
                                         "avg_launch_us": round(per_plain * 1e3, 3),
                                         "algorithmic_bytes_per_launch": bytes_plain,
                                         "traffic": pmc_traffic("decode_m1")}},
                "ceiling": dict(ceiling, sclk_mhz=clock,
                                frac_of_ceiling=round(achieved / ceiling["read_gbs"], 4) if ceiling["read_gbs"] else None)}
    log(f"[bench] decode kernel with LoRA {per_lora * 1e3:.2f} us ({achieved:.1f} GB/s), without "
        f"{per_plain * 1e3:.2f} us ({ach_plain:.1f} GB/s); plain read of the same bytes {ceiling['read_us']} us "
        f"({ceiling['read_gbs']} GB/s); sclk {clock} MHz")

    rows = {}
    if not args.skip_rows:
        rows = other_rows(args, torch, fp4w, W, decode, dev, bf16, sync, time_loop, time_graph, rank)

    cpu = cpu_baseline(args, W, decode, rank, step_bytes)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Qwen-2.5-7B decode projections (18944x3584, 3584x18944, 3584x3584), "
                               "NVFP4 W4A16, M=1, LoRA r=16, weights rotated over >1 GiB",
                   "batch_rows": 1, "lora_rank": rank, "format": "nvfp4",
                   "step_algorithmic_bytes": step_bytes, "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   "timing": "HIP graph replay of the timed steps", "eager_us_per_step": round(ms_eager * 1e3, 2),
                   "wall_s_timed_region": round(wall, 4)},
        "roofline": roofline, "cpu_baseline": cpu, "rows": rows,
    }
    print(json.dumps(out), flush=True)


# ---- profile summaries (rocprofv3 csv -> profiles/*.txt, no GPU) ---------------------

def _csv_rows(d, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _is_target(name, target):
    base = name.split("(")[0]
    return any(k in base for k in TARGET_KERNELS[target])


def _per_dispatch(rows, counter, reduce="sum"):
    """{dispatch id: (kernel name, value)} of one counter, its instances (XCDs,
    shader engines) added, or their maximum (a clock such as GRBM_GUI_ACTIVE)."""
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        d = r["Dispatch_Id"]
        x = float(r["Counter_Value"])
        if d in out:
            name, v = out[d]
            out[d] = (name, v + x if reduce == "sum" else max(v, x))
        else:
            out[d] = (r["Kernel_Name"], x)
    return out


def _median(v):
    v = sorted(v)
    return v[len(v) // 2] if v else float("nan")


def _calibration(rows, counter):
    """The counter of the 256 MiB calibration copies: the copy dispatches within 10%
    of the largest value of that counter among copy kernels."""
    vals = [v for n, v in _per_dispatch(rows, counter).values() if "copyBuffer" in n or "copy" in n.lower()]
    if not vals:
        return None
    top = max(vals)
    return _median([v for v in vals if v >= 0.9 * top])


def _algorithmic(target):
    """(algorithmic bytes per call, flops per call or None, what a call is)."""
    import importlib
    W = importlib.import_module("mxfp4_bit_weight_amd.workloads")
    n, k = W.QWEN7B_SHAPES["gate_up"]
    r = W.LORA_RANK
    if target == "decode_m1_lora":
        return linear_bytes(0, 1, n, k, r), linear_flops(1, n, k, r), "fp4w_linear, m = 1, LoRA r = 16"
    if target == "decode_m1":
        return linear_bytes(0, 1, n, k, 0), linear_flops(1, n, k, 0), "fp4w_linear, m = 1, no LoRA"
    if target == "decode_m8_lora":
        return linear_bytes(0, 8, n, k, r), linear_flops(8, n, k, r), "fp4w_linear, m = 8, LoRA r = 16"
    if target == "quantize_nvfp4":
        return quant_bytes(0, n * k), None, "fp4w_quantize NVFP4 (amax + encode launches)"
    m = W.PREFILL_M
    return 2 * m * k + n * k // 2 + n * k // 16 + 2 * m * n, linear_flops(m, n, k, r), \
        f"fp4w_linear, m = {m}, LoRA r = 16 (GEMM launch; the LoRA down-projection is its own launch)"


def summarize_profile(args):
    t = args.summarize
    lines = []
    add = lines.append
    nbytes, flops, what = _algorithmic(t)
    shape = "(18944, 3584) Qwen-2.5-7B gate/up"
    add(f"# {t}: W {shape}, NVFP4 unless stated; {what}")
    add("# commands (repo root on the GPU box; each counter pass a run of its own):")
    if args.commands:
        for c in open(args.commands):
            if c.strip():
                add("#   " + c.strip())
    add("# summarized by: python bench.py --summarize " + t + " --trace <dir> --fetch <dir> --write <dir>"
        + (" --sq <dir>" if args.sq else "") + " --commands <file> --bench-json <file>")
    # kernel trace
    tr = _csv_rows(args.trace, "kernel_trace.csv")
    durs = {}
    for r in tr:
        if _is_target(r["Kernel_Name"], t):
            key = r["Kernel_Name"].split("(")[0].replace("void ", "")
            durs.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    add("kernel trace (us per dispatch): kernel, dispatches, median, mean, min")
    call_us = 0.0
    for key, v in durs.items():
        add(f"  {key}: {len(v)} {_median(v):.3f} {sum(v) / len(v):.3f} {min(v):.3f}")
        call_us += _median(v)
    add(f"median kernel time per call (us): {call_us:.3f}")
    if args.bench_json and os.path.exists(args.bench_json):
        for line in open(args.bench_json):
            line = line.strip()
            if line.startswith("{"):
                j = json.loads(line)
                if "per_launch_us" in j:
                    add(f"bench.py HIP-event time per call over the same graph (us, includes launch gaps): "
                        f"{j['per_launch_us']}")
                if "rows" in j:
                    for name, row in j["rows"].items():
                        add(f"bench.py {name}: {row.get('ms')} ms per call")
    # HBM traffic
    fetch_rows = _csv_rows(args.fetch, "counter_collection.csv")
    write_rows = _csv_rows(args.write, "counter_collection.csv")
    cf = _calibration(fetch_rows, "FETCH_SIZE")
    cw = _calibration(write_rows, "WRITE_SIZE")
    copy_kib = 256 * 1024
    ff = cf / copy_kib if cf else None
    fw = cw / copy_kib if cw else None
    add(f"calibration copy 256 MiB: FETCH_SIZE {cf} KiB (factor {ff}), WRITE_SIZE {cw} KiB (factor {fw})")
    fv = [v for n, v in _per_dispatch(fetch_rows, "FETCH_SIZE").values() if _is_target(n, t)]
    wv = [v for n, v in _per_dispatch(write_rows, "WRITE_SIZE").values() if _is_target(n, t)]
    kernels_per_call = max(1, len(durs))
    fetch_b = _median(fv) * 1024 / ff * kernels_per_call if fv and ff else float("nan")
    write_b = _median(wv) * 1024 / fw * kernels_per_call if wv and fw else float("nan")
    if t == "quantize_nvfp4" or t == "gemm":      # per kernel medians, then the call's sum
        fetch_b = write_b = 0.0
        for k in TARGET_KERNELS[t]:
            fk = [v for n, v in _per_dispatch(fetch_rows, "FETCH_SIZE").values() if k in n.split("(")[0]]
            wk = [v for n, v in _per_dispatch(write_rows, "WRITE_SIZE").values() if k in n.split("(")[0]]
            if fk and ff:
                fetch_b += _median(fk) * 1024 / ff
            if wk and fw:
                write_b += _median(wk) * 1024 / fw
    add(f"dispatches counted: {len(fv)} (FETCH_SIZE run), {len(wv)} (WRITE_SIZE run)")
    add(f"HBM bytes read per call: {fetch_b:.0f}")
    add(f"HBM bytes written per call: {write_b:.0f}")
    add(f"algorithmic bytes per call: {nbytes}")
    add(f"traffic / algorithmic: {(fetch_b + write_b) / nbytes:.4f}")
    add(f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}")
    if call_us > 0:
        add(f"achieved (algorithmic bytes / median kernel time): {nbytes / (call_us * 1e-6) / 1e9:.1f} GB/s "
            f"= {100 * nbytes / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f} GB/s")
        if flops:
            add(f"achieved: {flops / (call_us * 1e-6) / 1e12:.1f} TFLOP/s "
                f"= {100 * flops / (call_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS:.1f}% of the dense bf16 peak")
    if args.sq:
        sq = _csv_rows(args.sq, "counter_collection.csv")
        names = sorted({r["Counter_Name"] for r in sq})
        add("SQ counters (median per dispatch of the target kernel):")
        med = {}
        for c in names:
            red = "max" if c.startswith("GRBM_") else "sum"
            v = [x for n, x in _per_dispatch(sq, c, red).values() if _is_target(n, t) and "lora_down" not in n]
            med[c] = _median(v)
            add(f"  {c} ({red} over instances): {med[c]:.0f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med and "SQ_BUSY_CU_CYCLES" in med and med["SQ_BUSY_CU_CYCLES"] > 0:
            # per SIMD against the busy cycles of its CU (4 SIMDs per CU); GRBM_GUI_ACTIVE
            # as read here runs several times faster than the shader clock, so it is listed only
            add(f"MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES)): "
                f"{100 * med['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * med['SQ_BUSY_CU_CYCLES']):.1f}%")
            add(f"CU busy cycles per CU (SQ_BUSY_CU_CYCLES / 256) over the kernel time: "
                f"{med['SQ_BUSY_CU_CYCLES'] / 256 / (call_us * 1e3):.3f} GHz")
        if "SQ_WAIT_INST_ANY" in med and "SQ_WAVE_CYCLES" in med and med["SQ_WAVE_CYCLES"] > 0:
            # both in the same (quad-cycle) unit, summed over waves
            add(f"waves' cycles waiting on an instruction's operands (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES): "
                f"{100 * med['SQ_WAIT_INST_ANY'] / med['SQ_WAVE_CYCLES']:.1f}%")
        if "SQ_ACTIVE_INST_VALU" in med and "SQ_WAVE_CYCLES" in med and med["SQ_WAVE_CYCLES"] > 0:
            add(f"waves' cycles issuing VALU (SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES): "
                f"{100 * med['SQ_ACTIVE_INST_VALU'] / med['SQ_WAVE_CYCLES']:.1f}%")
        if "SQ_WAVE_CYCLES" in med and "SQ_WAVES" in med and med["SQ_WAVES"] > 0:
            add(f"mean wave lifetime (4 x SQ_WAVE_CYCLES / SQ_WAVES, shader cycles): "
                f"{4 * med['SQ_WAVE_CYCLES'] / med['SQ_WAVES']:.0f}")
        if "SQ_LDS_BANK_CONFLICT" in med and "SQ_LDS_IDX_ACTIVE" in med and med["SQ_LDS_IDX_ACTIVE"] > 0:
            add(f"LDS bank conflict cycles / LDS active cycles: "
                f"{med['SQ_LDS_BANK_CONFLICT'] / med['SQ_LDS_IDX_ACTIVE']:.4f}")
    add(f"kernel_sources_sha256: {kernel_sources_sha256(t)}")
    out = os.path.join(ROOT, "profiles", PROFILE_FILES[t])
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def pmc_traffic(target):
    """HBM bytes per launch of a profiled kernel from its committed rocprofv3 --pmc
    summary, if that was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", PROFILE_FILES[target])
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("kernel_sources_sha256") != kernel_sources_sha256(target):
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def kernel_sources_sha256(target):
    h = hashlib.sha256()
    for f in TARGET_SOURCES[target]:
        h.update(open(os.path.join(ROOT, "mxfp4_bit_weight_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def calibration_copy(torch, dev, sync):
    """A plain 256 MiB device copy: the profiler's FETCH_SIZE / WRITE_SIZE for a
    launch of known size, which scales the counters of the profiled kernel."""
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    sync()
    return src.numel()


def _membench():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "mxfp4_bit_weight_amd", "libfp4w_membench.so"))
    lib.fp4w_membench_read.restype = ctypes.c_int
    lib.fp4w_membench_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.fp4w_membench_clock.restype = ctypes.c_int
    lib.fp4w_membench_clock.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    return lib


def sclk_mhz(torch, dev, sync):
    """The shader clock right after the decode launches: cycle counter against the
    100 MHz counter over 50 us on one wave (median of 5)."""
    import ctypes
    lib = _membench()
    out = torch.zeros(2, dtype=torch.int64, device=dev)
    vals = []
    for _ in range(5):
        st = lib.fp4w_membench_clock(5000, ctypes.c_void_p(out.data_ptr()),
                                     ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        if st != 0:
            return None
        sync()
        cyc, ticks = (int(v) for v in out.cpu().tolist())
        if ticks > 0:
            vals.append(100.0 * cyc / ticks)
    return round(sorted(vals)[len(vals) // 2], 1) if vals else None


def read_ceiling(torch, dev, sync, time_graph, nbytes, launches, warmup):
    """What a memory-bound launch of `nbytes` can reach here: a plain streaming
    read of the same byte count from buffers rotated over more than 1 GiB, timed
    like the decode kernel (graph of back-to-back launches, HIP events); the best
    of a few grid sizes."""
    import ctypes
    lib = _membench()
    nb = (nbytes + 15) // 16 * 16
    copies = max(2, -(-ROTATE_BYTES // nb))
    bufs = [torch.ones(nb, dtype=torch.uint8, device=dev) for _ in range(copies)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    best = None
    for blocks in (1024, 2048, 4096, 8192):
        def f(i, blocks=blocks):
            st = lib.fp4w_membench_read(ctypes.c_void_p(bufs[i % copies].data_ptr()), nb, blocks,
                                        ctypes.c_void_p(sink.data_ptr()),
                                        ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
            if st != 0:
                raise RuntimeError(f"fp4w_membench_read: status {st}")
        per, _ = time_graph(f, launches, warmup)
        if best is None or per < best[0]:
            best = (per, blocks)
    del bufs
    per, blocks = best
    return {"read_us": round(per * 1e3, 3), "read_gbs": round(nbytes / (per * 1e-3) / 1e9, 1),
            "read_frac_of_peak": round(nbytes / (per * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "read_blocks": blocks,
            "what": "plain 16-byte streaming read of the kernel's algorithmic bytes, same rotation and timing"}


def gemm_rows(torch, fp4w, W, dev, bf16, time_loop, rank, weights, prefill_only=False):
    """The prefill GEMM: x 16384 x 3584, W (18944, 3584), LoRA r = 16, both formats
    (weights[fmt] = (qweight, A, B, n, k)); 10 untimed calls first, as the clock
    ramps up under this load.  prefill_only: that GEMM alone (profiler runs)."""
    rows = {}
    mrows = W.PREFILL_M
    for fmt in (0, 1):
        q, a, b, n, k = weights[fmt]
        x = bf16(W.normal_bf16(300, W.TID_X, (mrows, k), 1.0))
        y = torch.empty((mrows, n), dtype=torch.bfloat16, device=dev)
        wsg = torch.zeros(fp4w.linear_workspace_bytes(mrows, n, k, rank), dtype=torch.uint8, device=dev)
        gms, _ = time_loop(lambda i: fp4w.linear(x, q, a, b, out=y, workspace=wsg), 10, 10)
        fl = linear_flops(mrows, n, k, rank)
        tf = fl / (gms * 1e-3) / 1e12
        name = "nvfp4" if fmt == 0 else "mxfp4"
        rows[f"prefill_gemm_{name}"] = {"m": mrows, "n": n, "k": k, "ms": round(gms, 3), "TFLOP/s": round(tf, 1),
                                        "pct_bf16_peak": round(100 * tf / BF16_PEAK_TFLOPS, 1), "algorithmic_flop": fl}
        log(f"[bench] prefill GEMM {name} {gms:.3f} ms, {tf:.1f} TFLOP/s")
        if prefill_only:
            del x, y, wsg
            continue
        # the input gradient through the frozen base for the same shape: dX = dY deq(W),
        # dY the forward's output (m x n), dX m x k
        dx = torch.empty((mrows, k), dtype=torch.bfloat16, device=dev)
        bms, _ = time_loop(lambda i: fp4w.linear_backward_dx(y, q, out=dx), 10, 10)
        bfl = 2 * mrows * n * k
        btf = bfl / (bms * 1e-3) / 1e12
        rows[f"backward_dx_{name}"] = {"m": mrows, "n": n, "k": k, "ms": round(bms, 3), "TFLOP/s": round(btf, 1),
                                       "pct_bf16_peak": round(100 * btf / BF16_PEAK_TFLOPS, 1), "algorithmic_flop": bfl}
        log(f"[bench] backward dX {name} {bms:.3f} ms, {btf:.1f} TFLOP/s")
        # the adapter's gradients (u = dY B, dA = u^T x, dB = dY^T (x A^T)) and the
        # input gradient with the adapter's term u A, same layer and tokens
        if fmt == 0:
            ga = torch.empty((rank, k), dtype=torch.float32, device=dev)
            gb = torch.empty((n, rank), dtype=torch.float32, device=dev)
            uu = torch.empty((mrows, rank), dtype=torch.float32, device=dev)
            wsl = torch.empty(fp4w.lora_backward_workspace_bytes(mrows, n, k, rank), dtype=torch.uint8, device=dev)

            def lgrad(i):
                fp4w._check(fp4w._lora_bwd(fp4w._ptr(y), mrows, n, fp4w._ptr(x), k, fp4w._ptr(a), fp4w._ptr(b), rank,
                                           fp4w._ptr(uu), fp4w._ptr(ga), fp4w._ptr(gb), fp4w._ptr(wsl), wsl.numel(),
                                           fp4w._stream(dev)), "fp4w_lora_backward")
            lms, _ = time_loop(lgrad, 10, 5)
            lfl = 2 * mrows * rank * (2 * n + 2 * k)
            lbytes = 2 * (2 * mrows * n + 2 * mrows * k)            # dY and x, each read twice
            rows["lora_backward"] = {"m": mrows, "n": n, "k": k, "r": rank, "ms": round(lms, 3),
                                     "GB/s": round(lbytes / (lms * 1e-3) / 1e9, 1),
                                     "pct_hbm_peak": round(100 * lbytes / (lms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
                                     "algorithmic_bytes": lbytes, "algorithmic_flop": lfl,
                                     "bound": "hbm (dY and x streamed twice: products over their rows and columns)"}
            log(f"[bench] LoRA backward {lms:.3f} ms")
            xms, _ = time_loop(lambda i: fp4w.linear_backward_dx(y, q, out=dx, lora_u=uu, lora_a=a), 10, 5)
            xfl = bfl + 2 * mrows * rank * k
            rows["backward_dx_with_lora_nvfp4"] = {"m": mrows, "n": n, "k": k, "r": rank, "ms": round(xms, 3),
                                                   "TFLOP/s": round(xfl / (xms * 1e-3) / 1e12, 1),
                                                   "pct_bf16_peak": round(100 * xfl / (xms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 1),
                                                   "algorithmic_flop": xfl}
            log(f"[bench] backward dX + u A {xms:.3f} ms")
            del ga, gb, uu, wsl
        # the Scale-QLoRA delta gradient of the same layer: dY = y, X = x
        gout = torch.empty((n, k // (16 if fmt == 0 else 32)), dtype=torch.float32, device=dev)
        dms, _ = time_loop(lambda i: fp4w.scale_delta_grad(y, x, q, out=gout), 10, 10)
        dtf = bfl / (dms * 1e-3) / 1e12
        rows[f"scale_delta_grad_{name}"] = {"m": mrows, "n": n, "k": k, "ms": round(dms, 3), "TFLOP/s": round(dtf, 1),
                                            "pct_bf16_peak": round(100 * dtf / BF16_PEAK_TFLOPS, 1),
                                            "algorithmic_flop": bfl}
        log(f"[bench] scale delta grad {name} {dms:.3f} ms, {dtf:.1f} TFLOP/s")
        del dx, gout
        if fmt == 1:
            # W4A4: the same x quantized to MXFP4 (outside the timed region), then
            # the block-scaled fp4 product against the same MXFP4 weight
            xq = fp4w.quantize(x, 1)
            ams, _ = time_loop(lambda i: fp4w.linear_w4a4(xq, q, out=y), 10, 10)
            afl = 2 * mrows * n * k
            atf = afl / (ams * 1e-3) / 1e12
            rows["prefill_w4a4_mxfp4"] = {"m": mrows, "n": n, "k": k, "ms": round(ams, 3), "TFLOP/s": round(atf, 1),
                                          "pct_fp4_peak": round(100 * atf / FP4_PEAK_TFLOPS, 1), "algorithmic_flop": afl}
            log(f"[bench] prefill W4A4 mxfp4 {ams:.3f} ms, {atf:.1f} TFLOP/s")
            del xq
        del x, y, wsg
    return rows


def other_rows(args, torch, fp4w, W, decode, dev, bf16, sync, time_loop, time_graph, rank):
    rows = {}
    reps = max(100, args.steps)          # graph launches per row (fewer would carry the graph's start per call)
    ws_bytes = max(fp4w.linear_workspace_bytes(m, n, k, rank) for (n, k) in W.QWEN7B_SHAPES.values() for m in (1, 8))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    # decode linears, every shape, M = 1 and 8, both formats
    dec = {}
    for (fmt, name), d in decode.items():
        for m in (1, 8):
            x = d["x1"] if m == 1 else d["x8"]
            y = torch.empty((m, d["n"]), dtype=torch.bfloat16, device=dev)

            def f(i, d=d, x=x, y=y):
                q, a, b = d["qs"][i % len(d["qs"])]
                fp4w.linear(x, q, a, b, out=y, workspace=ws)
            ms, _ = time_graph(f, reps, reps, replays=3)   # the median of three replays
            nb = linear_bytes(fmt, m, d["n"], d["k"], rank)
            gbs = nb / (ms * 1e-3) / 1e9
            dec[f"{'nvfp4' if fmt == 0 else 'mxfp4'}/{name}/M{m}"] = {
                "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                "algorithmic_bytes": nb}
    rows["decode_linear_with_lora"] = dec
    log("[bench] decode rows done")

    # the noisy RMSNorm prologue (m = 1, k = 3584) alone and ahead of the gate/up
    # decode linear (NVFP4, LoRA r = 16): two launches per call
    d = decode[(0, "gate_up")]
    gam = bf16(W.normal_bf16(301, W.TID_X, (d["k"],), 1.0))
    noise = torch.from_numpy(np.random.default_rng(302).standard_normal(d["k"]).astype(np.float32)).to(dev)
    xn = torch.empty_like(d["x1"])
    sig = fp4w.aqn_sigma(100, 1000)
    ams, _ = time_graph(lambda i: fp4w.aqn_rmsnorm(d["x1"], gam, noise, sig, 1e-6, out=xn), reps, reps)
    aqn = {}
    for m in (1, 8):
        xm = d["x1"] if m == 1 else d["x8"]
        xnm = torch.empty_like(xm)
        ym = torch.empty((m, d["n"]), dtype=torch.bfloat16, device=dev)

        def norm_linear(i, xm=xm, xnm=xnm, ym=ym):
            q, a, b = d["qs"][i % len(d["qs"])]
            fp4w.aqn_rmsnorm(xm, gam, noise, sig, 1e-6, out=xnm)
            fp4w.linear(xnm, q, a, b, out=ym, workspace=ws)
        nms, _ = time_graph(norm_linear, reps, reps)
        aws = torch.zeros(fp4w.linear_aqn_workspace_bytes(m, d["n"], d["k"], rank), dtype=torch.uint8, device=dev)

        def fused(i, xm=xm, ym=ym, aws=aws):
            q, a, b = d["qs"][i % len(d["qs"])]
            fp4w.linear_aqn(xm, gam, noise, sig, q, a, b, eps=1e-6, out=ym, workspace=aws)
        fms, _ = time_graph(fused, reps, reps)
        aqn[m] = (nms, fms)
    nms, fms = aqn[1]
    rows["aqn_rmsnorm_m1_k3584"] = {"us": round(ams * 1e3, 2),
                                    "us_with_gate_up_linear_nvfp4": round(nms * 1e3, 2),
                                    "us_fused_into_gate_up_linear_nvfp4": round(fms * 1e3, 2),
                                    "linear_alone_us": dec["nvfp4/gate_up/M1"]["us"],
                                    "m8": {"us_with_gate_up_linear_nvfp4": round(aqn[8][0] * 1e3, 2),
                                           "us_fused_into_gate_up_linear_nvfp4": round(aqn[8][1] * 1e3, 2),
                                           "linear_alone_us": dec["nvfp4/gate_up/M8"]["us"]}}
    log(f"[bench] noisy RMSNorm {ams * 1e3:.2f} us, then the gate/up linear {nms * 1e3:.2f} us, "
        f"fused {fms * 1e3:.2f} us")

    weights = {fmt: (*decode[(fmt, "gate_up")]["qs"][0], decode[(fmt, "gate_up")]["n"], decode[(fmt, "gate_up")]["k"])
               for fmt in (0, 1)}
    rows.update(gemm_rows(torch, fp4w, W, dev, bf16, time_loop, rank, weights))
    torch.cuda.empty_cache()

    # quantize over a 7B-shaped set: 28 layers x {2 x (18944,3584), (3584,18944), 4 x (3584,3584)}
    for fmt in (0, 1):
        base = {}
        for name, (n, k) in W.QWEN7B_SHAPES.items():
            base[(n, k)] = bf16(decode[(fmt, name)]["host"][0])      # the decode weights of this format
        tensors, outs = [], []
        for _ in range(W.QWEN7B_LAYERS):
            for (n, k) in W.QWEN7B_LAYER:
                tensors.append(base[(n, k)].clone())
                outs.append(fp4w.empty_qweight(fmt, n, k, dev))
        count = sum(t.numel() for t in tensors)

        def qpass(i):
            for t, o in zip(tensors, outs):
                fp4w.quantize(t, fmt, out=o)
        ms, _ = time_graph(qpass, 3, 1)
        nb = sum(quant_bytes(fmt, t.numel()) for t in tensors)
        gbs = nb / (ms * 1e-3) / 1e9
        rows[f"quantize_7b_set_{'nvfp4' if fmt == 0 else 'mxfp4'}"] = {
            "weights": count, "tensors": len(tensors), "ms": round(ms, 3), "GB/s": round(gbs, 1),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1), "weights_per_s": round(count / (ms * 1e-3), 1),
            "algorithmic_bytes": nb}
        log(f"[bench] quantize fmt={fmt}: {ms:.2f} ms, {gbs:.1f} GB/s")
        # dequantize the same set (bf16 out)
        deq = [torch.empty((o.n, o.k), dtype=torch.bfloat16, device=dev) for o in outs[:7]]

        def dpass(i):
            for j, o in enumerate(outs):
                fp4w.dequantize(o, out=deq[j % 7])
        ms_d, _ = time_graph(dpass, 3, 1)
        nbd = sum(o.n * o.k * 2 + o.n * o.k // 2 + o.n * o.k // (16 if fmt == 0 else 32) for o in outs)
        rows[f"dequantize_7b_set_{'nvfp4' if fmt == 0 else 'mxfp4'}"] = {
            "ms": round(ms_d, 3), "GB/s": round(nbd / (ms_d * 1e-3) / 1e9, 1), "algorithmic_bytes": nbd}
        # fused fake-quant (dequantize(quantize(W)) in one pass) over the same set: reads 2 B/w,
        # writes 2 B/w and the block scales
        fq = [torch.empty((o.n, o.k), dtype=torch.bfloat16, device=dev) for o in outs[:7]]
        fq_s = [torch.empty_like(o.scales) for o in outs[:7]]
        fq_t = torch.empty(1, dtype=torch.float32, device=dev)

        def fpass(i):
            for j, t in enumerate(tensors):
                y = fq[j % 7]
                ts = fq_t if fmt == 0 else None
                fp4w._check(fp4w._fake_quant(fmt, fp4w._ptr(t), t.shape[0], t.shape[1], fp4w._ptr(y),
                                             fp4w._ptr(fq_s[j % 7]), fp4w._ptr(ts), 0, fp4w._stream(dev)),
                            "fp4w_fake_quant")
        ms_f, _ = time_graph(fpass, 3, 1)
        nbf = sum(t.numel() * 4 + t.numel() // (16 if fmt == 0 else 32) for t in tensors)
        rows[f"fake_quant_7b_set_{'nvfp4' if fmt == 0 else 'mxfp4'}"] = {
            "ms": round(ms_f, 3), "GB/s": round(nbf / (ms_f * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * nbf / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS, 1), "algorithmic_bytes": nbf}
        log(f"[bench] fake-quant fmt={fmt}: {ms_f:.2f} ms, {nbf / (ms_f * 1e-3) / 1e9:.1f} GB/s")
        del fq, fq_s
        if fmt == 0:
            # scale-only merge of the (18944, 3584) weight (new scales, codes kept); ratio to re-quantizing it
            o = outs[0]
            s_t = o.scales.reshape(-1).cpu()
            dec_s = s_t.view(torch.float8_e4m3fn).to(torch.float32).numpy()
            z = W.merge_noise(401, o.scales.numel())
            deltas = torch.from_numpy((np.float32(0.05) * dec_s * z).astype(np.float32)).to(dev).reshape(o.scales.shape)
            # rotated over copies of more than 1 GiB together, so each call reads HBM
            nbm = o.scales.numel() * (1 + 4 + 1)
            mcopies = max(2, -(-(1 << 30) // nbm))
            msets = [(fp4w.QWeight(0, o.codes, o.scales.clone(), o.tensor_scale, o.n, o.k), deltas.clone(),
                      torch.empty_like(o.scales)) for _ in range(mcopies)]

            def mpass(i):
                qm, dm, om = msets[i % mcopies]
                fp4w.merge_scales(qm, dm, scales_out=om)
            ms_m, _ = time_graph(mpass, 200, 20, replays=3)
            ms_q, _ = time_graph(lambda i: fp4w.quantize(tensors[0], 0, out=outs[0]), 20, 3)
            del msets
            rows["merge_scales_nvfp4"] = {"blocks": o.scales.numel(), "us": round(ms_m * 1e3, 2),
                                          "GB/s": round(nbm / (ms_m * 1e-3) / 1e9, 1), "algorithmic_bytes": nbm,
                                          "requantize_same_tensor_us": round(ms_q * 1e3, 2),
                                          "speedup_vs_requantize": round(ms_q / ms_m, 1)}
        del tensors, outs, base, deq
        torch.cuda.empty_cache()
    log("[bench] quantize/dequantize/merge rows done")

    # grouped MoE: 128 experts, gate/up (768, 2048), down (2048, 768), 64 tokens top-8
    cfg = W.MOE
    row_index, offsets = W.moe_routing(500)
    active = int((np.diff(offsets) > 0).sum())
    ri, off = torch.from_numpy(row_index).to(dev), torch.from_numpy(offsets).to(dev)
    x = bf16(W.normal_bf16(500, W.TID_X, (cfg["tokens"], cfg["d_model"]), 1.0))
    xd = bf16(W.normal_bf16(500, W.TID_DOWN_IN, (row_index.size, cfg["d_ff"]), 1.0))
    rid = torch.arange(row_index.size, dtype=torch.int32, device=dev)
    experts = {}
    for ti, (n, k, tag) in enumerate([(cfg["d_ff"], cfg["d_model"], "gate"), (cfg["d_ff"], cfg["d_model"], "up"),
                                      (cfg["d_model"], cfg["d_ff"], "down")]):
        wd = bf16(W.moe_expert_weights(600 + ti, cfg["experts"], n, k))
        codes = torch.empty((cfg["experts"], n, k // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((cfg["experts"], n, k // 16), dtype=torch.uint8, device=dev)
        ts = torch.empty(cfg["experts"], dtype=torch.float32, device=dev)
        for e in range(cfg["experts"]):          # per-expert tensor scale
            fp4w.quantize(wd[e], 0, out=fp4w.QWeight(0, codes[e], scales[e], ts[e:e + 1], n, k))
        experts[tag] = (codes, scales, ts, n, k)
        del wd
    copies = 4
    moe = [{tag: (c.clone(), s.clone(), t.clone(), n, k) for tag, (c, s, t, n, k) in experts.items()}
           for _ in range(copies)]
    yg = torch.empty((row_index.size, cfg["d_ff"]), dtype=torch.bfloat16, device=dev)
    yd = torch.empty((row_index.size, cfg["d_model"]), dtype=torch.bfloat16, device=dev)

    def moe_pass(i):
        e = moe[i % copies]
        for tag in ("gate", "up"):
            c, s, t, n, k = e[tag]
            fp4w.grouped_linear(x, ri, off, 0, c, s, t, out=yg)
        c, s, t, n, k = e["down"]
        fp4w.grouped_linear(xd, rid, off, 0, c, s, t, out=yd)
    ms, _ = time_graph(moe_pass, 40, 8, replays=3)
    nb = 0
    for tag, (c, s, t, n, k) in experts.items():
        nb += active * (n * k // 2 + n * k // 16 + 4)
    nb += 2 * (2 * cfg["tokens"] * cfg["d_model"] + 2 * row_index.size * cfg["d_ff"])
    nb += 2 * row_index.size * cfg["d_ff"] + 2 * row_index.size * cfg["d_model"]
    gbs = nb / (ms * 1e-3) / 1e9
    rows["grouped_moe_nvfp4"] = {"experts": cfg["experts"], "active_experts": active, "rows": int(row_index.size),
                                 "us_per_gate_up_down": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                                 "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1), "algorithmic_bytes": nb}
    log(f"[bench] grouped MoE {ms * 1e3:.1f} us, {gbs:.1f} GB/s")
    return rows


def cpu_baseline(args, W, decode, rank, step_bytes):
    """The CPU oracle (test infrastructure, binary64, OpenMP) on the host cores it
    is given: the headline decode step for about --cpu-seconds, then a bounded
    sample of each other row (a few seconds each), in the same units as the GPU
    rows.  The oracle is used as it stands, never tuned for this."""
    import oracle as O
    host = {name: decode[(0, name)]["host"] for name in W.QWEN7B_SHAPES}
    prepared = {}
    for name, (w, x1, a, b) in host.items():
        c, s, st = O.quantize(O.NVFP4, w)
        prepared[name] = (x1, c, s, st, a, b)
    reps = 0
    t0 = time.perf_counter()
    while True:
        for name, (x1, c, s, st, a, b) in prepared.items():
            O.linear(O.NVFP4, x1, c, s, st, a, b)
        reps += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    dt = time.perf_counter() - t0
    total = dt

    def timed(fn, budget=2.0):
        n_, t_ = 0, time.perf_counter()
        while True:
            fn()
            n_ += 1
            if time.perf_counter() - t_ >= budget:
                return n_, time.perf_counter() - t_

    rows = {}
    w, x1, a, b = host["gate_up"]
    n, k = w.shape
    for fmt, tag in ((O.NVFP4, "nvfp4"), (O.MXFP4, "mxfp4")):
        cnt, sec = timed(lambda: O.quantize(fmt, w))
        total += sec
        rate = cnt * w.size / sec
        rows[f"quantize_{tag}"] = {"weights_per_s": round(rate, 1),
                                   "GB/s": round(rate * quant_bytes(fmt, w.size) / w.size / 1e9, 3),
                                   "sample": f"{cnt} quantizations of W (18944, 3584), {sec:.1f} s"}
    x1n, c, sc, st, an, bn = prepared["gate_up"]
    g = np.random.default_rng(401)
    deltas = (0.01 * g.standard_normal(sc.size)).astype(np.float32)
    cnt, sec = timed(lambda: O.merge_scales(O.NVFP4, sc, deltas))
    total += sec
    rows["merge_scales_nvfp4"] = {"us": round(1e6 * sec / cnt, 1), "GB/s": round(cnt * sc.size * 6 / sec / 1e9, 4),
                                  "sample": f"{cnt} in-place merges of 4,243,456 blocks, {sec:.1f} s"}
    x8 = W.normal_bf16(100, W.TID_X + 50, (8, k), 1.0)
    cnt, sec = timed(lambda: O.linear(O.NVFP4, x8, c, sc, st, an, bn))
    total += sec
    rows["decode_nvfp4_gate_up_M8"] = {"us": round(1e6 * sec / cnt, 1),
                                       "GB/s": round(cnt * linear_bytes(0, 8, n, k, rank) / sec / 1e9, 4),
                                       "sample": f"{cnt} linears x (8, 3584) W (18944, 3584) LoRA r=16, {sec:.1f} s"}
    slice_rows = 32
    xs = W.normal_bf16(300, W.TID_X, (slice_rows, k), 1.0)
    cnt, sec = timed(lambda: O.linear(O.NVFP4, xs, c, sc, st, an, bn), budget=3.0)
    total += sec
    per_row = sec / cnt / slice_rows
    full_s = per_row * W.PREFILL_M
    rows["prefill_gemm_nvfp4"] = {
        "TFLOP/s": round(linear_flops(W.PREFILL_M, n, k, rank) / full_s / 1e12, 6),
        "extrapolated_ms": round(1e3 * full_s, 1),
        "sample": f"{cnt} x a {slice_rows}-row slice of x (16384, 3584) against W (18944, 3584), LoRA r=16, "
                  f"{sec:.1f} s; extrapolated per row to 16384 rows (labelled: not a full run)"}
    cfg = W.MOE
    row_index, offsets = W.moe_routing(500)
    xm = W.normal_bf16(500, W.TID_X, (cfg["tokens"], cfg["d_model"]), 1.0)
    ex = W.moe_expert_weights(600, cfg["experts"], cfg["d_ff"], cfg["d_model"])
    qe = [O.quantize(O.NVFP4, ex[e]) for e in range(cfg["experts"])]
    ce = np.stack([q[0] for q in qe])
    se = np.stack([q[1] for q in qe])
    te = np.array([q[2] for q in qe], np.float32)
    active = int((np.diff(offsets) > 0).sum())
    cnt, sec = timed(lambda: O.grouped_linear(O.NVFP4, xm, row_index, offsets, ce, se, te))
    total += sec
    nbm = active * (cfg["d_ff"] * cfg["d_model"] * 9 // 16 + 4) + 2 * (cfg["tokens"] * cfg["d_model"]
                                                                      + row_index.size * cfg["d_ff"])
    rows["grouped_moe_gate_nvfp4"] = {"us": round(1e6 * sec / cnt, 1), "GB/s": round(cnt * nbm / sec / 1e9, 4),
                                      "sample": f"{cnt} grouped gate projections (128 experts (768, 2048), "
                                                f"64 tokens top-8), {sec:.1f} s"}
    return {"value": round(step_bytes * reps / dt / 1e9, 3), "unit": "GB/s", "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"{reps} decode steps (the three Qwen-2.5-7B shapes at M=1, NVFP4, LoRA r=16), binary64 "
                      f"oracle with OpenMP, {dt:.1f} s",
            "affinity_cpus": len(os.sched_getaffinity(0)), "total_cpu_seconds": round(total, 1), "rows": rows}


if __name__ == "__main__":
    main()
