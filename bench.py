"""Throughput of the quantized-attention hot path on one MI355X.

One step = the whole forward hot path on one batch of resident synthetic input:
smoothing/quantization prologue + fused attention (sage_attn_fwd_ex).  The
headline workload is the LLM-prefill shape (INT8 QK^T, FP8 P~V, causal,
B=1 H=32 N=4096 d=128).  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra] [--copy-calib]
  python bench.py --traffic FETCH_DIR WRITE_DIR   (turn two rocprofv3 --pmc runs into a profile summary)

Roofline traffic: run this script twice under rocprofv3 with --copy-calib, once with
--pmc FETCH_SIZE and once with --pmc WRITE_SIZE (--output-format csv), then
--traffic on the two output directories.  The summary lands in profiles/ with a hash of
the kernel sources; the bench reports it as roofline.traffic only while the hash matches.
"""
import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HEADLINE = "int8_fp8_causal_b1h32n4096d128"
METRIC = "attention TOPS (4·B·H·N²·d/s, ½ if causal) at d=128; % of MI355X MFMA peak"
# MI355X dense peaks (TFLOP/s or TOP/s)
PEAK = {"int8_fp8": 5000.0, "mxfp4_fp8": 1.0 / (0.5 / 10100.0 + 0.5 / 5000.0), "mxfp4_mxfp4": 10100.0,
        "int8_f16": 1.0 / (0.5 / 5000.0 + 0.5 / 2500.0)}   # half the ops on each product's matrix path
HBM_PEAK_GBS = 8000.0
COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_fwd_int8_fp8_causal_b1h32n4096d128.txt")
KERNEL_SOURCES = ["bit_quantized_attention_smooth_amd/csrc/attn_fwd.hip",
                  "bit_quantized_attention_smooth_amd/csrc/sage_device.hpp"]


def kernel_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the fused kernel from the committed counter summary, if current."""
    try:
        kv = dict(line.strip().split("=", 1) for line in open(TRAFFIC_FILE) if "=" in line and not line.startswith("#"))
    except OSError:
        return None
    if kv.get("source_sha256_16") != kernel_hash():
        return None
    return float(kv["hbm_bytes_per_launch"])


def _short(kname):
    return kname.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0]


def dispatch_counters(path):
    """{(kernel, grid): {counter: [per-dispatch values]}} plus per-dispatch durations (ns)."""
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    per, dur = {}, {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]) // int(r["Workgroup_Size"]))
            d = per.setdefault(key, {}).setdefault(r["Counter_Name"], {})
            did = (f, r["Dispatch_Id"])
            d[did] = d.get(did, 0.0) + float(r["Counter_Value"])
            dur.setdefault(key, {})[did] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return ({k: {c: list(v.values()) for c, v in cs.items()} for k, cs in per.items()},
            {k: list(v.values()) for k, v in dur.items()})


def counter_summary(sq_dir, fetch_dir, write_dir, out_path):
    """Markdown profile: MFMA busy share per fused-kernel launch shape and of the backward's main
    kernels (SQ counters), and the prologue kernels' HBM bytes (FETCH_SIZE / WRITE_SIZE,
    copy-calibrated) per launch."""
    mean = lambda v: sum(v) / len(v)
    sq, _ = dispatch_counters(sq_dir)
    lines = ["# MFMA busy share of the fused forward and backward kernels, and HBM bytes of the prologue", "",
             "Commands (repository root, one MI355X):", "",
             "    rocprofv3 --pmc SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_VALU "
             "SQ_INSTS_MFMA SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES SQ_WAIT_ANY --output-format csv -d <sq_dir> -- "
             "python bench.py --steps 5 --warmup 2 --no-cpu",
             "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -- python bench.py --steps 3 --warmup 1 "
             "--no-cpu --no-extra --copy-calib",
             "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write_dir> -- python bench.py --steps 3 --warmup 1 "
             "--no-cpu --no-extra --copy-calib",
             "    python bench.py --counters <sq_dir> <fetch_dir> <write_dir>", "",
             "## Fused kernels: MFMA busy share", "",
             "SQ_BUSY_CYCLES is summed over the 32 shader engines and SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs,",
             "so MFMA busy = MFMA_BUSY / (1024 * BUSY / 32): the share of the kernel's time the matrix cores of",
             "an average SIMD were busy.  Co-exec is the share of MFMA busy time that overlapped vector issue.",
             "VALU busy = 4 SQ_ACTIVE_INST_VALU / (1024 * BUSY / 32) (the counter is in quad-cycles): the share",
             "of the kernel's time an average SIMD issued vector instructions.",
             "Template arguments: <head dim, QK format (1 INT8, 3 MXFP4), causal, I/O dtype, P~V format (2 FP8,",
             "3 MXFP4, 4 MXFP8, 5 fp16), finer INT8 steps>.", "",
             "| kernel | workgroups | dispatches | MFMA busy | VALU busy | co-exec | VALU instr. per MFMA | wait share of wave cycles |",
             "|---|---|---|---|---|---|---|---|"]
    def sq_rows(match):
        for (k, g), cs in sorted(sq.items(), key=lambda kv: (kv[0][0], -kv[0][1])):
            if not match(k) or "SQ_BUSY_CYCLES" not in cs:
                continue
            busy = mean(cs["SQ_BUSY_CYCLES"]) / 32.0
            mfma = mean(cs.get("SQ_VALU_MFMA_BUSY_CYCLES", [0])) / 1024.0
            coex = mean(cs.get("SQ_VALU_MFMA_COEXEC_CYCLES", [0])) / 1024.0
            valu = 4.0 * mean(cs.get("SQ_ACTIVE_INST_VALU", [0])) / 1024.0
            vpm = mean(cs.get("SQ_INSTS_VALU", [0])) / max(1.0, mean(cs.get("SQ_INSTS_MFMA", [1])))
            wait = mean(cs.get("SQ_WAIT_ANY", [0])) / max(1.0, mean(cs.get("SQ_WAVE_CYCLES", [1])))
            lines.append(f"| `{k}` | {g} | {len(cs['SQ_BUSY_CYCLES'])} | {100 * mfma / busy:.1f} % | "
                         f"{100 * valu / busy:.1f} % | {100 * coex / max(mfma, 1e-9):.0f} % | {vpm:.1f} | "
                         f"{100 * wait:.0f} % |")

    sq_rows(lambda k: "attn_fwd_kernel" in k)
    lines += ["", "## Backward kernels (training workloads B=8 H=16 N=2048, causal; d = 64 and 128)", "",
              "Template arguments: d = 64 kernels <head dim, causal, I/O dtype>; d = 128 kernels <causal, I/O",
              "dtype, waves per workgroup> (two waves per 32-token group, two workgroups per CU).", "",
              "| kernel | workgroups | dispatches | MFMA busy | VALU busy | co-exec | VALU instr. per MFMA | wait share of wave cycles |",
              "|---|---|---|---|---|---|---|---|"]
    sq_rows(lambda k: any(x in k for x in ("bwd_dq_kernel", "bwd_dkdv_kernel", "bwd_dq_split_kernel",
                                           "bwd_dkdv_split_kernel")))
    fe, fdur = dispatch_counters(fetch_dir)
    wr, _ = dispatch_counters(write_dir)
    copy = lambda d, c: max(mean(v[c]) for k, v in d.items() if "sage" not in k[0] and c in v)
    ff = COPY_BYTES / (copy(fe, "FETCH_SIZE") * 1024.0)
    fw = COPY_BYTES / (copy(wr, "WRITE_SIZE") * 1024.0)
    lines += ["", "## Prologue kernels on the headline workload (B=1 H=32 N=4096 d=128, INT8-QK / FP8-PV)", "",
              f"FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by {ff:.4f} and {fw:.4f}: the byte counts a",
              f"plain {COPY_BYTES >> 20} MiB device copy reads and writes in the same runs.  The durations are the",
              "counter runs' own dispatch timestamps (serialised dispatches), so the rates are a floor.", "",
              "| kernel | workgroups | HBM read (MB) | HBM write (MB) | duration (us) | GB/s |", "|---|---|---|---|---|---|"]
    for (k, g), cs in sorted(fe.items()):
        if not ("stats_kernel" in k or "quant_" in k) or (k, g) not in wr:
            continue
        rd = mean(cs["FETCH_SIZE"]) * 1024.0 * ff / 1e6
        wt = mean(wr[(k, g)]["WRITE_SIZE"]) * 1024.0 * fw / 1e6
        us = mean(fdur[(k, g)]) / 1e3
        lines.append(f"| `{k}` | {g} | {rd:.1f} | {wt:.1f} | {us:.1f} | {(rd + wt) * 1e3 / us:.0f} |")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counters(path, name):
    """Mean per-dispatch value of counter `name` for our fused kernel, and the copy kernel's value."""
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    per = {}
    kname = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != name:
                continue
            key = (f, r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
            kname[key] = r["Kernel_Name"]
    ours = [v for k, v in per.items() if "attn_fwd_kernel" in kname[k]]
    others = [v for k, v in per.items() if "sage" not in kname[k]]
    return sum(ours) / len(ours), max(others)


def traffic_summary(fetch_dir, write_dir):
    f_k, f_copy = counters(fetch_dir, "FETCH_SIZE")
    w_k, w_copy = counters(write_dir, "WRITE_SIZE")
    # the counters are in KiB; calibrate each by a plain copy of COPY_BYTES
    ff = COPY_BYTES / (f_copy * 1024.0)
    fw = COPY_BYTES / (w_copy * 1024.0)
    total = f_k * 1024.0 * ff + w_k * 1024.0 * fw
    lines = [
        "# HBM traffic of attn_fwd_kernel<128, INT8, causal, bf16> on the headline workload",
        "# (B=1 H=32 N=4096 d=128, causal, INT8-QK / FP8-PV), from two rocprofv3 counter runs:",
        "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -- python bench.py --steps 3 --warmup 1 --no-cpu --no-extra --copy-calib",
        "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write_dir> -- python bench.py --steps 3 --warmup 1 --no-cpu --no-extra --copy-calib",
        "#   python bench.py --traffic <fetch_dir> <write_dir>",
        "# Each counter (KiB per dispatch, averaged over the kernel's dispatches) is scaled by",
        f"# COPY_BYTES / (counter of a plain {COPY_BYTES >> 20} MiB device copy in the same run).",
        f"fetch_kib_per_launch={f_k:.1f}",
        f"write_kib_per_launch={w_k:.1f}",
        f"copy_fetch_kib={f_copy:.1f}",
        f"copy_write_kib={w_copy:.1f}",
        f"fetch_scale={ff:.4f}",
        f"write_scale={fw:.4f}",
        f"hbm_bytes_per_launch={total:.0f}",
        f"source_sha256_16={kernel_hash()}",
    ]
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def ktrace_summary(trace_dir, bench_json, out_path):
    """Markdown profile from a rocprofv3 --kernel-trace run of this script: per kernel and grid, the
    dispatch count and durations, beside the live HIP-event timing of the same run's JSON line."""
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
                   if "Grid_Size_X" in r else int(r["Grid_Size"]) // int(r["Workgroup_Size"]))
            per.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    live = json.loads(open(bench_json).read().strip().splitlines()[-1])
    head = "sage::attn_fwd_kernel<128, 1, true, 0, 2, false>"
    hd = per.get((head, 1024), [])
    lines = ["# Kernel trace: the forward hot path and the secondary workloads (bench.py)", "",
             "Commands (repository root, one MI355X):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d <trace_dir> -o k -- "
             "python -u bench.py --steps 20 --warmup 5 --no-cpu > <bench_json>",
             "    python bench.py --ktrace <trace_dir> <bench_json>", "",
             "The headline workload is B=1 H=32 N=4096 d=128, causal, INT8-QK / FP8-PV, bf16 I/O.  Template",
             "arguments: <head dim, QK format (1 INT8, 3 MXFP4), causal, I/O dtype, P~V format (2 FP8, 3 MXFP4,",
             "4 MXFP8, 5 fp16), finer INT8 steps>.", "",
             "## Headline fused kernel: trace vs. the live measurement of the same run", ""]
    if hd:
        lines += [f"- `{head}` on the headline grid (1024 workgroups): {len(hd)} dispatches, average "
                  f"{sum(hd) / len(hd):.1f} us, min {min(hd):.1f} us, max {max(hd):.1f} us (warm-up included).",
                  f"- bench.py's HIP events, kernel-only timed region: {1e3 * live['roofline']['kernel_ms']:.1f} us "
                  f"per launch ({live['roofline']['achieved']:.0f} TOPS, frac {live['roofline']['frac']:.3f}); "
                  f"full step {1e3 * live['ms_per_step']:.1f} us ({live['value']:.0f} TOPS).", ""]
    lines += ["## All kernels in the run", "", "| kernel | workgroups | calls | avg (us) | min (us) | max (us) |",
              "|---|---|---|---|---|---|"]
    for (k, g), v in sorted(per.items(), key=lambda kv: -sum(kv[1]) / len(kv[1])):
        lines.append(f"| `{k}` | {g} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} |")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def attn_ops(B, H, N, d, causal):
    ops = 4.0 * B * H * N * N * d
    return ops / 2 if causal else ops


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# Untimed back-to-back work before every timed region.  The GPU's clocks need tens of
# milliseconds of load to settle: measured on the headline step, the first 50-step region after
# 10 warmup steps ran at 182 us per step, the same region after 45 ms of load at 152 us, and
# after 2 s idle at 179 us again.  Throughput is quoted at the settled clocks.
WARM_S = 0.25


def time_region(fn, steps, warmup, torch):
    """At least `warmup` untimed steps, continued in synchronized batches until WARM_S seconds
    of back-to-back work have passed; then exactly `steps` steps timed with HIP events on the
    launch stream (torch's current stream, the one the library launches on)."""
    n, t_w = 0, time.perf_counter()
    while n < warmup or time.perf_counter() - t_w < WARM_S:
        for _ in range(20):
            fn()
        n += 20
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


MALL_EVICT_BYTES = 512 << 20    # twice the 256 MB Infinity Cache


def time_cold(fn, reps, torch, evict):
    """Average duration of single launches of fn, each after a 512 MB device write that evicts
    the Infinity Cache (so the launch reads its inputs from HBM); HIP events on the launch stream
    bracket the launch alone."""
    evs = []
    for i in range(reps):
        evict.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps


def run_workload(name, S, torch, steps, warmup, pv="fp8", qk=None):
    """Times the full step, the fused kernel alone and the prologue alone (HIP events on the launch stream)."""
    from bit_quantized_attention_smooth_amd.workloads import workload_inputs
    x, w = workload_inputs(name)
    dev = torch.device("cuda:0")
    g = {n: x[n].to(dev) for n in "qkv"}
    B, H, N, d, causal = w["B"], w["H"], w["N"], w["d"], w["causal"]
    qk = qk or w["qk_fmt"]
    p = S.problem(B, H, N, d, causal=causal, sm_scale=w["sm_scale"], dtype=g["q"].dtype, qk_fmt=qk, pv_fmt=pv)
    nbytes, _ = S.quant_size(p)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    o = torch.empty_like(g["q"])
    stream = S._stream()
    L = S.lib()
    import ctypes

    def step():
        S._check(L.sage_attn_fwd_ex(ctypes.byref(p), S._ptr(g["q"]), S._ptr(g["k"]), S._ptr(g["v"]), S._ptr(o),
                                    None, S._ptr(ws), nbytes, stream))

    def kernel():
        S._check(L.sage_attn_fwd_quantized(S._ptr(ws), nbytes, ctypes.byref(p), S._ptr(o), None, stream))

    def prologue():
        S._check(L.sage_quantize(S._ptr(g["q"]), S._ptr(g["k"]), S._ptr(g["v"]), ctypes.byref(p), S._ptr(ws),
                                 nbytes, stream))

    ms_step, wall = time_region(step, steps, warmup, torch)
    ms_kernel, _ = time_region(kernel, steps, warmup, torch)
    ms_pro, _ = time_region(prologue, steps, warmup, torch)
    evict = torch.empty(MALL_EVICT_BYTES, dtype=torch.uint8, device=dev)
    ms_pro_cold = time_cold(prologue, max(5, steps // 2), torch, evict)
    del evict
    ops = attn_ops(B, H, N, d, causal)
    E = B * H * N * d
    # prologue algorithmic bytes: read Q, K, V once (2 B each); write codes (1 B INT8/FP8, 0.5 B MXFP4)
    # plus the scales (INT8: 4 B per 64 tokens; MXFP4: 1 B per 32 elements) and the per-token LSE term
    # (MXFP4 V: 0.5 B codes + 1 B per 32 tokens and channel; MXFP8 V: 1 B codes + the same E8M0 bytes;
    # FP8 V: 1 B codes + a fp32 step per channel)
    v_b = {"fp8": E, "f16": 2 * E}.get(pv, (E // 2 if pv == "mxfp4" else E) + E // 32)
    code_b = (2 * E + v_b) if qk.startswith("int8") else (2 * (E // 2 + E // 32) + v_b)
    nqb = (N + 127) // 128     # per-block Q smoothing: a dS row per 128-query block
    scale_b = ({"int8": 2 * 4 * B * H * ((N + 63) // 64), "int8_token": 4 * B * H * (N + (N + 31) // 32),
                "mxfp4_qblock": 4 * B * H * N * nqb}.get(qk, 4 * B * H * N)) + \
        (4 * B * H * d if pv == "fp8" else 0) + 4 * B * H * N
    pro_bytes = 3 * 2 * E + code_b + scale_b
    return dict(name=name, B=B, H=H, N=N, d=d, causal=causal, qk=qk, pv=pv, ms_step=ms_step, wall=wall,
                ms_kernel=ms_kernel, ms_prologue=ms_pro, ms_prologue_cold=ms_pro_cold, ops=ops, pro_bytes=pro_bytes,
                dtype=w["dtype"], step_tops=ops / (ms_step * 1e-3) / 1e12, kernel_tops=ops / (ms_kernel * 1e-3) / 1e12,
                prologue_gbs=pro_bytes / (ms_pro * 1e-3) / 1e9,
                prologue_cold_gbs=pro_bytes / (ms_pro_cold * 1e-3) / 1e9)


def run_backward(name, S, torch, steps, warmup):
    """Forward (with LSE) and the 8-bit backward of the training workload."""
    import ctypes
    from bit_quantized_attention_smooth_amd.workloads import workload_inputs
    x, w = workload_inputs(name)
    dev = torch.device("cuda:0")
    g = {n: x[n].to(dev) for n in ("q", "k", "v", "do")}
    B, H, N, d, causal = w["B"], w["H"], w["N"], w["d"], w["causal"]
    p = S.problem(B, H, N, d, causal=causal, sm_scale=w["sm_scale"], dtype=g["q"].dtype)
    L = S.lib()
    nf, nb = ctypes.c_size_t(), ctypes.c_size_t()
    S._check(L.sage_attn_fwd_ws_size(ctypes.byref(p), ctypes.byref(nf)))
    S._check(L.sage_attn_bwd_ws_size(ctypes.byref(p), ctypes.byref(nb)))
    wsf = torch.empty(nf.value, dtype=torch.uint8, device=dev)
    wsb = torch.empty(nb.value, dtype=torch.uint8, device=dev)
    o = torch.empty_like(g["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(g["q"]) for _ in range(3))
    st = S._stream()

    def fwd():
        S._check(L.sage_attn_fwd_ex(ctypes.byref(p), S._ptr(g["q"]), S._ptr(g["k"]), S._ptr(g["v"]), S._ptr(o),
                                    S._ptr(lse), S._ptr(wsf), nf.value, st))

    def bwd():
        S._check(L.sage_attn_bwd(ctypes.byref(p), S._ptr(g["q"]), S._ptr(g["k"]), S._ptr(g["v"]), S._ptr(o),
                                 S._ptr(g["do"]), S._ptr(lse), S._ptr(dq), S._ptr(dk), S._ptr(dv), S._ptr(wsb),
                                 nb.value, st))

    def bwd_after_fwd():
        # the training step's backward: the forward quantized into wsb (below), and that
        # quantization of Q and K is reused (the backward does not modify it)
        S._check(L.sage_attn_bwd_after_fwd(ctypes.byref(p), S._ptr(g["q"]), S._ptr(g["k"]), S._ptr(g["v"]), S._ptr(o),
                                           S._ptr(g["do"]), S._ptr(lse), S._ptr(dq), S._ptr(dk), S._ptr(dv),
                                           S._ptr(wsb), nb.value, st))

    ms_f, _ = time_region(fwd, steps, warmup, torch)
    fwd()
    ms_b, _ = time_region(bwd, steps, warmup, torch)
    S._check(L.sage_attn_fwd_ex(ctypes.byref(p), S._ptr(g["q"]), S._ptr(g["k"]), S._ptr(g["v"]), S._ptr(o),
                                S._ptr(lse), S._ptr(wsb), nb.value, st))
    ms_r, _ = time_region(bwd_after_fwd, steps, warmup, torch)
    ops_f = attn_ops(B, H, N, d, causal)
    ops_b = 2.5 * ops_f          # 10 d ops per (query, key) pair vs 4 d in the forward
    return {"fwd_ms": round(ms_f, 4), "fwd_tops": round(ops_f / (ms_f * 1e-3) / 1e12, 1),
            "bwd_ms": round(ms_b, 4), "bwd_tops": round(ops_b / (ms_b * 1e-3) / 1e12, 1),
            "bwd_frac": round(ops_b / (ms_b * 1e-3) / 1e12 / PEAK["int8_fp8"], 4),
            "bwd_after_fwd_ms": round(ms_r, 4), "bwd_after_fwd_tops": round(ops_b / (ms_r * 1e-3) / 1e12, 1),
            "bwd_after_fwd_frac": round(ops_b / (ms_r * 1e-3) / 1e12 / PEAK["int8_fp8"], 4)}


def run_varlen(name, S, torch, steps, warmup):
    """Packed prefill step (prologue + fused kernel through sage_attn_varlen_fwd)."""
    import ctypes
    from bit_quantized_attention_smooth_amd.workloads import varlen_workload
    x, w = varlen_workload(name)
    dev = torch.device("cuda:0")
    g = {n: x[n].to(dev) for n in ("q", "k", "v", "cu_q", "cu_k")}
    T, H, Hkv, d = w["T"], w["H"], w["Hkv"], w["d"]
    p = S.varlen_problem(w["B"], H, Hkv, d, T, T, w["max_seqlen"], w["max_seqlen"], causal=w["causal"],
                         sm_scale=w["sm_scale"], dtype=g["q"].dtype)
    L = S.lib()
    n = ctypes.c_size_t()
    S._check(L.sage_varlen_ws_size(ctypes.byref(p), ctypes.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device=dev)
    o = torch.empty_like(g["q"])
    st = S._stream()

    def step():
        S._check(L.sage_attn_varlen_fwd(ctypes.byref(p), S._ptr(g["q"]), S._ptr(g["k"]), S._ptr(g["v"]),
                                        S._ptr(g["cu_q"]), S._ptr(g["cu_k"]), S._ptr(o), None, S._ptr(ws), n.value,
                                        st))

    ms, _ = time_region(step, steps, warmup, torch)
    ops = sum(attn_ops(1, H, n_b, d, w["causal"]) for n_b in w["lens"])
    return {"step_ms": round(ms, 4), "step_tops": round(ops / (ms * 1e-3) / 1e12, 1),
            "sequences": w["lens"], "heads": f"{H} query / {Hkv} KV"}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(name):
    """The CPU oracle (prologue + tiled quantized forward) over every head of the workload with
    every host thread (about 40 core-seconds on 16 cores), plus four heads on one thread (the
    per-core rate, about 5 s)."""
    import oracle
    from bit_quantized_attention_smooth_amd.workloads import workload_inputs, as_u16
    x, w = workload_inputs(name)
    B, H, N, d, causal, sm = w["B"], w["H"], w["N"], w["d"], w["causal"], w["sm_scale"]
    nh = B * H
    f = {n: oracle.widen(as_u16(x[n].reshape(B * H, N, d)[:nh]), w["dtype"]).reshape(nh, N, d) for n in "qkv"}
    oracle.lib()
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        cores = min(cores, int(omp))
    threads = oracle.set_threads(cores)

    def run(heads):
        t0 = time.perf_counter()
        qz = oracle.quant_int8_fp8(f["q"][:heads], f["k"][:heads], f["v"][:heads], sm)
        oracle.attn_int8_fp8(qz, N, d, causal, sm, 64)
        return time.perf_counter() - t0

    dt = run(nh)
    oracle.set_threads(1)
    n1 = min(4, nh)
    dt1 = run(n1)
    oracle.set_threads(threads)
    ops = attn_ops(1, nh, N, d, causal)
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "single_thread": {"value": attn_ops(1, n1, N, d, causal) / dt1 / 1e12, "unit": "TOPS", "cores": 1,
                              "sample": f"heads 0-{n1 - 1} of {name}, all {N} query rows, {dt1:.1f} s"},
            "sample": f"{nh} of {B * H} heads of {name}, all {N} query rows: prologue + tiled INT8/FP8 forward "
                      f"(fp64), {dt:.1f} s on {threads} threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--copy-calib", action="store_true", help="run one 1 GiB device copy at the end (counter calibration)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the roofline traffic summary from two rocprofv3 counter runs and exit")
    ap.add_argument("--ktrace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                    help="write the kernel-trace profile summary from a rocprofv3 --kernel-trace run and exit")
    ap.add_argument("--counters", nargs=3, metavar=("SQ_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the MFMA-busy / prologue-HBM profile summary from rocprofv3 counter runs and exit")
    args = ap.parse_args()
    if args.counters:
        counter_summary(*args.counters, os.path.join(ROOT, "profiles", "counters_attn_fwd_attn_bwd_and_prologue.md"))
        return
    if args.ktrace:
        ktrace_summary(*args.ktrace, os.path.join(ROOT, "profiles", "attn_fwd_int8_fp8_causal_b1h32n4096d128.md"))
        return
    if args.traffic:
        traffic_summary(*args.traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (heads shard over GPUs without "
              f"exchange, so N GPUs would run N independent copies of this step)", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_quantized_attention_smooth_amd as S
    S.lib()
    log(f"[bench] headline {HEADLINE}: steps={args.steps} warmup={args.warmup}")
    r = run_workload(HEADLINE, S, torch, args.steps, args.warmup)
    log(f"[bench] step {r['ms_step']:.4f} ms  kernel {r['ms_kernel']:.4f} ms  prologue {r['ms_prologue']:.4f} ms")
    path = "int8_fp8" if r["qk"] == "int8" else "mxfp4_fp8"
    achieved = r["kernel_tops"]
    out = {
        "metric": METRIC, "value": round(r["step_tops"], 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8+fp8",
        "timing": f"each timed region follows >= {args.warmup} untimed steps and >= {WARM_S} s of back-to-back "
                  f"untimed work (settled GPU clocks)",
        "data": "synthetic (seeded normal Q/K/V, K channel offsets, 1% outlier channels)",
        "config": {"workload": HEADLINE, "B": r["B"], "H": r["H"], "N": r["N"], "d": r["d"], "causal": r["causal"],
                   "qk_fmt": r["qk"], "pv_fmt": r["pv"], "io_dtype": r["dtype"], "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK[path], "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK[path], 4), "traffic": read_traffic(),
                     "kernel": "attn_fwd_kernel<128, INT8, causal, bf16>", "kernel_ms": round(r["ms_kernel"], 5)},
        "prologue": {"ms": round(r["ms_prologue_cold"], 5), "algorithmic_bytes": r["pro_bytes"],
                     "GB/s": round(r["prologue_cold_gbs"], 1),
                     "frac_of_hbm": round(r["prologue_cold_gbs"] / HBM_PEAK_GBS, 4),
                     "timing": "single launches, each after a 512 MB write that evicts the 256 MB Infinity Cache",
                     "back_to_back": {"ms": round(r["ms_prologue"], 5), "GB/s": round(r["prologue_gbs"], 1),
                                      "note": "inputs partly served by the Infinity Cache"}},
    }
    if not args.no_extra:
        extra = {}
        for name, pv, *qk in (("int8_fp8_b1h32n8192d128", "fp8"), ("int8_fp8_b1h32n8192d128", "f16"),
                              ("int8_fp8_causal_b1h32n4096d128", "fp8", "int8_token"),
                              ("int8_fp8_causal_b1h32n16384d128", "fp8"),
                         ("mxfp4_b4h32n8192d128", "fp8"), ("mxfp4_b4h32n8192d128", "fp8", "mxfp4_qblock"),
                         ("mxfp4_b4h32n8192d128", "mxfp4"),
                         ("mxfp4_b4h32n8192d128", "mxfp8"), ("int8_fp8_b2h24n16384d64", "fp8")):
            qk = qk[0] if qk else None
            log(f"[bench] secondary {name} (P~V {pv}{', QK ' + qk if qk else ''})")
            e = run_workload(name, S, torch, max(5, args.steps // 5), 3, pv=pv, qk=qk)
            # FP8 and MXFP8 V both run the P~V product on the FP8 matrix path
            pk = PEAK[("int8_f16" if pv == "f16" else "int8_fp8") if e["qk"].startswith("int8") else
                      ("mxfp4_mxfp4" if pv == "mxfp4" else "mxfp4_fp8")]
            key = (name if pv == "fp8" else name + "+pv_" + pv) + ("+qk_" + qk if qk else "")
            extra[key] = {"kernel_tops": round(e["kernel_tops"], 1), "frac": round(e["kernel_tops"] / pk, 4),
                           "step_tops": round(e["step_tops"], 1), "kernel_ms": round(e["ms_kernel"], 4),
                           "prologue_GB/s": round(e["prologue_gbs"], 1),
                           "prologue_cold_GB/s": round(e["prologue_cold_gbs"], 1)}
            if e["d"] == 128 and e["N"] >= 8192:
                # the d = 128, N >= 8192 points (and the long causal prefill): the kernel against its own roofline; for
                # MXFP4 QK both the format-mix peak and the literal MXFP4 peak
                rb = {"bound": "mfma", "achieved": round(e["kernel_tops"], 2), "peak": round(pk, 1),
                      "unit": "TFLOP/s", "frac": round(e["kernel_tops"] / pk, 4), "traffic": None,
                      "kernel_ms": round(e["ms_kernel"], 5)}
                if not e["qk"].startswith("int8"):
                    rb["peak_note"] = ("MXFP4 QK + MXFP4 P~V: 10.1 P" if pv == "mxfp4" else
                                       "MXFP4 QK + FP8 P~V: harmonic mix of 10.1 P and 5.0 P (half the ops each)")
                    rb["frac_of_mxfp4_peak"] = round(e["kernel_tops"] / PEAK["mxfp4_mxfp4"], 4)
                extra[key]["roofline"] = rb
            torch.cuda.empty_cache()
        log("[bench] secondary varlen_gqa_causal_b8h32kv8t16384d128 (packed sequences, grouped KV heads)")
        extra["varlen_gqa_causal_b8h32kv8t16384d128"] = run_varlen("varlen_gqa_causal_b8h32kv8t16384d128", S, torch,
                                                                   max(5, args.steps // 5), 3)
        torch.cuda.empty_cache()
        log("[bench] secondary train_causal_b8h16n2048d64 (forward + 8-bit backward)")
        extra["train_causal_b8h16n2048d64"] = run_backward("train_causal_b8h16n2048d64", S, torch,
                                                           max(5, args.steps // 5), 3)
        torch.cuda.empty_cache()
        log("[bench] secondary train_causal_b8h16n2048d128 (forward + 8-bit backward, d = 128)")
        extra["train_causal_b8h16n2048d128"] = run_backward("train_causal_b8h16n2048d128", S, torch,
                                                            max(5, args.steps // 5), 3)
        out["other_workloads"] = extra
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(HEADLINE)
    if args.copy_calib:
        log("[bench] copy calibration: 1 GiB read + 1 GiB write elementwise kernel")
        src = torch.zeros(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
