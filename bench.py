#!/usr/bin/env python3
"""Benchmark of the fused attention forward pass on one MI355X.

One step = one call of the library's forward entry point over the whole
workload (all of: Q/K/V tile loads, both MFMA products, the online softmax,
the masked tiles and the epilogue run inside that one kernel).  Inputs are
synthetic (seeded N(0,1), rounded to the working dtype) and resident in HBM
before the timed region starts.

Prints ONE JSON line on stdout:
  metric / value / unit   causal-adjusted TFLOP/s of the workload
  roofline                the kernel's achieved TFLOP/s against the dense
                          MFMA peak of its dtype (from per-launch HIP events on
                          the stream the kernel is launched on), plus measured
                          HBM traffic when the counter file matches the kernel
  cpu_baseline            the CPU oracle timed on a bounded sample of rows of
                          the same workload, on this host's cores

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--calibrate-copy BYTES]
       python bench.py --traffic-summary FETCH_CSV WRITE_CSV --copy-bytes BYTES

HBM traffic: run the bench twice under `rocprofv3 --pmc FETCH_SIZE` and
`rocprofv3 --pmc WRITE_SIZE` with --calibrate-copy BYTES, which first copies
BYTES bytes device-to-device.  The counters read for that plain copy give
the factor between counter units and bytes moved; --traffic-summary applies
it to the attention kernel's dispatches and writes profiles/hbm_traffic.json,
which later bench runs report as roofline.traffic (only while the kernel
sources still hash to the value recorded there).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "attention fwd TFLOP/s (causal-adjusted) and % of bf16 MFMA peak, 1 GPU"
METRIC_BWD = ("attention bwd TFLOP/s (causal-adjusted, 2.5x the forward's FLOPs: five products) "
              "and % of bf16 MFMA peak, 1 GPU")
# Published HBM3E bandwidth of one MI355X (GB/s): the bound of memory-bound
# (decode-shaped) calls, whose FLOPs per byte sit below the ridge.
PEAK_HBM_GBS = 8000.0
# Published dense MFMA peak of one MI355X for bf16 and fp16 (TFLOP/s).  The
# bench also prints the peak that the device's own compute-unit count and
# peak clock give (device_peak), beside this one.
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_code_hash(kernel: str):
    """sha256 (16 hex digits) of the generated instructions of `kernel` (its
    assembly up to the kernel descriptor; for the HIP C++ tile kernels, their
    source files), or None for a name neither makes.  Counter figures taken
    on other instructions no longer describe the kernel."""
    sys.path.insert(0, ROOT)
    try:
        from attention_forward_05_amd.asm.fa_fwd_gen import Gen
        from attention_forward_05_amd.asm.fa_fwd_x8 import Gen8
    finally:
        sys.path.pop(0)
    if "tile_kernel" in kernel:
        # the HIP C++ tile kernels (and the merge after a split): their sources
        srcs = ["fa_tile.hip", "fa_mfma.h", "fa_combine.hip"]
        h = hashlib.sha256()
        for s in srcs:
            with open(os.path.join(ROOT, "attention_forward_05_amd", "csrc", s), "rb") as f:
                h.update(f.read())
        return h.hexdigest()[:16]
    parts = kernel.split("_")   # fa_fwd_<dt>_d<D>[_x8|_x8s]_gfx950
    if len(parts) < 5 or parts[:2] != ["fa", "fwd"] or parts[-1] != "gfx950":
        return None
    dt, D, shape = parts[2], int(parts[3][1:]), parts[4:-1]
    if shape == []:
        gen = Gen(dt, D)
    elif shape in (["x8"], ["x8s"]):
        gen = Gen8(dt, shape == ["x8s"], D)
    else:
        return None
    text = gen.assemble_text()[0]
    code = text[:text.index(".amdhsa_kernel")]
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def measured_traffic(workload_name: str, kernel: str):
    """Bytes per launch from the committed counter summary, or None when the
    file is absent or its figures were taken on other instructions."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get("workloads", {}).get(workload_name)
    if not entry or entry.get("kernel") != kernel:
        return None
    if entry.get("kernel_code_sha256_16") != kernel_code_hash(kernel):
        return None
    return entry.get("bytes_per_launch")


def launched_kernel(w: workloads.Workload, cus: int) -> str:
    """Name of the kernel the library launches for this workload on a device
    with `cus` compute units, from the library's own plan query (with split
    key ranges a merge kernel follows it)."""
    import attention_forward_05_amd as fa
    st, kern, ranges, _ = fa.fa_fwd_plan(w.B, w.Sq, w.Skv, w.Hq, w.Hkv, w.D, int(w.causal), cus,
                                         True)
    if st != fa.FA_OK:
        raise fa.FAError(st, "fa_fwd_plan")
    merge = f" ({ranges} key ranges) + combine_kernel" if ranges > 1 else ""
    if kern == fa.FA_KERNEL_TILE_ROWS:
        return f"fwd_tile_kernel<{w.dtype}, D={w.D}, rows>{merge}"
    if kern == fa.FA_KERNEL_TILE_KEYS:
        return f"fwd_tile_kernel<{w.dtype}, D={w.D}, keys>{merge}"
    if kern == fa.FA_KERNEL_FOUR_WAVE:
        return f"fa_fwd_{w.dtype}_d{w.D}_gfx950"
    if ranges == 1:
        return f"fa_fwd_{w.dtype}_d{w.D}_x8_gfx950"
    return f"fa_fwd_{w.dtype}_d128_x8s_gfx950{merge}"


def device_peak(dtype: str):
    """Compute units and peak shader clock of device 0, read from the HIP
    runtime torch has loaded, and the dense MFMA peak they give
    (4096 bf16/fp16 FLOP per clock per compute unit: 4 SIMDs x 1024)."""
    import ctypes
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                path = line.split()[-1]
                break
    if path is None:
        return None
    hip = ctypes.CDLL(path)
    val = ctypes.c_int(0)
    # hipDeviceAttributeClockRate = 5 (kHz), hipDeviceAttributeMultiprocessorCount = 63
    if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, 0) != 0:
        return None
    khz = val.value
    if hip.hipDeviceGetAttribute(ctypes.byref(val), 63, 0) != 0:
        return None
    cus = val.value
    flop_per_clk_cu = 4096 if dtype in ("bf16", "f16") else None
    return {"compute_units": cus, "max_sclk_mhz": khz / 1e3,
            "peak_tflops_from_clock": round(cus * flop_per_clk_cu * khz * 1e3 / 1e12, 1)}


def algorithmic_bytes(w: workloads.Workload) -> int:
    """Bytes one launch must move at least: Q, K, V read once, O and LSE
    written once."""
    el = 2
    return (2 * w.B * w.Sq * w.Hq * w.D * el + 2 * w.B * w.Skv * w.Hkv * w.D * el
            + 4 * w.B * w.Hq * w.Sq)


def _pmc_rows(path):
    """(kernel name, dispatch id, counter value) of every row of a rocprofv3
    counter-collection CSV."""
    import csv
    out = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            out.append((row["Kernel_Name"], row.get("Dispatch_Id", ""), float(row["Counter_Value"])))
    return out


def traffic_summary(fetch_csv: str, write_csv: str, copy_bytes: int, workload_name: str):
    """Scale the attention kernel's FETCH_SIZE / WRITE_SIZE (KiB) by what the
    same counters read for the calibration copy of `copy_bytes` bytes."""
    res = {}
    for key, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = _pmc_rows(path)
        # per dispatch: sum the counter's rows (one per counter instance)
        per = {}
        for name, did, val in rows:
            per.setdefault((name, did), 0.0)
            per[(name, did)] += val
        def is_attn(n):
            return n.startswith("fa_fwd_") or "fwd_tile_kernel" in n

        fa_vals = [v for (n, _), v in per.items() if is_attn(n)]
        others = [(v, n) for (n, _), v in per.items() if not is_attn(n) and "combine" not in n]
        if not fa_vals or not others:
            raise SystemExit(f"{path}: no attention or no copy dispatch found")
        copy_kib, copy_name = max(others)
        factor = copy_kib * 1024.0 / copy_bytes
        res[key] = {"kernel_kib_avg": sum(fa_vals) / len(fa_vals), "dispatches": len(fa_vals),
                    "copy_kib": copy_kib, "copy_kernel": copy_name,
                    "factor_counter_bytes_per_byte": factor,
                    "bytes": sum(fa_vals) / len(fa_vals) * 1024.0 / factor}
    w = workloads.get(workload_name)
    return {
        "bytes_per_launch": round(res["fetch"]["bytes"] + res["write"]["bytes"]),
        "fetch_bytes": round(res["fetch"]["bytes"]),
        "write_bytes": round(res["write"]["bytes"]),
        "algorithmic_bytes": algorithmic_bytes(w),
        "copy_bytes": copy_bytes,
        "fetch": res["fetch"],
        "write": res["write"],
    }


def counter_summary(csv_path: str, w: workloads.Workload, which: str = "fwd"):
    """Per-dispatch averages of the counters in a rocprofv3 counter-collection
    CSV for the attention kernels, and the figures derived from them:
    MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES summed over all instances / (GPU
    clocks x SIMDs), the GPU clocks being GRBM_GUI_ACTIVE summed over its
    one-per-XCD instances / XCDs (counts from the run's agent info); LDS
    bank-conflict cycles per LDS-active cycle; GPU clock = GRBM_GUI_ACTIVE /
    dispatch duration;
    executed MFMA FLOPs = MOPS x 512 against the algorithmic count; and
    transcendental instructions x 64 lanes against the exponentials the
    method needs (one per visible (query, key) pair)."""
    import csv
    per = {}
    names = {}
    durations = {}
    for row in csv.DictReader(open(csv_path, newline="")):
        name = row["Kernel_Name"]
        if not (name.startswith(("fa_fwd_", "fa_bwd_")) or "tile_kernel" in name
                or "combine_kernel" in name or "bwd_" in name):
            continue
        did = row.get("Dispatch_Id", "")
        cname, val = row["Counter_Name"], float(row["Counter_Value"])
        per.setdefault(did, {}).setdefault(cname, 0.0)
        # rocprofv3 sums a counter's instances: for the per-SE / per-SIMD SQ
        # counters that is the whole chip's count; GRBM_GUI_ACTIVE has one
        # instance per XCD, each counting the same clocks (divided below)
        per[did][cname] += val
        names[did] = name
        if row.get("Start_Timestamp") and row.get("End_Timestamp"):
            durations[did] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
    kernels = sorted(set(names.values()))
    # the device's XCD and SIMD counts and peak clock, from the run's agent info
    xcc, simds, max_mhz = 8, 1024, None
    info = csv_path.replace("_counter_collection.csv", "_agent_info.csv")
    if os.path.exists(info):
        for row in csv.DictReader(open(info, newline="")):
            if int(row.get("Simd_Count", "0") or 0) > 0:
                xcc, simds = int(row["Num_Xcc"]), int(row["Simd_Count"])
                max_mhz = float(row.get("Max_Engine_Clk_Fcompute", 0) or 0) or None
    out = {"csv": os.path.basename(csv_path), "xcd": xcc, "simds": simds,
           "max_engine_clock_mhz": max_mhz, "kernels": {}}
    for kname in kernels:
        ds = [d for d in per if names[d] == kname]
        keys = sorted({c for d in ds for c in per[d]})
        avg = {c: sum(per[d].get(c, 0.0) for d in ds) / len(ds) for c in keys}
        if "GRBM_GUI_ACTIVE" in avg:
            avg["GRBM_GUI_ACTIVE"] /= xcc  # GPU clocks of the dispatch
        entry = {"dispatches": len(ds), "counters_avg_per_dispatch": avg}
        durs = [durations[d] for d in ds if d in durations]
        if durs and avg.get("GRBM_GUI_ACTIVE"):
            entry["dispatch_avg_us"] = round(sum(durs) / len(durs) / 1e3, 2)
            entry["gpu_clock_mhz"] = round(avg["GRBM_GUI_ACTIVE"] / (sum(durs) / len(durs)) * 1e3, 1)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and avg.get("GRBM_GUI_ACTIVE"):
            entry["mfma_busy_pct"] = round(100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"]
                                           / (avg["GRBM_GUI_ACTIVE"] * simds), 2)
        if avg.get("SQ_LDS_IDX_ACTIVE"):
            entry["lds_bank_conflict_per_active_cycle"] = round(
                avg.get("SQ_LDS_BANK_CONFLICT", 0.0) / avg["SQ_LDS_IDX_ACTIVE"], 5)
        flops = workloads.attention_flops(w.B, w.Sq, w.Skv, w.Hq, w.D, w.causal)
        if which == "bwd":
            flops *= 2.5
        mops = avg.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + avg.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)
        if mops:
            entry["mfma_flops_executed"] = mops * 512
            entry["mfma_flops_over_algorithmic"] = round(mops * 512 / flops, 4)
        if "SQ_INSTS_VALU_TRANS_F32" in avg:
            exps = flops / (4.0 * w.D) * (1.0 if which == "fwd" else 1.0 / 2.5)
            entry["trans_f32_lanes"] = avg["SQ_INSTS_VALU_TRANS_F32"] * 64
            entry["exp_needed"] = exps
            entry["trans_lanes_over_exp"] = round(avg["SQ_INSTS_VALU_TRANS_F32"] * 64 / exps, 4)
        out["kernels"][kname] = entry
    return out


def cpu_baseline(w: workloads.Workload, q, k, v, target_s: float = 12.0):
    """Time the CPU oracle on uniformly sampled rows of the workload and
    scale to TFLOP/s with the same per-row FLOP count as the GPU metric."""
    import numpy as np
    import oracle

    rng = np.random.default_rng(1234)
    n_rows_total = w.B * w.Hq * w.Sq

    def rows_and_flops(n):
        r = np.stack([rng.integers(0, w.B, n), rng.integers(0, w.Hq, n),
                      rng.integers(0, w.Sq, n)], axis=1).astype(np.int64)
        i = r[:, 2]
        if w.causal:
            vis = np.clip(i + (w.Skv - w.Sq) + 1, 0, w.Skv)
        else:
            vis = np.full(n, w.Skv)
        return r, float((4.0 * w.D * vis).sum())

    # widen once (not timed: the oracle's inputs are fp64 arrays)
    qd, kd, vd = oracle._f64(q), oracle._f64(k), oracle._f64(v)
    # two pilots size the sample: 64 rows, then about a second's worth (the
    # first overstates the time per row: thread start-up dominates it)
    n = 64
    for budget in (1.0, target_s):
        r, fl = rows_and_flops(n)
        t0 = time.perf_counter()
        oracle.attn_rows(qd, kd, vd, w.causal, w.scale, r)
        t_pilot = max(time.perf_counter() - t0, 1e-3)
        n = int(min(n_rows_total, max(64, n * budget / t_pilot)))
    r, fl = rows_and_flops(n)
    t0 = time.perf_counter()
    oracle.attn_rows(qd, kd, vd, w.causal, w.scale, r)
    dt = time.perf_counter() - t0
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"{n} of {n_rows_total} query rows drawn uniformly over (b, hq, i); "
                  f"{fl / 1e9:.1f} GFLOP in {dt:.2f} s (fp64, OpenMP over rows)",
    }


def cpu_baseline_bwd(w: workloads.Workload, q, k, v, target_s: float = 12.0):
    """Time the CPU oracle's backward on whole (batch, kv-head group) slices
    of the workload -- every row and key of the q-heads of one kv-head --
    adding slices until about target_s seconds, and scale to TFLOP/s with the
    backward's FLOP count (2.5x the forward's) of those slices."""
    import numpy as np
    import torch
    import oracle

    gen = torch.Generator().manual_seed(w.seed + 1000)
    do = torch.randn(q.shape, generator=gen, dtype=torch.float32).to(q.dtype)
    g = w.Hq // w.Hkv
    slices, t_used, fl = 0, 0.0, 0.0
    total = w.B * w.Hkv
    while slices < total and t_used < target_s:
        b, hk = divmod(slices, w.Hkv)
        hs = slice(hk * g, (hk + 1) * g)
        qs = oracle._f64(q[b:b + 1, :, hs])
        ks = oracle._f64(k[b:b + 1, :, hk:hk + 1])
        vs = oracle._f64(v[b:b + 1, :, hk:hk + 1])
        ds = oracle._f64(do[b:b + 1, :, hs])
        t0 = time.perf_counter()
        oracle.attn_bwd(qs, ks, vs, ds, w.causal, w.scale)
        t_used += time.perf_counter() - t0
        fl += 2.5 * workloads.attention_flops(1, w.Sq, w.Skv, g, w.D, w.causal)
        slices += 1
    del np
    return {
        "value": fl / t_used / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"{slices} of {total} (batch, kv-head) slices, each with its {g} q-heads, all "
                  f"rows and keys; {fl / 1e9:.1f} GFLOP (2.5x forward count) in {t_used:.2f} s "
                  "(fp64, OpenMP over rows and keys)",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=workloads.HEADLINE.name,
                    help="a named workload (" + ", ".join(workloads.BY_NAME) + ") or an ad-hoc "
                    "shape B,Hq,Hkv,Sq,Skv,D,causal,dtype")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward pass (default) or the backward pass (fa_bwd)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="first copy BYTES bytes device-to-device (HBM counter calibration)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--counter-summary", nargs="+", metavar="CSV",
                    help="summarise rocprofv3 counter CSVs of this workload's attention kernels")
    ap.add_argument("--compute-units", type=int, default=256,
                    help="with --traffic-summary: compute units of the profiled device")
    args = ap.parse_args()

    if args.counter_summary:
        w = workloads.get(args.workload)
        for path in args.counter_summary:
            print(json.dumps(counter_summary(path, w, args.which), indent=1))
        return

    if args.traffic_summary:
        entry = traffic_summary(args.traffic_summary[0], args.traffic_summary[1],
                                args.copy_bytes, args.workload)
        kernel = launched_kernel(workloads.get(args.workload), args.compute_units)
        entry["kernel"] = kernel
        entry["kernel_code_sha256_16"] = kernel_code_hash(kernel)
        try:
            with open(TRAFFIC_FILE) as f:
                doc = json.load(f)
        except (OSError, ValueError):
            doc = {}
        doc.setdefault("workloads", {})[args.workload] = entry
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(doc, f, indent=1, sort_keys=True)
            f.write("\n")
        print(json.dumps(entry))
        return

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the kernel has no multi-GPU path to time.", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_forward_05_amd as fa

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    fa.load()

    w = workloads.get(args.workload)
    dev = torch.device("cuda:0")
    if args.calibrate_copy > 0:
        src = torch.ones(args.calibrate_copy, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    q, k, v = workloads.workload_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    od = torch.empty_like(qd)
    lsed = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # the workspace for split key ranges, allocated before the timed region
    _, _, _, ws_bytes = fa.fa_fwd_plan(w.B, w.Sq, w.Skv, w.Hq, w.Hkv, w.D, int(w.causal), cus,
                                       True)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    dt = fa.FA_DTYPE_BF16 if w.dtype == "bf16" else fa.FA_DTYPE_F16

    def step():
        st = fa.fa_fwd_ws(dt, qd, kd, vd, od, lsed, w.B, w.Sq, w.Skv, w.Hq, w.Hkv, w.D,
                          int(w.causal), w.scale, ws, ws_bytes, sh)
        if st != fa.FA_OK:
            raise fa.FAError(st, "fa_fwd_ws")

    if args.which == "bwd":
        # the forward's O and LSE, an upstream gradient, the gradients and
        # the workspace (l2 and delta per query row), all before the timed region
        step()
        gen = torch.Generator().manual_seed(w.seed + 1000)
        dod = torch.randn(q.shape, generator=gen, dtype=torch.float32).to(q.dtype).to(dev)
        dqd, dkd, dvd = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        bws = torch.empty(max(8 * w.B * w.Hq * w.Sq, 16), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

        def step():  # noqa: F811 -- the timed step is the backward pass
            st = fa.fa_bwd(dt, qd, kd, vd, od, lsed, dod, dqd, dkd, dvd, w.B, w.Sq, w.Skv, w.Hq,
                           w.Hkv, w.D, int(w.causal), w.scale, bws, bws.numel(), sh)
            if st != fa.FA_OK:
                raise fa.FAError(st, "fa_bwd")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole timed region
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps

    # per-launch durations (same stream), for the roofline figure
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    launch_ms = sorted(a.elapsed_time(b) for a, b in evs)
    launch_avg_ms = sum(launch_ms) / len(launch_ms)

    flops = workloads.attention_flops(w.B, w.Sq, w.Skv, w.Hq, w.D, w.causal)
    if args.which == "bwd":
        flops *= 2.5
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (launch_avg_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    kernel = launched_kernel(w, cus) if args.which == "fwd" else \
        f"bwd_delta_kernel + fa_bwd_dkv_{w.dtype}_d{w.D}_gfx950 + fa_bwd_dq_{w.dtype}_d{w.D}_gfx950"
    dev_peak = device_peak(w.dtype)
    traffic = measured_traffic(w.name, kernel) if args.which == "fwd" else None
    log(f"[bench] {w.name} ({args.which}): {ms_per_step * 1e3:.1f} us/step, {value:.1f} TFLOP/s "
        f"({100 * value / peak:.1f}% of {peak:.0f}); launch avg {launch_avg_ms * 1e3:.1f} us, "
        f"min {launch_ms[0] * 1e3:.1f} us, median {launch_ms[len(launch_ms) // 2] * 1e3:.1f} us")
    # the bound: matrix cores, unless the call's FLOPs per algorithmic byte
    # sit below the ridge (peak FLOP/s over HBM bandwidth): then HBM
    abytes = algorithmic_bytes(w) if args.which == "fwd" else None
    if abytes and flops / abytes < peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        gbs = abytes / (launch_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                "algorithmic_bytes": abytes}
        log(f"[bench] memory-bound: {gbs:.0f} GB/s of algorithmic bytes ({abytes / 1e6:.1f} MB)")
    else:
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic}
    roof.update({
        "kernel_launch_avg_us": round(launch_avg_ms * 1e3, 2),
        "timing": f"HIP events around each of {args.steps} launches on the launch stream",
        "kernel": kernel,
        "device": dev_peak,
    })

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        cpu = cpu_baseline(w, q, k, v) if args.which == "fwd" else cpu_baseline_bwd(w, q, k, v)
        log(f"[bench] cpu oracle: {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC if args.which == "fwd" else METRIC_BWD,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs rounded to the dtype, resident in HBM)",
        "config": {
            "workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq,
            "Skv": w.Skv, "D": w.D, "causal": w.causal, "scale": w.scale,
            "flops_per_step": flops, "parallelism": "single GPU",
        },
        "pct_of_peak": round(100 * value / peak, 2),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if args.which == "bwd":
        out["config"]["pass"] = "bwd"
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
