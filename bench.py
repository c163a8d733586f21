#!/usr/bin/env python3
"""Throughput of the KroQuant online quantizer on one MI355X.

One step = one kq_quantize pass over the largest single-GPU workload: the
65536 x 12288 bf16 activation of the bandwidth sweep (N(0,1), 1% outlier
channels x50, 0.1% each of all-zero, subnormal, near-min-normal and exact-tie
blocks; synthetic, from synth/inputs.py), with the configured
[[1,1],[1,-1]]/sqrt(2) factors (the normalised Walsh-Hadamard-32 block,
shared by every block): bf16 -> Kronecker transform -> MXFP4 codes + E8M0
scales.

  value     = algorithmic bytes of the K timed steps / their wall time (GB/s)
              algorithmic bytes = 2.53125 B per element (2 read, 0.5 + 1/32 written)
  roofline  = the quantizer kernel's average launch against the 8 TB/s HBM peak,
              timed with HIP events on the launch stream around the timed graph
  comparison = in the same run and on the same input: the strip kernel on the
              same shared set, 384 per-block factor sets, the SmoothQuant
              kernel, the butterfly variant, the K2 (LU) form, the
              Walsh-Hadamard-32 kernel and the 4:1 copy ceiling (every copy
              form, the fastest reported); plus per-shape entries (KroQuant with
              the configuration's per-block sets and with one shared set,
              SmoothQuant, copy ceiling) for every other configured workload
              but the tiny one: the DiT CFG batch (8192 x 1152, 8192 x 4608),
              the mid widths (2048 x 2240, 2048 x 8960), the double-stream
              inputs (4608 x 3072, 4608 x 12288) and the sweep (4096 and
              16384 x 12288)
  cpu_baseline = the CPU oracle on the first 4096 rows of the same input

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu] [--no-per-shape]

HBM traffic (the roofline's "traffic" field) comes from two rocprofv3 counter
passes over `bench.py --traffic-run` (FETCH_SIZE, then WRITE_SIZE), which
launches a plain bf16->fp32 copy of known size as the calibration kernel and
then the quantizer steps eagerly; `bench.py --summarize-traffic FETCH_DIR
WRITE_DIR` turns the two runs' counter CSVs into the traffic profile under
profiles/, which this script reads back while the kernel source hash still
matches.
"""
import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantizer GB/s (bf16→MXFP4+E8M0) and % HBM peak, KroQuant vs SmoothQuant"
HBM_PEAK_GBS = 8000.0
BYTES_PER_ELEM = 2.0 + 0.5 + 1.0 / 32.0
ROTATE_BYTES = 1 << 30
HEADLINE = ("sweep_65536", 65536, 12288)
# every other configured workload except the tiny one: KroQuant (its configured
# per-block factor sets, and one shared set), SmoothQuant and the copy ceiling each
PER_SHAPE = [("dit_1152", 8192, 1152), ("dit_4608", 8192, 4608), ("mid_2240", 2048, 2240), ("mid_8960", 2048, 8960),
             ("dbl_3072", 4608, 3072), ("dbl_12288", 4608, 12288), ("sweep_4096", 4096, 12288),
             ("sweep_16384", 16384, 12288)]
KERNEL_SYMBOL = "kq_flat_kernel<true"  # the headline's kernel (one shared factor set)
RAMP_S = 0.3  # untimed replays before the warm-up steps, for the GPU clocks to leave their idle state
CPU_ROWS = 4096  # rows of the headline input the CPU oracle is timed on


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extras", action="store_true", help="skip the comparison legs and per-shape entries")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-per-shape", action="store_true",
                    help="skip the per-shape entries (the comparison legs at the headline shape still run)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum wall time of the CPU-oracle baseline")
    ap.add_argument("--traffic-run", action="store_true",
                    help="eager calibration copy + quantizer steps only, for rocprofv3 counter passes")
    ap.add_argument("--all-configs", action="store_true",
                    help="per-configuration table: KroQuant (MFMA per-block and shared, butterfly), SmoothQuant "
                         "and the copy ceiling, each timed alone")
    ap.add_argument("--hot", action="store_true",
                    help="one buffer set replayed (no rotation), so the caches may serve part of each launch: K2 "
                         "(LU), FWHT-32, the matrix-core and butterfly KroQuant forms and SmoothQuant; reported as "
                         "times and ratios, never as a fraction of HBM peak")
    ap.add_argument("--adaln", action="store_true",
                    help="AdaLN front-end fused with the quantizer against the unfused pipeline, hidden widths")
    ap.add_argument("--gemm", action="store_true",
                    help="W4A4 consumer (mx_gemm) on the DiT layer shapes, against its roofline")
    ap.add_argument("--gemm-library", action="store_true",
                    help="mx_gemm against torch's MXFP4 scaled_mm (hipBLASLt) on the qkv and proj layer shapes")
    ap.add_argument("--summarize-trace-runs", metavar="KERNEL_TRACE_CSV",
                    help="per-leg kernel times from a rocprofv3 --kernel-trace csv: runs of consecutive dispatches "
                         "of one kernel and grid (no GPU needed)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic profile from two rocprofv3 --pmc output folders (no GPU needed)")
    return ap.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("kq_kernels.hip", "kq_device.h", "kq_capi.hip", "kq_internal.h"):
        with open(os.path.join(ROOT, "mxfp4_act_quantizer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "kq_flat_sweep65536_traffic.md")
# calibration copy of the counter runs: bf16 -> fp32, 2^27 elements
CAL_ELEMS = 1 << 27
CAL_READ, CAL_WRITE = 2 * CAL_ELEMS, 4 * CAL_ELEMS
CAL_REPEAT = 4


def load_traffic(src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter runs (the json
    block of the traffic profile), if they were taken on the current kernel
    source; otherwise None."""
    try:
        with open(TRAFFIC_PROFILE) as fh:
            text = fh.read()
        t = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, ValueError, IndexError):
        return None
    if t.get("kernel_source_hash") != src_hash:
        return None
    return t.get("hbm_bytes_per_launch")


def _read_counters(folder):
    """(dispatch id, kernel name, grid, counter, value) rows of a rocprofv3 --pmc csv run."""
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]), r["Counter_Name"],
                             float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    return sorted(rows)


def summarize_trace_runs(path, min_calls=5):
    """Kernel durations of a rocprofv3 --kernel-trace csv, split into runs of
    consecutive dispatches of one kernel at one grid size: each timed leg of
    this script is such a run (its ramp, warm-up and timed graph), so a
    run's statistics are that leg's kernel time.  Prints one line per run of
    at least min_calls dispatches."""
    import csv
    import re
    with open(path) as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Start_Timestamp"]))
    runs = []
    for r in rows:
        key = (re.sub(r"\(.*", "", r["Kernel_Name"].replace("(anonymous namespace)::", "")), r.get("Grid_Size_X", ""))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if runs and runs[-1][0] == key:
            runs[-1][1].append(dur)
        else:
            runs.append([key, [dur]])
    for i, ((name, grid), v) in enumerate(runs):
        if len(v) < min_calls:
            continue
        v = sorted(v)
        print(f"| {i} | `{name}` | {grid} | {len(v)} | {sum(v) / len(v):.2f} | {v[len(v) // 2]:.2f} | {v[0]:.2f} |")


def summarize_traffic(fetch_dir, write_dir):
    """Counter runs -> calibrated HBM bytes per quantizer launch -> the traffic profile."""
    cal, kq = {}, {}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for _, name, grid, cname, val in _read_counters(folder):
            if cname != counter:
                continue
            if KERNEL_SYMBOL in name:
                kq.setdefault(counter, []).append(val * 1024.0)
                kq["grid"] = grid
                kq["name"] = name
            elif "copy" in name and ("BFloat16" in name or "bfloat16" in name):
                cal.setdefault((name, grid), {}).setdefault(counter, []).append(val * 1024.0)
    cal = [v for v in cal.values() if len(v.get("FETCH_SIZE", [])) >= CAL_REPEAT]
    if len(cal) != 1:
        raise SystemExit(f"expected one calibration copy kernel, found {len(cal)}")
    cal = cal[0]
    f_fetch = CAL_READ / float(np.median(cal["FETCH_SIZE"]))
    f_write = CAL_WRITE / float(np.median(cal["WRITE_SIZE"]))
    name, M, d = HEADLINE
    rd = float(np.mean(kq["FETCH_SIZE"])) * f_fetch
    wr = float(np.mean(kq["WRITE_SIZE"])) * f_write
    alg = M * d * BYTES_PER_ELEM
    blob = {"kernel": kq["name"], "workload": f"{name} ({M} x {d})", "kernel_source_hash": kernel_source_hash(),
            "grid": kq["grid"], "dispatches": len(kq["FETCH_SIZE"]),
            "read_bytes": round(rd), "write_bytes": round(wr),
            "hbm_bytes_per_launch": round(rd + wr), "algorithmic_bytes_per_launch": round(alg),
            "ratio": round((rd + wr) / alg, 4),
            "fetch_scale": round(f_fetch, 4), "write_scale": round(f_write, 4),
            "calibration": {"kernel": "torch bf16->fp32 copy", "elements": CAL_ELEMS,
                            "read_bytes": CAL_READ, "write_bytes": CAL_WRITE,
                            "fetch_kib_median": float(np.median(cal["FETCH_SIZE"])) / 1024,
                            "write_kib_median": float(np.median(cal["WRITE_SIZE"])) / 1024}}
    lines = [
        f"# HBM traffic of the KroQuant quantizer kernel, {M} x {d} bf16 (Hadamard factors, one shared set)",
        "",
        "Commands (from the repository root, on one MI355X; each counter pass is a run of its own):",
        "",
        f"    timeout -s KILL 240 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o fetch -- "
        "python3 bench.py --traffic-run --steps 10",
        f"    timeout -s KILL 240 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o write -- "
        "python3 bench.py --traffic-run --steps 10",
        f"    python3 bench.py --summarize-traffic {fetch_dir} {write_dir}",
        "",
        f"Calibration: a plain bf16->fp32 copy of {CAL_ELEMS} elements reads {CAL_READ} B and writes {CAL_WRITE} B; "
        f"its counters read FETCH_SIZE {blob['calibration']['fetch_kib_median']:.0f} KiB and WRITE_SIZE "
        f"{blob['calibration']['write_kib_median']:.0f} KiB per dispatch, so FETCH_SIZE is scaled by "
        f"{f_fetch:.4f} and WRITE_SIZE by {f_write:.4f}.",
        "",
        "| kernel | grid | dispatches | HBM read B | HBM write B | algorithmic B | HBM / algorithmic |",
        "|---|---|---|---|---|---|---|",
        f"| `{kq['name']}` | {kq['grid']} | {blob['dispatches']} | {blob['read_bytes']} | {blob['write_bytes']} | "
        f"{blob['algorithmic_bytes_per_launch']} | {blob['ratio']} |",
        "", "```json", json.dumps(blob, indent=1), "```", ""]
    with open(TRAFFIC_PROFILE, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(x_rows, f, tiny, min_seconds=10.0):
    """The oracle, as it stands (single-threaded C, untuned), over a bounded
    sample of the headline input (its first rows), spread over host threads
    by row ranges (ctypes releases the GIL), repeated until at least
    min_seconds of wall time; plus a one-thread figure on the tiny
    configuration (256 x 1152, one shared factor set)."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as O
    O.lib()
    host_cores = os.cpu_count() or 1
    threads = max(1, min(16, host_cores))  # at most 16 threads: the host CPU share of one GPU
    rows = x_rows.shape[0]
    chunk = max(1, (rows + 4 * threads - 1) // (4 * threads))
    jobs = [np.ascontiguousarray(x_rows[r0:r0 + chunk]) for r0 in range(0, rows, chunk)]
    passes = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            list(ex.map(lambda a: O.kq_quantize(a, f), jobs))
            passes += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
    dt = time.perf_counter() - t0
    elems = x_rows.size
    xt, ft = tiny
    n1, t1 = 0, time.perf_counter()
    while True:
        O.kq_quantize(xt, ft)
        n1 += 1
        if time.perf_counter() - t1 >= 2.0:
            break
    dt1 = time.perf_counter() - t1
    name, M, d = HEADLINE
    return {
        "value": round(passes * elems * BYTES_PER_ELEM / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the first {rows} of the {M} rows of the {name} input ({rows} x {d}, Hadamard factors), "
                  f"{passes} passes, {passes * elems} elements in {dt:.1f} s wall on {threads} threads over row "
                  f"ranges; same byte formula as the GPU value",
        "rows_per_s": round(passes * rows / dt, 1),
        "host_cores": host_cores,
        "cpu_model": cpu_model(),
        "one_thread_tiny": {"value": round(n1 * xt.size * BYTES_PER_ELEM / dt1 / 1e9, 4), "unit": "GB/s",
                            "rows_per_s": round(n1 * xt.shape[0] / dt1, 1),
                            "sample": f"tiny configuration {xt.shape[0]} x {xt.shape[1]}, one shared factor set, "
                                      f"{n1} passes on 1 thread"},
    }


def _time_leg(fn, nsets, steps):
    """Average time of one call of fn(set index): a graph of `steps` calls over
    the rotating sets, captured on a side stream, replayed after the clocks
    are up, timed with HIP events on that stream."""
    import torch
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        fn(0)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cs):
            for i in range(steps):
                fn(i % nsets)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.1:  # clocks up
        g.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cs):
        e0.record(cs)
        g.replay()
        e1.record(cs)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / steps


def best_copy(K, src_of, dst_of, nsets, steps):
    """Every 4:1 copy form on the given buffers; (best seconds per call, best
    form, {form: seconds})."""
    import torch
    per = {}
    for form in range(K.KQ_COPY_FORMS):
        per[form] = _time_leg(lambda i, form=form: K.measure_copy41(src_of(i), dst_of(i), form=form,
                                                                     stream=torch.cuda.current_stream()),
                              nsets, steps)
    best = min(per, key=per.get)
    return per[best], best, per


def all_configs(args):
    """Every configured shape (except the tiny smoke case): the MFMA quantizer
    with per-block factors (strip kernel) and with one shared set (flat kernel,
    and the strip kernel beside it), the butterfly variant, SmoothQuant
    and the 4:1 copy ceiling, each as a graph of `--steps` launches over
    rotating buffers (>= 1 GB per cycle), timed with HIP events.  Inputs are
    N(0,1) bf16 with 1% outlier channels x50 drawn on the GPU (the kernels'
    time does not depend on the values)."""
    import torch

    import mxfp4_act_quantizer_amd as K
    from synth import inputs as I
    dev = torch.device("cuda:0")
    table = []
    for name, (M, d, _) in I.CONFIGS.items():
        if name == "tiny":
            continue
        elems = M * d
        alg = elems * BYTES_PER_ELEM
        nsets = max(2, int(np.ceil(ROTATE_BYTES / alg)))
        gen = torch.Generator(device=dev)
        gen.manual_seed(I.data_seed(name))
        chan = torch.ones(d, device=dev)
        chan[torch.randperm(d, generator=gen, device=dev)[:max(1, d // 100)]] = 50.0
        bufs = []
        for _ in range(nsets):
            x = (torch.randn(M, d, generator=gen, device=dev) * chan).to(torch.bfloat16)
            bufs.append(dict(x=x, q=torch.empty((M, d // 2), dtype=torch.uint8, device=dev),
                             s=torch.empty((M, d // 32), dtype=torch.uint8, device=dev),
                             s16=torch.empty((M, d // 16), dtype=torch.uint8, device=dev)))
        amax = bufs[0]["x"].float().abs().amax(dim=0)
        scale = torch.sqrt(torch.clamp(amax, min=1e-5))
        f_pb = torch.from_numpy(I.random_factors(d // 32, I.factor_seed(name))).to(dev)
        f_sh = torch.from_numpy(I.random_factors(1, I.factor_seed(name))).to(dev)
        lu_pb = torch.from_numpy(I.random_lu(d // 32, I.factor_seed(name) + 77)).to(dev)
        f16 = torch.from_numpy(I.random_factors16(d // 16, I.factor_seed(name) + 16)).to(dev)
        f16_sh = torch.from_numpy(I.random_factors16(1, I.factor_seed(name) + 16)).to(dev)
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream
        legs = {
            "kq_mfma_perblock": lambda b: K.kq_quantize(b["x"], f_pb, b["q"], b["s"], stream=cur(), variant=1),
            "kq_mfma_shared": lambda b: K.kq_quantize(b["x"], f_sh, b["q"], b["s"], stream=cur(), variant=1),
            "kq_strip_shared": lambda b: K.kq_quantize(b["x"], f_sh, b["q"], b["s"], stream=cur(), variant=1,
                                                       tuning={"shared_form": 1}),
            "kq_butterfly_perblock": lambda b: K.kq_quantize(b["x"], f_pb, b["q"], b["s"], stream=cur(), variant=2),
            "kq_lu_perblock": lambda b: K.kq_quantize_lu(b["x"], lu_pb, b["q"], b["s"], stream=cur()),
            "fwht": lambda b: K.fwht_quantize(b["x"], b["q"], b["s"], stream=cur()),
            "kq16_perblock": lambda b: K.kq_quantize16(b["x"], f16, b["q"], b["s16"], stream=cur()),
            "kq16_shared": lambda b: K.kq_quantize16(b["x"], f16_sh, b["q"], b["s16"], stream=cur()),
            "smoothquant": lambda b: K.sq_quantize(b["x"], scale, b["q"], b["s"], stream=cur()),
        }
        row = {"config": name, "M": M, "d": d, "algorithmic_bytes": int(alg)}
        for leg, fn in legs.items():
            g = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            cs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cs):
                fn(bufs[0])
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=cs):
                    for i in range(args.steps):
                        fn(bufs[i % nsets])
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.1:  # clocks up
                g.replay()
                torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / args.steps
            # copy: 2 + 0.5 B per element; 16-element blocks: 2 + 0.5 + 1/16
            nbytes = elems * (2.5 + 1.0 / 16) if leg.startswith("kq16") else alg
            row[leg] = {"us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
                        "hbm_pct": round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 1), "rows/s": round(M / us * 1e6, 1)}
        cp, cp_form, _ = best_copy(K, lambda i: bufs[i]["x"], lambda i: bufs[i]["q"], nsets, args.steps)
        row["copy41"] = {"us": round(cp * 1e6, 2), "GB/s": round(elems * 2.5 / cp / 1e9, 1),
                         "hbm_pct": round(100 * elems * 2.5 / cp / 1e9 / HBM_PEAK_GBS, 1), "form": cp_form}
        row["kq_over_sq_speed"] = round(row["smoothquant"]["us"] / row["kq_mfma_perblock"]["us"], 4)
        row["kq_shared_over_sq_speed"] = round(row["smoothquant"]["us"] / row["kq_mfma_shared"]["us"], 4)
        row["kq_over_copy41_speed"] = round(row["copy41"]["us"] / row["kq_mfma_perblock"]["us"], 4)
        row["k2_lu_over_fwht_speed"] = round(row["fwht"]["us"] / row["kq_lu_perblock"]["us"], 4)
        table.append(row)
        print(json.dumps(row), flush=True)
        del bufs
        torch.cuda.empty_cache()
    print("| config | M x d | KQ MFMA per-block us (GB/s, %peak) | KQ shared, flat kernel us (GB/s, %peak) | "
          "KQ shared, strip kernel us | KQ butterfly us | K2 LU us | FWHT us | SmoothQuant us (GB/s, %peak) | "
          "copy 4:1 us (GB/s) | KQ/SQ speed (per-block, shared) | KQ/copy speed | K2/FWHT speed | "
          "KQ16 per-block, strip kernel us (GB/s) | KQ16 shared, flat kernel us (GB/s) |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for r in table:
        a, b, bs, c, l2, fw, q, cp = (r[k] for k in ("kq_mfma_perblock", "kq_mfma_shared", "kq_strip_shared",
                                                       "kq_butterfly_perblock", "kq_lu_perblock", "fwht",
                                                       "smoothquant", "copy41"))
        print(f"| {r['config']} | {r['M']}x{r['d']} | {a['us']} ({a['GB/s']}, {a['hbm_pct']}%) | "
              f"{b['us']} ({b['GB/s']}, {b['hbm_pct']}%) | {bs['us']} | "
              f"{c['us']} | {l2['us']} | {fw['us']} | {q['us']} ({q['GB/s']}, {q['hbm_pct']}%) | "
              f"{cp['us']} ({cp['GB/s']}) | {r['kq_over_sq_speed']}, {r['kq_shared_over_sq_speed']} | "
              f"{r['kq_over_copy41_speed']} | "
              f"{r['k2_lu_over_fwht_speed']} | {r['kq16_perblock']['us']} ({r['kq16_perblock']['GB/s']}) | "
              f"{r['kq16_shared']['us']} ({r['kq16_shared']['GB/s']}) |", flush=True)


# shapes whose x, q and s of one call fit the 256 MB last-level cache
HOT_SHAPES = [("dit_1152", 8192, 1152), ("dit_4608", 8192, 4608), ("sweep_4096", 4096, 12288)]


def hot_bench(args):
    """The transform kernels on one buffer set per shape, replayed as a graph
    of `--steps` launches (no rotation), so the caches may serve part of each
    launch.  The kernels read x with nontemporal loads, which stream past the
    caches, so this is not a cache-resident measurement: it only shows how
    much the kernels gain when the data were just touched.  The K2 form (LU
    scalars rebuilt in the kernel) against the Walsh-Hadamard-32 kernel is the
    comparison the pages make; the matrix-core forms (per-block and one shared
    set), the butterfly form and SmoothQuant are timed beside it.  Times and
    ratios only, no fraction of HBM peak."""
    import torch

    import mxfp4_act_quantizer_amd as K
    from synth import inputs as I
    dev = torch.device("cuda:0")
    cur = torch.cuda.current_stream
    rows = []
    for name, M, d in HOT_SHAPES:
        gen = torch.Generator(device=dev)
        gen.manual_seed(I.data_seed(name))
        chan = torch.ones(d, device=dev)
        chan[torch.randperm(d, generator=gen, device=dev)[:max(1, d // 100)]] = 50.0
        x = (torch.randn(M, d, generator=gen, device=dev) * chan).to(torch.bfloat16)
        q = torch.empty((M, d // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((M, d // 32), dtype=torch.uint8, device=dev)
        amax = x.float().abs().amax(dim=0)
        scale = torch.sqrt(torch.clamp(amax, min=1e-5))
        f_pb = torch.from_numpy(I.random_factors(d // 32, I.factor_seed(name))).to(dev)
        f_h = torch.from_numpy(I.hadamard_factors(1)).to(dev)
        lu_pb = torch.from_numpy(I.random_lu(d // 32, I.factor_seed(name) + 77)).to(dev)
        torch.cuda.synchronize()
        legs = {
            "k2_lu_perblock": lambda i: K.kq_quantize_lu(x, lu_pb, q, sc, stream=cur()),
            "fwht": lambda i: K.fwht_quantize(x, q, sc, stream=cur()),
            "kq_mfma_perblock": lambda i: K.kq_quantize(x, f_pb, q, sc, stream=cur(), variant=1),
            "kq_mfma_hadamard_shared": lambda i: K.kq_quantize(x, f_h, q, sc, stream=cur(), variant=1),
            "kq_butterfly_perblock": lambda i: K.kq_quantize(x, f_pb, q, sc, stream=cur(), variant=2),
            "smoothquant": lambda i: K.sq_quantize(x, scale, q, sc, stream=cur()),
        }
        row = {"config": name, "M": M, "d": d, "footprint_MB": round(M * d * BYTES_PER_ELEM / 1e6, 2)}
        for leg, fn in legs.items():
            # best of three replays of the same graph (each a graph of --steps launches)
            row[leg] = {"us": round(min(_time_leg(fn, 1, args.steps) for _ in range(3)) * 1e6, 2)}
        row["k2_lu_over_fwht_speed"] = round(row["fwht"]["us"] / row["k2_lu_perblock"]["us"], 4)
        row["kq_perblock_over_smoothquant_speed"] = round(row["smoothquant"]["us"] / row["kq_mfma_perblock"]["us"], 4)
        row["kq_shared_over_smoothquant_speed"] = round(
            row["smoothquant"]["us"] / row["kq_mfma_hadamard_shared"]["us"], 4)
        row["mfma_over_butterfly_speed"] = round(
            row["kq_butterfly_perblock"]["us"] / row["kq_mfma_perblock"]["us"], 4)
        row["note"] = "one buffer set replayed (x read with nontemporal loads), not an HBM-peak figure"
        rows.append(row)
        print(json.dumps(row), flush=True)
        del x, q, sc
        torch.cuda.empty_cache()


FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 matrix peak (TFLOP/s)
# DiT (d = 1152, MLP 4608) linear layers on the CFG batch of 8192 tokens: (name, M, N, K)
GEMM_SHAPES = [("qkv", 8192, 3456, 1152), ("proj", 8192, 1152, 1152), ("mlp_up", 8192, 4608, 1152),
               ("mlp_down", 8192, 1152, 4608)]


def gemm_bench(args):
    """mx_gemm (bf16 out) on the DiT layer shapes; operands from the quantizer's
    own kernels on synthetic data; each shape a graph of --steps launches over
    rotating operand sets, timed with HIP events.  Roofline per shape:
    max(2MNK / FP4 peak, bytes / HBM peak) with bytes = A, B codes and scales
    plus the bf16 output.  The per-tile kernel (the fallback for shapes the
    persistent kernel does not take) is timed on the same operands beside it, and
    so is the quantizer of the activation followed by the product."""
    import torch

    import mxfp4_act_quantizer_amd as K
    from synth import inputs as I
    dev = torch.device("cuda:0")
    rows = []
    for name, M, N, Kd in GEMM_SHAPES:
        gen = torch.Generator(device=dev)
        gen.manual_seed(M + N + Kd)
        nbytes = M * Kd // 2 + M * Kd // 32 + N * Kd // 2 + N * Kd // 32 + M * N * 2
        nsets = max(2, int(np.ceil(ROTATE_BYTES / nbytes)))
        f = torch.from_numpy(I.hadamard_factors(Kd // 32)).to(dev)
        sets = []
        for _ in range(nsets):
            x = torch.randn(M, Kd, generator=gen, device=dev).to(torch.bfloat16)
            qa, sa = K.kq_quantize(x, f)
            w = torch.randn(N, Kd, generator=gen, device=dev) / math.sqrt(Kd)
            qb, sb = K.mx_quantize_f32(w)
            sets.append((qa, sa, qb, sb, torch.empty((M, N), dtype=torch.bfloat16, device=dev), x))
            del w
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            K.mx_gemm(*sets[0][:4], out=sets[0][4], stream=cs)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=cs):
                for i in range(args.steps):
                    b = sets[i % nsets]
                    K.mx_gemm(*b[:4], out=b[4], stream=torch.cuda.current_stream())
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.1:
            g.replay()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        # the per-tile kernel on the same operands, for comparison
        us_tile = _time_leg(lambda i: K.mx_gemm(*sets[i][:4], out=sets[i][4], stream=torch.cuda.current_stream(),
                                                tuning={"gemm_kernel": 1}), nsets, args.steps) * 1e6
        # the activation quantizer followed by the product, as a layer runs them
        us_pipe = _time_leg(lambda i: (K.kq_quantize(sets[i][5], f, sets[i][0], sets[i][1],
                                                     stream=torch.cuda.current_stream()),
                                       K.mx_gemm(*sets[i][:4], out=sets[i][4], stream=torch.cuda.current_stream())),
                            nsets, args.steps) * 1e6
        flops = 2.0 * M * N * Kd
        t_mfma = flops / (FP4_PEAK_TFLOPS * 1e12) * 1e6
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9) * 1e6
        bound = "mfma" if t_mfma >= t_hbm else "hbm"
        row = {"layer": name, "M": M, "N": N, "K": Kd, "us": round(us, 2), "TFLOP/s": round(flops / us / 1e6, 1),
               "GB/s": round(nbytes / us / 1e3, 1), "bound": bound,
               "roofline_us": round(max(t_mfma, t_hbm), 2), "frac": round(max(t_mfma, t_hbm) / us, 4),
               "per_tile_kernel_us": round(us_tile, 2), "quantize_then_product_us": round(us_pipe, 2)}
        rows.append(row)
        print(json.dumps(row), flush=True)
        del sets
        torch.cuda.empty_cache()
    tot_us = sum(r["us"] for r in rows)
    tot_roof = sum(r["roofline_us"] for r in rows)
    print(json.dumps({"gemm_block_us": round(tot_us, 2), "roofline_us": round(tot_roof, 2),
                      "frac": round(tot_roof / tot_us, 4),
                      "per_tile_kernel_block_us": round(sum(r["per_tile_kernel_us"] for r in rows), 2)}), flush=True)


def gemm_library_bench(args):
    """mx_gemm against the library MXFP4 product this image offers
    (torch.nn.functional.scaled_mm with 1x32 E8M0 block scales, which runs
    hipBLASLt), on the same operands: the quantizer's codes and scales as they
    are, viewed as float4_e2m1fn_x2 and float8_e8m0fnu.  Both timed eagerly,
    back to back, with HIP events.  Only the qkv and proj shapes: at the MLP
    shapes the library's kernel generator fails in this build and retries
    for minutes."""
    import torch
    import torch.nn.functional as F

    import mxfp4_act_quantizer_amd as K
    from synth import inputs as I
    dev = torch.device("cuda:0")

    def eager_us(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    for name, M, N, Kd in GEMM_SHAPES[:2]:
        gen = torch.Generator(device=dev)
        gen.manual_seed(M + N + Kd)
        f = torch.from_numpy(I.hadamard_factors(Kd // 32)).to(dev)
        x = torch.randn(M, Kd, generator=gen, device=dev).to(torch.bfloat16)
        qa, sa = K.kq_quantize(x, f)
        qb, sb = K.mx_quantize_f32(torch.randn(N, Kd, generator=gen, device=dev) / math.sqrt(Kd))
        ref = K.mx_gemm(qa, sa, qb, sb, out_dtype=torch.float32)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ours = eager_us(lambda: K.mx_gemm(qa, sa, qb, sb, out=out), args.steps)
        a4, b4 = qa.view(torch.float4_e2m1fn_x2), qb.view(torch.float4_e2m1fn_x2)
        ea, eb = sa.view(torch.float8_e8m0fnu), sb.view(torch.float8_e8m0fnu)

        def lib():
            return F.scaled_mm(a4, b4.t(), ea, F.ScalingType.BlockWise1x32, eb, F.ScalingType.BlockWise1x32,
                               F.SwizzleType.NO_SWIZZLE, F.SwizzleType.NO_SWIZZLE, output_dtype=torch.bfloat16)
        row = {"layer": name, "M": M, "N": N, "K": Kd, "mx_gemm_us": round(ours, 2)}
        try:
            got = lib()
            torch.cuda.synchronize()
            row["library_us"] = round(eager_us(lib, args.steps), 2)
            row["library_max_rel_diff"] = float(((got.float() - ref).abs().max() / ref.abs().max()).item())
            row["mx_gemm_max_rel_diff"] = float(((out.float() - ref).abs().max() / ref.abs().max()).item())
        except (RuntimeError, TypeError, AttributeError) as e:
            row["library_error"] = f"{type(e).__name__}: {str(e)[:200]}"
        print(json.dumps(row), flush=True)


ADALN_WORKLOADS = ("dit_1152", "mid_2240", "dbl_3072")  # the hidden widths AdaLN normalises
ADALN_EPS = 1e-6


def adaln_bench(args):
    """The AdaLN front-end fused with the quantizer (kq_adaln_quantize) against
    the unfused pipeline (adaln_modulate writing bf16 x, then kq_quantize with
    the MFMA or the butterfly transform) and against torch's layer_norm and
    modulation (bf16 out) followed by kq_quantize, at the hidden widths, two samples
    (CFG) per batch.  The fused call runs its automatic form (two launches,
    second pass on the matrix cores); more fused legs force the one-launch form
    (whole rows in LDS), the matrix-core second pass in strips of 4 blocks and
    the butterfly second pass.  Fused algorithmic bytes: 2.53125 B per element (h read,
    codes and scales written) plus the modulation; unfused: 6.53125 (x
    written and read back).  Per-block factor sets; h drawn on the GPU as
    N(0,1) with 1% outlier channels x50 (the time does not depend on the
    values)."""
    import torch

    import mxfp4_act_quantizer_amd as K
    from synth import inputs as I
    dev = torch.device("cuda:0")
    rows = []
    for name in ADALN_WORKLOADS:
        M, d, _ = I.CONFIGS[name]
        T = I.tokens_per_sample(name)
        elems = M * d
        alg = elems * BYTES_PER_ELEM
        nsets = max(2, int(np.ceil(ROTATE_BYTES / alg)))
        gen = torch.Generator(device=dev)
        gen.manual_seed(I.data_seed(name))
        chan = torch.ones(d, device=dev)
        chan[torch.randperm(d, generator=gen, device=dev)[:max(1, d // 100)]] = 50.0
        shift, scale = (torch.from_numpy(a).to(dev) for a in I.adaln_modulation((M + T - 1) // T, d, I.adaln_seed(name)))
        f = torch.from_numpy(I.random_factors(d // 32, I.factor_seed(name))).to(dev)
        sets = []
        for _ in range(nsets):
            sets.append(dict(h=(torch.randn(M, d, generator=gen, device=dev) * chan).to(torch.bfloat16),
                             x=torch.empty((M, d), dtype=torch.bfloat16, device=dev),
                             q=torch.empty((M, d // 2), dtype=torch.uint8, device=dev),
                             s=torch.empty((M, d // 32), dtype=torch.uint8, device=dev),
                             w=torch.empty((M, 2), dtype=torch.float64, device=dev)))
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream

        def fused(i):
            b = sets[i]
            K.kq_adaln_quantize(b["h"], shift, scale, T, ADALN_EPS, f, b["q"], b["s"], stats=b["w"], stream=cur())

        def modulate(i):
            b = sets[i]
            K.adaln_modulate(b["h"], shift, scale, T, ADALN_EPS, b["x"], stats=b["w"], stream=cur())

        def unfused(variant):
            def run(i):
                b = sets[i]
                K.adaln_modulate(b["h"], shift, scale, T, ADALN_EPS, b["x"], stats=b["w"], stream=cur())
                K.kq_quantize(b["x"], f, b["q"], b["s"], stream=cur(), variant=variant)
            return run

        nS = (M + T - 1) // T

        def torch_unfused(i):
            # torch's own layer norm and modulation (several kernels, bf16 out), then the quantizer
            b = sets[i]
            n = torch.nn.functional.layer_norm(b["h"], (d,), eps=ADALN_EPS)
            if M % T == 0:
                x = (n.view(nS, T, d) * (1.0 + scale[:, None, :]) + shift[:, None, :]).to(torch.bfloat16).view(M, d)
            else:
                idx = torch.arange(M, device=dev) // T
                x = (n * (1.0 + scale[idx]) + shift[idx]).to(torch.bfloat16)
            K.kq_quantize(x, f, b["q"], b["s"], stream=cur())

        def fused_with(knobs):
            def run(i):
                b = sets[i]
                K.kq_adaln_quantize(b["h"], shift, scale, T, ADALN_EPS, f, b["q"], b["s"], stats=b["w"],
                                    stream=cur(), tuning=knobs)
            return run

        t = {"fused": _time_leg(fused, nsets, args.steps),
             "fused_one_launch": _time_leg(fused_with({"adaln_pass": 3}), nsets, args.steps),
             "fused_butterfly_pass": _time_leg(fused_with({"adaln_pass": 2}), nsets, args.steps),
             "fused_mfma_strip4": _time_leg(fused_with({"adaln_pass": 1, "adaln_strip": 4}), nsets, args.steps),
             "torch_layernorm_then_kq_mfma": _time_leg(torch_unfused, nsets, args.steps),
             "unfused_mfma": _time_leg(unfused(1), nsets, args.steps),
             "unfused_butterfly": _time_leg(unfused(2), nsets, args.steps),
             "modulate_alone": _time_leg(modulate, nsets, args.steps)}
        fused_gbs = alg / t["fused"] / 1e9
        row = {"workload": name, "M": M, "d": d, "tokens_per_sample": T,
               "us": {k: round(v * 1e6, 2) for k, v in t.items()},
               "fused_GB/s": round(fused_gbs, 1),
               "fused_roofline": {"bound": "hbm", "achieved": round(fused_gbs, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(fused_gbs / HBM_PEAK_GBS, 4)},
               "fused_speedup_vs_unfused_mfma": round(t["unfused_mfma"] / t["fused"], 3),
               "fused_speedup_vs_unfused_butterfly": round(t["unfused_butterfly"] / t["fused"], 3),
               "fused_speedup_vs_torch_layernorm": round(t["torch_layernorm_then_kq_mfma"] / t["fused"], 3),
               "unfused_mfma_GB/s_at_6.53B": round(elems * 6.53125 / t["unfused_mfma"] / 1e9, 1)}
        rows.append(row)
        print(json.dumps(row), flush=True)
        del sets
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_trace_runs:
        summarize_trace_runs(args.summarize_trace_runs)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the quantizer shards by "
              f"rows with no communication, so N GPUs run N independent copies of this step)", file=sys.stderr)
        sys.exit(2)
    if args.all_configs or args.gemm or args.adaln or args.gemm_library or args.hot:
        if args.all_configs:
            all_configs(args)
        elif args.hot:
            hot_bench(args)
        elif args.gemm:
            gemm_bench(args)
        elif args.gemm_library:
            gemm_library_bench(args)
        else:
            adaln_bench(args)
        return
    import torch

    import mxfp4_act_quantizer_amd as K
    from synth import inputs as I
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no GPU visible)", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    cur = torch.cuda.current_stream

    # ---- the headline input, generated on the host from the seeded recipe
    name, M, d = HEADLINE
    t_gen = time.perf_counter()
    x_bits = I.act_sweep_special(M, d, I.data_seed(name))[0]
    print(f"[bench] {name} {M} x {d} generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    f_h = I.hadamard_factors(1)
    step_bytes = M * d * BYTES_PER_ELEM
    nsets = max(2, int(np.ceil(ROTATE_BYTES / step_bytes)))
    x0 = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    sets = [dict(x=x0 if k == 0 else x0.clone(), q=torch.empty((M, d // 2), dtype=torch.uint8, device=dev),
                 s=torch.empty((M, d // 32), dtype=torch.uint8, device=dev)) for k in range(nsets)]
    fh_d = torch.from_numpy(f_h).to(dev)
    torch.cuda.synchronize()

    def step(i):
        b = sets[i % nsets]
        K.kq_quantize(b["x"], fh_d, b["q"], b["s"], stream=cur())

    def capture(fn, count):
        """A HIP graph of `count` calls fn(0..count-1), captured on a side stream."""
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            fn(0)  # one eager call on the capture stream first
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=cs):
                for i in range(count):
                    fn(i)
        torch.cuda.synchronize()
        return g, cs

    if args.traffic_run:
        src = torch.randn(CAL_ELEMS, device=dev).to(torch.bfloat16)
        dst = torch.empty(CAL_ELEMS, dtype=torch.float32, device=dev)
        for _ in range(CAL_REPEAT):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        for i in range(args.warmup + args.steps):
            step(i)
        torch.cuda.synchronize()
        print(f"traffic run: {CAL_REPEAT} calibration copies, {args.warmup + args.steps} quantizer steps", flush=True)
        return

    # ---- the timed region: exactly K steps, launched as one graph (launch
    # gaps would otherwise show between kernels), bracketed by synchronisation
    g_warm, _ = capture(step, max(1, args.warmup))
    g_main, cs_main = capture(step, args.steps)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < RAMP_S:  # clocks out of their idle state
        g_warm.replay()
        torch.cuda.synchronize()
    ramp_s = round(time.perf_counter() - t0, 3)
    g_warm.replay()  # the W warm-up steps
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(cs_main):
        e0.record(cs_main)  # HIP events on the stream the kernels run on
        g_main.replay()
        e1.record(cs_main)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = e0.elapsed_time(e1) * 1e-3
    value = step_bytes * args.steps / wall / 1e9
    avg_launch = ev / args.steps
    achieved = step_bytes / avg_launch / 1e9
    # per-launch spread, outside the timed region: K single launches on the
    # same stream, each between its own pair of HIP events
    pairs = []
    with torch.cuda.stream(cs_main):
        for i in range(args.steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(cs_main)
            step(i)
            b.record(cs_main)
            pairs.append((a, b))
    torch.cuda.synchronize()
    per_launch = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
    shape = K.kq_flat_launch_shape(M, d)
    src_hash = kernel_source_hash()
    kname = f"kq_flat_kernel<true, {'true' if shape['nt_codes'] else 'false'}, {shape['ring']}>"
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(src_hash),
                "kernel": kname, "avg_launch_us": round(avg_launch * 1e6, 2), "launches_timed": args.steps,
                "algorithmic_bytes_per_launch": round(step_bytes),
                "timing": "HIP events on the launch stream around the timed graph of K steps (one launch each)",
                "launch_shape": shape,
                "per_launch_us": {"median": round(float(np.median(per_launch)), 2),
                                  "mean": round(float(np.mean(per_launch)), 2),
                                  "min": round(per_launch[0], 2), "max": round(per_launch[-1], 2),
                                  "launches": len(per_launch),
                                  "timing": "K more launches after the timed region, each between its own "
                                            "pair of HIP events on the launch stream"}}
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"bandwidth sweep, largest single-GPU configuration: {M} x {d} bf16 activation "
                               f"(N(0,1), 1% outlier channels x50, 0.1% each zero / subnormal / near-min-normal / "
                               f"exact-tie blocks), [[1,1],[1,-1]]/sqrt(2) factors shared by all blocks "
                               f"(normalised Walsh-Hadamard-32), MXFP4 + E8M0 out",
                   "M": M, "d": d, "nT": 1, "factors": "hadamard", "rotating_sets": nsets, "accumulate": "fp32",
                   "launch": "HIP graph of the K timed steps", "clock_ramp_s": ramp_s,
                   "hbm_pct": round(100 * value / HBM_PEAK_GBS, 2),
                   "rows_per_s": round(M * args.steps / wall, 1),
                   "kernel_source_hash": src_hash,
                   "library_sources": K.kq_build_info().rsplit(" ", 1)[-1]},
        "roofline": roofline,
    }

    if not args.no_extras:
        steps = args.steps
        scale_d = torch.from_numpy(I.smoothquant_scale(x_bits)).to(dev)
        f_pb = torch.from_numpy(I.random_factors(d // 32, I.factor_seed(name))).to(dev)
        f_id = torch.from_numpy(I.identity_factors(1)).to(dev)
        lu_pb = torch.from_numpy(I.random_lu(d // 32, I.factor_seed(name) + 77)).to(dev)

        def leg(fn):
            return _time_leg(fn, nsets, steps)

        b = lambda i: sets[i]
        t = {
            "kq_hadamard_shared": avg_launch,
            "kq_hadamard_shared_strip_kernel": leg(lambda i: K.kq_quantize(b(i)["x"], fh_d, b(i)["q"], b(i)["s"],
                                                                           stream=cur(), tuning={"shared_form": 1})),
            "kq_perblock_384": leg(lambda i: K.kq_quantize(b(i)["x"], f_pb, b(i)["q"], b(i)["s"], stream=cur())),
            "kq_identity": leg(lambda i: K.kq_quantize(b(i)["x"], f_id, b(i)["q"], b(i)["s"], stream=cur())),
            "smoothquant": leg(lambda i: K.sq_quantize(b(i)["x"], scale_d, b(i)["q"], b(i)["s"], stream=cur())),
            "kq_butterfly_perblock": leg(lambda i: K.kq_quantize(b(i)["x"], f_pb, b(i)["q"], b(i)["s"],
                                                                 stream=cur(), variant=2)),
            "k2_lu_perblock": leg(lambda i: K.kq_quantize_lu(b(i)["x"], lu_pb, b(i)["q"], b(i)["s"], stream=cur())),
            "fwht": leg(lambda i: K.fwht_quantize(b(i)["x"], b(i)["q"], b(i)["s"], stream=cur())),
        }
        c_best, c_form, c_per = best_copy(K, lambda i: sets[i]["x"], lambda i: sets[i]["q"], nsets, steps)
        legs = {}
        for k, sec in t.items():
            legs[k] = {"us": round(sec * 1e6, 2), "GB/s": round(step_bytes / sec / 1e9, 1),
                       "hbm_pct": round(100 * step_bytes / sec / 1e9 / HBM_PEAK_GBS, 2),
                       "rows/s": round(M / sec, 1)}
        copy_bytes = M * d * 2.5
        legs["copy41_ceiling"] = {"us": round(c_best * 1e6, 2), "GB/s": round(copy_bytes / c_best / 1e9, 1),
                                  "hbm_pct": round(100 * copy_bytes / c_best / 1e9 / HBM_PEAK_GBS, 2),
                                  "form": c_form, "us_per_form": {f: round(s * 1e6, 2) for f, s in c_per.items()}}
        sq = t["smoothquant"]
        out["comparison"] = {
            "legs": legs,
            "smoothquant_GB/s": legs["smoothquant"]["GB/s"],
            "smoothquant_rows/s": legs["smoothquant"]["rows/s"],
            "smoothquant_hbm_pct": legs["smoothquant"]["hbm_pct"],
            "kroquant_over_smoothquant_speed": round(sq / avg_launch, 4),
            "flat_over_strip_kernel_speed": round(t["kq_hadamard_shared_strip_kernel"] / avg_launch, 4),
            "kroquant_perblock_over_smoothquant_speed": round(sq / t["kq_perblock_384"], 4),
            "k2_lu_over_fwht_speed": round(t["fwht"] / t["k2_lu_perblock"], 4),
            "copy41_ceiling_GB/s": legs["copy41_ceiling"]["GB/s"],
            "kroquant_over_copy41_speed": round(c_best / avg_launch, 4),
            "notes": "every leg on the same input and buffers, graphs of K launches timed with HIP events; "
                     "copy41: fastest of the 4:1 streaming copy forms (2 B read, 0.5 B written per element; "
                     "GB/s at 2.5 B per element)",
        }
        del scale_d
        # ---- per-shape entries: every other configured workload but the tiny one
        per_shape = {}
        for sname, sM, sd in ([] if args.no_per_shape else PER_SHAPE):
            xs = I.make_activation(sname)
            fs = torch.from_numpy(I.make_factors(sname)).to(dev)
            fsh = torch.from_numpy(I.make_factors(sname, shared=True)).to(dev)
            ss = torch.from_numpy(I.smoothquant_scale(xs)).to(dev)
            sbytes = sM * sd * BYTES_PER_ELEM
            ns = max(2, int(np.ceil(ROTATE_BYTES / sbytes)))
            xd = torch.from_numpy(xs.view(np.int16)).to(dev).view(torch.bfloat16)
            bufs = [dict(x=xd if k == 0 else xd.clone(), q=torch.empty((sM, sd // 2), dtype=torch.uint8, device=dev),
                         s=torch.empty((sM, sd // 32), dtype=torch.uint8, device=dev)) for k in range(ns)]
            torch.cuda.synchronize()
            kq_t = _time_leg(lambda i: K.kq_quantize(bufs[i]["x"], fs, bufs[i]["q"], bufs[i]["s"], stream=cur()),
                             ns, steps)
            kqs_t = _time_leg(lambda i: K.kq_quantize(bufs[i]["x"], fsh, bufs[i]["q"], bufs[i]["s"], stream=cur()),
                              ns, steps)
            sq_t = _time_leg(lambda i: K.sq_quantize(bufs[i]["x"], ss, bufs[i]["q"], bufs[i]["s"], stream=cur()),
                             ns, steps)
            cp_t, cp_form, _ = best_copy(K, lambda i: bufs[i]["x"], lambda i: bufs[i]["q"], ns, steps)
            per_shape[sname] = {
                "M": sM, "d": sd, "nT": sd // 32, "launch_shape": K.kq_launch_shape(sM, sd),
                "kq_us": round(kq_t * 1e6, 2), "kq_GB/s": round(sbytes / kq_t / 1e9, 1),
                "kq_hbm_pct": round(100 * sbytes / kq_t / 1e9 / HBM_PEAK_GBS, 2), "kq_rows/s": round(sM / kq_t, 1),
                "kq_shared_us": round(kqs_t * 1e6, 2), "kq_shared_GB/s": round(sbytes / kqs_t / 1e9, 1),
                "kq_shared_hbm_pct": round(100 * sbytes / kqs_t / 1e9 / HBM_PEAK_GBS, 2),
                "kq_shared_launch_shape": K.kq_flat_launch_shape(sM, sd),
                "kq_shared_over_sq_speed": round(sq_t / kqs_t, 4),
                "sq_us": round(sq_t * 1e6, 2), "sq_GB/s": round(sbytes / sq_t / 1e9, 1),
                "sq_rows/s": round(sM / sq_t, 1), "kq_over_sq_speed": round(sq_t / kq_t, 4),
                "copy41_us": round(cp_t * 1e6, 2), "copy41_form": cp_form,
                "kq_over_copy41_speed": round(cp_t / kq_t, 4)}
            print(f"[bench] {sname}: {per_shape[sname]}", file=sys.stderr, flush=True)
            del bufs, xd
            torch.cuda.empty_cache()
        out["per_shape"] = per_shape

    if not args.no_cpu:
        tiny = (I.make_activation("tiny"), I.make_factors("tiny"))
        out["cpu_baseline"] = cpu_baseline(np.ascontiguousarray(x_bits[:CPU_ROWS]), f_h, tiny, args.cpu_seconds)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
