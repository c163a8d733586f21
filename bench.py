#!/usr/bin/env python3
"""Throughput of the KroQuant online quantizer on one MI355X.

One step = the quantizer pass over one CFG-doubled DiT batch: both activation
matrices of the DiT configuration (M = 8192 tokens, d = 1152 with 36 factor
sets and d = 4608 with 144 factor sets, bf16, synthetic: per-token lognormal
rows, 1% outlier channels x50), each through kq_quantize (bf16 -> per-block
Kronecker transform -> MXFP4 codes + E8M0 scales).

  value     = algorithmic bytes of the step / step time  (GB/s)
              algorithmic bytes = 2.53125 B per element (2 read, 0.5 + 1/32 written)
  roofline  = the quantizer kernel's average launch against the 8 TB/s HBM peak,
              timed with HIP events around graphs of back-to-back launches
  cpu_baseline = the CPU oracle on a bounded sample of the same workload

Inputs and outputs rotate over enough buffer sets (>= 1 GB per cycle) that
every launch reads from HBM rather than the 256 MB last-level cache.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]

HBM traffic (the roofline's "traffic" field) comes from two rocprofv3 counter
passes over `bench.py --traffic-run` (FETCH_SIZE, then WRITE_SIZE), which
launches a plain bf16->fp32 copy of known size as the calibration kernel and
then the quantizer steps eagerly; `bench.py --summarize-traffic FETCH_DIR
WRITE_DIR` turns the two runs' counter CSVs into profiles/kq_mfma_dit_traffic.md,
which this script reads back while the kernel source hash still matches.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantizer GB/s (bf16→MXFP4+E8M0) and % HBM peak, KroQuant vs SmoothQuant"
HBM_PEAK_GBS = 8000.0
BYTES_PER_ELEM = 2.0 + 0.5 + 1.0 / 32.0
ROTATE_BYTES = 1 << 30
WORKLOAD = [("dit_1152", 8192, 1152), ("dit_4608", 8192, 4608)]
KERNEL_SYMBOL = "kq_mfma_kernel<true"  # both strip-width instances: <true, 8> and <true, 16>
RAMP_S = 0.3  # untimed replays before the warm-up steps, for the GPU clocks to leave their idle state


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--variant", type=int, default=0, help="0 auto, 1 mfma, 2 butterfly")
    ap.add_argument("--no-extras", action="store_true", help="skip the SmoothQuant / butterfly comparison legs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum wall time of the CPU-oracle baseline")
    ap.add_argument("--traffic-run", action="store_true",
                    help="eager calibration copy + quantizer steps only, for rocprofv3 counter passes")
    ap.add_argument("--all-configs", action="store_true",
                    help="per-configuration table: KroQuant (MFMA per-block and shared, butterfly), SmoothQuant "
                         "and the copy ceiling, each timed alone")
    ap.add_argument("--adaln", action="store_true",
                    help="AdaLN front-end fused with the quantizer against the unfused pipeline, hidden widths")
    ap.add_argument("--gemm", action="store_true",
                    help="W4A4 consumer (mx_gemm) on the DiT layer shapes, against its roofline")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic profile from two rocprofv3 --pmc output folders (no GPU needed)")
    return ap.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("kq_kernels.hip", "kq_device.h", "kq_capi.hip", "kq_internal.h"):
        with open(os.path.join(ROOT, "mxfp4_act_quantizer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "kq_mfma_dit_traffic.md")
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
    """(dispatch id, kernel name, counter, value) rows of a rocprofv3 --pmc csv run."""
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


def summarize_traffic(fetch_dir, write_dir):
    """Counter runs -> calibrated HBM bytes per quantizer launch -> the traffic profile.

    The traffic run launches the shapes of WORKLOAD in turn, so the n-th
    quantizer dispatch of a run is shape n mod len(WORKLOAD)."""
    cal, kq = {}, {}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        n = 0
        for _, name, grid, cname, val in _read_counters(folder):
            if cname != counter:
                continue
            if KERNEL_SYMBOL in name:
                kq.setdefault((n % len(WORKLOAD), grid), {}).setdefault(counter, []).append(val * 1024.0)
                n += 1
            elif "copy" in name and ("BFloat16" in name or "bfloat16" in name):
                cal.setdefault((name, grid), {}).setdefault(counter, []).append(val * 1024.0)
    cal = [v for v in cal.values() if len(v.get("FETCH_SIZE", [])) >= CAL_REPEAT]
    if len(cal) != 1:
        raise SystemExit(f"expected one calibration copy kernel, found {len(cal)}")
    cal = cal[0]
    f_fetch = CAL_READ / float(np.median(cal["FETCH_SIZE"]))
    f_write = CAL_WRITE / float(np.median(cal["WRITE_SIZE"]))
    if sorted(k[0] for k in kq) != list(range(len(WORKLOAD))):
        raise SystemExit(f"quantizer dispatches do not alternate over the {len(WORKLOAD)} shapes: {sorted(kq)}")
    shapes = {}
    tot = 0.0
    for (k, grid), v in sorted(kq.items()):
        name, M, d = WORKLOAD[k]
        rd = float(np.mean(v["FETCH_SIZE"])) * f_fetch
        wr = float(np.mean(v["WRITE_SIZE"])) * f_write
        alg = M * d * BYTES_PER_ELEM
        shapes[name] = {"grid": grid, "dispatches": len(v["FETCH_SIZE"]), "read_bytes": round(rd),
                        "write_bytes": round(wr), "hbm_bytes": round(rd + wr), "algorithmic_bytes": round(alg),
                        "ratio": round((rd + wr) / alg, 4)}
        tot += rd + wr
    blob = {"kernel": "kq_mfma_kernel<true, kW>", "kernel_source_hash": kernel_source_hash(),
            "hbm_bytes_per_launch": round(tot / len(shapes)),
            "algorithmic_bytes_per_launch": round(sum(M * d for _, M, d in WORKLOAD) * BYTES_PER_ELEM / len(WORKLOAD)),
            "fetch_scale": round(f_fetch, 4), "write_scale": round(f_write, 4),
            "calibration": {"kernel": "torch bf16->fp32 copy", "elements": CAL_ELEMS,
                            "read_bytes": CAL_READ, "write_bytes": CAL_WRITE,
                            "fetch_kib_median": float(np.median(cal["FETCH_SIZE"])) / 1024,
                            "write_kib_median": float(np.median(cal["WRITE_SIZE"])) / 1024},
            "per_shape": shapes}
    lines = [
        "# HBM traffic of the KroQuant quantizer kernel, DiT CFG workload (8192 tokens, d=1152 and d=4608)",
        "",
        "Commands (from the repository root, on one MI355X; each counter pass is a run of its own):",
        "",
        "    timeout -s KILL 240 rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o fetch -- "
        "python3 bench.py --traffic-run --steps 20",
        "    timeout -s KILL 240 rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o write -- "
        "python3 bench.py --traffic-run --steps 20",
        "    python3 bench.py --summarize-traffic gpurun_out/pmc_fetch gpurun_out/pmc_write",
        "",
        f"Calibration: a plain bf16->fp32 copy of {CAL_ELEMS} elements reads {CAL_READ} B and writes {CAL_WRITE} B; "
        f"its counters read FETCH_SIZE {blob['calibration']['fetch_kib_median']:.0f} KiB and WRITE_SIZE "
        f"{blob['calibration']['write_kib_median']:.0f} KiB per dispatch, so FETCH_SIZE is scaled by "
        f"{f_fetch:.4f} and WRITE_SIZE by {f_write:.4f}.",
        "",
        "| shape | grid | dispatches | HBM read B | HBM write B | algorithmic B | HBM / algorithmic |",
        "|---|---|---|---|---|---|---|",
    ]
    for name, v in shapes.items():
        lines.append(f"| {name} | {v['grid']} | {v['dispatches']} | {v['read_bytes']} | {v['write_bytes']} | "
                     f"{v['algorithmic_bytes']} | {v['ratio']} |")
    lines += ["", "Per launch (average of the two shapes, as the roofline's `achieved`): "
              f"{blob['hbm_bytes_per_launch']} HBM bytes against {blob['algorithmic_bytes_per_launch']} algorithmic bytes.",
              "", "```json", json.dumps(blob, indent=1), "```", ""]
    with open(TRAFFIC_PROFILE, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def make_inputs():
    from synth import inputs as I
    mats = []
    for name, M, d in WORKLOAD:
        x = I.make_activation(name)
        f = I.make_factors(name)
        scale = I.smoothquant_scale(x)
        assert x.shape == (M, d)
        mats.append((name, x, f, scale))
    return mats


def cpu_baseline(mats, min_seconds=10.0):
    """The oracle, as it stands, over the whole step (every row of both
    matrices), spread over host threads by row ranges (ctypes releases the
    GIL), repeated until at least min_seconds of wall time."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as O
    O.lib()
    threads = max(1, min(16, os.cpu_count() or 1))
    jobs = []
    for _, x, f, _ in mats:
        rows = x.shape[0]
        chunk = max(1, (rows + 4 * threads - 1) // (4 * threads))
        for r0 in range(0, rows, chunk):
            jobs.append((np.ascontiguousarray(x[r0:r0 + chunk]), f))
    passes = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            list(ex.map(lambda a: O.kq_quantize(a[0], a[1]), jobs))
            passes += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
    dt = time.perf_counter() - t0
    elems = sum(x.size for _, x, _, _ in mats)
    return {
        "value": round(passes * elems * BYTES_PER_ELEM / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the full step (both DiT matrices, all 8192 rows, per-block factor sets) {passes} times, "
                  f"{passes * elems} elements in {dt:.1f} s wall on {threads} threads; same byte formula as the GPU value",
    }


def all_configs(args):
    """Every configured shape (except the tiny smoke case): the MFMA quantizer
    with per-block and with shared factors, the butterfly variant, SmoothQuant
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
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream
        legs = {
            "kq_mfma_perblock": lambda b: K.kq_quantize(b["x"], f_pb, b["q"], b["s"], stream=cur(), variant=1),
            "kq_mfma_shared": lambda b: K.kq_quantize(b["x"], f_sh, b["q"], b["s"], stream=cur(), variant=1),
            "kq_butterfly_perblock": lambda b: K.kq_quantize(b["x"], f_pb, b["q"], b["s"], stream=cur(), variant=2),
            "kq_lu_perblock": lambda b: K.kq_quantize_lu(b["x"], lu_pb, b["q"], b["s"], stream=cur()),
            "fwht": lambda b: K.fwht_quantize(b["x"], b["q"], b["s"], stream=cur()),
            "kq16_perblock": lambda b: K.kq_quantize16(b["x"], f16, b["q"], b["s16"], stream=cur()),
            "smoothquant": lambda b: K.sq_quantize(b["x"], scale, b["q"], b["s"], stream=cur()),
            "copy41": lambda b: K.measure_copy41(b["x"], b["q"], stream=cur()),
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
            nbytes = elems * 2.5 if leg == "copy41" else (elems * (2.5 + 1.0 / 16) if leg == "kq16_perblock" else alg)
            row[leg] = {"us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
                        "hbm_pct": round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 1), "rows/s": round(M / us * 1e6, 1)}
        row["kq_over_sq_speed"] = round(row["smoothquant"]["us"] / row["kq_mfma_perblock"]["us"], 4)
        row["kq_over_copy41_speed"] = round(row["copy41"]["us"] / row["kq_mfma_perblock"]["us"], 4)
        row["k2_lu_over_fwht_speed"] = round(row["fwht"]["us"] / row["kq_lu_perblock"]["us"], 4)
        table.append(row)
        print(json.dumps(row), flush=True)
        del bufs
        torch.cuda.empty_cache()
    print("| config | M x d | KQ MFMA per-block us (GB/s, %peak) | KQ MFMA shared us | KQ butterfly us | "
          "K2 LU us | FWHT us | SmoothQuant us (GB/s, %peak) | copy 4:1 us (GB/s) | KQ/SQ speed | "
          "KQ/copy speed | K2/FWHT speed | KQ16 butterfly us (GB/s) |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for r in table:
        a, b, c, l2, fw, q, cp = (r[k] for k in ("kq_mfma_perblock", "kq_mfma_shared", "kq_butterfly_perblock",
                                                   "kq_lu_perblock", "fwht", "smoothquant", "copy41"))
        print(f"| {r['config']} | {r['M']}x{r['d']} | {a['us']} ({a['GB/s']}, {a['hbm_pct']}%) | {b['us']} | "
              f"{c['us']} | {l2['us']} | {fw['us']} | {q['us']} ({q['GB/s']}, {q['hbm_pct']}%) | "
              f"{cp['us']} ({cp['GB/s']}) | {r['kq_over_sq_speed']} | {r['kq_over_copy41_speed']} | "
              f"{r['k2_lu_over_fwht_speed']} | {r['kq16_perblock']['us']} ({r['kq16_perblock']['GB/s']}) |", flush=True)


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
        K.set_tuning(7, 1)
        try:
            us_tile = _time_leg(lambda i: K.mx_gemm(*sets[i][:4], out=sets[i][4],
                                                    stream=torch.cuda.current_stream()), nsets, args.steps) * 1e6
        finally:
            K.set_tuning(7, 0)
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


ADALN_WORKLOADS = ("dit_1152", "mid_2240", "dbl_3072")  # the hidden widths AdaLN normalises
ADALN_EPS = 1e-6


def adaln_bench(args):
    """The AdaLN front-end fused with the quantizer (kq_adaln_quantize) against
    the unfused pipeline (adaln_modulate writing bf16 x, then kq_quantize with
    the MFMA or the butterfly transform) and against torch's layer_norm and
    modulation (bf16 out) followed by kq_quantize, at the hidden widths, two samples
    (CFG) per batch.  Two more fused legs select the butterfly second pass and
    the matrix-core second pass in strips of 4 blocks.  Fused algorithmic bytes: 2.53125 B per element (h read,
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
                for key, val in knobs.items():
                    K.set_tuning(key, val)
                try:
                    fused(i)
                finally:
                    for key in knobs:
                        K.set_tuning(key, 0)
            return run

        t = {"fused": _time_leg(fused, nsets, args.steps),
             "fused_butterfly_pass": _time_leg(fused_with({8: 2}), nsets, args.steps),
             "fused_mfma_strip4": _time_leg(fused_with({8: 1, 9: 4}), nsets, args.steps),
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
    if args.all_configs or args.gemm or args.adaln:
        if args.gpus != 1:
            sys.exit(2)
        if args.all_configs:
            all_configs(args)
        elif args.gemm:
            gemm_bench(args)
        else:
            adaln_bench(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the quantizer shards by "
              f"rows with no communication, so N GPUs run N independent copies of this step)", file=sys.stderr)
        sys.exit(2)
    import torch

    import mxfp4_act_quantizer_amd as K
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no GPU visible)", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    mats = make_inputs()
    from synth import inputs as I

    # ---- device buffers, rotated so one cycle touches >= 1 GB
    step_bytes = sum(x.size * BYTES_PER_ELEM for _, x, _, _ in mats)
    nsets = max(2, int(np.ceil(ROTATE_BYTES / step_bytes)))
    sets = []
    for _ in range(nsets):
        one = []
        for name, x, f, scale in mats:
            M, d = x.shape
            xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
            lu = I.random_lu(d // 32, I.factor_seed(name) + 77)
            one.append(dict(x=xd, f=torch.from_numpy(f).to(dev), scale=torch.from_numpy(scale).to(dev),
                            lu=torch.from_numpy(lu).to(dev),
                            q=torch.empty((M, d // 2), dtype=torch.uint8, device=dev),
                            s=torch.empty((M, d // 32), dtype=torch.uint8, device=dev)))
        sets.append(one)
    torch.cuda.synchronize()

    def step_kq(i, variant):
        for b in sets[i % nsets]:
            K.kq_quantize(b["x"], b["f"], b["q"], b["s"], stream=torch.cuda.current_stream(), variant=variant)

    def step_sq(i):
        for b in sets[i % nsets]:
            K.sq_quantize(b["x"], b["scale"], b["q"], b["s"], stream=torch.cuda.current_stream())

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
        return g

    def timed_graph(g, replays=1):
        """Replay a graph: wall and event time of the replays, bracketed by synchronisation."""
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) / 1e3

    def clock_ramp(g):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < RAMP_S:
            g.replay()
            torch.cuda.synchronize()
        return round(time.perf_counter() - t0, 3)

    variant = args.variant
    if args.traffic_run:
        src = torch.randn(CAL_ELEMS, device=dev).to(torch.bfloat16)
        dst = torch.empty(CAL_ELEMS, dtype=torch.float32, device=dev)
        for _ in range(CAL_REPEAT):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        for i in range(args.warmup + args.steps):
            step_kq(i, variant)
        torch.cuda.synchronize()
        print(f"traffic run: {CAL_REPEAT} calibration copies, {args.warmup + args.steps} quantizer steps", flush=True)
        return
    # the timed region: exactly K steps, launched as one graph (the launches
    # themselves would otherwise leave the GPU idle between short kernels)
    g_warm = capture(lambda i: step_kq(i, variant), max(1, args.warmup))
    g_main = capture(lambda i: step_kq(i, variant), args.steps)
    # the GPU idles in a low-power state: untimed replays until its clocks
    # have ramped (about RAMP_S seconds), then the W warm-up steps, then K
    ramp_s = clock_ramp(g_warm)
    timed_graph(g_warm)
    wall, ev = timed_graph(g_main)
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (wall / args.steps) / 1e9

    # roofline of the quantizer kernel: per shape, a graph of back-to-back
    # launches over the rotating buffers, timed with events on its stream
    LAUNCHES = 40
    launch_bytes = [x.size * BYTES_PER_ELEM for _, x, _, _ in mats]
    per_shape = {}
    for k, (name, x, _, _) in enumerate(mats):
        def one(i, k=k):
            b = sets[i % nsets][k]
            K.kq_quantize(b["x"], b["f"], b["q"], b["s"], stream=torch.cuda.current_stream(), variant=variant)
        g = capture(one, LAUNCHES)
        timed_graph(g)
        _, t = timed_graph(g, 3)
        avg = t / (3 * LAUNCHES)
        per_shape[name] = {"avg_us": round(avg * 1e6, 2), "GB/s": round(launch_bytes[k] / avg / 1e9, 1),
                           "rows/s": round(x.shape[0] / avg, 1), "hbm_pct": round(100 * launch_bytes[k] / avg / 8e12, 2)}
    # achieved: the timed region itself (its HIP events), per quantizer launch
    n_launch = args.steps * len(mats)
    achieved = step_bytes * args.steps / ev / 1e9
    src_hash = kernel_source_hash()
    traffic = load_traffic(src_hash)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": ("kq_mfma_kernel<true, kW> (kW = 8 at d=1152, 16 at d=4608)" if variant in (0, 1)
                           else "stream_kernel<2>"),
                "avg_launch_us": round(ev / n_launch * 1e6, 2), "launches_timed": n_launch,
                "algorithmic_bytes_per_launch": round(step_bytes / len(mats)),
                "timing": "HIP events on the launch stream around the timed graph of K steps",
                "per_shape": per_shape, "per_shape_timing": f"graphs of {LAUNCHES} launches of one shape, replayed 3x"}

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "DiT CFG batch: 2x4096 tokens, d=1152 (36 factor sets) + d=4608 (144 factor sets), "
                               "bf16 in, MXFP4 + E8M0 out, per-block Kronecker transforms",
                   "M": 8192, "d": [1152, 4608], "nT": [36, 144], "variant": ["auto", "mfma", "butterfly"][variant],
                   "rows_per_step": 2 * 8192, "rotating_sets": nsets, "accumulate": "fp32",
                   "launch": "HIP graph of the K timed steps", "clock_ramp_s": ramp_s,
                   "hbm_pct": round(100 * value / HBM_PEAK_GBS, 2),
                   "rows_per_s": round(2 * 8192 / (wall / args.steps), 1),
                   "kernel_source_hash": src_hash},
        "roofline": roofline,
    }

    if not args.no_extras:
        g_sq = capture(step_sq, args.steps)
        timed_graph(capture(step_sq, max(1, args.warmup)))
        sq_wall, _ = timed_graph(g_sq)
        sq_value = step_bytes / (sq_wall / args.steps) / 1e9
        other = 2 if variant in (0, 1) else 1
        g_o = capture(lambda i: step_kq(i, other), args.steps)
        timed_graph(capture(lambda i: step_kq(i, other), max(1, args.warmup)))
        o_wall, _ = timed_graph(g_o)
        def step_lu(i):
            for b in sets[i % nsets]:
                K.kq_quantize_lu(b["x"], b["lu"], b["q"], b["s"], stream=torch.cuda.current_stream())

        def step_fwht(i):
            for b in sets[i % nsets]:
                K.fwht_quantize(b["x"], b["q"], b["s"], stream=torch.cuda.current_stream())

        walls = {}
        for nm, fn in (("lu", step_lu), ("fwht", step_fwht)):
            g = capture(fn, args.steps)
            timed_graph(capture(fn, max(1, args.warmup)))
            walls[nm], _ = timed_graph(g)

        def step_copy(i):
            for b in sets[i % nsets]:
                K.measure_copy41(b["x"], b["q"], stream=torch.cuda.current_stream())
        g_c = capture(step_copy, args.steps)
        timed_graph(capture(step_copy, max(1, args.warmup)))
        c_wall, _ = timed_graph(g_c)
        copy_bytes = sum(x.size * 2.5 for _, x, _, _ in mats)
        out["comparison"] = {
            "smoothquant_GB/s": round(sq_value, 1),
            "smoothquant_hbm_pct": round(100 * sq_value / HBM_PEAK_GBS, 2),
            "kroquant_over_smoothquant_speed": round(sq_wall / wall, 4),
            ("butterfly_GB/s" if other == 2 else "mfma_GB/s"): round(step_bytes / (o_wall / args.steps) / 1e9, 1),
            "k2_lu_GB/s": round(step_bytes / (walls["lu"] / args.steps) / 1e9, 1),
            "fwht_GB/s": round(step_bytes / (walls["fwht"] / args.steps) / 1e9, 1),
            "k2_lu_over_fwht_speed": round(walls["fwht"] / walls["lu"], 4),
            "k2": "factor sets as 15 LU scalars per block, rebuilt in the kernel (kq_quantize_lu); "
                  "fwht: fixed normalised Walsh-Hadamard-32 + MXFP4 (fwht_quantize)",
            "copy41_ceiling_GB/s": round(copy_bytes / (c_wall / args.steps) / 1e9, 1),
            "kroquant_over_copy41_speed": round(c_wall / wall, 4),
            "copy41": "plain streaming copy of the same x (2 B read) into the q buffers (0.5 B written) per element",
        }

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(mats, args.cpu_seconds)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
