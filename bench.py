"""Benchmark of the exact tiled attention hot path on one MI355X.

One step = one forward pass (S = scale Q K^T, online softmax, P V, LSE) and one backward pass
(D pre-pass, dK/dV, dQ) over one batch of seeded synthetic input of the chosen workload, inputs
resident in device memory.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long] [--no-cpu-baseline]
                    [--copy-calibration MIB]
    python bench.py --traffic-from FETCH_CSV WRITE_CSV [--workload long]
    python bench.py --linear-sweep [--copy-calibration 256]     (under rocprofv3 --pmc)
    python bench.py --sweep-from FETCH_CSV WRITE_CSV
    python bench.py --mfma-from COUNTER_CSV
    python bench.py --counters-from COUNTER_CSV
    python bench.py --data-sensitivity [--workload long]       (alone, or under rocprofv3 --pmc)
    python bench.py --data-sensitivity-from COUNTER_CSV

HBM traffic: run the bench twice under `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE` with
`--copy-calibration 256`, which first copies 256 MiB with the runtime's copy kernel.  The two
counters read a fixed fraction of the true bytes on this part; the copy of known size gives that
fraction.  `--traffic-from` turns the two counter files into profiles/hbm_traffic.json (bytes
per launch of each attention kernel, tagged with a digest of the kernel sources so that a later
kernel change voids it) and prints a markdown summary.

FLOP convention: forward 4*B*H*N^2*d (halved for causal; block-sparse counts active 128x128
blocks), backward 2.5x forward.  value = (forward + backward flops) / step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 bf16 flop/clk x 2.4 GHz (dense)
PEAK_FP8_TFLOPS = 5033.2    # 256 CU x 8192 fp8 flop/clk x 2.4 GHz (dense)
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd/bwd TFLOP/s (bf16, d=64/128) and % of MI355X MFMA peak"
CSRC = os.path.join(ROOT, "exact_io_aware_flash_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def csrc_digest() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def kernel_flops(w, block_mask):
    import workloads

    f = workloads.flops_fwd(w.B, w.H, w.N, w.d, w.causal, block_mask)
    return {
        # MFMA work each kernel performs by definition: fwd S and PV; dK/dV kernel recomputes S,
        # computes dP, dV, dK; dQ kernel recomputes S and dP, computes dQ.
        "fwd": f,
        "bwd_dkdv": 2.0 * f,
        "bwd_dq": 1.5 * f,
    }


def preprocess_bytes(w):
    # reads O and dO (bf16), writes D (float32)
    return 2 * w.B * w.H * w.N * w.d * 2 + w.B * w.H * w.N * 4


KERNEL_KEYS = {"fwd_bf16_kernel": "fwd", "fwd_pingpong_kernel": "fwd_pingpong", "bwd_delta_kernel": "bwd_preprocess",
               "bwd_dkdv_kernel": "bwd_dkdv", "bwd_dkdv_wave_kernel": "bwd_dkdv", "bwd_dq_kernel": "bwd_dq", "fwd_mxfp8_kernel": "fwd_mxfp8",
               "mx_quantize_rows_kernel": "mxfp8_quantize_rows", "mx_quantize_vt_kernel": "mxfp8_quantize_vt"}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_label(name: str):
    """Short label of a library kernel from its profiler name (None for other kernels); the bf16
    forward without the causal mask is labelled apart from the causal one."""
    for key, short in KERNEL_KEYS.items():
        if key in name:
            if short == "fwd" and "<" in name and name.split("<", 1)[1].split(",")[1].strip() == "false":
                return "fwd_noncausal"
            if short == "fwd_pingpong" and "<false" in name:
                return "fwd_pingpong_noncausal"
            return short
    return None


def check_one_kernel_per_label(names_by_label: dict, path: str):
    """A label must stand for one kernel instantiation: a counter run that also launched the
    kernels of other shapes (the d = 64 workloads of the default bench line) would mix them."""
    mixed = {k: sorted(v) for k, v in names_by_label.items() if len(v) > 1}
    if mixed:
        raise SystemExit(f"{path}: several kernels under one label {sorted(mixed)}; profile the bench with "
                         "--no-other-workloads --no-gemm")


def read_counter(path: str, counter: str):
    """{dispatch id: (kernel name, counter value summed over the rows of that dispatch)}."""
    import csv

    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, v = per.get(d, (r["Kernel_Name"], 0.0))
            per[d] = (name, v + float(r["Counter_Value"]))
    return per


def traffic_from(fetch_csv: str, write_csv: str, workload: str, copy_mib: int = 256):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by the copy kernel's reading of a copy of
    known size, write profiles/hbm_traffic.json and return a markdown summary."""
    import statistics

    copy_bytes = copy_mib * 2 ** 20
    out = {"csrc_sha256": csrc_digest(), "workload": workload, "copy_bytes": copy_bytes,
           "sources": [os.path.relpath(fetch_csv, ROOT), os.path.relpath(write_csv, ROOT)], "kernels": []}
    per_kernel = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = read_counter(path, counter)
        copies = [v for name, v in vals.values() if COPY_KERNEL in name]
        if not copies:
            raise SystemExit(f"{path}: no {COPY_KERNEL} dispatch; run the bench with --copy-calibration {copy_mib}")
        factor = copy_bytes / (statistics.median(copies) * 1024.0)
        out[counter.lower() + "_factor"] = factor
        names = {}
        for name, v in vals.values():
            short = kernel_label(name)
            if short:
                names.setdefault(short, set()).add(name)
                per_kernel.setdefault(short, {}).setdefault(counter, []).append(v * 1024.0 * factor)
        check_one_kernel_per_label(names, path)
    lines = [f"| kernel | dispatches | FETCH bytes/launch | WRITE bytes/launch | HBM bytes/launch |",
             "|---|---|---|---|---|"]
    for short, c in per_kernel.items():
        fb = statistics.median(c.get("FETCH_SIZE", [0.0]))
        wb = statistics.median(c.get("WRITE_SIZE", [0.0]))
        out["kernels"].append({"kernel": short, "workload": workload, "dispatches": len(c.get("FETCH_SIZE", [])),
                               "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                               "hbm_bytes_per_launch": fb + wb})
        lines.append(f"| {short} | {len(c.get('FETCH_SIZE', []))} | {fb:.4g} | {wb:.4g} | {fb + wb:.4g} |")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    head = (f"copy calibration: {copy_mib} MiB copy; FETCH_SIZE factor {out['fetch_size_factor']:.3f}, "
            f"WRITE_SIZE factor {out['write_size_factor']:.3f}\n\n")
    return head + "\n".join(lines)


LINEAR_NS = (4096, 8192, 16384, 32768, 65536)


def linear_sweep(dev):
    """Causal forward at B=1, H=8, d=128 for each N in LINEAR_NS (seeded device-side Gaussian
    inputs), two calls each; for a counter run that shows how HBM bytes per call grow with N."""
    import torch

    import exact_io_aware_flash_amd as fa

    for N in LINEAR_NS:
        g = torch.Generator(device=dev)
        g.manual_seed(N)
        q, k, v = (torch.randn(1, 8, N, 128, device=dev, generator=g).to(torch.bfloat16) for _ in range(3))
        o = torch.empty_like(q)
        lse = torch.empty((1, 8, N), dtype=torch.float32, device=dev)
        for _ in range(2):
            fa.fwd(q, k, v, 1.0 / 128 ** 0.5, True, None, out=o, lse=lse)
        torch.cuda.synchronize()
        print(f"# linear sweep N={N} done", file=sys.stderr, flush=True)
        del q, k, v, o, lse


def sweep_from(fetch_csv: str, write_csv: str, copy_mib: int = 256) -> str:
    """Markdown table of forward HBM bytes per call against N from two counter files of a
    --linear-sweep run (the forward grid, N/128 * 8 workgroups, identifies N)."""
    import statistics

    factors, per_n = {}, {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        import csv

        rows = list(csv.DictReader(open(path)))
        vals, grids = {}, {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            dsp = int(r["Dispatch_Id"])
            vals[dsp] = vals.get(dsp, 0.0) + float(r["Counter_Value"])
            grids[dsp] = (r["Kernel_Name"], int(r["Grid_Size"]))
        copies = [vals[d_] for d_, (n, _) in grids.items() if COPY_KERNEL in n]
        factors[counter] = copy_mib * 2 ** 20 / (statistics.median(copies) * 1024.0)
        for d_, (n, grid) in grids.items():
            if "fwd_bf16_kernel" in n:
                N = grid // 256 // 8 * 128
                per_n.setdefault(N, {}).setdefault(counter, []).append(vals[d_] * 1024.0 * factors[counter])
    lines = [f"FETCH_SIZE factor {factors['FETCH_SIZE']:.3f}, WRITE_SIZE factor {factors['WRITE_SIZE']:.3f} "
             f"(from the {copy_mib} MiB copy)\n",
             "| N | algorithmic bytes (Q, K, V read; O, LSE written) | measured HBM bytes/call | measured ÷ algorithmic | "
             "S+P materialisation (16·N²·H bytes) |", "|---|---|---|---|---|"]
    for N in sorted(per_n):
        meas = statistics.median(per_n[N]["FETCH_SIZE"]) + statistics.median(per_n[N]["WRITE_SIZE"])
        alg = 8 * (4 * N * 128 * 2 + 4 * N)
        lines.append(f"| {N} | {alg / 1e6:.1f} MB | {meas / 1e6:.1f} MB | {meas / alg:.2f} | {16 * N * N * 8 / 1e9:.1f} GB |")
    return "\n".join(lines)


def mfma_from(csv_path: str) -> str:
    """Markdown table of MFMA utilisation per attention kernel from a counter run with
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA and GRBM_GUI_ACTIVE (summed over the 8 XCDs)."""
    import csv
    import statistics

    per = {}
    for r in csv.DictReader(open(csv_path)):
        dsp = int(r["Dispatch_Id"])
        e = per.setdefault(dsp, {"name": r["Kernel_Name"], "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = {}
    check_one_kernel_per_label({lab: {e["name"] for e in per.values() if kernel_label(e["name"]) == lab}
                                for lab in {kernel_label(e["name"]) for e in per.values()} if lab}, csv_path)
    for e in per.values():
        short = kernel_label(e["name"])
        if short and "SQ_VALU_MFMA_BUSY_CYCLES" in e:
            cycles = e["GRBM_GUI_ACTIVE"] / 8.0  # per XCD
            util = e["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024.0 * cycles) if cycles else 0.0
            out.setdefault(short, []).append((util, cycles / (e["ns"] * 1e-9) / 1e9, e.get("SQ_INSTS_MFMA", 0.0)))
    lines = ["| kernel | dispatches | MFMA busy ÷ (1024 SIMDs × kernel cycles) | kernel clock from GRBM_GUI_ACTIVE ÷ duration | "
             "MFMA instructions |", "|---|---|---|---|---|"]
    for short, v in out.items():
        u = statistics.median(x[0] for x in v)
        c = statistics.median(x[1] for x in v)
        n = statistics.median(x[2] for x in v)
        lines.append(f"| {short} | {len(v)} | {100 * u:.1f}% | {c:.2f} GHz | {n:.4g} |")
    return "\n".join(lines)


GEMM_N = 8192                       # the library GEMM timed beside the attention kernels
SENS_CALLS = 7                      # calls per case in --data-sensitivity (2 warm-up + 5 timed)


def timed_calls(fn, warm: int = 2, n: int = 5) -> float:
    """Median milliseconds of n event-timed calls of fn after warm untimed ones (torch's stream)."""
    import torch

    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return sorted(ts)[len(ts) // 2]


def library_gemm(dev, n: int = GEMM_N, fill: str = "randn", warm: int = 2, calls: int = 5):
    """Rate of the vendor library's bf16 GEMM (torch.matmul, n x n x n) on the same kind of
    inputs: a reference for what the matrix cores sustain on this part under this data, not a
    step of the attention path."""
    import torch

    g = torch.Generator(device=dev)
    g.manual_seed(n)
    if fill == "randn":
        a, b = (torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16) for _ in range(2))
    else:
        a, b = (torch.zeros(n, n, device=dev, dtype=torch.bfloat16) for _ in range(2))
    ms = timed_calls(lambda: torch.matmul(a, b), warm, calls)
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"shape": f"{n}x{n}x{n} bf16 {'N(0,1)' if fill == 'randn' else 'zeros'}", "ms": ms, "TFLOP/s": tf,
            "frac_of_peak": tf / PEAK_BF16_TFLOPS}


def data_sensitivity(dev, w, q, k, v):
    """Causal forward at the workload's shape on its N(0,1) inputs, on those inputs times 0.01, on
    zeros and on ones; then the library GEMM on N(0,1) and on zeros.  Same kernels, same work:
    any difference is the part's power limit reacting to the data.  SENS_CALLS calls per case,
    in that order (the counter parser relies on it)."""
    import torch

    import exact_io_aware_flash_amd as fa

    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ff = 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if w.causal else 1.0)
    cases = [("N(0,1) (the workload's inputs)", (q, k, v)),
             ("N(0,1) x 0.01", tuple((x.float() * 0.01).to(torch.bfloat16) for x in (q, k, v))),
             ("zeros", tuple(torch.zeros_like(q) for _ in range(3))),
             ("ones", tuple(torch.ones_like(q) for _ in range(3)))]
    lines = ["| kernel | inputs | ms (median of 5) | TFLOP/s | % of bf16 peak |", "|---|---|---|---|---|"]
    for name, (a, b, c) in cases:
        ms = timed_calls(lambda: fa.fwd(a, b, c, w.scale, w.causal, None, out=o, lse=lse), 2, SENS_CALLS - 2)
        tf = ff / (ms * 1e-3) / 1e12
        lines.append(f"| attention forward ({w.name}) | {name} | {ms:.3f} | {tf:.0f} | {100 * tf / PEAK_BF16_TFLOPS:.1f} |")
        print(lines[-1], file=sys.stderr, flush=True)
    for n in (GEMM_N, 2 * GEMM_N):
        for fill in ("randn", "zeros"):
            r = library_gemm(dev, n, fill, 2, SENS_CALLS - 2)
            lines.append(f"| torch.matmul (vendor library) | {r['shape']} | {r['ms']:.3f} | {r['TFLOP/s']:.0f} | "
                         f"{100 * r['frac_of_peak']:.1f} |")
            print(lines[-1], file=sys.stderr, flush=True)
    return "\n".join(lines)


def data_sensitivity_from(csv_path: str) -> str:
    """Clock and MFMA busy fraction per case of a --data-sensitivity counter run (counters as in
    --mfma-from).  Dispatches of the forward come in blocks of SENS_CALLS per input case, and so do
    those of the GEMM kernel (the most frequent other kernel with MFMA instructions)."""
    import csv
    import statistics

    per = {}
    for r in csv.DictReader(open(csv_path)):
        dsp = int(r["Dispatch_Id"])
        e = per.setdefault(dsp, {"name": r["Kernel_Name"], "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    order = [per[d] for d in sorted(per)]
    fwd = [e for e in order if kernel_label(e["name"]) == "fwd"]
    others = {}
    for e in order:
        if kernel_label(e["name"]) is None and e.get("SQ_INSTS_MFMA", 0.0) > 0:
            others.setdefault(e["name"], []).append(e)
    gemm = max(others.values(), key=len) if others else []
    f_cases = ["N(0,1)", "N(0,1) x 0.01", "zeros", "ones"]
    g_cases = [f"{GEMM_N}^3 N(0,1)", f"{GEMM_N}^3 zeros", f"{2 * GEMM_N}^3 N(0,1)", f"{2 * GEMM_N}^3 zeros"]
    lines = ["| kernel | inputs | dispatches | MFMA busy ÷ (1024 SIMDs × kernel cycles) | kernel clock (GHz) |",
             "|---|---|---|---|---|"]
    for label, seq, names in (("attention forward", fwd, f_cases), ("library GEMM", gemm, g_cases)):
        for i, case in enumerate(names):
            blk = seq[i * SENS_CALLS:(i + 1) * SENS_CALLS][2:]  # the timed calls
            if not blk:
                continue
            util, clk = [], []
            for e in blk:
                cycles = e["GRBM_GUI_ACTIVE"] / 8.0
                util.append(e["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024.0 * cycles) if cycles else 0.0)
                clk.append(cycles / (e["ns"] * 1e-9) / 1e9)
            lines.append(f"| {label} | {case} | {len(blk)} | {100 * statistics.median(util):.1f}% | "
                         f"{statistics.median(clk):.2f} |")
    return "\n".join(lines)


OTHER_WORKLOADS = ("bert", "gpt2", "sparse")


def percentiles(ms_list):
    """p10 / p50 / p90 of a list of per-call milliseconds (nearest rank)."""
    v = sorted(ms_list)
    pick = lambda q: v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]
    return {"p10_ms": pick(0.1), "p50_ms": pick(0.5), "p90_ms": pick(0.9)}


def time_workload(fa, w, dev, steps: int, warmup: int):
    """Forward and the three backward kernels of one workload on its seeded inputs.  Each kernel
    is launched `steps` times back to back (at least 20), captured into a HIP graph on torch's
    current stream (the stream the library launches on) and replayed between one pair of events,
    so that the host's launch overhead of these microsecond kernels stays out of the figure;
    TFLOP/s under the same convention as the main figure."""
    import numpy as np
    import torch

    import workloads

    t = workloads.make(w, with_do=True)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v, do = (to_dev(x) for x in (t.q, t.k, t.v, t.do))
    mask = torch.from_numpy(t.block_mask).to(dev) if t.block_mask is not None else None
    B, H, N, d = w.B, w.H, w.N, w.d
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = fa.new_workspace(B, H, N, d, dev)
    calls = [lambda: fa.fwd(q, k, v, w.scale, w.causal, mask, out=o, lse=lse),
             lambda: fa.bwd_preprocess(q, o, do, ws),
             lambda: fa.bwd_dkdv(q, k, v, do, lse, ws, w.scale, w.causal, mask, dk, dv),
             lambda: fa.bwd_dq(q, k, v, do, lse, ws, w.scale, w.causal, mask, dq)]
    n = max(20, steps)
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()

    def replayed(c):
        # n launches captured into one HIP graph and replayed between two events: the kernels run
        # back to back with no host launch gaps (the library makes no allocation or memset, so
        # its launches capture as they are)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                c()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    per = [replayed(c) for c in calls]
    ff = workloads.flops_fwd(B, H, N, d, w.causal, t.block_mask)
    fwd_ms, bwd_ms = per[0], sum(per[1:])
    return {"config": w.description, "launches_per_kernel": n, "timing": "HIP graph of n launches, replayed once",
            "fwd_ms": fwd_ms, "bwd_preprocess_ms": per[1],
            "bwd_dkdv_ms": per[2], "bwd_dq_ms": per[3], "bwd_ms": bwd_ms,
            "fwd_TFLOP/s": ff / (fwd_ms * 1e-3) / 1e12, "bwd_TFLOP/s": 2.5 * ff / (bwd_ms * 1e-3) / 1e12,
            "fwd+bwd_TFLOP/s": 3.5 * ff / ((fwd_ms + bwd_ms) * 1e-3) / 1e12}


def counters_from(csv_path: str) -> str:
    """Markdown table of every counter in a rocprofv3 counter file, per attention kernel: the
    median over its dispatches of each counter summed over the dispatch's rows, and for the SQ
    wait / active counters their ratio to SQ_WAVE_CYCLES (the share of the waves' cycles)."""
    import csv
    import statistics

    per = {}
    for r in csv.DictReader(open(csv_path)):
        e = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    check_one_kernel_per_label({lab: {e["name"] for e in per.values() if kernel_label(e["name"]) == lab}
                                for lab in {kernel_label(e["name"]) for e in per.values()} if lab}, csv_path)
    names = sorted({k for e in per.values() for k in e if k != "name"})
    by = {}
    for e in per.values():
        lab = kernel_label(e["name"])
        if lab:
            by.setdefault(lab, []).append(e)
    lines = ["| kernel | dispatches | " + " | ".join(names) + " |", "|---|---|" + "---|" * len(names)]
    for lab, es in by.items():
        cells = []
        for n in names:
            v = statistics.median(e.get(n, 0.0) for e in es)
            cell = f"{v:.4g}"
            wc = statistics.median(e.get("SQ_WAVE_CYCLES", 0.0) for e in es)
            if wc and (n.startswith("SQ_WAIT") or n.startswith("SQ_ACTIVE_INST")):
                cell += f" ({100 * v / wc:.1f}%)"
            cells.append(cell)
        lines.append(f"| {lab} | {len(es)} | " + " | ".join(cells) + " |")
    return "\n".join(lines)


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the current
    kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("csrc_sha256") != csrc_digest():
        return None
    import workloads

    if kernel == "fwd" and not workloads.WORKLOADS[workload].causal:
        kernel = "fwd_noncausal"
    for k in rec.get("kernels", []):
        if k.get("kernel") == kernel and k.get("workload") == workload:
            return k.get("hbm_bytes_per_launch")
    return None


_CPU_T = None  # the workload's host tensors, shared with the forked oracle workers


def _single_thread_blas():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:  # noqa: BLE001
        pass


def _oracle_head(task):
    """One (b, h) of the oracle in a worker process (forward, and backward unless forward-only)."""
    import numpy as np

    import oracle
    import workloads

    b, h, scale, causal, fwd_only = task
    f = lambda name: workloads.bf16_bits_to_f32(getattr(_CPU_T, name)[b, h]).astype(np.float64)
    t0 = time.perf_counter()
    q, k, v = f("q"), f("k"), f("v")
    oracle.forward_head(q, k, v, scale, causal, _CPU_T.block_mask)
    if not fwd_only:
        oracle.backward_head(q, k, v, f("do"), scale, causal, _CPU_T.block_mask)
    return time.perf_counter() - t0


def cpu_workers() -> int:
    """Host cores this process may use (its CPU affinity), at most 16 (one GPU's share of a box)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(w, t, heads: int | None = None):
    """The fp64 oracle timed on the host: a pool of one process per usable core (BLAS limited to
    one thread each), one (b, h) per task, `heads` heads of the same inputs (default: one per
    worker), forward + backward.  Run before the GPU is initialised, and the pool is joined, so
    no process outlives it."""
    import multiprocessing

    global _CPU_T
    workers = cpu_workers()
    heads = min(heads or workers, w.B * w.H)
    tasks = [(i // w.H, i % w.H, w.scale, w.causal, w.fwd_only) for i in range(heads)]
    _CPU_T = t
    ctx = multiprocessing.get_context("fork")
    t0 = time.perf_counter()
    pool = ctx.Pool(workers, initializer=_single_thread_blas)
    try:
        per_head = pool.map(_oracle_head, tasks, chunksize=1)
    finally:
        pool.close()
        pool.join()
    dt = time.perf_counter() - t0
    _CPU_T = None
    import workloads

    one = workloads.flops_fwd(1, 1, w.N, w.d, w.causal, t.block_mask)
    flops = heads * (one if w.fwd_only else 3.5 * one)
    cpu = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{heads} of {w.B * w.H} heads (b,h) of the same workload, fp64 numpy "
                  f"{'forward' if w.fwd_only else 'forward+backward'}, one head per task on a pool of "
                  f"{workers} processes with one BLAS thread each; {dt:.1f} s wall "
                  f"(per head {min(per_head):.1f}-{max(per_head):.1f} s), {cpu}",
        "seconds": dt,
    }


def fp8_forward(fa, w, q, k, v, mask, flops, iters):
    """The MX-FP8 forward on the same inputs, as a separate figure (not the metric): the
    quantisation of Q, K (row blocks) and V (transposed) and the forward, each timed with events
    on the library's stream."""
    import torch

    def timed(fn, n):
        for _ in range(2):
            fn()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        e[0].record()
        for _ in range(n):
            fn()
        e[1].record()
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / n

    Q8, K8, V8 = fa.mxfp8_quantize(q), fa.mxfp8_quantize(k), fa.mxfp8_quantize(v, transposed=True)
    o8, l8 = fa.fwd_mxfp8(Q8, K8, V8, w.scale, w.causal, mask)
    ms = timed(lambda: fa.fwd_mxfp8(Q8, K8, V8, w.scale, w.causal, mask, out=o8, lse=l8), iters)
    qms = timed(lambda: (fa.mxfp8_quantize(q), fa.mxfp8_quantize(k), fa.mxfp8_quantize(v, transposed=True)), iters)
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": ms, "TFLOP/s": tf, "frac_of_bf16_peak": tf / PEAK_BF16_TFLOPS,
            "roofline": {"kernel": "fwd_mxfp8", "bound": "mfma", "achieved": tf, "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / PEAK_FP8_TFLOPS, "traffic": traffic_for("fwd_mxfp8", w.name)},
            "quantize_qkv_ms": qms, "TFLOP/s_with_quantize": flops / ((ms + qms) * 1e-3) / 1e12,
            "dtype": "MX-FP8 E4M3 operands, fp32 accumulation and softmax"}


def fp8_cpu_baseline(w, t):
    """The oracle of the FP8 forward on the host: host MX-FP8 quantisation of one head, then the
    fp64 forward on the dequantised inputs."""
    import numpy as np

    import oracle
    import workloads
    from oracle import mx

    f = lambda name: workloads.bf16_bits_to_f32(getattr(t, name)[0, 0]).astype(np.float64)
    t0 = time.perf_counter()
    qd = mx.dequantize(*mx.quantize(f("q"), axis=-1), axis=-1)
    kd = mx.dequantize(*mx.quantize(f("k"), axis=-1), axis=-1)
    vd = mx.dequantize(*mx.quantize(f("v"), axis=0), axis=0)
    oracle.forward_head(qd, kd, vd, w.scale, w.causal, t.block_mask)
    dt = time.perf_counter() - t0
    return {"value": workloads.flops_fwd(1, 1, w.N, w.d, w.causal, t.block_mask) / dt / 1e12, "unit": "TFLOP/s",
            "kind": "oracle", "sample": f"head (0,0): host MX-FP8 quantisation + fp64 forward, {dt:.1f} s",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the MX-FP8 forward figure")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads the oracle times on the host (default: one per usable core, at most 16)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="copy MIB MiB with the runtime's copy kernel before the bench (counter scaling)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from two rocprofv3 counter files and exit")
    ap.add_argument("--linear-sweep", action="store_true",
                    help="run the causal forward at B=1 H=8 d=128 for N = 4k .. 64k (for a counter run) and exit")
    ap.add_argument("--sweep-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print HBM bytes per forward call against N from a --linear-sweep counter run and exit")
    ap.add_argument("--mfma-from", metavar="CSV",
                    help="print MFMA utilisation per kernel from an SQ counter run and exit")
    ap.add_argument("--counters-from", metavar="CSV",
                    help="print every counter of a counter run per kernel (with shares of SQ_WAVE_CYCLES) and exit")
    ap.add_argument("--data-sensitivity", action="store_true",
                    help="time the forward and the library GEMM on N(0,1), scaled, zero and one inputs and exit")
    ap.add_argument("--data-sensitivity-from", metavar="CSV",
                    help="print clock and MFMA busy per case from a --data-sensitivity counter run and exit")
    ap.add_argument("--no-gemm", action="store_true", help="skip the library GEMM reference figure")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the figures of the d = 64 workloads (BERT-, GPT-2-shaped, block-sparse)")
    args = ap.parse_args()
    if args.traffic_from:
        print(traffic_from(*args.traffic_from, workload=args.workload, copy_mib=args.copy_calibration or 256))
        return
    if args.sweep_from:
        print(sweep_from(*args.sweep_from, copy_mib=args.copy_calibration or 256))
        return
    if args.mfma_from:
        print(mfma_from(args.mfma_from))
        return
    if args.counters_from:
        print(counters_from(args.counters_from))
        return
    if args.data_sensitivity_from:
        print(data_sensitivity_from(args.data_sensitivity_from))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "heads are independent, so the multi-GPU figure is the one-GPU figure on each GPU's share "
              "of B*H.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_io_aware_flash_amd as fa
    import workloads

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration * 2 ** 20 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.linear_sweep:
        linear_sweep(dev)
        return
    t_gen = time.perf_counter()
    t = workloads.make(w, with_do=not w.fwd_only)
    # the oracle on the host cores first, before anything initialises the GPU: its worker
    # processes are forked from a process without GPU state and are all joined here
    cpu_line = fp8_cpu_line = None
    if not args.no_cpu_baseline and not args.data_sensitivity:
        cpu_line = cpu_baseline(w, t, args.cpu_heads or None)
        if not args.no_fp8:
            fp8_cpu_line = fp8_cpu_baseline(w, t)
        print(f"# cpu baseline done in {cpu_line['seconds']:.1f}s", file=sys.stderr, flush=True)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to_dev(t.q), to_dev(t.k), to_dev(t.v)
    do = to_dev(t.do) if not w.fwd_only else None
    mask = torch.from_numpy(t.block_mask).to(dev) if t.block_mask is not None else None
    print(f"# inputs ready in {time.perf_counter() - t_gen:.1f}s: {w.description}", file=sys.stderr, flush=True)
    if args.data_sensitivity:
        print(data_sensitivity(dev, w, q, k, v), flush=True)
        return
    B, H, N, d = w.B, w.H, w.N, w.d
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if not w.fwd_only:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = fa.new_workspace(B, H, N, d, dev)

    names = ["fwd"] if w.fwd_only else ["fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq"]

    def step(ev):
        # torch.cuda.Event records on torch's current stream, which is the stream every call below
        # hands to the library, so each pair of events brackets exactly one kernel launch
        if ev:
            ev[0].record()
        fa.fwd(q, k, v, w.scale, w.causal, mask, out=o, lse=lse)
        if ev:
            ev[1].record()
        if w.fwd_only:
            return
        fa.bwd_preprocess(q, o, do, ws)
        if ev:
            ev[2].record()
        fa.bwd_dkdv(q, k, v, do, lse, ws, w.scale, w.causal, mask, dk, dv)
        if ev:
            ev[3].record()
        fa.bwd_dq(q, k, v, do, lse, ws, w.scale, w.causal, mask, dq)
        if ev:
            ev[4].record()

    for _ in range(args.warmup):
        step(None)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1000.0 / args.steps
    kern_ms = {n: sum(e[j].elapsed_time(e[j + 1]) for e in events) / args.steps for j, n in enumerate(names)}
    kern_pct = {n: percentiles([e[j].elapsed_time(e[j + 1]) for e in events]) for j, n in enumerate(names)}
    gpu_ms = sum(kern_ms.values())

    ff = workloads.flops_fwd(B, H, N, d, w.causal, t.block_mask)
    fb = 0.0 if w.fwd_only else 2.5 * ff
    value = (ff + fb) / (ms_per_step * 1e-3) / 1e12
    kf = kernel_flops(w, t.block_mask)
    kernels = {}
    for n in names:
        ms = kern_ms[n]
        if n == "bwd_preprocess":
            kernels[n] = {"ms": ms, "GB/s": preprocess_bytes(w) / (ms * 1e-3) / 1e9}
        else:
            tf = kf[n] / (ms * 1e-3) / 1e12
            kernels[n] = {"ms": ms, "TFLOP/s": tf, "frac_of_peak": tf / PEAK_BF16_TFLOPS}
        kernels[n].update(kern_pct[n])
    dom = max(names, key=lambda n: kern_ms[n])
    if dom == "bwd_preprocess":
        ach = preprocess_bytes(w) / (kern_ms[dom] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS, "traffic": traffic_for(dom, w.name)}
    else:
        ach = kf[dom] / (kern_ms[dom] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_BF16_TFLOPS, "traffic": traffic_for(dom, w.name)}
    fwd_tf = ff / (kern_ms["fwd"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.description, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "block_sparse": w.sparse, "pass": "forward" if w.fwd_only else "forward+backward"},
        "frac_of_peak": value / PEAK_BF16_TFLOPS,
        "fwd_TFLOP/s": fwd_tf,
        "fwd_frac_of_peak": fwd_tf / PEAK_BF16_TFLOPS,
        "bwd_TFLOP/s": (fb / (sum(kern_ms[n] for n in names[1:]) * 1e-3) / 1e12) if not w.fwd_only else None,
        "gpu_ms_per_step": gpu_ms,
        "kernels": kernels,
        "roofline": roof,
    }
    if w.causal and mask is None:
        # the same shape without the causal mask (a figure beside the metric, not part of it)
        fnc = workloads.flops_fwd(B, H, N, d, False, None)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for _ in range(2):
            fa.fwd(q, k, v, w.scale, False, None, out=o, lse=lse)
        torch.cuda.synchronize()
        e[0].record()
        for _ in range(max(3, args.steps // 2)):
            fa.fwd(q, k, v, w.scale, False, None, out=o, lse=lse)
        e[1].record()
        torch.cuda.synchronize()
        ms_nc = e[0].elapsed_time(e[1]) / max(3, args.steps // 2)
        tf_nc = fnc / (ms_nc * 1e-3) / 1e12
        line["fwd_noncausal"] = {"ms": ms_nc, "TFLOP/s": tf_nc, "frac_of_peak": tf_nc / PEAK_BF16_TFLOPS}
    if d == 128 and mask is None:
        # the wave-specialised schedule beside the in-wave interleave of the metric's forward: both
        # timed the same way (back-to-back calls between one event pair), alternating, same inputs
        n_pp = max(5, args.steps)
        def back_to_back(fn):
            for _ in range(2):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(n_pp):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n_pp
        pp, il = [], []
        for _ in range(2):
            pp.append(back_to_back(lambda: fa.fwd_pingpong(q, k, v, w.scale, w.causal, out=o, lse=lse)))
            il.append(back_to_back(lambda: fa.fwd(q, k, v, w.scale, w.causal, None, out=o, lse=lse)))
        pp_ms, il_ms = min(pp), min(il)
        line["pingpong_forward"] = {"ms": pp_ms, "TFLOP/s": ff / (pp_ms * 1e-3) / 1e12,
                                    "frac_of_peak": ff / (pp_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                    "interleave_ms": il_ms, "interleave_TFLOP/s": ff / (il_ms * 1e-3) / 1e12,
                                    "pingpong_over_interleave_time": pp_ms / il_ms,
                                    "schedule": "waves w and w+4 of each SIMD alternate matrix and softmax phases"}
    if args.workload == "long" and not args.no_other_workloads:
        # the other bf16 workloads (d = 64), each timed kernel by kernel the same way
        line["other_workloads"] = {n: time_workload(fa, workloads.WORKLOADS[n], dev, max(5, args.steps // 2), 2)
                                   for n in OTHER_WORKLOADS}
    if not args.no_gemm:
        # the vendor library's bf16 GEMM on N(0,1) inputs in the same process: what the matrix
        # cores sustain on this part under Gaussian data (context for the fractions above)
        line["library_gemm"] = library_gemm(dev)
    if not args.no_fp8:
        line["mxfp8_forward"] = fp8_forward(fa, w, q, k, v, mask, ff, max(3, args.steps))
        if fp8_cpu_line:
            line["mxfp8_forward"]["cpu_baseline"] = fp8_cpu_line
    if cpu_line:
        line["cpu_baseline"] = cpu_line
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
