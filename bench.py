"""W4A16 GEMM throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload sweep|llama7b]

Default workload (the one the metric is quoted on): the large single layer
K = 18432, N = 73728 (the 72k x 18k layer of the MARLIN note's first figure),
group 128, at every batch size M = 1, 2, 4, 8, 16, 32, 64, 128.  One step runs
the eight GEMMs once.  Inputs are seeded synthetic data (A ~ N(0,1) in FP16,
uniform codes, FP16 scales uniform on [0.005, 0.02]), resident in HBM before
timing starts.  Weights, scales and activations exist in several copies and
the copy a launch reads rotates, so that no launch finds its operands in the
256 MB Infinity Cache from an earlier one.

Warmup runs the W steps asked for and continues until at least half a
second of steps has run (the GPU's clocks ramp up from idle).  Then five
timed regions of exactly K steps each, synchronised on both sides; the
median is ``value`` (all five are listed).  The Llama-2-7B layer step (four
layers at M = 1, 16, 128) is timed the same way and reported under
``secondary``.

Prints one JSON line: whole-step TFLOP/s (the metric), achieved HBM TB/s,
per-GEMM times, the roofline object of the dominant kernel (per-launch
durations from HIP events around back-to-back batches of each GEMM on the
launch stream), measured ceilings (a plain 2 GiB read and an FP16
matrix-instruction loop, libw4a16_probes.so) beside the published peaks,
the clocks under load (rocm-smi) and the CPU oracle timed on the host on a
bounded slice of the same workload.

Counter-based HBM traffic (``roofline.traffic``) comes from two rocprofv3
counter runs of this script, summarised into profiles/ by
``--pmc-summary``; it is reported only while the kernel sources still hash
to the value recorded with the counters:

    rocprofv3 --pmc FETCH_SIZE -d OUT/fetch -o run -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-graph --no-secondary --no-probes --no-clocks --copy-probe
    rocprofv3 --pmc WRITE_SIZE -d OUT/write -o run -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-graph --no-secondary --no-probes --no-clocks --copy-probe
    python3 bench.py --pmc-summary OUT/fetch OUT/write profiles/pmc_traffic_large_layer_sweep.json

The kernel durations come from a trace of the same workload, summarised by
``--trace-summary``:

    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/kt -o run -- python3 bench.py --steps 10 --warmup 2 --no-cpu-baseline --no-graph --no-secondary --no-probes --no-clocks
    python3 bench.py --trace-summary OUT/kt/run_kernel_stats.csv profiles/kernel_trace_large_layer_sweep.md

``--configs-report OUT.md`` instead times every workload shape one GEMM at a
time (the single 4096 x 4096 layer, the Llama-2-7B layers, the 18432 x 73728
batch sweep, the 8192 x 28672 prefill layer and the deep-K layers with group
128 and group K) and writes a table of time, TFLOP/s, HBM TB/s and roofline
fraction per call, with the 2:4-sparse GEMM on the same codes beside it.
``--single M K N [--sparse24]`` times one GEMM and prints one JSON line: the
short program for counter runs, summarised by ``--pmc-kernels OUT DIR...``
(MFMA utilisation, HBM bytes per dispatch).
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sqlite3
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

LAYERS = [("qkv", 4096, 12288), ("o", 4096, 4096), ("gate_up", 4096, 22016),
          ("down", 11008, 4096)]
BATCHES = [1, 16, 128]
GROUP = 128
WEIGHT_COPIES = 8   # 8 x 101 MB of packed weights: far beyond the 256 MB MALL
COPY_PROBE_BYTES = 512 * 2**20   # one-dispatch device copy of known size, counter calibration
COPY_PROBE_RUNS = 4
SIMDS = 256 * 4                 # MI355X: 256 compute units of four SIMDs
XCDS = 8                        # accelerator complex dies
WARMUP_MIN_S = 0.5   # untimed steps run at least this long before timing
REPEATS = 5          # timed regions of exactly --steps steps; the median is reported
PROBE_READ_BYTES = 2 * 2**30    # the stream-read ceiling: a 2 GiB buffer read once per launch
PROBE_MFMA_ITERS = 2048
PROBE_MFMA_BLOCKS = 1024         # four waves per SIMD
# the kernel-trace run behind profiles/kernel_trace_large_layer_sweep.md
TRACE_RUN_FLAGS = ("--steps 10 --warmup 2 --no-cpu-baseline --no-graph --no-secondary --no-probes "
                   "--no-clocks")
# the counter runs behind roofline.traffic (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)
PMC_RUN_FLAGS = ("--steps 2 --warmup 1 --no-cpu-baseline --no-graph --no-secondary --no-probes "
                 "--no-clocks --copy-probe")

# The workloads.  "sweep" is the one the metric is quoted on: the large
# single layer at every batch size from 1 to 128.
WORKLOADS = {
    "sweep": {
        "layers": [("large", 18432, 73728)],
        "batches": [1, 2, 4, 8, 16, 32, 64, 128],
        "copies": 2,     # 2 x 680 MB of packed weights
        "workload": "Large single W4A16 layer K=18432, N=73728 (the 72k x 18k layer), group "
                    "128, batch sweep M in {1,2,4,8,16,32,64,128}; one step = the 8 GEMMs",
        "traffic": os.path.join(ROOT, "profiles", "pmc_traffic_large_layer_sweep.json"),
    },
    "llama7b": {
        "layers": LAYERS,
        "batches": BATCHES,
        "copies": WEIGHT_COPIES,
        "workload": "Llama-2-7B-shaped W4A16 linear layers (qkv 4096x12288, o 4096x4096, "
                    "gate/up 4096x22016, down 11008x4096), group 128, M in {1,16,128}; "
                    "one step = the 12 GEMMs",
        "traffic": os.path.join(ROOT, "profiles", "pmc_traffic_llama7b_step.json"),
    },
}

# Every workload shape, for --configs-report: (label, K, N, group, batch sizes).
REPORT_SHAPES = [
    ("single layer 4096x4096", 4096, 4096, 128, [16]),
    ("Llama-2-7B qkv", 4096, 12288, 128, [1, 16, 128]),
    ("Llama-2-7B o", 4096, 4096, 128, [1, 16, 128]),
    ("Llama-2-7B gate/up", 4096, 22016, 128, [1, 16, 128]),
    ("Llama-2-7B down", 11008, 4096, 128, [1, 16, 128]),
    ("large layer 18432x73728", 18432, 73728, 128, [1, 2, 4, 8, 16, 32, 64, 128]),
    ("prefill 8192x28672", 8192, 28672, 128, [512, 1024, 4096]),
    ("deep K 28672x8192, group 128", 28672, 8192, 128, [1, 8, 32]),
    ("deep K 28672x8192, group K", 28672, 8192, 28672, [1, 8, 32]),
    ("deep K 13824x5120, group 128", 13824, 5120, 128, [1, 8, 32]),
    ("deep K 13824x5120, group K", 13824, 5120, 13824, [1, 8, 32]),
]
ROTATE_BYTES = 512 * 10**6   # weight copies cycled per shape: beyond the 256 MB MALL


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="sweep",
                    help="the workload of the headline line (default: the large-layer "
                         "batch sweep the metric is quoted on)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other workload (reported under 'secondary')")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the stream-read and MFMA-loop ceiling probes")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip the rocm-smi clock readout under load")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step (profiler runs)")
    ap.add_argument("--cpu-sample-cols", type=int, default=12288,
                    help="output columns per layer for the CPU oracle (0 = whole layers)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, run a one-dispatch elementwise copy (negation) "
                         "of 512 MiB a few times: calibrates the HBM byte counters")
    ap.add_argument("--configs-report", metavar="OUT",
                    help="time every workload shape, one GEMM at a time, write a "
                         "markdown table to OUT and exit")
    ap.add_argument("--epilogue-report", metavar="OUT",
                    help="time the fused output stage (bias + SiLU inside the GEMM) "
                         "against the plain GEMM and against the plain GEMM followed by "
                         "torch's bias add and SiLU, write a markdown table to OUT and exit")
    ap.add_argument("--formats-report", metavar="OUT",
                    help="time the weight formats (FP16, FP16 with zero points, BF16, BF16 "
                         "with zero points, 8-bit weights) side by side, write a markdown "
                         "table to OUT and exit")
    ap.add_argument("--single", nargs=3, type=int, metavar=("M", "K", "N"),
                    help="time one GEMM shape (group 128) with rotating weight copies, "
                         "print one JSON line and exit: a short program for counter runs")
    ap.add_argument("--sparse24", action="store_true",
                    help="with --single: the 2:4-sparse GEMM on the same codes")
    ap.add_argument("--pmc-kernels", nargs="+", metavar=("OUT", "DIR"),
                    help="summarise rocprofv3 --pmc runs (one DIR each) into OUT (JSON): "
                         "per GEMM kernel and counter, the value per dispatch")
    ap.add_argument("--trace-summary", nargs=2, metavar=("STATS_CSV", "OUT"),
                    help="write a rocprofv3 kernel-stats table as markdown")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) "
                         "of this script into a traffic file and exit")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of the HIP sources: counter figures are valid for this code only."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_only_int4_gemm_amd", "csrc")
    for path in sorted(glob.glob(os.path.join(csrc, "*.hip")) +
                       glob.glob(os.path.join(csrc, "*.hpp"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short_kernel_name(name: str) -> str:
    """Kernel name as w4a16_describe() prints it, e.g. 'gemm_tile_kernel<8,2,2>',
    from a demangled ('void w4a16::gemm_tile_kernel<8, 2, 2>(...)') or mangled
    ('_ZN5w4a1616gemm_tile_kernelILi8ELi2ELi2EEEv...') profiler name."""
    import re
    if name.startswith("_ZN"):
        # length-prefixed name segments, then I <template args> E
        i, seg = 3, ""
        while i < len(name) and name[i].isdigit():
            j = i
            while name[j].isdigit():
                j += 1
            n = int(name[i:j])
            seg, i = name[j:j + n], j + n
        if name[i:i + 1] == "I":
            end = name.find("EE", i)
            targs = name[i:end + 2]
            # the plan's integer arguments come before the first bool (the
            # fused-epilogue switch); the weight format after it is not part
            # of the plan's name
            if "Lb" in targs:
                targs = targs[:targs.index("Lb")]
            args = re.findall(r"Li(-?\d+)E", targs)
            return f"{seg}<{','.join(args)}>"
        return seg
    base = name.split("(")[0].replace("void ", "").strip()
    head, lt, rest = base.partition("<")
    # the fused-epilogue switch (a bool) and the weight format after it are
    # not part of the plan's name
    rest = rest.replace(" ", "")
    for flag in (",false", ",true"):
        if flag in rest:
            rest = rest[:rest.index(flag)] + ">"
    return head.split("::")[-1] + lt + rest


def _pmc_values(run_dir: str, counter: str):
    """{kernel name: [value per dispatch]} from a rocprofv3 database."""
    dbs = glob.glob(os.path.join(run_dir, "**", "*_results.db"), recursive=True)
    if not dbs:
        raise SystemExit(f"no rocprofv3 results database under {run_dir}")
    out = {}
    for db in dbs:
        con = sqlite3.connect(db)
        for kname, cname, value in con.execute(
                "select kernel_name, counter_name, value from counters_collection"):
            if cname == counter:
                out.setdefault(kname, []).append(float(value))
        con.close()
    return out


def pmc_summary(fetch_dir: str, write_dir: str, out_path: str, workload: str = "sweep") -> None:
    fetch = _pmc_values(fetch_dir, "FETCH_SIZE")
    write = _pmc_values(write_dir, "WRITE_SIZE")

    def median(v):
        v = sorted(v)
        return v[len(v) // 2]

    # the calibration copy: the elementwise negation kernel of the probe
    copies = [(median(v), k) for k, v in fetch.items()
              if "neg" in k.lower() and len(v) >= COPY_PROBE_RUNS]
    if not copies:
        raise SystemExit("no copy-kernel dispatches found (run with --copy-probe)")
    copy_fetch_kib, copy_name = max(copies)
    copy_write_kib = median([x for x in write.get(copy_name, [0.0])])
    expect_kib = COPY_PROBE_BYTES / 1024
    fetch_scale = expect_kib / copy_fetch_kib if copy_fetch_kib else None
    write_scale = expect_kib / copy_write_kib if copy_write_kib else None
    kernels = {}
    for k, v in fetch.items():
        if "gemm" not in k:
            continue
        short = _short_kernel_name(k)
        f = sum(v) / len(v)
        w_list = write.get(k, [])
        w = sum(w_list) / len(w_list) if w_list else 0.0
        kernels[short] = {
            "dispatches": len(v),
            "fetch_kib_per_dispatch": f,
            "write_kib_per_dispatch": w,
            "hbm_bytes_per_dispatch": (f * (fetch_scale or 1) + w * (write_scale or 1)) * 1024,
        }
    wflag = "" if workload == "sweep" else f" --workload {workload}"
    summary = {
        "what": f"HBM bytes per dispatch of each GEMM kernel of bench.py's {workload} workload "
                f"({WORKLOADS[workload]['workload']}), from rocprofv3 FETCH_SIZE and WRITE_SIZE, "
                "each scaled by what the counter reads for a device copy of known size",
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE -d OUT/fetch -o run -- python3 bench.py{wflag} "
            f"{PMC_RUN_FLAGS}",
            f"rocprofv3 --pmc WRITE_SIZE -d OUT/write -o run -- python3 bench.py{wflag} "
            f"{PMC_RUN_FLAGS}",
            f"python3 bench.py{wflag} --pmc-summary OUT/fetch OUT/write "
            + os.path.relpath(out_path, ROOT),
        ],
        "kernel_source_hash": kernel_source_hash(),
        "copy_probe": {"kernel": copy_name, "bytes": COPY_PROBE_BYTES,
                       "fetch_kib": copy_fetch_kib, "write_kib": copy_write_kib,
                       "fetch_scale": fetch_scale, "write_scale": write_scale},
        "kernels": kernels,
    }
    with open(out_path, "w") as f:
        json.dump(summary, f, indent=1)
        f.write("\n")
    print(json.dumps(summary, indent=1))


def trace_summary(stats_csv: str, out_path: str, workload: str = "sweep") -> None:
    """A rocprofv3 --kernel-trace --stats kernel table as markdown: calls,
    average, min and max duration and share of GPU time per kernel."""
    import csv
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            rows.append((_short_kernel_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]),
                         float(r["MinNs"]), float(r["MaxNs"]), float(r["Percentage"])))
    rows.sort(key=lambda r: -r[1] * r[2])
    wl = WORKLOADS[workload]
    wflag = "" if workload == "sweep" else f" --workload {workload}"
    lines = [
        "# Kernel trace: bench.py " + ("default workload" if workload == "sweep"
                                       else f"{workload} workload"),
        "",
        f"Workload: {wl['workload']}.",
        "",
        "Command (from the repository root on the GPU box; `OUT` a scratch directory), then the "
        "summary:",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
        f"-d OUT/kt -o run -- python3 $REPO/bench.py{wflag} {TRACE_RUN_FLAGS}",
        f"python3 bench.py{wflag} --trace-summary OUT/kt/run_kernel_stats.csv "
        + os.path.relpath(out_path, ROOT),
        "```",
        "",
        "The calls are the warm-up steps (at least half a second of them), five timed regions of "
        "10 steps, then each GEMM launched back to back between two HIP events (bench.py's "
        "per-launch durations).  The averages are the kernels' own durations and should agree "
        "with bench.py's `roofline.avg_launch_us` for the dominant kernel.",
        "",
        f"Kernel source hash (bench.py `kernel_source_hash`): `{kernel_source_hash()}`",
        "",
        "| kernel | calls | average us | min us | max us | share of GPU time |",
        "|---|---|---|---|---|---|",
    ]
    for name, calls, avg, mn, mx, pct in rows:
        lines.append(f"| `{name}` | {calls} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} "
                     f"| {pct:.1f}% |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def pmc_kernels(out_path: str, run_dirs) -> None:
    """Per GEMM kernel and counter of each rocprofv3 --pmc run: the value per
    dispatch (rows of one dispatch summed; and their maximum), averaged over
    dispatches.  rocprofv3 stores one value per dispatch, already summed over
    the counter's instances.  MFMA utilisation as rocprofv3's own derived
    MfmaUtil defines it: SQ_VALU_MFMA_BUSY_CYCLES summed over SIMDs, over
    (GRBM_GUI_ACTIVE of one XCD times the SIMD count); GRBM_GUI_ACTIVE comes
    summed over the eight XCDs, which are active over the same span, so one
    XCD's value is that sum over eight."""
    out = {"commands": "rocprofv3 --pmc <counters> -d DIR -o run -- python3 bench.py "
                       "--single M K N [--sparse24]; python3 bench.py --pmc-kernels OUT DIR...",
           "kernel_source_hash": kernel_source_hash(), "runs": {}}
    for d in run_dirs:
        dbs = glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True)
        if not dbs:
            raise SystemExit(f"no rocprofv3 results database under {d}")
        per = {}
        cols = None
        for db in dbs:
            con = sqlite3.connect(db)
            cur = con.execute("select * from counters_collection")
            cols = [c[0] for c in cur.description]
            disp = next((c for c in cols if "dispatch" in c.lower() and "id" in c.lower()), None)
            for row in cur:
                r = dict(zip(cols, row))
                k = _short_kernel_name(str(r["kernel_name"]))
                if "gemm" not in k:
                    continue
                key = (db, r[disp]) if disp else (db, id(row))
                per.setdefault(k, {}).setdefault(r["counter_name"], {}).setdefault(
                    key, []).append(float(r["value"]))
            con.close()
        kern = {}
        for k, ctrs in per.items():
            entry = {}
            for c, bydisp in ctrs.items():
                vals = list(bydisp.values())
                entry[c] = {"dispatches": len(vals),
                            "sum_per_dispatch": sum(sum(v) for v in vals) / len(vals),
                            "max_per_dispatch": sum(max(v) for v in vals) / len(vals),
                            "rows_per_dispatch": sum(len(v) for v in vals) / len(vals)}
            if "SQ_VALU_MFMA_BUSY_CYCLES" in entry and "GRBM_GUI_ACTIVE" in entry:
                gui_one_xcd = entry["GRBM_GUI_ACTIVE"]["sum_per_dispatch"] / XCDS
                entry["mfma_util_percent"] = (100 * entry["SQ_VALU_MFMA_BUSY_CYCLES"]["sum_per_dispatch"]
                                              / (gui_one_xcd * SIMDS))
            if "MfmaUtil" in entry:
                entry["mfma_util_percent_rocprof"] = entry["MfmaUtil"]["sum_per_dispatch"]
            kern[k] = entry
        out["runs"][os.path.basename(os.path.normpath(d))] = {"columns": cols, "kernels": kern}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


def measured_traffic(kernel: str, path: str):
    """Counter-measured HBM bytes per launch of `kernel`, or None when there
    is no summary or the kernel sources changed since it was taken."""
    try:
        with open(path) as f:
            summ = json.load(f)
    except (OSError, ValueError):
        return None
    if summ.get("kernel_source_hash") != kernel_source_hash():
        return None
    entry = summ.get("kernels", {}).get(kernel)
    return None if entry is None else entry["hbm_bytes_per_dispatch"]


def measured_ceilings(torch, dev):
    """What this chip sustains (libw4a16_probes.so), beside the published
    peaks: a plain read of a 2 GiB buffer with 16-byte non-temporal loads,
    and independent FP16 matrix instructions on register operands in every
    wave of a full grid.  Median of five timed launches each."""
    import ctypes
    import numpy as np
    from weight_only_int4_gemm_amd import roofline
    path = os.path.join(ROOT, "weight_only_int4_gemm_amd", "libw4a16_probes.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.w4a16_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_void_p]
    lib.w4a16_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    lib.w4a16_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.w4a16_probe_mfma_flops.restype = ctypes.c_double
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    buf = torch.ones(PROBE_READ_BYTES // 4, dtype=torch.int32, device=dev)

    def timed(launch, reps=5):
        launch()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return float(np.median(ts))

    # Short-lived workgroups read fastest in this grid-stride form (one box,
    # 2 GiB: 6.2 TB/s with 1024 or 2048 workgroups of 512, 6.6 with 4096,
    # 7.0 with 8192): 8192 of them, four rounds of eight loads per thread.
    read_blocks = 256 * 32
    t_read = timed(lambda: lib.w4a16_probe_read(buf.data_ptr(), PROBE_READ_BYTES,
                                                sink.data_ptr(), read_blocks, sh))
    del buf
    mfma_blocks = PROBE_MFMA_BLOCKS
    t_mfma = timed(lambda: lib.w4a16_probe_mfma(sink.data_ptr(), mfma_blocks, PROBE_MFMA_ITERS,
                                                sh))
    flops = lib.w4a16_probe_mfma_flops(mfma_blocks, PROBE_MFMA_ITERS)
    read_gbps = PROBE_READ_BYTES / t_read / 1e9
    mfma_tflops = flops / t_mfma / 1e12
    return {
        "hbm_read_gbps": read_gbps,
        "hbm_read_frac_of_peak": read_gbps / (roofline.HBM_PEAK_BYTES_PER_S / 1e9),
        "mfma_f16_tflops": mfma_tflops,
        "mfma_frac_of_peak": mfma_tflops / (roofline.MFMA_F16_PEAK_FLOPS / 1e12),
        "probe": "2 GiB read once with 16-byte non-temporal loads (8192 workgroups of 512); "
                 f"{PROBE_MFMA_ITERS} rounds of 16 independent v_mfma_f32_16x16x32_f16 per wave, "
                 f"{PROBE_MFMA_BLOCKS} workgroups of 4 waves; median of 5 launches each",
    }


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, sample_cols: int):
    """The oracle, as it stands, on this host: every GEMM of one step of the
    workload on the first ``sample_cols`` output columns of each layer (full
    K, every batch size; 0 = whole layers), timed call by call."""
    import numpy as np
    import oracle
    from synth import make_inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    total_flops = 0
    t_total = 0.0
    for name, K, N in wl["layers"]:
        cols = N if sample_cols <= 0 else min(N, sample_cols)
        _, Bq, S = make_inputs(1, K, cols, GROUP, seed=0)
        for M in wl["batches"]:
            A, _, _ = make_inputs(M, K, 8, GROUP, seed=M)
            t0 = time.perf_counter()
            oracle.gemm(A, Bq, S, GROUP)
            t_total += time.perf_counter() - t0
            total_flops += 2 * M * K * cols
    what = "every GEMM of one step" if sample_cols <= 0 else \
        f"every GEMM of one step on the first {sample_cols} output columns of each layer " \
        f"(full K, all {len(wl['batches'])} batch sizes)"
    return {
        "value": total_flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{what}; float64 accumulation, numpy; {t_total:.1f} s",
        "cpu_model": _cpu_model(),
        "logical_cpus": os.cpu_count(),
    }


def _time_calls(calls, launches: int, repeats: int) -> float:
    """Median over ``repeats`` of the mean time of ``launches`` back-to-back
    calls (cycling over ``calls``), from HIP events on the current stream."""
    import numpy as np
    import torch
    # the same calls for at least 0.2 s first: the host work that prepares a
    # shape's inputs leaves the GPU idle long enough for its clocks to drop
    t0 = time.perf_counter()
    i = 0
    while i < max(5, len(calls)) or time.perf_counter() - t0 < 0.2:
        calls[i % len(calls)]()
        i += 1
        if i % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    times = []
    for _ in range(repeats):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(launches):
            calls[i % len(calls)]()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3 / launches)
    return float(np.median(times))


def _warm_clocks(seconds: float = 1.0) -> None:
    """Keep the GPU busy for ``seconds`` so its clocks leave the idle state
    before anything is timed."""
    import torch
    x = torch.randn(4096, 4096, device="cuda", dtype=torch.float16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            torch.matmul(x, x)
        torch.cuda.synchronize()


def _gpu_clocks() -> str:
    """The current clocks as rocm-smi reports them (empty if unavailable)."""
    import subprocess
    try:
        out = subprocess.run(["rocm-smi", "--showclocks"], stdout=subprocess.PIPE,
                             stderr=subprocess.STDOUT, text=True, timeout=30).stdout
    except (OSError, subprocess.SubprocessError):
        return ""
    keep = [l.strip() for l in out.splitlines() if "sclk" in l or "mclk" in l or "fclk" in l]
    return "; ".join(keep)


def configs_report(out_path: str, repeats: int = 3, launches: int = 20) -> None:
    """Time each workload shape one GEMM at a time: hipEvents around
    ``launches`` back-to-back calls that cycle over enough copies of the
    packed weights to exceed the Infinity Cache, median of ``repeats``.
    Next to it, an FP16 GEMM (torch.matmul, i.e. hipBLASLt) on the same
    weights dequantised to FP16, the comparison the pages make."""
    import numpy as np
    import torch

    import weight_only_int4_gemm_amd as w4
    from weight_only_int4_gemm_amd import roofline
    from synth import make_activations, make_inputs, make_mask24

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = w4.load()
    sh = torch.cuda.current_stream().cuda_stream
    _warm_clocks()
    clocks_before = _gpu_clocks()
    rows = []
    for label, K, N, group, batches in REPORT_SHAPES:
        _, Bq, S = make_inputs(1, K, N, group, seed=0)
        Bq_d = torch.from_numpy(Bq.view(np.int32)).to(dev)
        first = w4.alloc_packed(K, N)
        w4.w4a16_repack(Bq_d, first, K, N)
        # the same codes under a two-of-four mask, for the 2:4-sparse column
        sfirst = w4.alloc_packed_sparse24(K, N)
        w4.w4a16_sparse24_repack(Bq_d, torch.from_numpy(make_mask24(K, N, seed=1)).to(dev),
                                 sfirst, K, N)
        nsp = max(1, -(-ROTATE_BYTES // (K * N * 3 // 8)))
        scopies = [sfirst] + [sfirst.clone() for _ in range(nsp - 1)]
        del Bq_d, Bq
        ncopy = max(1, -(-ROTATE_BYTES // (K * N // 2)))
        copies = [first] + [first.clone() for _ in range(ncopy - 1)]
        S_d = torch.from_numpy(S).to(dev)
        # the same weights as FP16 for the comparison, with their own rotation
        W = torch.empty((K, N), dtype=torch.float16, device=dev)
        w4.w4a16_dequant_debug(first, S_d, W, K, N, group)
        nw = max(1, -(-ROTATE_BYTES // (K * N * 2)))
        wcopies = [W] + [W.clone() for _ in range(nw - 1)]
        for M in batches:
            A_d = torch.from_numpy(make_activations(M, K, seed=M)).to(dev)
            C_d = torch.empty((M, N), dtype=torch.float16, device=dev)
            ws = torch.zeros(max(w4.w4a16_workspace_bytes(M, K, N, group),
                                 w4.w4a16_sparse24_workspace_bytes(M, K, N, group), 256),
                             dtype=torch.uint8, device=dev)

            def sparse_call(c):
                args = (A_d.data_ptr(), c.data_ptr(), S_d.data_ptr(), C_d.data_ptr(), M, K, N,
                        group, ws.data_ptr(), sh)

                def run():
                    rc = lib.w4a16_sparse24_gemm(*args)
                    if rc != 0:
                        raise RuntimeError(
                            f"w4a16_sparse24_gemm failed: {w4.w4a16_status_string(rc)}")
                return run

            def gemm_call(c):
                args = (A_d.data_ptr(), c.data_ptr(), S_d.data_ptr(), C_d.data_ptr(), M, K, N,
                        group, ws.data_ptr(), sh)

                def run():
                    rc = lib.w4a16_gemm(*args)
                    if rc != 0:
                        raise RuntimeError(f"w4a16_gemm failed: {w4.w4a16_status_string(rc)}")
                return run

            t = _time_calls([gemm_call(c) for c in copies], launches, repeats)
            C16 = torch.empty((M, N), dtype=torch.float16, device=dev)
            t16 = _time_calls([(lambda w=w: torch.matmul(A_d, w, out=C16)) for w in wcopies],
                              launches, repeats)
            tsp = _time_calls([sparse_call(c) for c in scopies], launches, repeats)
            flops = roofline.flops(M, K, N)
            nbytes = roofline.algorithmic_bytes(M, K, N, group)
            # 2:4: three quarters of the code bytes, the rest unchanged
            sbytes = nbytes - K * N // 2 + K * N * 3 // 8
            rows.append(dict(shape=label, M=M, K=K, N=N, group=group, us=t * 1e6,
                             sp24_us=tsp * 1e6, sp24_tbps=sbytes / tsp / 1e12,
                             tflops=flops / t / 1e12, tbps=nbytes / t / 1e12,
                             bound=roofline.bound(M, K, N, group),
                             frac=roofline.roofline_seconds(M, K, N, group) / t,
                             fp16_us=t16 * 1e6, speedup=t16 / t,
                             plan=w4.w4a16_describe(M, K, N, group).split(" workspace")[0]))
            print(json.dumps(rows[-1]), flush=True)
            del A_d, C_d, ws, C16
        del copies, first, S_d, W, wcopies, scopies, sfirst
        torch.cuda.empty_cache()
    clocks_after = _gpu_clocks()

    lines = [
        "# W4A16 GEMM on one MI355X: every workload shape",
        "",
        "Command (repository root, GPU box): `python3 bench.py --configs-report " +
        os.path.relpath(out_path, ROOT) + "`",
        "",
        f"Kernel source hash: `{kernel_source_hash()}`. Per call: hipEvents around "
        f"{launches} back-to-back launches cycling over enough copies of the packed weights "
        f"to exceed 512 MB (so weights come from HBM, not the Infinity Cache), median of "
        f"{repeats} repeats, after at least 0.2 s of the same calls; the time includes launch "
        "gaps. Inputs: seeded synthetic data "
        "(weights seed 0, activations seed M). Roofline: HBM 8 TB/s, dense FP16 MFMA "
        "2.5 PFLOP/s; `frac` is the bound's time over the measured time. `FP16 us` is "
        "torch.matmul (hipBLASLt) on the same weights dequantised to FP16, timed the same "
        "way with its own rotation of weight copies; `x FP16` is its time over ours. "
        "`2:4 us` is `w4a16_sparse24_gemm` on the same codes under a two-of-four mask (seed 1), "
        "with its own rotation and plan; `2:4 TB/s` counts its bytes (three quarters of the "
        "code bytes).",
        "",
        f"Clocks after a one-second warm-up, before the first shape (rocm-smi): "
        f"{clocks_before or 'n/a'}",
        "",
        f"Clocks after: {clocks_after or 'n/a'}",
        "",
        "| shape | M | us | TFLOP/s | HBM TB/s | bound | frac | FP16 us | x FP16 | 2:4 us | "
        "2:4 TB/s | plan |",
        "|---|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    for r in rows:
        lines.append(f"| {r['shape']} | {r['M']} | {r['us']:.1f} | {r['tflops']:.1f} | "
                     f"{r['tbps']:.2f} | {r['bound']} | {r['frac']:.3f} | {r['fp16_us']:.1f} | "
                     f"{r['speedup']:.2f} | {r['sp24_us']:.1f} | {r['sp24_tbps']:.2f} | "
                     f"`{r['plan']}` |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


# Shapes for --epilogue-report: (label, K, N, batch sizes).
EPILOGUE_SHAPES = [
    ("Llama-2-7B gate/up", 4096, 22016, [1, 16, 128]),
    ("Llama-2-7B qkv", 4096, 12288, [1, 128]),
    ("prefill 8192x28672", 8192, 28672, [1024]),
]


def epilogue_report(out_path: str, repeats: int = 7, launches: int = 50) -> None:
    """Per call, timed like --configs-report: the plain GEMM; the fused
    entry point with a bias and SiLU; and the plain GEMM followed by the same
    operation as two torch kernels (in-place bias add, in-place SiLU) -- the
    extra pass over C that fusing removes."""
    import numpy as np
    import torch
    import torch.nn.functional as F

    import weight_only_int4_gemm_amd as w4
    from synth import make_activations, make_bias, make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = w4.load()
    sh = torch.cuda.current_stream().cuda_stream
    _warm_clocks()
    rows = []
    for label, K, N, batches in EPILOGUE_SHAPES:
        _, Bq, S = make_inputs(1, K, N, GROUP, seed=0)
        Bq_d = torch.from_numpy(Bq.view(np.int32)).to(dev)
        first = w4.alloc_packed(K, N)
        w4.w4a16_repack(Bq_d, first, K, N)
        del Bq_d, Bq
        ncopy = max(1, -(-ROTATE_BYTES // (K * N // 2)))
        copies = [first] + [first.clone() for _ in range(ncopy - 1)]
        S_d = torch.from_numpy(S).to(dev)
        bias = torch.from_numpy(make_bias(N, seed=1)).to(dev)
        for M in batches:
            A_d = torch.from_numpy(make_activations(M, K, seed=M)).to(dev)
            C_d = torch.empty((M, N), dtype=torch.float16, device=dev)
            ws = torch.zeros(max(w4.w4a16_workspace_bytes(M, K, N, GROUP), 256),
                             dtype=torch.uint8, device=dev)

            def call(c, fused):
                if fused:
                    args = (A_d.data_ptr(), c.data_ptr(), S_d.data_ptr(), bias.data_ptr(),
                            w4.W4A16_ACT_SILU, C_d.data_ptr(), M, K, N, GROUP, ws.data_ptr(), sh)
                    fn = lib.w4a16_gemm_fused
                else:
                    args = (A_d.data_ptr(), c.data_ptr(), S_d.data_ptr(), C_d.data_ptr(), M, K,
                            N, GROUP, ws.data_ptr(), sh)
                    fn = lib.w4a16_gemm

                def run():
                    rc = fn(*args)
                    if rc != 0:
                        raise RuntimeError(f"gemm failed: {w4.w4a16_status_string(rc)}")
                return run

            plain = [call(c, False) for c in copies]

            def unfused(i):
                def run():
                    plain[i]()
                    C_d.add_(bias)
                    F.silu(C_d, inplace=True)
                return run

            # the three forms interleaved, repeat by repeat: the clock drifts
            # over a run by more than the differences measured here
            forms = [plain, [call(c, True) for c in copies],
                     [unfused(i) for i in range(len(copies))]]
            times = [[], [], []]
            for _ in range(repeats):
                for f, form in enumerate(forms):
                    times[f].append(_time_calls(form, launches, 1))
            t_plain, t_fused, t_unf = (float(np.median(t)) for t in times)
            rows.append(dict(shape=label, M=M, K=K, N=N, plain_us=t_plain * 1e6,
                             fused_us=t_fused * 1e6, unfused_us=t_unf * 1e6,
                             plan=w4.w4a16_describe(M, K, N, GROUP).split(" workspace")[0]))
            print(json.dumps(rows[-1]), flush=True)
            del A_d, C_d, ws
        del copies, first, S_d, bias
        torch.cuda.empty_cache()
    lines = [
        "# Fused output stage (bias + SiLU) on one MI355X",
        "",
        "Command (repository root, GPU box): `python3 bench.py --epilogue-report " +
        os.path.relpath(out_path, ROOT) + "`",
        "",
        f"Kernel source hash: `{kernel_source_hash()}`. Per form: hipEvents around "
        f"{launches} back-to-back calls cycling over weight copies beyond 512 MB; the three "
        f"forms are timed in turn, {repeats} rounds, median per form. `plain`: w4a16_gemm. `fused`: w4a16_gemm_fused with "
        "an FP16 bias and SiLU. `unfused`: w4a16_gemm, then torch's in-place bias add and "
        "in-place SiLU on C (two more kernels, two more passes over C).",
        "",
        "| shape | M | plain us | fused us | unfused us | fused - plain | unfused - fused | plan |",
        "|---|---|---|---|---|---|---|---|",
    ]
    for r in rows:
        lines.append(f"| {r['shape']} | {r['M']} | {r['plain_us']:.1f} | {r['fused_us']:.1f} | "
                     f"{r['unfused_us']:.1f} | {r['fused_us'] - r['plain_us']:+.1f} | "
                     f"{r['unfused_us'] - r['fused_us']:+.1f} | `{r['plan']}` |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


# Shapes for --formats-report: (label, K, N, batch sizes).
FORMAT_SHAPES = [
    ("Llama-2-7B qkv", 4096, 12288, [1, 16, 128]),
    ("Llama-2-7B gate/up", 4096, 22016, [1, 16, 128]),
    ("Llama-2-7B down", 11008, 4096, [1, 16, 128]),
    ("prefill 8192x28672", 8192, 28672, [1024]),
]
FORMATS = [("FP16", 0, False), ("FP16 + zero points", 0, True), ("BF16", 1, False),
           ("BF16 + zero points", 1, True), ("8-bit weights", None, False),
           ("2:4 sparse", "sp24", False)]


def formats_report(out_path: str, repeats: int = 7, launches: int = 50) -> None:
    """Per shape, the four weight formats through w4a16_gemm_awq, timed in
    turn (interleaved rounds, median), weight copies rotating beyond 512 MB."""
    import numpy as np
    import torch

    import weight_only_int4_gemm_amd as w4
    from weight_only_int4_gemm_amd import roofline
    from synth import make_inputs_awq, make_mask24, make_words

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = w4.load()
    sh = torch.cuda.current_stream().cuda_stream
    _warm_clocks()
    rows = []
    for label, K, N, batches in FORMAT_SHAPES:
        _, Bq, S16, Z = make_inputs_awq(1, K, N, GROUP, seed=0)
        _, _, Sb, _ = make_inputs_awq(1, K, N, GROUP, seed=0, bf16=True)
        Bq_d = torch.from_numpy(Bq.view(np.int32)).to(dev)
        first = w4.alloc_packed(K, N)
        w4.w4a16_repack(Bq_d, first, K, N)
        del Bq_d, Bq
        ncopy = max(1, -(-ROTATE_BYTES // (K * N // 2)))
        copies = [first] + [first.clone() for _ in range(ncopy - 1)]
        scales = {0: torch.from_numpy(S16.view(np.int16)).to(dev),
                  1: torch.from_numpy(Sb.view(np.int16)).to(dev)}
        zeros = torch.from_numpy(Z).to(dev)
        # 8-bit codes: uniform words [K/4][N], repacked, with their own rotation
        Bq8 = np.concatenate([make_words(K, N, 1), make_words(K, N, 2)])
        Bq8_d = torch.from_numpy(Bq8.view(np.int32)).to(dev)
        first8 = w4.alloc_packed8(K, N)
        w4.w8a16_repack(Bq8_d, first8, K, N)
        del Bq8_d, Bq8
        ncopy8 = max(1, -(-ROTATE_BYTES // (K * N)))
        copies8 = [first8] + [first8.clone() for _ in range(ncopy8 - 1)]
        # 2:4-sparse codes: the 4-bit words under a two-of-four mask
        _, Bqs, _, _ = make_inputs_awq(1, K, N, GROUP, seed=0)
        Bqs_d = torch.from_numpy(Bqs.view(np.int32)).to(dev)
        mask_d = torch.from_numpy(make_mask24(K, N, seed=1)).to(dev)
        firsts = w4.alloc_packed_sparse24(K, N)
        w4.w4a16_sparse24_repack(Bqs_d, mask_d, firsts, K, N)
        del Bqs_d, Bqs, mask_d
        ncopys = max(1, -(-ROTATE_BYTES // (K * N * 3 // 8)))
        copiess = [firsts] + [firsts.clone() for _ in range(ncopys - 1)]
        for M in batches:
            A16, _, _, _ = make_inputs_awq(M, K, 8, GROUP, seed=M)
            Ab, _, _, _ = make_inputs_awq(M, K, 8, GROUP, seed=M, bf16=True)
            acts = {0: torch.from_numpy(A16.view(np.int16)).to(dev),
                    1: torch.from_numpy(Ab.view(np.int16)).to(dev)}
            C_d = torch.empty((M, N), dtype=torch.int16, device=dev)
            ws = torch.zeros(max(w4.w4a16_workspace_bytes(M, K, N, GROUP),
                                 w4.w8a16_workspace_bytes(M, K, N, GROUP),
                                 w4.w4a16_sparse24_workspace_bytes(M, K, N, GROUP), 256),
                             dtype=torch.uint8, device=dev)

            def form(dtype, zp):
                if dtype == "sp24":     # 2:4-sparse weights, FP16 activations
                    def calls(c):
                        args = (acts[0].data_ptr(), c.data_ptr(), scales[0].data_ptr(),
                                C_d.data_ptr(), M, K, N, GROUP, ws.data_ptr(), sh)

                        def run():
                            rc = lib.w4a16_sparse24_gemm(*args)
                            if rc != 0:
                                raise RuntimeError(
                                    f"w4a16_sparse24_gemm: {w4.w4a16_status_string(rc)}")
                        return run
                    return [calls(c) for c in copiess]
                if dtype is None:       # 8-bit weights, FP16 activations
                    def call8(c):
                        args = (acts[0].data_ptr(), c.data_ptr(), scales[0].data_ptr(),
                                C_d.data_ptr(), M, K, N, GROUP, ws.data_ptr(), sh)

                        def run():
                            rc = lib.w8a16_gemm(*args)
                            if rc != 0:
                                raise RuntimeError(f"w8a16_gemm: {w4.w4a16_status_string(rc)}")
                        return run
                    return [call8(c) for c in copies8]

                def call(c):
                    args = (acts[dtype].data_ptr(), c.data_ptr(), scales[dtype].data_ptr(),
                            zeros.data_ptr() if zp else None, C_d.data_ptr(), M, K, N, GROUP,
                            dtype, ws.data_ptr(), sh)

                    def run():
                        rc = lib.w4a16_gemm_awq(*args)
                        if rc != 0:
                            raise RuntimeError(f"w4a16_gemm_awq: {w4.w4a16_status_string(rc)}")
                    return run
                return [call(c) for c in copies]

            forms = [form(dt, zp) for _, dt, zp in FORMATS]
            times = [[] for _ in forms]
            for _ in range(repeats):
                for f, calls in enumerate(forms):
                    times[f].append(_time_calls(calls, launches, 1))
            med = [float(np.median(t)) for t in times]
            flops = roofline.flops(M, K, N)
            rows.append(dict(shape=label, M=M, us=[t * 1e6 for t in med],
                             tflops=[flops / t / 1e12 for t in med],
                             plan=w4.w4a16_describe(M, K, N, GROUP).split(" workspace")[0],
                             plan_sp24=w4.w4a16_sparse24_describe(M, K, N, GROUP)
                             .split(" workspace")[0]))
            print(json.dumps(rows[-1]), flush=True)
            del acts, C_d, ws
        del copies, first, scales, zeros, copies8, first8, copiess, firsts
        torch.cuda.empty_cache()
    lines = [
        "# Weight formats on one MI355X: FP16, zero points, BF16, 8-bit weights, 2:4 sparsity",
        "",
        "Command (repository root, GPU box): `python3 bench.py --formats-report " +
        os.path.relpath(out_path, ROOT) + "`",
        "",
        f"Kernel source hash: `{kernel_source_hash()}`. Each format through `w4a16_gemm_awq` "
        f"(FP16 without zero points is the plain kernel) or `w8a16_gemm`, hipEvents around {launches} "
        f"back-to-back calls cycling over weight copies beyond 512 MB; the four formats are "
        f"timed in turn, {repeats} rounds, median per format (the formats interleaved). Zero points: uint8 per group "
        "and column (one more byte per 64 code bytes at group 128). 8-bit weights: "
        "`w8a16_gemm` (twice the code bytes of 4-bit). 2:4 sparse: `w4a16_sparse24_gemm` "
        "on the same codes under a two-of-four mask (three quarters of the 4-bit bytes, "
        "half the products; its own plan).",
        "",
        "| shape | M | " + " | ".join(f"{n} us" for n, _, _ in FORMATS) + " | plan | 2:4 plan |",
        "|---|---|" + "---|" * len(FORMATS) + "---|---|",
    ]
    for r in rows:
        lines.append(f"| {r['shape']} | {r['M']} | " +
                     " | ".join(f"{u:.1f}" for u in r["us"]) +
                     f" | `{r['plan']}` | `{r['plan_sp24']}` |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def single_gemm(M: int, K: int, N: int, sparse: bool = False, launches: int = 20,
                repeats: int = 3) -> None:
    """One GEMM shape, group 128: warm clocks, then ``repeats`` batches of
    ``launches`` back-to-back calls over weight copies beyond the Infinity
    Cache; prints the median time per call and the plan as one JSON line."""
    import numpy as np
    import torch

    import weight_only_int4_gemm_amd as w4
    from weight_only_int4_gemm_amd import roofline
    from synth import make_activations, make_inputs, make_mask24

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = w4.load()
    sh = torch.cuda.current_stream().cuda_stream
    _, Bq, S = make_inputs(1, K, N, GROUP, seed=0)
    Bq_d = torch.from_numpy(Bq.view(np.int32)).to(dev)
    if sparse:
        first = w4.alloc_packed_sparse24(K, N)
        w4.w4a16_sparse24_repack(Bq_d, torch.from_numpy(make_mask24(K, N, seed=1)).to(dev),
                                 first, K, N)
        wbytes = K * N * 3 // 8
        ws_bytes = w4.w4a16_sparse24_workspace_bytes(M, K, N, GROUP)
        fn, desc = lib.w4a16_sparse24_gemm, w4.w4a16_sparse24_describe(M, K, N, GROUP)
    else:
        first = w4.alloc_packed(K, N)
        w4.w4a16_repack(Bq_d, first, K, N)
        wbytes = K * N // 2
        ws_bytes = w4.w4a16_workspace_bytes(M, K, N, GROUP)
        fn, desc = lib.w4a16_gemm, w4.w4a16_describe(M, K, N, GROUP)
    del Bq_d
    copies = [first] + [first.clone() for _ in range(max(1, -(-ROTATE_BYTES // wbytes)) - 1)]
    S_d = torch.from_numpy(S).to(dev)
    A_d = torch.from_numpy(make_activations(M, K, seed=M)).to(dev)
    C_d = torch.empty((M, N), dtype=torch.float16, device=dev)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def call(c):
        args = (A_d.data_ptr(), c.data_ptr(), S_d.data_ptr(), C_d.data_ptr(), M, K, N, GROUP,
                ws.data_ptr(), sh)

        def run():
            rc = fn(*args)
            if rc != 0:
                raise RuntimeError(f"GEMM failed: {w4.w4a16_status_string(rc)}")
        return run

    _warm_clocks(0.5)
    t = _time_calls([call(c) for c in copies], launches, repeats)
    print(json.dumps(dict(M=M, K=K, N=N, group=GROUP, sparse24=sparse, us=t * 1e6,
                          tflops=roofline.flops(M, K, N) / t / 1e12, plan=desc,
                          calls=max(5, len(copies)) + launches * repeats)), flush=True)


def _build_workload(wl, dev, torch, w4, make_inputs, np):
    """Inputs of a workload, resident in HBM: per layer `copies` copies of
    the packed weights, the scales and every batch's activations (the copy a
    launch reads rotates, so no launch finds its operands in the 256 MB
    Infinity Cache from an earlier one), one output per GEMM, one workspace.
    Returns the GEMMs of a step in launch order, the C-call arguments of the
    first `copies` steps (the rotation repeats after that) and the plans."""
    layers, batches, copies = wl["layers"], wl["batches"], wl["copies"]
    packed, scales, acts = {}, {}, {}
    for name, K, N in layers:
        _, Bq, S = make_inputs(1, K, N, GROUP, seed=0)
        Bq_d = torch.from_numpy(Bq.view(np.int32)).to(dev)
        del Bq
        first = w4.alloc_packed(K, N)
        w4.w4a16_repack(Bq_d, first, K, N)
        del Bq_d
        packed[name] = [first] + [first.clone() for _ in range(copies - 1)]
        s0 = torch.from_numpy(S).to(dev)
        scales[name] = [s0] + [s0.clone() for _ in range(copies - 1)]
        for M in batches:
            A, _, _ = make_inputs(M, K, 8, GROUP, seed=M)
            a0 = torch.from_numpy(A).to(dev)
            acts[(name, M)] = [a0] + [a0.clone() for _ in range(copies - 1)]
    outs, ws_bytes = {}, 0
    for name, K, N in layers:
        for M in batches:
            outs[(name, M)] = torch.empty((M, N), dtype=torch.float16, device=dev)
            ws_bytes = max(ws_bytes, w4.w4a16_workspace_bytes(M, K, N, GROUP))
    workspace = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    gemms = [(name, K, N, M) for M in batches for (name, K, N) in layers]
    plans = {g: w4.w4a16_describe(g[3], g[1], g[2], GROUP) for g in gemms}
    uses = len(batches)   # uses of one layer per step

    def args_for(g, copy, stream_handle):
        name, K, N, M = g
        return (acts[(name, M)][copy].data_ptr(), packed[name][copy].data_ptr(),
                scales[name][copy].data_ptr(), outs[(name, M)].data_ptr(), M, K, N, GROUP,
                workspace.data_ptr(), stream_handle)

    # the t-th use of a layer over the run reads copy t % copies
    def calls(stream_handle):
        return [[args_for(g, (uses * s + batches.index(g[3])) % copies, stream_handle)
                 for g in gemms] for s in range(copies)]
    keep = (packed, scales, acts, outs, workspace)
    return gemms, calls, plans, keep


def _time_workload(wl, args, lib, torch, w4, roofline, stream, make_inputs, np, dev,
                   graph: bool):
    """Time one workload: warmup, then REPEATS timed regions of exactly
    args.steps steps each (synchronised on both sides; the median is the
    result), per-GEMM launch durations from HIP events on the launch stream,
    and optionally the same steps replayed from HIP graphs."""
    gemms, calls, plans, keep = _build_workload(wl, dev, torch, w4, make_inputs, np)
    copies = wl["copies"]
    sh = stream.cuda_stream
    calls_per_step = calls(sh)

    def run_step(s):
        for a in calls_per_step[s % copies]:
            rc = lib.w4a16_gemm(*a)
            if rc != 0:
                raise RuntimeError(f"w4a16_gemm failed: {w4.w4a16_status_string(rc)}")

    # Warmup: the W steps asked for, continued (untimed) until at least
    # WARMUP_MIN_S of back-to-back steps have run: from idle the GPU takes a
    # fraction of a second to reach its working clocks.
    t_w = time.perf_counter()
    warmup_run = 0
    while warmup_run < args.warmup or time.perf_counter() - t_w < WARMUP_MIN_S:
        run_step(warmup_run)
        warmup_run += 1
        if warmup_run % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # ---- timed regions: launches only, exactly args.steps steps each ----
    walls = []
    s_next = warmup_run
    for _ in range(REPEATS):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            run_step(s_next + s)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
        s_next += args.steps
    wall = sorted(walls)[len(walls) // 2]

    # Per-GEMM launch durations: each GEMM launched n_rep times back to back
    # (its copies rotating) between two HIP events on the launch stream;
    # duration per launch = span / n_rep.
    n_rep = max(args.steps, 2 * copies, 10)
    spans = {}
    torch.cuda.synchronize()
    for gi, g in enumerate(gemms):
        gcalls = [calls_per_step[s][gi] for s in range(copies)]
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(n_rep):
            rc = lib.w4a16_gemm(*gcalls[r % copies])
            if rc != 0:
                raise RuntimeError(f"w4a16_gemm failed: {w4.w4a16_status_string(rc)}")
        e1.record(stream)
        spans[g] = (e0, e1)
    torch.cuda.synchronize()
    launch_s = {g: e0.elapsed_time(e1) / n_rep / 1e3 for g, (e0, e1) in spans.items()}

    graph_wall = None
    if graph:
        # one graph per rotation step, captured once on a side stream
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        graphs = []
        cap_calls = calls(cap.cuda_stream)
        with torch.cuda.stream(cap):
            for s in range(copies):
                gph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gph, stream=cap):
                    for a in cap_calls[s]:
                        rc = lib.w4a16_gemm(*a)
                        if rc != 0:
                            raise RuntimeError(
                                f"w4a16_gemm failed: {w4.w4a16_status_string(rc)}")
                graphs.append(gph)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        n_warm = max(args.warmup, 2 * copies)
        for s in range(n_warm):
            graphs[s % copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            graphs[(n_warm + s) % copies].replay()
        torch.cuda.synchronize()
        graph_wall = time.perf_counter() - t0
        del graphs

    step_flops = sum(roofline.flops(M, K, N) for (_, K, N, M) in gemms)
    step_bytes = sum(roofline.algorithmic_bytes(M, K, N, GROUP) for (_, K, N, M) in gemms)
    step_roof_s = sum(roofline.roofline_seconds(M, K, N, GROUP) for (_, K, N, M) in gemms)
    per_gemm = []
    for g in gemms:
        name, K, N, M = g
        t = launch_s[g]
        per_gemm.append({
            "layer": name, "M": M, "K": K, "N": N, "us": round(t * 1e6, 2),
            "tflops": round(roofline.flops(M, K, N) / t / 1e12, 2),
            "tbps": round(roofline.algorithmic_bytes(M, K, N, GROUP) / t / 1e12, 3),
            "roofline_frac": round(roofline.roofline_seconds(M, K, N, GROUP) / t, 3),
            "bound": roofline.bound(M, K, N, GROUP), "plan": plans[g],
        })
    res = {
        "workload": wl["workload"],
        "value": step_flops / (wall / args.steps) / 1e12,
        "unit": "TFLOP/s",
        "ms_per_step": wall * 1e3 / args.steps,
        "repeat_ms_per_step": [round(w * 1e3 / args.steps, 4) for w in walls],
        "hbm_tbps": step_bytes / (wall / args.steps) / 1e12,
        "step_roofline_frac": step_roof_s / (wall / args.steps),
        "warmup_steps_run": warmup_run,
        "events_ms_per_step": sum(launch_s.values()) * 1e3,
        "graph": None if graph_wall is None else {
            "launch": f"one HIP graph per step ({len(gemms)} kernel nodes), replayed",
            "ms_per_step": graph_wall * 1e3 / args.steps,
            "value": step_flops / (graph_wall / args.steps) / 1e12, "unit": "TFLOP/s"},
        "per_gemm": per_gemm,
        "weight_copies": copies,
    }
    res["roofline"] = _dominant_roofline(gemms, plans, launch_s, roofline, wl["traffic"])
    res["_run_step"] = run_step
    res["_next_step"] = s_next
    res["_keep"] = keep
    return res


def _dominant_roofline(gemms, plans, launch_s, roofline, traffic_path):
    """The roofline object of the kernel variant with the most time in a
    step: algorithmic flops (MFMA-bound) or bytes (HBM-bound) per launch over
    its average launch duration."""
    by_kernel = {}
    for g in gemms:
        name, K, N, M = g
        kname = plans[g].split()[0]
        d = by_kernel.setdefault(kname, {"s": 0.0, "launches": 0, "bytes": 0, "flops": 0,
                                         "hbm": 0, "mfma": 0})
        d["s"] += launch_s[g]
        d["launches"] += 1
        d["bytes"] += roofline.algorithmic_bytes(M, K, N, GROUP)
        d["flops"] += roofline.flops(M, K, N)
        d[roofline.bound(M, K, N, GROUP)] += 1
    dom_name, dom = max(by_kernel.items(), key=lambda kv: kv[1]["s"])
    avg_s = dom["s"] / dom["launches"]
    if dom["hbm"] >= dom["mfma"]:
        achieved = dom["bytes"] / dom["launches"] / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved,
                "peak": roofline.HBM_PEAK_BYTES_PER_S / 1e9, "unit": "GB/s"}
    else:
        achieved = dom["flops"] / dom["launches"] / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved,
                "peak": roofline.MFMA_F16_PEAK_FLOPS / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom_name, traffic_path)
    roof["traffic_unit"] = "bytes per launch"
    roof["algorithmic_bytes"] = dom["bytes"] / dom["launches"]
    roof["algorithmic_flops"] = dom["flops"] / dom["launches"]
    roof["kernel"] = dom_name
    roof["avg_launch_us"] = avg_s * 1e6
    roof["launches_per_step"] = dom["launches"]
    return roof


def _clocks_under_load(run_step, first_step: int, torch, seconds: float = 2.0) -> str:
    """rocm-smi's clock readout taken while steps keep the GPU busy."""
    import subprocess
    import threading
    out = {}

    def read():
        out["clocks"] = _gpu_clocks()

    th = threading.Thread(target=read)
    t0 = time.perf_counter()
    th.start()
    s = first_step
    while th.is_alive() and time.perf_counter() - t0 < seconds + 30:
        run_step(s)
        s += 1
        if s % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    th.join()
    return out.get("clocks", "")


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, workload=args.workload)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary, workload=args.workload)
        return
    if args.pmc_kernels:
        pmc_kernels(args.pmc_kernels[0], args.pmc_kernels[1:])
        return
    if args.configs_report:
        configs_report(args.configs_report)
        return
    if args.epilogue_report:
        epilogue_report(args.epilogue_report)
        return
    if args.formats_report:
        formats_report(args.formats_report)
        return
    if args.single:
        single_gemm(*args.single, sparse=args.sparse24)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the W4A16 GEMM runs on a single device and "
              "this build has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import weight_only_int4_gemm_amd as w4
    from weight_only_int4_gemm_amd import roofline
    from synth import make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = w4.load()
    stream = torch.cuda.current_stream()

    primary = WORKLOADS[args.workload]
    res = _time_workload(primary, args, lib, torch, w4, roofline, stream, make_inputs, np, dev,
                         graph=not args.no_graph)
    clocks = "" if args.no_clocks else _clocks_under_load(res["_run_step"], res["_next_step"],
                                                          torch)
    del res["_run_step"], res["_next_step"], res["_keep"]
    torch.cuda.empty_cache()

    secondary = None
    if not args.no_secondary:
        other = WORKLOADS["llama7b" if args.workload == "sweep" else "sweep"]
        sec = _time_workload(other, args, lib, torch, w4, roofline, stream, make_inputs, np,
                             dev, graph=not args.no_graph)
        del sec["_run_step"], sec["_next_step"], sec["_keep"]
        torch.cuda.empty_cache()
        secondary = sec

    ceilings = None
    if not args.no_probes:
        ceilings = measured_ceilings(torch, dev)

    if args.copy_probe:
        # torch's elementwise negation: one dispatch that reads and writes
        # COPY_PROBE_BYTES each (a device-to-device memcpy is split into
        # many blit dispatches and cannot serve as the reference)
        n = COPY_PROBE_BYTES // 2
        src = torch.empty(n, dtype=torch.float16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(COPY_PROBE_RUNS):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(primary, args.cpu_sample_cols)

    line = {
        "metric": "W4A16 GEMM TFLOP/s + achieved HBM TB/s (% roofline) at M=1..128, 1 MI355X",
        "value": res["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": res["warmup_steps_run"],
        "ms_per_step": res["ms_per_step"],
        "repeats": REPEATS,
        "repeat_ms_per_step": res["repeat_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": primary["workload"],
            "group": GROUP, "batches": primary["batches"],
            "weight_copies": primary["copies"],
            "parallelism": "single GPU",
        },
        "hbm_tbps": res["hbm_tbps"],
        "step_roofline_frac": res["step_roofline_frac"],
        "events_ms_per_step": res["events_ms_per_step"],
        "graph": res["graph"],
        "roofline": res["roofline"],
        "ceilings": ceilings,
        "cpu_baseline": cpu,
        "per_gemm": res["per_gemm"],
        "secondary": secondary,
        "sclk": clocks,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
