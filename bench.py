"""W4A16 GEMM throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: the Llama-2-7B-shaped linear layers as W4A16 GEMMs (K x N =
4096 x 12288 fused qkv, 4096 x 4096 o, 4096 x 22016 fused gate/up,
11008 x 4096 down), group 128, at batch M = 1, 16 and 128.  One step runs
all twelve GEMMs once.  Inputs are seeded synthetic data (A ~ N(0,1) in
FP16, uniform codes, FP16 scales uniform on [0.005, 0.02]), resident in HBM
before timing starts.  Each of the twelve GEMMs of a step reads its own copy
of the layer's weights, and the copies rotate over steps, so that no weight
read is served by the 256 MB Infinity Cache from an earlier launch.

Prints one JSON line: whole-step TFLOP/s (the metric), achieved HBM TB/s,
the roofline object of the dominant kernel (measured with HIP events on the
launch stream over the timed region), and the CPU oracle timed on the host.
"""

from __future__ import annotations

import argparse
import json
import os
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-cols", type=int, default=0,
                    help="columns per GEMM for the CPU oracle (0 = whole GEMMs)")
    return ap.parse_args()


def cpu_baseline(sample_cols: int):
    """The oracle, as it stands, on this host: the step's twelve GEMMs (or the
    first ``sample_cols`` columns of each)."""
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
    for name, K, N in LAYERS:
        cols = N if sample_cols <= 0 else min(N, sample_cols)
        _, Bq, S = make_inputs(1, K, cols, GROUP, seed=0)
        for M in BATCHES:
            A, _, _ = make_inputs(M, K, 8, GROUP, seed=M)
            t0 = time.perf_counter()
            oracle.gemm(A, Bq, S, GROUP)
            t_total += time.perf_counter() - t0
            total_flops += 2 * M * K * cols
    what = "all twelve GEMMs of one step" if sample_cols <= 0 else \
        f"the first {sample_cols} output columns of each of the twelve GEMMs"
    return {
        "value": total_flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{what} (float64 accumulation, numpy), {t_total:.1f} s on "
                  f"{os.cpu_count()} logical CPUs",
    }


def main():
    args = parse()
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
    sh = stream.cuda_stream

    # ---- inputs, resident in HBM -------------------------------------------
    packed = {}     # layer -> list of WEIGHT_COPIES packed buffers
    scales = {}
    for name, K, N in LAYERS:
        _, Bq, S = make_inputs(1, K, N, GROUP, seed=0)
        Bq_d = torch.from_numpy(Bq.view(np.int32)).to(dev)
        first = w4.alloc_packed(K, N)
        w4.w4a16_repack(Bq_d, first, K, N)
        packed[name] = [first] + [first.clone() for _ in range(WEIGHT_COPIES - 1)]
        scales[name] = torch.from_numpy(S).to(dev)
        del Bq_d
    acts, outs = {}, {}
    ws_bytes = 0
    for name, K, N in LAYERS:
        for M in BATCHES:
            A, _, _ = make_inputs(M, K, 8, GROUP, seed=M)
            acts[(name, M)] = torch.from_numpy(A).to(dev)
            outs[(name, M)] = torch.empty((M, N), dtype=torch.float16, device=dev)
            ws_bytes = max(ws_bytes, w4.w4a16_workspace_bytes(M, K, N, GROUP))
    workspace = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # the twelve GEMMs of a step, in order; copy index rotates per launch
    gemms = [(name, K, N, M) for M in BATCHES for (name, K, N) in LAYERS]
    plans = {g: w4.w4a16_describe(g[3], g[1], g[2], GROUP) for g in gemms}

    def args_for(g, copy):
        name, K, N, M = g
        return (acts[(name, M)].data_ptr(), packed[name][copy].data_ptr(),
                scales[name].data_ptr(), outs[(name, M)].data_ptr(), M, K, N, GROUP,
                workspace.data_ptr(), sh)

    # A layer is used three times a step (once per batch); its t-th use over
    # the run reads copy t % WEIGHT_COPIES, so between two reads of the same
    # copy every layer has been read WEIGHT_COPIES - 1 more times (~700 MB).
    n_launch = len(gemms)
    calls_per_step = [[args_for(g, (len(BATCHES) * s + BATCHES.index(g[3])) % WEIGHT_COPIES)
                       for g in gemms] for s in range(WEIGHT_COPIES)]

    def run_step(s, events=None):
        calls = calls_per_step[s % WEIGHT_COPIES]
        for i, a in enumerate(calls):
            if events is not None:
                events[i].record(stream)
            rc = lib.w4a16_gemm(*a)
            if rc != 0:
                raise RuntimeError(f"w4a16_gemm failed: {w4.w4a16_status_string(rc)}")

    for s in range(args.warmup):
        run_step(s)
    torch.cuda.synchronize()

    # ---- timed region ------------------------------------------------------
    step_events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_launch)]
                   for _ in range(args.steps)]
    end_event = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        run_step(s, step_events[s])
    end_event.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-launch durations from the events
    per_gemm_ms = {g: [] for g in gemms}
    for s in range(args.steps):
        evs = step_events[s] + ([step_events[s + 1][0]] if s + 1 < args.steps else [end_event])
        for i, g in enumerate(gemms):
            per_gemm_ms[g].append(evs[i].elapsed_time(evs[i + 1]))
    gpu_ms_total = step_events[0][0].elapsed_time(end_event)

    step_flops = sum(roofline.flops(M, K, N) for (_, K, N, M) in gemms)
    step_bytes = sum(roofline.algorithmic_bytes(M, K, N, GROUP) for (_, K, N, M) in gemms)
    step_roof_s = sum(roofline.roofline_seconds(M, K, N, GROUP) for (_, K, N, M) in gemms)
    ms_per_step = wall * 1e3 / args.steps
    value = step_flops / (wall / args.steps) / 1e12

    # ---- the dominant kernel: the variant with the most time in the step ----
    by_kernel = {}
    for g in gemms:
        kname = plans[g].split()[0]
        d = by_kernel.setdefault(kname, {"ms": 0.0, "launches": 0, "bytes": 0, "flops": 0,
                                         "hbm": 0, "mfma": 0})
        d["ms"] += sum(per_gemm_ms[g])
        d["launches"] += len(per_gemm_ms[g])
        name, K, N, M = g
        d["bytes"] += roofline.algorithmic_bytes(M, K, N, GROUP) * len(per_gemm_ms[g])
        d["flops"] += roofline.flops(M, K, N) * len(per_gemm_ms[g])
        d[roofline.bound(M, K, N, GROUP)] += 1
    dom_name, dom = max(by_kernel.items(), key=lambda kv: kv[1]["ms"])
    avg_s = dom["ms"] / dom["launches"] / 1e3
    if dom["hbm"] >= dom["mfma"]:
        achieved = dom["bytes"] / dom["launches"] / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": roofline.HBM_PEAK_BYTES_PER_S / 1e9,
                "unit": "GB/s"}
    else:
        achieved = dom["flops"] / dom["launches"] / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved,
                "peak": roofline.MFMA_F16_PEAK_FLOPS / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = dom_name
    roof["avg_launch_us"] = avg_s * 1e6
    roof["launches_per_step"] = dom["launches"] // args.steps

    per_gemm = []
    for g in gemms:
        name, K, N, M = g
        t = sorted(per_gemm_ms[g])[len(per_gemm_ms[g]) // 2] / 1e3
        per_gemm.append({
            "layer": name, "M": M, "K": K, "N": N, "us": round(t * 1e6, 2),
            "tflops": round(roofline.flops(M, K, N) / t / 1e12, 2),
            "gbps": round(roofline.algorithmic_bytes(M, K, N, GROUP) / t / 1e9, 1),
            "roofline_frac": round(roofline.roofline_seconds(M, K, N, GROUP) / t, 3),
            "bound": roofline.bound(M, K, N, GROUP), "plan": plans[g],
        })

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_sample_cols)

    line = {
        "metric": "W4A16 GEMM TFLOP/s + achieved HBM TB/s (% roofline) at M=1..128, 1 MI355X",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "Llama-2-7B-shaped W4A16 linear layers (qkv 4096x12288, o 4096x4096, "
                        "gate/up 4096x22016, down 11008x4096), group 128, M in {1,16,128}; "
                        "one step = the 12 GEMMs",
            "group": GROUP, "batches": BATCHES, "weight_copies": WEIGHT_COPIES,
            "parallelism": "single GPU",
        },
        "hbm_tbps": step_bytes / (wall / args.steps) / 1e12,
        "step_roofline_frac": step_roof_s / (wall / args.steps),
        "gpu_ms_per_step": gpu_ms_total / args.steps,
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_gemm": per_gemm,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
