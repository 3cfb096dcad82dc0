#!/usr/bin/env python3
"""Benchmark of the rotate + quantize hot path on one MI355X.

Workload: the HARP MLP weight, 4096 x 11008 bfloat16 (0.02 * Student-t(3),
0.5% outlier input channels x30), left plan (16,16,16) and right plan
(43,16,16) with per-group random orthogonal blocks and random signs, then
3-bit group-128 absmax quantization and LSB-first packing.  One step = one
brq_rotate_quantize_pack call (W' = M_U W M_V^T, quantize, pack) on one
resident input; four input copies rotate so the working set exceeds the
256 MB Infinity Cache.

Metric: algorithmic HBM GB/s = (input read once + codes + scales + plan
arrays read once) / step time, and its fraction of the 8 TB/s peak.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Prints one JSON line.  --gpus above 1 exits: this build runs on one GPU.
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

M, N, BITS, GROUP = 4096, 11008, 3, 128
LEFT_RADIX, RIGHT_RADIX = (16, 16, 16), (43, 16, 16)
HBM_PEAK_GBS = 8000.0
FP32_VECTOR_PEAK_TFLOPS = 157.3   # 256 CUs x 2.4 GHz x 256 flop/clk (packed FMA)
FP32_MFMA_PEAK_TFLOPS = 157.3
N_BUFFERS = 4


def plan_bytes(d, radix, signs=True):
    """float32 blocks read once (d * b_t per stage) + float32 signs."""
    return 4 * sum(d * b for b in radix) + (4 * d if signs else 0)


def algorithmic_bytes():
    return (M * N * 2 + M * N * BITS // 8 + M * (N // GROUP) * 4
            + plan_bytes(M, LEFT_RADIX) + plan_bytes(N, RIGHT_RADIX))


def kernel_work(name: str):
    """(bound, algorithmic amount per launch, unit, peak) of a kernel of this
    workload, from the stages its name lists: a dense b x b stage is b FMA
    (2b flop) per element, over all M*N elements.  The fast-path kernels
    contract on fp32 MFMA; the generic tile pass on the fp32 vector ALU."""
    import re
    flop = 0
    for grp in re.findall(r"\(([0-9,]+)\)", name):
        for b in grp.split(","):
            flop += 2 * int(b) * M * N
    if name.startswith("fused"):
        return "mfma", flop / 1e12, "TFLOP/s", FP32_MFMA_PEAK_TFLOPS
    return "alu", flop / 1e12, "TFLOP/s", FP32_VECTOR_PEAK_TFLOPS


def measured_traffic(kernel_name: str):
    """HBM bytes per launch of `kernel_name` from the committed counter
    summary (rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by what the
    same counter reads for a plain copy of known size), or None when the
    summary is missing or was taken on a different kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_fused_harp_mlp_4096x11008.md")
    src = os.path.join(ROOT, "butterfly_rotation_quantization_amd", "csrc", "fused_kernels.hip")
    if not os.path.exists(path) or not os.path.exists(src):
        return None
    sha = hashlib.sha1(open(src, "rb").read()).hexdigest()
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().strip("`").split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha1") != sha:
        return None
    key = "fused_b" if kernel_name.startswith("fusedB") else "fused_a"
    try:
        fetch = float(vals[f"{key}_fetch_kib"]) * float(vals["copy_fetch_scale"])
        write = float(vals[f"{key}_write_kib"]) * float(vals["copy_write_scale"])
    except KeyError:
        return None
    return round((fetch + write) * 1024)


def cpu_baseline(cfg, rows_sample: int):
    """The oracle, as written, on `rows_sample` seeded rows of the workload:
    rows of M_U (factor by factor), times W, then the dense M_V^T (formed from
    its stages inside the timed region), group absmax and packing."""
    import numpy as np
    import synthetic as S
    from oracle import quant as Q
    from oracle import transform as T

    threads = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        threads = min(threads, int(omp))
    left, right = cfg["left"], cfg["right"]
    w64 = S.storage_to_f64(cfg["w"], "bf16")
    rows = np.sort(np.random.default_rng(99).choice(M, size=rows_sample, replace=False))
    t0 = time.perf_counter()
    U = T.Plan(left.d, left.radix, left.mode, left.blocks, left.signs.astype(float))
    V = T.Plan(right.d, right.radix, right.mode, right.blocks, right.signs.astype(float))
    y = T.left_rows(U, rows) @ w64
    y = T.apply_right(V, y, method="dense")
    codes, _alpha = Q.absmax_quantize(y, BITS, GROUP)
    Q.pack(codes, BITS)
    dt = time.perf_counter() - t0
    share = rows_sample / M
    return {
        "value": round(algorithmic_bytes() * share / dt / 1e9, 6),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{rows_sample} of {M} seeded rows of the same workload (left plan rows "
                   f"factor by factor, dense right plan formed in the timed region, absmax, "
                   f"pack); {dt:.1f} s"),
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=M)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device-to-device copy of MIB MiB (3 times) before the "
                         "steps, as the reference kernel for HBM byte counters")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the path needs no "
              "collectives and multi-GPU runs are out of scope here.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import butterfly_rotation_quantization_amd as brq
    import synthetic as S

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    cfg = S.harp_mlp()
    w_host = torch.from_numpy(cfg["w"].view(np.int16)).view(torch.bfloat16)
    bufs = [w_host.to(dev) for _ in range(N_BUFFERS)]
    U = brq.Plan(cfg["left"].d, cfg["left"].radix, "per_group", cfg["left"].blocks,
                 cfg["left"].signs)
    V = brq.Plan(cfg["right"].d, cfg["right"].radix, "per_group", cfg["right"].blocks,
                 cfg["right"].signs)
    codes = torch.empty((M, N * BITS // 8), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, N // GROUP), dtype=torch.float32, device=dev)
    ws = brq.workspace(U, V, M, N, dev)
    stream = torch.cuda.current_stream()

    def step(i):
        brq.rotate_quantize_pack(U, V, bufs[i % N_BUFFERS], BITS, GROUP, codes=codes,
                                 scales=scales, ws=ws, stream=stream)

    if a.copy_calibration:
        nel = a.copy_calibration * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    brq.profile_reset()
    brq.profile_enable(True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(a.steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    brq.profile_enable(False)
    ms = start.elapsed_time(end) / a.steps
    kernels = brq.profile_read()

    alg = algorithmic_bytes()
    value = alg / (ms * 1e-3) / 1e9
    dom_name, (dom_ms, dom_n) = max(kernels.items(), key=lambda kv: kv[1][0])
    bound, work, unit, peak = kernel_work(dom_name)
    avg_ms = dom_ms / max(dom_n, 1)
    achieved = work / (avg_ms * 1e-3)
    line = {
        "metric": "HBM GB/s & % of peak: fused 2-sided rotate+quantize, 4096x11008 bf16",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "harp_mlp_4096x11008_bf16_two_sided_(16,16,16)x(43,16,16)_absmax3_g128",
            "m": M, "n": N, "bits": BITS, "group": GROUP,
            "hbm_peak_frac": round(value / HBM_PEAK_GBS, 5),
            "elements_per_s": round(M * N / (ms * 1e-3), 1),
            "algorithmic_bytes": alg,
            "kernels_ms_per_step": {k: round(v[0] / max(v[1], 1), 5) for k, v in kernels.items()},
        },
        "roofline": {
            "bound": bound,
            "kernel": dom_name,
            "achieved": round(achieved, 4),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 5),
            "traffic": measured_traffic(dom_name),
        },
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, a.cpu_rows)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
