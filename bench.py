#!/usr/bin/env python3
"""Benchmark of the rotate + quantize hot path on one MI355X.

Default workload (the headline line): the HARP MLP weight, 4096 x 11008
bfloat16 (0.02 * Student-t(3), 0.5% outlier input channels x30), left plan
(16,16,16) and right plan (43,16,16) with per-group random orthogonal blocks
and random signs, then 3-bit group-128 absmax quantization and LSB-first
packing.  One step = one brq_rotate_quantize_pack call (W' = M_U W M_V^T,
quantize, pack) on one resident input; several input copies rotate so the
working set exceeds the 256 MB Infinity Cache.

Metric: algorithmic HBM GB/s = (input read once + codes + scales + plan
arrays read once) / step time, and its fraction of the 8 TB/s peak.

--workload names one of the other shapes of the hot path (each prints the
same kind of line; "all" prints one line per workload):

  llama7b_weight   4096 x 4096 bf16, two-sided RHT d=4096, absmax g128 at
                   2, 3 and 4 bits (one step = the three calls)
  llama7b_act      online right-side RHT of activations 2048 x 4096 bf16
  polar_quant      the 7 projections of a decoder block (hidden 4096, FFN
                   12288), block-128 Walsh-Hadamard, per-block norm, 4-bit
                   Lloyd-Max codebook (one step = 7 calls)
  polar_dequant    dequantize + unrotate of the same 7 matrices to bf16
  llama70b_weight  8192 x 28672 bf16, left (32,16,16) and right (7,16,16,16)
                   per-group plans, absmax 2-bit g64
  decode_t1/16/256 online right-side rotation of T x 28672 fp16 activations
                   with the (7,16,16,16) plan: latency per call
  polar_requant    PolarQuant's downstream chain on the same 7 matrices: Q5
                   codes restored and quantized again with absmax INT4 g128
                   in one pass (one step = 7 calls)
  qlinear_t1/16/256 the quantized 70B down projection at decode: T x 28672
                   f16 activations rotated (7,16,16,16), times the 2-bit g64
                   weight 8192 x 28672, the output rotated back (32,16,16):
                   latency per call
  orp_geo          ORP GEO quantization of the 7B weight 4096 x 4096 bf16: 3-bit
                   power-of-two basis, stride-4 orthogonal residual basis,
                   least-squares scales per group of 128
  orp_geo_dequant  its dequantization back to bf16
  harp_build       HARP blocks built on the device from int8 parameters for
                   the 70B schedules (left (32,16,16) d=8192, right
                   (7,16,16,16) d=28672): latency of the seven launches

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline]

--gpus above 1 exits: the benchmark runs on one GPU.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# fp32 peaks: MFMA (v_mfma_f32_16x16x4f32: 256 flop/clk/CU) and vector ALU
# (256 CUs x 64 lanes x 2 (FMA) x 2 (dual issue) x 2.4 GHz); both 157.3 TFLOP/s.
FP32_VECTOR_PEAK_TFLOPS = 157.3
FP32_MFMA_PEAK_TFLOPS = 157.3
FP64_VECTOR_PEAK_TFLOPS = 78.6
F16_MFMA_PEAK_TFLOPS = 2500.0  # dense f16 / bf16 MFMA
MALL_BYTES = 256 << 20


def plan_bytes(d, radix, blocks=True, signs=True):
    """float32 blocks read once (d * b_t per stage) + float32 signs."""
    return (4 * sum(d * b for b in radix) if blocks else 0) + (4 * d if signs else 0)


def cpu_threads():
    threads = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        threads = min(threads, int(omp))
    return threads


def copies_for(nbytes, floor=2):
    """Input copies that together exceed the Infinity Cache."""
    return max(floor, math.ceil(1.25 * MALL_BYTES / max(nbytes, 1)) + 1)


def stage_flops(radix, hadamard, elems):
    """Algorithmic flops of applying one side's stages to `elems` elements: a
    dense b x b stage is b FMA (2b flop) per element, a Hadamard stage of
    radix b is a log2(b)-level butterfly (log2(b) add/sub per element)."""
    if hadamard:
        return sum(int(round(math.log2(b))) for b in radix) * elems
    return sum(2 * b for b in radix) * elems


def roofline_of(bytes_, flops, engine):
    """(bound, achieved-per-second function inputs) for one kernel: the
    resource whose time floor is larger at peak binds."""
    t_hbm = bytes_ / (HBM_PEAK_GBS * 1e9)
    peak = {"mfma": FP32_MFMA_PEAK_TFLOPS, "alu64": FP64_VECTOR_PEAK_TFLOPS,
            "mfma16": F16_MFMA_PEAK_TFLOPS}.get(engine, FP32_VECTOR_PEAK_TFLOPS)
    t_fl = flops / (peak * 1e12)
    if t_hbm >= t_fl:
        return "hbm", bytes_ / 1e9, "GB/s", HBM_PEAK_GBS
    return ("mfma" if engine.startswith("mfma") else "alu"), flops / 1e12, "TFLOP/s", peak


def measured_traffic(workload: str, kernel_name: str):
    """HBM bytes per launch of `kernel_name` from the committed counter
    summary of this workload (rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled
    by what the same counter reads for a plain copy of known size), or None
    when the summary is missing or was taken on a different kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().strip("`").split("=", 1)
            vals[k.strip()] = v.strip()
    h = hashlib.sha1()
    for name in vals.get("kernel_source", "").split(","):
        src = os.path.join(ROOT, "butterfly_rotation_quantization_amd", "csrc", name.strip())
        if not name.strip() or not os.path.isfile(src):
            return None
        h.update(open(src, "rb").read())
    if vals.get("kernel_source_sha1") != h.hexdigest():
        return None
    key = vals.get(f"kernel[{kernel_name}]")
    if key is None:
        return None
    try:
        fetch = float(vals[f"{key}_fetch_kib"]) * float(vals["copy_fetch_scale"])
        write = float(vals[f"{key}_write_kib"]) * float(vals["copy_write_scale"])
    except KeyError:
        return None
    return round((fetch + write) * 1024)


def storage_tensor(arr, dtype, dev):
    """A device tensor holding the bit pattern of a synthetic storage array."""
    import numpy as np
    import torch
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(dev)
    if dtype == "f16":
        return torch.from_numpy(arr).to(dev)
    return torch.from_numpy(arr).to(dev)


def oracle_plan(side):
    from oracle import transform as T
    return T.Plan(side.d, side.radix, side.mode, side.blocks,
                  None if side.signs is None else side.signs.astype(float))


# ---------------------------------------------------------------- workloads

class Workload:
    """One shape of the hot path: device set-up, the step, the algorithmic
    bytes and flops of each kernel it launches, and the oracle's timing."""
    name = ""
    metric = ""
    unit = "GB/s"
    higher_is_better = True
    dtype = "f32"

    def setup(self, brq, dev, stream):
        raise NotImplementedError

    def step(self, i):
        raise NotImplementedError

    def alg_bytes(self):
        raise NotImplementedError

    def kernel_cost(self, name):
        """(algorithmic bytes, algorithmic flops, engine) of one launch."""
        raise NotImplementedError

    def value(self, ms):
        return self.alg_bytes() / (ms * 1e-3) / 1e9

    def config(self):
        return {}

    def elements(self):
        """Matrix elements one step transforms."""
        raise NotImplementedError

    def cpu_baseline(self, budget_s):
        return None


def quant_bytes(m, n, bits, group, scale_bytes):
    return m * n * bits // 8 + m * (n // group) * scale_bytes


def _two_sided_parity(self):
    """The GPU's codes on the oracle's sampled rows against the oracle's codes
    of the same rows: mismatches, the decision band's population (elements
    within 1e-6 relative of a threshold), and mismatches outside the band."""
    import numpy as np
    from oracle import quant as Q
    if getattr(self, "_oracle_sample", None) is None:
        return None
    rows, y, codes = self._oracle_sample
    out = {"rows": int(len(rows)), "elements": 0, "mismatches": 0, "band": 0,
           "mismatches_outside_band": 0}
    for b in self.bits_list:
        got = Q.unpack(self.out[b][0].cpu().numpy()[rows], b, self.N)
        band = Q.absmax_band(y, b, self.group)
        mism = got != codes[b]
        out["elements"] += int(got.size)
        out["mismatches"] += int(mism.sum())
        out["band"] += int(band.sum())
        out["mismatches_outside_band"] += int((mism & ~band).sum())
    out["band_frac"] = out["band"] / max(out["elements"], 1)
    return out


class TwoSidedWeight(Workload):
    """Two-sided rotate + quantize + pack of one weight matrix."""
    kind = "absmax"

    def __init__(self, name, metric, cfg_fn, bits_list, group):
        self.name, self.metric = name, metric
        self.cfg_fn = cfg_fn
        self.bits_list = tuple(bits_list)
        self.group = group

    def setup(self, brq, dev, stream):
        import torch
        self.brq = brq
        self.cfg = cfg = self.cfg_fn()
        self.M, self.N = cfg["w"].shape
        w = storage_tensor(cfg["w"], cfg["dtype"], dev)
        self.bufs = [w] + [w.clone() for _ in range(copies_for(w.numel() * 2) - 1)]
        L, R = cfg["left"], cfg["right"]
        self.U = brq.Plan(L.d, L.radix, L.mode, L.blocks, L.signs)
        self.V = brq.Plan(R.d, R.radix, R.mode, R.blocks, R.signs)
        self.out = {b: (torch.empty((self.M, self.N * b // 8), dtype=torch.uint8, device=dev),
                        torch.empty((self.M, self.N // self.group), dtype=torch.float32,
                                    device=dev)) for b in self.bits_list}
        self.ws = brq.workspace(self.U, self.V, self.M, self.N, dev)
        self.stream = stream

    def step(self, i):
        w = self.bufs[i % len(self.bufs)]
        for b in self.bits_list:
            c, s = self.out[b]
            self.brq.rotate_quantize_pack(self.U, self.V, w, b, self.group, codes=c, scales=s,
                                          ws=self.ws, stream=self.stream)

    def elements(self):
        return self.M * self.N * len(self.bits_list)

    def _plans_bytes(self):
        L, R = self.cfg["left"], self.cfg["right"]
        return (plan_bytes(L.d, L.radix, L.mode != "hadamard", L.signs is not None)
                + plan_bytes(R.d, R.radix, R.mode != "hadamard", R.signs is not None))

    def alg_bytes(self):
        M, N = self.M, self.N
        return sum(M * N * 2 + quant_bytes(M, N, b, self.group, 4) + self._plans_bytes()
                   for b in self.bits_list)

    def kernel_cost(self, name):
        M, N, E = self.M, self.N, self.M * self.N
        L, R = self.cfg["left"], self.cfg["right"]
        had = L.mode == "hadamard"
        qb = re.search(r"quant b(\d+)", name)
        bits = int(qb.group(1)) if qb else self.bits_list[0]
        q_out = quant_bytes(M, N, bits, self.group, 4)
        if name.startswith("fusedA"):
            # U_0 and V_0 of the plans (Hadamard plans: the first four levels)
            fl = (stage_flops((16,), True, E) * 2 if had
                  else stage_flops((L.radix[0], R.radix[0]), False, E))
            blk = 0 if had else 4 * (M * L.radix[0] + N * R.radix[0])
            # products on split-f16 MFMA: the f16 peak applies
            return E * 2 + E * 4 + blk + 4 * (M + N), fl, "mfma16"
        if name.startswith("fusedB"):
            fl = (stage_flops((16, 16), True, E) * 2 if had
                  else stage_flops(L.radix[1:] + R.radix[1:], False, E))
            blk = 0 if had else 4 * (M * sum(L.radix[1:]) + N * sum(R.radix[1:]))
            return E * 4 + q_out + blk, fl, "mfma16"
        if name.startswith("rowhad quant"):  # quantizer pass over the float32 intermediate
            return E * 4 + q_out, 0, "alu"
        # stage pass ("stage L(b) S..") or generic tile pass ("pass L(..) R(..) [quant]")
        radices = []
        for side, d, plan in (("L", M, L), ("R", N, R)):
            m_ = re.search(side + r"\(([0-9,]+)\)", name)
            if m_:
                rs = tuple(int(x) for x in m_.group(1).split(","))
                radices.append((rs, d))
        fl = sum(stage_flops(rs, had, E) for rs, _ in radices)
        blk = 0 if had else sum(4 * d * sum(rs) for rs, d in radices)
        first = self._first_kernel == name
        bytes_in = E * 2 if first else E * 4
        bytes_out = q_out if name.endswith("quant") else E * 4
        return bytes_in + bytes_out + blk, fl, "alu"

    def config(self):
        L, R = self.cfg["left"], self.cfg["right"]
        return {"m": self.M, "n": self.N, "bits": list(self.bits_list), "group": self.group,
                "left": {"d": L.d, "radix": list(L.radix), "mode": L.mode},
                "right": {"d": R.d, "radix": list(R.radix), "mode": R.mode},
                "input_copies": len(self.bufs)}

    parity_sample = _two_sided_parity

    def cpu_baseline(self, budget_s):
        """The oracle on seeded rows: rows of M_U (factor by factor), times W,
        then M_V^T (dense from its stages when d <= 11008, else factor by
        factor), group absmax and packing."""
        import numpy as np
        import synthetic as S
        from oracle import quant as Q
        from oracle import transform as T
        U, V = oracle_plan(self.cfg["left"]), oracle_plan(self.cfg["right"])
        method = "dense" if V.d <= 11008 else "factored"
        w64 = S.storage_to_f64(self.cfg["w"], self.cfg["dtype"])
        rng = np.random.default_rng(99)

        def run(k):
            rows = np.sort(rng.choice(self.M, size=k, replace=False))
            t0 = time.perf_counter()
            y = T.left_rows(U, rows) @ w64
            y = T.apply_right(V, y, method=method)
            codes = {}
            for b in self.bits_list:
                codes[b], _alpha = Q.absmax_quantize(y, b, self.group)
                Q.pack(codes[b], b)
            dt = time.perf_counter() - t0
            self._oracle_sample = (rows, y, codes)
            return dt

        k = self._cpu_rows
        dt = run(k)
        share = k / self.M
        return {
            "value": round(self.alg_bytes() * share / dt / 1e9, 6),
            "unit": "GB/s",
            "cores": cpu_threads(),
            "kind": "oracle",
            "sample": (f"{k} of {self.M} seeded rows of the same workload (left plan rows "
                       f"factor by factor, right plan {method}, absmax at "
                       f"{'/'.join(map(str, self.bits_list))} bits, pack); {dt:.1f} s"),
        }


class RightRotate(Workload):
    """Online right-side rotation of activations (Y = X M_V^T, same dtype)."""

    def __init__(self, name, metric, side, x, dtype, latency=False):
        self.name, self.metric = name, metric
        self.side, self.x_host, self.xdtype = side, x, dtype
        self.latency = latency
        if latency:
            self.unit, self.higher_is_better = "us", False

    def setup(self, brq, dev, stream):
        import torch
        self.brq = brq
        P = self.side
        self.T, self.N = self.x_host.shape
        x = storage_tensor(self.x_host, self.xdtype, dev)
        # Latency runs keep one activation buffer (it comes fresh from the
        # previous kernel) and rotate over copies of the plan, as the layers
        # of a model would, so the plan arrays are not cache-resident.
        xb = x.numel() * 2
        pb = plan_bytes(P.d, P.radix, P.mode != "hadamard", P.signs is not None)
        self.bufs = [x] + ([] if self.latency else
                           [x.clone() for _ in range(copies_for(xb) - 1)])
        nplans = copies_for(pb, floor=1) if self.latency and P.mode != "hadamard" else 1
        self.plans = [brq.Plan(P.d, P.radix, P.mode, P.blocks, P.signs) for _ in range(nplans)]
        self.y = torch.empty_like(x)
        self.ws = brq.workspace(None, self.plans[0], self.T, self.N, dev)
        self.stream = stream

    def step(self, i):
        self.brq.rotate(self.plans[i % len(self.plans)], self.bufs[i % len(self.bufs)], self.y,
                        side="right", ws=self.ws, stream=self.stream)

    @property
    def step_warm(self):
        """Latency runs also time the same call with one plan, whose blocks
        then stay in the caches (warm), beside the plan rotation (cold)."""
        if not self.latency:
            return None
        return lambda i, stream=None: self.brq.rotate(self.plans[0], self.bufs[0], self.y,
                                                      side="right", ws=self.ws,
                                                      stream=stream or self.stream)

    def elements(self):
        return self.T * self.N

    def alg_bytes(self):
        P = self.side
        return 4 * self.T * self.N + plan_bytes(P.d, P.radix, P.mode != "hadamard",
                                                P.signs is not None)

    def value(self, ms):
        if self.latency:
            return ms * 1e3
        return super().value(ms)

    def kernel_cost(self, name):
        P, E = self.side, self.T * self.N
        had = P.mode == "hadamard"
        m_ = re.search(r"\(([0-9,]+)\)", name)
        rs = tuple(int(x) for x in m_.group(1).split(",")) if m_ else P.radix
        if name.startswith("rowhad"):
            hd = int(re.search(r"H(\d+)", name).group(1))
            return 4 * E + 4 * P.d, int(round(math.log2(hd))) * E, "alu"
        fl = stage_flops(rs, had, E)
        blk = 0 if had else 4 * P.d * sum(rs)
        first, last = self._first_kernel == name, self._last_kernel == name
        return (2 if first else 4) * E + (2 if last else 4) * E + blk, fl, "alu"

    def config(self):
        P = self.side
        return {"tokens": self.T, "n": self.N, "d": P.d, "radix": list(P.radix),
                "mode": P.mode, "io_dtype": self.xdtype, "input_copies": len(self.bufs),
                "plan_copies": len(self.plans)}

    def cpu_baseline(self, budget_s):
        import numpy as np
        import synthetic as S
        from oracle import transform as T
        V = oracle_plan(self.side)
        x64 = S.storage_to_f64(self.x_host, self.xdtype)
        k = min(self.T, self._cpu_rows)
        method = "dense" if V.d <= 4096 else "factored"
        t0 = time.perf_counter()
        y = T.apply_right(V, x64[:k], method=method)
        S.to_storage(y, self.xdtype)
        dt = time.perf_counter() - t0
        share = k / self.T
        if self.latency:
            val, unit = round(dt * 1e6 / share, 3), "us"
        else:
            val, unit = round(self.alg_bytes() * share / dt / 1e9, 6), "GB/s"
        return {"value": val, "unit": unit, "cores": cpu_threads(), "kind": "oracle",
                "sample": (f"{k} of {self.T} seeded rows (right plan {method}, rounded to "
                           f"{self.xdtype}); {dt:.2f} s")}


class PolarBlock(Workload):
    """PolarQuant-style quantization (or dequantization) of the 7 projections
    of one decoder block with block-128 Walsh-Hadamard and a 4-bit codebook."""
    dequant = False

    def __init__(self, name, metric, dequant):
        self.name, self.metric, self.dequant = name, metric, dequant

    def setup(self, brq, dev, stream):
        import numpy as np
        import torch
        import synthetic as S
        from oracle import lloydmax as LM
        self.brq = brq
        self.cfg = cfg = S.polar()
        self.cb = LM.lloyd_max_gaussian(cfg["bits"])[0].astype(np.float32)
        R = cfg["right"]
        self.H = brq.Plan(R.d, R.radix, R.mode, R.blocks, R.signs)
        self.mats = {}
        for name, arr in cfg["mats"].items():
            m, n = arr.shape
            w = storage_tensor(arr, "bf16", dev)
            codes = torch.empty((m, n * cfg["bits"] // 8), dtype=torch.uint8, device=dev)
            scales = torch.empty((m, n // cfg["group"]), dtype=torch.float16, device=dev)
            self.mats[name] = (w, codes, scales)
        if self.dequant:  # codes and norms of the same matrices
            for w, codes, scales in self.mats.values():
                brq.rotate_quantize_pack(None, self.H, w, cfg["bits"], cfg["group"],
                                         "codebook_norm", self.cb, codes=codes, scales=scales)
            torch.cuda.synchronize()
        self.stream = stream

    def step(self, i):
        b, g = self.cfg["bits"], self.cfg["group"]
        for w, codes, scales in self.mats.values():
            if self.dequant:
                self.brq.dequant_unrotate(None, self.H, codes, scales, w.shape[0], w.shape[1],
                                          b, g, "codebook_norm", self.cb, out=w,
                                          stream=self.stream)
            else:
                self.brq.rotate_quantize_pack(None, self.H, w, b, g, "codebook_norm", self.cb,
                                              codes=codes, scales=scales, stream=self.stream)

    def elements(self):
        return sum(a.size for a in self.cfg["mats"].values())

    def alg_bytes(self):
        b, g = self.cfg["bits"], self.cfg["group"]
        return sum(a.size * 2 + quant_bytes(a.shape[0], a.shape[1], b, g, 2)
                   for a in self.cfg["mats"].values())

    def kernel_cost(self, name):
        # every launch of the step has the same per-element cost; the profile
        # aggregates the 7 calls, so use the mean launch
        E = sum(a.size for a in self.cfg["mats"].values()) / 7.0
        return self.alg_bytes() / 7.0, 7 * E, "alu"

    def config(self):
        return {"matrices": {k: list(v.shape) for k, v in self.cfg["mats"].items()},
                "d": 128, "bits": self.cfg["bits"], "group": self.cfg["group"],
                "quantizer": "codebook_norm (Lloyd-Max N(0,1), fp16 norms)",
                "direction": "dequant+unrotate to bf16" if self.dequant else
                "rotate+quantize+pack"}

    def cpu_baseline(self, budget_s):
        """The oracle on the first `_cpu_rows` rows of every projection."""
        import numpy as np
        import synthetic as S
        from oracle import quant as Q
        from oracle import transform as T
        H = oracle_plan(self.cfg["right"])
        b, g = self.cfg["bits"], self.cfg["group"]
        k = self._cpu_rows
        dt, done = 0.0, 0
        for arr in self.cfg["mats"].values():
            x64 = S.storage_to_f64(arr[:k], "bf16")
            if self.dequant:  # codes and norms first, outside the timed region
                codes, r64 = Q.codebook_norm_quantize(T.apply_right(H, x64), self.cb, g)[:2]
                t0 = time.perf_counter()
                v = Q.codebook_dequant(codes, r64.astype(np.float16), self.cb, g)
                S.to_storage(T.apply_right(H, v, inverse=True), "bf16")
            else:
                t0 = time.perf_counter()
                codes = Q.codebook_norm_quantize(T.apply_right(H, x64), self.cb, g)[0]
                Q.pack(codes, b)
            dt += time.perf_counter() - t0
            done += x64.size
        share = done / sum(a.size for a in self.cfg["mats"].values())
        return {"value": round(self.alg_bytes() * share / dt / 1e9, 6), "unit": "GB/s",
                "cores": cpu_threads(), "kind": "oracle",
                "sample": (f"the first {k} rows of each of the 7 projections "
                           f"({100 * share:.0f}% of the elements; right plan dense); {dt:.2f} s")}


class PolarRequant(Workload):
    """PolarQuant's downstream chain on the 7 projections: Q5 codes and fp16
    norms (block-128 Walsh-Hadamard, 5-bit Lloyd-Max) restored and quantized
    again with absmax INT4, group 128, in one pass (brq_requant)."""
    bits_in, bits_out, g_out = 5, 4, 128

    def __init__(self, name, metric):
        self.name, self.metric = name, metric

    def setup(self, brq, dev, stream):
        import numpy as np
        import torch
        import synthetic as S
        from oracle import lloydmax as LM
        self.brq, self.stream = brq, stream
        self.cfg = cfg = S.polar()
        self.g_in = cfg["group"]
        self.cb = LM.lloyd_max_gaussian(self.bits_in)[0].astype(np.float32)
        R = cfg["right"]
        self.H = brq.Plan(R.d, R.radix, R.mode, R.blocks, R.signs)
        self.mats = []
        for arr in cfg["mats"].values():
            m, n = arr.shape
            w = storage_tensor(arr, "bf16", dev)
            codes, norms = brq.rotate_quantize_pack(None, self.H, w, self.bits_in, self.g_in,
                                                    "codebook_norm", self.cb)
            del w
            out = torch.empty((m, n * self.bits_out // 8), dtype=torch.uint8, device=dev)
            sc = torch.empty((m, n // self.g_out), dtype=torch.float32, device=dev)
            self.mats.append((m, n, codes, norms, out, sc))
        torch.cuda.synchronize()

    def step(self, i):
        for m, n, codes, norms, out, sc in self.mats:
            self.brq.requant(self.H, codes, norms, m, n, self.bits_in, self.g_in, self.bits_out,
                             self.g_out, codebook=self.cb, codes_out=out, scales_out=sc,
                             stream=self.stream)

    def elements(self):
        return sum(m * n for m, n, *_ in self.mats)

    def alg_bytes(self):
        return sum(quant_bytes(m, n, self.bits_in, self.g_in, 2) +
                   quant_bytes(m, n, self.bits_out, self.g_out, 4) for m, n, *_ in self.mats)

    def kernel_cost(self, name):
        E = self.elements() / 7.0
        return self.alg_bytes() / 7.0, 7 * E, "alu"

    def config(self):
        return {"matrices": {k: list(v.shape) for k, v in self.cfg["mats"].items()}, "d": 128,
                "in": f"codebook_norm {self.bits_in}-bit g{self.g_in} (Lloyd-Max N(0,1), fp16 norms)",
                "out": f"absmax {self.bits_out}-bit g{self.g_out} (float32 scales)"}

    def cpu_baseline(self, budget_s):
        import numpy as np
        from oracle import chain as C
        from oracle import quant as Q
        H = oracle_plan(self.cfg["right"])
        k = self._cpu_rows
        dt, done = 0.0, 0
        for m, n, codes, norms, *_ in self.mats:
            ci = Q.unpack(codes[:k].cpu().numpy(), self.bits_in, n)
            r16 = norms[:k].cpu().numpy()
            t0 = time.perf_counter()
            c, a, _ = C.requant(ci, r16, self.cb, self.g_in, H, self.bits_out, self.g_out)
            Q.pack(c, self.bits_out)
            dt += time.perf_counter() - t0
            done += k * n
        share = done / self.elements()
        return {"value": round(self.alg_bytes() * share / dt / 1e9, 6), "unit": "GB/s",
                "cores": cpu_threads(), "kind": "oracle",
                "sample": (f"the first {k} rows of each of the 7 projections "
                           f"({100 * share:.0f}% of the elements); {dt:.2f} s")}


class DecodeLinear(Workload):
    """The quantized down projection of a 70B decoder layer at decode
    (brq_qlinear): T tokens x 28672 f16 activations rotated with the right plan
    (7,16,16,16), times the 2-bit g64 absmax weight 8192 x 28672 (dequantized
    in the product's prologue), the output rotated back with the left plan
    (32,16,16)."""
    unit, higher_is_better, dtype = "us", False, "f16"
    m, n, bits, group = 8192, 28672, 2, 64

    def __init__(self, name, metric, tokens):
        self.name, self.metric, self.T = name, metric, tokens

    def setup(self, brq, dev, stream):
        import numpy as np
        import torch
        import synthetic as S
        self.brq, self.stream = brq, stream
        cfg = S.llama70b(rows=1, tokens=(self.T,))
        self.Ls, self.Rs = cfg["left"], cfg["right"]
        rng = S.streams(7100, 1)[0]
        m, n, b = self.m, self.n, self.bits
        # the weight: seeded codes and scales (any W' has this form)
        self.codes_h = rng.integers(0, 256, size=(m, n * b // 8), dtype=np.int64).astype(np.uint8)
        self.alpha_h = ((0.5 + rng.random((m, n // self.group))) * 0.05).astype(np.float32)
        self.x_h = cfg["acts"][self.T]
        self.U = brq.Plan(self.Ls.d, self.Ls.radix, self.Ls.mode, self.Ls.blocks, self.Ls.signs)
        self.V = brq.Plan(self.Rs.d, self.Rs.radix, self.Rs.mode, self.Rs.blocks, self.Rs.signs)
        # several weight copies so that the step streams the weight from HBM
        wb = self.codes_h.nbytes + self.alpha_h.nbytes
        self.ws_copies = [(torch.from_numpy(self.codes_h).to(dev), torch.from_numpy(self.alpha_h).to(dev))
                          for _ in range(copies_for(wb))]
        self.x = torch.from_numpy(self.x_h).to(dev)
        self.y = torch.empty((self.T, m), dtype=torch.float16, device=dev)
        q = brq.make_quant(b, self.group, "absmax")
        nb = brq.lib().brq_qlinear_workspace_bytes(self.U.handle, self.V.handle, ctypes.byref(q),
                                                   self.T, m, n)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        self.latency = True

    def step(self, i):
        codes, alpha = self.ws_copies[i % len(self.ws_copies)]
        self.brq.qlinear(self.U, self.V, self.x, codes, alpha, self.m, self.n, self.bits,
                         self.group, y=self.y, ws=self.ws, stream=self.stream)

    def step_warm(self, i, stream=None):
        """The same call on one weight copy (as far as the caches hold it)."""
        codes, alpha = self.ws_copies[0]
        self.brq.qlinear(self.U, self.V, self.x, codes, alpha, self.m, self.n, self.bits,
                         self.group, y=self.y, ws=self.ws, stream=stream or self.stream)

    def value(self, ms):
        return ms * 1e3

    def elements(self):
        return self.m * self.n

    def alg_bytes(self):
        m, n, T_ = self.m, self.n, self.T
        return (quant_bytes(m, n, self.bits, self.group, 4) + 2 * T_ * n + 2 * T_ * m +
                plan_bytes(self.Rs.d, self.Rs.radix) + plan_bytes(self.Ls.d, self.Ls.radix))

    def kernel_cost(self, name):
        m, n, T_ = self.m, self.n, self.T
        if name.startswith("qlinear b"):
            return (quant_bytes(m, n, self.bits, self.group, 4) + 2 * T_ * n,
                    2 * T_ * m * n, "mfma16")
        if name.startswith("qlinear reduce"):
            return 8 * T_ * m, T_ * m, "alu"
        # the rotations' stage passes
        d = self.Rs.d if name.startswith("stage R(") else self.Ls.d  # R^T: the output's
        b = int(re.search(r"\((\d+)", name).group(1))
        return 8 * T_ * d + 4 * d * b, 2 * b * T_ * d, "alu"

    def config(self):
        return {"tokens": self.T, "m": self.m, "n": self.n, "bits": self.bits, "group": self.group,
                "left": {"d": self.Ls.d, "radix": list(self.Ls.radix)},
                "right": {"d": self.Rs.d, "radix": list(self.Rs.radix)},
                "weight_copies": len(self.ws_copies)}

    def cpu_baseline(self, budget_s):
        import numpy as np
        import synthetic as S
        from oracle import linear as OL
        from oracle import quant as Q
        Uo, Vo = oracle_plan(self.Ls), oracle_plan(self.Rs)
        rows = 256  # output rows of the weight in the sample
        t0 = time.perf_counter()
        xt = OL.rotate_acts(Vo, S.storage_to_f64(self.x_h, "f16"))
        w = OL.weight(Q.unpack(self.codes_h[:rows], self.bits, self.n), self.alpha_h[:rows].astype(np.float64),
                      self.bits, self.group)
        z = xt @ w.T
        dt = time.perf_counter() - t0
        share = rows / self.m
        return {"value": round(dt * 1e6 / share, 1), "unit": "us", "cores": cpu_threads(),
                "kind": "oracle",
                "sample": (f"rotation of the {self.T} tokens and {rows} of the {self.m} weight rows "
                           f"(scaled by {1 / share:.0f}); the output rotation left out; {dt:.2f} s")}


class OrpGeo(Workload):
    """ORP GEO quantization (or dequantization) of the 7B-shaped weight,
    4096 x 4096 bf16 (0.02 * Student-t(3), 0.5% outlier input channels x30):
    power-of-two primary basis, stride-4 exchange secondary basis,
    least-squares scales per group of 128, 3 bits (one step = one call)."""
    bits, group, stride = 3, 128, 4

    def __init__(self, name, metric, dequant):
        self.name, self.metric, self.dequant = name, metric, dequant

    def setup(self, brq, dev, stream):
        import torch
        import synthetic as S
        self.brq, self.stream = brq, stream
        self.cfg = S.llama7b(act_tokens=1)
        self.w_h = self.cfg["w"]
        self.M, self.N = self.w_h.shape
        w = storage_tensor(self.w_h, "bf16", dev)
        self.bufs = [w] + [w.clone() for _ in range(copies_for(w.numel() * 2) - 1)]
        self.codes, self.signs, self.coef = brq.orp_geo_quantize(w, self.bits, self.group,
                                                                 self.stride, stream=stream)
        if self.dequant:
            n_out = copies_for(w.numel() * 2)
            self.outs = [torch.empty_like(w) for _ in range(n_out)]

    def step(self, i):
        if self.dequant:
            self.brq.orp_geo_dequant(self.codes, self.signs, self.coef, self.M, self.N, self.bits,
                                     self.group, self.stride, out=self.outs[i % len(self.outs)],
                                     stream=self.stream)
        else:
            self.brq.orp_geo_quantize(self.bufs[i % len(self.bufs)], self.bits, self.group,
                                      self.stride, codes=self.codes, signs=self.signs,
                                      coef=self.coef, stream=self.stream)

    def elements(self):
        return self.M * self.N

    def alg_bytes(self):
        E = self.M * self.N
        return 2 * E + E * self.bits // 8 + E // 16 + 8 * E // self.group

    def kernel_cost(self, name):
        return self.alg_bytes(), 0, "alu"

    def config(self):
        return {"m": self.M, "n": self.N, "bits": self.bits, "group": self.group,
                "stride": self.stride, "io_dtype": "bf16",
                "copies": len(self.outs) if self.dequant else len(self.bufs)}

    def cpu_baseline(self, budget_s):
        import synthetic as S
        from oracle import orp as O
        k = self._cpu_rows
        w64 = S.storage_to_f64(self.w_h[:k], "bf16")
        t0 = time.perf_counter()
        codes, sigma, coef, b1, b2, _ = O.geo_quantize(w64, self.bits, self.group, self.stride)
        if self.dequant:
            O.geo_dequant(codes, sigma, coef, self.bits, self.group, self.stride)
        dt = time.perf_counter() - t0
        share = k / self.M
        return {"value": round(self.alg_bytes() * share / dt / 1e9, 6), "unit": "GB/s",
                "cores": cpu_threads(), "kind": "oracle",
                "sample": (f"{k} of {self.M} rows ({'quantize + dequantize' if self.dequant else 'quantize'} "
                           f"in the oracle); {dt:.2f} s")}


class HarpBuild(Workload):
    """HARP blocks built on the device from int8 parameters: every stage of a
    left and a right schedule in one brq_harp_blocks_batch call (the stages of
    radix 3..32 share one launch, others launch alone)."""
    unit, higher_is_better, dtype = "us", False, "f64"

    def __init__(self, name, metric, sides):
        self.name, self.metric = name, metric
        self.sides = sides  # [(d, radix)]

    def setup(self, brq, dev, stream):
        import numpy as np
        import torch
        import synthetic as S
        self.brq, self.stream = brq, stream
        rng = S.streams(7000, 1)[0]
        self.jobs = []
        for d, radix in self.sides:
            for b in radix:
                ng = d // b
                npar = 1 if b == 2 else b * (b - 1) // 2
                q = rng.integers(-127, 128, size=(ng, npar)).astype(np.int8)
                base = None if b & (b - 1) == 0 else S.random_orthogonal(rng, b).astype(np.float32)
                self.jobs.append((b, q, base,
                                  torch.from_numpy(q).to(dev),
                                  None if base is None else torch.from_numpy(base).to(dev),
                                  torch.empty((ng, b, b), dtype=torch.float32, device=dev)))

    def step(self, i):
        self.brq.harp_blocks_batch([(b, q, 0.004, base, out) for b, _, _, q, base, out in self.jobs],
                                   stream=self.stream)

    def value(self, ms):
        return ms * 1e3

    def elements(self):
        return sum(out.numel() for *_, out in self.jobs)

    @staticmethod
    def _cost(b, ng, sylvester):
        npar = 1 if b == 2 else b * (b - 1) // 2
        # Gauss-Jordan on [I - A | I + A] (b pivots x 2b columns x b rows, an
        # FMA each: 4 b^3 flop) and the product Q G: b^3 FMA for a given G,
        # a Walsh-Hadamard transform of each row (b^2 log2 b additions) for
        # the Sylvester one
        if b == 2:
            return ng * (npar + 4 * b * b), ng * 16  # Givens: Q G only
        prod = b * b * (b.bit_length() - 1) if sylvester else 2 * b ** 3
        return ng * (npar + 4 * b * b), ng * (4 * b ** 3 + prod)

    def alg_bytes(self):
        return sum(self._cost(b, out.shape[0], base is None)[0] + (0 if base is None else 4 * b * b)
                   for b, _, _, _, base, out in self.jobs)

    def kernel_cost(self, name):
        if name.endswith("batch"):  # every job of radix 3..32 in the one launch
            costs = [self._cost(bb, out.shape[0], base is None) for bb, _, _, _, base, out in self.jobs
                     if 3 <= bb <= 32]
            return sum(c[0] for c in costs), sum(c[1] for c in costs), "alu64"
        b = int(re.search(r"b(\d+)$", name).group(1))
        costs = [self._cost(bb, out.shape[0], base is None) for bb, _, _, _, base, out in self.jobs if bb == b]
        n = len(costs)
        return (sum(c[0] for c in costs) // n, sum(c[1] for c in costs) // n, "alu64")

    def config(self):
        return {"schedules": [{"d": d, "radix": list(r)} for d, r in self.sides],
                "scale": 0.004, "blocks": self.elements()}

    def cpu_baseline(self, budget_s):
        from oracle import harp as OH
        t0 = time.perf_counter()
        done = total = 0.0
        for b, q, base, *_ in self.jobs:
            k = min(q.shape[0], 64)
            OH.stage_blocks(b, k, q[:k], 0.004, None if base is None else base.astype("float64"))
            done += k
            total += q.shape[0]
        dt = time.perf_counter() - t0
        return {"value": round(dt * 1e6 * total / done, 1), "unit": "us", "cores": cpu_threads(),
                "kind": "oracle",
                "sample": f"64 blocks of each stage ({int(done)} of {int(total)}); {dt:.2f} s"}


def make_workload(name):
    import synthetic as S
    if name == "harp_mlp":
        w = TwoSidedWeight(name, "HBM GB/s & % of peak: fused 2-sided rotate+quantize, "
                           "4096x11008 bf16", S.harp_mlp, (3,), 128)
        w.workload = "harp_mlp_4096x11008_bf16_two_sided_(16,16,16)x(43,16,16)_absmax3_g128"
        w._cpu_rows = 4096
        return w
    if name == "llama7b_weight":
        w = TwoSidedWeight(name, "HBM GB/s: two-sided RHT d=4096 + absmax g128 at 2/3/4 bits, "
                           "4096x4096 bf16", lambda: S.llama7b(act_tokens=1), (2, 3, 4), 128)
        w.workload = "llama7b_weight_4096x4096_bf16_two_sided_rht4096_absmax234_g128"
        w._cpu_rows = 4096
        return w
    if name == "llama70b_weight":
        w = TwoSidedWeight(name, "HBM GB/s: two-sided HARP (32,16,16)x(7,16,16,16) + absmax2 "
                           "g64, 8192x28672 bf16", lambda: S.llama70b(tokens=()), (2,), 64)
        w.workload = "llama70b_weight_8192x28672_bf16_two_sided_(32,16,16)x(7,16,16,16)_absmax2_g64"
        w._cpu_rows = 2048
        return w
    if name == "llama7b_act":
        cfg = S.llama7b(rows=1)
        w = RightRotate(name, "HBM GB/s: online right-side RHT d=4096, 2048x4096 bf16",
                        cfg["right"], cfg["x"], "bf16")
        w.workload = "llama7b_act_2048x4096_bf16_rht4096"
        w._cpu_rows = 2048
        return w
    if name.startswith("decode_t"):
        t = int(name[len("decode_t"):])
        cfg = S.llama70b(rows=1, tokens=(t,))
        w = RightRotate(name, f"latency per call: online rotation of {t}x28672 fp16 "
                        "activations, HARP (7,16,16,16)", cfg["right"], cfg["acts"][t], "f16",
                        latency=True)
        w.workload = f"decode_{t}x28672_f16_(7,16,16,16)"
        w._cpu_rows = t
        return w
    if name.startswith("qlinear_t"):
        t = int(name[len("qlinear_t"):])
        w = DecodeLinear(name, f"latency per call: quantized 70B down projection at decode, {t} "
                         "tokens (rotate, 2-bit g64 product, unrotate)", t)
        w.workload = f"qlinear_{t}x28672_f16_w8192x28672_absmax2_g64_(32,16,16)x(7,16,16,16)"
        return w
    if name == "polar_requant":
        w = PolarRequant(name, "HBM GB/s: PolarQuant Q5 -> restore -> absmax INT4 g128 in one "
                         "pass, 7 projections (hidden 4096, FFN 12288)")
        w.workload = "polar_requant_7proj_4096_12288_q5_h128_to_absmax4_g128"
        w._cpu_rows = 512
        return w
    if name == "harp_build":
        w = HarpBuild(name, "latency: HARP blocks from int8 parameters (Cayley / Givens times "
                      "the base mixer), 70B schedules U (32,16,16) d=8192 + V (7,16,16,16) "
                      "d=28672", [(8192, (32, 16, 16)), (28672, (7, 16, 16, 16))])
        w.workload = "harp_build_70b_U(32,16,16)_d8192_V(7,16,16,16)_d28672_int8"
        return w
    if name in ("orp_geo", "orp_geo_dequant"):
        dq = name == "orp_geo_dequant"
        w = OrpGeo(name, "HBM GB/s: ORP GEO " + ("dequantize" if dq else "quantize") +
                   " (power-of-two + orthogonal residual basis, 3-bit, g128, stride 4), "
                   "4096x4096 bf16", dq)
        w.workload = f"{name}_7b_4096x4096_bf16_b3_g128_s4"
        w._cpu_rows = 1024
        return w
    if name in ("polar_quant", "polar_dequant"):
        dq = name == "polar_dequant"
        w = PolarBlock(name, ("HBM GB/s: PolarQuant dequant+unrotate" if dq else
                              "HBM GB/s: PolarQuant rotate+quantize+pack")
                       + ", 7 projections (hidden 4096, FFN 12288) bf16, H128, 4-bit codebook",
                       dq)
        w.workload = f"{name}_7proj_4096_12288_bf16_h128_codebook4_g128"
        w._cpu_rows = 1024
        return w
    raise SystemExit(f"unknown workload {name!r}")


WORKLOADS = ("harp_mlp", "llama7b_weight", "llama7b_act", "polar_quant", "polar_dequant",
             "llama70b_weight", "decode_t1", "decode_t16", "decode_t256", "harp_build",
             "polar_requant", "qlinear_t1", "qlinear_t16", "qlinear_t256", "orp_geo",
             "orp_geo_dequant")


def _pct(vals, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(vals, dtype=float), q)), 5)


def time_steps(wl, steps, torch, stream, step=None):
    """Per-step durations (ms) of `steps` consecutive steps, from HIP events
    recorded between the steps on the launch stream; no per-launch events."""
    step = step or wl.step
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(steps):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]) / steps, per


def graph_latency(wl, steps, warmup, torch):
    """Per-call latency of the warm call replayed from a graph captured once
    (the call's kernels and arguments; a replay saves the host launch path
    and the gaps between dependent launches).  The hot calls only launch
    kernels on the given stream, which makes them capturable."""
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            wl.step_warm(0, stream=s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            wl.step_warm(0, stream=s)
        torch.cuda.synchronize()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record(cur)
        for i in range(steps):
            g.replay()
            evs[i + 1].record(cur)
        torch.cuda.synchronize()
        per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
        del g
        return {"median": _pct(per, 50), "p10": _pct(per, 10), "p90": _pct(per, 90)}
    except Exception as e:  # a failed capture leaves the line without the figure
        return {"error": str(e)[:160]}


def stream_copy_gbs(torch, dev, mib=1024, reps=10):
    """A plain device-to-device copy of `mib` MiB (torch's copy kernel):
    bytes read + written per second, the practical HBM ceiling."""
    src = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * mib * (1 << 20) / (ms * 1e-3) / 1e9, 1)


def host_description():
    """CPU model, logical CPUs in the affinity mask, and numpy's BLAS with the
    threads its pool runs (what the oracle's matrix products use)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        for info in threadpool_info():
            if info.get("user_api") == "blas":
                blas = f"{info.get('internal_api')} {info.get('version')}"
                threads = info.get("num_threads")
                break
    except Exception:
        pass
    return {"cpu_model": model, "cpus_in_mask": len(os.sched_getaffinity(0)), "blas": blas,
            "blas_threads": threads}


def run_workload(wl, a, brq, torch, dev, stream, copy_gbs=None):
    wl.setup(brq, dev, stream)
    if a.copy_calibration:
        nel = a.copy_calibration * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(a.warmup):
        wl.step(i)
    torch.cuda.synchronize()
    # The timed region runs with per-launch profiling off; each step is
    # bracketed by events on the launch stream, which give the median and
    # p10/p90.  Per-kernel durations come from a second run of the same steps
    # with an event pair around every launch.
    brq.profile_enable(False)
    ms, per = time_steps(wl, a.steps, torch, stream)
    brq.profile_reset()
    brq.profile_enable(True)
    for i in range(a.steps):
        wl.step(i)
    torch.cuda.synchronize()
    brq.profile_enable(False)
    kernels = brq.profile_read()
    names = list(kernels)
    wl._first_kernel, wl._last_kernel = names[0], names[-1]
    warm = graph = None
    if getattr(wl, "step_warm", None) is not None:
        for i in range(a.warmup):
            wl.step_warm(i)
        _, wper = time_steps(wl, a.steps, torch, stream, wl.step_warm)
        warm = {"median": _pct(wper, 50), "p10": _pct(wper, 10), "p90": _pct(wper, 90)}
        graph = graph_latency(wl, a.steps, a.warmup, torch)

    value = wl.value(ms)
    alg = wl.alg_bytes()
    dom_name, (dom_ms, dom_n) = max(kernels.items(), key=lambda kv: kv[1][0])
    kb, kf, engine = wl.kernel_cost(dom_name)
    bound, work, unit, peak = roofline_of(kb, kf, engine)
    avg_ms = dom_ms / max(dom_n, 1)
    achieved = work / (avg_ms * 1e-3)
    cfg = {"workload": wl.workload}
    cfg.update(wl.config())
    cfg.update({
        "algorithmic_bytes": alg,
        "hbm_gbs": round(alg / (ms * 1e-3) / 1e9, 3),
        "hbm_peak_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
        "step_ms": {"mean": round(ms, 5), "median": _pct(per, 50), "p10": _pct(per, 10),
                    "p90": _pct(per, 90)},
        "kernels_ms_per_step": {k: round(v[0] / a.steps, 5) for k, v in kernels.items()},
        "launches_per_step": {k: v[1] / a.steps for k, v in kernels.items()},
    })
    if warm is not None:
        cfg["step_ms_warm"] = warm
        cfg["step_ms_cold"] = cfg["step_ms"]
        cfg["step_ms_graph"] = graph
    if copy_gbs is not None:
        cfg["stream_copy_gbs"] = copy_gbs
        cfg["hbm_frac_of_copy"] = round(alg / (ms * 1e-3) / 1e9 / copy_gbs, 5)
    cfg["elements_per_s"] = round(wl.elements() / (ms * 1e-3), 1)
    line = {
        "metric": wl.metric,
        "value": round(value, 3),
        "unit": wl.unit,
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": wl.higher_is_better,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": cfg,
        "roofline": {
            "bound": bound,
            "kernel": dom_name,
            "achieved": round(achieved, 4),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 5),
            "traffic": measured_traffic(wl.name, dom_name),
            "algorithmic_bytes": kb,
            "algorithmic_flops": kf,
            "avg_launch_ms": round(avg_ms, 5),
        },
    }
    if not a.no_cpu_baseline:
        cb = wl.cpu_baseline(None)
        if cb is not None:
            cb.update(host_description())
        line["cpu_baseline"] = cb
        par = getattr(wl, "parity_sample", None)
        if par is not None:
            line["parity"] = par()
    print(json.dumps(line), flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="harp_mlp", choices=WORKLOADS + ("all",))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="oracle sample size in rows (0: the workload's default)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device-to-device copy of MIB MiB (3 times) before the "
                         "steps, as the reference kernel for HBM byte counters")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the path needs no "
              "collectives and multi-GPU runs are out of scope here.", file=sys.stderr)
        return 2

    import torch

    import butterfly_rotation_quantization_amd as brq

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    names = WORKLOADS if a.workload == "all" else (a.workload,)
    copy_gbs = stream_copy_gbs(torch, dev)
    for name in names:
        wl = make_workload(name)
        if a.cpu_rows:
            wl._cpu_rows = a.cpu_rows
        run_workload(wl, a, brq, torch, dev, stream, copy_gbs)
        del wl
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
