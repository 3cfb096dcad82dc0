"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module only draws random numbers and rounds them to storage types; it
holds none of the rotation or quantization arithmetic.  Every array it returns
is the one input both the HIP path and the oracle receive.

Generator: numpy PCG64 through ``SeedSequence(base).spawn(8)``; the child
streams are used in a fixed order: 0 values, 1 outlier columns, 2 signs of the
left side, 3 signs of the right side, 4 blocks of the left side (stage by
stage), 5 blocks of the right side (stage by stage), 6 activations.

Values are drawn in float64 and rounded to the storage type: float32 by
round-to-nearest-even, bfloat16 by rounding that float32 to nearest-even on
its top 16 bits, float16 by numpy's direct rounding.

Workloads (shapes of the layers the pages quantize; heavy tails and outlier
input channels as the pages describe weights and activations):

* ``tiny``      64 x 256 float32, N(0,1), 1% of the columns x20.
* ``llama7b``   4096 x 4096 bfloat16, 0.02 * Student-t(3), 0.5% of the
                columns x30; activations 2048 x 4096 bfloat16, N(0,1) with the
                same columns x30.
* ``harp_mlp``  4096 x 11008 bfloat16, 0.02 * Student-t(3), 0.5% columns x30.
* ``polar``     the 7 projections of one decoder block at hidden 4096 and FFN
                12288 (q, k, v, o 4096 x 4096; gate, up 12288 x 4096; down
                4096 x 12288), bfloat16, 0.02 * (N(0,1) with probability 0.99,
                N(0, 10^2) with probability 0.01).
* ``llama70b``  8192 x 28672 bfloat16, 0.02 * Student-t(3), 0.5% columns x30;
                decode activations T x 28672 float16 for T in {1, 16, 256}.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

STREAM_VALUES, STREAM_OUTLIERS, STREAM_SIGNS_U, STREAM_SIGNS_V = 0, 1, 2, 3
STREAM_BLOCKS_U, STREAM_BLOCKS_V, STREAM_ACT = 4, 5, 6


def streams(base_seed: int, n: int = 8) -> List[np.random.Generator]:
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(base_seed).spawn(n)]


# ---------------------------------------------------------------- storage rounding

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values -> stored array (float32, float16, or uint16 bf16 bits)."""
    if dtype == "f32":
        return np.asarray(x64, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x64, dtype=np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(np.asarray(x64, dtype=np.float32))
    raise ValueError(dtype)


def storage_to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------- draws

def outlier_columns(rng: np.random.Generator, n: int, frac: float) -> np.ndarray:
    k = int(round(frac * n))
    return np.sort(rng.choice(n, size=k, replace=False))


def signs(rng: np.random.Generator, d: int) -> np.ndarray:
    """Random +-1 vector as int8."""
    return np.where(rng.integers(0, 2, size=d) == 1, 1, -1).astype(np.int8)


def random_orthogonal(rng: np.random.Generator, b: int) -> np.ndarray:
    """A seeded random orthogonal b x b matrix: Q of the QR factorisation of a
    Gaussian matrix, column signs fixed so that R has a positive diagonal."""
    q, r = np.linalg.qr(rng.standard_normal((b, b)))
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return q * s[None, :]


def radix_blocks(rng: np.random.Generator, d: int, radix: Sequence[int],
                 per_group: bool = True, dtype=np.float32) -> List[np.ndarray]:
    """Random orthogonal blocks for every stage, rounded to ``dtype`` (the
    library takes float32 blocks): per_group -> (d/b_t, b_t, b_t) per stage,
    else (b_t, b_t)."""
    out = []
    for b in radix:
        if per_group:
            arr = np.stack([random_orthogonal(rng, b) for _ in range(d // b)])
        else:
            arr = random_orthogonal(rng, b)
        out.append(arr.astype(dtype))
    return out


def student_t_weights(rng: np.random.Generator, m: int, n: int, scale: float = 0.02,
                      nu: float = 3.0) -> np.ndarray:
    return scale * rng.standard_t(nu, size=(m, n))


def gaussian_mixture_weights(rng: np.random.Generator, m: int, n: int,
                             scale: float = 0.02, p_wide: float = 0.01,
                             wide_sigma: float = 10.0) -> np.ndarray:
    wide = rng.random((m, n)) < p_wide
    x = rng.standard_normal((m, n))
    return scale * np.where(wide, wide_sigma * x, x)


# ---------------------------------------------------------------- workloads

@dataclass
class SidePlan:
    """Arrays that define one side of a transform (inputs of both paths)."""
    d: int
    radix: tuple
    mode: str                       # "hadamard" | "shared" | "per_group"
    blocks: Optional[List[np.ndarray]] = None
    signs: Optional[np.ndarray] = None


def hadamard_side(rng: Optional[np.random.Generator], d: int, radix: Sequence[int],
                  with_signs: bool = True) -> SidePlan:
    return SidePlan(d, tuple(radix), "hadamard", None,
                    signs(rng, d) if with_signs else None)


def dense_side(rng_signs: Optional[np.random.Generator], rng_blocks: np.random.Generator,
               d: int, radix: Sequence[int], per_group: bool = True,
               with_signs: bool = True) -> SidePlan:
    return SidePlan(d, tuple(radix), "per_group" if per_group else "shared",
                    radix_blocks(rng_blocks, d, radix, per_group),
                    signs(rng_signs, d) if with_signs else None)


def tiny(seed: int = 1000) -> Dict:
    r = streams(seed)
    m, n = 64, 256
    x = r[STREAM_VALUES].standard_normal((m, n))
    cols = outlier_columns(r[STREAM_OUTLIERS], n, 0.01)
    x[:, cols] *= 20.0
    sv = signs(r[STREAM_SIGNS_V], n)
    return {
        "w": to_storage(x, "f32"), "dtype": "f32", "outliers": cols,
        "rht": SidePlan(n, (2,) * 8, "hadamard", None, sv),
        "harp": SidePlan(n, (4, 4, 16), "per_group",
                         radix_blocks(r[STREAM_BLOCKS_V], n, (4, 4, 16)), sv),
        "bits": 4, "group": 128,
    }


def llama7b(seed: int = 2000, rows: int = 4096, act_tokens: int = 2048) -> Dict:
    r = streams(seed)
    m = n = 4096
    w = student_t_weights(r[STREAM_VALUES], rows, n)
    cols = outlier_columns(r[STREAM_OUTLIERS], n, 0.005)
    w[:, cols] *= 30.0
    x = r[STREAM_ACT].standard_normal((act_tokens, n))
    x[:, cols] *= 30.0
    return {
        "w": to_storage(w, "bf16"), "dtype": "bf16", "outliers": cols,
        "left": hadamard_side(r[STREAM_SIGNS_U], m, (2,) * 12),
        "right": hadamard_side(r[STREAM_SIGNS_V], n, (2,) * 12),
        "x": to_storage(x, "bf16"),
        "bits": (2, 3, 4), "group": 128,
    }


def harp_mlp(seed: int = 3000, rows: int = 4096) -> Dict:
    r = streams(seed)
    m, n = 4096, 11008
    w = student_t_weights(r[STREAM_VALUES], rows, n)
    cols = outlier_columns(r[STREAM_OUTLIERS], n, 0.005)
    w[:, cols] *= 30.0
    return {
        "w": to_storage(w, "bf16"), "dtype": "bf16", "outliers": cols,
        "left": dense_side(r[STREAM_SIGNS_U], r[STREAM_BLOCKS_U], m, (16, 16, 16)),
        "right": dense_side(r[STREAM_SIGNS_V], r[STREAM_BLOCKS_V], n, (43, 16, 16)),
        "bits": 3, "group": 128,
    }


POLAR_SHAPES = {
    "q_proj": (4096, 4096), "k_proj": (4096, 4096), "v_proj": (4096, 4096),
    "o_proj": (4096, 4096), "gate_proj": (12288, 4096), "up_proj": (12288, 4096),
    "down_proj": (4096, 12288),
}


def polar(seed: int = 4000, names: Optional[Sequence[str]] = None,
          row_limit: Optional[int] = None) -> Dict:
    """The 7 projections (optionally a subset, optionally only the first
    row_limit rows of each: the draws for later rows are then not made)."""
    r = streams(seed)
    mats = {}
    for name, (m, n) in POLAR_SHAPES.items():
        rows = m if row_limit is None else min(m, row_limit)
        w = gaussian_mixture_weights(r[STREAM_VALUES], rows, n)
        if names is None or name in names:
            mats[name] = to_storage(w, "bf16")
    return {
        "mats": mats, "dtype": "bf16",
        "right": SidePlan(128, (2,) * 7, "hadamard", None, None),
        "bits": 4, "group": 128,
    }


def llama70b(seed: int = 5000, rows: int = 8192, tokens: Sequence[int] = (1, 16, 256)) -> Dict:
    r = streams(seed)
    m, n = 8192, 28672
    w = student_t_weights(r[STREAM_VALUES], rows, n)
    cols = outlier_columns(r[STREAM_OUTLIERS], n, 0.005)
    w[:, cols] *= 30.0
    acts = {}
    for t in tokens:
        x = r[STREAM_ACT].standard_normal((t, n))
        x[:, cols] *= 30.0
        acts[t] = to_storage(x, "f16")
    return {
        "w": to_storage(w, "bf16"), "dtype": "bf16", "outliers": cols,
        "left": dense_side(r[STREAM_SIGNS_U], r[STREAM_BLOCKS_U], m, (32, 16, 16)),
        "right": dense_side(r[STREAM_SIGNS_V], r[STREAM_BLOCKS_V], n, (7, 16, 16, 16)),
        "acts": acts, "bits": 2, "group": 64,
    }


def random_plan(rng: np.random.Generator, radix: Sequence[int], mode: str,
                with_signs: bool = True, dtype=np.float32) -> SidePlan:
    """A plan with the given radices for small parity cases."""
    d = int(np.prod(radix))
    s = signs(rng, d) if with_signs else None
    if mode == "hadamard":
        return SidePlan(d, tuple(radix), mode, None, s)
    return SidePlan(d, tuple(radix), mode,
                    radix_blocks(rng, d, radix, per_group=(mode == "per_group"),
                                 dtype=dtype), s)
