"""Oracle: PolarQuant's downstream chain, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed ([PolarQuant] section 3, the downstream INT4 finding):
weights quantized with PolarQuant (block Walsh-Hadamard rotation, per-block
norm, Lloyd-Max codebook) are restored -- dequantized and rotated back -- and
the restored weights are quantized again with group absmax at 4 bits.  The
pages run the second quantizer from an external library; its formula is the
same absmax reading as ``quant`` (section 1 of the page).

Readings: the restored weights go to the second quantizer in float32 (the
chain is one pass here and never materialises them in a 16-bit type); the
second quantizer's groups are contiguous along a row, like the first's; the
restore uses the inverse of the same right-side plan (for PolarQuant the
block-128 Hadamard matrix, its own inverse).
"""

from __future__ import annotations

import numpy as np

from . import quant as Q
from . import transform as T


def restore(codes: np.ndarray, norms16: np.ndarray, centroids: np.ndarray, g_in: int,
            right: T.Plan) -> np.ndarray:
    """Dequantize the codebook-norm codes and apply the inverse right-side
    transform: the weights PolarQuant gives back, float64 [m, n]."""
    v = Q.codebook_dequant(codes, norms16, centroids, g_in)
    method = "dense" if right.d <= 4096 else "factored"
    return T.apply_right(right, v, inverse=True, method=method)


def requant(codes: np.ndarray, norms16: np.ndarray, centroids: np.ndarray, g_in: int,
            right: T.Plan, bits_out: int, g_out: int):
    """The chain: restore, then group absmax at bits_out with groups of g_out.
    Returns (codes_out, alpha_out, restored); decisions in float32 from the
    float32 restored values, as in ``quant.absmax_quantize``."""
    w = restore(codes, norms16, centroids, g_in, right)
    c, a = Q.absmax_quantize(w, bits_out, g_out)
    return c, a, w
