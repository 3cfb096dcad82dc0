"""Oracle: the quantized linear layer at decode time, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed ([HARP] section 2: the two-sided processor W' = M_U W M_V^T
with W' quantized; section 2.4 and the latency comparison: at inference the
activations are rotated online and multiplied by the stored quantized weight).
With W = M_U^T W' M_V, a layer Y = X W^T becomes

    X~ = X M_V^T             (online rotation of the activations, right plan)
    Z  = X~ W'^T             (the quantized weight: absmax-dequantized codes)
    Y  = Z M_U               (every row z becomes M_U^T z: the left plan's inverse)

Readings: the weight is the absmax-quantized W' of ``quant`` (codes and
float32 scales, groups along the input index); X~ is rounded to the
activation dtype before the product (the rotation writes it in that type);
either plan may be absent (identity).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import quant as Q
from . import transform as T


def weight(codes: np.ndarray, alpha: np.ndarray, bits: int, group: int) -> np.ndarray:
    """W'^ [m, n] in float64 from absmax codes and scales."""
    return Q.absmax_dequant(codes, alpha, bits, group)


def _method(p: T.Plan) -> str:
    return "dense" if p.d <= 4096 else "factored"


def rotate_acts(right: Optional[T.Plan], x: np.ndarray) -> np.ndarray:
    """X~ = X M_V^T (rows of x, block-diagonal when d < n)."""
    x = np.asarray(x, dtype=np.float64)
    return x if right is None else T.apply_right(right, x, method=_method(right))


def qlinear(left: Optional[T.Plan], right: Optional[T.Plan], x_tilde: np.ndarray,
            codes: np.ndarray, alpha: np.ndarray, bits: int, group: int):
    """Z = X~ W'^T and Y = Z M_U (rows z -> M_U^T z).  x_tilde is the rotated
    activation as the product sees it.  Returns (Y, Z)."""
    z = np.asarray(x_tilde, dtype=np.float64) @ weight(codes, alpha, bits, group).T
    y = z if left is None else T.apply_right(left, z, inverse=True, method=_method(left))
    return y, z
