"""Oracle: HARP blocks from their parameters, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed ([HARP] section 2.2): every block of a stage is a learnable
orthogonal factor times a fixed base mixer, B_{t,c}(theta) = Q_{t,c}(theta) G_{b_t}.
Q is a Givens rotation when b_t = 2 and the Cayley map of a skew-symmetric
matrix when b_t > 2; G is the normalised Sylvester Hadamard matrix for a power
of two and a QR fallback otherwise ([HARP] section 2.1).  All parameters start
at zero, where Q = I and B = G, so the transform starts out as the RHT.  The
parameters may be stored as int8 ([HARP] section 2.4).

Readings (the pages name the maps but give no formulas or layouts):

* Cayley map: Q = (I - A)^{-1} (I + A) with A skew-symmetric (the textbook
  form; (I + A)(I - A)^{-1} is the same matrix because the factors commute).
* A from theta: b(b-1)/2 parameters per block, the strict upper triangle in
  row-major order, A[i][j] = theta[p(i, j)] for i < j and A[j][i] = -A[i][j],
  with p(i, j) = i*b - i*(i+1)/2 + (j - i - 1).
* Givens: one parameter per block, Q = [[cos theta, -sin theta],
  [sin theta, cos theta]].
* int8 storage: theta = s_t * q with q an int8 in [-127, 127] and one float32
  scale s_t per stage.
* Layout of a side's parameters: stage by stage, group c by group c (c as in
  the index reading of ``transform``), each group's parameters contiguous.
* G for a radix that is not a power of two is given by the caller (the QR
  fallback of a seeded Gaussian matrix, ``transform.base_mixer``).
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from . import transform as T


def n_params(b: int) -> int:
    """Parameters of one block: 1 for a Givens rotation (b = 2), b(b-1)/2 for
    the Cayley map (b > 2)."""
    return 1 if b == 2 else b * (b - 1) // 2


def skew(theta: np.ndarray, b: int) -> np.ndarray:
    """Skew-symmetric A (b x b) from the strict upper triangle, row-major."""
    theta = np.asarray(theta, dtype=np.float64).reshape(-1)
    if theta.size != b * (b - 1) // 2:
        raise ValueError("a b x b skew matrix has b(b-1)/2 parameters")
    a = np.zeros((b, b))
    iu = np.triu_indices(b, k=1)  # row-major order of the strict upper triangle
    a[iu] = theta
    return a - a.T


def givens(theta: float) -> np.ndarray:
    """Q for b = 2: rotation by theta."""
    c, s = np.cos(theta), np.sin(theta)
    return np.array([[c, -s], [s, c]])


def cayley(theta: np.ndarray, b: int) -> np.ndarray:
    """Q for b > 2: (I - A)^{-1} (I + A).  I - A is invertible for any real
    skew A (its eigenvalues are 1 - i*lambda)."""
    a = skew(theta, b)
    eye = np.eye(b)
    return np.linalg.solve(eye - a, eye + a)


def q_block(theta: np.ndarray, b: int) -> np.ndarray:
    """The learnable orthogonal factor of one block ([HARP] section 2.2)."""
    theta = np.asarray(theta, dtype=np.float64).reshape(-1)
    if b == 2:
        if theta.size != 1:
            raise ValueError("a Givens block has one parameter")
        return givens(float(theta[0]))
    return cayley(theta, b)


def dequant_theta(q: np.ndarray, scale: float) -> np.ndarray:
    """int8 storage ([HARP] section 2.4): theta = scale * q, q in [-127, 127]."""
    q = np.asarray(q)
    if q.dtype != np.int8 or (q == -128).any():
        raise ValueError("parameters are int8 in [-127, 127]")
    return float(np.float32(scale)) * q.astype(np.float64)


def stage_blocks(b: int, ngroups: int, theta_q: np.ndarray, scale: float,
                 base: Optional[np.ndarray] = None) -> np.ndarray:
    """(ngroups, b, b) blocks Q(theta_c) G of one stage.  theta_q holds the
    int8 parameters group by group; base is G (b x b), None for the normalised
    Sylvester matrix (powers of two)."""
    g = T.base_mixer(b) if base is None else np.asarray(base, dtype=np.float64).reshape(b, b)
    npar = n_params(b)
    th = dequant_theta(np.asarray(theta_q).reshape(ngroups, npar), scale)
    out = np.empty((ngroups, b, b))
    for c in range(ngroups):
        out[c] = q_block(th[c], b) @ g
    return out


def harp_plan(d: int, radix: Sequence[int], theta_q: np.ndarray, scales: Sequence[float],
              bases: Optional[Sequence[Optional[np.ndarray]]] = None,
              signs: Optional[np.ndarray] = None) -> T.Plan:
    """A per-group plan whose blocks come from int8 parameters (layout in the
    module docstring); bases[t] is G of stage t (None: Sylvester)."""
    radix = tuple(int(b) for b in radix)
    theta_q = np.asarray(theta_q).reshape(-1)
    blocks: List[np.ndarray] = []
    off = 0
    for t, b in enumerate(radix):
        ng = d // b
        cnt = ng * n_params(b)
        base = None if bases is None else bases[t]
        blocks.append(stage_blocks(b, ng, theta_q[off:off + cnt], scales[t], base))
        off += cnt
    if off != theta_q.size:
        raise ValueError("parameter count does not match the schedule")
    return T.Plan(d, radix, T.PER_GROUP, blocks, signs)


def total_params(d: int, radix: Sequence[int]) -> int:
    """Parameters of one side: sum over stages of (d / b_t) * n_params(b_t)."""
    return sum((d // int(b)) * n_params(int(b)) for b in radix)
