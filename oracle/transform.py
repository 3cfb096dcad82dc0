"""Oracle: the structured orthogonal transform, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed ([HARP] section 2.1): for a dimension d and a mixed-radix
schedule b = (b_0, ..., b_{m-1}) with prod(b) = d, stage t applies a
block-diagonal orthogonal matrix B_t whose b_t x b_t blocks act on groups of
coordinates that lie a fixed stride apart.  The rotation is the product of the
stages, preceded by the fixed random sign flip of the randomized Hadamard
transform ([HARP] section 1; section 2.2 says the learnable form starts out
equal to that transform, so it carries the same signs).

Readings (the pages name the stride permutation but not its indices):

* Index convention.  i = sum_t i_t * S_t with S_t = prod_{s>t} b_s, so digit 0
  is the most significant and the last stage has stride 1.  Stage t changes
  digit t only; its groups are {base + k*S_t : k < b_t}; the group index is
  c = hi*S_t + lo with hi = i // (b_t*S_t) and lo = i % S_t.
* Order.  M = B_{m-1} ... B_1 B_0 D, D = diag(signs): signs first, stage 0
  next.  With Hadamard blocks this gives H_d D / sqrt(d) exactly, so the
  "fixed permutation convention" of [HARP] section 2.2 is the identity.
* Blocks are indexed per group (B_{t,c}, the subscript c of [HARP] section
  2.2); a single block shared by all groups of a stage is a special case.
* Normalisation: the RHT is orthonormal, H_d D / sqrt(d) ([HARP] section 1
  calls it exactly orthogonal); Hadamard blocks are H_b / sqrt(b) ([HARP]
  section 2.2, "normalised Sylvester Hadamard").

Two-sided use ([HARP] section 2, "two-sided orthogonal processor"):
W' = M_U W M_V^T, with U acting on the row index (d = rows) and V on the
column index (d = cols, or a divisor of cols for a block-diagonal right side).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import scipy.sparse as sp

HADAMARD = "hadamard"
SHARED = "shared"
PER_GROUP = "per_group"


def strides(radix: Sequence[int]) -> List[int]:
    """S_t = product of the radices after stage t (digit 0 most significant)."""
    out = []
    for t in range(len(radix)):
        s = 1
        for b in radix[t + 1:]:
            s *= int(b)
        out.append(s)
    return out


def digits(i: int, radix: Sequence[int]) -> List[int]:
    """Mixed-radix digits (i_0, ..., i_{m-1}) of i, digit 0 most significant."""
    out = []
    for s, b in zip(strides(radix), radix):
        out.append((i // s) % b)
    return out


def sylvester(n: int) -> np.ndarray:
    """The +-1 Sylvester Hadamard matrix H_n (n a power of two), natural order:
    H_1 = [1], H_{2k} = [[H_k, H_k], [H_k, -H_k]]."""
    if n < 1 or n & (n - 1):
        raise ValueError("Sylvester Hadamard needs a power-of-two size")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def qr_orthogonal(g: np.ndarray) -> np.ndarray:
    """Deterministic orthogonal matrix from the QR factorisation of a given
    Gaussian matrix ([HARP] section 2.1: fallback mixer for radices that are
    not powers of two).  The sign of each column is fixed so that R has a
    positive diagonal, which makes Q a function of g alone."""
    q, r = np.linalg.qr(np.asarray(g, dtype=np.float64))
    sgn = np.sign(np.diag(r))
    sgn[sgn == 0] = 1.0
    return q * sgn[None, :]


def base_mixer(b: int, gaussian: Optional[np.ndarray] = None) -> np.ndarray:
    """G_b of [HARP] section 2.2: normalised Sylvester Hadamard H_b/sqrt(b) for a
    power of two, otherwise the QR fallback of a fixed Gaussian b x b matrix."""
    if b >= 1 and not (b & (b - 1)):
        return sylvester(b) / np.sqrt(b)
    if gaussian is None:
        raise ValueError("a non-power-of-two base mixer needs its Gaussian matrix")
    return qr_orthogonal(gaussian)


@dataclass
class Plan:
    """One side's transform.

    mode HADAMARD: every stage uses G_b = H_b/sqrt(b) (powers of two only).
    mode SHARED:   blocks[t] is one (b_t, b_t) matrix used by every group.
    mode PER_GROUP: blocks[t] is (d/b_t, b_t, b_t), indexed by group c.
    signs: None (all +1) or a length-d vector of +-1.
    """

    d: int
    radix: tuple
    mode: str = HADAMARD
    blocks: Optional[list] = None
    signs: Optional[np.ndarray] = None
    _dense: Optional[np.ndarray] = field(default=None, repr=False, compare=False)

    def __post_init__(self):
        self.radix = tuple(int(b) for b in self.radix)
        if int(np.prod(self.radix)) != self.d:
            raise ValueError("prod(radix) must equal d")
        if self.mode == HADAMARD:
            for b in self.radix:
                if b < 2 or b & (b - 1):
                    raise ValueError("Hadamard stages need power-of-two radices")
        elif self.mode not in (SHARED, PER_GROUP):
            raise ValueError("unknown mode")
        if self.signs is not None:
            self.signs = np.asarray(self.signs, dtype=np.float64).reshape(self.d)

    def stage_blocks(self, t: int) -> np.ndarray:
        """(d/b_t, b_t, b_t) float64 array of the blocks of stage t."""
        b = self.radix[t]
        ng = self.d // b
        if self.mode == HADAMARD:
            blk = base_mixer(b)
            return np.broadcast_to(blk, (ng, b, b))
        arr = np.asarray(self.blocks[t], dtype=np.float64)
        if self.mode == SHARED:
            return np.broadcast_to(arr.reshape(b, b), (ng, b, b))
        return arr.reshape(ng, b, b)

    def sign_vector(self) -> np.ndarray:
        return np.ones(self.d) if self.signs is None else self.signs


def stage_matrix(plan: Plan, t: int) -> sp.csr_matrix:
    """Stage t as a sparse d x d matrix: y[base + j*S] = sum_k B_{t,c}[j,k] x[base + k*S]
    for every group c ([HARP] section 2.1, block-diagonal B_t on stride-separated
    groups)."""
    b = plan.radix[t]
    s = strides(plan.radix)[t]
    blocks = plan.stage_blocks(t)
    rows, cols, vals = [], [], []
    for c in range(plan.d // b):
        hi, lo = divmod(c, s)
        base = hi * b * s + lo
        idx = base + s * np.arange(b)
        rows.append(np.repeat(idx, b))
        cols.append(np.tile(idx, b))
        vals.append(blocks[c].reshape(-1))
    return sp.csr_matrix(
        (np.concatenate(vals), (np.concatenate(rows), np.concatenate(cols))),
        shape=(plan.d, plan.d),
    )


def dense(plan: Plan) -> np.ndarray:
    """The explicit orthogonal matrix M = B_{m-1} ... B_0 D (cached on the plan)."""
    if plan._dense is None:
        m = np.diag(plan.sign_vector())
        for t in range(len(plan.radix)):
            m = stage_matrix(plan, t) @ m
        plan._dense = np.asarray(m)
    return plan._dense


def apply_factored(plan: Plan, x: np.ndarray, inverse: bool = False) -> np.ndarray:
    """Apply M (or M^T) to every length-d vector on the last axis of x by
    multiplying the factors of the definition one after another: D, then
    B_0, ..., B_{m-1} (inverse: B_{m-1}^T, ..., B_0^T, then D)."""
    x = np.asarray(x, dtype=np.float64)
    lead = x.shape[:-1]
    y = x.reshape(-1, plan.d).copy()
    st = strides(plan.radix)
    order = range(len(plan.radix))
    if not inverse:
        y *= plan.sign_vector()[None, :]
    else:
        order = reversed(list(order))
    for t in order:
        b, s = plan.radix[t], st[t]
        h = plan.d // (b * s)
        blk = plan.stage_blocks(t).reshape(h, s, b, b)
        v = y.reshape(-1, h, b, s)
        if not inverse:
            v = np.einsum("hljk,nhkl->nhjl", blk, v)
        else:
            v = np.einsum("hlkj,nhkl->nhjl", blk, v)
        y = v.reshape(-1, plan.d)
    if inverse:
        y = y * plan.sign_vector()[None, :]
    return y.reshape(*lead, plan.d)


def apply_right(plan: Plan, x: np.ndarray, inverse: bool = False,
                method: str = "dense") -> np.ndarray:
    """Right side: every row (or every d-chunk of a row, block-diagonal when
    cols > d) x becomes M x, i.e. Y = X M^T; inverse uses M^T."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    if cols % plan.d:
        raise ValueError("d must divide the row length")
    v = x.reshape(rows * (cols // plan.d), plan.d)
    if method == "factored":
        y = apply_factored(plan, v, inverse)
    else:
        m = dense(plan)
        y = v @ (m if inverse else m.T)
    return y.reshape(rows, cols)


def apply_left(plan: Plan, x: np.ndarray, inverse: bool = False,
               method: str = "dense") -> np.ndarray:
    """Left side: every column x becomes M x (Y = M X); inverse uses M^T."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[0] != plan.d:
        raise ValueError("left side needs d == rows")
    if method == "factored":
        return apply_factored(plan, x.T, inverse).T
    m = dense(plan)
    return (m.T if inverse else m) @ x


def two_sided(left: Optional[Plan], right: Optional[Plan], w: np.ndarray,
              method: str = "dense") -> np.ndarray:
    """W' = M_U W M_V^T ([HARP] section 2: two-sided processor); a missing
    side is the identity."""
    y = np.asarray(w, dtype=np.float64)
    if left is not None:
        y = apply_left(left, y, method=method)
    if right is not None:
        y = apply_right(right, y, method=method)
    return y


def two_sided_inverse(left: Optional[Plan], right: Optional[Plan], w: np.ndarray,
                      method: str = "dense") -> np.ndarray:
    """W = M_U^T W' M_V (the inverse of two_sided)."""
    y = np.asarray(w, dtype=np.float64)
    if right is not None:
        y = apply_right(right, y, inverse=True, method=method)
    if left is not None:
        y = apply_left(left, y, inverse=True, method=method)
    return y


def left_rows(plan: Plan, rows: np.ndarray) -> np.ndarray:
    """Selected rows of M (for checks on sampled output rows): M[r, :] = (M^T e_r)^T."""
    e = np.zeros((len(rows), plan.d))
    e[np.arange(len(rows)), rows] = 1.0
    return apply_factored(plan, e, inverse=True)
