"""Oracle: ORP's GEO mode, a two-basis power-of-two quantizer, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: [ORPQuant] "ORPQuant: geometric orthogonal residual projection for
multiplier-free power-of-two transformer quantization", technical summary,
section 2 ("geometric discrete basis search", "data-driven joint scaling",
GEO mode) and its hardware dataflow (a per-output-channel diagonal scale on
each of the two basis products).

For each vector w (a contiguous group of g inputs of one output row):

1. Preconditioning: w_p = w * s with a per-input-channel smoothing vector s
   (the page derives s from calibration statistics; here it is an input,
   and absent means all ones).
2. Primary basis: b1 = the point of an asymmetric power-of-two lattice with
   an exact zero state nearest to w_p / alpha, alpha = max |w_p|.
3. Residual: r = w_p - (<w_p, b1> / ||b1||^2) b1 (Gram-Schmidt).
4. Secondary basis: inside micro-blocks of 2S consecutive entries, entry i
   of the first half pairs with entry i + S (a local index exchange at
   stride S), and b2 takes the pair (b1[i], b1[i+S]) to
   sigma * (-b1[i+S], b1[i]) (a sign flip), so every pair of b2 is
   orthogonal to the same pair of b1, b2 is orthogonal to b1 exactly, and
   ||b2|| = ||b1||.  The sign sigma of each pair is the one that points b2
   along the residual: sigma = +1 if <r_pair, (-b1[i+S], b1[i])> >= 0,
   else -1.  Deterministic, one pass, O(N).
5. GEO scales: the least-squares coefficients of w_p on (b1, b2), which for
   orthogonal bases are c_i = <w_p, b_i> / ||b_i||^2.

Readings (the page leaves these open; each is the plainest one that fits
the rest of the page):

* The lattice at b bits has 2^b levels: zero, 2^(b-1) negative powers of
  two -1, -1/2, ..., -2^-(2^(b-1)-1) and 2^(b-1)-1 positive ones 1, 1/2,
  ..., 2^-(2^(b-1)-2) -- the page's 3-bit example runs from -1 through 0 to
  1 and calls the lattice asymmetric; the extra state goes to the negative
  side as in two's complement.  Codes index the levels in ascending order.
* "Nearest" is in value, a tie going to the lower code (as the codebook
  search does); the decision is taken in float32: u = fl(w_p * fl(1/alpha)),
  code = #{midpoints tau_k < u}.
* The sign of a pair depends on w_p only: the residual's component along
  (-b1[i+S], b1[i]) is d = w_p[i+S] b1[i] - w_p[i] b1[i+S] (the b1 part
  cancels); d = 0 takes sigma = +1.  Then <w_p, b2> = sum |d| over pairs.
* A group whose alpha is 0 gets the zero code everywhere and c1 = c2 = 0.
* Storage: codes LSB-first b-bit streams per row; one sign bit per pair
  (1 for sigma = -1), pairs numbered p = (i // 2S) * S + i % 2S by their
  first entry i, LSB-first per row (n/2 bits); (c1, c2) float32 per group.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

BAND_REL = 1e-6


def levels(bits: int) -> np.ndarray:
    """The asymmetric power-of-two lattice with zero, ascending (float64)."""
    if not 2 <= bits <= 5:
        raise ValueError("bits must be in 2..5")
    h = 1 << (bits - 1)
    neg = [-(2.0 ** -k) for k in range(h)]          # -1 ... -2^-(h-1)
    pos = [2.0 ** -k for k in range(h - 1)]          # 1 ... 2^-(h-2)
    return np.array(sorted(neg + [0.0] + pos))


def thresholds(bits: int) -> np.ndarray:
    """Midpoints of consecutive levels (exact in float32: sums of two powers
    of two, halved)."""
    lv = levels(bits)
    return (lv[:-1] + lv[1:]) / 2.0


def _groups(v: np.ndarray, g: int) -> np.ndarray:
    m, n = v.shape
    if n % g:
        raise ValueError("group size must divide the row length")
    return v.reshape(m, n // g, g)


def precondition(w: np.ndarray, smooth: Optional[np.ndarray]) -> np.ndarray:
    """w_p = w * s per input channel, rounded to float32 as the kernel forms
    it (one float32 product); s = None leaves w unchanged."""
    w = np.asarray(w, dtype=np.float64)
    if smooth is None:
        return w
    s32 = np.asarray(smooth, dtype=np.float32)
    return (w.astype(np.float32) * s32[None, :]).astype(np.float64)


def primary_codes(wp: np.ndarray, bits: int, g: int):
    """Codes of b1 [m, n] and alpha [m, n/g], deciding in float32 from the
    float32 w_p."""
    w32 = _groups(np.asarray(wp, dtype=np.float32), g)
    alpha = np.abs(w32).max(axis=2)
    with np.errstate(divide="ignore"):
        k = (np.float32(1.0) / alpha).astype(np.float32)
    k = np.where(alpha > 0, k, np.float32(0))
    u = (w32 * k[..., None]).astype(np.float32)
    tau = thresholds(bits).astype(np.float32)
    code = (u[..., None] > tau).sum(axis=-1)
    zero = int(np.flatnonzero(levels(bits) == 0.0)[0])
    code = np.where(alpha[..., None] > 0, code, zero)
    m = code.shape[0]
    return code.reshape(m, -1).astype(np.uint8), alpha.astype(np.float64)


def band(wp: np.ndarray, bits: int, g: int, rel: float = BAND_REL) -> np.ndarray:
    """Elements whose exact u = w_p / alpha lies within rel * max(|tau|,
    smallest level gap) of a decision threshold."""
    vg = _groups(np.asarray(wp, dtype=np.float64), g)
    a = np.abs(vg).max(axis=2)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(a > 0, vg / a, 0.0)
    tau = thresholds(bits)
    gap = np.diff(levels(bits)).min()
    width = rel * np.maximum(np.abs(tau), gap)
    hit = (np.abs(u[..., None] - tau) <= width).any(axis=-1) & (a > 0)
    return hit.reshape(vg.shape[0], -1)


def pair_index(n: int, stride: int):
    """(first, second) entry indices of every pair, in pair order p."""
    i = np.arange(n)
    first = i[(i % (2 * stride)) < stride]
    return first, first + stride


def secondary(wp: np.ndarray, b1: np.ndarray, stride: int):
    """b2 [m, n] and the pair signs sigma [m, n/2] (+1 / -1)."""
    wp = np.asarray(wp, dtype=np.float64)
    b1 = np.asarray(b1, dtype=np.float64)
    m, n = b1.shape
    f, s = pair_index(n, stride)
    d = wp[:, s] * b1[:, f] - wp[:, f] * b1[:, s]
    sigma = np.where(d >= 0, 1.0, -1.0)
    b2 = np.zeros_like(b1)
    b2[:, f] = -sigma * b1[:, s]
    b2[:, s] = sigma * b1[:, f]
    return b2, sigma


def geo_quantize(w: np.ndarray, bits: int, g: int, stride: int,
                 smooth: Optional[np.ndarray] = None):
    """GEO mode.  Returns codes [m, n] (b1 as indices into levels(bits)),
    sigma [m, n/2], coefficients [m, n/g, 2] = (c1, c2), and b1, b2, w_p."""
    if g % (2 * stride):
        raise ValueError("micro-blocks of 2*stride must tile the group")
    wp = precondition(w, smooth)
    codes, _alpha = primary_codes(wp, bits, g)
    b1 = levels(bits)[codes]
    b2, sigma = secondary(wp, b1, stride)
    m, n = wp.shape
    wg, b1g, b2g = _groups(wp, g), _groups(b1, g), _groups(b2, g)
    nn = (b1g * b1g).sum(axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        c1 = np.where(nn > 0, (wg * b1g).sum(axis=2) / nn, 0.0)
        c2 = np.where(nn > 0, (wg * b2g).sum(axis=2) / nn, 0.0)
    coef = np.stack([c1, c2], axis=-1)
    return codes, sigma, coef, b1, b2, wp


def basis_from_codes(codes: np.ndarray, sigma: np.ndarray, bits: int, stride: int):
    """(b1, b2) from stored codes and signs."""
    b1 = levels(bits)[np.asarray(codes)]
    f, s = pair_index(b1.shape[1], stride)
    b2 = np.zeros_like(b1)
    b2[:, f] = -sigma * b1[:, s]
    b2[:, s] = sigma * b1[:, f]
    return b1, b2


def geo_dequant(codes: np.ndarray, sigma: np.ndarray, coef: np.ndarray, bits: int, g: int,
                stride: int) -> np.ndarray:
    """w_p^ = c1 b1 + c2 b2 (in the preconditioned domain), float64."""
    b1, b2 = basis_from_codes(codes, sigma, bits, stride)
    c = np.asarray(coef, dtype=np.float64)
    m = b1.shape[0]
    out = c[..., 0:1] * _groups(b1, g) + c[..., 1:2] * _groups(b2, g)
    return out.reshape(m, -1)


def pack_signs(sigma: np.ndarray) -> np.ndarray:
    """One bit per pair, 1 for sigma = -1, LSB-first per row."""
    bits = (np.asarray(sigma) < 0).astype(np.uint8)
    return np.packbits(bits, axis=1, bitorder="little")


def unpack_signs(packed: np.ndarray, npairs: int) -> np.ndarray:
    b = np.unpackbits(np.asarray(packed, dtype=np.uint8), axis=1, bitorder="little")[:, :npairs]
    return np.where(b == 1, -1.0, 1.0)
