"""Oracle: group quantizers, decision bands and bit packing.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Absmax ([PolarQuant] section 1: a linear map that assumes the values are
uniform on [-alpha, alpha]).  Reading: the interval is mapped onto the whole
code range, endpoints to endpoints, so all L = 2^bits codes are used:

    alpha = max |v| over the group,  h = (L - 1) / 2,
    code  = clamp(rint(h * v / alpha + h), 0, L - 1)   (rint: half to even),
    v_hat = alpha * (code / h - 1).

A group with alpha = 0 gets codes 0 and scale 0 (reading).

Norm-scaled codebook ([PolarQuant] section 2): per block of g values,
r = ||v||_2, z = sqrt(g) * v / r, code = index of the nearest centroid of a
Gaussian codebook (searched through midpoint thresholds, a tie going to the
lower index), stored scale = fp16(r), v_hat = r16 * c[code] / sqrt(g).  The
rotation before it is the Walsh-Hadamard block transform, applied by the
transform oracle.

Decisions.  The hot path takes each code decision in float32; the
``decide_f32`` mode below does the same from float32 inputs, so two sides that
agree on v agree on the code.  Elements whose exact value lies within 1e-6 (relative, in the
quantizer's normalised domain) of a decision threshold form the "band"; there
either neighbouring code is accepted, and the band size is reported.

Packing (reading of "packed codes"): within a row, code k occupies bits
[k*bits, (k+1)*bits) of a little-endian bit stream: stream bit p is bit
(p mod 8) of byte p // 8.
"""

from __future__ import annotations

import numpy as np

BAND_REL = 1e-6


# ---------------------------------------------------------------- absmax

def _groups(v: np.ndarray, g: int) -> np.ndarray:
    v = np.asarray(v)
    m, n = v.shape
    if n % g:
        raise ValueError("group size must divide the row length")
    return v.reshape(m, n // g, g)


def absmax_scales(v: np.ndarray, g: int) -> np.ndarray:
    """alpha = max |v| of every contiguous group of g along a row, float64."""
    return np.abs(_groups(np.asarray(v, dtype=np.float64), g)).max(axis=2)


def absmax_quantize(v: np.ndarray, bits: int, g: int, decide_f32: bool = True):
    """Codes [m, n] (uint8) and alpha [m, n/g].

    decide_f32=True evaluates the decision in float32 from float32(v): alpha
    in float32, k = fl32(h / alpha), t = fl32(v * k + h) (the product of two
    float32 numbers is exact in float64; the sum is rounded to float64, then
    to float32), code = rint(t).
    decide_f32=False evaluates the same formula in float64.
    """
    lv = (1 << bits) - 1
    h = lv / 2.0
    if decide_f32:
        v32 = _groups(np.asarray(v, dtype=np.float32), g)
        alpha = np.abs(v32).max(axis=2)  # exact in float32
        with np.errstate(divide="ignore"):
            k = (np.float32(h) / alpha).astype(np.float32)
        k = np.where(alpha > 0, k, np.float32(0))
        t = (v32.astype(np.float64) * k.astype(np.float64)[..., None] + h).astype(np.float32)
        t = t.astype(np.float64)
        alpha_out = alpha.astype(np.float64)
    else:
        vg = _groups(np.asarray(v, dtype=np.float64), g)
        alpha_out = np.abs(vg).max(axis=2)
        with np.errstate(divide="ignore", invalid="ignore"):
            t = np.where(alpha_out[..., None] > 0, h * vg / alpha_out[..., None] + h, 0.0)
    code = np.clip(np.rint(t), 0, lv)
    code = np.where(alpha_out[..., None] > 0, code, 0)
    m = code.shape[0]
    return code.reshape(m, -1).astype(np.uint8), alpha_out


def absmax_dequant(codes: np.ndarray, alpha: np.ndarray, bits: int, g: int) -> np.ndarray:
    """v_hat = alpha * (code / h - 1), float64."""
    h = ((1 << bits) - 1) / 2.0
    c = _groups(np.asarray(codes, dtype=np.float64), g)
    a = np.asarray(alpha, dtype=np.float64)[..., None]
    return (a * (c / h - 1.0)).reshape(c.shape[0], -1)


def absmax_band(v: np.ndarray, bits: int, g: int, rel: float = BAND_REL) -> np.ndarray:
    """Boolean [m, n]: u = v/alpha lies within rel*max(|tau_k|, 2/(L-1)) of a
    threshold tau_k = -1 + (2k+1)/(L-1), k = 0..L-2 (exact float64 v)."""
    lv = (1 << bits) - 1
    vg = _groups(np.asarray(v, dtype=np.float64), g)
    a = np.abs(vg).max(axis=2)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(a > 0, vg / a, 0.0)
    tau = -1.0 + (2.0 * np.arange(lv) + 1.0) / lv
    width = rel * np.maximum(np.abs(tau), 2.0 / lv)
    dist = np.abs(u[..., None] - tau) - width
    band = (dist <= 0).any(axis=-1) & (a > 0)
    return band.reshape(vg.shape[0], -1)


# ---------------------------------------------------------------- codebook

def thresholds_f32(centroids: np.ndarray) -> np.ndarray:
    """Midpoints of consecutive float32 centroids, evaluated in float32."""
    c = np.asarray(centroids, dtype=np.float32)
    return ((c[:-1] + c[1:]) * np.float32(0.5)).astype(np.float32)


def codebook_norm_quantize(v: np.ndarray, centroids: np.ndarray, g: int,
                           decide_f32: bool = True):
    """Codes [m, n], norms r [m, n/g] (float64) and z [m, n] (float64).

    Float32 decision: r32 = fl32(sqrt(sum v^2)) from float32 v,
    z32 = fl32(v * fl32(sqrt(g) / r32)), code = #{k : z32 > tau_k} with
    float32 thresholds.  Float64 decision: the same in float64.
    """
    cb = np.asarray(centroids, dtype=np.float32)
    vg64 = _groups(np.asarray(v, dtype=np.float64), g)
    r64 = np.sqrt((vg64 * vg64).sum(axis=2))
    with np.errstate(divide="ignore", invalid="ignore"):
        z64 = np.where(r64[..., None] > 0, np.sqrt(g) * vg64 / r64[..., None], 0.0)
    if decide_f32:
        v32 = _groups(np.asarray(v, dtype=np.float32), g)
        r32 = np.sqrt((v32.astype(np.float64) ** 2).sum(axis=2)).astype(np.float32)
        with np.errstate(divide="ignore"):
            k = (np.float32(np.sqrt(np.float32(g))) / r32).astype(np.float32)
        k = np.where(r32 > 0, k, np.float32(0))
        z = (v32.astype(np.float64) * k.astype(np.float64)[..., None]).astype(np.float32)
        tau = thresholds_f32(cb)
        code = (z[..., None] > tau).sum(axis=-1)
        code = np.where(r32[..., None] > 0, code, 0)
    else:
        tau = (cb[:-1].astype(np.float64) + cb[1:].astype(np.float64)) / 2.0
        code = (z64[..., None] > tau).sum(axis=-1)
        code = np.where(r64[..., None] > 0, code, 0)
    m = vg64.shape[0]
    return code.reshape(m, -1).astype(np.uint8), r64, z64.reshape(m, -1)


def nearest_centroid(z: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """Brute-force argmin_k |z - c_k|, ties to the lower index (check of the
    threshold search)."""
    c = np.asarray(centroids, dtype=np.float64)
    d = np.abs(np.asarray(z, dtype=np.float64)[..., None] - c)
    return d.argmin(axis=-1)


def codebook_dequant(codes: np.ndarray, norms16: np.ndarray, centroids: np.ndarray,
                     g: int) -> np.ndarray:
    """v_hat = r16 * c[code] / sqrt(g), float64."""
    c = np.asarray(centroids, dtype=np.float32).astype(np.float64)
    cg = _groups(np.asarray(codes), g)
    r = np.asarray(norms16, dtype=np.float16).astype(np.float64)[..., None]
    return (r * c[cg] / np.sqrt(g)).reshape(cg.shape[0], -1)


def codebook_band(z: np.ndarray, centroids: np.ndarray, rel: float = BAND_REL) -> np.ndarray:
    """Boolean: z within rel*max(|tau_k|, smallest centroid gap) of a threshold."""
    c = np.asarray(centroids, dtype=np.float32).astype(np.float64)
    tau = (c[:-1] + c[1:]) / 2.0
    gap = np.min(np.diff(c))
    width = rel * np.maximum(np.abs(tau), gap)
    return (np.abs(np.asarray(z, dtype=np.float64)[..., None] - tau) <= width).any(axis=-1)


# ---------------------------------------------------------------- packing

def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """LSB-first bit stream per row: [m, n] codes -> [m, n*bits/8] bytes."""
    c = np.asarray(codes, dtype=np.uint64)
    m, n = c.shape
    if (n * bits) % 8:
        raise ValueError("row bit length must be a whole number of bytes")
    if c.size and c.max() >= (1 << bits):
        raise ValueError("code out of range")
    bitplane = ((c[..., None] >> np.arange(bits, dtype=np.uint64)) & 1).astype(np.uint8)
    stream = bitplane.reshape(m, n * bits)
    return np.packbits(stream, axis=1, bitorder="little")


def unpack(packed: np.ndarray, bits: int, n: int) -> np.ndarray:
    """Inverse of pack: [m, n*bits/8] bytes -> [m, n] codes (uint8)."""
    p = np.asarray(packed, dtype=np.uint8)
    stream = np.unpackbits(p, axis=1, bitorder="little")[:, : n * bits]
    planes = stream.reshape(p.shape[0], n, bits).astype(np.uint32)
    return (planes << np.arange(bits, dtype=np.uint32)).sum(axis=2).astype(np.uint8)
