"""Comparison rules between the HIP path and the oracle (test helper).

* float32 output: max |y - y_ref| / ||row of y_ref||_2 <= 2e-5.
* bfloat16 / float16 output: |y - y_ref| <= 1 ulp of the storage type at
  |y_ref| + 1e-6 * ||row of y_ref||_2.  The kernels compute in float32 and
  round once; the second term is what that float32 arithmetic needs (its
  measured error is a few 1e-8 of the row norm), so a value far below the row
  norm is still held to about one ulp, and a second rounding or a dropped
  small term fails.
* codes: equal except where the exact value is within the decision band
  (1e-6 relative of a threshold).  Every mismatch must lie in the band, the
  mismatches must number <= max(1e-5 * N, 4), and for N >= 1e6 the band's own
  population must be <= 1e-5 * N (the cap is stated on the band; below 1e6
  elements its count is a handful of elements, too few to be a fraction).
  The population cap applies to quantizers of at most 4 bits (absmax at 2, 3
  and 4 bits and the 4-bit codebook); at 5 bits there are 31 thresholds and
  a band of 1e-6 relative width around each holds about 1e-5 of
  Gaussian-like data by itself, whatever computed the codes, so there the
  count is recorded and the mismatch rules alone are asserted.
* absmax scales: within 2e-5 * row norm; float16 norms within 1 fp16 ulp.

Every code comparison appends its counts (elements, band, mismatches) to a
JSON-lines record, ``$BRQ_PARITY_RECORD`` or ``gpurun_out/parity_records.jsonl``
under the repository root, so the counts outlive pytest's captured output.
"""

from __future__ import annotations

import json
import os
import time

import numpy as np

ROT_TOL = 2e-5
F32_ROUNDING_TOL = 1e-6
BAND_FRAC = 1e-5
BAND_CAP_MIN_ELEMENTS = 1_000_000
BAND_CAP_MAX_BITS = 4

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def record_path() -> str:
    return os.environ.get("BRQ_PARITY_RECORD",
                          os.path.join(_ROOT, "gpurun_out", "parity_records.jsonl"))


def record(entry: dict) -> None:
    """Append one parity record (best effort: a read-only tree skips it)."""
    path = record_path()
    try:
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "a") as f:
            f.write(json.dumps(dict(entry, time=time.strftime("%Y-%m-%dT%H:%M:%S"))) + "\n")
    except OSError:
        pass


def row_norms(y_ref: np.ndarray) -> np.ndarray:
    return np.linalg.norm(np.asarray(y_ref, dtype=np.float64), axis=1)


def ulp(x: np.ndarray, mant_bits: int) -> np.ndarray:
    """Spacing of a float with `mant_bits` stored mantissa bits at |x|."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 1e-300)))
    return np.exp2(e - mant_bits)


def check_rotation(y: np.ndarray, y_ref: np.ndarray, dtype: str, what: str = "") -> dict:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    nrm = row_norms(y_ref)[:, None]
    nrm = np.where(nrm > 0, nrm, 1.0)
    err = np.abs(y - y_ref)
    rel = float((err / nrm).max()) if y.size else 0.0
    info = {"max_rel_err": rel}
    if dtype == "f32":
        assert rel <= ROT_TOL, f"{what}: float32 rotation error {rel:.3g} > {ROT_TOL}"
        return info
    mant = 7 if dtype == "bf16" else 10
    u = ulp(y_ref, mant)
    tol = u + F32_ROUNDING_TOL * nrm
    bad = err > tol
    info["beyond_one_ulp"] = int((err > u).sum())
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond 1 {dtype} ulp + "
                           f"{F32_ROUNDING_TOL:g} of the row norm; worst "
                           f"{float((err / tol).max()):.3g}x")
    return info


def check_codes(codes: np.ndarray, codes_ref: np.ndarray, band: np.ndarray, what: str = "",
                bits: int = 0) -> dict:
    codes = np.asarray(codes)
    codes_ref = np.asarray(codes_ref)
    mism = codes != codes_ref
    outside = mism & ~band
    n = codes.size
    nb = int(band.sum())
    nm = int(mism.sum())
    info = {"mismatches": nm, "band": nb, "elements": n,
            "band_frac": nb / n if n else 0.0, "mismatch_frac": nm / n if n else 0.0}
    record(dict(info, case=what, bits=bits, outside_band=int(outside.sum())))
    assert not outside.any(), (f"{what}: {int(outside.sum())} code mismatches outside the "
                               f"band (of {nm} mismatches)")
    cap = max(BAND_FRAC * n, 4.0)
    assert nm <= cap, f"{what}: {nm} in-band mismatches > {cap:.3g}"
    if n >= BAND_CAP_MIN_ELEMENTS and bits <= BAND_CAP_MAX_BITS:
        assert nb <= BAND_FRAC * n, (f"{what}: the decision band holds {nb} of {n} elements "
                                     f"({nb / n:.3g} > {BAND_FRAC:g})")
    return info


def check_absmax_scales(alpha: np.ndarray, alpha_ref: np.ndarray, y_ref: np.ndarray,
                        what: str = "") -> float:
    nrm = row_norms(y_ref)[:, None]
    rel = float((np.abs(np.asarray(alpha, np.float64) - alpha_ref) / np.maximum(nrm, 1e-300)).max())
    assert rel <= ROT_TOL, f"{what}: scale error {rel:.3g} of the row norm"
    return rel


def check_f16_norms(r16: np.ndarray, r_ref: np.ndarray, what: str = "") -> int:
    ref16 = np.asarray(r_ref, dtype=np.float16).astype(np.float64)
    got = np.asarray(r16, dtype=np.float16).astype(np.float64)
    tol = ulp(ref16, 10)
    bad = np.abs(got - ref16) > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} norms beyond 1 fp16 ulp"
    return int((got != ref16).sum())


def gamma_tilde(p: int, lam: float = 8.0) -> float:
    """Probabilistic rounding-error constant of a sum whose terms each pass
    through at most p float32 roundings (Higham and Mary, "A new approach to
    probabilistic rounding error analysis", SIAM J. Sci. Comput. 41 (2019)):
    |error| <= gamma~_p(lam) * sum |terms| with probability at least
    1 - 2 exp(-lam^2 (1 - u)^2 / 2), gamma~_p(lam) = exp(lam sqrt(p) u +
    p u^2 / (1 - u)) - 1, u = 2^-24.  lam = 8 puts the failure probability
    of one element below 3e-14."""
    u = 2.0 ** -24
    return float(np.expm1(lam * np.sqrt(p) * u + p * u * u / (1.0 - u)))


def quantized_dot_path(n: int, group: int) -> int:
    """Roundings along the longest path of a group-blocked quantized dot
    product: up to `group` additions inside a group, one for the group's
    scale, then at most n/group + 2 additions across groups, however the
    groups are split and the parts summed."""
    return group + n // group + 3


def check_quantized_dot(z: np.ndarray, z_ref: np.ndarray, s_abs: np.ndarray, p: int,
                        what: str = "") -> dict:
    """Element-wise |z - z_ref| <= gamma~_p(8) * s_abs, with z_ref the exact
    product of the same operands and s_abs = sum_k |x_k w_k|."""
    z = np.asarray(z, dtype=np.float64)
    z_ref = np.asarray(z_ref, dtype=np.float64)
    tol = gamma_tilde(p) * np.asarray(s_abs, dtype=np.float64)
    err = np.abs(z - z_ref)
    bad = err > tol
    worst = float((err / np.maximum(tol, 1e-300)).max()) if z.size else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {z.size} outputs beyond the "
                           f"accumulation bound; worst {worst:.3g}x")
    return {"worst_frac_of_bound": worst}
