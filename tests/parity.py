"""Comparison rules between the HIP path and the oracle (test helper).

* float32 output: max |y - y_ref| / ||row of y_ref||_2 <= 2e-5.
* bfloat16 / float16 output: |y - y_ref| <= 1 ulp of the storage type at
  |y_ref|; where that ulp is below the float32 rotation tolerance
  (2e-5 * row norm) the float32 tolerance applies instead (reading: the
  ulp rule cannot hold for values far below the row norm, whose absolute
  float32 error is set by the row norm).
* codes: equal except where the exact value is within the decision band
  (1e-6 relative of a threshold); the excepted elements -- mismatches, all of
  them inside the band -- must number <= 1e-5 of the elements (reading: the
  count bounded is that of the exceptions to bit-exactness; the band's own
  population is reported -- for the 4-bit Gaussian codebook it is ~1e-5 by
  itself, a property of the data and not of the kernel).  Below 4e5 elements
  the cap is 4 elements, where the fraction rule would forbid a single
  in-band flip.
* absmax scales: within 2e-5 * row norm; float16 norms within 1 fp16 ulp.
"""

from __future__ import annotations

import numpy as np

ROT_TOL = 2e-5
BAND_FRAC = 1e-5


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
    tol = np.maximum(ulp(y_ref, mant), ROT_TOL * nrm)
    bad = err > tol
    info["floor_used"] = int((ulp(y_ref, mant) < ROT_TOL * nrm).sum())
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond 1 {dtype} ulp; "
                           f"worst {float((err / tol).max()):.3g}x")
    return info


def check_codes(codes: np.ndarray, codes_ref: np.ndarray, band: np.ndarray, what: str = "") -> dict:
    codes = np.asarray(codes)
    codes_ref = np.asarray(codes_ref)
    mism = codes != codes_ref
    outside = mism & ~band
    n = codes.size
    nb = int(band.sum())
    nm = int(mism.sum())
    info = {"mismatches": nm, "band": nb, "elements": n}
    assert not outside.any(), (f"{what}: {int(outside.sum())} code mismatches outside the "
                               f"band (of {nm} mismatches)")
    cap = max(BAND_FRAC * n, 4.0)
    assert nm <= cap, f"{what}: {nm} in-band mismatches > {cap:.3g}"
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
