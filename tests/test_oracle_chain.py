"""Pins of the chain oracle (PolarQuant restore, then absmax INT4) against a
brute-force route: entrywise dequantization by loops, scipy's Hadamard
matrix, and the nearest absmax level by exhaustive search; plus the error
bound of the second quantizer."""

import numpy as np
import pytest
import scipy.linalg

from oracle import chain as C
from oracle import lloydmax as LM
from oracle import quant as Q
from oracle import transform as T


def _inputs(rng, m, n, bits, g):
    cent = LM.lloyd_max_gaussian(bits)[0]
    cent = np.asarray(cent, dtype=np.float32)
    codes = rng.integers(0, 1 << bits, size=(m, n)).astype(np.uint8)
    norms = (rng.random((m, n // g)) * 3 + 0.1).astype(np.float16)
    return codes, norms, cent


@pytest.mark.parametrize("bits_in,bits_out,g_out", [(5, 4, 128), (4, 4, 64), (5, 2, 256)])
def test_chain_matches_brute_force(bits_in, bits_out, g_out):
    rng = np.random.default_rng(bits_in * 10 + bits_out)
    m, n, d = 3, 512, 128
    codes, norms, cent = _inputs(rng, m, n, bits_in, d)
    plan = T.Plan(d, (2,) * 7, T.HADAMARD)
    c_out, a_out, w = C.requant(codes, norms, cent, d, plan, bits_out, g_out)
    # brute force: loops, scipy's Hadamard (symmetric, so its own inverse)
    h = scipy.linalg.hadamard(d) / np.sqrt(d)
    wb = np.zeros((m, n))
    for r in range(m):
        for b in range(n // d):
            v = np.array([float(norms[r, b]) * float(cent[codes[r, b * d + i]]) / np.sqrt(d)
                          for i in range(d)])
            wb[r, b * d:(b + 1) * d] = h @ v
    assert np.abs(w - wb).max() < 1e-12
    lv = (1 << bits_out) - 1
    for r in range(m):
        for gi in range(n // g_out):
            grp = wb[r, gi * g_out:(gi + 1) * g_out]
            alpha = np.abs(grp).max()
            assert abs(a_out[r, gi] - np.float32(alpha)) <= 1e-7 * alpha
            levels = alpha * (np.arange(lv + 1) * 2.0 / lv - 1.0)
            best = np.abs(grp[:, None] - levels[None, :]).argmin(axis=1)
            got = c_out[r, gi * g_out:(gi + 1) * g_out]
            band = Q.absmax_band(grp[None, :], bits_out, g_out)[0]
            assert ((got == best) | band).all()


def test_chain_error_bound():
    """Each restored weight is within half a level of its re-quantized value."""
    rng = np.random.default_rng(9)
    codes, norms, cent = _inputs(rng, 4, 1024, 5, 128)
    plan = T.Plan(128, (16, 8), T.HADAMARD)
    c_out, a_out, w = C.requant(codes, norms, cent, 128, plan, 4, 128)
    wq = Q.absmax_dequant(c_out, a_out, 4, 128)
    half = np.repeat(a_out / 7.5, 128, axis=1) / 2
    assert (np.abs(wq - w) <= half * (1 + 1e-6) + 1e-12).all()


def test_pins_catch_a_forward_restore(monkeypatch):
    """Restoring with the forward transform instead of the inverse fails the
    brute-force pin (the plan with signs is not its own inverse)."""
    rng = np.random.default_rng(3)
    codes, norms, cent = _inputs(rng, 1, 128, 5, 128)
    sg = np.where(rng.random(128) < 0.5, -1.0, 1.0)
    plan = T.Plan(128, (2,) * 7, T.HADAMARD, signs=sg)
    ref = C.restore(codes, norms, cent, 128, plan)
    orig = T.apply_right
    monkeypatch.setattr(T, "apply_right", lambda p, x, inverse=False, method="dense": orig(p, x, False, method))
    bad = C.restore(codes, norms, cent, 128, plan)
    assert np.abs(bad - ref).max() > 1e-3
