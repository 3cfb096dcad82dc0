"""Pins of the Lloyd-Max oracle: the 1-bit closed form, the optimality
conditions checked by independent numerical integration, Max's published table
(tests/golden), symmetry, and local optimality of the MSE."""

import os

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import lloydmax as LM

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _table():
    rows = {}
    with open(os.path.join(GOLDEN, "lloyd_max_gaussian_max1960.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                lv, thr, out, mse = [p.strip() for p in line.split("|")]
                rows[int(lv)] = ([float(x) for x in thr.split()],
                                 [float(x) for x in out.split()], float(mse))
    return rows


def test_one_bit_closed_form():
    c, t, mse = LM.lloyd_max_gaussian(1)
    assert np.allclose(c, [-np.sqrt(2 / np.pi), np.sqrt(2 / np.pi)], atol=1e-14)
    assert t.tolist() == [0.0]
    assert mse == pytest.approx(1 - 2 / np.pi, abs=1e-14)


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_centroid_condition_by_quadrature(bits):
    """c_k = E[X | cell k], with the conditional mean integrated numerically
    (scipy.integrate.quad of x * pdf), independent of the erfc closed form."""
    c, t, _ = LM.lloyd_max_gaussian(bits)
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    for k in range(len(c)):
        a, b = edges[k], edges[k + 1]
        p, _ = integrate.quad(stats.norm.pdf, a, b, epsabs=1e-14)
        m, _ = integrate.quad(lambda x: x * stats.norm.pdf(x), a, b, epsabs=1e-14)
        assert c[k] == pytest.approx(m / p, abs=1e-9)
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=1e-15)
    assert LM.stationarity_residual(c) < 1e-12


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_matches_max_1960_table(bits):
    thr, out, mse = _table()[1 << bits]
    c, t, m = LM.lloyd_max_gaussian(bits)
    half = len(c) // 2
    assert np.allclose(c[half:], out, atol=1e-3)
    assert np.allclose(t[half - 1:], thr, atol=1e-3)
    assert m == pytest.approx(mse, rel=2e-3)


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_symmetric_and_middle_threshold_zero(bits):
    c, t, _ = LM.lloyd_max_gaussian(bits)
    assert np.allclose(c, -c[::-1], atol=1e-15)
    assert t[len(t) // 2] == 0.0
    assert np.all(np.diff(c) > 0)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_mse_by_quadrature_and_local_optimality(bits):
    c, t, mse = LM.lloyd_max_gaussian(bits)

    def mse_of(cent):
        th = 0.5 * (cent[:-1] + cent[1:])
        e = np.concatenate([[-np.inf], th, [np.inf]])
        tot = 0.0
        for k in range(len(cent)):
            v, _ = integrate.quad(lambda x: (x - cent[k]) ** 2 * stats.norm.pdf(x),
                                  e[k], e[k + 1], epsabs=1e-14)
            tot += v
        return tot

    assert mse == pytest.approx(mse_of(c), abs=1e-10)
    rng = np.random.default_rng(bits)
    for _ in range(3):
        pert = c + 1e-3 * rng.standard_normal(len(c))
        assert mse_of(np.sort(pert)) > mse
