"""Pins of the decode linear oracle: the rotate-the-activations route equals
the unrotate-the-weight route (Y = X W^T with W = M_U^T W'^ M_V, formed by
the two-sided inverse), a brute-force loop on a tiny case, and the reading
that an all-identity layer is a plain product with the dequantized weight."""

import numpy as np
import pytest

from oracle import linear as L
from oracle import quant as Q
from oracle import transform as T
import synthetic as S


def _plan(seed, radix, mode="per_group"):
    side = S.random_plan(np.random.default_rng(seed), radix, mode, dtype=np.float64)
    return T.Plan(side.d, side.radix, side.mode, side.blocks, side.signs.astype(np.float64))


@pytest.mark.parametrize("m_radix,n_radix,bits,group", [((4, 16), (4, 4, 16), 2, 64),
                                                        ((8, 8), (16, 16), 3, 128),
                                                        ((2, 32), (7, 16, 4), 4, 64)])
def test_rotated_activations_equal_unrotated_weight(m_radix, n_radix, bits, group):
    U, V = _plan(1, m_radix), _plan(2, n_radix)
    m, n = U.d, V.d
    rng = np.random.default_rng(3)
    w = rng.standard_normal((m, n))
    codes, alpha = Q.absmax_quantize(T.two_sided(U, V, w), bits, group)
    x = rng.standard_normal((5, n))
    y, _ = L.qlinear(U, V, L.rotate_acts(V, x), codes, alpha, bits, group)
    w_back = T.two_sided_inverse(U, V, Q.absmax_dequant(codes, alpha, bits, group))
    assert np.abs(y - x @ w_back.T).max() < 1e-10 * max(1.0, np.abs(y).max())


def test_tiny_brute_force():
    U, V = _plan(4, (2, 2)), _plan(5, (4, 2))
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 4, size=(4, 8)).astype(np.uint8)
    alpha = rng.random((4, 1)) + 0.5
    x = rng.standard_normal((3, 8))
    xt = L.rotate_acts(V, x)
    y, z = L.qlinear(U, V, xt, codes, alpha, 2, 8)
    mv, mu = T.dense(V), T.dense(U)
    for t in range(3):
        xr = [sum(mv[j, k] * x[t, k] for k in range(8)) for j in range(8)]
        zz = [sum(xr[j] * alpha[i, 0] * (codes[i, j] / 1.5 - 1.0) for j in range(8)) for i in range(4)]
        yy = [sum(mu[i, r] * zz[i] for i in range(4)) for r in range(4)]
        assert np.allclose(z[t], zz, atol=1e-12) and np.allclose(y[t], yy, atol=1e-12)


def test_identity_plans_are_a_plain_product():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, size=(6, 128)).astype(np.uint8)
    alpha = rng.random((6, 2))
    x = rng.standard_normal((2, 128))
    y, z = L.qlinear(None, None, L.rotate_acts(None, x), codes, alpha, 4, 64)
    assert np.array_equal(y, z)
    assert np.allclose(y, x @ Q.absmax_dequant(codes, alpha, 4, 64).T, atol=1e-12)
