"""Pins of the HARP parameter oracle (oracle.harp) against facts fixed
outside it: the zero-parameter identity the pages state, closed forms of the
Cayley map (a hand-worked 3 x 3 case, the 2 x 2 angle formula), an independent
route through the eigendecomposition, orthogonality and determinant, and the
parameter layout by brute force.  A dropped term, a sign error, a transposed
factor or a misplaced parameter fails at least one of them.
"""

import numpy as np
import pytest
import scipy.linalg

from oracle import harp as H
from oracle import transform as T
import synthetic as S

RADICES = [2, 3, 4, 7, 16, 43, 64]


def _theta(rng, b, scale=0.3):
    return scale * rng.standard_normal(H.n_params(b))


@pytest.mark.parametrize("b", RADICES)
def test_zero_parameters_give_the_base_mixer(b):
    """[HARP] section 2.2: at theta = 0, Q = I and B = G."""
    q = H.q_block(np.zeros(H.n_params(b)), b)
    assert np.array_equal(q, np.eye(b))
    g = None if b & (b - 1) == 0 else T.base_mixer(b, np.random.default_rng(b).standard_normal((b, b)))
    blk = H.stage_blocks(b, 3, np.zeros(3 * H.n_params(b), dtype=np.int8), 0.01, g)
    ref = T.base_mixer(b) if g is None else g
    for c in range(3):
        assert np.array_equal(blk[c], ref)


@pytest.mark.parametrize("radix", [(2,) * 8, (4, 4, 16), (16, 16), (2, 8, 4)])
def test_zero_parameter_plan_is_the_rht(radix):
    """[HARP] section 2.2: with all parameters zero the transform is the RHT,
    H_d D / sqrt(d) with scipy's Hadamard matrix."""
    d = int(np.prod(radix))
    rng = np.random.default_rng(d)
    sg = S.signs(rng, d).astype(np.float64)
    p = H.harp_plan(d, radix, np.zeros(H.total_params(d, radix), dtype=np.int8),
                    [0.02] * len(radix), signs=sg)
    ref = scipy.linalg.hadamard(d) * sg[None, :] / np.sqrt(d)
    assert np.allclose(T.dense(p), ref, atol=1e-13, rtol=0)


@pytest.mark.parametrize("b", RADICES)
def test_blocks_orthogonal_with_determinant_one(b):
    rng = np.random.default_rng(100 + b)
    q = H.q_block(_theta(rng, b), b)
    assert np.abs(q.T @ q - np.eye(b)).max() < 1e-12
    assert abs(np.linalg.det(q) - 1.0) < 1e-10  # rotations: Givens and Cayley images lie in SO(b)


@pytest.mark.parametrize("b", [3, 4, 7, 16, 43])
def test_cayley_matches_eigendecomposition(b):
    """Independent route: iA is Hermitian, iA = V diag(mu) V^H, so A has
    eigenvalues -i mu and (I - A)^{-1}(I + A) = V diag((1 - i mu)/(1 + i mu)) V^H."""
    rng = np.random.default_rng(200 + b)
    th = _theta(rng, b, 0.7)
    a = H.skew(th, b)
    mu, v = np.linalg.eigh(1j * a)
    lam = (1 - 1j * mu) / (1 + 1j * mu)
    q = (v * lam[None, :]) @ v.conj().T
    assert np.abs(q.imag).max() < 1e-12
    assert np.abs(H.cayley(th, b) - q.real).max() < 1e-12


def test_cayley_worked_example_3x3():
    """A = [[0, 1, 0], [-1, 0, 0], [0, 0, 0]]: I - A = [[1, -1, 0], [1, 1, 0],
    [0, 0, 1]], its inverse is [[1, 1, 0], [-1, 1, 0], [0, 0, 2]] / 2, and
    times I + A = [[1, 1, 0], [-1, 1, 0], [0, 0, 1]] gives a quarter turn of
    the first two coordinates (worked by hand)."""
    q = H.cayley(np.array([1.0, 0.0, 0.0]), 3)
    assert np.allclose(q, [[0, 1, 0], [-1, 0, 0], [0, 0, 1]], atol=1e-15, rtol=0)


@pytest.mark.parametrize("a", [-2.0, -0.3, 0.0, 0.05, 1.0, 7.0])
def test_cayley_2x2_is_a_rotation_by_minus_twice_atan(a):
    """For b = 2, (I - A)^{-1}(I + A) with A = [[0, a], [-a, 0]] is
    [[1 - a^2, 2a], [-2a, 1 - a^2]] / (1 + a^2): the Givens rotation by
    -2 atan(a)."""
    closed = np.array([[1 - a * a, 2 * a], [-2 * a, 1 - a * a]]) / (1 + a * a)
    assert np.allclose(H.cayley(np.array([a]), 2), closed, atol=1e-15, rtol=0)
    assert np.allclose(H.givens(-2 * np.arctan(a)), closed, atol=1e-15, rtol=0)


def test_givens_quarter_turn():
    """Givens(pi/2) maps e_0 to e_1 and e_1 to -e_0."""
    q = H.givens(np.pi / 2)
    assert np.allclose(q @ [1, 0], [0, 1], atol=1e-15)
    assert np.allclose(q @ [0, 1], [-1, 0], atol=1e-15)


@pytest.mark.parametrize("b", [2, 3, 7, 16])
def test_negated_parameters_invert(b):
    rng = np.random.default_rng(300 + b)
    th = _theta(rng, b)
    assert np.abs(H.q_block(-th, b) - H.q_block(th, b).T).max() < 1e-13


@pytest.mark.parametrize("b", [3, 16])
def test_first_order_term(b):
    """Q(eps theta) = I + 2 eps A + O(eps^2)."""
    rng = np.random.default_rng(400 + b)
    th = _theta(rng, b, 1.0)
    for eps in (1e-3, 1e-4):
        err = np.abs(H.cayley(eps * th, b) - np.eye(b) - 2 * eps * H.skew(th, b)).max()
        assert err < 10 * b * eps * eps


@pytest.mark.parametrize("b", [3, 5, 16])
def test_parameter_layout_by_brute_force(b):
    th = np.arange(1, H.n_params(b) + 1, dtype=np.float64)
    a = H.skew(th, b)
    for i in range(b):
        assert a[i, i] == 0
        for j in range(i + 1, b):
            p = i * b - i * (i + 1) // 2 + (j - i - 1)
            assert a[i, j] == th[p] and a[j, i] == -th[p]


def test_int8_dequant():
    q = np.array([-127, -1, 0, 5, 127], dtype=np.int8)
    assert np.array_equal(H.dequant_theta(q, 0.5), [-63.5, -0.5, 0.0, 2.5, 63.5])
    with pytest.raises(ValueError):
        H.dequant_theta(np.array([-128], dtype=np.int8), 1.0)
    with pytest.raises(ValueError):
        H.dequant_theta(np.array([1], dtype=np.int16), 1.0)


def test_plan_layout_one_nonzero_group():
    """Only group c of stage t has nonzero parameters: only that block differs
    from G, and it equals Q(theta) G for that group's parameters."""
    radix = (4, 2, 8)
    d = 64
    n = H.total_params(d, radix)
    off = (d // 4) * H.n_params(4)  # stage 1 starts here
    c = 5
    tq = np.zeros(n, dtype=np.int8)
    tq[off + c] = 40  # stage 1 is radix 2: one Givens angle per group
    p = H.harp_plan(d, radix, tq, [0.1, 0.025, 0.1])
    for t, b in enumerate(radix):
        blk = p.stage_blocks(t)
        for g in range(d // b):
            ref = T.base_mixer(b)
            if t == 1 and g == c:
                ref = H.givens(float(np.float32(0.025)) * 40) @ ref  # the scale is a float32
            assert np.allclose(blk[g], ref, atol=1e-15, rtol=0), (t, g)


def test_pins_catch_a_transposed_cayley(monkeypatch):
    orig = H.cayley
    monkeypatch.setattr(H, "cayley", lambda th, b: orig(th, b).T)
    with pytest.raises(AssertionError):
        test_cayley_worked_example_3x3()
