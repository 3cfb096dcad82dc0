"""Pins of the transform oracle against facts fixed outside it.

Each test checks oracle.transform against a library routine (scipy's
Hadamard, numpy's Kronecker product), a brute-force entrywise formula, or an
algebraic invariant, so that a dropped term, a wrong sign, a wrong index or a
transposed operand in the oracle fails at least one of them.
"""

import os

import numpy as np
import pytest
import scipy.linalg

from oracle import transform as T
import synthetic as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _plan(side: S.SidePlan) -> T.Plan:
    return T.Plan(side.d, side.radix, side.mode, side.blocks,
                  None if side.signs is None else side.signs.astype(np.float64))


def _rand_plan(seed, radix, mode, with_signs=True, dtype=np.float64):
    """Float64 blocks unless asked: the pins below hold to rounding of fp64."""
    return _plan(S.random_plan(np.random.default_rng(seed), radix, mode, with_signs, dtype))


# ------------------------------------------------------------ Hadamard

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64, 256, 1024])
def test_sylvester_matches_scipy_hadamard(n):
    assert np.array_equal(T.sylvester(n), scipy.linalg.hadamard(n).astype(float))


@pytest.mark.parametrize("n", [2, 16, 128, 4096])
def test_hadamard_rows_orthogonal(n):
    h = T.sylvester(n)
    assert np.array_equal(h @ h.T, n * np.eye(n))


@pytest.mark.parametrize("radix", [(2,) * 8, (4, 4, 16), (16, 16), (8, 2, 4), (2, 128),
                                   (4, 64), (2,) * 7, (16, 16, 16)])
def test_hadamard_blocks_reproduce_rht(radix):
    """With the normalised Sylvester blocks every power-of-two schedule gives
    the randomized Hadamard transform H_d D / sqrt(d) (HARP section 2.2: the
    processor equals the RHT at initialisation)."""
    d = int(np.prod(radix))
    s = S.signs(np.random.default_rng(d), d).astype(float)
    p = T.Plan(d, radix, T.HADAMARD, None, s)
    ref = scipy.linalg.hadamard(d) * s[None, :] / np.sqrt(d)
    assert np.abs(T.dense(p) - ref).max() < 1e-14


# ------------------------------------------------------------ structure

def test_strides_and_digits():
    radix = (3, 4, 5, 2)
    st = T.strides(radix)
    assert st == [40, 10, 2, 1]
    for i in range(120):
        dg = T.digits(i, radix)
        assert sum(a * b for a, b in zip(dg, st)) == i


@pytest.mark.parametrize("radix", [(4, 4, 16), (3, 4, 5), (2, 8, 4), (7, 5, 3, 2), (43,), (5, 2)])
def test_shared_blocks_are_kronecker_product(radix):
    """Shared blocks: M = kron(B_0, ..., B_{m-1}) D (digit 0 most significant)."""
    p = _rand_plan(11, radix, T.SHARED)
    k = np.ones((1, 1))
    for blk in p.blocks:
        k = np.kron(k, np.asarray(blk, dtype=np.float64))
    ref = k * p.sign_vector()[None, :]
    assert np.abs(T.dense(p) - ref).max() < 1e-13


def _path_formula(p: T.Plan) -> np.ndarray:
    """Brute force, entry by entry: M[i, j] = s_j * prod_t B_{t,c_t}[i_t, j_t]
    where after stage t-1 the coordinate carries digits (i_0..i_{t-1}, j_t..),
    so stage t's group is formed from the leading digits of i and the trailing
    digits of j: c_t = hi * S_t + lo, hi from i_0..i_{t-1}, lo from j_{t+1}.."""
    d, radix = p.d, p.radix
    m = len(radix)
    st = T.strides(radix)
    blocks = [p.stage_blocks(t) for t in range(m)]
    s = p.sign_vector()
    out = np.zeros((d, d))
    for i in range(d):
        di = T.digits(i, radix)
        for j in range(d):
            dj = T.digits(j, radix)
            val = s[j]
            for t in range(m):
                hi = 0
                for u in range(t):
                    hi = hi * radix[u] + di[u]
                lo = sum(dj[u] * st[u] for u in range(t + 1, m))
                val *= blocks[t][hi * st[t] + lo][di[t], dj[t]]
            out[i, j] = val
    return out


@pytest.mark.parametrize("radix", [(4, 4, 4), (3, 4, 5), (2, 8, 4), (7, 5, 2), (2, 3, 2, 2)])
def test_per_group_blocks_match_path_formula(radix):
    p = _rand_plan(12, radix, T.PER_GROUP)
    assert np.abs(T.dense(p) - _path_formula(p)).max() < 1e-13


def test_stage_changes_only_its_digit():
    radix = (3, 4, 5)
    p = _rand_plan(13, radix, T.PER_GROUP)
    for t in range(3):
        a = T.stage_matrix(p, t).tocoo()
        for r, c in zip(a.row, a.col):
            dr, dc = T.digits(r, radix), T.digits(c, radix)
            assert all(dr[u] == dc[u] for u in range(3) if u != t)


# ------------------------------------------------------------ invariants

@pytest.mark.parametrize("radix,mode", [((43, 16, 16), T.PER_GROUP), ((16, 16, 16), T.PER_GROUP),
                                        ((7, 16, 16), T.PER_GROUP), ((3, 4, 5), T.SHARED),
                                        ((2,) * 10, T.HADAMARD), ((8, 8, 8, 5, 2), T.PER_GROUP)])
def test_orthogonal_norm_and_round_trip(radix, mode):
    p = _rand_plan(14, radix, mode)
    rng = np.random.default_rng(1)
    if p.d <= 4096:
        m = T.dense(p)
        assert np.abs(m @ m.T - np.eye(p.d)).max() < 1e-12
    x = rng.standard_normal((5, p.d))
    y = T.apply_factored(p, x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.abs(T.apply_factored(p, y, inverse=True) - x).max() < 1e-12


def test_float32_blocks_orthogonal_to_rounding():
    """The library takes float32 blocks; their product is orthogonal to ~1e-7."""
    p = _rand_plan(22, (43, 16, 16), T.PER_GROUP, dtype=np.float32)
    x = np.random.default_rng(7).standard_normal((4, p.d))
    y = T.apply_factored(p, x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)
    assert np.abs(T.apply_factored(p, y, inverse=True) - x).max() < 1e-5


@pytest.mark.parametrize("radix,mode", [((4, 4, 16), T.PER_GROUP), ((43, 4), T.PER_GROUP),
                                        ((2,) * 8, T.HADAMARD), ((5, 3), T.SHARED)])
def test_factored_matches_dense(radix, mode):
    p = _rand_plan(15, radix, mode)
    x = np.random.default_rng(2).standard_normal((7, p.d))
    m = T.dense(p)
    assert np.abs(T.apply_factored(p, x) - x @ m.T).max() < 1e-12
    assert np.abs(T.apply_factored(p, x, inverse=True) - x @ m).max() < 1e-12


def test_block_diagonal_right_side():
    p = _rand_plan(16, (4, 8), T.PER_GROUP)
    x = np.random.default_rng(3).standard_normal((3, 4 * p.d))
    y = T.apply_right(p, x)
    m = T.dense(p)
    for c in range(4):
        seg = slice(c * p.d, (c + 1) * p.d)
        assert np.abs(y[:, seg] - x[:, seg] @ m.T).max() < 1e-13


def test_two_sided_associative_and_norm_preserving():
    u = _rand_plan(17, (4, 8), T.PER_GROUP)
    v = _rand_plan(18, (3, 16), T.PER_GROUP)
    w = np.random.default_rng(4).standard_normal((32, 48))
    mu, mv = T.dense(u), T.dense(v)
    a = T.two_sided(u, v, w)
    assert np.abs(a - (mu @ w) @ mv.T).max() < 1e-12
    assert np.abs(a - mu @ (w @ mv.T)).max() < 1e-12
    assert np.isclose(np.linalg.norm(a), np.linalg.norm(w), rtol=1e-13)
    assert np.abs(T.two_sided_inverse(u, v, a) - w).max() < 1e-12
    f = T.two_sided(u, v, w, method="factored")
    assert np.abs(a - f).max() < 1e-12


def test_left_rows_are_rows_of_dense():
    p = _rand_plan(19, (4, 4, 16), T.PER_GROUP)
    rows = np.array([0, 5, 77, 255])
    assert np.abs(T.left_rows(p, rows) - T.dense(p)[rows]).max() < 1e-14


# ------------------------------------------------------------ pages' examples

def _read_schedules():
    out = []
    with open(os.path.join(GOLDEN, "harp_radix_schedules.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                d, r = line.split("|")
                out.append((int(d), tuple(int(x) for x in r.split())))
    return out


def test_harp_page_schedule_5120():
    """HARP section 2.1: d = 5120 with radices (8, 8, 8, 5, 2); base mixers G_b
    (Hadamard for powers of two, QR fallback for 5) give an orthogonal M."""
    for d, radix in _read_schedules():
        assert int(np.prod(radix)) == d
        rng = np.random.default_rng(d)
        blocks = [T.base_mixer(b, rng.standard_normal((b, b))) for b in radix]
        p = T.Plan(d, radix, T.SHARED, blocks, None)
        x = np.random.default_rng(5).standard_normal((4, d))
        y = T.apply_factored(p, x)
        assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
        assert np.abs(T.apply_factored(p, y, inverse=True) - x).max() < 1e-12


def test_base_mixer_qr_fallback_is_orthogonal_and_deterministic():
    g = np.random.default_rng(6).standard_normal((5, 5))
    q1, q2 = T.base_mixer(5, g), T.base_mixer(5, g.copy())
    assert np.array_equal(q1, q2)
    assert np.abs(q1 @ q1.T - np.eye(5)).max() < 1e-14
    assert np.abs(T.base_mixer(8) - scipy.linalg.hadamard(8) / np.sqrt(8)).max() < 1e-15


# ------------------------------------------------------------ planted mistakes

def test_pins_catch_a_transposed_stage(monkeypatch):
    """A transposed block in the stage matrix must break the Kronecker pin."""
    p = _rand_plan(20, (3, 4), T.SHARED)
    orig = T.Plan.stage_blocks

    def transposed(self, t):
        return np.swapaxes(orig(self, t), 1, 2)

    monkeypatch.setattr(T.Plan, "stage_blocks", transposed)
    p._dense = None
    k = np.kron(p.blocks[0].astype(float), p.blocks[1].astype(float)) * p.sign_vector()[None, :]
    assert np.abs(T.dense(p) - k).max() > 1e-3


def test_pins_catch_a_wrong_stage_order():
    """Per-group stages do not commute: the product in the wrong order
    (B_0 B_1 D instead of B_1 B_0 D) must disagree with the path formula."""
    p = _rand_plan(21, (4, 4), T.PER_GROUP)
    ref = _path_formula(p)
    m = np.diag(p.sign_vector())
    m = T.stage_matrix(p, 0) @ (T.stage_matrix(p, 1) @ m)
    assert np.abs(np.asarray(m) - ref).max() > 1e-3
    assert np.abs(T.dense(p) - ref).max() < 1e-13
