"""Pins of the ORP GEO oracle ([ORPQuant] technical summary, section 2).

* The 3-bit lattice is the page's example: it runs from -1 through -1/2 to
  0 and up to 1, every level zero or a signed power of two, one state more
  on the negative side (asymmetric).
* b1 is the brute-force nearest lattice point outside the decision band.
* b1 and b2 are exactly orthogonal, b2 is b1 with entries exchanged at
  stride S inside micro-blocks of 2S and signs flipped, ||b2|| = ||b1||.
* (c1, c2) equal numpy's least-squares solution on the two bases, and the
  two-basis residual never exceeds the b1-only one.
* The chosen pair signs minimise the two-basis residual over every sign
  pattern (brute force on short vectors).
* A hand-worked 4-element case, and bit extraction of the packed signs.
"""

import itertools

import numpy as np
import pytest

from oracle import orp as O


def test_three_bit_lattice_is_the_pages_example():
    lv = O.levels(3)
    assert len(lv) == 8 and len(set(lv)) == 8
    assert lv[0] == -1.0 and lv[1] == -0.5 and lv[-1] == 1.0 and 0.0 in lv
    nz = lv[lv != 0]
    assert np.all(np.log2(np.abs(nz)) == np.round(np.log2(np.abs(nz))))  # powers of two
    assert (lv < 0).sum() == (lv > 0).sum() + 1


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_lattice_shape_at_every_width(bits):
    lv = O.levels(bits)
    assert len(lv) == 1 << bits
    assert np.all(np.diff(lv) > 0)
    assert lv.min() == -1.0 and lv.max() == 1.0
    assert (lv < 0).sum() == (1 << (bits - 1)) and (lv == 0).sum() == 1


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_primary_codes_equal_brute_force_nearest_point(bits):
    rng = np.random.default_rng(bits)
    w = rng.standard_t(3, size=(40, 256)) * 10.0 ** rng.uniform(-3, 1, size=(40, 1))
    w = w.astype(np.float32).astype(np.float64)
    codes, alpha = O.primary_codes(w, bits, 64)
    lv = O.levels(bits)
    u = (w.reshape(40, 4, 64) / np.abs(w.reshape(40, 4, 64)).max(axis=2, keepdims=True))
    dist = np.abs(u.reshape(40, 256)[..., None] - lv)
    brute = dist.argmin(axis=-1)  # ties to the lower index
    band = O.band(w, bits, 64)
    assert np.array_equal(codes[~band], brute[~band])
    assert band.mean() < 1e-3
    # the element holding alpha maps to -1 or +1 exactly
    for r in range(40):
        for gi in range(4):
            k = gi * 64 + int(np.abs(w[r, gi * 64:(gi + 1) * 64]).argmax())
            assert lv[codes[r, k]] == np.sign(w[r, k])


def test_band_sits_on_the_switching_points():
    bits = 3
    lv = O.levels(bits)
    tau = O.thresholds(bits)
    gap = np.diff(lv).min()
    w = np.zeros((1, 64))
    w[0, 0] = 1.0
    inside = tau + 0.5e-6 * np.maximum(np.abs(tau), gap)
    outside = tau + 3e-6 * np.maximum(np.abs(tau), gap)
    w[0, 1:1 + len(tau)] = inside
    w[0, 8:8 + len(tau)] = outside
    b = O.band(w, bits, 64)
    assert b[0, 1:1 + len(tau)].all() and not b[0, 8:8 + len(tau)].any()


@pytest.mark.parametrize("stride", [1, 2, 4, 32])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_bases_orthogonal_and_scales_are_least_squares(bits, stride):
    rng = np.random.default_rng(10 * bits + stride)
    g = 64
    w = rng.standard_t(3, size=(16, 4 * g))
    codes, sigma, coef, b1, b2, wp = O.geo_quantize(w, bits, g, stride)
    for r in range(16):
        for gi in range(4):
            sl = slice(gi * g, (gi + 1) * g)
            x1, x2, y = b1[r, sl], b2[r, sl], wp[r, sl]
            assert x1 @ x2 == 0.0                                  # exactly orthogonal
            assert x1 @ x1 == x2 @ x2
            c, *_ = np.linalg.lstsq(np.stack([x1, x2], axis=1), y, rcond=None)
            assert np.allclose(coef[r, gi], c, rtol=1e-12, atol=1e-15)
            res2 = np.linalg.norm(y - coef[r, gi, 0] * x1 - coef[r, gi, 1] * x2)
            res1 = np.linalg.norm(y - coef[r, gi, 0] * x1)
            assert res2 <= res1 * (1 + 1e-15)
            assert coef[r, gi, 1] >= 0.0                            # b2 points along r
    # b2 is a stride exchange of b1 with sign flips inside micro-blocks
    f, s = O.pair_index(4 * g, stride)
    assert np.array_equal(np.abs(b2[:, f]), np.abs(b1[:, s]))
    assert np.array_equal(np.abs(b2[:, s]), np.abs(b1[:, f]))
    assert np.all((f // (2 * stride)) == (s // (2 * stride)))


@pytest.mark.parametrize("stride", [1, 2, 4])
def test_pair_signs_minimise_the_residual_over_all_patterns(stride):
    rng = np.random.default_rng(50 + stride)
    g, bits = 16, 3
    for trial in range(6):
        w = rng.standard_normal((1, g))
        codes, sigma, coef, b1, b2, wp = O.geo_quantize(w, bits, g, stride)
        best = np.linalg.norm(wp[0] - coef[0, 0, 0] * b1[0] - coef[0, 0, 1] * b2[0])
        f, s = O.pair_index(g, stride)
        for pattern in itertools.product((1.0, -1.0), repeat=len(f)):
            sg = np.array(pattern)[None, :]
            _, b2p = O.basis_from_codes(codes, sg, bits, stride)
            A = np.stack([b1[0], b2p[0]], axis=1)
            c, *_ = np.linalg.lstsq(A, wp[0], rcond=None)
            assert np.linalg.norm(wp[0] - A @ c) >= best - 1e-12


def test_hand_worked_example():
    """w = (0.9, -0.3, 0.2, 1.0), 3 bits, one group, stride 1.
    alpha = 1.0; u = w; nearest levels: 0.9 -> 1, -0.3 -> -0.25, 0.2 -> 0.25,
    1.0 -> 1, so b1 = (1, -1/4, 1/4, 1), ||b1||^2 = 2.125,
    <w, b1> = 0.9 + 0.075 + 0.05 + 1.0 = 2.025, c1 = 2.025 / 2.125.
    Pairs (0, 1), (2, 3): d0 = w1 b1[0] - w0 b1[1] = -0.3 + 0.225 = -0.075
    -> sigma0 = -1, b2[0:2] = -(-b1[1], b1[0]) = (-0.25, -1);
    d1 = w3 b1[2] - w2 b1[3] = 0.25 - 0.2 = 0.05 -> sigma1 = +1,
    b2[2:4] = (-b1[3], b1[2]) = (-1, 0.25);
    <w, b2> = |d0| + |d1| = 0.125, c2 = 0.125 / 2.125."""
    w = np.array([[0.9, -0.3, 0.2, 1.0]])
    codes, sigma, coef, b1, b2, _ = O.geo_quantize(w, 3, 4, 1)
    assert np.array_equal(b1[0], [1.0, -0.25, 0.25, 1.0])
    assert np.array_equal(sigma[0], [-1.0, 1.0])
    assert np.array_equal(b2[0], [-0.25, -1.0, -1.0, 0.25])
    assert coef[0, 0, 0] == pytest.approx(2.025 / 2.125, rel=1e-15)
    assert coef[0, 0, 1] == pytest.approx(0.125 / 2.125, rel=1e-14)
    assert list(codes[0]) == [7, 2, 5, 7]


def test_zero_group_and_dequant_round_trip():
    rng = np.random.default_rng(9)
    w = rng.standard_normal((4, 128))
    w[1, :64] = 0.0
    codes, sigma, coef, b1, b2, wp = O.geo_quantize(w, 4, 64, 2)
    zero = int(np.flatnonzero(O.levels(4) == 0)[0])
    assert np.all(codes[1, :64] == zero) and np.all(coef[1, 0] == 0)
    back = O.geo_dequant(codes, sigma, coef, 4, 64, 2)
    ref = (np.repeat(coef[..., 0], 64, axis=1) * b1 + np.repeat(coef[..., 1], 64, axis=1) * b2)
    assert np.allclose(back, ref, rtol=0, atol=1e-15)
    # two bases reconstruct better than one on every nonzero group
    e2 = ((wp - back) ** 2).reshape(4, 2, 64).sum(axis=2)
    e1 = ((wp - np.repeat(coef[..., 0], 64, axis=1) * b1) ** 2).reshape(4, 2, 64).sum(axis=2)
    assert np.all(e2 <= e1)


def test_preconditioning_scales_input_channels():
    rng = np.random.default_rng(12)
    w = rng.standard_normal((3, 64))
    s = rng.uniform(0.5, 2.0, size=64)
    wp = O.precondition(w, s)
    assert np.array_equal(wp, (w.astype(np.float32) * s.astype(np.float32)).astype(np.float64))
    c1 = O.geo_quantize(w, 3, 64, 1, smooth=s)[0]
    c2 = O.geo_quantize(wp, 3, 64, 1)[0]
    assert np.array_equal(c1, c2)


def test_sign_packing_bit_extraction():
    rng = np.random.default_rng(13)
    sigma = np.where(rng.random((3, 40)) < 0.5, -1.0, 1.0)
    packed = O.pack_signs(sigma)
    assert packed.shape == (3, 5)
    for r in range(3):
        stream = int.from_bytes(bytes(packed[r]), "little")
        for p in range(40):
            assert ((stream >> p) & 1) == (1 if sigma[r, p] < 0 else 0)
    assert np.array_equal(O.unpack_signs(packed, 40), sigma)
