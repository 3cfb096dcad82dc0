"""Pins of the quantizer, band and packing oracles.

Absmax is checked against a brute-force nearest-level search and the error
bound of uniform rounding; the codebook search against a brute-force
nearest-centroid argmin; packing against bit extraction with Python integers;
the PolarQuant block pipeline against the identities its page states
(Hadamard self-inverse, unit-sphere normalisation, Gaussian coordinates).
"""

import numpy as np
import pytest
import scipy.linalg
import scipy.stats

from oracle import lloydmax as LM
from oracle import quant as Q
from oracle import transform as T


# ------------------------------------------------------------ absmax

@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_absmax_equals_brute_force_nearest_level(bits):
    """code = argmin_c |v - (-alpha + c * 2 alpha / (L-1))| for random groups."""
    rng = np.random.default_rng(bits)
    v = rng.standard_normal((6, 64)) * rng.uniform(0.1, 10, size=(6, 1))
    codes, alpha = Q.absmax_quantize(v, bits, 16, decide_f32=False)
    lv = (1 << bits) - 1
    for r in range(6):
        for gi in range(4):
            a = np.abs(v[r, gi * 16:(gi + 1) * 16]).max()
            assert alpha[r, gi] == a
            levels = -a + np.arange(lv + 1) * (2 * a / lv)
            for k in range(16):
                x = v[r, gi * 16 + k]
                best = int(np.argmin(np.abs(x - levels)))
                assert codes[r, gi * 16 + k] == best


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_absmax_error_bound_and_endpoints(bits):
    rng = np.random.default_rng(10 + bits)
    v = scipy.stats.t.rvs(3, size=(8, 256), random_state=rng)
    codes, alpha = Q.absmax_quantize(v, bits, 128, decide_f32=False)
    vh = Q.absmax_dequant(codes, alpha, bits, 128)
    lv = (1 << bits) - 1
    delta = np.repeat(2 * alpha / lv, 128, axis=1)
    assert np.all(np.abs(v - vh) <= delta / 2 * (1 + 1e-12))
    g = v.reshape(8, 2, 128)
    c = codes.reshape(8, 2, 128)
    idx = np.abs(g).argmax(axis=2)
    for r in range(8):
        for gi in range(2):
            x = g[r, gi, idx[r, gi]]
            assert c[r, gi, idx[r, gi]] == (lv if x > 0 else 0)
            assert vh.reshape(8, 2, 128)[r, gi, idx[r, gi]] == pytest.approx(x, rel=1e-15)


def test_absmax_scale_invariance_and_zero_group():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((4, 128))
    c1, _ = Q.absmax_quantize(v, 3, 128)
    c2, _ = Q.absmax_quantize(v * 8.0, 3, 128)
    assert np.array_equal(c1, c2)
    z = np.zeros((2, 128))
    cz, az = Q.absmax_quantize(z, 3, 128)
    assert not cz.any() and not az.any()


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_absmax_f32_and_f64_decisions_agree_outside_band(bits):
    rng = np.random.default_rng(20 + bits)
    v = rng.standard_normal((64, 512)).astype(np.float32).astype(np.float64)
    c32, _ = Q.absmax_quantize(v, bits, 128, decide_f32=True)
    c64, _ = Q.absmax_quantize(v, bits, 128, decide_f32=False)
    band = Q.absmax_band(v, bits, 128)
    assert np.array_equal(c32[~band], c64[~band])


def test_absmax_band_contains_threshold_points():
    bits, lv = 3, 7
    a = 2.0
    tau = -1 + (2 * np.arange(lv) + 1) / lv
    v = np.concatenate([[a], a * tau, a * (tau + 0.3 / lv)])
    v = np.concatenate([v, np.zeros(128 - len(v))])[None, :]
    band = Q.absmax_band(v, bits, 128)
    assert band[0, 1:1 + lv].all()
    assert not band[0, 1 + lv:1 + 2 * lv].any()


# ------------------------------------------------------------ codebook / PolarQuant

def test_codebook_threshold_search_equals_nearest_centroid():
    cb = LM.lloyd_max_gaussian(4)[0].astype(np.float32)
    rng = np.random.default_rng(4)
    z = rng.standard_normal(20000) * 1.5
    tau = (cb[:-1].astype(np.float64) + cb[1:].astype(np.float64)) / 2
    z = np.concatenate([z, tau])  # exact ties go to the lower index
    by_search = (z[:, None] > tau).sum(axis=1)
    assert np.array_equal(by_search, Q.nearest_centroid(z, cb))


def _switch_points(cb):
    """Where the brute-force nearest-centroid search changes its answer,
    found by bisection on nearest_centroid alone (no threshold formula)."""
    c = np.asarray(cb, dtype=np.float32).astype(np.float64)
    pts = []
    for k in range(len(c) - 1):
        lo, hi = c[k], c[k + 1]
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            if Q.nearest_centroid(np.array([mid]), cb)[0] <= k:
                lo = mid
            else:
                hi = mid
        pts.append(lo)
    return np.array(pts)


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_codebook_band_sits_on_the_decision_points(bits):
    """The band of the codebook search lies on the points where the nearest
    centroid changes: points 0.5 band widths from each switching point are in
    it, points 3 widths away are not; the width is 1e-6 relative, floored at
    1e-6 of the smallest centroid gap, so it is not empty at the threshold 0."""
    cb = LM.lloyd_max_gaussian(bits)[0].astype(np.float32)
    sw = _switch_points(cb)
    assert len(sw) == (1 << bits) - 1
    gap = float(np.diff(cb.astype(np.float64)).min())
    width = Q.BAND_REL * np.maximum(np.abs(sw), gap)
    mid = (1 << bits) // 2 - 1
    assert abs(sw[mid]) < 1e-15 and width[mid] > 0  # the middle threshold is 0
    for f in (-0.5, 0.5):
        assert Q.codebook_band(sw + f * width, cb).all()
    for f in (-3.0, 3.0):
        assert not Q.codebook_band(sw + f * width, cb).any()
    # far from every switching point: never in the band
    far = 0.5 * (sw[:-1] + sw[1:])
    assert not Q.codebook_band(far, cb).any()


@pytest.mark.parametrize("bits", [2, 4, 5])
@pytest.mark.parametrize("decide_f32", [True, False])
def test_codebook_codes_equal_brute_force_outside_band(bits, decide_f32):
    """codebook_norm_quantize's codes equal the brute-force nearest centroid
    of z = sqrt(g) v / ||v|| (computed in float64) everywhere outside the
    band, on Gaussian and heavy-tailed blocks, scaled over decades."""
    cb = LM.lloyd_max_gaussian(bits)[0].astype(np.float32)
    rng = np.random.default_rng(40 + bits)
    g = 128
    v = rng.standard_normal((400, 4 * g))
    v[:200] *= np.where(rng.random((200, 4 * g)) < 0.01, 10.0, 1.0)
    v *= 10.0 ** rng.uniform(-3, 2, size=(400, 1))
    v = v.astype(np.float32).astype(np.float64)
    codes, r, z = Q.codebook_norm_quantize(v, cb, g, decide_f32=decide_f32)
    vg = v.reshape(400, 4, g)
    z_bf = (np.sqrt(g) * vg / np.linalg.norm(vg, axis=2, keepdims=True)).reshape(400, -1)
    ref = Q.nearest_centroid(z_bf, cb)
    band = Q.codebook_band(z_bf, cb)
    assert np.array_equal(codes[~band], ref[~band])
    assert band.mean() < 1e-4


def test_polar_block_identities():
    """PolarQuant section 2: normalise the block onto the unit sphere, rotate
    by the Walsh-Hadamard matrix, scale by sqrt(d): sum z^2 = d; H/sqrt(d) is
    its own inverse; both orders of normalise/rotate agree."""
    d = 128
    hn = scipy.linalg.hadamard(d) / np.sqrt(d)
    assert np.abs(hn @ hn - np.eye(d)).max() < 1e-14
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, d)) * rng.uniform(0.01, 5, size=(50, 1))
    z1 = np.sqrt(d) * (x / np.linalg.norm(x, axis=1, keepdims=True)) @ hn.T
    p = T.Plan(d, (2,) * 7, T.HADAMARD)
    y = T.apply_right(p, x)
    _, r, z2 = Q.codebook_norm_quantize(y, LM.lloyd_max_gaussian(4)[0], d, decide_f32=False)
    assert np.abs(z1 - z2).max() < 1e-12
    assert np.allclose((z2 ** 2).sum(axis=1), d, rtol=1e-13)
    assert np.allclose(r[:, 0], np.linalg.norm(x, axis=1), rtol=1e-13)


def test_polar_rotated_coordinates_are_gaussian():
    """PolarQuant section 2: rotated unit-sphere coordinates tend to N(0, 1/d);
    after the sqrt(d) scale they are close to N(0, 1), even for heavy-tailed
    blocks."""
    d = 128
    rng = np.random.default_rng(6)
    x = np.where(rng.random((4000, d)) < 0.01, 10.0, 1.0) * rng.standard_normal((4000, d))
    p = T.Plan(d, (2,) * 7, T.HADAMARD)
    _, _, z = Q.codebook_norm_quantize(T.apply_right(p, x), LM.lloyd_max_gaussian(4)[0], d,
                                       decide_f32=False)
    zz = z.reshape(-1)
    assert abs(zz.mean()) < 0.01
    assert abs(np.mean(zz ** 2) - 1.0) < 1e-12  # exact: sum z^2 = d per block
    assert scipy.stats.kstest(zz[::7], "norm").statistic < 0.02


def test_codebook_dequant_round_trip_mse():
    """Quantize-dequantize of Gaussian blocks: per-coordinate MSE of z close
    to the Lloyd-Max MSE of the codebook."""
    d = 128
    cb, _, mse = LM.lloyd_max_gaussian(4)
    rng = np.random.default_rng(7)
    y = rng.standard_normal((2000, d))
    codes, r, z = Q.codebook_norm_quantize(y, cb, d)
    r16 = r.astype(np.float16)
    yh = Q.codebook_dequant(codes, r16, cb, d)
    zh = np.sqrt(d) * yh / np.repeat(r16.astype(np.float64), d, axis=1)
    assert abs(np.mean((z - zh) ** 2) - mse) < 0.1 * mse


def test_codebook_f32_and_f64_decisions_agree_outside_band():
    cb = LM.lloyd_max_gaussian(4)[0].astype(np.float32)
    rng = np.random.default_rng(8)
    v = rng.standard_normal((64, 512)).astype(np.float32).astype(np.float64)
    c32, _, z = Q.codebook_norm_quantize(v, cb, 128, decide_f32=True)
    c64, _, _ = Q.codebook_norm_quantize(v, cb, 128, decide_f32=False)
    band = Q.codebook_band(z, cb)
    assert np.array_equal(c32[~band], c64[~band])


# ------------------------------------------------------------ packing

@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_pack_matches_bit_extraction(bits):
    rng = np.random.default_rng(30 + bits)
    n = 64
    codes = rng.integers(0, 1 << bits, size=(3, n)).astype(np.uint8)
    packed = Q.pack(codes, bits)
    assert packed.shape == (3, n * bits // 8)
    for r in range(3):
        stream = int.from_bytes(bytes(packed[r]), "little")
        for k in range(n):
            assert (stream >> (k * bits)) & ((1 << bits) - 1) == codes[r, k]
    assert np.array_equal(Q.unpack(packed, bits, n), codes)


def test_pack_small_worked_example():
    """Codes 1,2,3,0,7,5,6,4 at 3 bits, LSB first, worked by hand:
    stream = 1 | 2<<3 | 3<<6 | 0<<9 | 7<<12 | 5<<15 | 6<<18 | 4<<21
    -> bytes 0xD1, 0xF0, 0x9A."""
    codes = np.array([[1, 2, 3, 0, 7, 5, 6, 4]], dtype=np.uint8)
    assert list(Q.pack(codes, 3)[0]) == [0xD1, 0xF0, 0x9A]
