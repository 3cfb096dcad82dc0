"""GPU parity of the ORP GEO quantizer (brq_orp_geo_quantize / _dequant)
against oracle.orp ([ORPQuant] technical summary, section 2).

* b1 codes: bit for bit everywhere.  No rotation precedes this quantizer:
  both sides decide in float32 on the same float32 values, so there is no
  rounding for a decision band to excuse.  Inputs stored in 16 bits put
  many ratios w / alpha exactly on a power-of-two midpoint (about 0.2% of
  bf16 weights); those ties are counted and recorded, and decided the same
  way on both sides (the lower code).
* pair signs: bit for bit on every pair whose two b1 codes agree.
* (c1, c2): |c - c_ref| * ||b1|| <= 2e-5 * ||w_p|| of the group (the
  projection lengths, at the rotation tolerance; float32 sums of g terms).
* dequant: from the GPU's own codes, signs and scales, the float32 output
  equals fl32(c1 b1 + c2 b2) bit for bit (c1 b1 and c2 b2 are exact), and a
  16-bit output equals that float32 value rounded to nearest-even.
"""

import numpy as np
import pytest

import synthetic as S
from oracle import orp as O
from parity import check_codes
from gpu_util import announce, from_dev, to_dev

pytestmark = pytest.mark.gpu

ROT_TOL = 2e-5


def _weights(rng, m, n, outlier_frac=0.005):
    w = 0.02 * rng.standard_t(3, size=(m, n))
    cols = rng.choice(n, size=max(1, int(round(outlier_frac * n))), replace=False)
    w[:, cols] *= 30.0
    return w


def _check(ws, dt, bits, group, stride, smooth=None, what="", out_dts=("f32",)):
    import butterfly_rotation_quantization_amd as brq
    import torch
    m, n = ws.shape
    w64 = S.storage_to_f64(ws, dt)
    wd = to_dev(ws, dt)
    sd = None if smooth is None else torch.from_numpy(smooth.astype(np.float32)).cuda()
    codes, signs, coef = brq.orp_geo_quantize(wd, bits, group, stride, smooth=sd)
    torch.cuda.synchronize()
    c_gpu = codes.cpu().numpy()
    s_gpu = signs.cpu().numpy()
    k_gpu = coef.cpu().numpy().astype(np.float64)
    codes_ref, sigma_ref, coef_ref, b1, b2, wp = O.geo_quantize(w64, bits, group, stride, smooth)
    got = Q_unpack(c_gpu, bits, n)
    ties = int(O.band(wp, bits, group).sum())
    info = check_codes(got, codes_ref, np.zeros(got.shape, dtype=bool), f"ORP {what}", bits)
    info["exact_ties"] = ties
    assert np.array_equal(Q_pack(got, bits), c_gpu)
    sig = O.unpack_signs(s_gpu, n // 2)
    f, s2 = O.pair_index(n, stride)
    agree = (got[:, f] == codes_ref[:, f]) & (got[:, s2] == codes_ref[:, s2])
    bad = (sig != sigma_ref) & agree
    assert not bad.any(), f"ORP {what}: {int(bad.sum())} pair signs differ"
    # scales, as projection lengths against the group norm
    wg = wp.reshape(m, n // group, group)
    nb1 = np.linalg.norm(b1.reshape(m, n // group, group), axis=2)
    nw = np.linalg.norm(wg, axis=2)
    rows_ok = np.ones(m, dtype=bool) if not (got != codes_ref).any() else ~(got != codes_ref).any(axis=1)
    err = np.abs(k_gpu - coef_ref) * nb1[..., None]
    lim = ROT_TOL * nw[..., None] + 1e-30
    assert (err[rows_ok] <= lim[rows_ok]).all(), \
        f"ORP {what}: scale error {float((err / lim).max()):.3g} x the tolerance"
    # dequant from the GPU's own outputs
    gb1, gb2 = O.basis_from_codes(got, sig, bits, stride)
    exact = (np.repeat(k_gpu[..., 0], group, axis=1) * gb1 +
             np.repeat(k_gpu[..., 1], group, axis=1) * gb2)
    ref32 = exact.astype(np.float32)
    for odt in out_dts:
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[odt]
        out = from_dev(brq.orp_geo_dequant(codes, signs, coef, m, n, bits, group, stride,
                                           out_dtype=tdt))
        want = ref32.astype(np.float64) if odt == "f32" else \
            S.storage_to_f64(S.to_storage(ref32.astype(np.float64), odt), odt)
        assert np.array_equal(out, want), \
            f"ORP {what}: dequant {odt} differs at {int((out != want).sum())} elements"
    print(f"ORP {what}", info, flush=True)
    return info


def Q_unpack(packed, bits, n):
    from oracle import quant as Q
    return Q.unpack(packed, bits, n)


def Q_pack(codes, bits):
    from oracle import quant as Q
    return Q.pack(codes, bits)


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
@pytest.mark.parametrize("stride", [1, 2, 4, 8, 32])
def test_orp_bits_and_strides(bits, stride):
    rng = np.random.default_rng(100 * bits + stride)
    m, n, group = 24, 1536, 128
    ws = S.to_storage(_weights(rng, m, n), "bf16")
    announce(f"ORP bits={bits} stride={stride} {m}x{n} g{group}")
    _check(ws, "bf16", bits, group, stride, what=f"b{bits} S{stride}", out_dts=("f32", "bf16"))


@pytest.mark.parametrize("group,stride", [(64, 32), (256, 128), (512, 256), (512, 1), (64, 1)])
def test_orp_groups(group, stride):
    rng = np.random.default_rng(group + stride)
    m, n = 16, 3072
    ws = S.to_storage(_weights(rng, m, n), "f16")
    announce(f"ORP group={group} stride={stride}")
    _check(ws, "f16", 3, group, stride, what=f"g{group} S{stride}", out_dts=("f32", "f16"))


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_orp_dtypes_ragged_chunk_and_smoothing(dt):
    """n = 11008: the last 512-element chunk of each row is half empty;
    with a per-input-channel smoothing vector."""
    rng = np.random.default_rng(7)
    m, n = 9, 11008
    ws = S.to_storage(_weights(rng, m, n), dt)
    smooth = rng.uniform(0.25, 4.0, size=n)
    announce(f"ORP {dt} {m}x{n} smoothing")
    _check(ws, dt, 3, 128, 4, smooth=smooth, what=f"{dt} smooth", out_dts=(dt,))
    _check(ws, dt, 4, 64, 16, what=f"{dt} ragged")


def test_orp_zero_groups_and_empty():
    import butterfly_rotation_quantization_amd as brq
    import torch
    rng = np.random.default_rng(8)
    m, n = 8, 1024
    w = _weights(rng, m, n)
    w[2, :] = 0.0
    w[5, 128:256] = 0.0
    ws = S.to_storage(w, "f32")
    announce("ORP zero groups")
    _check(ws, "f32", 3, 128, 2, what="zero groups")
    empty = torch.empty((0, n), dtype=torch.float32, device="cuda")
    c, s, k = brq.orp_geo_quantize(empty, 3, 128, 2)
    assert c.shape == (0, n * 3 // 8)


def test_orp_rejects_bad_arguments():
    import butterfly_rotation_quantization_amd as brq
    import torch
    w = torch.zeros((4, 256), dtype=torch.float32, device="cuda")
    for bits, group, stride in [(6, 128, 2), (3, 96, 2), (3, 128, 3), (3, 128, 128)]:
        with pytest.raises(brq.BrqError):
            brq.orp_geo_quantize(w, bits, group, stride)


@pytest.mark.parametrize("shape", [(4096, 4096), (4096, 11008)])
def test_orp_full_size(shape):
    """Weights of the 7B (4096 x 4096) and MLP (4096 x 11008) shapes, bf16,
    3 bits (the page's W3 setting), groups of 128, stride 4: every element."""
    rng = np.random.default_rng(shape[1])
    ws = S.to_storage(_weights(rng, *shape), "bf16")
    announce(f"ORP full size {shape}")
    info = _check(ws, "bf16", 3, 128, 4, what=f"full {shape[0]}x{shape[1]}")
    assert info["mismatches"] == 0
