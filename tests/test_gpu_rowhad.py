"""GPU parity of the row Hadamard path (right-side Hadamard plans with
16 <= d <= 4096, one pass per call) against the oracle: rotate and its
inverse in every dtype pair, rotate + quantize + pack for both quantizers
over bit widths and group sizes, and dequant + unrotate.  Row counts make the
last workgroup partial; each case checks that the row Hadamard kernel ran."""

import numpy as np
import pytest

import synthetic as S
from oracle import lloydmax as LM
from oracle import quant as Q
from oracle import transform as T
from parity import check_absmax_scales, check_codes, check_f16_norms, check_rotation
from gpu_util import announce, from_dev, lib_plan, orc_plan, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def _hadamard(l2d, seed, signs=True):
    rng = np.random.default_rng(seed)
    d = 1 << l2d
    return S.SidePlan(d, (2,) * l2d, "hadamard", None, S.signs(rng, d) if signs else None)


def _input(rows, cols, dtype, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols))
    x[:, rng.choice(cols, size=max(1, cols // 64), replace=False)] *= 25.0
    return S.to_storage(x, dtype)


def _ran_rowhad():
    import butterfly_rotation_quantization_amd as brq
    names = list(brq.profile_read())
    brq.profile_enable(False)
    assert names and all(k.startswith("rowhad") for k in names), names


def _profile_on():
    import butterfly_rotation_quantization_amd as brq
    brq.profile_reset()
    brq.profile_enable(True)


# (log2 d, rows, chunks per row, input dtype, output dtype, signs)
ROT = [
    (4, 33, 2, "bf16", "bf16", True),
    (5, 129, 3, "f32", "f32", True),
    (7, 50, 4, "bf16", "f32", False),
    (8, 17, 2, "f16", "f16", True),
    (10, 9, 2, "f32", "bf16", True),
    (11, 6, 1, "bf16", "f16", True),
    (12, 37, 1, "bf16", "bf16", True),
    (12, 3, 2, "f32", "f32", True),
]


@pytest.mark.parametrize("l2d,rows,cpr,xt,yt,signs", ROT)
def test_rowhad_rotate(l2d, rows, cpr, xt, yt, signs):
    import butterfly_rotation_quantization_amd as brq
    torch = pytest.importorskip("torch")
    side = _hadamard(l2d, 10 + l2d, signs)
    cols = cpr * side.d
    announce(f"rowhad rotate d={side.d} rows={rows} cols={cols} {xt}->{yt}")
    xs = _input(rows, cols, xt, l2d)
    x = to_dev(xs, xt)
    p = lib_plan(side)
    y = torch.empty((rows, cols), dtype=torch_dtype(yt), device="cuda")
    _profile_on()
    brq.rotate(p, x, y, side="right")
    _ran_rowhad()
    Po = orc_plan(side)
    ref = T.apply_right(Po, S.storage_to_f64(xs, xt), method="factored")
    check_rotation(from_dev(y), ref, yt, f"rowhad d={side.d}")
    xi = torch.empty((rows, cols), dtype=torch_dtype(yt), device="cuda")
    _profile_on()
    brq.rotate_inverse(p, y, xi, side="right")
    _ran_rowhad()
    refi = T.apply_right(Po, from_dev(y), inverse=True, method="factored")
    check_rotation(from_dev(xi), refi, yt, f"rowhad inverse d={side.d}")


# (log2 d, rows, chunks per row, bits, group, kind, dtype)
QNT = [
    (7, 40, 32, 4, 128, "codebook_norm", "bf16"),
    (7, 13, 96, 4, 128, "codebook_norm", "bf16"),
    (12, 19, 1, 3, 128, "absmax", "bf16"),
    (8, 11, 8, 2, 64, "absmax", "f32"),
    (5, 30, 64, 5, 256, "absmax", "f16"),
    (10, 7, 4, 4, 1024, "codebook_norm", "bf16"),
    (4, 70, 64, 3, 64, "absmax", "bf16"),
    (6, 21, 16, 2, 512, "codebook_norm", "f32"),
    (9, 5, 2, 5, 64, "codebook_norm", "bf16"),
]


@pytest.mark.parametrize("l2d,rows,cpr,bits,group,kind,dt", QNT)
def test_rowhad_quant_dequant(l2d, rows, cpr, bits, group, kind, dt):
    import butterfly_rotation_quantization_amd as brq
    side = _hadamard(l2d, 20 + l2d, signs=(kind == "absmax"))
    n = cpr * side.d
    announce(f"rowhad quant d={side.d} rows={rows} n={n} b{bits} g{group} {kind} {dt}")
    rng = np.random.default_rng(100 * l2d + bits)
    ws = S.to_storage(S.gaussian_mixture_weights(rng, rows, n), dt)
    cb = LM.lloyd_max_gaussian(bits)[0].astype(np.float32) if kind == "codebook_norm" else None
    p = lib_plan(side)
    _profile_on()
    codes, scales = brq.rotate_quantize_pack(None, p, to_dev(ws, dt), bits, group, kind, cb)
    _ran_rowhad()
    Po = orc_plan(side)
    y = T.apply_right(Po, S.storage_to_f64(ws, dt), method="factored")
    got = Q.unpack(codes.cpu().numpy(), bits, n)
    what = f"rowhad d={side.d} b{bits} g{group} {kind}"
    if kind == "absmax":
        ref, _ = Q.absmax_quantize(y, bits, group)
        band = Q.absmax_band(y, bits, group)
        check_absmax_scales(scales.cpu().numpy(), Q.absmax_scales(y, group), y, what)
    else:
        ref, r, z = Q.codebook_norm_quantize(y, cb, group)
        band = Q.codebook_band(z, cb)
        check_f16_norms(scales.cpu().numpy(), r, what)
    info = check_codes(got, ref, band, what, bits)
    assert np.array_equal(Q.pack(got, bits), codes.cpu().numpy())
    _profile_on()
    out = brq.dequant_unrotate(None, p, codes, scales, rows, n, bits, group, kind, cb)
    _ran_rowhad()
    if kind == "absmax":
        v = Q.absmax_dequant(got, scales.cpu().numpy().astype(np.float64), bits, group)
    else:
        v = Q.codebook_dequant(got, scales.cpu().numpy(), cb, group)
    back = T.apply_right(Po, v, inverse=True, method="factored")
    check_rotation(from_dev(out), back, "f32", what + " dequant")
    print(info, flush=True)
