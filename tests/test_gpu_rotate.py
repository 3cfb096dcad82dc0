"""GPU parity of the one-sided rotations against the oracle (small shapes that
span several tiles with ragged tails)."""

import numpy as np
import pytest

import synthetic as S
from oracle import transform as T
from parity import check_rotation
from gpu_util import announce, from_dev, lib_plan, method_for, orc_plan, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

PLANS = [
    ((2,) * 8, "hadamard"),
    ((4, 4, 16), "per_group"),
    ((16, 16), "shared"),
    ((43, 16, 16), "per_group"),
    ((3, 5, 7), "per_group"),
    ((2,) * 12, "hadamard"),
    ((16, 16, 16), "per_group"),
    ((7, 16, 16, 16), "per_group"),
    ((8, 8, 8, 5, 2), "per_group"),
    ((64, 2), "per_group"),
    ((2,) * 7, "hadamard"),
]


def _side(radix, mode, seed=7, signs=True):
    return S.random_plan(np.random.default_rng(seed), radix, mode, with_signs=signs)


def _input(rows, cols, dtype, seed=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols))
    x[:, rng.choice(cols, size=max(1, cols // 100), replace=False)] *= 30.0
    return S.to_storage(x, dtype)


@pytest.mark.parametrize("radix,mode", PLANS)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_right_rotate(radix, mode, dt):
    import butterfly_rotation_quantization_amd as brq
    side = _side(radix, mode)
    d = side.d
    rows = 37 if d <= 4096 else 5
    cols = 2 * d if d <= 512 else d
    announce(f"right rotate radix={radix} mode={mode} dt={dt} rows={rows} cols={cols}")
    xs = _input(rows, cols, dt)
    x = to_dev(xs, dt)
    p = lib_plan(side)
    y = brq.rotate(p, x, side="right")
    ref = T.apply_right(orc_plan(side), S.storage_to_f64(xs, dt), method=method_for(d))
    check_rotation(from_dev(y), ref, dt, f"right {radix}")
    xi = brq.rotate_inverse(p, y.float() if dt == "f32" else y, side="right")
    refi = T.apply_right(orc_plan(side), from_dev(y), inverse=True, method=method_for(d))
    check_rotation(from_dev(xi), refi, dt, f"right inverse {radix}")


# 45 columns: the tile kernels; 64: left stages of power-of-two radix run by
# whole rows (vector accesses need the column count a multiple of 4).
@pytest.mark.parametrize("radix,mode", [p for p in PLANS if np.prod(p[0]) <= 4096])
@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("cols", [45, 64])
def test_left_rotate(radix, mode, dt, cols):
    import butterfly_rotation_quantization_amd as brq
    side = _side(radix, mode, seed=9)
    d = side.d
    announce(f"left rotate radix={radix} mode={mode} dt={dt} cols={cols}")
    xs = _input(d, cols, dt, seed=4)
    x = to_dev(xs, dt)
    p = lib_plan(side)
    y = brq.rotate(p, x, side="left")
    ref = T.apply_left(orc_plan(side), S.storage_to_f64(xs, dt))
    check_rotation(from_dev(y).T, ref.T, dt, f"left {radix}")
    xi = brq.rotate_inverse(p, y, side="left")
    refi = T.apply_left(orc_plan(side), from_dev(y), inverse=True)
    check_rotation(from_dev(xi).T, refi.T, dt, f"left inverse {radix}")


@pytest.mark.parametrize("radix,mode", PLANS)
def test_tile_pass_both_sides(radix, mode):
    """The same rotations with every call on the multi-stage tile pass (the
    kernel that takes any plan and shape)."""
    import butterfly_rotation_quantization_amd as brq
    side = _side(radix, mode, seed=11)
    d = side.d
    rows = 37 if d <= 4096 else 5
    cols = 2 * d if d <= 512 else d
    announce(f"tile pass radix={radix} mode={mode}")
    xs = _input(rows, cols, "f32", seed=5)
    p = lib_plan(side)
    with brq.tile_path():
        y = brq.rotate(p, to_dev(xs, "f32"), side="right")
        xi = brq.rotate_inverse(p, y, side="right")
    ref = T.apply_right(orc_plan(side), xs.astype(np.float64), method=method_for(d))
    check_rotation(from_dev(y), ref, "f32", f"tile right {radix}")
    refi = T.apply_right(orc_plan(side), from_dev(y), inverse=True, method=method_for(d))
    check_rotation(from_dev(xi), refi, "f32", f"tile right inverse {radix}")
    if d <= 4096:
        xl = _input(d, 45, "f32", seed=6)
        with brq.tile_path():
            yl = brq.rotate(p, to_dev(xl, "f32"), side="left")
        refl = T.apply_left(orc_plan(side), xl.astype(np.float64))
        check_rotation(from_dev(yl).T, refl.T, "f32", f"tile left {radix}")


def test_mixed_dtypes_and_in_place():
    import butterfly_rotation_quantization_amd as brq
    torch = pytest.importorskip("torch")
    side = _side((4, 4, 16), "per_group", seed=11)
    xs = _input(19, 512, "bf16", seed=5)
    x = to_dev(xs, "bf16")
    p = lib_plan(side)
    y = torch.empty((19, 512), dtype=torch.float32, device="cuda")
    brq.rotate(p, x, y)
    ref = T.apply_right(orc_plan(side), S.storage_to_f64(xs, "bf16"))
    check_rotation(from_dev(y), ref, "f32", "bf16->f32")
    y16 = torch.empty((19, 512), dtype=torch.float16, device="cuda")
    brq.rotate(p, x, y16)
    check_rotation(from_dev(y16), ref, "f16", "bf16->f16")
    z = x.clone()
    brq.rotate(p, z, z)  # in place, same dtype
    check_rotation(from_dev(z), ref, "bf16", "in place")


def test_leading_dimension_and_empty():
    import butterfly_rotation_quantization_amd as brq
    torch = pytest.importorskip("torch")
    side = _side((16, 16), "per_group", seed=12)
    xs = _input(33, 300, "f32", seed=6)
    big = to_dev(xs, "f32")
    x = big[:, 20:276]  # ld 300 > cols 256
    y_big = torch.zeros((33, 290), dtype=torch.float32, device="cuda")
    y = y_big[:, 10:266]
    brq.rotate(lib_plan(side), x, y)
    ref = T.apply_right(orc_plan(side), xs[:, 20:276].astype(np.float64))
    check_rotation(from_dev(y), ref, "f32", "ld")
    assert not y_big[:, :10].any() and not y_big[:, 266:].any()
    e = torch.empty((0, 256), dtype=torch.float32, device="cuda")
    brq.rotate(lib_plan(side), e, e.clone())


@pytest.mark.parametrize("offset", [4, 2])
def test_left_leading_dimension(offset):
    """Left-side rotation of a column window of a wider matrix: an offset of
    4 floats keeps 16-byte vector accesses (whole-row stages), 2 does not
    (tile kernels); both must match, and the columns outside stay untouched."""
    import butterfly_rotation_quantization_amd as brq
    torch = pytest.importorskip("torch")
    side = _side((32, 16, 16), "per_group", seed=13)
    d = side.d
    xs = _input(d, 100, "f32", seed=8)
    big = to_dev(xs, "f32")
    x = big[:, offset:offset + 64]
    y_big = torch.zeros((d, 100), dtype=torch.float32, device="cuda")
    y = y_big[:, offset:offset + 64]
    brq.rotate(lib_plan(side), x, y, side="left")
    ref = T.apply_left(orc_plan(side), xs[:, offset:offset + 64].astype(np.float64))
    check_rotation(from_dev(y).T, ref.T, "f32", f"left ld offset {offset}")
    assert not y_big[:, :offset].any() and not y_big[:, offset + 64:].any()
    xi = torch.empty_like(y)
    brq.rotate_inverse(lib_plan(side), y.contiguous(), xi, side="left")
    check_rotation(from_dev(xi).T, xs[:, offset:offset + 64].astype(np.float64).T, "f32",
                   f"left ld offset {offset} round trip")


@pytest.mark.parametrize("radix,mode,rows", [((2, 16, 64), "per_group", 16),
                                             ((2, 16, 64), "per_group", 4096),
                                             ((7, 16, 16, 16), "per_group", 24),
                                             ((7, 16, 16, 16), "per_group", 64),
                                             ((4, 16, 64), "hadamard", 40)])
def test_right_stages_in_place(radix, mode, rows):
    """float32 in and out: every stage after the first updates the output in
    place, so a stage whose waves share rows must not write before all have
    read (radix 16 with groups in lanes)."""
    import butterfly_rotation_quantization_amd as brq
    side = _side(radix, mode, seed=21)
    d = side.d
    announce(f"right in place radix={radix} rows={rows}")
    xs = _input(rows, d, "f32", seed=9)
    p = lib_plan(side)
    y = brq.rotate(p, to_dev(xs, "f32"), side="right")
    ref = T.apply_right(orc_plan(side), xs.astype(np.float64), method=method_for(d))
    check_rotation(from_dev(y), ref, "f32", f"in place {radix}")
    xi = brq.rotate_inverse(p, y, side="right")
    check_rotation(from_dev(xi), xs.astype(np.float64), "f32", f"in place inverse {radix}")


@pytest.mark.parametrize("radix,mode,rows,chunks", [
    ((7, 16, 16, 16), "per_group", 1, 1), ((8, 8, 8, 5, 2), "per_group", 3, 1),
    ((2, 16, 64), "shared", 7, 2), ((3, 5, 7), "per_group", 4, 3), ((16, 4, 16), "per_group", 2, 1),
    ((7, 16, 16, 16), "per_group", 13, 1), ((8, 8, 8, 5, 2), "shared", 32, 1),
])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_right_stage_pairs_few_rows(radix, mode, rows, chunks, dt):
    """Up to 32 rows two consecutive stages of radix <= 16 run as one launch
    (outer stage first forward, inner first inverse, with the signs at the
    plan's stage 0): forward and inverse against the oracle."""
    import butterfly_rotation_quantization_amd as brq
    side = _side(radix, mode, seed=rows + chunks)
    d = side.d
    announce(f"right stage pairs radix={radix} mode={mode} rows={rows} dt={dt}")
    xs = _input(rows, chunks * d, dt, seed=rows)
    p = lib_plan(side)
    brq.profile_reset()
    brq.profile_enable(True)
    y = brq.rotate(p, to_dev(xs, dt), side="right")
    names = list(brq.profile_read())
    brq.profile_enable(False)
    assert any("," in n for n in names), names  # a pair launch ran
    ref = T.apply_right(orc_plan(side), S.storage_to_f64(xs, dt), method=method_for(d))
    check_rotation(from_dev(y), ref, dt, f"pairs {radix}")
    xi = brq.rotate_inverse(p, y, side="right")
    refi = T.apply_right(orc_plan(side), from_dev(y), inverse=True, method=method_for(d))
    check_rotation(from_dev(xi), refi, dt, f"pairs inverse {radix}")
