"""GPU parity of rotate+quantize+pack and dequant+unrotate against the oracle
on small shapes (the Tiny workload and variations of it)."""

import contextlib

import numpy as np
import pytest

import synthetic as S
from oracle import lloydmax as LM
from oracle import quant as Q
from oracle import transform as T
from parity import check_absmax_scales, check_codes, check_f16_norms, check_rotation
from gpu_util import announce, from_dev, lib_plan, orc_plan, to_dev

pytestmark = pytest.mark.gpu


def kernels(path):
    """The automatic kernel choice, or every call on the multi-stage tile pass."""
    import butterfly_rotation_quantization_amd as brq
    return brq.tile_path() if path == "tile" else contextlib.nullcontext()


def run_case(w_store, dtype, left, right, bits, group, kind="absmax", codebook=None,
             what="", method="dense"):
    """Quantize on the GPU and check codes, packed bytes, scales, then the
    dequant+unrotate of the GPU's own codes against the oracle's."""
    import butterfly_rotation_quantization_amd as brq
    m, n = w_store.shape
    w = to_dev(w_store, dtype)
    Lp = lib_plan(left) if left is not None else None
    Rp = lib_plan(right) if right is not None else None
    codes, scales = brq.rotate_quantize_pack(Lp, Rp, w, bits, group, kind, codebook)
    codes_np = codes.cpu().numpy()
    Lo = orc_plan(left) if left is not None else None
    Ro = orc_plan(right) if right is not None else None
    y = T.two_sided(Lo, Ro, S.storage_to_f64(w_store, dtype), method=method)
    got = Q.unpack(codes_np, bits, n)
    if kind == "absmax":
        ref, alpha = Q.absmax_quantize(y, bits, group)
        band = Q.absmax_band(y, bits, group)
        check_absmax_scales(scales.cpu().numpy(), Q.absmax_scales(y, group), y, what)
    else:
        ref, r, z = Q.codebook_norm_quantize(y, codebook, group)
        band = Q.codebook_band(z, codebook)
        check_f16_norms(scales.cpu().numpy(), r, what)
    info = check_codes(got, ref, band, what, bits)
    # packed stream: identical bytes to the oracle's packing of the same codes
    assert np.array_equal(Q.pack(got, bits), codes_np), f"{what}: packing layout differs"
    # inverse: both sides dequantize the GPU's codes and scales
    out = brq.dequant_unrotate(Lp, Rp, codes, scales, m, n, bits, group, kind, codebook)
    if kind == "absmax":
        v = Q.absmax_dequant(got, scales.cpu().numpy().astype(np.float64), bits, group)
    else:
        v = Q.codebook_dequant(got, scales.cpu().numpy(), codebook, group)
    back = T.two_sided_inverse(Lo, Ro, v, method=method)
    check_rotation(from_dev(out), back, "f32", what + " dequant")
    return info


@pytest.mark.parametrize("path", ["auto", "tile"])
def test_tiny_rht_and_harp(path):
    cfg = S.tiny()
    for name in ("rht", "harp"):
        announce(f"tiny {name} path={path}")
        with kernels(path):
            info = run_case(cfg["w"], "f32", None, cfg[name], cfg["bits"], cfg["group"],
                            what=f"tiny {name} {path}")
        print(name, info)


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
@pytest.mark.parametrize("group", [64, 128, 256])
def test_absmax_bits_groups(bits, group):
    rng = np.random.default_rng(bits * 100 + group)
    right = S.random_plan(rng, (4, 4, 16), "per_group")
    w = S.to_storage(0.02 * rng.standard_t(3, size=(45, 1024)), "bf16")
    announce(f"absmax bits={bits} group={group}")
    run_case(w, "bf16", None, right, bits, group, what=f"b{bits} g{group}")


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_codebook_norm(bits):
    rng = np.random.default_rng(40 + bits)
    cb = LM.lloyd_max_gaussian(bits)[0].astype(np.float32)
    right = S.SidePlan(128, (2,) * 7, "hadamard", None, None)
    w = S.to_storage(S.gaussian_mixture_weights(rng, 40, 512), "bf16")
    announce(f"codebook bits={bits}")
    run_case(w, "bf16", None, right, bits, 128, "codebook_norm", cb, what=f"cb{bits}")


@pytest.mark.parametrize("path", ["auto", "tile"])
def test_two_sided_small(path):
    rng = np.random.default_rng(50)
    left = S.random_plan(rng, (4, 4, 4), "per_group")
    right = S.random_plan(rng, (43, 16, 4), "per_group")
    w = S.to_storage(0.02 * rng.standard_t(3, size=(64, 2752)), "bf16")
    announce(f"two-sided small (4,4,4) x (43,16,4) path={path}")
    with kernels(path):
        run_case(w, "bf16", left, right, 3, 64, what=f"two-sided {path}")


@pytest.mark.parametrize("path", ["auto", "tile"])
def test_left_only_and_quant_only(path):
    rng = np.random.default_rng(51)
    left = S.random_plan(rng, (16, 8), "per_group")
    w = S.to_storage(rng.standard_normal((128, 320)), "f32")
    with kernels(path):
        announce(f"left only path={path}")
        run_case(w, "f32", left, None, 4, 64, what=f"left only {path}")
        announce(f"quant only path={path}")
        run_case(w, "f32", None, None, 3, 64, what=f"quant only {path}")


@pytest.mark.parametrize("path", ["auto", "tile"])
def test_zero_groups_and_ragged_rows(path):
    rng = np.random.default_rng(52)
    right = S.random_plan(rng, (16, 16), "per_group")
    x = rng.standard_normal((13, 512))
    x[3, :] = 0.0
    x[7, 256:] = 0.0
    w = S.to_storage(x, "f32")
    announce(f"zero groups path={path}")
    with kernels(path):
        run_case(w, "f32", None, right, 4, 128, what=f"zero groups {path}")


@pytest.mark.parametrize("bits,group", [(2, 64), (4, 128)])
def test_stage_head_pass_b_tail(bits, group):
    """Dense schedules ending in (16, 16) on both sides run as stage passes
    for the earlier stages and pass B for the last four and the quantizer
    (the 70B weight's route), here on a full matrix the oracle covers."""
    import butterfly_rotation_quantization_amd as brq
    rng = np.random.default_rng(60 + bits)
    left = S.random_plan(rng, (4, 16, 16), "per_group")
    right = S.random_plan(rng, (3, 16, 16, 16), "per_group")
    w = S.to_storage(0.02 * rng.standard_t(3, size=(1024, 12288)), "bf16")
    announce(f"stage head + pass B tail b{bits} g{group}")
    brq.profile_reset()
    brq.profile_enable(True)
    info = run_case(w, "bf16", left, right, bits, group, what=f"tail b{bits} g{group}",
                    method="factored")
    names = list(brq.profile_read())
    brq.profile_enable(False)
    assert any(n.startswith("fusedB") for n in names), names
    print(info)
