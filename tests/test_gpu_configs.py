"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark times.

Where the dense oracle would take minutes, the comparison uses seeded sampled
rows, which the oracle computes one by one: row r of W' = M_U W M_V^T is
(M_U[r, :] W) M_V^T, with M_U[r, :] = (M_U^T e_r)^T and M_V applied factor by
factor (both pinned equal to the dense definition in the oracle tests).
"""

import numpy as np
import pytest

import synthetic as S
from oracle import lloydmax as LM
from oracle import quant as Q
from oracle import transform as T
from parity import check_absmax_scales, check_codes, check_f16_norms, check_rotation
from gpu_util import announce, from_dev, lib_plan, orc_plan, to_dev

pytestmark = pytest.mark.gpu


_POLAR = {}


def polar_mats():
    """All 7 projections, generated once per session (0.44 GB of bf16)."""
    if not _POLAR:
        _POLAR.update(S.polar())
    return _POLAR


def sampled_rows(m: int, k: int, seed: int) -> np.ndarray:
    return np.sort(np.random.default_rng(seed).choice(m, size=min(k, m), replace=False))


def oracle_rows(left, right, w64, rows):
    """Rows `rows` of M_U W M_V^T (left/right oracle plans or None)."""
    a = w64[rows] if left is None else T.left_rows(left, rows) @ w64
    return a if right is None else T.apply_right(right, a, method="factored")


def unit_rows_of_transpose(plan, rows):
    """Rows `rows` of M^T, i.e. (M e_r)^T."""
    e = np.zeros((len(rows), plan.d))
    e[np.arange(len(rows)), rows] = 1.0
    return T.apply_factored(plan, e)


def check_quantized_rows(codes, scales, y_rows, rows, bits, group, what, kind="absmax", cb=None):
    n = y_rows.shape[1]
    got = Q.unpack(codes.cpu().numpy()[rows], bits, n)
    sc = scales.cpu().numpy()[rows]
    if kind == "absmax":
        ref, _ = Q.absmax_quantize(y_rows, bits, group)
        band = Q.absmax_band(y_rows, bits, group)
        check_absmax_scales(sc, Q.absmax_scales(y_rows, group), y_rows, what)
    else:
        ref, r, z = Q.codebook_norm_quantize(y_rows, cb, group)
        band = Q.codebook_band(z, cb)
        check_f16_norms(sc, r, what)
    info = check_codes(got, ref, band, what, bits)
    assert np.array_equal(Q.pack(got, bits), codes.cpu().numpy()[rows])
    print(what, info, flush=True)
    return got, sc


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_llama7b_two_sided_rht(bits):
    import butterfly_rotation_quantization_amd as brq
    announce(f"7B two-sided RHT 4096x4096 bits={bits}")
    cfg = S.llama7b()
    w = to_dev(cfg["w"], "bf16")
    U, V = lib_plan(cfg["left"]), lib_plan(cfg["right"])
    brq.profile_reset()
    brq.profile_enable(True)
    codes, scales = brq.rotate_quantize_pack(U, V, w, bits, 128)
    brq.profile_enable(False)
    # radix-2^12 Hadamard plans take the two-kernel fast path as (16,16,16)
    assert all(k.startswith("fused") for k in brq.profile_read()), brq.profile_read()
    Uo, Vo = orc_plan(cfg["left"]), orc_plan(cfg["right"])
    w64 = S.storage_to_f64(cfg["w"], "bf16")
    rows = sampled_rows(4096, 512, 7 + bits)
    y = oracle_rows(Uo, Vo, w64, rows)
    got, sc = check_quantized_rows(codes, scales, y, rows, bits, 128, f"7B b{bits}")
    # dequant + unrotate: every row of the result needs every row of codes
    out = brq.dequant_unrotate(U, V, codes, scales, 4096, 4096, bits, 128)
    allc = Q.unpack(codes.cpu().numpy(), bits, 4096)
    v = Q.absmax_dequant(allc, scales.cpu().numpy().astype(np.float64), bits, 128)
    back = T.apply_right(Vo, unit_rows_of_transpose(Uo, rows) @ v, inverse=True,
                         method="factored")
    check_rotation(from_dev(out)[rows], back, "f32", f"7B b{bits} dequant")


def test_llama7b_activations():
    import butterfly_rotation_quantization_amd as brq
    announce("7B activations 2048x4096 bf16 right RHT")
    cfg = S.llama7b()
    x = to_dev(cfg["x"], "bf16")
    V = lib_plan(cfg["right"])
    y = brq.rotate(V, x)
    ref = T.apply_right(orc_plan(cfg["right"]), S.storage_to_f64(cfg["x"], "bf16"))
    check_rotation(from_dev(y), ref, "bf16", "7B activations")


def test_harp_mlp_two_sided():
    """The benchmark workload: 4096 x 11008 bf16, U (16,16,16), V (43,16,16),
    per-group blocks and signs, 3-bit absmax, group 128."""
    import butterfly_rotation_quantization_amd as brq
    announce("HARP MLP 4096x11008 two-sided 3-bit")
    cfg = S.harp_mlp()
    w = to_dev(cfg["w"], "bf16")
    U, V = lib_plan(cfg["left"]), lib_plan(cfg["right"])
    codes, scales = brq.rotate_quantize_pack(U, V, w, 3, 128)
    Uo, Vo = orc_plan(cfg["left"]), orc_plan(cfg["right"])
    w64 = S.storage_to_f64(cfg["w"], "bf16")
    rows = sampled_rows(4096, 384, 11)
    y = oracle_rows(Uo, Vo, w64, rows)
    check_quantized_rows(codes, scales, y, rows, 3, 128, "HARP MLP")
    out = brq.dequant_unrotate(U, V, codes, scales, 4096, 11008, 3, 128)
    allc = Q.unpack(codes.cpu().numpy(), 3, 11008)
    v = Q.absmax_dequant(allc, scales.cpu().numpy().astype(np.float64), 3, 128)
    back = T.apply_right(Vo, unit_rows_of_transpose(Uo, rows) @ v, inverse=True,
                         method="factored")
    check_rotation(from_dev(out)[rows], back, "f32", "HARP MLP dequant")


@pytest.mark.parametrize("name", list(S.POLAR_SHAPES))
def test_polar_projection(name):
    """Every row of the projection: the block-128 oracle is cheap, so codes,
    norms and packing are compared over the whole matrix and the decision
    band's population is that of the whole matrix."""
    import butterfly_rotation_quantization_amd as brq
    announce(f"PolarQuant {name} {S.POLAR_SHAPES[name]}")
    cfg = polar_mats()
    ws = cfg["mats"][name]
    m, n = ws.shape
    cb = LM.lloyd_max_gaussian(4)[0].astype(np.float32)
    w = to_dev(ws, "bf16")
    V = lib_plan(cfg["right"])
    codes, scales = brq.rotate_quantize_pack(None, V, w, 4, 128, "codebook_norm", cb)
    out = brq.dequant_unrotate(None, V, codes, scales, m, n, 4, 128, "codebook_norm", cb,
                               out_dtype=w.dtype)
    codes_h, sc_h, out_h = codes.cpu().numpy(), scales.cpu().numpy(), from_dev(out)
    Vo = orc_plan(cfg["right"])
    gots, refs, bands = [], [], []
    worst = 0.0
    for r0 in range(0, m, 2048):
        rows = slice(r0, min(m, r0 + 2048))
        y = T.apply_right(Vo, S.storage_to_f64(ws[rows], "bf16"))
        ref, r, z = Q.codebook_norm_quantize(y, cb, 128)
        got = Q.unpack(codes_h[rows], 4, n)
        check_f16_norms(sc_h[rows], r, f"polar {name}")
        assert np.array_equal(Q.pack(got, 4), codes_h[rows])
        gots.append(got)
        refs.append(ref)
        bands.append(Q.codebook_band(z, cb))
        back = T.apply_right(Vo, Q.codebook_dequant(got, sc_h[rows], cb, 128), inverse=True)
        info = check_rotation(out_h[rows], back, "bf16", f"polar {name} dequant")
        worst = max(worst, info["max_rel_err"])
    info = check_codes(np.concatenate(gots), np.concatenate(refs), np.concatenate(bands),
                       f"polar {name} (all rows)", 4)
    print(f"polar {name}", info, "dequant max rel err", worst, flush=True)


def test_llama70b_two_sided():
    import butterfly_rotation_quantization_amd as brq
    import torch
    announce("70B 8192x28672 two-sided 2-bit g64")
    cfg = S.llama70b()
    w = to_dev(cfg["w"], "bf16")
    U, V = lib_plan(cfg["left"]), lib_plan(cfg["right"])
    codes, scales = brq.rotate_quantize_pack(U, V, w, 2, 64)
    Uo, Vo = orc_plan(cfg["left"]), orc_plan(cfg["right"])
    rows = sampled_rows(8192, 256, 17)
    w64 = S.storage_to_f64(cfg["w"], "bf16")
    y = oracle_rows(Uo, Vo, w64, rows)
    del w64, w
    check_quantized_rows(codes, scales, y, rows, 2, 64, "70B")
    del y
    # dequant + unrotate at the same shape, on the same sampled rows
    out = brq.dequant_unrotate(U, V, codes, scales, 8192, 28672, 2, 64)
    out_rows = from_dev(out[torch.from_numpy(rows).cuda()])
    del out
    allc = Q.unpack(codes.cpu().numpy(), 2, 28672)
    v = Q.absmax_dequant(allc, scales.cpu().numpy().astype(np.float64), 2, 64)
    del allc
    back = T.apply_right(Vo, unit_rows_of_transpose(Uo, rows) @ v, inverse=True,
                         method="factored")
    check_rotation(out_rows, back, "f32", "70B dequant")


@pytest.mark.parametrize("tokens", [1, 16, 256])
def test_llama70b_decode_activations(tokens):
    import butterfly_rotation_quantization_amd as brq
    announce(f"70B decode activations T={tokens} x 28672 fp16")
    cfg = S.llama70b(rows=1, tokens=(1, 16, 256))
    xs = cfg["acts"][tokens]
    x = to_dev(xs, "f16")
    V = lib_plan(cfg["right"])
    brq.profile_reset()
    brq.profile_enable(True)
    y = brq.rotate(V, x)
    names = list(brq.profile_read())
    brq.profile_enable(False)
    # stages 2 and 3 as one launch; up to 32 tokens stages 0 and 1 as well
    assert len(names) == (2 if tokens <= 32 else 3) and all(n.startswith("stage R(") for n in names), names
    ref = T.apply_right(orc_plan(cfg["right"]), xs.astype(np.float64), method="factored")
    check_rotation(from_dev(y), ref, "f16", f"70B decode T={tokens}")
    xi = brq.rotate_inverse(V, y)
    refi = T.apply_right(orc_plan(cfg["right"]), from_dev(y), inverse=True, method="factored")
    check_rotation(from_dev(xi), refi, "f16", f"70B decode inverse T={tokens}")
