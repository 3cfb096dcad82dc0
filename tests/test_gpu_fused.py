"""GPU parity of the two-kernel fast path (left (16,16,16) over 4096 rows,
right (bv,16,16) per row chunk) for the radix, block mode, dtype, bit width
and group variants it covers; sampled rows against the oracle."""

import numpy as np
import pytest

import synthetic as S
from oracle import lloydmax as LM
from oracle import quant as Q
from oracle import transform as T
from parity import check_absmax_scales, check_codes, check_f16_norms
from gpu_util import announce, lib_plan, orc_plan, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    (43, "per_group", 1, 3, 128, "bf16", "absmax"),
    (16, "per_group", 1, 4, 128, "f32", "absmax"),
    (32, "shared", 1, 2, 64, "f16", "absmax"),
    (64, "per_group", 1, 5, 128, "bf16", "absmax"),
    (7, "per_group", 2, 4, 64, "bf16", "absmax"),
    (16, "hadamard", 1, 2, 128, "bf16", "absmax"),
    (43, "per_group", 1, 4, 128, "bf16", "codebook_norm"),
]


@pytest.mark.parametrize("bv,mode,chunks,bits,group,dt,kind", CASES)
def test_fused_two_sided(bv, mode, chunks, bits, group, dt, kind):
    import butterfly_rotation_quantization_amd as brq
    announce(f"fused bv={bv} {mode} chunks={chunks} b{bits} g{group} {dt} {kind}")
    rng = np.random.default_rng(1000 + bv)
    umode = "hadamard" if mode == "hadamard" else "per_group"
    left = S.random_plan(rng, (16, 16, 16), umode)
    right = S.random_plan(rng, (bv, 16, 16), mode)
    m, n = 4096, bv * 256 * chunks
    x = 0.02 * rng.standard_t(3, size=(m, n))
    x[:, rng.choice(n, size=n // 200, replace=False)] *= 30.0
    ws = S.to_storage(x, dt)
    w = to_dev(ws, dt)
    cb = LM.lloyd_max_gaussian(bits)[0].astype(np.float32) if kind == "codebook_norm" else None
    U, V = lib_plan(left), lib_plan(right)
    brq.profile_reset()
    brq.profile_enable(True)
    codes, scales = brq.rotate_quantize_pack(U, V, w, bits, group, kind, cb)
    brq.profile_enable(False)
    names = list(brq.profile_read())
    assert len(names) == 2 and all(k.startswith("fused") for k in names), names
    Uo, Vo = orc_plan(left), orc_plan(right)
    rows = np.sort(rng.choice(m, size=128, replace=False))
    y = T.left_rows(Uo, rows) @ S.storage_to_f64(ws, dt)
    y = T.apply_right(Vo, y, method="factored")
    got = Q.unpack(codes.cpu().numpy()[rows], bits, n)
    sc = scales.cpu().numpy()[rows]
    if kind == "absmax":
        ref, _ = Q.absmax_quantize(y, bits, group)
        band = Q.absmax_band(y, bits, group)
        check_absmax_scales(sc, Q.absmax_scales(y, group), y, "fused")
    else:
        ref, r, z = Q.codebook_norm_quantize(y, cb, group)
        band = Q.codebook_band(z, cb)
        check_f16_norms(sc, r, "fused")
    info = check_codes(got, ref, band, "fused", bits)
    assert np.array_equal(Q.pack(got, bits), codes.cpu().numpy()[rows])
    print(info, flush=True)


def test_fused_deterministic_and_matches_generic():
    """Same inputs twice give identical bytes; the other routes for the same
    plans agree outside the decision band: stage passes + pass B (taken for an
    input whose rows are only 8-byte aligned) and the multi-stage tile pass."""
    import butterfly_rotation_quantization_amd as brq
    torch = pytest.importorskip("torch")
    announce("fused determinism and agreement with the other routes")
    cfg = S.harp_mlp()
    U, V = lib_plan(cfg["left"]), lib_plan(cfg["right"])
    w = to_dev(cfg["w"], "bf16")
    c1, s1 = brq.rotate_quantize_pack(U, V, w, 3, 128)
    c2, s2 = brq.rotate_quantize_pack(U, V, w, 3, 128)
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    a = Q.unpack(c1.cpu().numpy(), 3, 11008)
    # a copy with leading dimension n + 4 (8-byte row alignment): pass A does
    # not take it, so stage passes apply the first stages and pass B the rest
    wide = torch.zeros((4096, 11008 + 4), dtype=torch.bfloat16, device="cuda")
    wide[:, :11008] = w
    for route in ("stages + pass B", "tile pass"):
        brq.profile_reset()
        brq.profile_enable(True)
        if route == "tile pass":
            with brq.tile_path():
                c3, s3 = brq.rotate_quantize_pack(U, V, w, 3, 128)
        else:
            c3, s3 = brq.rotate_quantize_pack(U, V, wide[:, :11008], 3, 128)
        names = list(brq.profile_read())
        brq.profile_enable(False)
        if route == "tile pass":
            assert all(k.startswith("pass") for k in names), names
        else:
            assert names[-1].startswith("fusedB") and all(k.startswith("stage") for k in names[:-1]), names
        b = Q.unpack(c3.cpu().numpy(), 3, 11008)
        diff = a != b
        assert diff.mean() < 1e-5, (route, diff.sum())
        rel = (s1 - s3).abs().max().item() / s1.abs().max().item()
        assert rel < 1e-5, (route, rel)


LONGER = [
    ((32, 16, 16), (7, 16, 16), 3, 128, "bf16"),
    ((32, 16, 16), (3, 2, 16, 16), 4, 64, "f16"),
    ((16, 2, 16, 16), (16, 16, 16), 2, 128, "f32"),
]


@pytest.mark.parametrize("uradix,vradix,bits,group,dt", LONGER)
def test_fused_longer_schedules(uradix, vradix, bits, group, dt):
    """Stage 0 of radix 32 on the left, stages between stage 0 and the last
    two (run as stage passes between pass A and pass B): sampled rows against
    the oracle."""
    import butterfly_rotation_quantization_amd as brq
    announce(f"fused longer {uradix} x {vradix} b{bits} g{group} {dt}")
    rng = np.random.default_rng(7 + bits)
    left = S.random_plan(rng, uradix, "per_group")
    right = S.random_plan(rng, vradix, "per_group")
    m, n = left.d, right.d
    x = 0.02 * rng.standard_t(3, size=(m, n))
    x[:, rng.choice(n, size=max(1, n // 200), replace=False)] *= 30.0
    ws = S.to_storage(x, dt)
    w = to_dev(ws, dt)
    U, V = lib_plan(left), lib_plan(right)
    brq.profile_reset()
    brq.profile_enable(True)
    codes, scales = brq.rotate_quantize_pack(U, V, w, bits, group)
    brq.profile_enable(False)
    names = list(brq.profile_read())
    assert names[0].startswith("fusedA") and names[-1].startswith("fusedB"), names
    assert len(names) == 2 + (len(uradix) - 3) + (len(vradix) - 3), names
    Uo, Vo = orc_plan(left), orc_plan(right)
    rows = np.sort(rng.choice(m, size=96, replace=False))
    y = T.left_rows(Uo, rows) @ S.storage_to_f64(ws, dt)
    y = T.apply_right(Vo, y, method="factored")
    got = Q.unpack(codes.cpu().numpy()[rows], bits, n)
    ref, _ = Q.absmax_quantize(y, bits, group)
    band = Q.absmax_band(y, bits, group)
    check_absmax_scales(scales.cpu().numpy()[rows], Q.absmax_scales(y, group), y, "fused longer")
    info = check_codes(got, ref, band, "fused longer", bits)
    print(info, flush=True)
