"""GPU parity of the quantized linear layer at decode (brq_qlinear) against
oracle.linear.  Codes and scales are seeded inputs given to both sides.  The
oracle rotates the activations in float64 and rounds them to the activation
type, as the library does; a rounding there may land one ulp apart, so the
tolerance is the error bound that follows: one ulp of each rotated
activation (floored at the float32 rotation tolerance) times |W'|, plus the
float32 accumulation, plus the output rotation and the output rounding."""

import numpy as np
import pytest

import synthetic as S
from oracle import linear as OL
from oracle import quant as Q
from oracle import transform as T
from gpu_util import announce, from_dev, lib_plan, method_for, orc_plan, to_dev

pytestmark = pytest.mark.gpu

ROT_TOL = 2e-5


def _ulp(v, mant):
    """One ulp (2^(e - mant)) at |v|, normal range of f16 (mant 10) / bf16 (7)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - mant)


def _case(rng, T_, m, n, bits, group):
    codes = rng.integers(0, 256, size=(m, n * bits // 8), dtype=np.int64).astype(np.uint8)
    alpha = (0.5 + rng.random((m, n // group))).astype(np.float32) * 0.05
    x = rng.standard_normal((T_, n))
    x[:, rng.choice(n, size=max(1, n // 200), replace=False)] *= 20.0
    return codes, alpha, x


def _check(y, xs, dt, U, V, codes, alpha, bits, group, out_dt, what):
    mant = 10 if dt == "f16" else 7
    x64 = S.storage_to_f64(xs, dt)
    xt = OL.rotate_acts(V, x64)
    xt16 = S.storage_to_f64(S.to_storage(xt, dt), dt)
    y_ref, z_ref = OL.qlinear(U, V, xt16, Q.unpack(codes, bits, xs.shape[1]), alpha.astype(np.float64),
                              bits, group)
    w = np.abs(OL.weight(Q.unpack(codes, bits, xs.shape[1]), alpha.astype(np.float64), bits, group))
    nx = np.linalg.norm(x64, axis=1)[:, None]
    dx = np.maximum(_ulp(xt, mant), ROT_TOL * nx) if V is not None else 0.0 * xt
    bound_z = (dx + np.abs(xt16) * xs.shape[1] * 2.0 ** -23) @ w.T + 1e-30
    out_mant = {"f32": 23, "f16": 10, "bf16": 7}[out_dt]
    if U is None:
        err = np.abs(y - z_ref)
        tol = bound_z + (_ulp(z_ref, out_mant) if out_dt != "f32" else 0.0)
        assert (err <= tol).all(), f"{what}: worst {float((err / tol).max()):.3g} x the bound"
    else:
        err = np.linalg.norm(y - y_ref, axis=1)
        tol = (np.linalg.norm(bound_z, axis=1) + ROT_TOL * np.linalg.norm(y_ref, axis=1) +
               (np.linalg.norm(_ulp(y_ref, out_mant), axis=1) if out_dt != "f32" else 0.0))
        assert (err <= tol).all(), f"{what}: worst {float((err / tol).max()):.3g} x the bound"


@pytest.mark.parametrize("T_", [1, 16, 37])
@pytest.mark.parametrize("bits,group", [(2, 64), (4, 128), (3, 64)])
@pytest.mark.parametrize("sides", ["both", "none"])
def test_qlinear_small(T_, bits, group, sides):
    import butterfly_rotation_quantization_amd as brq
    rng = np.random.default_rng(T_ * 10 + bits)
    m, n = 256, 1792
    codes, alpha, x = _case(rng, T_, m, n, bits, group)
    dt = "f16"
    xs = S.to_storage(x, dt)
    Ls = S.random_plan(rng, (16, 16), "per_group") if sides == "both" else None
    Rs = S.random_plan(rng, (7, 16, 16), "per_group") if sides == "both" else None
    announce(f"qlinear T={T_} m={m} n={n} b{bits} g{group} {sides}")
    U, V = (lib_plan(Ls), lib_plan(Rs)) if sides == "both" else (None, None)
    y = brq.qlinear(U, V, to_dev(xs, dt), to_dev(codes, "u8"), to_dev(alpha, "f32"), m, n, bits,
                    group)
    Uo, Vo = (orc_plan(Ls), orc_plan(Rs)) if sides == "both" else (None, None)
    _check(from_dev(y), xs, dt, Uo, Vo, codes, alpha, bits, group, dt, f"T={T_} b{bits} {sides}")


@pytest.mark.parametrize("T_", [1, 37])
@pytest.mark.parametrize("bits,group", [(2, 64), (3, 64), (4, 128), (5, 64)])
@pytest.mark.parametrize("n", [1024, 3584])
def test_qlinear_stream_chunks(T_, bits, group, n):
    """n a multiple of the 512-input chunk: the weight rows pass through LDS
    (when the staging fits), with one or several chunks per split and fewer
    chunks than the split target."""
    import butterfly_rotation_quantization_amd as brq
    rng = np.random.default_rng(T_ * 100 + bits * 10 + n)
    m = 512
    codes, alpha, x = _case(rng, T_, m, n, bits, group)
    xs = S.to_storage(x, "f16")
    Rs = S.random_plan(rng, (n // 256, 16, 16), "per_group")
    announce(f"qlinear stream T={T_} m={m} n={n} b{bits} g{group}")
    y = brq.qlinear(None, lib_plan(Rs), to_dev(xs, "f16"), to_dev(codes, "u8"), to_dev(alpha, "f32"),
                    m, n, bits, group)
    _check(from_dev(y), xs, "f16", None, orc_plan(Rs), codes, alpha, bits, group, "f16",
           f"stream T={T_} b{bits} n={n}")


def test_qlinear_bf16_and_f32_out():
    import butterfly_rotation_quantization_amd as brq
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    m, n, bits, group = 256, 1024, 2, 64
    codes, alpha, x = _case(rng, 9, m, n, bits, group)
    xs = S.to_storage(x, "bf16")
    Rs = S.random_plan(rng, (4, 16, 16), "per_group")
    y = brq.qlinear(None, lib_plan(Rs), to_dev(xs, "bf16"), to_dev(codes, "u8"), to_dev(alpha, "f32"),
                    m, n, bits, group, out_dtype=torch.float32)
    _check(from_dev(y), xs, "bf16", None, orc_plan(Rs), codes, alpha, bits, group, "f32", "bf16 in")


@pytest.mark.parametrize("T_", [1, 16, 256])
def test_qlinear_70b_down_proj(T_):
    """The 70B down projection: 8192 outputs, 28672 inputs, left (32,16,16),
    right (7,16,16,16), 2-bit g64, f16 activations."""
    import butterfly_rotation_quantization_amd as brq
    rng = np.random.default_rng(700 + T_)
    cfg_rng = np.random.default_rng(5000)
    m, n, bits, group = 8192, 28672, 2, 64
    codes, alpha, x = _case(rng, T_, m, n, bits, group)
    xs = S.to_storage(x, "f16")
    Ls = S.random_plan(cfg_rng, (32, 16, 16), "per_group")
    Rs = S.random_plan(cfg_rng, (7, 16, 16, 16), "per_group")
    announce(f"qlinear 70B down_proj T={T_}")
    y = brq.qlinear(lib_plan(Ls), lib_plan(Rs), to_dev(xs, "f16"), to_dev(codes, "u8"),
                    to_dev(alpha, "f32"), m, n, bits, group)
    _check(from_dev(y), xs, "f16", orc_plan(Ls), orc_plan(Rs), codes, alpha, bits, group, "f16",
           f"70B T={T_}")


@pytest.mark.parametrize("T_", [1, 37])
def test_qlinear_direct_kernel_matches_stream(T_):
    """Codes 4 bytes off a 16-byte boundary take the direct kernel, aligned
    codes the streaming one.  Both form each group's sum with the same MFMA
    steps on the same operands and add a split's groups in the same order,
    so the two outputs agree bit for bit (and the aligned one with the
    oracle)."""
    import butterfly_rotation_quantization_amd as brq
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(90 + T_)
    m, n, bits, group = 512, 2048, 2, 64
    codes, alpha, x = _case(rng, T_, m, n, bits, group)
    xs = S.to_storage(x, "f16")
    Ls = S.random_plan(rng, (32, 16), "per_group")
    Rs = S.random_plan(rng, (8, 16, 16), "per_group")
    announce(f"qlinear direct vs stream T={T_}")
    U, V = lib_plan(Ls), lib_plan(Rs)
    xd, sd = to_dev(xs, "f16"), to_dev(alpha, "f32")
    aligned = to_dev(codes, "u8")
    buf = torch.zeros(codes.size + 16, dtype=torch.uint8, device="cuda")
    shifted = buf[4:4 + codes.size].view(m, -1)
    shifted.copy_(aligned)
    assert aligned.data_ptr() % 16 == 0 and shifted.data_ptr() % 16 == 4
    y1 = brq.qlinear(U, V, xd, aligned, sd, m, n, bits, group)
    y2 = brq.qlinear(U, V, xd, shifted, sd, m, n, bits, group)
    assert torch.equal(y1, y2)
    _check(from_dev(y1), xs, "f16", orc_plan(Ls), orc_plan(Rs), codes, alpha, bits, group, "f16",
           f"direct vs stream T={T_}")
