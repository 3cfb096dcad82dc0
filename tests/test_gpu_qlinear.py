"""GPU parity of the quantized linear layer at decode (brq_qlinear) against
oracle.linear, one step at a time.  Codes and scales are seeded inputs given
to both sides.

* X~ = X M_V^T: the library leaves its rotated activations at the start of
  the workspace; they are checked against the oracle's rotation at the
  16-bit rule (one ulp plus the float32 allowance).
* Z = X~ W'^T: the GPU's own X~ goes into the oracle, so the product is
  judged alone, element by element, against the probabilistic float32
  accumulation bound gamma~_p(8) * sum |x~ w| with p the roundings along a
  group-blocked path (tests/parity.py; at 28672 inputs the bound is about
  1e-3 of |z|, and tests/test_parity_rules.py shows that one dropped split
  part or one doubled group scale fails it).  Z is read from a call without
  the left plan and with float32 output, which runs the same product and
  reduction.
* Y: with a left plan, Y = Z M_U is checked against the oracle's inverse
  rotation of that Z at the rotation rule; without one, Y must be the
  round-to-nearest-even of Z in the output type, bit for bit.
"""

import numpy as np
import pytest

import synthetic as S
from oracle import linear as OL
from oracle import quant as Q
from oracle import transform as T
from parity import check_quantized_dot, check_rotation, quantized_dot_path
from gpu_util import announce, from_dev, lib_plan, method_for, orc_plan, to_dev

pytestmark = pytest.mark.gpu


def _case(rng, T_, m, n, bits, group):
    codes = rng.integers(0, 256, size=(m, n * bits // 8), dtype=np.int64).astype(np.uint8)
    alpha = (0.5 + rng.random((m, n // group))).astype(np.float32) * 0.05
    x = rng.standard_normal((T_, n))
    x[:, rng.choice(n, size=max(1, n // 200), replace=False)] *= 20.0
    return codes, alpha, x


def _run_and_check(Ls, Rs, xs, dt, codes, alpha, m, n, bits, group, out_dt, what,
                   codes_dev=None):
    import butterfly_rotation_quantization_amd as brq
    import torch
    T_ = xs.shape[0]
    U = lib_plan(Ls) if Ls is not None else None
    V = lib_plan(Rs) if Rs is not None else None
    Uo = orc_plan(Ls) if Ls is not None else None
    Vo = orc_plan(Rs) if Rs is not None else None
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
    xd, sd = to_dev(xs, dt), to_dev(alpha, "f32")
    cd = to_dev(codes, "u8") if codes_dev is None else codes_dev
    ws = torch.empty(max(1, brq.qlinear_workspace_bytes(U, V, bits, group, T_, m, n)),
                     dtype=torch.uint8, device="cuda")
    y = brq.qlinear(U, V, xd, cd, sd, m, n, bits, group, out_dtype=tdt[out_dt], ws=ws)
    torch.cuda.synchronize()
    if V is not None:
        xt_gpu = from_dev(ws[: T_ * n * 2].view(tdt[dt]).reshape(T_, n))
    else:
        xt_gpu = S.storage_to_f64(xs, dt)
    y_gpu = from_dev(y)
    z_gpu = from_dev(brq.qlinear(None, V, xd, cd, sd, m, n, bits, group,
                                 out_dtype=torch.float32))
    # 1. the online rotation
    if Vo is not None:
        x_ref = OL.rotate_acts(Vo, S.storage_to_f64(xs, dt))
        check_rotation(xt_gpu, x_ref, dt, f"{what}: X~")
    # 2. the product, from the GPU's own X~
    w = OL.weight(Q.unpack(codes, bits, n), alpha.astype(np.float64), bits, group)
    z_ref = xt_gpu @ w.T
    s_abs = np.abs(xt_gpu) @ np.abs(w).T
    info = check_quantized_dot(z_gpu, z_ref, s_abs, quantized_dot_path(n, group), f"{what}: Z")
    # 3. the output
    if Uo is not None:
        y_ref = T.apply_right(Uo, z_gpu, inverse=True, method=method_for(Uo.d))
        check_rotation(y_gpu, y_ref, out_dt, f"{what}: Y")
    elif out_dt == "f32":
        assert np.array_equal(y_gpu, z_gpu), f"{what}: Y differs from Z"
    else:
        y_round = S.storage_to_f64(S.to_storage(z_gpu, out_dt), out_dt)
        assert np.array_equal(y_gpu, y_round), f"{what}: Y is not Z rounded to {out_dt}"
    print(what, info, flush=True)
    return y


@pytest.mark.parametrize("T_", [1, 16, 37])
@pytest.mark.parametrize("bits,group", [(2, 64), (4, 128), (3, 64)])
@pytest.mark.parametrize("sides", ["both", "none"])
def test_qlinear_small(T_, bits, group, sides):
    rng = np.random.default_rng(T_ * 10 + bits)
    m, n = 256, 1792
    codes, alpha, x = _case(rng, T_, m, n, bits, group)
    dt = "f16"
    xs = S.to_storage(x, dt)
    Ls = S.random_plan(rng, (16, 16), "per_group") if sides == "both" else None
    Rs = S.random_plan(rng, (7, 16, 16), "per_group") if sides == "both" else None
    announce(f"qlinear T={T_} m={m} n={n} b{bits} g{group} {sides}")
    _run_and_check(Ls, Rs, xs, dt, codes, alpha, m, n, bits, group, dt,
                   f"T={T_} b{bits} {sides}")


@pytest.mark.parametrize("T_", [1, 37])
@pytest.mark.parametrize("bits,group", [(2, 64), (3, 64), (4, 128), (5, 64)])
@pytest.mark.parametrize("n", [1024, 3584])
def test_qlinear_stream_chunks(T_, bits, group, n):
    """n a multiple of the 512-input chunk: the weight rows pass through LDS
    (when the staging fits), with one or several chunks per split and fewer
    chunks than the split target."""
    rng = np.random.default_rng(T_ * 100 + bits * 10 + n)
    m = 512
    codes, alpha, x = _case(rng, T_, m, n, bits, group)
    xs = S.to_storage(x, "f16")
    Rs = S.random_plan(rng, (n // 256, 16, 16), "per_group")
    announce(f"qlinear stream T={T_} m={m} n={n} b{bits} g{group}")
    _run_and_check(None, Rs, xs, "f16", codes, alpha, m, n, bits, group, "f16",
                   f"stream T={T_} b{bits} n={n}")


@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_qlinear_bf16_in(out_dt):
    rng = np.random.default_rng(3)
    m, n, bits, group = 256, 1024, 2, 64
    codes, alpha, x = _case(rng, 9, m, n, bits, group)
    xs = S.to_storage(x, "bf16")
    Rs = S.random_plan(rng, (4, 16, 16), "per_group")
    announce(f"qlinear bf16 in, {out_dt} out")
    _run_and_check(None, Rs, xs, "bf16", codes, alpha, m, n, bits, group, out_dt,
                   f"bf16 in {out_dt} out")


@pytest.mark.parametrize("T_", [64, 130, 256, 1030])
@pytest.mark.parametrize("bits,group,dt", [(2, 64, "f16"), (3, 128, "f16"), (4, 64, "bf16"), (5, 64, "f16")])
def test_qlinear_gemm_kernel(T_, bits, group, dt):
    """64 tokens and more with a multiple of 256 weight rows: the GEMM-shaped
    kernel (128 tokens x 256 rows per workgroup, 256-input chunks, one split
    per XCD and token tile, a single split from nine token tiles), including
    a ragged last token tile."""
    rng = np.random.default_rng(T_ * 7 + bits * 3 + group)
    m, n = 512, 2048
    codes, alpha, x = _case(rng, T_, m, n, bits, group)
    xs = S.to_storage(x, dt)
    Ls = S.random_plan(rng, (32, 16), "per_group")
    Rs = S.random_plan(rng, (8, 16, 16), "per_group")
    announce(f"qlinear gemm T={T_} m={m} n={n} b{bits} g{group} {dt}")
    _run_and_check(Ls, Rs, xs, dt, codes, alpha, m, n, bits, group, dt,
                   f"gemm T={T_} b{bits} g{group} {dt}")


@pytest.mark.parametrize("T_", [1, 16, 256])
def test_qlinear_70b_down_proj(T_):
    """The 70B down projection: 8192 outputs, 28672 inputs, left (32,16,16),
    right (7,16,16,16), 2-bit g64, f16 activations; every output element
    checked."""
    rng = np.random.default_rng(700 + T_)
    cfg_rng = np.random.default_rng(5000)
    m, n, bits, group = 8192, 28672, 2, 64
    codes, alpha, x = _case(rng, T_, m, n, bits, group)
    xs = S.to_storage(x, "f16")
    Ls = S.random_plan(cfg_rng, (32, 16, 16), "per_group")
    Rs = S.random_plan(cfg_rng, (7, 16, 16, 16), "per_group")
    announce(f"qlinear 70B down_proj T={T_}")
    _run_and_check(Ls, Rs, xs, "f16", codes, alpha, m, n, bits, group, "f16", f"70B T={T_}")


@pytest.mark.parametrize("T_", [1, 37])
def test_qlinear_direct_kernel_matches_stream(T_):
    """Codes 4 bytes off a 16-byte boundary take the direct kernel, aligned
    codes the streaming one.  Both form each group's sum with the same MFMA
    steps on the same operands and add a split's groups in the same order,
    so the two outputs agree bit for bit; each is checked against the
    oracle on its own."""
    import butterfly_rotation_quantization_amd as brq
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(90 + T_)
    m, n, bits, group = 512, 2048, 2, 64
    codes, alpha, x = _case(rng, T_, m, n, bits, group)
    xs = S.to_storage(x, "f16")
    Ls = S.random_plan(rng, (32, 16), "per_group")
    Rs = S.random_plan(rng, (8, 16, 16), "per_group")
    announce(f"qlinear direct vs stream T={T_}")
    aligned = to_dev(codes, "u8")
    buf = torch.zeros(codes.size + 16, dtype=torch.uint8, device="cuda")
    shifted = buf[4:4 + codes.size].view(m, -1)
    shifted.copy_(aligned)
    assert aligned.data_ptr() % 16 == 0 and shifted.data_ptr() % 16 == 4
    y1 = _run_and_check(Ls, Rs, xs, "f16", codes, alpha, m, n, bits, group, "f16",
                        f"stream T={T_}", codes_dev=aligned)
    y2 = _run_and_check(Ls, Rs, xs, "f16", codes, alpha, m, n, bits, group, "f16",
                        f"direct T={T_}", codes_dev=shifted)
    assert torch.equal(y1, y2)
