"""The decode linear's no-allocation entry point (brq_qlinear_noalloc),
called through the C ABI: bit for bit the same output as brq_qlinear with a
workspace, on two calls in a row (the second smaller, so the scratch array
holds the first call's contents), and a clear error beyond its limit."""

import ctypes

import numpy as np
import pytest

import synthetic as S
from gpu_util import announce, lib_plan, to_dev

pytestmark = pytest.mark.gpu


def _case(rng, T_, m, n, bits, group):
    codes = rng.integers(0, 256, size=(m, n * bits // 8), dtype=np.int64).astype(np.uint8)
    alpha = (0.5 + rng.random((m, n // group))).astype(np.float32) * 0.05
    x = rng.standard_normal((T_, n))
    return codes, alpha, S.to_storage(x, "f16")


def _noalloc(brq, U, V, xd, cd, sd, m, n, bits, group, y):
    q = brq.make_quant(bits, group, "absmax")
    return brq.lib().brq_qlinear_noalloc(
        U.handle if U else None, V.handle if V else None, xd.data_ptr(), brq.dtype_code(xd),
        xd.stride(0), xd.shape[0], cd.data_ptr(), sd.data_ptr(), ctypes.byref(q), m, n,
        y.data_ptr(), brq.dtype_code(y), y.stride(0), None)


@pytest.mark.parametrize("shapes", [
    # (T, m, n, bits, group, left radix, right radix): first call, then a smaller one
    [(16, 8192, 28672, 2, 64, (32, 16, 16), (7, 16, 16, 16)),
     (1, 8192, 28672, 2, 64, (32, 16, 16), (7, 16, 16, 16))],
    [(37, 512, 3584, 3, 64, (32, 16), (14, 16, 16)),
     (5, 256, 1792, 4, 128, (16, 16), (7, 16, 16))],
])
def test_noalloc_matches_workspace_call(shapes):
    import butterfly_rotation_quantization_amd as brq
    import torch
    lim = brq.lib().brq_qlinear_noalloc_limit()
    assert lim == 64 << 20
    for k, (T_, m, n, bits, group, lr, rr) in enumerate(shapes):
        rng = np.random.default_rng(31 + k)
        codes, alpha, xs = _case(rng, T_, m, n, bits, group)
        U = lib_plan(S.random_plan(rng, lr, "per_group"))
        V = lib_plan(S.random_plan(rng, rr, "per_group"))
        announce(f"noalloc call {k}: T={T_} {m}x{n} b{bits} g{group}")
        xd, cd, sd = to_dev(xs, "f16"), to_dev(codes, "u8"), to_dev(alpha, "f32")
        ref = brq.qlinear(U, V, xd, cd, sd, m, n, bits, group)
        y = torch.full((T_, m), float("nan"), dtype=torch.float16, device="cuda")
        st = _noalloc(brq, U, V, xd, cd, sd, m, n, bits, group, y)
        assert st == 0, brq.lib().brq_last_error()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"call {k}: {int((y != ref).sum())} outputs differ"


def test_noalloc_rejects_beyond_limit():
    import butterfly_rotation_quantization_amd as brq
    import torch
    rng = np.random.default_rng(40)
    T_, m, n, bits, group = 256, 8192, 28672, 2, 64
    U = lib_plan(S.random_plan(rng, (32, 16, 16), "per_group"))
    V = lib_plan(S.random_plan(rng, (7, 16, 16, 16), "per_group"))
    need = brq.qlinear_workspace_bytes(U, V, bits, group, T_, m, n)
    assert need > brq.lib().brq_qlinear_noalloc_limit()
    xd = torch.zeros((T_, n), dtype=torch.float16, device="cuda")
    cd = torch.zeros((m, n * bits // 8), dtype=torch.uint8, device="cuda")
    sd = torch.zeros((m, n // group), dtype=torch.float32, device="cuda")
    y = torch.empty((T_, m), dtype=torch.float16, device="cuda")
    st = _noalloc(brq, U, V, xd, cd, sd, m, n, bits, group, y)
    assert st == 4 and b"no-allocation" in brq.lib().brq_last_error()
