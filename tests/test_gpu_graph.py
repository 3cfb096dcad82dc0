"""Decode calls replayed from a captured graph.

The hot calls launch kernels on the caller's stream and nothing else (no
allocation, no memset, no synchronisation), so a graph captured from one call
replays it.  Each replay is compared with the eager call bit for bit (the same
kernels on the same inputs); between the replays the test runs eager work of
its own, clears the graph's output and synchronises.
"""

import numpy as np
import pytest

import synthetic as S
from gpu_util import announce, lib_plan, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _check_replays(torch, capture, eager_other, out_graph, ref):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        capture()  # once outside the capture (the library's first-call set-up)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        capture()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        out_graph.zero_()
        eager_other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_graph, ref), f"replay {r} differs from the eager call"


def test_graph_decode_rotation():
    """The 70B right rotation at one token (two stage-pair launches)."""
    import butterfly_rotation_quantization_amd as brq
    import torch
    announce("graph: decode rotation T=1 (7,16,16,16)")
    rng = np.random.default_rng(11)
    Rs = S.random_plan(rng, (7, 16, 16, 16), "per_group")
    V = lib_plan(Rs)
    n = Rs.d
    x = to_dev(S.to_storage(rng.standard_normal((1, n)), "f16"), "f16")
    x2 = to_dev(S.to_storage(rng.standard_normal((1, n)), "f16"), "f16")
    ws = brq.workspace(None, V, 1, n, "cuda")
    ref = torch.empty_like(x)
    brq.rotate(V, x, ref, side="right", ws=ws)
    torch.cuda.synchronize()
    yg, yo = torch.empty_like(x), torch.empty_like(x)
    _check_replays(torch, lambda: brq.rotate(V, x, yg, side="right", ws=ws),
                   lambda: brq.rotate(V, x2, yo, side="right", ws=ws), yg, ref)


@pytest.mark.parametrize("T_", [1, 130])
def test_graph_decode_linear(T_):
    """The quantized linear layer at one token (input rotation, streaming
    product, reduction, output rotation) and at 130 tokens (the GEMM-shaped
    product, the reduction folded into the first output stage)."""
    import butterfly_rotation_quantization_amd as brq
    import torch
    announce(f"graph: decode linear T={T_} m=256 n=1792")
    rng = np.random.default_rng(12 + T_)
    m, n, bits, group = 256, 1792, 2, 64
    codes = rng.integers(0, 256, size=(m, n * bits // 8), dtype=np.int64).astype(np.uint8)
    alpha = (0.5 + rng.random((m, n // group))).astype(np.float32) * 0.05
    U = lib_plan(S.random_plan(rng, (16, 16), "per_group"))
    V = lib_plan(S.random_plan(rng, (7, 16, 16), "per_group"))
    x = to_dev(S.to_storage(rng.standard_normal((T_, n)), "f16"), "f16")
    x2 = to_dev(S.to_storage(rng.standard_normal((T_, n)), "f16"), "f16")
    cd, sd = to_dev(codes, "u8"), to_dev(alpha, "f32")
    nb = brq.qlinear_workspace_bytes(U, V, bits, group, T_, m, n)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ref = torch.empty((T_, m), dtype=torch.float16, device="cuda")
    brq.qlinear(U, V, x, cd, sd, m, n, bits, group, y=ref, ws=ws)
    torch.cuda.synchronize()
    yg, yo = torch.empty_like(ref), torch.empty_like(ref)
    _check_replays(torch, lambda: brq.qlinear(U, V, x, cd, sd, m, n, bits, group, y=yg, ws=ws),
                   lambda: brq.qlinear(U, V, x2, cd, sd, m, n, bits, group, y=yo, ws=ws2), yg, ref)
