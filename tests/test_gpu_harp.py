"""GPU parity of the HARP block builder (brq_harp_blocks, brq_plan_create_harp)
against oracle.harp: blocks element by element, and rotations with plans
built from parameters, including the zero-parameter plan that must be the
RHT."""

import numpy as np
import pytest

import synthetic as S
from oracle import harp as OH
from oracle import transform as T
from parity import check_rotation
from gpu_util import announce, from_dev, method_for, to_dev

pytestmark = pytest.mark.gpu

# The kernel works in float64 and rounds each entry once to float32: within
# one float32 ulp of the float64 oracle (the float64 elimination error, about
# b * 1e-16, can only move a value across a rounding boundary).
ULP32 = 2.0 ** -23


def _theta(rng, n):
    q = rng.integers(-127, 128, size=n, dtype=np.int64).astype(np.int8)
    q[rng.random(n) < 0.05] = 0
    return q


def _base(rng, b):
    """G of a radix: None (Sylvester) for powers of two, else a seeded
    orthogonal matrix from the input generator, in float32."""
    if b & (b - 1) == 0:
        return None
    return S.random_orthogonal(rng, b).astype(np.float32)


def check_blocks(got, ref, what):
    err = np.abs(got - ref)
    tol = ULP32 * np.maximum(np.abs(ref), 2.0 ** -20) + 1e-12
    assert (err <= tol).all(), f"{what}: worst {float((err / tol).max()):.3g} x tolerance"


@pytest.mark.parametrize("b", [2, 3, 4, 7, 16, 32, 43, 64])
@pytest.mark.parametrize("scale", [0.02, 0.0005])
def test_harp_blocks_parity(b, scale):
    import butterfly_rotation_quantization_amd as brq
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(b * 7 + int(scale * 1e4))
    ng = 37
    announce(f"harp blocks b={b} scale={scale} groups={ng}")
    tq = _theta(rng, ng * OH.n_params(b))
    base = _base(rng, b)
    th_dev = torch.from_numpy(tq.reshape(ng, -1)).cuda()
    base_dev = None if base is None else torch.from_numpy(base).cuda()
    got = from_dev(brq.harp_blocks(b, th_dev, scale, base_dev))
    ref = OH.stage_blocks(b, ng, tq, scale, None if base is None else base.astype(np.float64))
    check_blocks(got, ref, f"b={b}")
    # the built blocks are orthogonal to float32 rounding
    for c in (0, ng - 1):
        assert np.abs(got[c] @ got[c].T - np.eye(b)).max() < 4 * b * 2.0 ** -24


def test_harp_blocks_zero_parameters_give_the_base():
    import butterfly_rotation_quantization_amd as brq
    torch = pytest.importorskip("torch")
    for b in (2, 4, 16, 64):
        th = torch.zeros((5, OH.n_params(b)), dtype=torch.int8, device="cuda")
        got = from_dev(brq.harp_blocks(b, th, 0.3))
        ref = np.broadcast_to(T.base_mixer(b).astype(np.float32), (5, b, b))
        assert np.array_equal(got, ref), b


@pytest.mark.parametrize("radix", [(16, 16, 16), (4, 4, 16), (2,) * 8])
def test_zero_parameter_plan_is_the_rht(radix):
    """[HARP] section 2.2: a plan from all-zero parameters rotates exactly as
    the RHT, H_d D / sqrt(d)."""
    import butterfly_rotation_quantization_amd as brq
    d = int(np.prod(radix))
    rng = np.random.default_rng(d)
    sg = S.signs(rng, d)
    announce(f"harp zero plan radix={radix}")
    p = brq.Plan.from_harp(d, radix, np.zeros(OH.total_params(d, radix), dtype=np.int8),
                           [0.05] * len(radix), signs=sg)
    x = rng.standard_normal((33, 2 * d)).astype(np.float32)
    y = from_dev(brq.rotate(p, to_dev(x, "f32"), side="right"))
    rht = T.Plan(d, radix, T.HADAMARD, None, sg.astype(np.float64))
    check_rotation(y, T.apply_right(rht, x.astype(np.float64)), "f32", f"zero harp {radix}")


@pytest.mark.parametrize("side,radix,lines", [
    ("right", (7, 16, 16), 37), ("right", (43, 16, 16), 9), ("left", (32, 16), 64),
    ("left", (8, 3, 16), 45), ("right", (2, 2, 64), 20),
])
def test_harp_plan_rotation(side, radix, lines):
    """Rotations with a plan whose blocks the device built from int8
    parameters match the oracle plan built from the same parameters."""
    import butterfly_rotation_quantization_amd as brq
    d = int(np.prod(radix))
    rng = np.random.default_rng(d + lines)
    tq = _theta(rng, OH.total_params(d, radix))
    scales = [0.01 * (t + 1) for t in range(len(radix))]
    bases = [_base(rng, b) for b in radix]
    sg = S.signs(rng, d)
    announce(f"harp plan {side} radix={radix} lines={lines}")
    lib_bases = None
    if any(g is not None for g in bases):
        lib_bases = [T.base_mixer(b).astype(np.float32) if g is None else g for b, g in zip(radix, bases)]
    p = brq.Plan.from_harp(d, radix, tq, scales, lib_bases, sg)
    orc = OH.harp_plan(d, radix, tq, scales,
                       [None if g is None else g.astype(np.float64) for g in bases],
                       sg.astype(np.float64))
    if side == "right":
        x = rng.standard_normal((lines, d)).astype(np.float32)
        y = from_dev(brq.rotate(p, to_dev(x, "f32"), side="right"))
        ref = T.apply_right(orc, x.astype(np.float64), method=method_for(d))
        check_rotation(y, ref, "f32", f"harp right {radix}")
    else:
        x = rng.standard_normal((d, lines)).astype(np.float32)
        y = from_dev(brq.rotate(p, to_dev(x, "f32"), side="left"))
        ref = T.apply_left(orc, x.astype(np.float64), method=method_for(d))
        check_rotation(y.T, ref.T, "f32", f"harp left {radix}")


def test_harp_blocks_70b_shapes():
    """Every stage of the 70B schedules, U = (32, 16, 16) at d = 8192 and
    V = (7, 16, 16, 16) at d = 28672, built on the device; 64 sampled groups
    per stage against the oracle."""
    import butterfly_rotation_quantization_amd as brq
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(70)
    for d, radix in ((8192, (32, 16, 16)), (28672, (7, 16, 16, 16))):
        for t, b in enumerate(radix):
            ng = d // b
            announce(f"harp 70B d={d} stage {t} b={b} groups={ng}")
            npar = OH.n_params(b)
            tq = _theta(rng, ng * npar)
            base = _base(rng, b)
            got = from_dev(brq.harp_blocks(
                b, torch.from_numpy(tq.reshape(ng, npar)).cuda(), 0.004,
                None if base is None else torch.from_numpy(base).cuda()))
            for c in rng.choice(ng, size=64, replace=False):
                ref = OH.stage_blocks(b, 1, tq[c * npar:(c + 1) * npar], 0.004,
                                      None if base is None else base.astype(np.float64))[0]
                check_blocks(got[c], ref, f"d={d} t={t} c={c}")


@pytest.mark.parametrize("kind", ["blocks", "harp"])
def test_plan_image_rotates_identically(kind):
    """A plan rebuilt from its byte image gives bit-identical rotations."""
    import butterfly_rotation_quantization_amd as brq
    rng = np.random.default_rng(11)
    radix = (7, 16, 16)
    d = int(np.prod(radix))
    if kind == "harp":
        tq = _theta(rng, OH.total_params(d, radix))
        bases = [S.random_orthogonal(rng, 7).astype(np.float32), T.base_mixer(16).astype(np.float32),
                 T.base_mixer(16).astype(np.float32)]
        p = brq.Plan.from_harp(d, radix, tq, [0.01, 0.02, 0.03], bases, S.signs(rng, d))
    else:
        side = S.random_plan(rng, radix, "per_group")
        p = brq.Plan(side.d, side.radix, side.mode, side.blocks, side.signs)
    announce(f"plan image {kind}")
    img = p.serialize()
    q = brq.Plan.deserialize(img)
    assert q.serialize() == img
    x = to_dev(rng.standard_normal((40, 2 * d)).astype(np.float32), "f32")
    a = brq.rotate(p, x, side="right")
    b = brq.rotate(q, x, side="right")
    assert bool((a == b).all())


def test_harp_blocks_batch_equals_single_calls():
    """brq_harp_blocks_batch builds every job as brq_harp_blocks does (the
    same elimination per block), bit for bit: radices 3..32 in one launch,
    2 and above 32 on their own, an empty job among them; sampled blocks
    against the oracle as well."""
    import butterfly_rotation_quantization_amd as brq
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(606)
    spec = [(16, 1792, 0.004), (2, 37, 0.3), (32, 256, 0.002), (7, 300, 0.01), (43, 5, 0.005),
            (64, 3, 0.003), (3, 50, 0.05), (16, 0, 0.01)]
    announce("harp blocks batch of 8 jobs")
    jobs, singles, refs = [], [], []
    for b, ng, sc in spec:
        tq = _theta(rng, ng * OH.n_params(b)).reshape(ng, OH.n_params(b))
        base = _base(rng, b)
        th_dev = torch.from_numpy(tq).cuda()
        base_dev = None if base is None else torch.from_numpy(base).cuda()
        out = torch.full((ng, b, b), float("nan"), dtype=torch.float32, device="cuda")
        jobs.append((b, th_dev, sc, base_dev, out))
        singles.append(brq.harp_blocks(b, th_dev, sc, base_dev))
        refs.append((tq, base))
    brq.harp_blocks_batch(jobs)
    for (b, _, sc, _, out), one, (tq, base) in zip(jobs, singles, refs):
        assert torch.equal(out, one), f"b={b}"
        ng = out.shape[0]
        got = from_dev(out)
        for c in (rng.choice(ng, size=min(ng, 4), replace=False) if ng else []):
            npar = OH.n_params(b)
            ref = OH.stage_blocks(b, 1, tq.reshape(-1)[c * npar:(c + 1) * npar], sc,
                                  None if base is None else base.astype(np.float64))[0]
            check_blocks(got[c], ref, f"batch b={b} c={c}")
