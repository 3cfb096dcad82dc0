"""CPU dry run of every launch the GPU tests and the benchmark make.

libbrq_dryrun.so is the same host layer (validation, pass planning, dispatch)
built with host memory for plans and, in place of each kernel launch, a walk
over every index the kernel would touch: global rows/columns, LDS slots, block
and code offsets; it also checks that the tiles of each pass cover every
matrix element exactly once.  Device pointers handed to it are never
dereferenced, so fake addresses are used.
"""

import ctypes

import numpy as np
import pytest

import butterfly_rotation_quantization_amd as brq
import synthetic as S

X, Y, WS, CODES, SCALES = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


@pytest.fixture(scope="module")
def dl():
    import os
    # BRQ_DRYRUN_LIB selects another build of the same library (the
    # AddressSanitizer one, from test_host_asan.py)
    path = os.environ.get("BRQ_DRYRUN_LIB", brq.DRYRUN_LIB_PATH)
    if not os.path.exists(path):
        pytest.fail(f"{os.path.basename(path)} is not built")
    lib = brq.load_library(path)
    lib.brq_dryrun_violation.restype = ctypes.c_char_p
    lib.brq_dryrun_launches.restype = ctypes.c_longlong
    lib.brq_dryrun_rows_launches.restype = ctypes.c_longlong
    lib.brq_dryrun_lanes_launches.restype = ctypes.c_longlong
    return lib


def _ok(dl, st, what):
    msg = dl.brq_last_error().decode()
    viol = dl.brq_dryrun_violation().decode()
    assert st == 0 and not viol, f"{what}: status {st} {msg!r} violation {viol!r}"


class DPlan:
    def __init__(self, dl, side: S.SidePlan):
        r = np.asarray(side.radix, dtype=np.int32)
        blk = None
        if side.blocks is not None:
            blk = np.ascontiguousarray(np.concatenate([b.reshape(-1) for b in side.blocks]),
                                       dtype=np.float32)
        sg = None if side.signs is None else np.ascontiguousarray(side.signs, dtype=np.int8)
        self.h = ctypes.c_void_p()
        mode = {"hadamard": 0, "shared": 1, "per_group": 2}[side.mode]
        st = dl.brq_plan_create(ctypes.byref(self.h), side.d, len(r), r.ctypes.data,
                                None if blk is None else blk.ctypes.data, mode,
                                None if sg is None else sg.ctypes.data)
        _ok(dl, st, f"plan {side.radix}")
        self.dl = dl

    def __del__(self):
        self.dl.brq_plan_destroy(self.h)


def _rotate(dl, plan, side, rows, cols, xt=0, yt=0, inverse=False):
    dl.brq_dryrun_reset()
    fn = dl.brq_rotate_inverse if inverse else dl.brq_rotate
    ws = dl.brq_workspace_bytes(plan.h if side else None, None if side else plan.h, rows, cols)
    st = fn(plan.h, side, X, xt, cols, Y, yt, cols, rows, cols, WS, ws, None)
    _ok(dl, st, f"rotate side={side} inverse={inverse} {rows}x{cols}")
    assert dl.brq_dryrun_launches() >= 1


def _rqp(dl, left, right, m, n, bits, group, kind=0):
    q = brq.make_quant(bits, group, kind,
                       np.linspace(-2, 2, 1 << bits) if kind == 1 else None)
    ws = dl.brq_workspace_bytes(left.h if left else None, right.h if right else None, m, n)
    dl.brq_dryrun_reset()
    st = dl.brq_rotate_quantize_pack(left.h if left else None, right.h if right else None, X, 1,
                                     m, n, n, ctypes.byref(q), CODES, SCALES, WS, ws, None)
    _ok(dl, st, f"rqp {m}x{n} b{bits} g{group}")
    dl.brq_dryrun_reset()
    st = dl.brq_dequant_unrotate(left.h if left else None, right.h if right else None, CODES,
                                 SCALES, ctypes.byref(q), m, n, Y, 0, n, WS, ws, None)
    _ok(dl, st, f"dequant {m}x{n} b{bits} g{group}")


ROTATE_PLANS = [
    ((2,) * 8, "hadamard"), ((4, 4, 16), "per_group"), ((16, 16), "shared"),
    ((43, 16, 16), "per_group"), ((3, 5, 7), "per_group"), ((2,) * 12, "hadamard"),
    ((16, 16, 16), "per_group"), ((7, 16, 16, 16), "per_group"),
    ((8, 8, 8, 5, 2), "per_group"), ((64, 2), "per_group"), ((2,) * 7, "hadamard"),
    ((32, 16, 16), "per_group"), ((2,) * 16, "hadamard"),
]


@pytest.mark.parametrize("radix,mode", ROTATE_PLANS)
def test_rotate_launches(dl, radix, mode):
    side = S.random_plan(np.random.default_rng(1), radix, mode)
    p = DPlan(dl, side)
    d = side.d
    for inverse in (False, True):
        _rotate(dl, p, 0, 37 if d <= 4096 else 5, 2 * d if d <= 512 else d, inverse=inverse)
        _rotate(dl, p, 0, 1, d, 1, 2, inverse=inverse)
        if d <= 8192:
            _rotate(dl, p, 1, d, 45, 2, 0, inverse=inverse)
            _rotate(dl, p, 1, d, 1, inverse=inverse)


def test_quant_launches_small(dl):
    rng = np.random.default_rng(2)
    tiny = S.tiny()
    for name in ("rht", "harp"):
        _rqp(dl, None, DPlan(dl, tiny[name]), 64, 256, 4, 128)
    r = DPlan(dl, S.random_plan(rng, (4, 4, 16), "per_group"))
    for bits in (2, 3, 4, 5):
        for group in (64, 128, 256):
            _rqp(dl, None, r, 45, 1024, bits, group)
    h = DPlan(dl, S.SidePlan(128, (2,) * 7, "hadamard", None, None))
    for bits in (2, 3, 4, 5):
        _rqp(dl, None, h, 40, 512, bits, 128, kind=1)
    left = DPlan(dl, S.random_plan(rng, (4, 4, 4), "per_group"))
    right = DPlan(dl, S.random_plan(rng, (43, 16, 4), "per_group"))
    _rqp(dl, left, right, 64, 2752, 3, 64)
    l2 = DPlan(dl, S.random_plan(rng, (16, 8), "per_group"))
    _rqp(dl, l2, None, 128, 320, 4, 64)
    _rqp(dl, None, None, 128, 320, 3, 64)
    r16 = DPlan(dl, S.random_plan(rng, (16, 16), "per_group"))
    _rqp(dl, None, r16, 13, 512, 4, 128)


def test_quant_launches_workload_shapes(dl):
    """The shapes of the benchmark workload and the full-size parity cases."""
    rng = np.random.default_rng(3)
    u = DPlan(dl, S.random_plan(rng, (16, 16, 16), "per_group"))
    v = DPlan(dl, S.random_plan(rng, (43, 16, 16), "per_group"))
    _rqp(dl, u, v, 4096, 11008, 3, 128)
    hu = DPlan(dl, S.SidePlan(4096, (2,) * 12, "hadamard", None, S.signs(rng, 4096)))
    hv = DPlan(dl, S.SidePlan(4096, (2,) * 12, "hadamard", None, S.signs(rng, 4096)))
    _rqp(dl, hu, hv, 4096, 4096, 4, 128)
    _rotate(dl, hv, 0, 2048, 4096, 1, 1)
    h = DPlan(dl, S.SidePlan(128, (2,) * 7, "hadamard", None, None))
    _rqp(dl, None, h, 12288, 4096, 4, 128, kind=1)


@pytest.mark.parametrize("bv,mode,chunks,bits,group,wt", [
    (43, "per_group", 1, 3, 128, 1), (16, "per_group", 1, 4, 128, 0), (32, "shared", 1, 2, 64, 2),
    (64, "per_group", 1, 5, 128, 1), (7, "per_group", 2, 4, 64, 1), (16, "hadamard", 1, 2, 128, 1),
    (43, "per_group", 1, 4, 64, 0),
])
def test_fused_two_sided_launches(dl, bv, mode, chunks, bits, group, wt):
    """Two-sided (16,16,16) x (bv,16,16) calls take the two-kernel fast path
    (2 launches) and every index of both kernels stays in bounds."""
    rng = np.random.default_rng(bv)
    umode = "hadamard" if mode == "hadamard" else "per_group"
    u = DPlan(dl, S.random_plan(rng, (16, 16, 16), umode))
    v = DPlan(dl, S.random_plan(rng, (bv, 16, 16), mode))
    m, n = 4096, bv * 256 * chunks
    q = brq.make_quant(bits, group)
    ws = dl.brq_workspace_bytes(u.h, v.h, m, n)
    dl.brq_dryrun_reset()
    st = dl.brq_rotate_quantize_pack(u.h, v.h, X, wt, m, n, n, ctypes.byref(q), CODES, SCALES,
                                     WS, ws, None)
    _ok(dl, st, f"fused bv={bv} {mode}")
    assert dl.brq_dryrun_launches() == 2


@pytest.mark.parametrize("uradix,vradix,m,n,bits,group,wt", [
    ((32, 16, 16), (7, 16, 16, 16), 8192, 28672, 2, 64, 1),   # the 70B weight
    ((32, 16, 16), (7, 16, 16), 8192, 1792, 3, 128, 0),
    ((32, 16, 16), (3, 2, 16, 16), 8192, 3072, 4, 128, 2),
    ((16, 2, 16, 16), (16, 16, 16), 8192, 4096, 3, 64, 1),
])
def test_fused_longer_schedules_launches(dl, uradix, vradix, m, n, bits, group, wt):
    """Stage 0 of radix 16 or 32 on the left and up to 64 on the right at any
    stride, stages between stage 0 and the last two as stage passes in place,
    then pass B: every index of the passes stays in bounds and every output
    element is written once."""
    rng = np.random.default_rng(m + n)
    u = DPlan(dl, S.random_plan(rng, uradix, "per_group"))
    v = DPlan(dl, S.random_plan(rng, vradix, "per_group"))
    q = brq.make_quant(bits, group)
    ws = dl.brq_workspace_bytes(u.h, v.h, m, n)
    dl.brq_dryrun_reset()
    st = dl.brq_rotate_quantize_pack(u.h, v.h, X, wt, m, n, n, ctypes.byref(q), CODES, SCALES,
                                     WS, ws, None)
    _ok(dl, st, f"fused {uradix} x {vradix}")
    assert dl.brq_dryrun_launches() == 2 + (len(uradix) - 3) + (len(vradix) - 3)


# The row Hadamard path: one launch per call, for every chunk length it
# takes, with partial last workgroups, every dtype pair and group size.
@pytest.mark.parametrize("l2d,rows,cpr", [(4, 33, 2), (5, 129, 3), (7, 50, 4), (8, 17, 2),
                                           (10, 9, 2), (11, 6, 1), (12, 37, 1), (12, 3, 2),
                                           (7, 12288, 32)])
def test_rowhad_launches(dl, l2d, rows, cpr):
    d = 1 << l2d
    rng = np.random.default_rng(l2d)
    p = DPlan(dl, S.SidePlan(d, (2,) * l2d, "hadamard", None, S.signs(rng, d)))
    n = cpr * d
    for xt, yt in ((0, 0), (1, 1), (2, 2), (1, 0), (0, 2)):
        for inverse in (False, True):
            dl.brq_dryrun_reset()
            fn = dl.brq_rotate_inverse if inverse else dl.brq_rotate
            st = fn(p.h, 0, X, xt, n, Y, yt, n, rows, n, None, 0, None)
            _ok(dl, st, f"rowhad rotate d={d} {xt}->{yt} inverse={inverse}")
            assert dl.brq_dryrun_launches() == 1
    for bits in (2, 3, 4, 5):
        for group in (64, 128, 256, 512, 1024):
            if n % group:
                continue
            for kind in (0, 1):
                _rqp(dl, None, p, rows, n, bits, group, kind)
                assert dl.brq_dryrun_launches() == 1


def _right_launches(radices, lines, mode, inverse):
    """Launches of a right-side stage pass: in application order, a
    forward (16, 16) at strides 16, 1 (or its inverse) is one launch; up to
    32 rows of a dense plan, so are two consecutive stages of radix <= 16
    with a product <= 256; every other stage is a launch of its own."""
    n = len(radices)
    S = [int(np.prod(radices[t + 1:])) for t in range(n)]
    order = list(range(n))[::-1] if inverse else list(range(n))
    i = launches = 0
    while i < n:
        if i + 1 < n:
            to, ti = sorted((order[i], order[i + 1]))
            pair16 = radices[to] == 16 and radices[ti] == 16 and S[to] == 16 and S[ti] == 1
            pair2 = (lines <= 32 and mode != "hadamard" and not pair16 and radices[to] <= 16 and
                     radices[ti] <= 16 and radices[to] * radices[ti] <= 256)
            if pair16 or pair2:
                launches += 1
                i += 2
                continue
        launches += 1
        i += 1
    return launches


# The stage pass: one launch per stage for rotations of few lines (decode-time
# activations on the right side, a few columns on the left side).
@pytest.mark.parametrize("radix,mode,lines,chunks", [
    ((7, 16, 16, 16), "per_group", 1, 1), ((7, 16, 16, 16), "per_group", 16, 1),
    ((7, 16, 16, 16), "per_group", 256, 1), ((43, 16, 16), "per_group", 33, 2),
    ((3, 5, 7), "shared", 70, 3), ((2,) * 13, "hadamard", 5, 1), ((64, 2), "per_group", 1024, 1),
    ((32, 16, 16), "per_group", 9, 1), ((8, 8, 8, 5, 2), "per_group", 3, 1), ((2, 16, 64), "shared", 7, 2),
    ((3, 5, 7), "per_group", 4, 2),
])
def test_stage_pass_launches(dl, radix, mode, lines, chunks):
    side = S.random_plan(np.random.default_rng(len(radix) + lines), radix, mode)
    p = DPlan(dl, side)
    d = side.d
    nst = len(radix) if mode != "hadamard" else -(-int(np.log2(d)) // 4)
    radices = radix if mode != "hadamard" else (16,) * (nst - 1) + (d // 16 ** (nst - 1),)
    if mode == "hadamard" and d % 16 ** (nst - 1) == 0 and 16 ** nst != d:
        radices = (d // 16 ** (nst - 1),) + (16,) * (nst - 1)
    for inverse in (False, True):
        want = _right_launches(radices, lines, mode, inverse)
        for xt, yt in ((2, 2), (1, 0), (0, 1)):
            _rotate(dl, p, 0, lines, chunks * d, xt, yt, inverse=inverse)
            assert dl.brq_dryrun_launches() == want
        if d <= 8192:
            _rotate(dl, p, 1, d, lines, 1, 1, inverse=inverse)
            assert dl.brq_dryrun_launches() == nst


def test_stage_head_pass_b_tail_launches(dl):
    """Dense two-sided schedules ending in (16, 16) on both sides: stage passes
    for the earlier stages, then pass B (tiles of 256 rows over any number of
    256-row blocks)."""
    rng = np.random.default_rng(77)
    u = DPlan(dl, S.random_plan(rng, (4, 16, 16), "per_group"))
    v = DPlan(dl, S.random_plan(rng, (3, 16, 16, 16), "per_group"))
    m, n = 1024, 12288
    q = brq.make_quant(2, 64)
    ws = dl.brq_workspace_bytes(u.h, v.h, m, n)
    dl.brq_dryrun_reset()
    st = dl.brq_rotate_quantize_pack(u.h, v.h, X, 1, m, n, n, ctypes.byref(q), CODES, SCALES,
                                     WS, ws, None)
    _ok(dl, st, "stage head + pass B tail")
    assert dl.brq_dryrun_launches() == 1 + 2 + 1  # L(4), R(3), R(16) S256, pass B


# Left-side stages whose radix is a power of two up to 64 run by whole rows
# when the column count, leading dimensions and pointers allow vector accesses
# and one side is float32; the rest keep the tile kernel.
@pytest.mark.parametrize("radix,mode,cols,xt,yt,rows_launches", [
    ((32, 16, 16), "per_group", 512, 1, 1, 3),    # bf16 -> f32 -> f32 -> bf16
    ((16, 16, 16), "per_group", 64, 0, 0, 3),
    ((64, 2), "per_group", 8, 2, 2, 2),           # radix 64: one column per thread
    ((2,) * 12, "hadamard", 36, 1, 1, 3),         # canonical radix-16 stages
    ((32, 16, 16), "per_group", 6, 1, 1, 1),      # 6 columns: radix 32 takes pairs, 16 needs 4
    ((32, 16, 16), "per_group", 9, 1, 1, 0),      # odd column count
    ((3, 5, 7), "shared", 64, 0, 0, 0),           # radices that are not powers of two
    ((4,), "shared", 64, 1, 1, 0),                # one stage bf16 -> bf16
])
def test_left_rows_kernel(dl, radix, mode, cols, xt, yt, rows_launches):
    side = S.random_plan(np.random.default_rng(cols), radix, mode)
    p = DPlan(dl, side)
    for inverse in (False, True):
        _rotate(dl, p, 1, side.d, cols, xt, yt, inverse=inverse)
        assert dl.brq_dryrun_rows_launches() == rows_launches


# HARP blocks from parameters: the launch geometry, the parameter indices of
# every (i < j) pair once each, and the LDS system, for every radix; then a
# whole plan built that way goes through the ordinary plan set-up.
@pytest.mark.parametrize("b", [2, 3, 4, 5, 7, 8, 16, 32, 43, 64])
def test_harp_blocks_walk(dl, b):
    dl.brq_dryrun_reset()
    base = None if b & (b - 1) == 0 else 0x2000
    st = dl.brq_harp_blocks(b, 37, 0x1000, ctypes.c_float(0.05), base, 0x3000, None)
    _ok(dl, st, f"harp blocks b={b}")
    assert dl.brq_dryrun_launches() == 1


@pytest.mark.parametrize("radix,with_base", [((32, 16, 16), False), ((7, 16, 16, 16), True),
                                             ((2,) * 6, False), ((43, 2), True)])
def test_plan_create_harp_walk(dl, radix, with_base):
    import oracle.harp as OH  # parameter counts only
    d = int(np.prod(radix))
    th = np.zeros(OH.total_params(d, radix), dtype=np.int8)
    sc = np.full(len(radix), 0.01, dtype=np.float32)
    bases = None
    if with_base:
        bases = np.concatenate([np.eye(b, dtype=np.float32).reshape(-1) for b in radix])
    r = np.asarray(radix, dtype=np.int32)
    h = ctypes.c_void_p()
    dl.brq_dryrun_reset()
    st = dl.brq_plan_create_harp(ctypes.byref(h), d, len(r), r.ctypes.data, th.ctypes.data,
                                 sc.ctypes.data, None if bases is None else bases.ctypes.data,
                                 None)
    _ok(dl, st, f"harp plan {radix}")
    # the stages of radix 3..32 share one launch, the others go one by one
    batched = [b for b in radix if 3 <= b <= 32]
    assert dl.brq_dryrun_launches() == (1 if batched else 0) + len(radix) - len(batched)
    assert dl.brq_dryrun_harp_batches() == (1 if batched else 0)
    dl.brq_plan_destroy(h)


def _jobs(spec):
    arr = (brq.HarpJob * len(spec))()
    out = 0x100000
    for i, (b, ng) in enumerate(spec):
        arr[i] = brq.HarpJob(b, ng, 0x1000, 0.05, None if b & (b - 1) == 0 else 0x2000, out)
        out += 4 * ng * b * b
    return arr


def test_harp_blocks_batch_walk(dl):
    """Radix 3..32 jobs share launches of at most 16 jobs; radix 2 and above
    32 launch alone; empty jobs launch nothing; one invalid job launches
    nothing at all."""
    dl.brq_dryrun_reset()
    spec = [(16, 1792), (2, 5), (32, 256), (7, 4096), (43, 3), (16, 0), (64, 2), (3, 9)]
    _ok(dl, dl.brq_harp_blocks_batch(len(spec), _jobs(spec), None), "batch")
    assert dl.brq_dryrun_harp_batches() == 1
    assert dl.brq_dryrun_launches() == 1 + 3
    dl.brq_dryrun_reset()
    many = [(16, 10)] * 20
    _ok(dl, dl.brq_harp_blocks_batch(len(many), _jobs(many), None), "20 jobs")
    assert dl.brq_dryrun_harp_batches() == 2 and dl.brq_dryrun_launches() == 2
    dl.brq_dryrun_reset()
    bad = _jobs([(16, 10), (7, 10)])
    bad[1].base = None  # radix 7 without a base mixer
    assert dl.brq_harp_blocks_batch(2, bad, None) == 1
    assert dl.brq_dryrun_launches() == 0


# Plan images: serialise, deserialise, serialise again gives the same bytes
# (host memory stands in for the device here); damaged images are refused.
def _image(dl, h):
    n = ctypes.c_size_t()
    assert dl.brq_plan_serialize(h, None, 0, ctypes.byref(n)) == 0
    buf = ctypes.create_string_buffer(n.value)
    assert dl.brq_plan_serialize(h, buf, n.value, ctypes.byref(n)) == 0
    return buf.raw[:n.value]


@pytest.mark.parametrize("radix,mode", [((2,) * 6, "hadamard"), ((4, 16), "shared"),
                                        ((7, 16, 16), "per_group"), ((3, 5, 7), "per_group")])
def test_plan_image_round_trip(dl, radix, mode):
    p = DPlan(dl, S.random_plan(np.random.default_rng(3), radix, mode))
    img = _image(dl, p.h)
    assert img[:4] == b"BRQP"
    h2 = ctypes.c_void_p()
    _ok(dl, dl.brq_plan_deserialize(ctypes.byref(h2), img, len(img)), "deserialize")
    assert _image(dl, h2) == img
    dl.brq_plan_destroy(h2)


def test_harp_plan_image_holds_the_int8_parameters(dl):
    import oracle.harp as OH  # parameter counts only
    radix, d = (7, 16, 16, 16), 28672
    rng = np.random.default_rng(4)
    th = rng.integers(-127, 128, size=OH.total_params(d, radix)).astype(np.int8)
    sc = np.asarray([0.004, 0.003, 0.002, 0.001], dtype=np.float32)
    bases = np.concatenate([np.eye(b, dtype=np.float32).reshape(-1) for b in radix])
    sg = S.signs(rng, d)
    r = np.asarray(radix, dtype=np.int32)
    h = ctypes.c_void_p()
    _ok(dl, dl.brq_plan_create_harp(ctypes.byref(h), d, 4, r.ctypes.data, th.ctypes.data,
                                    sc.ctypes.data, bases.ctypes.data, sg.ctypes.data), "harp plan")
    img = _image(dl, h)
    # header 28 + radices 16 + scales 16 + bases + parameters + signs + hash 8
    assert len(img) == 28 + 16 + 16 + 4 * bases.size + th.size + d + 8
    assert img.find(th.tobytes()) > 0
    h2 = ctypes.c_void_p()
    _ok(dl, dl.brq_plan_deserialize(ctypes.byref(h2), img, len(img)), "deserialize harp")
    assert _image(dl, h2) == img
    # int8 parameters are 8.6x smaller than the float32 blocks they make
    nblk = sum((d // b) * b * b for b in radix)
    assert 4 * nblk / th.size > 8
    dl.brq_plan_destroy(h2)
    dl.brq_plan_destroy(h)


def test_plan_image_damage_is_refused(dl):
    p = DPlan(dl, S.random_plan(np.random.default_rng(5), (4, 16), "per_group"))
    img = bytearray(_image(dl, p.h))
    h = ctypes.c_void_p()
    for bad in (bytes(img[:-1]), bytes(img[:20]), b"XXXX" + bytes(img[4:])):
        assert dl.brq_plan_deserialize(ctypes.byref(h), bad, len(bad)) == 1
    flipped = bytearray(img)
    flipped[100] ^= 1
    assert dl.brq_plan_deserialize(ctypes.byref(h), bytes(flipped), len(flipped)) == 1
    assert b"hash" in dl.brq_last_error()
    n = ctypes.c_size_t()
    small = ctypes.create_string_buffer(16)
    assert dl.brq_plan_serialize(p.h, small, 16, ctypes.byref(n)) == 1


# PolarQuant's downstream chain: one fused pass for right Hadamard plans with
# d = 64..256, else dequantize + unrotate into the workspace and quantize.
@pytest.mark.parametrize("d,m,n,bits_in,bits_out,g_out,fused", [
    (128, 64, 4096, 5, 4, 128, True), (128, 5, 12288, 4, 4, 64, True),
    (256, 3, 1024, 5, 2, 1024, True), (64, 7, 192, 3, 5, 64, True),
    (512, 4, 1024, 5, 4, 128, False), (4096, 2, 4096, 5, 4, 128, False),
])
def test_requant_walk(dl, d, m, n, bits_in, bits_out, g_out, fused):
    p = DPlan(dl, S.random_plan(np.random.default_rng(d), (2,) * int(np.log2(d)), "hadamard", False))
    qi = brq.make_quant(bits_in, min(d, 1024), 1, np.linspace(-2.5, 2.5, 1 << bits_in))
    qo = brq.make_quant(bits_out, g_out, 0)
    nb = dl.brq_requant_workspace_bytes(p.h, ctypes.byref(qi), ctypes.byref(qo), m, n)
    assert nb == (0 if fused else 2 * m * n * 4)
    dl.brq_dryrun_reset()
    st = dl.brq_requant(p.h, CODES, SCALES, ctypes.byref(qi), m, n, ctypes.byref(qo), X, Y,
                        WS, nb, None)
    _ok(dl, st, f"requant d={d}")
    assert dl.brq_dryrun_launches() == (1 if fused else 2)
    # the downstream quantizer must be absmax
    qc = brq.make_quant(bits_out, g_out, 1, np.linspace(-2, 2, 1 << bits_out))
    assert dl.brq_requant(p.h, CODES, SCALES, ctypes.byref(qi), m, n, ctypes.byref(qc), X, Y,
                          WS, nb, None) == 1


# Right-side stages of radix <= 8 whose stride is a multiple of 64 keep one
# group per lane (its block in registers); the rest keep the tile kernel.
@pytest.mark.parametrize("radix,mode,rows,chunks,lanes", [
    ((7, 16, 16, 16), "per_group", 4096, 1, 2),   # the 70B right schedule: stages 0, 1
    ((7, 16, 16, 16), "per_group", 1, 1, 0),      # decode T = 1: the tile kernel
    ((7, 16, 16, 16), "per_group", 16, 1, 0),     # decode T = 16: the tile kernel up to 32 rows
    ((7, 16, 16), "shared", 37, 2, 1),            # block-diagonal, shared block
    ((8, 8, 8, 5, 2), "per_group", 40, 1, 1),     # S = 640 at stage 0; 80 and 10 are not
    ((2, 4, 64), "per_group", 33, 3, 2),          # S = 256 and 64
    ((43, 16, 16), "per_group", 9, 1, 0),         # radix 43; radix 16 at strides 16 and 1
    ((7, 16, 16, 16), "shared", 64, 1, 1),        # radix 7 (radix 16: block rows not 16-byte aligned)
    ((7, 16, 16, 16), "per_group", 256, 1, 1),    # radix 16 only for <= 32 or >= 4096 rows
    ((2, 16, 64), "shared", 5, 2, 0),             # below 8 rows: (2, 16) as one pair launch
    ((2, 16, 64), "shared", 17, 2, 0),            # 17 rows: the tile kernel
    ((2, 4, 16, 64), "shared", 33, 1, 2),         # radix 2 (S = 4096) and 4 (S = 1024)
])
def test_right_lanes_kernel(dl, radix, mode, rows, chunks, lanes):
    side = S.random_plan(np.random.default_rng(rows), radix, mode)
    p = DPlan(dl, side)
    for inverse in (False, True):
        _rotate(dl, p, 0, rows, chunks * side.d, 2, 2, inverse=inverse)
        assert dl.brq_dryrun_lanes_launches() == lanes


# The quantized linear layer: rotation passes, the split product and its
# reduction, and the output rotation.
@pytest.mark.parametrize("T,m,n,bits,group,sides", [
    (1, 512, 4096, 2, 64, "both"), (16, 512, 4096, 3, 128, "both"), (40, 256, 1024, 4, 64, "right"),
    (5, 256, 2048, 5, 128, "left"), (3, 256, 512, 2, 64, "none"), (70, 128, 1024, 3, 64, "none"),
    (9, 256, 1792, 2, 64, "none"),  # n not a multiple of the staging chunk
    # 64 tokens and more with 256-row blocks: the GEMM-shaped kernel
    (64, 256, 1024, 2, 64, "both"), (130, 512, 2048, 3, 128, "right"), (256, 256, 768, 5, 64, "none"),
    (300, 512, 1280, 4, 64, "left"),
    (128, 384, 1024, 2, 64, "none"),  # m not a multiple of 256: the direct kernel
    (1100, 256, 512, 2, 64, "none"),  # nine token tiles: a single split
])
def test_qlinear_walk(dl, T, m, n, bits, group, sides):
    left = DPlan(dl, S.random_plan(np.random.default_rng(m), (m // 16, 16), "per_group")) \
        if sides in ("both", "left") else None
    right = DPlan(dl, S.random_plan(np.random.default_rng(n), (n // 64, 4, 16), "per_group")) \
        if sides in ("both", "right") else None
    q = brq.make_quant(bits, group, 0)
    lh, rh = (left.h if left else None), (right.h if right else None)
    nb = dl.brq_qlinear_workspace_bytes(lh, rh, ctypes.byref(q), T, m, n)
    assert nb > 0
    dl.brq_dryrun_reset()
    st = dl.brq_qlinear(lh, rh, X, 2, n, T, CODES, SCALES, ctypes.byref(q), m, n, Y, 2, m, WS, nb, None)
    _ok(dl, st, f"qlinear T={T} {sides}")
    assert dl.brq_dryrun_launches() >= 2  # the product and its reduction, plus the rotations
    # too small a workspace, a codebook weight and bf32 activations are refused
    assert dl.brq_qlinear(lh, rh, X, 2, n, T, CODES, SCALES, ctypes.byref(q), m, n, Y, 2, m, WS,
                          nb - 1, None) == 4
    qc = brq.make_quant(bits, group, 1, np.linspace(-2, 2, 1 << bits))
    assert dl.brq_qlinear(lh, rh, X, 2, n, T, CODES, SCALES, ctypes.byref(qc), m, n, Y, 2, m, WS,
                          nb, None) == 1
    assert dl.brq_qlinear(lh, rh, X, 0, n, T, CODES, SCALES, ctypes.byref(q), m, n, Y, 2, m, WS,
                          nb, None) == 1


# The ORP GEO quantizer and dequantizer: every lane's element run, code
# bytes, sign bytes and coefficient pairs, each written exactly once; pair
# partners inside their group and micro-block; ragged last chunks.
@pytest.mark.parametrize("m,n,bits,group,stride", [
    (3, 1024, 3, 128, 1), (2, 11008, 3, 128, 4), (4, 1536, 2, 64, 32), (2, 3072, 5, 512, 256),
    (5, 640, 4, 64, 8), (1, 4096, 4, 256, 2), (2, 1152, 3, 128, 64), (7, 64, 2, 64, 16),
])
def test_orp_walk(dl, m, n, bits, group, stride):
    q = brq.Orp(bits, group, stride)
    SIGNS, COEF = 0x60000000, 0x70000000
    for wt in (0, 1):
        dl.brq_dryrun_reset()
        st = dl.brq_orp_geo_quantize(X, wt, m, n, n, None, ctypes.byref(q), CODES, SIGNS, COEF, None)
        _ok(dl, st, f"orp quant {m}x{n} b{bits} g{group} S{stride}")
        assert dl.brq_dryrun_launches() == 1
    dl.brq_dryrun_reset()
    st = dl.brq_orp_geo_dequant(CODES, SIGNS, COEF, ctypes.byref(q), m, n, Y, 1, n, None)
    _ok(dl, st, f"orp dequant {m}x{n}")
    # validation: a stride that does not fit the group, a group not dividing n,
    # misaligned rows
    bad = brq.Orp(bits, group, group)
    assert dl.brq_orp_geo_quantize(X, 0, m, n, n, None, ctypes.byref(bad), CODES, SIGNS, COEF,
                                   None) == 1
    assert dl.brq_orp_geo_quantize(X, 0, m, n + 8, n + 8, None, ctypes.byref(q), CODES, SIGNS,
                                   COEF, None) == 1
    assert dl.brq_orp_geo_quantize(X + 4, 0, m, n, n, None, ctypes.byref(q), CODES, SIGNS, COEF,
                                   None) == 3
