"""Host-side checks of libbrq: the library loads, exports every entry point
include/brq.h declares, validates arguments before touching the device, and
its host Lloyd-Max helper agrees with the oracle.  No kernel is launched."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import butterfly_rotation_quantization_amd as brq
from oracle import lloydmax as LM

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "brq.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(brq.LIB_PATH):
        pytest.fail("libbrq.so is not built (python -m butterfly_rotation_quantization_amd.build)")
    return brq.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(brq_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(brq.EXPORTED), names
    out = subprocess.run(["nm", "-D", "--defined-only", brq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (brq_[a-z_0-9]+)\b", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib, n)


def test_status_strings(lib):
    for code, name in brq.STATUS.items():
        assert lib.brq_status_string(code).decode() == name
    assert lib.brq_version() >= 100


def _create(lib, d, radix, blocks=None, mode=0, signs=None, out=True):
    r = np.asarray(radix, dtype=np.int32)
    h = ctypes.c_void_p()
    b = None if blocks is None else np.ascontiguousarray(blocks, dtype=np.float32)
    s = None if signs is None else np.ascontiguousarray(signs, dtype=np.int8)
    st = lib.brq_plan_create(ctypes.byref(h) if out else None, d, len(r), r.ctypes.data,
                             None if b is None else b.ctypes.data, mode,
                             None if s is None else s.ctypes.data)
    if st == 0:
        lib.brq_plan_destroy(h)
    return st, lib.brq_last_error().decode()


@pytest.mark.parametrize("d,radix,mode,blocks,signs,expect", [
    (256, (2,) * 8, 0, None, None, None),                  # valid (HIP only without a GPU)
    (1, (1,), 0, None, None, 1),                            # d < 2
    (256, (4, 4, 4), 0, None, None, 1),                     # product != d
    (16, (16, 1), 0, None, None, 1),                        # radix < 2
    (96, (96,), 1, np.zeros(96 * 96), None, 2),             # radix > 64
    (12, (3, 4), 0, None, None, 2),                         # Hadamard radix not 2^k
    (12, (3, 4), 2, None, None, 1),                         # blocks missing
    (8, (8,), 0, None, np.array([1, -1, 0, 1, 1, 1, 1, 1]), 1),  # sign not +-1
    (8, (8,), 7, None, None, 1),                            # unknown mode
])
def test_plan_create_validation(lib, d, radix, mode, blocks, signs, expect):
    st, msg = _create(lib, d, radix, blocks, mode, signs)
    if expect is None:
        assert st in (0, 5), (st, msg)
    else:
        assert st == expect, (st, msg)
        assert msg


def test_plan_create_null_out_and_stages(lib):
    st, _ = _create(lib, 8, (8,), out=False)
    assert st == 1
    r = np.full(17, 2, dtype=np.int32)
    h = ctypes.c_void_p()
    assert lib.brq_plan_create(ctypes.byref(h), 1 << 17, 17, r.ctypes.data, None, 0, None) == 1
    assert lib.brq_plan_destroy(None) == 0
    assert lib.brq_plan_dim(None) == 0


def test_call_validation_without_device(lib):
    q = brq.make_quant(3, 128)
    # NULL plan
    assert lib.brq_rotate(None, 0, None, 0, 256, None, 0, 256, 4, 256, None, 0, None) == 1
    # bits out of range, group not dividing n, group not a power of two
    for bits, group, n, expect in [(1, 128, 256, 1), (6, 128, 256, 1), (3, 128, 200, 1),
                                   (4, 96, 192, 2), (3, 32, 256, 2)]:
        qq = brq.make_quant(bits, group)
        st = lib.brq_rotate_quantize_pack(None, None, None, 0, 4, n, n, ctypes.byref(qq), None,
                                          None, None, 0, None)
        assert st == expect, (bits, group, n, st, lib.brq_last_error())
    # bad dtype, ld < n, NULL data with rows > 0 (no kernel is reached)
    assert lib.brq_rotate_quantize_pack(None, None, None, 9, 4, 256, 256, ctypes.byref(q), None,
                                        None, None, 0, None) == 1
    assert lib.brq_rotate_quantize_pack(None, None, None, 0, 4, 256, 100, ctypes.byref(q), None,
                                        None, None, 0, None) == 1
    assert lib.brq_rotate_quantize_pack(None, None, None, 0, 4, 256, 256, ctypes.byref(q), None,
                                        None, None, 0, None) == 1
    # codebook must ascend
    qc = brq.make_quant(2, 128, "codebook_norm", [0.0, 1.0, 0.5, 2.0])
    assert lib.brq_dequant_unrotate(None, None, None, None, ctypes.byref(qc), 4, 256, None, 0,
                                    256, None, 0, None) == 1
    # zero rows is a no-op that succeeds without touching the device
    assert lib.brq_rotate_quantize_pack(None, None, None, 0, 0, 256, 256, ctypes.byref(q), None,
                                        None, None, 0, None) == 0


def test_workspace_bytes(lib):
    assert lib.brq_workspace_bytes(None, None, 0, 10) == 0
    assert lib.brq_workspace_bytes(None, None, 4, 256) == 4 * 256 * 4


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_library_lloyd_max_matches_oracle(lib, bits):
    got = brq.lloyd_max_gaussian(bits).astype(np.float64)
    ref = LM.lloyd_max_gaussian(bits)[0]
    # both solve the same conditions to ~1e-13; the float32 roundings agree
    assert np.all(np.abs(got - ref) <= np.spacing(np.abs(ref).astype(np.float32)))
    assert np.array_equal(got, -got[::-1])


def test_lloyd_max_validation(lib):
    buf = np.zeros(64, dtype=np.float32)
    assert lib.brq_lloyd_max_gaussian(0, buf.ctypes.data) == 1
    assert lib.brq_lloyd_max_gaussian(6, buf.ctypes.data) == 1
    assert lib.brq_lloyd_max_gaussian(3, None) == 1


def test_path_selection(lib):
    assert lib.brq_set_path(1) == 0
    assert lib.brq_set_path(0) == 0
    assert lib.brq_set_path(7) == 1  # INVALID_ARGUMENT
    assert b"unknown path" in lib.brq_last_error()


@pytest.mark.parametrize("b,ng,base,scale,expect", [
    (1, 4, False, 0.1, 1),            # radix below 2
    (65, 4, True, 0.1, 1),            # radix above 64
    (7, 4, False, 0.1, 1),            # not a power of two and no base mixer
    (16, -1, False, 0.1, 1),          # negative group count
    (16, 1 << 31, False, 0.1, 1),     # too many groups
    (16, 4, False, float("nan"), 1),  # scale not finite
    (16, 0, False, 0.1, 0),           # nothing to do
])
def test_harp_blocks_validation(lib, b, ng, base, scale, expect):
    """Arguments are checked before any launch (fake device addresses, never
    dereferenced on these paths)."""
    st = lib.brq_harp_blocks(b, ng, 0x1000, ctypes.c_float(scale), 0x2000 if base else None,
                             0x3000, None)
    assert st == expect, (st, lib.brq_last_error().decode())


def test_plan_create_harp_validation(lib):
    r = np.asarray((7, 16), dtype=np.int32)
    th = np.zeros(16 * 21 + 7 * 1, dtype=np.int8)
    sc = np.asarray([0.1, 0.1], dtype=np.float32)
    h = ctypes.c_void_p()
    # radix 7 without base mixers
    st = lib.brq_plan_create_harp(ctypes.byref(h), 112, 2, r.ctypes.data, th.ctypes.data,
                                  sc.ctypes.data, None, None)
    assert st == 1 and "base" in lib.brq_last_error().decode()
    st = lib.brq_plan_create_harp(ctypes.byref(h), 100, 2, r.ctypes.data, th.ctypes.data,
                                  sc.ctypes.data, None, None)
    assert st == 1
    st = lib.brq_plan_create_harp(None, 112, 2, r.ctypes.data, th.ctypes.data, sc.ctypes.data,
                                  None, None)
    assert st == 1
