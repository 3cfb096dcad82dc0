"""Python binding of libbrq (structured rotation + group quantization, gfx950).

Argument marshalling only: every step of the rotation and quantization runs
in the HIP kernels of ``lib/libbrq.so``; PyTorch supplies device memory and
the current stream.  There is no CPU fallback: a missing library raises.

Names follow the C ABI in ``include/brq.h`` without the ``brq_`` prefix.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libbrq.so")
DRYRUN_LIB_PATH = os.path.join(_PKG, "lib", "libbrq_dryrun.so")

F32, BF16, F16 = 0, 1, 2
HADAMARD, SHARED, PER_GROUP = 0, 1, 2
RIGHT, LEFT = 0, 1
ABSMAX, CODEBOOK_NORM = 0, 1
_MODES = {"hadamard": HADAMARD, "shared": SHARED, "per_group": PER_GROUP}
_KINDS = {"absmax": ABSMAX, "codebook_norm": CODEBOOK_NORM}
_SIDES = {"right": RIGHT, "left": LEFT}

STATUS = {0: "BRQ_OK", 1: "BRQ_ERR_INVALID_ARGUMENT", 2: "BRQ_ERR_UNSUPPORTED",
          3: "BRQ_ERR_ALIGNMENT", 4: "BRQ_ERR_WORKSPACE", 5: "BRQ_ERR_HIP"}

EXPORTED = (
    "brq_status_string", "brq_last_error", "brq_version", "brq_plan_create",
    "brq_plan_destroy", "brq_plan_dim", "brq_workspace_bytes", "brq_rotate",
    "brq_rotate_inverse", "brq_rotate_quantize_pack", "brq_dequant_unrotate",
    "brq_lloyd_max_gaussian", "brq_profile_enable", "brq_profile_reset", "brq_profile_count",
    "brq_profile_read", "brq_set_path", "brq_harp_blocks", "brq_harp_blocks_batch", "brq_plan_create_harp",
    "brq_plan_serialize", "brq_plan_deserialize", "brq_requant_workspace_bytes", "brq_requant",
    "brq_qlinear_workspace_bytes", "brq_qlinear", "brq_orp_geo_quantize", "brq_orp_geo_dequant",
    "brq_qlinear_noalloc_limit", "brq_qlinear_noalloc",
)


class BrqError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


class Orp(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32), ("stride", ctypes.c_int32)]


class Quant(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group", ctypes.c_int32), ("codebook", ctypes.c_float * 32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libbrq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m butterfly_rotation_quantization_amd.build` (no CPU fallback exists)")
    # PyTorch ships its own HIP runtime.  Loading it first makes libbrq.so bind
    # to that same runtime (same soname): one runtime per process, and tensors
    # and streams from PyTorch are valid in the library.  Loaded the other way
    # round, PyTorch would find the system runtime already in place and see no
    # GPU.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = bind(ctypes.CDLL(path))
    if path == LIB_PATH:
        _lib = lib
    return lib


def bind(lib):
    """Declare the argument and result types of the C ABI on a loaded library."""
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.brq_status_string.argtypes = [i32]
    lib.brq_status_string.restype = ctypes.c_char_p
    lib.brq_last_error.argtypes = []
    lib.brq_last_error.restype = ctypes.c_char_p
    lib.brq_version.restype = i32
    lib.brq_plan_create.argtypes = [ctypes.POINTER(vp), i32, i32, vp, vp, i32, vp]
    lib.brq_plan_create.restype = i32
    lib.brq_plan_destroy.argtypes = [vp]
    lib.brq_plan_destroy.restype = i32
    lib.brq_plan_dim.argtypes = [vp]
    lib.brq_plan_dim.restype = i32
    lib.brq_workspace_bytes.argtypes = [vp, vp, i64, i64]
    lib.brq_workspace_bytes.restype = sz
    rot = [vp, i32, vp, i32, i64, vp, i32, i64, i64, i64, vp, sz, vp]
    lib.brq_rotate.argtypes = rot
    lib.brq_rotate.restype = i32
    lib.brq_rotate_inverse.argtypes = rot
    lib.brq_rotate_inverse.restype = i32
    lib.brq_rotate_quantize_pack.argtypes = [vp, vp, vp, i32, i64, i64, i64,
                                             ctypes.POINTER(Quant), vp, vp, vp, sz, vp]
    lib.brq_rotate_quantize_pack.restype = i32
    lib.brq_dequant_unrotate.argtypes = [vp, vp, vp, vp, ctypes.POINTER(Quant), i64, i64,
                                         vp, i32, i64, vp, sz, vp]
    lib.brq_dequant_unrotate.restype = i32
    lib.brq_lloyd_max_gaussian.argtypes = [i32, vp]
    lib.brq_lloyd_max_gaussian.restype = i32
    lib.brq_profile_enable.argtypes = [i32]
    lib.brq_profile_enable.restype = i32
    lib.brq_profile_reset.argtypes = []
    lib.brq_profile_reset.restype = i32
    lib.brq_profile_count.argtypes = []
    lib.brq_profile_count.restype = i32
    lib.brq_profile_read.argtypes = [i32, ctypes.c_char_p, sz, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(i64)]
    lib.brq_profile_read.restype = i32
    if hasattr(lib, "brq_harp_blocks"):
        lib.brq_harp_blocks.argtypes = [i32, i64, vp, ctypes.c_float, vp, vp, vp]
        lib.brq_harp_blocks.restype = i32
    if hasattr(lib, "brq_harp_blocks_batch"):
        lib.brq_harp_blocks_batch.argtypes = [i32, ctypes.POINTER(HarpJob), vp]
        lib.brq_harp_blocks_batch.restype = i32
        lib.brq_plan_create_harp.argtypes = [ctypes.POINTER(vp), i32, i32, vp, vp, vp, vp, vp]
        lib.brq_plan_create_harp.restype = i32
    if hasattr(lib, "brq_requant"):
        lib.brq_requant_workspace_bytes.argtypes = [vp, ctypes.POINTER(Quant), ctypes.POINTER(Quant),
                                                    i64, i64]
        lib.brq_requant_workspace_bytes.restype = sz
        lib.brq_requant.argtypes = [vp, vp, vp, ctypes.POINTER(Quant), i64, i64,
                                    ctypes.POINTER(Quant), vp, vp, vp, sz, vp]
        lib.brq_requant.restype = i32
    if hasattr(lib, "brq_qlinear"):
        lib.brq_qlinear_workspace_bytes.argtypes = [vp, vp, ctypes.POINTER(Quant), i64, i64, i64]
        lib.brq_qlinear_workspace_bytes.restype = sz
        lib.brq_qlinear.argtypes = [vp, vp, vp, i32, i64, i64, vp, vp, ctypes.POINTER(Quant), i64,
                                    i64, vp, i32, i64, vp, sz, vp]
        lib.brq_qlinear.restype = i32
    if hasattr(lib, "brq_qlinear_noalloc"):
        lib.brq_qlinear_noalloc_limit.argtypes = []
        lib.brq_qlinear_noalloc_limit.restype = sz
        lib.brq_qlinear_noalloc.argtypes = [vp, vp, vp, i32, i64, i64, vp, vp, ctypes.POINTER(Quant),
                                            i64, i64, vp, i32, i64, vp]
        lib.brq_qlinear_noalloc.restype = i32
    if hasattr(lib, "brq_orp_geo_quantize"):
        lib.brq_orp_geo_quantize.argtypes = [vp, i32, i64, i64, i64, vp, ctypes.POINTER(Orp), vp, vp,
                                             vp, vp]
        lib.brq_orp_geo_quantize.restype = i32
        lib.brq_orp_geo_dequant.argtypes = [vp, vp, vp, ctypes.POINTER(Orp), i64, i64, vp, i32, i64,
                                            vp]
        lib.brq_orp_geo_dequant.restype = i32
    if hasattr(lib, "brq_plan_serialize"):
        lib.brq_plan_serialize.argtypes = [vp, vp, sz, ctypes.POINTER(sz)]
        lib.brq_plan_serialize.restype = i32
        lib.brq_plan_deserialize.argtypes = [ctypes.POINTER(vp), vp, sz]
        lib.brq_plan_deserialize.restype = i32
    if hasattr(lib, "brq_set_path"):  # libraries built before the path switch lack it
        lib.brq_set_path.argtypes = [i32]
        lib.brq_set_path.restype = i32
    return lib


def lib():
    return load_library()


def check(status: int):
    if status != 0:
        raise BrqError(status, lib().brq_last_error().decode())


# ---------------------------------------------------------------- plans

class Plan:
    """A device transform plan (owns the brq_plan*)."""

    def __init__(self, d: int, radix: Sequence[int], mode="hadamard",
                 blocks: Optional[Sequence[np.ndarray]] = None,
                 signs: Optional[np.ndarray] = None):
        L = lib()
        mode_i = _MODES[mode] if isinstance(mode, str) else int(mode)
        r = np.ascontiguousarray(np.asarray(radix, dtype=np.int32))
        blk = None
        if blocks is not None:
            blk = np.ascontiguousarray(
                np.concatenate([np.asarray(b, dtype=np.float32).reshape(-1) for b in blocks]))
        sg = None if signs is None else np.ascontiguousarray(np.asarray(signs, dtype=np.int8))
        h = ctypes.c_void_p()
        check(L.brq_plan_create(ctypes.byref(h), int(d), len(r), r.ctypes.data,
                                None if blk is None else blk.ctypes.data, mode_i,
                                None if sg is None else sg.ctypes.data))
        self._h = h
        self.d = int(d)
        self.radix = tuple(int(x) for x in r)
        self.mode = mode_i

    @classmethod
    def from_harp(cls, d: int, radix: Sequence[int], theta_q: np.ndarray, scales: Sequence[float],
                  bases: Optional[Sequence[Optional[np.ndarray]]] = None,
                  signs: Optional[np.ndarray] = None) -> "Plan":
        """A per-group plan whose blocks the device builds from int8 HARP
        parameters (brq_plan_create_harp).  bases[t] is G of stage t; None
        for all stages means Sylvester everywhere."""
        L = lib()
        r = np.ascontiguousarray(np.asarray(radix, dtype=np.int32))
        th = np.ascontiguousarray(np.asarray(theta_q, dtype=np.int8).reshape(-1))
        sc = np.ascontiguousarray(np.asarray(scales, dtype=np.float32))
        bs = None
        if bases is not None:
            bs = np.ascontiguousarray(np.concatenate(
                [np.asarray(g, dtype=np.float32).reshape(-1) for g in bases]))
        sg = None if signs is None else np.ascontiguousarray(np.asarray(signs, dtype=np.int8))
        h = ctypes.c_void_p()
        check(L.brq_plan_create_harp(ctypes.byref(h), int(d), len(r), r.ctypes.data,
                                     th.ctypes.data if th.size else None, sc.ctypes.data,
                                     None if bs is None else bs.ctypes.data,
                                     None if sg is None else sg.ctypes.data))
        self = cls.__new__(cls)
        self._h = h
        self.d = int(d)
        self.radix = tuple(int(x) for x in r)
        self.mode = _MODES["per_group"]
        return self

    def serialize(self) -> bytes:
        """Byte image of the plan (brq_plan_serialize)."""
        L = lib()
        n = ctypes.c_size_t()
        check(L.brq_plan_serialize(self._h, None, 0, ctypes.byref(n)))
        buf = ctypes.create_string_buffer(n.value)
        check(L.brq_plan_serialize(self._h, buf, n.value, ctypes.byref(n)))
        return buf.raw[:n.value]

    @classmethod
    def deserialize(cls, image: bytes) -> "Plan":
        """Rebuild a plan from brq_plan_serialize's image on the current device."""
        L = lib()
        h = ctypes.c_void_p()
        check(L.brq_plan_deserialize(ctypes.byref(h), image, len(image)))
        self = cls.__new__(cls)
        self._h = h
        self.d = int(L.brq_plan_dim(h))
        self.radix = None
        self.mode = None
        return self

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().brq_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _h(plan: Optional[Plan]):
    return None if plan is None else plan.handle


# ---------------------------------------------------------------- torch marshalling

def dtype_code(t) -> int:
    import torch
    return {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}[t.dtype]


def _torch_dtype(code: int):
    import torch
    return {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}[code]


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ld(t) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return int(t.stride(0))


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def workspace_bytes(left: Optional[Plan], right: Optional[Plan], m: int, n: int) -> int:
    return int(lib().brq_workspace_bytes(_h(left), _h(right), int(m), int(n)))


def workspace(left, right, m, n, device="cuda"):
    import torch
    nb = workspace_bytes(left, right, m, n)
    return torch.empty(max(nb, 4) // 4 + 1, dtype=torch.float32, device=device)


def _ws_args(ws):
    if ws is None:
        return None, 0
    return int(ws.data_ptr()), int(ws.numel() * ws.element_size())


def harp_blocks(b: int, theta_q, scale: float, base=None, out=None, stream=None):
    """Blocks Q(theta) G of one stage from device int8 parameters theta_q
    [ngroups, np] (brq_harp_blocks); base is a device float32 [b, b] G or
    None (Sylvester).  Returns out, a device float32 [ngroups, b, b]."""
    import torch
    ng = theta_q.shape[0]
    if out is None:
        out = torch.empty((ng, b, b), dtype=torch.float32, device=theta_q.device)
    check(lib().brq_harp_blocks(int(b), int(ng), _ptr(theta_q), float(scale),
                                None if base is None else _ptr(base), _ptr(out), _stream(stream)))
    return out


class HarpJob(ctypes.Structure):
    """brq_harp_job: one stage's blocks for brq_harp_blocks_batch."""
    _fields_ = [("b", ctypes.c_int32), ("ngroups", ctypes.c_int64), ("theta_q", ctypes.c_void_p),
                ("scale", ctypes.c_float), ("base", ctypes.c_void_p), ("blocks", ctypes.c_void_p)]


def harp_blocks_batch(jobs, stream=None):
    """Several stages' blocks in one call (brq_harp_blocks_batch): jobs is a
    list of (b, theta_q, scale, base or None, out) with device tensors as for
    harp_blocks (out a device float32 [ngroups, b, b])."""
    arr = (HarpJob * max(1, len(jobs)))()
    for i, (b, theta_q, scale, base, out) in enumerate(jobs):
        arr[i] = HarpJob(int(b), int(theta_q.shape[0]), _ptr(theta_q), float(scale),
                         None if base is None else _ptr(base), _ptr(out))
    check(lib().brq_harp_blocks_batch(len(jobs), arr, _stream(stream)))


def rotate(plan: Plan, x, y=None, side="right", ws=None, stream=None, inverse=False):
    """Y = X M^T (side "right", rows or d-chunks of rows) or Y = M X (side
    "left"); inverse=True applies M^T.  Returns y."""
    import torch
    side_i = _SIDES[side] if isinstance(side, str) else int(side)
    if y is None:
        y = torch.empty_like(x)
    if ws is None:
        ws = workspace(plan if side_i == LEFT else None, plan if side_i == RIGHT else None,
                       x.shape[0], x.shape[1], x.device)
    wp, wb = _ws_args(ws)
    fn = lib().brq_rotate_inverse if inverse else lib().brq_rotate
    check(fn(plan.handle, side_i, _ptr(x), dtype_code(x), _ld(x), _ptr(y), dtype_code(y), _ld(y),
             int(x.shape[0]), int(x.shape[1]), wp, wb, _stream(stream)))
    return y


def rotate_inverse(plan: Plan, x, y=None, side="right", ws=None, stream=None):
    return rotate(plan, x, y, side, ws, stream, inverse=True)


def make_quant(bits: int, group: int, kind="absmax", codebook=None) -> Quant:
    q = Quant()
    q.kind = _KINDS[kind] if isinstance(kind, str) else int(kind)
    q.bits = int(bits)
    q.group = int(group)
    if codebook is not None:
        cb = np.asarray(codebook, dtype=np.float32).reshape(-1)
        for i, v in enumerate(cb):
            q.codebook[i] = float(v)
    return q


def rotate_quantize_pack(left: Optional[Plan], right: Optional[Plan], w, bits: int, group: int,
                         kind="absmax", codebook=None, codes=None, scales=None, ws=None,
                         stream=None):
    """W' = M_U W M_V^T, then group quantization along rows and LSB-first
    packing.  Returns (codes uint8 [m, n*bits/8], scales [m, n/group])."""
    import torch
    m, n = int(w.shape[0]), int(w.shape[1])
    q = make_quant(bits, group, kind, codebook)
    if codes is None:
        codes = torch.empty((m, n * bits // 8), dtype=torch.uint8, device=w.device)
    if scales is None:
        sd = torch.float32 if q.kind == ABSMAX else torch.float16
        scales = torch.empty((m, n // group), dtype=sd, device=w.device)
    if ws is None:
        ws = workspace(left, right, m, n, w.device)
    wp, wb = _ws_args(ws)
    check(lib().brq_rotate_quantize_pack(_h(left), _h(right), _ptr(w), dtype_code(w), m, n,
                                         _ld(w), ctypes.byref(q), _ptr(codes), _ptr(scales),
                                         wp, wb, _stream(stream)))
    return codes, scales


def dequant_unrotate(left: Optional[Plan], right: Optional[Plan], codes, scales, m: int, n: int,
                     bits: int, group: int, kind="absmax", codebook=None, out=None,
                     out_dtype=None, ws=None, stream=None):
    """W = M_U^T deq(codes) M_V.  Returns out [m, n]."""
    import torch
    q = make_quant(bits, group, kind, codebook)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype or torch.float32, device=codes.device)
    if ws is None:
        ws = workspace(left, right, m, n, codes.device)
    wp, wb = _ws_args(ws)
    check(lib().brq_dequant_unrotate(_h(left), _h(right), _ptr(codes), _ptr(scales),
                                     ctypes.byref(q), int(m), int(n), _ptr(out), dtype_code(out),
                                     _ld(out), wp, wb, _stream(stream)))
    return out


def requant(right: Optional[Plan], codes, scales, m: int, n: int, bits_in: int, group_in: int,
            bits_out: int, group_out: int, kind_in="codebook_norm", codebook=None,
            codes_out=None, scales_out=None, ws=None, stream=None):
    """Restore (dequantize + inverse right plan), then absmax-quantize the
    restored rows at bits_out / group_out (brq_requant).  Returns
    (codes_out uint8 [m, n*bits_out/8], scales_out float32 [m, n/group_out])."""
    import torch
    L = lib()
    qi = make_quant(bits_in, group_in, kind_in, codebook)
    qo = make_quant(bits_out, group_out, "absmax")
    dev = codes.device
    if codes_out is None:
        codes_out = torch.empty((m, n * bits_out // 8), dtype=torch.uint8, device=dev)
    if scales_out is None:
        scales_out = torch.empty((m, n // group_out), dtype=torch.float32, device=dev)
    if ws is None:
        nb = L.brq_requant_workspace_bytes(_h(right), ctypes.byref(qi), ctypes.byref(qo), int(m), int(n))
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev) if nb else None
    wp, wb = _ws_args(ws)
    check(L.brq_requant(_h(right), _ptr(codes), _ptr(scales), ctypes.byref(qi), int(m), int(n),
                        ctypes.byref(qo), _ptr(codes_out), _ptr(scales_out), wp, wb, _stream(stream)))
    return codes_out, scales_out


def qlinear_workspace_bytes(left: Optional[Plan], right: Optional[Plan], bits: int, group: int,
                            T: int, m: int, n: int) -> int:
    """Bytes of device workspace brq_qlinear needs for T tokens."""
    q = make_quant(bits, group, "absmax")
    return int(lib().brq_qlinear_workspace_bytes(_h(left), _h(right), ctypes.byref(q), int(T),
                                                 int(m), int(n)))


def qlinear(left: Optional[Plan], right: Optional[Plan], x, codes, scales, m: int, n: int,
            bits: int, group: int, y=None, out_dtype=None, ws=None, stream=None):
    """Y = X W^T for the weight W = M_U^T W' M_V stored as the absmax codes and
    scales of W' (brq_qlinear): rotate X, the quantized product, unrotate.
    x [T, n] f16/bf16.  Returns y [T, m]."""
    import torch
    L = lib()
    T = int(x.shape[0])
    q = make_quant(bits, group, "absmax")
    if y is None:
        y = torch.empty((T, m), dtype=out_dtype or x.dtype, device=x.device)
    if ws is None:
        nb = L.brq_qlinear_workspace_bytes(_h(left), _h(right), ctypes.byref(q), T, int(m), int(n))
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=x.device)
    wp, wb = _ws_args(ws)
    check(L.brq_qlinear(_h(left), _h(right), _ptr(x), dtype_code(x), _ld(x), T, _ptr(codes),
                        _ptr(scales), ctypes.byref(q), int(m), int(n), _ptr(y), dtype_code(y),
                        _ld(y), wp, wb, _stream(stream)))
    return y


def qlinear_noalloc(left: Optional[Plan], right: Optional[Plan], x, codes, scales, m: int, n: int,
                    bits: int, group: int, y=None, out_dtype=None, stream=None):
    """brq_qlinear without a workspace (brq_qlinear_noalloc): the library's
    per-device scratch array is used; returns y [T, m]."""
    import torch
    T = int(x.shape[0])
    q = make_quant(bits, group, "absmax")
    if y is None:
        y = torch.empty((T, m), dtype=out_dtype or x.dtype, device=x.device)
    check(lib().brq_qlinear_noalloc(_h(left), _h(right), _ptr(x), dtype_code(x), _ld(x), T,
                                    _ptr(codes), _ptr(scales), ctypes.byref(q), int(m), int(n),
                                    _ptr(y), dtype_code(y), _ld(y), _stream(stream)))
    return y


def orp_geo_quantize(w, bits: int, group: int, stride: int, smooth=None, codes=None, signs=None,
                     coef=None, stream=None):
    """ORP GEO quantizer (brq_orp_geo_quantize): w [m, n] f32/bf16/f16 on the
    device, optional float32 smoothing vector [n].  Returns (codes [m, n*bits/8]
    uint8, signs [m, n/16] uint8, coef [m, n/group, 2] float32)."""
    import torch
    m, n = int(w.shape[0]), int(w.shape[1])
    dev = w.device
    if codes is None:
        codes = torch.empty((m, n * bits // 8), dtype=torch.uint8, device=dev)
    if signs is None:
        signs = torch.empty((m, n // 16), dtype=torch.uint8, device=dev)
    if coef is None:
        coef = torch.empty((m, n // group, 2), dtype=torch.float32, device=dev)
    q = Orp(bits, group, stride)
    check(lib().brq_orp_geo_quantize(_ptr(w), dtype_code(w), m, n, _ld(w), _ptr(smooth),
                                     ctypes.byref(q), _ptr(codes), _ptr(signs), _ptr(coef),
                                     _stream(stream)))
    return codes, signs, coef


def orp_geo_dequant(codes, signs, coef, m: int, n: int, bits: int, group: int, stride: int,
                    out=None, out_dtype=None, stream=None):
    """w_p^ = c1 b1 + c2 b2 (brq_orp_geo_dequant).  Returns out [m, n]."""
    import torch
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype or torch.float32, device=codes.device)
    q = Orp(bits, group, stride)
    check(lib().brq_orp_geo_dequant(_ptr(codes), _ptr(signs), _ptr(coef), ctypes.byref(q), int(m),
                                    int(n), _ptr(out), dtype_code(out), _ld(out), _stream(stream)))
    return out


def profile_enable(on: bool = True):
    """Bracket every kernel launch of the hot calls with HIP events on its stream."""
    check(lib().brq_profile_enable(1 if on else 0))


def profile_reset():
    check(lib().brq_profile_reset())


def profile_read() -> dict:
    """{kernel name: (total ms, launches)} since the last reset (waits for the events)."""
    L = lib()
    out = {}
    for i in range(L.brq_profile_count()):
        buf = ctypes.create_string_buffer(256)
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        check(L.brq_profile_read(i, buf, 256, ctypes.byref(ms), ctypes.byref(n)))
        out[buf.value.decode()] = (ms.value, n.value)
    return out


PATH_AUTO, PATH_TILE = 0, 1


def set_path(path: int):
    """Kernel selection: PATH_AUTO (fastest kernel that takes a call) or
    PATH_TILE (every call on the multi-stage tile pass)."""
    check(lib().brq_set_path(int(path)))


class tile_path:
    """Context manager: run the enclosed calls on the tile pass."""

    def __enter__(self):
        set_path(PATH_TILE)
        return self

    def __exit__(self, *exc):
        set_path(PATH_AUTO)
        return False


def lloyd_max_gaussian(bits: int) -> np.ndarray:
    """2^bits float32 Lloyd-Max centroids for N(0,1), computed by the library."""
    out = np.zeros(1 << bits, dtype=np.float32)
    check(lib().brq_lloyd_max_gaussian(int(bits), out.ctypes.data))
    return out
