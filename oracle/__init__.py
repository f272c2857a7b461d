"""CPU oracle for MoE expert-parallel dispatch and combine, and the
expert-major layout of the received rows.

TEST INFRASTRUCTURE ONLY. A plain, slow, single-threaded C definition of what
dispatch and combine compute (``ep_oracle.c``), bound here with ctypes over
numpy arrays. Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import it; the GPU library never does, and the two
share no code. Passages followed and readings taken are listed in
``ep_oracle.h``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

BF16 = 0
FP16 = 1


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    P = ctypes.c_void_p
    I = ctypes.c_int
    Z = ctypes.c_size_t
    lib.oracle_dispatch.argtypes = [I, I, I, I, Z, Z, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.oracle_dispatch.restype = I
    lib.oracle_layout_by_sort.argtypes = [I, I, I, I, P, P, P, P]
    lib.oracle_layout_by_sort.restype = I
    lib.oracle_combine.argtypes = [I, I, I, I, I, P, P, P, P, P, P]
    lib.oracle_combine.restype = I
    lib.oracle_combine_push.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P]
    lib.oracle_combine_push.restype = I
    lib.oracle_expert_layout.argtypes = [I, I, I, I, I, Z, Z, P, P, P, P, P, P, P, P, P, P]
    lib.oracle_expert_layout.restype = I
    lib.oracle_expert_combine.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P]
    lib.oracle_expert_combine.restype = I
    lib.oracle_expert_combine_wire.argtypes = [I, I, I, I, I, I, I, I, P, P, P, P, P, P]
    lib.oracle_expert_combine_wire.restype = I
    lib.oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_e4m3.restype = ctypes.c_uint8
    lib.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_e2m1.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_e2m1.restype = ctypes.c_uint8
    lib.oracle_e2m1_to_f32.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_to_f32.restype = ctypes.c_float
    lib.oracle_cast_to_e4m3_n.argtypes = [P, I, P, Z]
    lib.oracle_cast_to_e4m3_n.restype = None
    lib.oracle_quantize_rows.argtypes = [ctypes.c_int64, I, I, I, P, P, P]
    lib.oracle_quantize_rows.restype = I
    lib.oracle_combine_wire.argtypes = [I, I, I, I, I, I, P, P, P, P, P]
    lib.oracle_combine_wire.restype = I
    for name in ("oracle_f32_to_bf16_n", "oracle_f32_to_f16_n",
                 "oracle_bf16_to_f32_n", "oracle_f16_to_f32_n"):
        getattr(lib, name).argtypes = [P, P, Z]
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype is not None:
        assert a.dtype == dtype, (a.dtype, dtype)
    return a


def dispatch(W, M, k, Er, ntok, x, idx, w=None, scales=None):
    """Dispatch by definition. ``x`` is any contiguous array shaped [W, M, ...]
    whose trailing bytes form one payload row; ``scales`` likewise (or None).
    Returns a dict of out_x (uint8 [W, W*M, row_bytes]), out_idx, out_w,
    out_scales (uint8 rows), recv [W], src_pos [W, W*M], fwd [W, M, min(W,k)].
    Rows that receive nothing stay zero."""
    lib = _load()
    ntok = _c(np.asarray(ntok, dtype=np.int32))
    x = _c(x)
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    scales = _c(scales)
    WM = W * M
    P = min(W, k)
    row_bytes = x.nbytes // (W * M)
    scale_bytes = 0 if scales is None else scales.nbytes // (W * M)
    out = dict(
        out_x=np.zeros((W, WM, row_bytes), np.uint8),
        out_idx=np.zeros((W, WM, k), np.int32),
        out_w=None if w is None else np.zeros((W, WM, k), np.float32),
        out_scales=None if scales is None else np.zeros((W, WM, scale_bytes), np.uint8),
        recv=np.zeros(W, np.int32),
        src_pos=np.full((W, WM), -1, np.int32),
        fwd=np.full((W, M, P), -1, np.int32),
    )
    rc = lib.oracle_dispatch(W, M, k, Er, row_bytes, scale_bytes, _ptr(ntok), _ptr(x), _ptr(idx),
                             _ptr(w), _ptr(scales), _ptr(out["out_x"]), _ptr(out["out_idx"]),
                             _ptr(out["out_w"]), _ptr(out["out_scales"]), _ptr(out["recv"]),
                             _ptr(out["src_pos"]), _ptr(out["fwd"]))
    if rc != 0:
        raise RuntimeError(f"oracle_dispatch failed ({rc})")
    return out


def layout_by_sort(W, M, k, Er, ntok, idx):
    """Second formulation of the receive layout (sort of (d, r, t) triples).
    Returns (recv [W], src_pos [W, W*M])."""
    lib = _load()
    ntok = _c(np.asarray(ntok, dtype=np.int32))
    idx = _c(idx, np.int32)
    recv = np.zeros(W, np.int32)
    src_pos = np.full((W, W * M), -1, np.int32)
    rc = lib.oracle_layout_by_sort(W, M, k, Er, _ptr(ntok), _ptr(idx), _ptr(recv), _ptr(src_pos))
    if rc != 0:
        raise RuntimeError(f"oracle_layout_by_sort failed ({rc})")
    return recv, src_pos


def combine(W, M, k, H, dtype, ntok, fwd, y, y_w=None):
    """Combine by definition (gather form). ``y`` holds 16-bit words
    [W, W*M, H] (bf16 when dtype == BF16, fp16 when FP16). Returns
    (out uint16 [W, M, H], out_w float32 [W, M, k] or None); rows of absent
    tokens stay zero."""
    lib = _load()
    ntok = _c(np.asarray(ntok, dtype=np.int32))
    fwd = _c(fwd, np.int32)
    y = _c(y).view(np.uint16)
    y_w = _c(y_w, np.float32)
    out = np.zeros((W, M, H), np.uint16)
    out_w = None if y_w is None else np.zeros((W, M, k), np.float32)
    rc = lib.oracle_combine(W, M, k, H, dtype, _ptr(ntok), _ptr(fwd), _ptr(y), _ptr(y_w),
                            _ptr(out), _ptr(out_w))
    if rc != 0:
        raise RuntimeError(f"oracle_combine failed ({rc})")
    return out, out_w


def combine_push(W, M, k, Er, H, dtype, ntok, idx, recv, src_pos, y, y_w=None):
    """Combine, second formulation (push form through src_pos)."""
    lib = _load()
    ntok = _c(np.asarray(ntok, dtype=np.int32))
    idx = _c(idx, np.int32)
    recv = _c(recv, np.int32)
    src_pos = _c(src_pos, np.int32)
    y = _c(y).view(np.uint16)
    y_w = _c(y_w, np.float32)
    out = np.zeros((W, M, H), np.uint16)
    out_w = None if y_w is None else np.zeros((W, M, k), np.float32)
    rc = lib.oracle_combine_push(W, M, k, Er, H, dtype, _ptr(ntok), _ptr(idx), _ptr(recv),
                                 _ptr(src_pos), _ptr(y), _ptr(y_w), _ptr(out), _ptr(out_w))
    if rc != 0:
        raise RuntimeError(f"oracle_combine_push failed ({rc})")
    return out, out_w


def expert_layout(W, M, k, Er, cap, recv, src_pos, x, idx, scales=None, fill=-1):
    """Expert-major layout of dispatch outputs by definition. ``x`` is any
    contiguous array shaped [W, W*M, ...] (one payload row per trailing block),
    ``idx`` int32 [W, W*M, k], ``scales`` likewise or None. Returns a dict of
    px (uint8 [W, Er, cap, row_bytes]), psc (uint8 rows or None), count
    [W, Er], src_info [W, Er, cap] (slots past the kept rows hold ``fill``),
    layout_range int64 [W, Er, W]. Unwritten payload bytes stay zero."""
    lib = _load()
    WM = W * M
    recv = _c(np.asarray(recv, dtype=np.int32))
    src_pos = _c(src_pos, np.int32)
    x = _c(x)
    idx = _c(idx, np.int32)
    scales = _c(scales)
    row_bytes = x.nbytes // (W * WM)
    scale_bytes = 0 if scales is None else scales.nbytes // (W * WM)
    out = dict(
        px=np.zeros((W, Er, cap, row_bytes), np.uint8),
        psc=None if scales is None else np.zeros((W, Er, cap, scale_bytes), np.uint8),
        count=np.zeros((W, Er), np.int32),
        src_info=np.full((W, Er, cap), fill, np.int32),
        layout_range=np.zeros((W, Er, W), np.int64),
    )
    rc = lib.oracle_expert_layout(W, M, k, Er, cap, row_bytes, scale_bytes, _ptr(recv),
                                  _ptr(src_pos), _ptr(x), _ptr(idx), _ptr(scales),
                                  _ptr(out["px"]), _ptr(out["psc"]), _ptr(out["count"]),
                                  _ptr(out["src_info"]), _ptr(out["layout_range"]))
    if rc != 0:
        raise RuntimeError(f"oracle_expert_layout failed ({rc})")
    return out


def expert_combine(W, M, k, Er, cap, H, dtype, recv, idx, py, w=None):
    """Inverse of the expert-major layout by definition: ``py`` holds 16-bit
    words [W, Er, cap, H]; ``w`` the dispatched weight rows float32
    [W, W*M, k] for the weighted form (None: unweighted). Returns y uint16
    [W, W*M, H]; rows past recv[d] stay zero."""
    lib = _load()
    recv = _c(np.asarray(recv, dtype=np.int32))
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    py = _c(py).view(np.uint16)
    y = np.zeros((W, W * M, H), np.uint16)
    rc = lib.oracle_expert_combine(W, M, k, Er, cap, H, dtype, _ptr(recv), _ptr(idx), _ptr(w),
                                   _ptr(py), _ptr(y))
    if rc != 0:
        raise RuntimeError(f"oracle_expert_combine failed ({rc})")
    return y


def expert_combine_wire(W, M, k, Er, cap, H, dtype, wire, recv, idx, py, py_scales, w=None):
    """The inverse with the packed expert outputs on a wire: ``py`` uint8 wire
    rows [W, Er, cap, ...], ``py_scales`` their scale rows (float32 or uint8
    E8M0); otherwise as expert_combine."""
    lib = _load()
    recv = _c(np.asarray(recv, dtype=np.int32))
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    py = _c(py, np.uint8)
    py_scales = _c(py_scales)
    y = np.zeros((W, W * M, H), np.uint16)
    rc = lib.oracle_expert_combine_wire(W, M, k, Er, cap, H, dtype, wire, _ptr(recv), _ptr(idx),
                                        _ptr(w), _ptr(py), _ptr(py_scales), _ptr(y))
    if rc != 0:
        raise RuntimeError(f"oracle_expert_combine_wire failed ({rc})")
    return y


WIRE_FP8_BLOCK128 = 1
WIRE_MXFP4 = 2


def f32_to_e4m3(v):
    return _load().oracle_f32_to_e4m3(float(v))


def e4m3_to_f32(c):
    return _load().oracle_e4m3_to_f32(int(c))


def f32_to_e2m1(v):
    return _load().oracle_f32_to_e2m1(float(v))


def e2m1_to_f32(c):
    return _load().oracle_e2m1_to_f32(int(c))


def cast_to_e4m3(words, dtype):
    """bf16 (dtype BF16) / fp16 (FP16) words -> E4M3 codes, direct cast."""
    lib = _load()
    words = np.ascontiguousarray(words, dtype=np.uint16)
    out = np.empty(words.shape, np.uint8)
    lib.oracle_cast_to_e4m3_n(_ptr(words), dtype, _ptr(out), words.size)
    return out


def quantize_rows(words, dtype, wire):
    """Rows [..., H] of bf16 / fp16 words into a wire format. Returns (codes,
    scales): FP8 block-128: uint8 [..., H] and float32 [..., H/128]; MXFP4:
    uint8 [..., H/2] packed and uint8 E8M0 [..., H/32]."""
    lib = _load()
    words = np.ascontiguousarray(words, dtype=np.uint16)
    H = words.shape[-1]
    lead = words.shape[:-1]
    n = words.size // H
    if wire == WIRE_FP8_BLOCK128:
        out = np.zeros(lead + (H,), np.uint8)
        scales = np.zeros(lead + (H // 128,), np.float32)
    else:
        out = np.zeros(lead + (H // 2,), np.uint8)
        scales = np.zeros(lead + (H // 32,), np.uint8)
    rc = lib.oracle_quantize_rows(n, H, dtype, wire, _ptr(words), _ptr(out), _ptr(scales))
    if rc != 0:
        raise RuntimeError(f"oracle_quantize_rows failed ({rc})")
    return out, scales


def combine_wire(W, M, k, H, dtype, wire, ntok, fwd, y, y_scales):
    """Combine by definition from wire rows y [W, W*M, ...] and their scales.
    Returns out uint16 [W, M, H]; rows of absent tokens stay zero."""
    lib = _load()
    ntok = _c(np.asarray(ntok, dtype=np.int32))
    fwd = _c(fwd, np.int32)
    y = _c(y)
    y_scales = _c(y_scales)
    out = np.zeros((W, M, H), np.uint16)
    rc = lib.oracle_combine_wire(W, M, k, H, dtype, wire, _ptr(ntok), _ptr(fwd), _ptr(y),
                                 _ptr(y_scales), _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_combine_wire failed ({rc})")
    return out


def _conv(name, a, in_dtype, out_dtype):
    lib = _load()
    a = np.ascontiguousarray(a, dtype=in_dtype)
    out = np.empty(a.shape, out_dtype)
    getattr(lib, name)(_ptr(a), _ptr(out), a.size)
    return out


def f32_to_bf16(a):
    return _conv("oracle_f32_to_bf16_n", a, np.float32, np.uint16)


def f32_to_f16(a):
    return _conv("oracle_f32_to_f16_n", a, np.float32, np.uint16)


def bf16_to_f32(a):
    return _conv("oracle_bf16_to_f32_n", a, np.uint16, np.float32)


def f16_to_f32(a):
    return _conv("oracle_f16_to_f32_n", a, np.uint16, np.float32)
