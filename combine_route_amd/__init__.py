"""Python binding of the combine_route_amd C ABI (include/ep.h).

MoE expert-parallel dispatch and combine for W virtual ranks held in one
MI355X's HBM, computed by the gfx950 kernels of libcombine_route_amd.so. This
module only marshals arguments: the functions below carry the C names and
pass tensor addresses through; torch provides device memory and streams.
Before a pointer reaches the library, each tensor is checked to be a
contiguous device tensor at least as large as the call will touch, so a
wrong-sized buffer raises here instead of faulting the GPU.

There is no CPU fallback: if the library is not built, importing succeeds but
the first call raises.
"""
import ctypes
import os
import weakref
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcombine_route_amd.so")

EP_BF16, EP_FP16, EP_FP8_E4M3 = 0, 1, 2
EP_OK, EP_ERR_NULL, EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_SIZE, EP_ERR_STATE, EP_ERR_HIP = (
    0, -1, -2, -3, -4, -5, -6)
EP_KERNEL_ROUTE, EP_KERNEL_SCAN, EP_KERNEL_COPY, EP_KERNEL_COMBINE = 0, 1, 2, 3
(EP_KERNEL_EXPERT_COUNT, EP_KERNEL_EXPERT_SCAN, EP_KERNEL_EXPERT_COPY,
 EP_KERNEL_EXPERT_COMBINE) = 4, 5, 6, 7
(EP_KERNEL_STANDARD_COUNT, EP_KERNEL_STANDARD_SCAN, EP_KERNEL_STANDARD_COPY,
 EP_KERNEL_STANDARD_COMBINE) = 8, 9, 10, 11
EP_CACHE_AUTO, EP_CACHE_STREAM, EP_CACHE_KEEP = 0, 1, 2
EP_LAYOUT_AUTO, EP_LAYOUT_KERNELS, EP_LAYOUT_SCAN_IN_COPY, EP_LAYOUT_IN_COPY = 0, 1, 2, 3

EP_WIRE_NONE, EP_WIRE_FP8_BLOCK128, EP_WIRE_MXFP4 = 0, 1, 2
EP_CAST_NONE, EP_CAST_FP8_FROM_BF16, EP_CAST_FP8_FROM_FP16 = 0, 1, 2
CASTS = {None: EP_CAST_NONE, "none": EP_CAST_NONE, "bf16": EP_CAST_FP8_FROM_BF16,
         "fp16": EP_CAST_FP8_FROM_FP16}

DTYPES = {"bf16": EP_BF16, "fp16": EP_FP16, "fp8": EP_FP8_E4M3}
WIRES = {None: EP_WIRE_NONE, "none": EP_WIRE_NONE, "fp8_block128": EP_WIRE_FP8_BLOCK128,
         "mxfp4": EP_WIRE_MXFP4}
ELEM_BYTES = {EP_BF16: 2, EP_FP16: 2, EP_FP8_E4M3: 1}

EXPORTED = ("ep_workspace_bytes", "ep_plan_create", "ep_plan_destroy", "ep_dispatch",
            "ep_combine", "ep_get_src_token_pos", "ep_last_error", "ep_plan_set_launch",
            "ep_plan_get_launch", "ep_plan_set_timing", "ep_plan_kernel_time",
            "ep_expert_workspace_bytes", "ep_expert_plan_create", "ep_expert_plan_destroy",
            "ep_convert_dispatch_output", "ep_convert_combine_input", "ep_quantize_rows",
            "ep_dispatch_standard_moe", "ep_combine_standard_moe", "ep_probe_pattern",
            "ep_probe_forward_map", "ep_plan_static")
EP_STATIC_SCRATCH_BYTES = 4 << 20
EP_PROBE_READ, EP_PROBE_WRITE, EP_PROBE_COPY, EP_PROBE_FANOUT, EP_PROBE_GATHER = range(5)


class EpConfig(ctypes.Structure):
    """ep_config_t: after the pages' EpDispatchCombineConfig."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "world_size", "hidden_dim", "scale_dim", "scale_type_size", "max_num_inp_token_per_rank",
        "num_experts_per_rank", "num_experts_per_token", "dispatch_dtype", "combine_dtype",
        "combine_wire", "dispatch_cast")]


class EpDispatchArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "num_tokens", "x", "indices", "weights", "scales", "out_x", "out_indices",
        "out_weights", "out_scales", "recv_num_token")]


class EpCombineArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("y", "y_weights", "out", "out_weights",
                                               "y_scales")]


class EpLaunch(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "tile_tokens", "dispatch_waves", "dispatch_row_split", "combine_waves",
        "combine_row_split", "cache_policy", "layout", "expert_waves", "expert_row_split",
        "expert_combine_waves", "expert_combine_row_split", "expert_cache_policy",
        "expert_token_split", "dispatch_token_split")]


class EpConvertDispatchArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "indices", "weights", "scales", "recv_num_token", "packed_x", "packed_scales",
        "packed_count", "packed_src_info", "packed_layout_range")]


class EpConvertCombineArgs(ctypes.Structure):
    _fields_ = [("packed_y", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("apply_weights", ctypes.c_int32)]


class EpDispatchStandardArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "num_tokens", "x", "indices", "scales", "packed_x", "packed_scales", "packed_count",
        "packed_src_info", "packed_layout_range")]


class EpCombineStandardArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("packed_y", "indices", "weights", "out",
                                               "packed_y_scales")]


class EpProbeArgs(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("row_bytes", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("src", ctypes.c_void_p), ("dst", ctypes.c_void_p),
                ("map", ctypes.c_void_p), ("map_rows", ctypes.c_int64),
                ("stride", ctypes.c_int32), ("pieces", ctypes.c_int32),
                ("waves", ctypes.c_int32)]


class EpError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


_lib = None


def load():
    """The loaded library. Raises if it was not built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m combine_route_amd.build` "
                           "(or __graft_entry__.build()) first; there is no CPU fallback")
    lib = ctypes.CDLL(LIB_PATH)
    V, I, Z, P = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.POINTER
    lib.ep_workspace_bytes.argtypes = [P(EpConfig)]
    lib.ep_workspace_bytes.restype = Z
    lib.ep_plan_create.argtypes = [P(EpConfig), V, Z, P(V)]
    lib.ep_plan_destroy.argtypes = [V]
    lib.ep_plan_static.argtypes = [P(EpConfig), P(V)]
    lib.ep_dispatch.argtypes = [V, P(EpDispatchArgs), V]
    lib.ep_combine.argtypes = [V, P(EpCombineArgs), V]
    lib.ep_get_src_token_pos.argtypes = [V, ctypes.c_int32, P(V)]
    lib.ep_last_error.argtypes = []
    lib.ep_last_error.restype = ctypes.c_char_p
    lib.ep_plan_set_launch.argtypes = [V, P(EpLaunch)]
    lib.ep_plan_get_launch.argtypes = [V, V, P(EpLaunch)]
    lib.ep_plan_set_timing.argtypes = [V, I]
    lib.ep_plan_kernel_time.argtypes = [V, I, P(ctypes.c_int32), P(ctypes.c_double)]
    lib.ep_expert_workspace_bytes.argtypes = [V, ctypes.c_int32]
    lib.ep_expert_workspace_bytes.restype = Z
    lib.ep_expert_plan_create.argtypes = [V, ctypes.c_int32, V, Z, P(V)]
    lib.ep_expert_plan_destroy.argtypes = [V]
    lib.ep_convert_dispatch_output.argtypes = [V, P(EpConvertDispatchArgs), V]
    lib.ep_convert_combine_input.argtypes = [V, P(EpConvertCombineArgs), V]
    lib.ep_dispatch_standard_moe.argtypes = [V, P(EpDispatchStandardArgs), V]
    lib.ep_combine_standard_moe.argtypes = [V, P(EpCombineStandardArgs), V]
    lib.ep_quantize_rows.argtypes = [V, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, V, V, V, ctypes.c_int64, V]
    lib.ep_probe_pattern.argtypes = [P(EpProbeArgs), V]
    lib.ep_probe_forward_map.argtypes = [V, P(V), P(ctypes.c_int32)]
    for name in EXPORTED:
        if name not in ("ep_workspace_bytes", "ep_last_error", "ep_expert_workspace_bytes"):
            getattr(lib, name).restype = I
    _lib = lib
    return lib


def ep_last_error() -> str:
    return load().ep_last_error().decode()


def _check(fn, rc):
    if rc != EP_OK:
        raise EpError(fn, rc, ep_last_error())


def make_config(world_size, hidden_dim, max_num_inp_token_per_rank, num_experts_per_rank,
                num_experts_per_token, dispatch_dtype="bf16", combine_dtype=None,
                scale_dim=0, scale_type_size=4, combine_wire=None, dispatch_cast=None) -> EpConfig:
    """dispatch_cast: None, or "bf16" / "fp16": x of that type received as
    FP8 E4M3 (dispatch_dtype must then be "fp8")."""
    dd = DTYPES[dispatch_dtype] if isinstance(dispatch_dtype, str) else dispatch_dtype
    if combine_dtype is None:
        combine_dtype = EP_FP16 if dd == EP_FP16 else EP_BF16
    cd = DTYPES[combine_dtype] if isinstance(combine_dtype, str) else combine_dtype
    cw = WIRES[combine_wire] if combine_wire is None or isinstance(combine_wire, str) \
        else combine_wire
    dc = CASTS[dispatch_cast] if dispatch_cast is None or isinstance(dispatch_cast, str) \
        else dispatch_cast
    return EpConfig(world_size, hidden_dim, scale_dim, scale_type_size if scale_dim else 0,
                    max_num_inp_token_per_rank, num_experts_per_rank, num_experts_per_token,
                    dd, cd, cw, dc)


def ep_workspace_bytes(cfg: EpConfig) -> int:
    n = load().ep_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise EpError("ep_workspace_bytes", EP_ERR_ARG, ep_last_error())
    return n


_I32 = (torch.int32,)
_F32 = (torch.float32,)


def _payload(dtype_code):
    """Element types accepted for rows of an EP_* type: the type itself, or
    raw bytes (uint8) holding its encodings."""
    return (_TORCH[dtype_code], torch.uint8)


def _scale_types(elem_bytes):
    """Scale rows are copied as bytes: uint8, or any type of the config's
    scale element size."""
    return (torch.uint8,) + tuple(t for t in (torch.float32, torch.int32, torch.float16,
                                              torch.bfloat16, torch.int16, torch.float64,
                                              torch.int64, torch.int8)
                                  if torch.empty((), dtype=t).element_size() == elem_bytes)


def _dev(t: Optional[torch.Tensor], name: str, nbytes: int, dtypes=None):
    """Address of a contiguous device tensor of at least nbytes whose element
    type is one of dtypes (any when None), or None. The type is checked first:
    an int64 id tensor has enough bytes for the int32 ids it is mistaken for,
    and would be misread without an error."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, not {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes; this call needs {nbytes}")
    return t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device_index: Optional[int] = None) -> Optional[int]:
    """hipStream_t handle: the given stream, else torch's current stream."""
    if stream is None:
        if _raw_stream is not None and device_index is not None:
            return _raw_stream(device_index)
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def ep_plan_create(cfg: EpConfig, workspace: torch.Tensor) -> int:
    """Create a plan over a caller-owned workspace tensor (keep it alive)."""
    need = ep_workspace_bytes(cfg)
    ws = _dev(workspace, "workspace", need)
    out = ctypes.c_void_p()
    _check("ep_plan_create", load().ep_plan_create(
        ctypes.byref(cfg), ws, workspace.numel() * workspace.element_size(), ctypes.byref(out)))
    return out.value


def ep_plan_static(cfg: EpConfig) -> int:
    """ep_plan_static(): the current device's plan over the library's static
    scratch (no allocation). Every call returns the same plan, reset to cfg;
    calls that overlap on one device race (include/ep.h)."""
    out = ctypes.c_void_p()
    _check("ep_plan_static", load().ep_plan_static(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def ep_plan_destroy(plan: int) -> None:
    _check("ep_plan_destroy", load().ep_plan_destroy(plan))


def _sizes(cfg: EpConfig):
    W, M, k = cfg.world_size, cfg.max_num_inp_token_per_rank, cfg.num_experts_per_token
    row = cfg.hidden_dim * ELEM_BYTES[cfg.dispatch_dtype]
    crow = cfg.hidden_dim * 2
    srow = cfg.scale_dim * cfg.scale_type_size
    return W, M, k, row, crow, srow


def _dispatch_args(cfg: EpConfig, num_tokens: Sequence[int], x, indices, weights, scales, out_x,
                   out_indices, out_weights, out_scales, recv_num_token):
    """Checked ep_dispatch_args_t, and the ctypes array it points into."""
    W, M, k, row, _, srow = _sizes(cfg)
    xrow = cfg.hidden_dim * 2 if cfg.dispatch_cast else row
    WM = W * M
    if len(num_tokens) != W:
        raise ValueError(f"num_tokens has {len(num_tokens)} entries; world_size is {W}")
    nt = (ctypes.c_int32 * W)(*[int(v) for v in num_tokens])
    xt = _payload(cfg.dispatch_cast - 1) if cfg.dispatch_cast else _payload(cfg.dispatch_dtype)
    st = _scale_types(cfg.scale_type_size)
    a = EpDispatchArgs(
        ctypes.cast(nt, ctypes.c_void_p),
        _dev(x, "x", W * M * xrow, xt), _dev(indices, "indices", W * M * k * 4, _I32),
        _dev(weights, "weights", W * M * k * 4, _F32), _dev(scales, "scales", W * M * srow, st),
        _dev(out_x, "out_x", W * WM * row, _payload(cfg.dispatch_dtype)),
        _dev(out_indices, "out_indices", W * WM * k * 4, _I32),
        _dev(out_weights, "out_weights", W * WM * k * 4, _F32),
        _dev(out_scales, "out_scales", W * WM * srow, st),
        _dev(recv_num_token, "recv_num_token", W * 4, _I32))
    return a, nt


def wire_row_bytes(cfg: EpConfig):
    """(bytes of one combine input row, bytes of its scale row) for the
    config's combine wire."""
    H = cfg.hidden_dim
    if cfg.combine_wire == EP_WIRE_FP8_BLOCK128:
        return H, H // 128 * 4
    if cfg.combine_wire == EP_WIRE_MXFP4:
        return H // 2, H // 32
    return H * 2, 0


def wire_types(cfg: EpConfig):
    """(element types accepted for combine input rows, for their scales)."""
    if cfg.combine_wire == EP_WIRE_FP8_BLOCK128:
        return (torch.uint8, torch.float8_e4m3fn), (torch.float32, torch.uint8)
    if cfg.combine_wire == EP_WIRE_MXFP4:
        return (torch.uint8,), (torch.uint8,)
    return _payload(cfg.combine_dtype), None


def _combine_args(cfg: EpConfig, y, y_weights, out, out_weights, y_scales=None):
    W, M, k, _, crow, _ = _sizes(cfg)
    WM = W * M
    yrow, srow = wire_row_bytes(cfg)
    yt, yst = wire_types(cfg)
    return EpCombineArgs(_dev(y, "y", W * WM * yrow, yt),
                         _dev(y_weights, "y_weights", W * WM * k * 4, _F32),
                         _dev(out, "out", W * M * crow, _payload(cfg.combine_dtype)),
                         _dev(out_weights, "out_weights", W * M * k * 4, _F32),
                         _dev(y_scales, "y_scales", W * WM * srow, yst))


def ep_dispatch(plan: int, cfg: EpConfig, num_tokens: Sequence[int], x, indices, weights,
                scales, out_x, out_indices, out_weights, out_scales, recv_num_token,
                stream=None) -> None:
    """ep_dispatch(); tensors as in include/ep.h, sizes checked against cfg."""
    a, nt = _dispatch_args(cfg, num_tokens, x, indices, weights, scales, out_x, out_indices,
                           out_weights, out_scales, recv_num_token)
    _check("ep_dispatch", load().ep_dispatch(plan, ctypes.byref(a), _stream(stream)))


def ep_combine(plan: int, cfg: EpConfig, y, y_weights, out, out_weights, stream=None,
               y_scales=None) -> None:
    """ep_combine(); tensors as in include/ep.h, sizes checked against cfg."""
    a = _combine_args(cfg, y, y_weights, out, out_weights, y_scales)
    _check("ep_combine", load().ep_combine(plan, ctypes.byref(a), _stream(stream)))


def _same_tensors(held, given):
    """The very same tensor objects as before, still over the same memory,
    with the same size, element type and contiguity: a tensor changed in place
    (resize_, set_, a transpose_) misses and is checked again."""
    if len(held) != len(given):
        return False
    for h, g in zip(held, given):
        if h is None or g is None:
            if h is not g:
                return False
            continue
        ref, ptr, nbytes, dtype = h
        if (ref() is not g or g.data_ptr() != ptr or g.nbytes != nbytes or g.dtype != dtype
                or not g.is_contiguous()):
            return False
    return True


def _hold(tensors):
    """Weak references to the tensors a cached argument struct was built from,
    with their addresses, sizes and element types: the cache keeps none of the
    caller's tensors alive, and a tensor that is gone can only miss."""
    return tuple(None if t is None else (weakref.ref(t), t.data_ptr(), t.nbytes, t.dtype)
                 for t in tensors)


def ep_quantize_rows(rows: torch.Tensor, wire, out: torch.Tensor, scales: torch.Tensor,
                     stream=None, counts: Optional[torch.Tensor] = None) -> None:
    """ep_quantize_rows(): rows [..., H] bf16 / fp16 into the wire format
    (EP_WIRE_* or its name); out and scales sized as include/ep.h says.
    counts: an int32 device tensor of one count per leading index of rows
    ([G, R, H] rows with counts [G]); only the first counts[g] rows of group
    g are converted (recv_num_token for a combine's input)."""
    w = WIRES[wire] if wire is None or isinstance(wire, str) else wire
    H = rows.shape[-1]
    n = rows.numel() // H if H else 0
    dt = {torch.bfloat16: EP_BF16, torch.float16: EP_FP16}.get(rows.dtype)
    if dt is None:
        raise ValueError(f"rows must be bf16 or fp16, not {rows.dtype}")
    if w == EP_WIRE_FP8_BLOCK128:
        need_out, need_sc = n * H, n * (H // 128) * 4
    elif w == EP_WIRE_MXFP4:
        need_out, need_sc = n * H // 2, n * (H // 32)
    else:
        raise ValueError(f"wire must be fp8_block128 or mxfp4, not {wire!r}")
    cp, group = None, 0
    if counts is not None:
        if rows.dim() < 2 or rows.shape[0] == 0:
            raise ValueError("counts needs rows of shape [G, ..., H] with G >= 1")
        if counts.dtype != torch.int32:
            raise ValueError(f"counts must be int32, not {counts.dtype}")
        group = n // rows.shape[0]
        cp = _dev(counts, "counts", rows.shape[0] * 4)
    ot = (torch.uint8, torch.float8_e4m3fn) if w == EP_WIRE_FP8_BLOCK128 else (torch.uint8,)
    stt = (torch.float32, torch.uint8) if w == EP_WIRE_FP8_BLOCK128 else (torch.uint8,)
    _check("ep_quantize_rows", load().ep_quantize_rows(
        _dev(rows, "rows", n * H * 2), n, H, dt, w, _dev(out, "out", need_out, ot),
        _dev(scales, "scales", need_sc, stt), cp, group, _stream(stream, rows.device.index)))


def ep_probe_pattern(kind: int, row_bytes: int, rows: int, src=None, dst=None, map=None,
                     map_rows: int = 0, stride: int = 1, pieces: int = 1, waves: int = 8,
                     stream=None) -> None:
    """ep_probe_pattern() (include/ep_probe.h): one access-pattern probe
    launch, for measurement. src / dst are device tensors (or None), map a
    device int32 tensor or a device address (int), sizes checked here."""
    rb, n = int(row_bytes), int(rows)
    src_need = {EP_PROBE_READ: n * rb, EP_PROBE_COPY: n * rb, EP_PROBE_FANOUT: n * rb,
                EP_PROBE_GATHER: int(map_rows) * rb}.get(kind, 0)
    dst_need = {EP_PROBE_READ: n * pieces * 4, EP_PROBE_WRITE: n * rb, EP_PROBE_COPY: n * rb,
                EP_PROBE_FANOUT: int(map_rows) * rb, EP_PROBE_GATHER: n * rb}.get(kind, 0)
    mp = map if isinstance(map, int) or map is None else _dev(map, "map", n * stride * 4, _I32)
    a = EpProbeArgs(kind, rb, n, _dev(src, "src", src_need), _dev(dst, "dst", dst_need), mp,
                    int(map_rows), int(stride), int(pieces), int(waves))
    dev_index = (dst if dst is not None else src).device.index
    _check("ep_probe_pattern", load().ep_probe_pattern(ctypes.byref(a), _stream(stream, dev_index)))


def ep_probe_forward_map(plan: int):
    """(device address of the plan's forward map [W][M][stride] int32, stride)."""
    p = ctypes.c_void_p()
    st = ctypes.c_int32()
    _check("ep_probe_forward_map", load().ep_probe_forward_map(plan, ctypes.byref(p),
                                                                ctypes.byref(st)))
    return p.value, st.value


def ep_get_src_token_pos(plan: int, rank: int) -> int:
    """Device address of rank `rank`'s src_token_pos array (int32 [W*M])."""
    p = ctypes.c_void_p()
    _check("ep_get_src_token_pos", load().ep_get_src_token_pos(plan, rank, ctypes.byref(p)))
    return p.value


def ep_plan_set_launch(plan: int, launch: Optional[dict] = None) -> None:
    l = None if launch is None else ctypes.byref(EpLaunch(**{
        f: int(launch.get(f, 0)) for f, _ in EpLaunch._fields_}))
    _check("ep_plan_set_launch", load().ep_plan_set_launch(plan, l))


def ep_plan_get_launch(plan: int, num_tokens: Sequence[int]) -> dict:
    nt = (ctypes.c_int32 * len(num_tokens))(*[int(v) for v in num_tokens])
    out = EpLaunch()
    _check("ep_plan_get_launch", load().ep_plan_get_launch(
        plan, ctypes.cast(nt, ctypes.c_void_p), ctypes.byref(out)))
    return {f: getattr(out, f) for f, _ in EpLaunch._fields_}


def ep_plan_set_timing(plan: int, enable: bool) -> None:
    _check("ep_plan_set_timing", load().ep_plan_set_timing(plan, 1 if enable else 0))


def ep_plan_kernel_time(plan: int, kernel: int):
    """(launches timed, total milliseconds) of one EP_KERNEL_* kernel."""
    c = ctypes.c_int32()
    ms = ctypes.c_double()
    _check("ep_plan_kernel_time", load().ep_plan_kernel_time(
        plan, kernel, ctypes.byref(c), ctypes.byref(ms)))
    return c.value, ms.value


def ep_expert_workspace_bytes(plan: int, cap: int) -> int:
    n = load().ep_expert_workspace_bytes(plan, int(cap))
    if n == 0:
        raise EpError("ep_expert_workspace_bytes", EP_ERR_ARG, ep_last_error())
    return n


def ep_expert_plan_create(plan: int, cap: int, workspace: torch.Tensor) -> int:
    """Create an expert plan of capacity cap over a caller-owned workspace
    tensor (keep it alive, and the plan too, until ep_expert_plan_destroy)."""
    need = ep_expert_workspace_bytes(plan, cap)
    ws = _dev(workspace, "workspace", need)
    out = ctypes.c_void_p()
    _check("ep_expert_plan_create", load().ep_expert_plan_create(
        plan, int(cap), ws, workspace.numel() * workspace.element_size(), ctypes.byref(out)))
    return out.value


def ep_expert_plan_destroy(eplan: int) -> None:
    _check("ep_expert_plan_destroy", load().ep_expert_plan_destroy(eplan))


def _convert_dispatch_args(cfg: EpConfig, cap: int, x, indices, weights, scales,
                           recv_num_token, packed_x, packed_scales, packed_count,
                           packed_src_info, packed_layout_range):
    W, M, k, row, _, srow = _sizes(cfg)
    WM = W * M
    Er = cfg.num_experts_per_rank
    xt, st = _payload(cfg.dispatch_dtype), _scale_types(cfg.scale_type_size)
    return EpConvertDispatchArgs(
        _dev(x, "x", W * WM * row, xt), _dev(indices, "indices", W * WM * k * 4, _I32),
        _dev(weights, "weights", W * WM * k * 4, _F32),
        _dev(scales, "scales", W * WM * srow, st),
        _dev(recv_num_token, "recv_num_token", W * 4, _I32),
        _dev(packed_x, "packed_x", W * Er * cap * row, xt),
        _dev(packed_scales, "packed_scales", W * Er * cap * srow, st),
        _dev(packed_count, "packed_count", W * Er * 4, _I32),
        _dev(packed_src_info, "packed_src_info", W * Er * cap * 4, _I32),
        _dev(packed_layout_range, "packed_layout_range", W * Er * W * 8, (torch.int64,)))


def _convert_combine_args(cfg: EpConfig, cap: int, packed_y, y, apply_weights=False):
    W, M, _, _, crow, _ = _sizes(cfg)
    Er = cfg.num_experts_per_rank
    ct = _payload(cfg.combine_dtype)
    return EpConvertCombineArgs(_dev(packed_y, "packed_y", W * Er * cap * crow, ct),
                                _dev(y, "y", W * W * M * crow, ct), 1 if apply_weights else 0)


def ep_convert_dispatch_output(eplan: int, cfg: EpConfig, cap: int, x, indices, weights,
                               scales, recv_num_token, packed_x, packed_scales, packed_count,
                               packed_src_info, packed_layout_range, stream=None) -> None:
    """ep_convert_dispatch_output(); tensors as in include/ep.h."""
    a = _convert_dispatch_args(cfg, cap, x, indices, weights, scales, recv_num_token, packed_x,
                               packed_scales, packed_count, packed_src_info, packed_layout_range)
    _check("ep_convert_dispatch_output",
           load().ep_convert_dispatch_output(eplan, ctypes.byref(a), _stream(stream)))


def ep_convert_combine_input(eplan: int, cfg: EpConfig, cap: int, packed_y, y,
                             apply_weights=False, stream=None) -> None:
    """ep_convert_combine_input(); tensors as in include/ep.h."""
    a = _convert_combine_args(cfg, cap, packed_y, y, apply_weights)
    _check("ep_convert_combine_input",
           load().ep_convert_combine_input(eplan, ctypes.byref(a), _stream(stream)))


def _dispatch_standard_args(cfg: EpConfig, cap: int, num_tokens: Sequence[int], x, indices,
                            scales, packed_x, packed_scales, packed_count, packed_src_info,
                            packed_layout_range):
    W, M, k, row, _, srow = _sizes(cfg)
    xrow = cfg.hidden_dim * 2 if cfg.dispatch_cast else row
    Er = cfg.num_experts_per_rank
    if len(num_tokens) != W:
        raise ValueError(f"num_tokens has {len(num_tokens)} entries; world_size is {W}")
    arr = (ctypes.c_int32 * W)(*[int(t) for t in num_tokens])
    xt = _payload(cfg.dispatch_cast - 1) if cfg.dispatch_cast else _payload(cfg.dispatch_dtype)
    st = _scale_types(cfg.scale_type_size)
    a = EpDispatchStandardArgs(
        ctypes.addressof(arr), _dev(x, "x", W * M * xrow, xt),
        _dev(indices, "indices", W * M * k * 4, _I32), _dev(scales, "scales", W * M * srow, st),
        _dev(packed_x, "packed_x", W * Er * cap * row, _payload(cfg.dispatch_dtype)),
        _dev(packed_scales, "packed_scales", W * Er * cap * srow, st),
        _dev(packed_count, "packed_count", W * Er * 4, _I32),
        _dev(packed_src_info, "packed_src_info", W * Er * cap * 4, _I32),
        _dev(packed_layout_range, "packed_layout_range", W * Er * W * 8, (torch.int64,)))
    return a, arr


def _combine_standard_args(cfg: EpConfig, cap: int, packed_y, indices, weights, out,
                           packed_y_scales=None):
    W, M, k, _, crow, _ = _sizes(cfg)
    Er = cfg.num_experts_per_rank
    yrow, srow = wire_row_bytes(cfg) if cfg.combine_wire else (crow, 0)
    yt, yst = wire_types(cfg)
    return EpCombineStandardArgs(
        _dev(packed_y, "packed_y", W * Er * cap * yrow, yt),
        _dev(indices, "indices", W * M * k * 4, _I32),
        _dev(weights, "weights", W * M * k * 4, _F32),
        _dev(out, "out", W * M * crow, _payload(cfg.combine_dtype)),
        _dev(packed_y_scales, "packed_y_scales", W * Er * cap * srow, yst))


def ep_dispatch_standard_moe(eplan: int, cfg: EpConfig, cap: int, num_tokens, x, indices, scales,
                             packed_x, packed_scales, packed_count, packed_src_info,
                             packed_layout_range, stream=None) -> None:
    """ep_dispatch_standard_moe(); tensors as in include/ep.h."""
    a, arr = _dispatch_standard_args(cfg, cap, num_tokens, x, indices, scales, packed_x,
                                     packed_scales, packed_count, packed_src_info,
                                     packed_layout_range)
    _check("ep_dispatch_standard_moe",
           load().ep_dispatch_standard_moe(eplan, ctypes.byref(a), _stream(stream)))


def ep_combine_standard_moe(eplan: int, cfg: EpConfig, cap: int, packed_y, indices, weights, out,
                            stream=None, packed_y_scales=None) -> None:
    """ep_combine_standard_moe(); tensors as in include/ep.h."""
    a = _combine_standard_args(cfg, cap, packed_y, indices, weights, out, packed_y_scales)
    _check("ep_combine_standard_moe",
           load().ep_combine_standard_moe(eplan, ctypes.byref(a), _stream(stream)))


_TORCH = {EP_BF16: torch.bfloat16, EP_FP16: torch.float16, EP_FP8_E4M3: torch.float8_e4m3fn}


class EpDispatchCombineOp:
    """One plan with its workspace and output buffers, allocated once with
    torch on the current device and reused by every call, in the manner of the
    pages' EpDispatchCombineOp ("MORI-EP User Guide", section 3). dispatch()
    and combine() return views of those buffers, valid until the next
    dispatch ("MORI (ROCm/mori) — L2 Distillation", section 9)."""

    def __init__(self, cfg: EpConfig, device=None, with_weights=True, expert_capacity=None):
        self.cfg = cfg
        # rows kept per local expert by convert_dispatch_output (W * M: none
        # dropped); its buffers are allocated on first use
        self.expert_capacity = (cfg.world_size * cfg.max_num_inp_token_per_rank
                                if expert_capacity is None else int(expert_capacity))
        self._ex = None
        dev = torch.device("cuda") if device is None else torch.device(device)
        W, M, k, _, _, srow = _sizes(cfg)
        WM = W * M
        H = cfg.hidden_dim
        self.workspace = torch.empty(ep_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
        self.out_x = torch.empty((W, WM, H), dtype=_TORCH[cfg.dispatch_dtype], device=dev)
        self.out_indices = torch.empty((W, WM, k), dtype=torch.int32, device=dev)
        self.out_weights = (torch.empty((W, WM, k), dtype=torch.float32, device=dev)
                            if with_weights else None)
        self.out_scales = (torch.empty((W, WM, srow), dtype=torch.uint8, device=dev)
                           if cfg.scale_dim else None)
        self.recv_num_token = torch.empty((W,), dtype=torch.int32, device=dev)
        self.combine_out = torch.empty((W, M, H), dtype=_TORCH[cfg.combine_dtype], device=dev)
        self.combine_weights = (torch.empty((W, M, k), dtype=torch.float32, device=dev)
                                if with_weights else None)
        self.plan = ep_plan_create(cfg, self.workspace)
        self._src_pos_off = [ep_get_src_token_pos(self.plan, r) - self.workspace.data_ptr()
                             for r in range(W)]
        # Checked argument structs of the last call, reused while the same
        # tensor objects (over the same memory, same size and type) and token
        # counts come back: the per-tensor checks cost more host time than a
        # small call's GPU work. The cache holds weak references only, so it
        # keeps none of the caller's tensors alive; a tensor that is gone, or
        # changed in place, misses and is checked again.
        self._dcache = None
        self._ccache = None
        self._lib = load()
        self._dev_index = dev.index if dev.index is not None else torch.cuda.current_device()

    def dispatch(self, num_tokens, x, indices, weights=None, scales=None, stream=None):
        given = (x, indices, weights, scales)
        nt = tuple(num_tokens)
        c = self._dcache
        if c is None or c[1] != nt or not _same_tensors(c[0], given):
            a, arr = _dispatch_args(self.cfg, nt, x, indices, weights, scales, self.out_x,
                                    self.out_indices,
                                    self.out_weights if weights is not None else None,
                                    self.out_scales if scales is not None else None,
                                    self.recv_num_token)
            c = self._dcache = (_hold(given), nt, a, arr)
        _check("ep_dispatch", self._lib.ep_dispatch(self.plan, ctypes.byref(c[2]),
                                                    _stream(stream, self._dev_index)))
        return (self.out_x, self.out_weights, self.out_scales, self.out_indices,
                self.recv_num_token)

    def combine(self, y, y_weights=None, stream=None, y_scales=None):
        """With a combine wire in the config, y holds wire rows and y_scales
        their scales (ep_quantize_rows writes both)."""
        given = (y, y_weights, y_scales)
        c = self._ccache
        if c is None or not _same_tensors(c[0], given):
            a = _combine_args(self.cfg, y, y_weights, self.combine_out,
                              self.combine_weights if y_weights is not None else None, y_scales)
            c = self._ccache = (_hold(given), a)
        _check("ep_combine", self._lib.ep_combine(self.plan, ctypes.byref(c[1]),
                                                  _stream(stream, self._dev_index)))
        return self.combine_out, (self.combine_weights if y_weights is not None else None)

    def src_token_pos(self, rank: int) -> torch.Tensor:
        """int32 [W*M] view of rank's reverse map inside the workspace."""
        WM = self.cfg.world_size * self.cfg.max_num_inp_token_per_rank
        off = self._src_pos_off[rank]
        return self.workspace[off: off + 4 * WM].view(torch.int32)

    def set_launch(self, launch: Optional[dict] = None):
        ep_plan_set_launch(self.plan, launch)

    def _expert_state(self):
        if self._ex is None:
            cfg, cap = self.cfg, self.expert_capacity
            W, M, _, _, _, srow = _sizes(cfg)
            Er, H = cfg.num_experts_per_rank, cfg.hidden_dim
            dev = self.workspace.device
            ws = torch.empty(ep_expert_workspace_bytes(self.plan, cap), dtype=torch.uint8,
                             device=dev)
            ex = dict(
                workspace=ws,
                packed_x=torch.empty((W, Er, cap, H), dtype=_TORCH[cfg.dispatch_dtype],
                                     device=dev),
                packed_scales=(torch.empty((W, Er, cap, srow), dtype=torch.uint8, device=dev)
                               if cfg.scale_dim else None),
                packed_count=torch.empty((W, Er), dtype=torch.int32, device=dev),
                packed_src_info=torch.empty((W, Er, cap), dtype=torch.int32, device=dev),
                packed_layout_range=torch.empty((W, Er, W), dtype=torch.int64, device=dev),
                y=torch.empty((W, W * M, H), dtype=_TORCH[cfg.combine_dtype], device=dev),
                cache=None)
            ex["plan"] = ep_expert_plan_create(self.plan, cap, ws)
            self._ex = ex
        return self._ex

    def convert_dispatch_output(self, dispatch_out_x, dispatch_out_topk_idx,
                                dispatch_out_scales=None, dispatch_out_weights=None,
                                stream=None):
        """The last dispatch's received rows regrouped by local expert ("MORI-EP
        User Guide", section 4, convert_dispatch_output). Returns
        (packed_recv_x, packed_recv_count, packed_recv_src_info,
        packed_recv_layout_range); packed_recv_x is (rows, scale rows) when
        the config has scales. Views of buffers the next call overwrites.
        With dispatch_out_weights, each kept pair records its expert's weight
        for a weighted convert_combine_input."""
        ex = self._expert_state()
        given = (dispatch_out_x, dispatch_out_topk_idx, dispatch_out_scales,
                 dispatch_out_weights)
        c = ex["cache"]
        if c is None or not _same_tensors(c[0], given):
            a = _convert_dispatch_args(self.cfg, self.expert_capacity, dispatch_out_x,
                                       dispatch_out_topk_idx, dispatch_out_weights,
                                       dispatch_out_scales,
                                       self.recv_num_token, ex["packed_x"], ex["packed_scales"],
                                       ex["packed_count"], ex["packed_src_info"],
                                       ex["packed_layout_range"])
            c = ex["cache"] = (_hold(given), a)
        _check("ep_convert_dispatch_output", self._lib.ep_convert_dispatch_output(
            ex["plan"], ctypes.byref(c[1]), _stream(stream, self._dev_index)))
        px = ex["packed_x"] if ex["packed_scales"] is None else (ex["packed_x"],
                                                                  ex["packed_scales"])
        return px, ex["packed_count"], ex["packed_src_info"], ex["packed_layout_range"]

    def convert_combine_input(self, packed_recv_y, packed_recv_src_info=None,
                              packed_recv_layout_range=None, apply_weights=False, stream=None):
        """One combine input row per received row from the experts' outputs
        ("MORI-EP User Guide", section 4, convert_combine_input). The
        positions come from this op's last convert_dispatch_output;
        packed_recv_src_info / packed_recv_layout_range, if given, must be the
        tensors it returned. apply_weights scales each output by its expert's
        routing weight (the conversion must have had weights). Returns y
        [W, W*M, H] for combine()."""
        ex = self._ex
        if ex is None:
            raise EpError("ep_convert_combine_input", EP_ERR_STATE,
                          "convert_combine_input before any convert_dispatch_output")
        for t, key, name in ((packed_recv_src_info, "packed_src_info", "packed_recv_src_info"),
                             (packed_recv_layout_range, "packed_layout_range",
                              "packed_recv_layout_range")):
            if t is not None and t is not ex[key]:
                raise ValueError(f"{name} must be the tensor convert_dispatch_output returned")
        a = _convert_combine_args(self.cfg, self.expert_capacity, packed_recv_y, ex["y"],
                                  apply_weights)
        _check("ep_convert_combine_input", self._lib.ep_convert_combine_input(
            ex["plan"], ctypes.byref(a), _stream(stream, self._dev_index)))
        return ex["y"]

    def dispatch_standard_moe(self, input, weights, scales, indices, num_tokens=None,
                              stream=None):
        """Dispatch straight into the expert-major layout ("MORI-EP User
        Guide", section 4, dispatch_standard_moe): the same four results as
        dispatch() followed by convert_dispatch_output(), without the 2-D
        receive buffer. input [W, M, H] and indices [W, M, k] hold every
        rank's tokens; num_tokens (default: M each) the tokens T_r of each
        rank. weights is taken for the pages' argument order and is not part
        of the layout: give it to combine_standard_moe to apply it."""
        if weights is not None and (weights.dtype != torch.float32 or
                                    tuple(weights.shape[-1:]) != (self.cfg.num_experts_per_token,)):
            raise ValueError("weights must be float32 [W, M, k] or None")
        ex = self._expert_state()
        W, M = self.cfg.world_size, self.cfg.max_num_inp_token_per_rank
        nt = tuple([M] * W if num_tokens is None else num_tokens)
        given = (input, indices, scales)
        c = ex.get("scache")
        if c is None or c[1] != nt or not _same_tensors(c[0], given):
            a, arr = _dispatch_standard_args(self.cfg, self.expert_capacity, nt, input, indices,
                                             scales, ex["packed_x"], ex["packed_scales"],
                                             ex["packed_count"], ex["packed_src_info"],
                                             ex["packed_layout_range"])
            c = ex["scache"] = (_hold(given), nt, a, arr)
        _check("ep_dispatch_standard_moe", self._lib.ep_dispatch_standard_moe(
            ex["plan"], ctypes.byref(c[2]), _stream(stream, self._dev_index)))
        ex["ccache"] = None
        px = ex["packed_x"] if ex["packed_scales"] is None else (ex["packed_x"],
                                                                  ex["packed_scales"])
        return px, ex["packed_count"], ex["packed_src_info"], ex["packed_layout_range"]

    def combine_standard_moe(self, input, weights, indices, call_reset=False, stream=None,
                             input_scales=None):
        """Combine straight from the expert-major layout ("MORI-EP User Guide",
        section 4, combine_standard_moe): input [W, Er, cap, H] holds the
        experts' outputs for the last dispatch_standard_moe, indices its ids;
        weights [W, M, k] (or None for the plain sum) are applied as
        convert_combine_input(apply_weights=True) would. The result equals
        convert_combine_input() followed by combine(). call_reset is taken
        for the pages' signature: nothing needs resetting. With a combine
        wire in the config, input holds wire rows and input_scales their
        scales (ep_quantize_rows writes both, with counts=packed_count).
        Returns [W, M, H] (rows t < T_r written), a view of the op's combine
        output buffer."""
        ex = self._ex
        if ex is None:
            raise EpError("ep_combine_standard_moe", EP_ERR_STATE,
                          "combine_standard_moe before any dispatch_standard_moe")
        given = (input, weights, indices, input_scales)
        c = ex.get("ccache")
        if c is None or not _same_tensors(c[0], given):
            a = _combine_standard_args(self.cfg, self.expert_capacity, input, indices, weights,
                                       self.combine_out, input_scales)
            c = ex["ccache"] = (_hold(given), a)
        _check("ep_combine_standard_moe", self._lib.ep_combine_standard_moe(
            ex["plan"], ctypes.byref(c[1]), _stream(stream, self._dev_index)))
        return self.combine_out

    def close(self):
        self._dcache = self._ccache = None
        if self._ex is not None:
            ex, self._ex = self._ex, None
            ep_expert_plan_destroy(ex["plan"])
        if self.plan:
            ep_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
