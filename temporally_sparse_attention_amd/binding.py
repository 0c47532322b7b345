"""ctypes binding of liblite_attn.so (the C ABI in include/lite_attn.h).

Argument marshalling only: tensors are passed as device pointers together with torch's
current HIP stream; every step of the computation runs in the library's kernels. Importing
this module fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblite_attn.so")

ABI_VERSION = 2
OPT_IN_STEP_SKIP = 1
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_NO_MEMORY = range(5)
DTYPES = {"bf16": 0, "fp32": 1}
ORDERS = {"asc": 0, "alt": 1}

#: Every function the C header declares (checked against include/lite_attn.h by the tests).
EXPORTS = (
    "lite_attn_create",
    "lite_attn_destroy",
    "lite_attn_mask_bytes",
    "lite_attn_mask_geometry",
    "lite_attn_step",
    "lite_attn_step_refresh",
    "lite_attn_workspace_bytes",
    "lite_attn_step_scheduled",
    "lite_attn_step_scheduled_static",
    "lite_attn_reset_mask",
    "lite_attn_mask_popcount",
    "lite_attn_output_max_abs_diff",
    "lite_attn_calibrate_workspace_bytes",
    "lite_attn_calibrate",
    "lite_attn_status_string",
    "lite_attn_last_error",
    "lite_attn_last_launch",
)


class LiteAttnConfig(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("tile_q", ctypes.c_int32),
        ("tile_k", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("order", ctypes.c_int32),
        ("dense_prefix", ctypes.c_int32),
        ("stride_b", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
        ("stride_n", ctypes.c_int64),
        ("options", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


class LiteAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def _hip_runtimes_mapped():
    """Paths of every libamdhip64 mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                parts = line.split()
                if parts and "libamdhip64" in parts[-1]:
                    paths.add(os.path.realpath(parts[-1]))
    except OSError:
        pass
    return sorted(paths)


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m temporally_sparse_attention_amd.build)")
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7) but loads it by
    # another file name. Loading torch first makes this library bind to that runtime instead of
    # bringing a second HIP/HSA runtime into the process (a second runtime sees no device).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded in this process (%s); load torch before "
                          "any other HIP library" % ", ".join(runtimes))
    vp, u32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32)
    lib.lite_attn_create.argtypes = [ctypes.POINTER(LiteAttnConfig), ctypes.POINTER(vp)]
    lib.lite_attn_create.restype = ctypes.c_int
    lib.lite_attn_destroy.argtypes = [vp]
    lib.lite_attn_destroy.restype = ctypes.c_int
    lib.lite_attn_mask_bytes.argtypes = [vp]
    lib.lite_attn_mask_bytes.restype = ctypes.c_size_t
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.lite_attn_mask_geometry.argtypes = [vp, i32p, i32p, i32p]
    lib.lite_attn_mask_geometry.restype = ctypes.c_int
    lib.lite_attn_step.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_int32, vp]
    lib.lite_attn_step.restype = ctypes.c_int
    lib.lite_attn_step_refresh.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                           ctypes.c_float, ctypes.c_int32, vp]
    lib.lite_attn_step_refresh.restype = ctypes.c_int
    lib.lite_attn_workspace_bytes.argtypes = [vp]
    lib.lite_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.lite_attn_step_scheduled.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_int32,
                                             vp, vp]
    lib.lite_attn_step_scheduled.restype = ctypes.c_int
    lib.lite_attn_step_scheduled_static.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                                    ctypes.c_int32, vp]
    lib.lite_attn_step_scheduled_static.restype = ctypes.c_int
    lib.lite_attn_reset_mask.argtypes = [vp, vp, vp]
    lib.lite_attn_reset_mask.restype = ctypes.c_int
    lib.lite_attn_mask_popcount.argtypes = [vp, vp, vp, vp]
    lib.lite_attn_mask_popcount.restype = ctypes.c_int
    lib.lite_attn_output_max_abs_diff.argtypes = [vp, vp, vp, vp, vp]
    lib.lite_attn_output_max_abs_diff.restype = ctypes.c_int
    lib.lite_attn_calibrate_workspace_bytes.argtypes = [vp]
    lib.lite_attn_calibrate_workspace_bytes.restype = ctypes.c_size_t
    f32p = ctypes.POINTER(ctypes.c_float)
    vpp = ctypes.POINTER(vp)
    lib.lite_attn_calibrate.argtypes = [vp, vpp, vpp, vpp, ctypes.c_int32, f32p, f32p,
                                        ctypes.c_int32, f32p, f32p, vp, vp]
    lib.lite_attn_calibrate.restype = ctypes.c_int
    lib.lite_attn_status_string.argtypes = [ctypes.c_int]
    lib.lite_attn_status_string.restype = ctypes.c_char_p
    lib.lite_attn_last_error.argtypes = []
    lib.lite_attn_last_error.restype = ctypes.c_char_p
    lib.lite_attn_last_launch.argtypes = [i32p, i32p]
    lib.lite_attn_last_launch.restype = ctypes.c_int
    del u32p
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def lite_attn_status_string(status: int) -> str:
    return _lib.lite_attn_status_string(int(status)).decode()


def lite_attn_last_error() -> str:
    return _lib.lite_attn_last_error().decode()


def lite_attn_last_launch() -> Tuple[int, int]:
    """(workgroups, queue) of the calling thread's most recent step launch; queue -1: one
    workgroup per query tile, no tile queue."""
    wg, qu = ctypes.c_int32(), ctypes.c_int32()
    _lib.lite_attn_last_launch(ctypes.byref(wg), ctypes.byref(qu))
    return wg.value, qu.value


def _check(status: int, what: str):
    if status != OK:
        raise LiteAttnError(status, f"{what}: {lite_attn_status_string(status)}: "
                                    f"{lite_attn_last_error()}")


class Handle:
    """Owns a lite_attn_t; keeps the validated configuration for marshalling checks."""

    def __init__(self, ptr: int, cfg: LiteAttnConfig):
        self.ptr = ctypes.c_void_p(ptr)
        self.cfg = cfg
        tq, tk, w = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.lite_attn_mask_geometry(self.ptr, ctypes.byref(tq), ctypes.byref(tk),
                                            ctypes.byref(w)), "lite_attn_mask_geometry")
        self.tiles_q, self.tiles_k, self.words_per_row = tq.value, tk.value, w.value

    @property
    def mask_shape(self) -> Tuple[int, int, int, int]:
        c = self.cfg
        return (c.batch, c.heads, self.tiles_q, self.words_per_row)

    def close(self):
        if self.ptr is not None and self.ptr.value:
            _lib.lite_attn_destroy(self.ptr)
        self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def make_config(batch: int, heads: int, seq_len: int, head_dim: int, *, tile_q: int = 128,
                tile_k: int = 64, dtype: str = "bf16", softmax_scale: float = 0.0,
                order: str = "alt", dense_prefix: int = 0,
                strides: Tuple[int, int, int] = (0, 0, 0),
                in_step_skip: bool = False) -> LiteAttnConfig:
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {list(DTYPES)}")
    if order not in ORDERS:
        raise ValueError(f"order must be one of {list(ORDERS)}")
    return LiteAttnConfig(ABI_VERSION, batch, heads, seq_len, head_dim, tile_q, tile_k,
                          DTYPES[dtype], float(softmax_scale), ORDERS[order], dense_prefix,
                          int(strides[0]), int(strides[1]), int(strides[2]),
                          OPT_IN_STEP_SKIP if in_step_skip else 0, 0)


def lite_attn_create(batch: int, heads: int, seq_len: int, head_dim: int, **kw) -> Handle:
    cfg = kw.pop("config", None) or make_config(batch, heads, seq_len, head_dim, **kw)
    out = ctypes.c_void_p()
    _check(_lib.lite_attn_create(ctypes.byref(cfg), ctypes.byref(out)), "lite_attn_create")
    return Handle(out.value, cfg)


def lite_attn_destroy(handle: Handle):
    handle.close()


def lite_attn_mask_bytes(handle: Handle) -> int:
    return int(_lib.lite_attn_mask_bytes(handle.ptr))


def lite_attn_mask_geometry(handle: Handle) -> Tuple[int, int, int]:
    return handle.tiles_q, handle.tiles_k, handle.words_per_row


# ---------------------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_ptr(stream, device) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _ptr(t, name: str, device=None) -> int:
    torch = _torch()
    if isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor or a device pointer")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return int(t.data_ptr())


def _check_qkvo(handle: Handle, t, name: str):
    torch = _torch()
    if isinstance(t, int):
        return
    c = handle.cfg
    want = torch.bfloat16 if c.dtype == DTYPES["bf16"] else torch.float32
    if t.dtype != want:
        raise TypeError(f"{name} has dtype {t.dtype}, the handle expects {want}")
    if tuple(t.shape) != (c.batch, c.heads, c.seq_len, c.head_dim):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected "
                         f"{(c.batch, c.heads, c.seq_len, c.head_dim)}")
    if t.numel() == 0:
        return
    if c.stride_b == 0 and c.stride_h == 0 and c.stride_n == 0:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous for a handle with default strides")
    else:
        st = t.stride()
        if (st[3] != 1 or (c.batch > 1 and st[0] != c.stride_b) or
                (c.heads > 1 and st[1] != c.stride_h) or (c.seq_len > 1 and st[2] != c.stride_n)):
            raise ValueError(f"{name} strides {st} differ from the handle's "
                             f"({c.stride_b}, {c.stride_h}, {c.stride_n}, 1)")


def _check_mask(handle: Handle, mask):
    torch = _torch()
    if isinstance(mask, int):
        return
    if mask.dtype not in (torch.int32, torch.uint32):
        raise TypeError("mask must be an int32 or uint32 tensor")
    if not mask.is_contiguous() or mask.numel() * 4 < lite_attn_mask_bytes(handle):
        raise ValueError(f"mask must be a contiguous tensor of shape {handle.mask_shape}")


def lite_attn_step(handle: Handle, q, k, v, out, mask, log_eps_t: float, step: int,
                   stream=None):
    """Enqueue one denoising step on `stream` (default: torch's current stream)."""
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _check_qkvo(handle, t, name)
    _check_mask(handle, mask)
    dev = None if isinstance(q, int) else q.device
    st = _stream_ptr(stream, dev)
    _check(_lib.lite_attn_step(handle.ptr, _ptr(q, "q", dev), _ptr(k, "k", dev),
                               _ptr(v, "v", dev), _ptr(out, "out", dev), _ptr(mask, "mask", dev),
                               ctypes.c_float(log_eps_t), ctypes.c_int32(step),
                               ctypes.c_void_p(st)),
           "lite_attn_step")


def lite_attn_step_refresh(handle: Handle, q, k, v, out, mask, tile_stats, refresh_delta: float,
                           log_eps_t: float, step: int, stream=None):
    """lite_attn_step with divergence-triggered refresh; `tile_stats` is a float32 device tensor
    of B*H*Tq references (NaN: none yet)."""
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _check_qkvo(handle, t, name)
    _check_mask(handle, mask)
    torch = _torch()
    if isinstance(tile_stats, torch.Tensor):
        c = handle.cfg
        if (tile_stats.dtype != torch.float32 or not tile_stats.is_contiguous() or
                tile_stats.numel() < c.batch * c.heads * handle.tiles_q):
            raise ValueError("tile_stats must be a contiguous float32 tensor of B*H*Tq elements")
    dev = None if isinstance(q, int) else q.device
    st = _stream_ptr(stream, dev)
    _check(_lib.lite_attn_step_refresh(handle.ptr, _ptr(q, "q", dev), _ptr(k, "k", dev),
                                       _ptr(v, "v", dev), _ptr(out, "out", dev),
                                       _ptr(mask, "mask", dev), _ptr(tile_stats, "tile_stats", dev),
                                       ctypes.c_float(refresh_delta), ctypes.c_float(log_eps_t),
                                       ctypes.c_int32(step), ctypes.c_void_p(st)),
           "lite_attn_step_refresh")


def lite_attn_workspace_bytes(handle: Handle) -> int:
    return int(_lib.lite_attn_workspace_bytes(handle.ptr))


def lite_attn_step_scheduled(handle: Handle, q, k, v, out, mask, log_eps_t: float, step: int,
                             workspace, stream=None):
    """lite_attn_step with a visit-count schedule (heavy tiles first, short last); `workspace` is a device tensor of at least
    lite_attn_workspace_bytes(handle) bytes, 256-byte aligned."""
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _check_qkvo(handle, t, name)
    _check_mask(handle, mask)
    torch = _torch()
    if isinstance(workspace, torch.Tensor):
        if (not workspace.is_contiguous() or
                workspace.numel() * workspace.element_size() < lite_attn_workspace_bytes(handle)):
            raise ValueError("workspace must be a contiguous tensor of at least "
                             f"{lite_attn_workspace_bytes(handle)} bytes")
    dev = None if isinstance(q, int) else q.device
    st = _stream_ptr(stream, dev)
    _check(_lib.lite_attn_step_scheduled(handle.ptr, _ptr(q, "q", dev), _ptr(k, "k", dev),
                                         _ptr(v, "v", dev), _ptr(out, "out", dev),
                                         _ptr(mask, "mask", dev), ctypes.c_float(log_eps_t),
                                         ctypes.c_int32(step), _ptr(workspace, "workspace", dev),
                                         ctypes.c_void_p(st)),
           "lite_attn_step_scheduled")


def lite_attn_step_scheduled_static(handle: Handle, q, k, v, out, mask, log_eps_t: float,
                                    step: int, stream=None):
    """lite_attn_step_scheduled with the library's static workspace (allocates nothing)."""
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _check_qkvo(handle, t, name)
    _check_mask(handle, mask)
    dev = None if isinstance(q, int) else q.device
    st = _stream_ptr(stream, dev)
    _check(_lib.lite_attn_step_scheduled_static(handle.ptr, _ptr(q, "q", dev), _ptr(k, "k", dev),
                                                _ptr(v, "v", dev), _ptr(out, "out", dev),
                                                _ptr(mask, "mask", dev), ctypes.c_float(log_eps_t),
                                                ctypes.c_int32(step), ctypes.c_void_p(st)),
           "lite_attn_step_scheduled_static")


def lite_attn_reset_mask(handle: Handle, mask, stream=None):
    _check_mask(handle, mask)
    dev = None if isinstance(mask, int) else mask.device
    _check(_lib.lite_attn_reset_mask(handle.ptr, _ptr(mask, "mask", dev),
                                     ctypes.c_void_p(_stream_ptr(stream, dev))),
           "lite_attn_reset_mask")


def lite_attn_mask_popcount(handle: Handle, mask, counts, stream=None):
    _check_mask(handle, mask)
    torch = _torch()
    if isinstance(counts, torch.Tensor):
        c = handle.cfg
        if counts.dtype not in (torch.int32, torch.uint32) or counts.numel() < c.batch * c.heads:
            raise ValueError("counts must be an int32/uint32 tensor with B*H elements")
    dev = None if isinstance(mask, int) else mask.device
    _check(_lib.lite_attn_mask_popcount(handle.ptr, _ptr(mask, "mask", dev),
                                        _ptr(counts, "counts", dev),
                                        ctypes.c_void_p(_stream_ptr(stream, dev))),
           "lite_attn_mask_popcount")


def lite_attn_output_max_abs_diff(handle: Handle, a, b, result, stream=None):
    """Enqueue result[0] = max |a - b| over the valid elements (float32 device tensor)."""
    for t, name in ((a, "a"), (b, "b")):
        _check_qkvo(handle, t, name)
    torch = _torch()
    if isinstance(result, torch.Tensor) and (result.dtype != torch.float32 or
                                             result.numel() < 1):
        raise ValueError("result must be a float32 tensor with at least one element")
    dev = None if isinstance(a, int) else a.device
    _check(_lib.lite_attn_output_max_abs_diff(handle.ptr, _ptr(a, "a", dev), _ptr(b, "b", dev),
                                              _ptr(result, "result", dev),
                                              ctypes.c_void_p(_stream_ptr(stream, dev))),
           "lite_attn_output_max_abs_diff")


def lite_attn_calibrate_workspace_bytes(handle: Handle) -> int:
    return int(_lib.lite_attn_calibrate_workspace_bytes(handle.ptr))


def lite_attn_calibrate(handle: Handle, qs, ks, vs, error_budgets, candidates, workspace,
                        stream=None):
    """Per-step budgets from per-step output-error limits; blocks until done. qs, ks, vs: one
    device tensor (or pointer) per step. Returns (log_eps, errors) as lists of floats."""
    steps = len(error_budgets)
    if not (len(qs) == len(ks) == len(vs) == steps):
        raise ValueError("one q, k, v and error budget per step is needed")
    for seq, name in ((qs, "q"), (ks, "k"), (vs, "v")):
        for t in seq:
            _check_qkvo(handle, t, name)
    torch = _torch()
    need = lite_attn_calibrate_workspace_bytes(handle)
    if isinstance(workspace, torch.Tensor):
        if (not workspace.is_contiguous() or
                workspace.numel() * workspace.element_size() < need):
            raise ValueError(f"workspace must be a contiguous tensor of at least {need} bytes")
    first = qs[0] if steps else None
    dev = None if (first is None or isinstance(first, int)) else first.device
    arr = ctypes.c_void_p * max(1, steps)
    qa = arr(*[_ptr(t, "q", dev) for t in qs])
    ka = arr(*[_ptr(t, "k", dev) for t in ks])
    va = arr(*[_ptr(t, "v", dev) for t in vs])
    fl = ctypes.c_float * max(1, steps)
    budgets = fl(*[float(x) for x in error_budgets])
    cands = (ctypes.c_float * max(1, len(candidates)))(*[float(x) for x in candidates])
    log_eps, errors = fl(), fl()
    ws = 0 if workspace is None else _ptr(workspace, "workspace", dev)
    _check(_lib.lite_attn_calibrate(handle.ptr, qa, ka, va, ctypes.c_int32(steps), budgets,
                                    cands, ctypes.c_int32(len(candidates)), log_eps, errors,
                                    ctypes.c_void_p(ws),
                                    ctypes.c_void_p(_stream_ptr(stream, dev) if steps else 0)),
           "lite_attn_calibrate")
    return [float(log_eps[t]) for t in range(steps)], [float(errors[t]) for t in range(steps)]
