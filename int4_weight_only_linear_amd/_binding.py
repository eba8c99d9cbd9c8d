"""ctypes binding of libw4a16 (include/w4a16.h).

Argument marshalling only: shapes, dtypes and pointers are read off torch
tensors (device memory) or numpy arrays (host memory) and handed to the C
entry points of the same names; every step of the computation runs in the
library.  There is no fallback: if libw4a16.so is missing or fails to load,
importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")

W4A16_OK = 0
W4A16_F16 = 0
W4A16_BF16 = 1
PATH_AUTO, PATH_GEMV, PATH_GEMM = 0, 1, 2
GEMV_MAX_M = 16
ABI_VERSION = 4

STATUS_NAMES = {
    0: "W4A16_OK", 1: "W4A16_ERR_INVALID_ARG", 2: "W4A16_ERR_UNSUPPORTED",
    3: "W4A16_ERR_ALIGNMENT", 4: "W4A16_ERR_DEVICE", 5: "W4A16_ERR_LAUNCH",
    6: "W4A16_ERR_WORKSPACE",
}

# the exported symbols of include/w4a16.h: name -> (restype, argtypes)
_c_int, _c_i32, _c_i64, _c_sz, _vp = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = {
    "w4a16_abi_version": (_c_int, []),
    "w4a16_reload_tuning": (None, []),
    "w4a16_last_error": (ctypes.c_char_p, []),
    "w4a16_pack_weights": (_c_int, [_vp, _c_i64, _c_i64, _vp]),
    "w4a16_unpack_weights": (_c_int, [_vp, _c_i64, _c_i64, _vp]),
    "w4a16_pack_zeros": (_c_int, [_vp, _c_i64, _c_i64, _vp]),
    "w4a16_unpack_zeros": (_c_int, [_vp, _c_i64, _c_i64, _vp]),
    "w4a16_check_args": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32]),
    "w4a16_select_path": (_c_int, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32]),
    "w4a16_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32]),
    "w4a16_linear": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32,
                              _vp, _c_sz, _vp]),
    "w4a16_linear_path": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i32,
                                   _c_i32, _vp, _c_sz, _vp, _c_i32]),
    "w4a16_linear_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i32,
                                      _c_i32, _vp]),
    "w4a16_dequant": (_c_int, [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i32, _c_i32, _vp]),
    "w4a16_unpack_device": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp]),
    "w4a16_linear_dense": (_c_int, [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i32, _vp, _c_sz,
                                    _vp]),
    "w4a16_dense_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32]),
    "w4a16_moe_linear": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64,
                                  _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _vp]),
}


class PlanInfo(ctypes.Structure):
    """w4a16_plan_info (include/w4a16.h)."""
    _fields_ = [("path", ctypes.c_int32), ("tile_features", ctypes.c_int32),
                ("tile_tokens", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("tiles", ctypes.c_int64), ("counter_tiles", ctypes.c_int64),
                ("launches", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("two_pass", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64), ("tail_tile_tokens", ctypes.c_int32),
                ("tail_tile_features", ctypes.c_int32), ("tail_tiles", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


SIGNATURES["w4a16_plan"] = (_c_int, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32,
                                     ctypes.POINTER(PlanInfo)])


class W4A16Error(RuntimeError):
    """A libw4a16 call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [{STATUS_NAMES.get(status, status)}]")
        self.status = status
        self.message = message


def _load():
    # One HIP runtime per process: when PyTorch is present, let it load its
    # own libamdhip64 first so that libw4a16's dependency (same soname)
    # resolves to that copy instead of a second runtime from /opt/rocm.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run int4_weight_only_linear_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.w4a16_abi_version() != ABI_VERSION:
        raise ImportError(f"libw4a16 ABI {lib.w4a16_abi_version()} != binding ABI {ABI_VERSION}")
    return lib


lib = _load()


def _check(status: int):
    if status != W4A16_OK:
        raise W4A16Error(status, lib.w4a16_last_error().decode())


def w4a16_abi_version() -> int:
    return lib.w4a16_abi_version()


def w4a16_last_error() -> str:
    return lib.w4a16_last_error().decode()


def w4a16_reload_tuning() -> None:
    """Re-read the tuning environment variables (the library reads them once)."""
    lib.w4a16_reload_tuning()


# ------------------------------------------------------------------ host ---

def _host(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def w4a16_pack_weights(q: np.ndarray) -> np.ndarray:
    """uint8 [N, K] codes (0..15) -> int32 [N, K/8] words."""
    q = _host(q, np.uint8)
    N, K = q.shape
    out = np.empty((N, K // 8 if K % 8 == 0 else 0), dtype=np.int32)
    _check(lib.w4a16_pack_weights(q.ctypes.data, N, K, out.ctypes.data))
    return out


def w4a16_unpack_weights(wq: np.ndarray, K: int | None = None) -> np.ndarray:
    """int32/uint32 [N, K/8] words -> uint8 [N, K] codes."""
    wq = np.ascontiguousarray(wq)
    if wq.dtype not in (np.int32, np.uint32):
        raise TypeError(f"weights must be int32 or uint32, got {wq.dtype}")
    N = wq.shape[0]
    K = wq.shape[1] * 8 if K is None else K
    out = np.empty((N, K), dtype=np.uint8)
    _check(lib.w4a16_unpack_weights(wq.ctypes.data, N, K, out.ctypes.data))
    return out


def w4a16_pack_zeros(z: np.ndarray) -> np.ndarray:
    """uint8 [N, G] zero points -> int32 [N/8, G] words."""
    z = _host(z, np.uint8)
    N, G = z.shape
    out = np.empty((N // 8 if N % 8 == 0 else 0, G), dtype=np.int32)
    _check(lib.w4a16_pack_zeros(z.ctypes.data, N, G, out.ctypes.data))
    return out


def w4a16_unpack_zeros(zpk: np.ndarray, N: int | None = None) -> np.ndarray:
    """int32/uint32 [N/8, G] words -> uint8 [N, G] zero points."""
    zpk = np.ascontiguousarray(zpk)
    if zpk.dtype not in (np.int32, np.uint32):
        raise TypeError(f"zero points must be int32 or uint32, got {zpk.dtype}")
    N = zpk.shape[0] * 8 if N is None else N
    G = zpk.shape[1]
    out = np.empty((N, G), dtype=np.uint8)
    _check(lib.w4a16_unpack_zeros(zpk.ctypes.data, N, G, out.ctypes.data))
    return out


def w4a16_select_path(M, N, K, group_size, dtype, has_zp) -> int:
    return int(lib.w4a16_select_path(M, N, K, group_size, dtype, int(bool(has_zp))))


def w4a16_workspace_size(M, N, K, group_size, dtype, has_zp, path=PATH_AUTO) -> int:
    return int(lib.w4a16_workspace_size(M, N, K, group_size, dtype, int(bool(has_zp)), path))


def w4a16_plan(M, N, K, group_size, dtype, has_zp, path=PATH_AUTO) -> dict:
    """How the library would run this problem (host only): path, tile shape,
    output tiles, K splits, launches, waves, workspace bytes."""
    info = PlanInfo()
    _check(lib.w4a16_plan(M, N, K, group_size, dtype, int(bool(has_zp)), path, ctypes.byref(info)))
    return info.as_dict()


def w4a16_check_args(x_ptr, wq_ptr, s_ptr, zp_ptr, bias_ptr, y_ptr, M, N, K, group_size, dtype):
    """Raw-pointer argument check (no device access); raises W4A16Error."""
    _check(lib.w4a16_check_args(x_ptr, wq_ptr, s_ptr, zp_ptr, bias_ptr, y_ptr, M, N, K,
                                group_size, dtype))


# ---------------------------------------------------------------- device ---

_ZP_MSG = "Zero points must be int32 or uint32 (packed 8x uint4 along dim 0), got {}"


def _torch():
    import torch
    return torch


def _act_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return W4A16_F16
    if t.dtype == torch.bfloat16:
        return W4A16_BF16
    raise TypeError(f"activations must be float16 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _require_device(t, name, device):
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_ws_lock = threading.Lock()
_ws_cache: dict = {}


def _workspace(device, stream_ptr: int, nbytes: int):
    """A zero-filled buffer of at least nbytes, reused per (device, stream).

    Calls on one stream run in order, and every call leaves the buffer's
    counters zero again, so reuse across calls on the same stream is safe.
    """
    if nbytes == 0:
        return None
    torch = _torch()
    key = (device.index, stream_ptr)
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
            _ws_cache[key] = buf
        return buf


def _linear_args(x, wq, scales, zp, bias, group_size, out):
    torch = _torch()
    dt = _act_code(x)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    if wq.dim() != 2 or wq.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
        raise TypeError(f"wq must be a 2-D int32 or uint32 tensor, got {wq.dtype}")
    N = wq.shape[0]
    if wq.shape[1] * 8 != K:
        raise ValueError(f"wq is {tuple(wq.shape)}, expected [N, K/8] with K={K}")
    if scales.dtype != x.dtype:
        raise TypeError(f"scales must be {x.dtype}, got {scales.dtype}")
    if group_size <= 0 or K % group_size:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")
    G = K // group_size
    if tuple(scales.shape) != (N, G):
        raise ValueError(f"scales are {tuple(scales.shape)}, expected {(N, G)}")
    if zp is not None:
        if zp.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
            raise RuntimeError(_ZP_MSG.format(zp.dtype))
        if tuple(zp.shape) != (N // 8, G) or N % 8:
            raise ValueError(f"zp is {tuple(zp.shape)}, expected {(N // 8, G)} (N % 8 == 0)")
    if bias is not None:
        if bias.dtype != x.dtype or tuple(bias.shape) != (N,):
            raise ValueError(f"bias must be {x.dtype} [{N}]")
    device = x.device
    for t, name in ((x, "x"), (wq, "wq"), (scales, "scales"), (zp, "zp"), (bias, "bias")):
        _require_device(t, name, device)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=device)
    else:
        if out.dtype != x.dtype or tuple(out.shape) != (M, N):
            raise ValueError(f"out must be {x.dtype} [{M}, {N}]")
        _require_device(out, "out", device)
    return dt, M, N, K, out


def w4a16_linear_path(x, wq, scales, zp=None, bias=None, *, group_size: int, path: int = PATH_AUTO,
                      out=None, workspace=None):
    """y = x . dequant(wq, scales, zp)^T (+ bias) on x's device and current stream."""
    torch = _torch()
    dt, M, N, K, out = _linear_args(x, wq, scales, zp, bias, group_size, out)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        need = w4a16_workspace_size(M, N, K, group_size, dt, zp is not None, path)
        if workspace is None:
            workspace = _workspace(x.device, stream, need)
        ws_ptr = None if workspace is None else workspace.data_ptr()
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib.w4a16_linear_path(x.data_ptr(), wq.data_ptr(), scales.data_ptr(), _ptr(zp),
                                     _ptr(bias), out.data_ptr(), M, N, K, group_size, dt, ws_ptr,
                                     ws_bytes, stream, path))
    return out


def w4a16_linear(x, wq, scales, zp=None, bias=None, *, group_size: int, out=None, workspace=None):
    """w4a16_linear_path with the library's own choice of kernel."""
    return w4a16_linear_path(x, wq, scales, zp, bias, group_size=group_size, path=PATH_AUTO,
                             out=out, workspace=workspace)


NOALLOC_SCRATCH_BYTES = 64 << 20


def w4a16_linear_noalloc(x, wq, scales, zp=None, bias=None, *, group_size: int, out):
    """w4a16_linear without a workspace: a K split uses the library's own
    per-GPU scratch (calls that overlap on one GPU race).  `out` is required,
    so that the call allocates nothing."""
    torch = _torch()
    dt, M, N, K, out = _linear_args(x, wq, scales, zp, bias, group_size, out)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        _check(lib.w4a16_linear_noalloc(x.data_ptr(), wq.data_ptr(), scales.data_ptr(), _ptr(zp),
                                        _ptr(bias), out.data_ptr(), M, N, K, group_size, dt, stream))
    return out


def w4a16_dequant(wq, scales, zp=None, *, group_size: int, out=None):
    """Dequantised weights [N, K] in the scales' dtype, rounded once to nearest-even."""
    torch = _torch()
    dt = _act_code(scales)
    N, K = wq.shape[0], wq.shape[1] * 8
    if zp is not None and zp.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
        raise RuntimeError(_ZP_MSG.format(zp.dtype))
    for t, name in ((wq, "wq"), (scales, "scales"), (zp, "zp")):
        _require_device(t, name, wq.device)
    if out is None:
        out = torch.empty((N, K), dtype=scales.dtype, device=wq.device)
    stream = torch.cuda.current_stream(wq.device).cuda_stream
    with torch.cuda.device(wq.device):
        _check(lib.w4a16_dequant(wq.data_ptr(), scales.data_ptr(), _ptr(zp), out.data_ptr(), N, K,
                                 group_size, dt, stream))
    return out


def w4a16_unpack_device(wq, out=None):
    """uint8 codes [N, K] unpacked on the device."""
    torch = _torch()
    N, K = wq.shape[0], wq.shape[1] * 8
    _require_device(wq, "wq", wq.device)
    if out is None:
        out = torch.empty((N, K), dtype=torch.uint8, device=wq.device)
    stream = torch.cuda.current_stream(wq.device).cuda_stream
    with torch.cuda.device(wq.device):
        _check(lib.w4a16_unpack_device(wq.data_ptr(), out.data_ptr(), N, K, stream))
    return out


def w4a16_dense_workspace_size(M, N, K, dtype, has_bias) -> int:
    return int(lib.w4a16_dense_workspace_size(M, N, K, dtype, int(bool(has_bias))))


def w4a16_linear_dense(x, w, bias=None, *, out=None, workspace=None):
    """y = x . w^T (+ bias) with w the dequantised weights [N, K] (w4a16_dequant),
    on x's device and current stream."""
    torch = _torch()
    dt = _act_code(x)
    if x.dim() != 2 or w.dim() != 2 or w.shape[1] != x.shape[1]:
        raise ValueError(f"x must be [M, K] and w [N, K], got {tuple(x.shape)} and {tuple(w.shape)}")
    if w.dtype != x.dtype or (bias is not None and bias.dtype != x.dtype):
        raise TypeError("x, w and bias must share one dtype")
    M, K = x.shape
    N = w.shape[0]
    if bias is not None and tuple(bias.shape) != (N,):
        raise ValueError(f"bias must be [{N}]")
    for t, name in ((x, "x"), (w, "w"), (bias, "bias")):
        _require_device(t, name, x.device)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        need = w4a16_dense_workspace_size(M, N, K, dt, bias is not None)
        if workspace is None:
            workspace = _workspace(x.device, stream, need)
        ws_ptr = None if workspace is None else workspace.data_ptr()
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib.w4a16_linear_dense(x.data_ptr(), w.data_ptr(), _ptr(bias), out.data_ptr(), M, N, K,
                                      dt, ws_ptr, ws_bytes, stream))
    return out


def w4a16_moe_linear(x, wq, scales, topk_ids, zp=None, bias=None, topk_weights=None, *,
                     group_size: int, x_per_slot: bool = False, out=None):
    """Expert-indexed decode: y[m*topk + j] = topk_weights[m, j] * (x_row . W_e^T + b_e),
    e = topk_ids[m, j], with stacks wq [E, N, K/8], scales [E, N, G], zp [E, N/8, G],
    bias [E, N]; x is [M, K] (or [M*topk, K] with x_per_slot).  Returns [M*topk, N]."""
    torch = _torch()
    dt = _act_code(x)
    if wq.dim() != 3:
        raise ValueError("wq must be [E, N, K/8]")
    E, N, K = wq.shape[0], wq.shape[1], wq.shape[2] * 8
    if topk_ids.dim() != 2 or topk_ids.dtype != torch.int32:
        raise TypeError("topk_ids must be int32 [M, topk]")
    M, topk = topk_ids.shape
    if x.dim() != 2 or x.shape[1] != K or x.shape[0] != (M * topk if x_per_slot else M):
        raise ValueError(f"x is {tuple(x.shape)}, expected [{M * topk if x_per_slot else M}, {K}]")
    if group_size <= 0 or K % group_size:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")
    G = K // group_size
    if scales.dtype != x.dtype or tuple(scales.shape) != (E, N, G):
        raise ValueError(f"scales must be {x.dtype} {(E, N, G)}")
    if zp is not None and (zp.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32))
                           or tuple(zp.shape) != (E, N // 8, G)):
        raise ValueError(f"zp must be int32 {(E, N // 8, G)}")
    if bias is not None and (bias.dtype != x.dtype or tuple(bias.shape) != (E, N)):
        raise ValueError(f"bias must be {x.dtype} {(E, N)}")
    if topk_weights is not None and (topk_weights.dtype != torch.float32
                                     or tuple(topk_weights.shape) != (M, topk)):
        raise ValueError(f"topk_weights must be float32 {(M, topk)}")
    for t, name in ((x, "x"), (wq, "wq"), (scales, "scales"), (zp, "zp"), (bias, "bias"),
                    (topk_ids, "topk_ids"), (topk_weights, "topk_weights")):
        _require_device(t, name, x.device)
    if out is None:
        out = torch.empty((M * topk, N), dtype=x.dtype, device=x.device)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        _check(lib.w4a16_moe_linear(x.data_ptr(), wq.data_ptr(), scales.data_ptr(), _ptr(zp), _ptr(bias),
                                    topk_ids.data_ptr(), _ptr(topk_weights), out.data_ptr(), M, topk, E,
                                    N, K, group_size, dt, int(bool(x_per_slot)), stream))
    return out
