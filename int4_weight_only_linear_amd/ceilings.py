"""ctypes binding of libw4a16_ceilings.so (include/w4a16_ceilings.h): the
measurement kernels the benchmark times beside the W4A16 path (HBM read rate,
the decode kernel's load pattern alone, the sustained MFMA rate).  Argument
marshalling only; raises on import if the library is not built."""
from __future__ import annotations

import ctypes
import os

from . import _binding  # noqa: F401  (loads torch's HIP runtime first, as for libw4a16)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4a16_ceilings.so")

_i32, _i64, _u32, _u64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p
SIGNATURES = {
    "w4a16c_stream_read": (ctypes.c_int, [_vp, _u64, _vp, _vp]),
    "w4a16c_decode_loads": (ctypes.c_int, [_vp, _u64, _i64, _i64, _i64, _i32, _i32, _vp, _vp]),
    "w4a16c_mfma_loop": (ctypes.c_int, [_i32, _i32, _u32, _vp, _vp]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run int4_weight_only_linear_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


lib = _load()


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed: hipError {rc}")


def stream_read(buf, sink, stream_ptr, nbytes=None):
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check(lib.w4a16c_stream_read(buf.data_ptr(), n, sink.data_ptr(), stream_ptr), "stream_read")


def decode_loads(wq, tiles, K, tile_stride, kpw, waves, sink, stream_ptr):
    _check(lib.w4a16c_decode_loads(wq.data_ptr(), wq.numel() * wq.element_size(), tiles, K, tile_stride,
                                   kpw, waves, sink.data_ptr(), stream_ptr), "decode_loads")


def mfma_loop(blocks, iters, seed, sink, stream_ptr):
    _check(lib.w4a16c_mfma_loop(blocks, iters, seed, sink.data_ptr(), stream_ptr), "mfma_loop")
