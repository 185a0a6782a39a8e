"""ctypes declarations for libwushkv.so (the C ABI in include/wushkv.h)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("WUSHKV_LIB", os.path.join(HERE, "libwushkv.so"))

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_ALIGNMENT, ERR_NO_DEVICE, ERR_HIP, ERR_OOM = range(7)
F32, BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 24 << 20  # WUSHKV_NOALLOC_SCRATCH_BYTES
Q_SYM_RMS, Q_AFFINE_PCT = 0, 1

# every symbol include/wushkv.h declares
EXPORTED = [
    "wushkv_transform_create", "wushkv_transform_destroy", "wushkv_rope_create", "wushkv_rope_destroy",
    "wushkv_rope_frequencies", "wushkv_quantize_keys", "wushkv_quantize_values", "wushkv_dequantize",
    "wushkv_debug_rope_transform", "wushkv_debug_rope_cos_sin", "wushkv_debug_time_next_launch",
    "wushkv_status_string", "wushkv_last_error", "wushkv_version", "wushkv_pair_queries",
    "wushkv_decode_attention_workspace", "wushkv_decode_attention", "wushkv_decode_attention_noalloc",
    "wushkv_quantize_kv", "wushkv_debug_check_arith", "wushkv_transform_create_hadamard",
]


class Quantizer(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("clip_alpha", ctypes.c_float), ("group", ctypes.c_int32),
                ("p_lo", ctypes.c_float), ("p_hi", ctypes.c_float)]


class Packed(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("slots", ctypes.c_void_p), ("n_rows", ctypes.c_int64)]


class WushKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libwushkv status {status}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libwushkv.so.  Raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libwushkv.so not found at {LIB_PATH}; build it with "
                          "`python -m bit_kv_cache_rope_amd.build` (there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    qp, pp = ctypes.POINTER(Quantizer), ctypes.POINTER(Packed)
    L.wushkv_transform_create.argtypes = [vp, i32, ctypes.POINTER(vp)]
    L.wushkv_transform_create_hadamard.argtypes = [i32, ctypes.POINTER(vp)]
    L.wushkv_transform_destroy.argtypes = [vp]
    L.wushkv_rope_create.argtypes = [f32, ctypes.c_int32, ctypes.POINTER(vp)]
    L.wushkv_rope_destroy.argtypes = [vp]
    L.wushkv_rope_frequencies.argtypes = [f32, vp]
    L.wushkv_quantize_keys.argtypes = [vp, i32, i64, i32, i64, vp, vp, vp, i32, qp, pp, vp]
    L.wushkv_quantize_values.argtypes = [vp, i32, i64, i32, i64, i32, qp, pp, vp]
    L.wushkv_quantize_kv.argtypes = [vp, vp, i32, i64, i32, i64, i64, vp, vp, vp, i32, qp, pp, pp, vp]
    L.wushkv_dequantize.argtypes = [pp, i64, i32, i32, qp, vp, vp, i32, vp]
    L.wushkv_debug_rope_transform.argtypes = [vp, i32, i64, i32, i64, vp, vp, vp, vp, vp]
    L.wushkv_debug_rope_cos_sin.argtypes = [vp, vp, i64, vp, vp]
    L.wushkv_debug_time_next_launch.argtypes = [vp, vp]
    L.wushkv_debug_check_arith.argtypes = [vp, vp]
    L.wushkv_pair_queries.argtypes = [vp, i32, i64, i32, i64, vp, vp, vp]
    L.wushkv_decode_attention_workspace.argtypes = [i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.wushkv_decode_attention.argtypes = [vp, i32, i32, pp, pp, i32, i32, qp, vp, vp, i32, f32, vp,
                                          ctypes.c_size_t, vp, vp]
    L.wushkv_decode_attention_noalloc.argtypes = [vp, i32, i32, pp, pp, i32, i32, qp, vp, vp, i32, f32, vp, vp]
    L.wushkv_status_string.argtypes = [i32]
    L.wushkv_status_string.restype = ctypes.c_char_p
    L.wushkv_last_error.argtypes = []
    L.wushkv_last_error.restype = ctypes.c_char_p
    L.wushkv_version.argtypes = []
    for name in EXPORTED:
        if name not in ("wushkv_status_string", "wushkv_last_error"):
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def check(status: int) -> None:
    if status != OK:
        L = load()
        msg = L.wushkv_last_error().decode() or L.wushkv_status_string(status).decode()
        raise WushKVError(status, msg)


def hip_runtimes_mapped() -> list:
    """Paths of HIP runtime libraries mapped into this process."""
    seen = []
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                p = line.split()[-1] if len(line.split()) >= 6 else ""
                if "libamdhip64" in p and p not in seen:
                    seen.append(p)
    except OSError:  # pragma: no cover
        pass
    return seen
