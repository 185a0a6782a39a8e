"""CPU oracle for the WUSH-KV cache write/read path (ctypes wrapper).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU
library (``bit_kv_cache_rope_amd``) never imports it, and the two share no
code.  The arithmetic lives in ``wushkv_oracle.cpp``; this module only
marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wushkv_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "libwushkv_oracle.so")

D = 128
SYM, AFFINE = 0, 1


class Quantizer(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("clip_alpha", ctypes.c_float), ("group", ctypes.c_int32),
                ("p_lo", ctypes.c_float), ("p_hi", ctypes.c_float)]


def sym(alpha: float = 2.0) -> Quantizer:
    return Quantizer(SYM, alpha, 128, 0.0, 100.0)


def affine(p_lo: float = 1.0, p_hi: float = 99.0) -> Quantizer:
    return Quantizer(AFFINE, 0.0, 32, p_lo, p_hi)


_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with g++ -O2, no contraction, no fast-math."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _lib_():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        qp = ctypes.POINTER(Quantizer)
        L.wko_round_bf16.argtypes = [f32]; L.wko_round_bf16.restype = f32
        L.wko_f32_to_f16.argtypes = [f32]; L.wko_f32_to_f16.restype = ctypes.c_uint16
        L.wko_f16_to_f32.argtypes = [ctypes.c_uint16]; L.wko_f16_to_f32.restype = f32
        L.wko_omega.argtypes = [f32, i32]; L.wko_omega.restype = f32
        L.wko_round_bf16_array.argtypes = [vp, vp, i64]; L.wko_round_bf16_array.restype = None
        L.wko_f32_to_f16_array.argtypes = [vp, vp, i64]; L.wko_f32_to_f16_array.restype = None
        L.wko_cos_sin.argtypes = [f32, vp, i64, vp]; L.wko_cos_sin.restype = None
        L.wko_rope.argtypes = [vp, ctypes.c_int32, f32, vp]; L.wko_rope.restype = None
        L.wko_pairwise_sum.argtypes = [vp, i32]; L.wko_pairwise_sum.restype = f32
        L.wko_sym_quantize.argtypes = [vp, i32, f32, vp, vp]; L.wko_sym_quantize.restype = None
        L.wko_affine_quantize_group.argtypes = [vp, i32, f32, f32, vp, vp, vp]
        L.wko_affine_quantize_group.restype = None
        L.wko_percentile32.argtypes = [vp, f32]; L.wko_percentile32.restype = f32
        L.wko_pack.argtypes = [vp, i32, vp]; L.wko_pack.restype = None
        L.wko_unpack.argtypes = [vp, i32, vp]; L.wko_unpack.restype = None
        L.wko_transform_f64.argtypes = [vp, vp, vp]; L.wko_transform_f64.restype = None
        L.wko_query_pair.argtypes = [vp, vp, vp]; L.wko_query_pair.restype = i32
        L.wko_quantize_keys.argtypes = [vp, i32, i64, i32, i64, vp, vp, f32, i32, qp, vp, vp, vp, vp,
                                        vp, i32]
        L.wko_quantize_keys.restype = i32
        L.wko_quantize_values.argtypes = [vp, i32, i64, i32, i64, i32, qp, vp, vp, vp, vp, i32]
        L.wko_quantize_values.restype = i32
        L.wko_dequantize.argtypes = [vp, vp, vp, vp, i64, i32, i32, qp, vp, vp, i32]
        L.wko_dequantize.restype = i32
        L.wko_pair_queries.argtypes = [vp, i32, i64, i32, i64, vp, i32, vp]
        L.wko_pair_queries.restype = i32
        L.wko_decode_attention.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, i64, i32, vp, vp, f32,
                                           vp, i32]
        L.wko_decode_attention.restype = i32
        _lib = L
    return _lib


def threads_default() -> int:
    v = os.environ.get("WUSHKV_ORACLE_THREADS", "1")
    if v == "all":
        try:
            return len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            return os.cpu_count() or 1
    return max(1, int(v))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- scalar / small building blocks -------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty_like(x)
    _lib_().wko_round_bf16_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _lib_().wko_f32_to_f16_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def f16_to_f32(h: int) -> float:
    return float(_lib_().wko_f16_to_f32(int(h)))


def omega(theta: float, i: int) -> float:
    return float(_lib_().wko_omega(theta, i))


def cos_sin(theta: float, pos) -> np.ndarray:
    pos = _c(pos, np.int32)
    cs = np.empty((pos.size, 64, 2), dtype=np.float32)
    _lib_().wko_cos_sin(theta, pos.ctypes.data, pos.size, cs.ctypes.data)
    return cs


def rope(k: np.ndarray, pos: int, theta: float) -> np.ndarray:
    k = _c(k, np.float32)
    x = np.empty(D, dtype=np.float32)
    _lib_().wko_rope(k.ctypes.data, int(pos), theta, x.ctypes.data)
    return x


def pairwise_sum(a: np.ndarray) -> float:
    a = _c(a, np.float32)
    return float(_lib_().wko_pairwise_sum(a.ctypes.data, a.size))


def sym_quantize(y: np.ndarray, bits: int, alpha: float = 2.0):
    y = _c(y, np.float32)
    q = np.empty(D, dtype=np.uint8)
    sc = np.zeros(1, dtype=np.uint16)
    _lib_().wko_sym_quantize(y.ctypes.data, bits, alpha, q.ctypes.data, sc.ctypes.data)
    return q, int(sc[0])


def affine_quantize_group(x: np.ndarray, bits: int, p_lo: float = 1.0, p_hi: float = 99.0):
    x = _c(x, np.float32)
    q = np.empty(32, dtype=np.uint8)
    sc = np.zeros(1, dtype=np.uint16)
    zr = np.zeros(1, dtype=np.uint16)
    _lib_().wko_affine_quantize_group(x.ctypes.data, bits, p_lo, p_hi, q.ctypes.data, sc.ctypes.data,
                                      zr.ctypes.data)
    return q, int(sc[0]), int(zr[0])


def percentile32(sorted_vals: np.ndarray, p: float) -> float:
    s = _c(sorted_vals, np.float32)
    return float(_lib_().wko_percentile32(s.ctypes.data, p))


def pack(q: np.ndarray, bits: int) -> np.ndarray:
    q = _c(q, np.uint8)
    rec = np.empty(16 * bits, dtype=np.uint8)
    _lib_().wko_pack(q.ctypes.data, bits, rec.ctypes.data)
    return rec


def unpack(rec: np.ndarray, bits: int) -> np.ndarray:
    rec = _c(rec, np.uint8)
    q = np.empty(D, dtype=np.uint8)
    _lib_().wko_unpack(rec.ctypes.data, bits, q.ctypes.data)
    return q


def transform_f64(T: np.ndarray, x: np.ndarray) -> np.ndarray:
    T = _c(T, np.float32)
    x = _c(x, np.float64)
    y = np.empty(D, dtype=np.float64)
    _lib_().wko_transform_f64(T.ctypes.data, x.ctypes.data, y.ctypes.data)
    return y


def query_pair(T: np.ndarray, q: np.ndarray) -> np.ndarray:
    T = _c(T, np.float32)
    q = _c(q, np.float64)
    qp = np.empty(D, dtype=np.float64)
    if _lib_().wko_query_pair(T.ctypes.data, q.ctypes.data, qp.ctypes.data) != 0:
        raise np.linalg.LinAlgError("singular transform")
    return qp


# ---- whole-tensor entry points ----------------------------------------------------------

def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:  # bf16 bit patterns
        return 1
    raise TypeError(a.dtype)


def _outputs(rows: int, H: int, bits: int, q: Quantizer):
    codes = np.zeros((rows, H, 16 * bits), dtype=np.uint8)
    nsc = 1 if q.kind == SYM else 4
    scales = np.zeros((rows, H, nsc) if nsc > 1 else (rows, H), dtype=np.uint16)
    zeros = np.zeros((rows, H, 4), dtype=np.uint16) if q.kind == AFFINE else None
    return codes, scales, zeros


def quantize_keys(K: np.ndarray, pos: np.ndarray, T: np.ndarray, theta: float, bits: int,
                  q: Quantizer, slots: np.ndarray | None = None, rows: int | None = None,
                  want_y: bool = False, threads: int | None = None):
    """K: [N][H][128] float32 or uint16 (bf16 bits).  Returns dict(codes, scales, zeros, y)."""
    K = np.ascontiguousarray(K)
    N, H = K.shape[0], K.shape[1]
    pos = _c(pos, np.int32)
    T = _c(T, np.float32)
    if slots is not None:
        slots = _c(slots, np.int64)
    rows = rows if rows is not None else (int(slots.max()) + 1 if slots is not None and N else N)
    codes, scales, zeros = _outputs(rows, H, bits, q)
    y = np.empty((N, H, D), dtype=np.float32) if want_y else None
    rc = _lib_().wko_quantize_keys(K.ctypes.data, _dtype_code(K), N, H, H * D, pos.ctypes.data,
                                   T.ctypes.data, theta, bits, ctypes.byref(q), codes.ctypes.data,
                                   scales.ctypes.data, _ptr(zeros), _ptr(slots), _ptr(y),
                                   threads or threads_default())
    if rc != 0:
        raise ValueError("oracle rejected arguments")
    return dict(codes=codes, scales=scales, zeros=zeros, y=y)


def quantize_values(V: np.ndarray, bits: int, q: Quantizer, slots: np.ndarray | None = None,
                    rows: int | None = None, threads: int | None = None):
    V = np.ascontiguousarray(V)
    N, H = V.shape[0], V.shape[1]
    if slots is not None:
        slots = _c(slots, np.int64)
    rows = rows if rows is not None else (int(slots.max()) + 1 if slots is not None and N else N)
    codes, scales, zeros = _outputs(rows, H, bits, q)
    rc = _lib_().wko_quantize_values(V.ctypes.data, _dtype_code(V), N, H, H * D, bits, ctypes.byref(q),
                                     codes.ctypes.data, scales.ctypes.data, _ptr(zeros), _ptr(slots),
                                     threads or threads_default())
    if rc != 0:
        raise ValueError("oracle rejected arguments")
    return dict(codes=codes, scales=scales, zeros=zeros)


def dequantize(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray | None, N: int, H: int,
               bits: int, q: Quantizer, Tinv: np.ndarray | None = None,
               slots: np.ndarray | None = None, threads: int | None = None) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint16)
    zeros = None if zeros is None else _c(zeros, np.uint16)
    Tinv = None if Tinv is None else _c(Tinv, np.float32)
    if slots is not None:
        slots = _c(slots, np.int64)
    out = np.empty((N, H, D), dtype=np.float32)
    rc = _lib_().wko_dequantize(codes.ctypes.data, scales.ctypes.data, _ptr(zeros), _ptr(slots), N, H,
                                bits, ctypes.byref(q), _ptr(Tinv), out.ctypes.data,
                                threads or threads_default())
    if rc != 0:
        raise ValueError("oracle rejected arguments")
    return out


def pair_queries(Q: np.ndarray, Tinv: np.ndarray) -> np.ndarray:
    """Q: [N][Hq][128] float32 or uint16 (bf16 bits); Tinv: [Hkv][128][128].
    Returns the paired queries as bf16 bits [N][Hq][128]."""
    Q = np.ascontiguousarray(Q)
    Tinv = _c(Tinv, np.float32)
    N, Hq = Q.shape[0], Q.shape[1]
    out = np.empty((N, Hq, D), dtype=np.uint16)
    rc = _lib_().wko_pair_queries(Q.ctypes.data, _dtype_code(Q), N, Hq, Hq * D, Tinv.ctypes.data,
                                  Tinv.shape[0], out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected arguments")
    return out


def decode_attention(qp: np.ndarray, k: dict, v: dict, bits: int, row0: np.ndarray, lens: np.ndarray,
                     scale: float, threads: int | None = None) -> np.ndarray:
    """qp: bf16 bits [B][Hq][128]; k, v: dicts with ``codes`` [rows][Hkv][16 bits] and
    ``scales``: symmetric [rows][Hkv]; affine (``zeros`` present in both) [rows][Hkv][4]
    steps and zeros.  Sequence b reads rows row0[b] + n, n < lens[b].  Returns fp32
    [B][Hq][128]."""
    qp = _c(qp, np.uint16)
    kc, ks = _c(k["codes"], np.uint8), _c(k["scales"], np.uint16)
    vc, vs = _c(v["codes"], np.uint8), _c(v["scales"], np.uint16)
    kz = None if k.get("zeros") is None else _c(k["zeros"], np.uint16)
    vz = None if v.get("zeros") is None else _c(v["zeros"], np.uint16)
    row0 = _c(row0, np.int64)
    lens = _c(lens, np.int32)
    B, Hq = qp.shape[0], qp.shape[1]
    out = np.empty((B, Hq, D), dtype=np.float32)
    rc = _lib_().wko_decode_attention(qp.ctypes.data, B, Hq, kc.shape[1], kc.ctypes.data, ks.ctypes.data,
                                      _ptr(kz), vc.ctypes.data, vs.ctypes.data, _ptr(vz), kc.shape[0], bits,
                                      row0.ctypes.data, lens.ctypes.data, scale, out.ctypes.data,
                                      threads or threads_default())
    if rc != 0:
        raise ValueError("oracle rejected arguments")
    return out
