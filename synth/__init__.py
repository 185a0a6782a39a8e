"""Seeded synthetic workloads for the WUSH-KV cache write/read path.

The five workloads below are stand-ins for the Qwen3 activations that the
WUSH-KV pages evaluate on (WikiText-2, FineWeb-Edu, RULER, MRCR); those
datasets and model weights are not used.  Shapes follow the pages' models
(Qwen3-8B / Qwen3-32B: 8 KV heads of dimension 128, 36 / 64 layers) and the
pages' context lengths.

This module only draws numbers (see ``wushkv_synth.c``).  Both the CPU
oracle and the GPU library consume its output; it contains none of the
method's arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wushkv_synth.c")
_LIB_PATH = os.path.join(_HERE, "libwushkv_synth.so")

DIST_GAUSS_OUTLIER = 0
DIST_HEAVY_T3 = 1
DIST_LOGNORMAL_GAUSS = 2

D = 128


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    layers: int
    heads: int
    tokens: int              # tokens per layer call
    dtype: str               # "f32" | "bf16" (input K/V element type)
    dist: int
    bits: tuple
    quant: str               # "sym" | "affine"
    theta: float = 1e6
    clip_alpha: float = 2.0
    group: int = 128
    p_lo: float = 1.0
    p_hi: float = 99.0
    positions: str = "arange"  # "arange" | "decode" | "per_sequence"
    seq_len: int = 0           # per-sequence length for "per_sequence"
    cache_rows: int = 0        # rows of the packed cache (decode: batch * 32768)
    round_trip: bool = False
    notes: str = field(default="")

    @property
    def seed(self) -> int:
        return 1000 + self.index


WORKLOADS = {
    "tiny": Workload(
        0, "tiny", layers=1, heads=2, tokens=256, dtype="f32",
        dist=DIST_GAUSS_OUTLIER, bits=(2,), quant="sym",
        notes="fp32 N(0,1) K/V with 4 outlier channels per head scaled x20"),
    "qwen3_8b_prefill": Workload(
        1, "qwen3_8b_prefill", layers=1, heads=8, tokens=32768, dtype="bf16",
        dist=DIST_HEAVY_T3, bits=(2,), quant="sym",
        notes="bf16 K/V = sigma[h,c] * t3, sigma ~ LogNormal(0,1)"),
    "decode_append": Workload(
        2, "decode_append", layers=36, heads=8, tokens=64, dtype="bf16",
        dist=DIST_GAUSS_OUTLIER, bits=(2,), quant="sym", positions="decode",
        cache_rows=64 * 32768,
        notes="batch 64, one token each at U[0,32768); slot = b*32768 + pos"),
    "qwen3_32b_full": Workload(
        3, "qwen3_32b_full", layers=64, heads=8, tokens=131072, dtype="bf16",
        dist=DIST_HEAVY_T3, bits=(3, 4), quant="sym", round_trip=True,
        notes="as qwen3_8b_prefill, 3- and 4-bit, dequantize through T_k^-1"),
    "affine_pct": Workload(
        4, "affine_pct", layers=36, heads=8, tokens=16 * 16384, dtype="bf16",
        dist=DIST_LOGNORMAL_GAUSS, bits=(2,), quant="affine", group=32,
        positions="per_sequence", seq_len=16384, round_trip=True,
        notes="bf16 K/V = sigma[h,c] * N(0,1); 16 sequences x 16384"),
}
WORKLOAD_ORDER = ["tiny", "qwen3_8b_prefill", "decode_append", "qwen3_32b_full", "affine_pct"]

_lib = None


def build(force: bool = False) -> str:
    """Compile the generator (gcc, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int
        vp = ctypes.c_void_p
        lib.synth_kv.argtypes = [u64, i32, i32, i32, i64, i64, i32, i32, vp, i32]
        lib.synth_kv.restype = i32
        lib.synth_transform.argtypes = [u64, i32, i32, vp, vp]
        lib.synth_transform.restype = i32
        lib.synth_uniform_ints.argtypes = [u64, i64, i64, vp]
        lib.synth_uniform_ints.restype = None
        lib.synth_outliers.argtypes = [u64, i32, i32, i32, vp]
        lib.synth_outliers.restype = None
        lib.synth_channel_sigma.argtypes = [u64, i32, i32, i32, vp]
        lib.synth_channel_sigma.restype = None
        lib.synth_draw.argtypes = [u64, u64, u64]
        lib.synth_draw.restype = u64
        lib.synth_normal.argtypes = [u64, u64, u64]
        lib.synth_normal.restype = ctypes.c_double
        lib.synth_t3.argtypes = [u64, u64, u64]
        lib.synth_t3.restype = ctypes.c_double
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def kv(w: Workload, layer: int, tensor: str, n0: int = 0, n: int | None = None,
       dtype: str | None = None, threads: int | None = None) -> np.ndarray:
    """Pre-RoPE keys (tensor="K") or values ("V") for tokens [n0, n0+n) of a layer.

    Returns a C-contiguous array [n][heads][128]: float32, or uint16 holding
    bf16 bit patterns.
    """
    if n is None:
        n = w.tokens - n0
    dtype = dtype or w.dtype
    t = {"K": 0, "V": 1}[tensor]
    out = np.empty((n, w.heads, D), dtype=np.uint16 if dtype == "bf16" else np.float32)
    rc = _load().synth_kv(w.seed, w.dist, layer, t, n0, n, w.heads, 1 if dtype == "bf16" else 0,
                          out.ctypes.data, threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"synth_kv failed ({rc})")
    return out


def transform(w: Workload, layer: int):
    """(T, T_inv), each float32 [heads][128][128] row-major; T = Q diag(s)."""
    T = np.empty((w.heads, D, D), dtype=np.float32)
    Ti = np.empty((w.heads, D, D), dtype=np.float32)
    rc = _load().synth_transform(w.seed, layer, w.heads, T.ctypes.data, Ti.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"synth_transform failed ({rc})")
    return T, Ti


def positions(w: Workload, n0: int = 0, n: int | None = None) -> np.ndarray:
    """int32 positions of tokens [n0, n0+n) (shared by all layers)."""
    if n is None:
        n = w.tokens - n0
    if w.positions == "arange":
        return np.arange(n0, n0 + n, dtype=np.int32)
    if w.positions == "per_sequence":
        return (np.arange(n0, n0 + n, dtype=np.int64) % w.seq_len).astype(np.int32)
    if w.positions == "decode":
        allp = np.empty(w.tokens, dtype=np.int32)
        _load().synth_uniform_ints(w.seed, w.tokens, 32768, allp.ctypes.data)
        return allp[n0:n0 + n].copy()
    raise ValueError(w.positions)


def slots(w: Workload) -> np.ndarray | None:
    """int64 cache rows for the decode workload: batch b writes row b*32768 + pos_b."""
    if w.positions != "decode":
        return None
    p = positions(w).astype(np.int64)
    return np.arange(w.tokens, dtype=np.int64) * 32768 + p


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def draw(seed: int, stream: int, idx: int) -> int:
    return int(_load().synth_draw(seed, stream, idx))


def normal(seed: int, stream: int, idx: int) -> float:
    return float(_load().synth_normal(seed, stream, idx))


def student_t3(seed: int, stream: int, idx: int) -> float:
    return float(_load().synth_t3(seed, stream, idx))


def outliers(w: Workload, layer: int, tensor: str, head: int) -> list:
    out = (ctypes.c_int * 4)()
    _load().synth_outliers(w.seed, layer, {"K": 0, "V": 1}[tensor], head, out)
    return list(out)


def channel_sigma(w: Workload, layer: int, tensor: str) -> np.ndarray:
    s = np.empty((w.heads, D), dtype=np.float64)
    _load().synth_channel_sigma(w.seed, layer, {"K": 0, "V": 1}[tensor], w.heads, s.ctypes.data)
    return s
