"""bit_kv_cache_rope_amd — Python binding of libwushkv (WUSH-KV cache path on MI355X).

Argument marshalling only: every step of the write and read path runs in the
HIP kernels of libwushkv.so.  PyTorch supplies device memory and the stream.
The functions keep the C names:

    wushkv_quantize_keys(K, pos, rope, T_k, bits, quantizer, out)
    wushkv_quantize_values(V, bits, quantizer, out)
    wushkv_dequantize(packed, n_tokens, n_heads, bits, quantizer, T_k_inv=None, ...)
    wushkv_pair_queries(Q, T_k_inv)
    wushkv_decode_attention(q_paired, k_cache, v_cache, n_kv_heads, bits, quantizer, seq_row0, seq_len, ...)
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch  # imported first: the library binds to the HIP runtime torch has loaded

from . import _lib
from ._lib import WushKVError, F32, BF16, Q_SYM_RMS, Q_AFFINE_PCT  # noqa: F401

__all__ = [
    "WushKVError", "Quantizer", "sym", "affine", "Transform", "Rope", "PackedCache", "alloc_packed",
    "wushkv_quantize_keys", "wushkv_quantize_values", "wushkv_dequantize", "wushkv_debug_rope_transform",
    "wushkv_debug_rope_cos_sin", "wushkv_debug_time_next_launch", "wushkv_decode_attention_noalloc",
    "wushkv_rope_frequencies", "library", "PreparedCall", "prepare_quantize_keys",
    "prepare_quantize_values", "prepare_dequantize", "wushkv_pair_queries", "wushkv_decode_attention_workspace",
    "wushkv_decode_attention", "prepare_decode_attention", "wushkv_quantize_kv", "prepare_quantize_kv",
    "wushkv_debug_check_arith",
]


_checked = False


def library() -> ctypes.CDLL:
    """The loaded libwushkv.so (raises ImportError if it is not built).  The
    first call also checks that a single HIP runtime is mapped (the one torch
    loaded)."""
    global _checked
    L = _lib.load()
    if not _checked:
        maps = _lib.hip_runtimes_mapped()
        if len(maps) > 1:
            raise RuntimeError(f"more than one HIP runtime mapped into this process: {maps}")
        _checked = True
    return L


@dataclass(frozen=True)
class Quantizer:
    kind: int = Q_SYM_RMS
    clip_alpha: float = 2.0
    group: int = 128
    p_lo: float = 1.0
    p_hi: float = 99.0

    def c(self) -> _lib.Quantizer:
        return _lib.Quantizer(self.kind, self.clip_alpha, self.group, self.p_lo, self.p_hi)

    @property
    def scales_per_head(self) -> int:
        return 1 if self.kind == Q_SYM_RMS else 4


def sym(clip_alpha: float = 2.0) -> Quantizer:
    return Quantizer(Q_SYM_RMS, clip_alpha, 128, 0.0, 100.0)


def affine(p_lo: float = 1.0, p_hi: float = 99.0) -> Quantizer:
    return Quantizer(Q_AFFINE_PCT, 0.0, 32, p_lo, p_hi)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Transform:
    """Key transform handle (T_k, or T_k^-1 for reads); T: [H][128][128] fp32, y = T x.
    Transform.hadamard(H) is the structured handle T = H_128 / 8 whose key path is a fast
    Walsh-Hadamard transform (wushkv_transform_create_hadamard)."""

    def __init__(self, T):
        T = torch.as_tensor(T).detach().to("cpu", torch.float32).contiguous()
        if T.dim() != 3 or T.shape[1:] != (128, 128):
            raise ValueError("T must be [n_heads][128][128]")
        self.n_heads = int(T.shape[0])
        h = ctypes.c_void_p()
        _lib.check(library().wushkv_transform_create(ctypes.c_void_p(T.data_ptr()), self.n_heads, ctypes.byref(h)))
        self._h = h

    @classmethod
    def hadamard(cls, n_heads: int) -> "Transform":
        t = cls.__new__(cls)
        t.n_heads = int(n_heads)
        h = ctypes.c_void_p()
        _lib.check(library().wushkv_transform_create_hadamard(t.n_heads, ctypes.byref(h)))
        t._h = h
        return t

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            library().wushkv_transform_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Rope:
    """RoPE handle: base theta, positions in [0, max_pos)."""

    def __init__(self, theta: float = 1e6, max_pos: int = 1 << 17):
        self.theta, self.max_pos = float(theta), int(max_pos)
        h = ctypes.c_void_p()
        _lib.check(library().wushkv_rope_create(ctypes.c_float(self.theta), self.max_pos, ctypes.byref(h)))
        self._h = h

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            library().wushkv_rope_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


@dataclass
class PackedCache:
    """Caller-owned packed cache: codes uint8 [rows][H][16*bits], scales fp16
    [rows][H] (sym) or [rows][H][4] (affine), zeros fp16 [rows][H][4] (affine)."""
    codes: torch.Tensor
    scales: torch.Tensor
    zeros: torch.Tensor | None = None
    slots: torch.Tensor | None = None

    @property
    def n_rows(self) -> int:
        return int(self.codes.shape[0])

    def c(self) -> _lib.Packed:
        return _lib.Packed(self.codes.data_ptr(), self.scales.data_ptr(),
                           None if self.zeros is None else self.zeros.data_ptr(),
                           None if self.slots is None else self.slots.data_ptr(), self.n_rows)

    def with_slots(self, slots: torch.Tensor | None) -> "PackedCache":
        return PackedCache(self.codes, self.scales, self.zeros, slots)


def alloc_packed(rows: int, n_heads: int, bits: int, quantizer: Quantizer, device="cuda",
                 slots: torch.Tensor | None = None) -> PackedCache:
    codes = torch.zeros((rows, n_heads, 16 * bits), dtype=torch.uint8, device=device)
    if quantizer.kind == Q_SYM_RMS:
        scales = torch.zeros((rows, n_heads), dtype=torch.float16, device=device)
        zeros = None
    else:
        scales = torch.zeros((rows, n_heads, 4), dtype=torch.float16, device=device)
        zeros = torch.zeros((rows, n_heads, 4), dtype=torch.float16, device=device)
    return PackedCache(codes, scales, zeros, slots)


def _kv_args(X: torch.Tensor):
    if not X.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if X.dtype == torch.bfloat16:
        dt = BF16
    elif X.dtype == torch.float32:
        dt = F32
    else:
        raise TypeError("K/V must be bfloat16 or float32")
    if X.dim() != 3 or X.shape[2] != 128 or X.stride(2) != 1 or X.stride(1) != 128:
        raise ValueError("K/V must be [n_tokens][n_heads][128] with contiguous heads")
    stride = X.stride(0) if X.shape[0] > 1 else X.shape[1] * 128
    return dt, int(X.shape[0]), int(X.shape[1]), int(stride)


def _check_device_tensor(t: torch.Tensor | None, name: str, dtype):
    if t is None:
        return
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor")


def wushkv_quantize_keys(K: torch.Tensor, pos: torch.Tensor, rope: Rope, T_k: Transform, bits: int,
                         quantizer: Quantizer, out: PackedCache, stream=None) -> None:
    dt, n, h, stride = _kv_args(K)
    _check_device_tensor(pos, "pos", torch.int32)
    _check_device_tensor(out.slots, "slots", torch.int64)
    q = quantizer.c()
    p = out.c()
    _lib.check(library().wushkv_quantize_keys(
        ctypes.c_void_p(K.data_ptr()), dt, n, h, stride, ctypes.c_void_p(pos.data_ptr()), rope.handle,
        T_k.handle, bits, ctypes.byref(q), ctypes.byref(p), _stream(stream)))


def wushkv_quantize_values(V: torch.Tensor, bits: int, quantizer: Quantizer, out: PackedCache,
                           stream=None) -> None:
    dt, n, h, stride = _kv_args(V)
    _check_device_tensor(out.slots, "slots", torch.int64)
    q = quantizer.c()
    p = out.c()
    _lib.check(library().wushkv_quantize_values(
        ctypes.c_void_p(V.data_ptr()), dt, n, h, stride, bits, ctypes.byref(q), ctypes.byref(p),
        _stream(stream)))


def _kv_fused_args(K: torch.Tensor, V: torch.Tensor, pos: torch.Tensor, rope: Rope, T_k: Transform, bits: int,
                   quantizer: Quantizer, k_out: PackedCache, v_out: PackedCache, stream):
    dk, n, h, ks = _kv_args(K)
    dv, nv, hv, vs = _kv_args(V)
    if (dk, n, h) != (dv, nv, hv):
        raise ValueError("K and V must have the same dtype, token count and head count")
    _check_device_tensor(pos, "pos", torch.int32)
    _check_device_tensor(k_out.slots, "slots", torch.int64)
    _check_device_tensor(v_out.slots, "slots", torch.int64)
    q, pk, pv = quantizer.c(), k_out.c(), v_out.c()
    args = (ctypes.c_void_p(K.data_ptr()), ctypes.c_void_p(V.data_ptr()), dk, n, h, ks, vs,
            ctypes.c_void_p(pos.data_ptr()), rope.handle, T_k.handle, bits, ctypes.byref(q), ctypes.byref(pk),
            ctypes.byref(pv), _stream(stream))
    return args, (K, V, pos, rope, T_k, q, pk, pv, k_out, v_out)


def wushkv_quantize_kv(K: torch.Tensor, V: torch.Tensor, pos: torch.Tensor, rope: Rope, T_k: Transform, bits: int,
                       quantizer: Quantizer, k_out: PackedCache, v_out: PackedCache, stream=None) -> None:
    """Keys and values of the same tokens in one kernel (the append path)."""
    args, _keep = _kv_fused_args(K, V, pos, rope, T_k, bits, quantizer, k_out, v_out, stream)
    _lib.check(library().wushkv_quantize_kv(*args))


def wushkv_dequantize(packed: PackedCache, n_tokens: int, n_heads: int, bits: int, quantizer: Quantizer,
                      T_k_inv: Transform | None = None, out: torch.Tensor | None = None,
                      out_dtype=torch.bfloat16, stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty((n_tokens, n_heads, 128), dtype=out_dtype, device=packed.codes.device)
    if out.dtype not in (torch.float32, torch.bfloat16) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 or bfloat16 tensor")
    _check_device_tensor(packed.slots, "slots", torch.int64)
    q = quantizer.c()
    p = packed.c()
    _lib.check(library().wushkv_dequantize(
        ctypes.byref(p), n_tokens, n_heads, bits, ctypes.byref(q), None if T_k_inv is None else T_k_inv.handle,
        ctypes.c_void_p(out.data_ptr()), F32 if out.dtype == torch.float32 else BF16, _stream(stream)))
    return out


def wushkv_debug_rope_transform(K: torch.Tensor, pos: torch.Tensor, rope: Rope, T_k: Transform,
                                stream=None) -> torch.Tensor:
    dt, n, h, stride = _kv_args(K)
    _check_device_tensor(pos, "pos", torch.int32)
    y = torch.empty((n, h, 128), dtype=torch.float32, device=K.device)
    _lib.check(library().wushkv_debug_rope_transform(
        ctypes.c_void_p(K.data_ptr()), dt, n, h, stride, ctypes.c_void_p(pos.data_ptr()), rope.handle,
        T_k.handle, ctypes.c_void_p(y.data_ptr()), _stream(stream)))
    return y


def wushkv_debug_rope_cos_sin(rope: Rope, pos: torch.Tensor, stream=None) -> torch.Tensor:
    _check_device_tensor(pos, "pos", torch.int32)
    cs = torch.empty((pos.numel(), 64, 2), dtype=torch.float32, device=pos.device)
    _lib.check(library().wushkv_debug_rope_cos_sin(rope.handle, ctypes.c_void_p(pos.data_ptr()), pos.numel(),
                                                   ctypes.c_void_p(cs.data_ptr()), _stream(stream)))
    return cs


class PreparedCall:
    """A libwushkv call with its arguments marshalled once; calling it launches
    again with the same tensors and stream (for tight loops and benchmarks)."""

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st:
            _lib.check(st)


def prepare_quantize_keys(K, pos, rope: Rope, T_k: Transform, bits: int, quantizer: Quantizer,
                          out: PackedCache, stream=None) -> PreparedCall:
    dt, n, h, stride = _kv_args(K)
    _check_device_tensor(pos, "pos", torch.int32)
    q, p = quantizer.c(), out.c()
    args = (ctypes.c_void_p(K.data_ptr()), dt, n, h, stride, ctypes.c_void_p(pos.data_ptr()), rope.handle,
            T_k.handle, bits, ctypes.byref(q), ctypes.byref(p), _stream(stream))
    return PreparedCall(library().wushkv_quantize_keys, args, (K, pos, rope, T_k, q, p, out))


def prepare_quantize_values(V, bits: int, quantizer: Quantizer, out: PackedCache, stream=None) -> PreparedCall:
    dt, n, h, stride = _kv_args(V)
    q, p = quantizer.c(), out.c()
    args = (ctypes.c_void_p(V.data_ptr()), dt, n, h, stride, bits, ctypes.byref(q), ctypes.byref(p),
            _stream(stream))
    return PreparedCall(library().wushkv_quantize_values, args, (V, q, p, out))


def prepare_quantize_kv(K, V, pos, rope: Rope, T_k: Transform, bits: int, quantizer: Quantizer,
                        k_out: PackedCache, v_out: PackedCache, stream=None) -> PreparedCall:
    args, keep = _kv_fused_args(K, V, pos, rope, T_k, bits, quantizer, k_out, v_out, stream)
    return PreparedCall(library().wushkv_quantize_kv, args, keep)


def prepare_dequantize(packed: PackedCache, n_tokens: int, n_heads: int, bits: int, quantizer: Quantizer,
                       out: torch.Tensor, T_k_inv: Transform | None = None, stream=None) -> PreparedCall:
    q, p = quantizer.c(), packed.c()
    args = (ctypes.byref(p), n_tokens, n_heads, bits, ctypes.byref(q), None if T_k_inv is None else T_k_inv.handle,
            ctypes.c_void_p(out.data_ptr()), F32 if out.dtype == torch.float32 else BF16, _stream(stream))
    return PreparedCall(library().wushkv_dequantize, args, (packed, q, p, out, T_k_inv))


def wushkv_debug_time_next_launch(start: torch.cuda.Event | None, stop: torch.cuda.Event | None) -> None:
    """The next library kernel launch on this thread records `start`/`stop`
    at its kernel's start and end (events that have been recorded once, so
    that they exist)."""
    def handle(e):
        if e is None:
            return None
        if not e.cuda_event:
            raise ValueError("record the event once before passing it")
        return ctypes.c_void_p(e.cuda_event)
    _lib.check(library().wushkv_debug_time_next_launch(handle(start), handle(stop)))


def wushkv_debug_check_arith(stream=None) -> list:
    """Mismatch counts [sqrt, / 3, / 7, / 15] of the device's fp32 square root and the
    kernels' division by 2^b - 1 over all 2^32 inputs (all zero when correctly rounded)."""
    counts = torch.empty(4, dtype=torch.int32, device="cuda")
    _lib.check(library().wushkv_debug_check_arith(ctypes.c_void_p(counts.data_ptr()), _stream(stream)))
    return [int(c) for c in counts.cpu().tolist()]


def wushkv_rope_frequencies(theta: float):
    out = (ctypes.c_float * 64)()
    _lib.check(library().wushkv_rope_frequencies(ctypes.c_float(theta), out))
    return list(out)


def wushkv_pair_queries(Q: torch.Tensor, T_k_inv: Transform, out: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """Paired queries q' = bf16(T~inv^T q), bf16 [n_tokens][n_q_heads][128]."""
    dt, n, hq, stride = _kv_args(Q)
    if out is None:
        out = torch.empty((n, hq, 128), dtype=torch.bfloat16, device=Q.device)
    _check_device_tensor(out, "out", torch.bfloat16)
    _lib.check(library().wushkv_pair_queries(
        ctypes.c_void_p(Q.data_ptr()), dt, n, hq, stride, T_k_inv.handle, ctypes.c_void_p(out.data_ptr()),
        _stream(stream)))
    return out


def wushkv_decode_attention_workspace(n_seqs: int, n_q_heads: int, n_kv_heads: int, max_seq_len: int) -> int:
    b = ctypes.c_size_t()
    _lib.check(library().wushkv_decode_attention_workspace(n_seqs, n_q_heads, n_kv_heads, max_seq_len,
                                                           ctypes.byref(b)))
    return int(b.value)


def _attention_args(q_paired, k_cache, v_cache, n_kv_heads, bits, quantizer, seq_row0, seq_len, max_seq_len,
                    scale, workspace, out, stream):
    if q_paired.dim() != 3 or q_paired.shape[2] != 128:
        raise ValueError("q_paired must be [n_seqs][n_q_heads][128]")
    _check_device_tensor(q_paired, "q_paired", torch.bfloat16)
    _check_device_tensor(seq_row0, "seq_row0", torch.int64)
    _check_device_tensor(seq_len, "seq_len", torch.int32)
    n_seqs, n_q_heads = int(q_paired.shape[0]), int(q_paired.shape[1])
    if workspace is None:
        nb = wushkv_decode_attention_workspace(n_seqs, n_q_heads, n_kv_heads, max_seq_len)
        workspace = torch.empty(max(nb // 4, 4), dtype=torch.float32, device=q_paired.device)
    if out is None:
        out = torch.empty((n_seqs, n_q_heads, 128), dtype=torch.float32, device=q_paired.device)
    _check_device_tensor(out, "out", torch.float32)
    q, kp, vp_ = quantizer.c(), k_cache.c(), v_cache.c()
    args = (ctypes.c_void_p(q_paired.data_ptr()), n_seqs, n_q_heads, ctypes.byref(kp), ctypes.byref(vp_), n_kv_heads,
            bits, ctypes.byref(q), ctypes.c_void_p(seq_row0.data_ptr()), ctypes.c_void_p(seq_len.data_ptr()),
            max_seq_len, ctypes.c_float(scale), ctypes.c_void_p(workspace.data_ptr()),
            workspace.numel() * workspace.element_size(), ctypes.c_void_p(out.data_ptr()), _stream(stream))
    return args, (q_paired, k_cache, v_cache, seq_row0, seq_len, workspace, out, q, kp, vp_), out


def wushkv_decode_attention(q_paired: torch.Tensor, k_cache: PackedCache, v_cache: PackedCache, n_kv_heads: int,
                            bits: int, quantizer: Quantizer, seq_row0: torch.Tensor, seq_len: torch.Tensor,
                            max_seq_len: int, scale: float, workspace: torch.Tensor | None = None,
                            out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode attention over the packed caches; fp32 [n_seqs][n_q_heads][128]."""
    args, _keep, out = _attention_args(q_paired, k_cache, v_cache, n_kv_heads, bits, quantizer, seq_row0, seq_len,
                                       max_seq_len, scale, workspace, out, stream)
    _lib.check(library().wushkv_decode_attention(*args))
    return out


def wushkv_decode_attention_noalloc(q_paired: torch.Tensor, k_cache: PackedCache, v_cache: PackedCache,
                                    n_kv_heads: int, bits: int, quantizer: Quantizer, seq_row0: torch.Tensor,
                                    seq_len: torch.Tensor, max_seq_len: int, scale: float, out: torch.Tensor,
                                    stream=None) -> torch.Tensor:
    """Decode attention with the library's own scratch buffer (no workspace argument; the
    call allocates nothing).  `out` (fp32 [n_seqs][n_q_heads][128]) is the caller's."""
    if q_paired.dim() != 3 or q_paired.shape[2] != 128:
        raise ValueError("q_paired must be [n_seqs][n_q_heads][128]")
    for t, name, dt in ((q_paired, "q_paired", torch.bfloat16), (seq_row0, "seq_row0", torch.int64),
                        (seq_len, "seq_len", torch.int32), (out, "out", torch.float32)):
        _check_device_tensor(t, name, dt)
    q, kp, vp_ = quantizer.c(), k_cache.c(), v_cache.c()
    _lib.check(library().wushkv_decode_attention_noalloc(
        ctypes.c_void_p(q_paired.data_ptr()), int(q_paired.shape[0]), int(q_paired.shape[1]), ctypes.byref(kp),
        ctypes.byref(vp_), n_kv_heads, bits, ctypes.byref(q), ctypes.c_void_p(seq_row0.data_ptr()),
        ctypes.c_void_p(seq_len.data_ptr()), max_seq_len, ctypes.c_float(scale), ctypes.c_void_p(out.data_ptr()),
        _stream(stream)))
    return out


def prepare_decode_attention(q_paired, k_cache: PackedCache, v_cache: PackedCache, n_kv_heads: int, bits: int,
                             quantizer: Quantizer, seq_row0, seq_len, max_seq_len: int, scale: float,
                             workspace: torch.Tensor, out: torch.Tensor, stream=None) -> PreparedCall:
    args, keep, _ = _attention_args(q_paired, k_cache, v_cache, n_kv_heads, bits, quantizer, seq_row0, seq_len,
                                    max_seq_len, scale, workspace, out, stream)
    return PreparedCall(library().wushkv_decode_attention, args, keep)

