"""Attention-output reconstruction harness for the quantized cache.

Mirrors the pages' ablation metric: the relative error of a module's output,
geometric mean over layers (ai4snews summary "WUSH-KV cuts 2-bit KV-cache
perplexity ...", experiments paragraph).  Here the module is one decode
attention over a synthetic Qwen3-8B-shaped layer, with no model weights.
Everything quantized runs through the library's kernels; the unquantized
reference is fp32 attention over the bf16 RoPE'd keys and the bf16 values.

Per layer and key transform T (identity, Hadamard / 8, the workload's T_k, and a
data-adaptive transform: Hadamard / 8 times diag(1 / rms) of the layer's
RoPE'd key channels, normalised to a geometric mean of 1):
  * keys-only error: keys quantized through T and read back through T^-1
    (wushkv_dequantize), values exact;
  * joint error: the deployed path, keys quantized through T, the queries paired
    with T^-1, values quantized, attention over the packed caches
    (wushkv_decode_attention).
And per layer, for the values:
  * values-only error, values quantized as stored;
  * values-only error, values rotated by an orthonormal Hadamard before
    quantization (a value transform folded into the weights, as in the method's
    deployment paragraph) and the output rotated back.  The joint error uses these
    rotated values.

Error = |o - o_ref|^2 / |o_ref|^2 over all queries and query heads.  The
reference softmax's mean entropy (and exp of it, the effective number of
attended tokens) is reported beside the errors.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (Transform, alloc_packed, sym, wushkv_decode_attention, wushkv_debug_rope_transform,
               wushkv_dequantize, wushkv_pair_queries, wushkv_quantize_keys, wushkv_quantize_values, Rope)

D = 128


def hadamard(n: int = D) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (entries +-1)."""
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def _rel(o: torch.Tensor, ref: torch.Tensor) -> float:
    return float(((o - ref) ** 2).sum() / (ref ** 2).sum())


def attention_fp32(Q: torch.Tensor, Kh: torch.Tensor, Vh: torch.Tensor, G: int, scale: float):
    """fp32 attention: Q [n_q][H G][128], Kh, Vh [H][N][128]; query head hq reads KV head hq // G.
    Returns the output [n_q][H G][128] and the softmax's mean entropy (nats)."""
    n_q, Hq = Q.shape[0], Q.shape[1]
    H = Kh.shape[0]
    Qh = Q.float().view(n_q, H, G, D).permute(1, 0, 2, 3).reshape(H, n_q * G, D).contiguous()
    p = torch.softmax(torch.matmul(Qh, Kh.transpose(1, 2).contiguous()) * scale, dim=-1)
    ent = float(-(p * torch.log(p.clamp_min(1e-30))).sum(dim=-1).mean())
    o = torch.matmul(p, Vh).view(H, n_q, G, D).permute(1, 0, 2, 3).reshape(n_q, Hq, D)
    return o, ent


def layer_errors(synth, w, layer: int, bits: int, dev, n_tok: int, n_q: int, q_scale: float, G: int = 4) -> dict:
    H = w.heads
    q = sym(w.clip_alpha)
    rope = Rope(w.theta, 1 << 17)
    scale = 1.0 / np.sqrt(D)
    ident = np.stack([np.eye(D, dtype=np.float32)] * H)
    pos = torch.from_numpy(synth.positions(w, 0, n_tok)).to(dev)
    K = torch.from_numpy(synth.kv(w, layer, "K", 0, n_tok).view(np.int16)).to(dev).view(torch.bfloat16)
    V = torch.from_numpy(synth.kv(w, layer, "V", 0, n_tok).view(np.int16)).to(dev).view(torch.bfloat16)
    X = wushkv_debug_rope_transform(K, pos, rope, Transform(ident))  # bf16(RoPE(k)), exact in fp32
    Xh = X.permute(1, 0, 2).contiguous()
    Vf = V.float()
    Vh = Vf.permute(1, 0, 2).contiguous()
    g = torch.Generator(device=dev)
    g.manual_seed(1000 + layer)
    Qb = (torch.randn((n_q, H * G, D), device=dev, generator=g) * q_scale).to(torch.bfloat16)
    ref, ent = attention_fp32(Qb, Xh, Vh, G, scale)

    # values: as stored, and rotated by the orthonormal Hadamard R (output rotated back by R^T)
    R = torch.from_numpy(hadamard() / np.sqrt(D)).float().to(dev)
    Vr = torch.matmul(Vf.reshape(-1, D), R).reshape(n_tok, H, D).to(torch.bfloat16).contiguous()
    out = {}
    for name, Vin, back in (("values_stored", V, None), ("values_rotated", Vr, R)):
        vc = alloc_packed(n_tok, H, bits, q, dev)
        wushkv_quantize_values(Vin, bits, q, vc)
        vhat = wushkv_dequantize(vc, n_tok, H, bits, q, out_dtype=torch.float32)
        if back is not None:
            vhat = torch.matmul(vhat.reshape(-1, D), back.t().contiguous()).reshape(n_tok, H, D)
        o, _ = attention_fp32(Qb, Xh, vhat.permute(1, 0, 2).contiguous(), G, scale)
        out[name] = _rel(o, ref)
        if back is not None:
            vc_rot = vc

    # key transforms
    Hd = hadamard()
    rms = torch.sqrt((Xh.double() ** 2).mean(dim=1)).cpu().numpy()  # [H][128]
    rms = np.maximum(rms, 1e-30)
    rms = rms / np.exp(np.log(rms).mean(axis=1, keepdims=True))
    T, Ti = synth.transform(w, layer)
    transforms = {
        "identity": (ident, ident),
        "hadamard": (np.stack([Hd / 8.0] * H).astype(np.float32), np.stack([Hd / 16.0] * H).astype(np.float32)),
        "T_k": (T, Ti),
        "adaptive": (np.stack([(Hd / 8.0) / rms[h][None, :] for h in range(H)]).astype(np.float32),
                     np.stack([rms[h][:, None] * (Hd / 16.0) for h in range(H)]).astype(np.float32)),
    }
    row0 = torch.zeros(n_q, dtype=torch.int64, device=dev)
    lens = torch.full((n_q,), n_tok, dtype=torch.int32, device=dev)
    for name, (Tm, Tim) in transforms.items():
        tk, tki = Transform(Tm), Transform(Tim)
        kc = alloc_packed(n_tok, H, bits, q, dev)
        wushkv_quantize_keys(K, pos, rope, tk, bits, q, kc)
        khat = wushkv_dequantize(kc, n_tok, H, bits, q, T_k_inv=tki, out_dtype=torch.float32)
        o, _ = attention_fp32(Qb, khat.permute(1, 0, 2).contiguous(), Vh, G, scale)
        out[f"keys_{name}"] = _rel(o, ref)
        qp = wushkv_pair_queries(Qb, tki)
        oj = wushkv_decode_attention(qp, kc, vc_rot, H, bits, q, row0, lens, n_tok, scale)
        oj = torch.matmul(oj.reshape(-1, D), R.t().contiguous()).reshape(oj.shape)
        out[f"joint_{name}"] = _rel(oj, ref)
    out["entropy"] = ent
    return out


def quality_report(synth, dev, bits: int = 2, layers: int = 2, n_tok: int = 4096, n_q: int = 32,
                   q_scale: float = 0.2) -> dict:
    """Geometric means over `layers` synthetic layers of the errors above, with the
    reference softmax's mean entropy and effective number of attended tokens."""
    w = synth.WORKLOADS["qwen3_8b_prefill"]
    rows = [layer_errors(synth, w, layer, bits, dev, n_tok, n_q, q_scale) for layer in range(layers)]
    torch.cuda.synchronize()
    keys = [k for k in rows[0] if k != "entropy"]
    gm = {k: float(np.exp(np.mean(np.log([max(r[k], 1e-30) for r in rows])))) for k in keys}
    ent = float(np.mean([r["entropy"] for r in rows]))
    return {
        "bits": bits, "layers": layers, "tokens": n_tok, "queries": n_q, "query_scale": q_scale,
        "softmax_entropy": round(ent, 3), "effective_tokens": round(float(np.exp(ent)), 1),
        "keys_only": {k[5:]: round(v, 5) for k, v in gm.items() if k.startswith("keys_")},
        "values_only": {k[7:]: round(v, 5) for k, v in gm.items() if k.startswith("values_")},
        "joint": {k[6:]: round(v, 5) for k, v in gm.items() if k.startswith("joint_")},
        "note": "relative attention-output error |o - o_ref|^2 / |o_ref|^2, geometric mean over layers; "
                "joint = keys through each transform + Hadamard-rotated values, packed-cache attention; "
                "synthetic heavy-tailed keys and values, no model weights",
    }
