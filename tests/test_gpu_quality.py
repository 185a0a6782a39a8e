"""GPU checks of the attention-output reconstruction harness (bit_kv_cache_rope_amd.quality).

* The quality chain (quantize keys and values -> pair the queries -> attend over
  the packed caches) through the C ABI against the oracle's own chain on one
  small layer: records and paired queries as in the parity tests, attention
  outputs within the attention tolerance, and the harness's error figure the
  same from either chain.
* The harness ranks what it is built to rank, with the orderings that the
  oracle's chain shows on the same synthetic layers (worked out on the CPU with
  the oracle): per-channel-scaled Hadamard < Hadamard < identity for the
  keys-only error at 2 and 4 bits; 4 bits well below 2 bits wherever the error
  is rounding error (not for the identity, whose error is the clipping of
  outlier channels); Hadamard-rotated values well below values as stored; and a
  softmax that is neither flat nor one-hot.
"""
import numpy as np
import pytest

from test_gpu_attention import ATT_TOL
from test_gpu_parity import account_keys, assert_same_packed, env, packed_host, run_keys, run_values, say, to_dev  # noqa: F401

pytestmark = pytest.mark.gpu


def attention_f64(Q, X, V, G, scale):
    """fp64 attention: Q [n_q][H G][128], X, V [N][H][128]; query head hq reads KV head hq // G."""
    n_q, Hq = Q.shape[0], Q.shape[1]
    out = np.zeros((n_q, Hq, 128))
    for hq in range(Hq):
        h = hq // G
        s = Q[:, hq].astype(np.float64) @ X[:, h].astype(np.float64).T * scale
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, hq] = p @ V[:, h].astype(np.float64)
    return out


@pytest.mark.parametrize("bits", [2, 4])
def test_quality_chain_matches_oracle(env, bits):
    s, o, bk = env["synth"], env["oracle"], env["bk"]
    w = s.WORKLOADS["qwen3_8b_prefill"]
    H, G, n_tok, n_q = w.heads, 4, 512, 8
    K = s.kv(w, 0, "K", 0, n_tok)
    V = s.kv(w, 0, "V", 0, n_tok)
    pos = s.positions(w, 0, n_tok)
    T, Ti = s.transform(w, 0)
    rng = np.random.default_rng(700 + bits)
    Qf = o.round_bf16((rng.standard_normal((n_q, H * G, 128)) * 0.2).astype(np.float32))
    Qbits = (Qf.view(np.uint32) >> 16).astype(np.uint16)
    scale = float(1 / np.sqrt(128))
    q = bk.sym(2.0)
    row0 = np.zeros(n_q, np.int64)
    lens = np.full(n_q, n_tok, np.int32)
    say(f"quality chain {bits}-bit: {n_tok} tokens, {n_q} queries x {H * G} heads")
    # the library's chain
    kc, vc = run_keys(env, K, pos, T, bits, q), run_values(env, V, bits, q)
    qp = bk.wushkv_pair_queries(to_dev(env, Qbits), bk.Transform(Ti))
    og = bk.wushkv_decode_attention(qp, kc, vc, H, bits, q, to_dev(env, row0), to_dev(env, lens), n_tok,
                                    scale).cpu().numpy().astype(np.float64)
    # the oracle's chain
    rk = o.quantize_keys(K, pos, T, w.theta, bits, o.sym())
    rv = o.quantize_values(V, bits, o.sym())
    qpo = o.pair_queries(Qbits, Ti)
    oo = o.decode_attention(qpo, rk, rv, bits, row0, lens, scale).astype(np.float64)
    # stage by stage
    assert_same_packed(packed_host(vc), rv, "chain values")
    qpg = qp.detach().cpu().view(dtype=env["torch"].int16).numpy().view(np.uint16)
    assert np.array_equal(qpg, qpo), "paired queries differ"
    mism, _, _ = account_keys(env, K, pos, T, bits, q, f"chain keys {bits}-bit", g=packed_host(kc))
    vhat = o.dequantize(rv["codes"], rv["scales"], None, n_tok, H, bits, o.sym())
    vmax = np.abs(vhat).max(axis=(0, 2))
    if mism == 0:
        bound = ATT_TOL * vmax[np.arange(H * G) // G][None, :, None]
        assert np.all(np.abs(og - oo) <= bound), f"attention outputs differ by up to {np.abs(og - oo).max():.3e}"
    # the harness's figure from either chain, against fp64 attention over bf16(RoPE(k)) and bf16 V
    ident = np.stack([np.eye(128, dtype=np.float32)] * H)
    X = o.quantize_keys(K, pos, ident, w.theta, bits, o.sym(), want_y=True)["y"]
    Vf = (V.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    ref = attention_f64(Qf, X, Vf, G, scale)
    eg = float(((og - ref) ** 2).sum() / (ref ** 2).sum())
    eo = float(((oo - ref) ** 2).sum() / (ref ** 2).sum())
    say(f"  relative output error: library chain {eg:.6f}, oracle chain {eo:.6f}")
    assert abs(eg - eo) <= 1e-3 * eo


def test_quality_report_ranks_transforms_and_widths(env):
    from bit_kv_cache_rope_amd import quality
    s = env["synth"]
    r = {b: quality.quality_report(s, "cuda", bits=b, layers=1, n_tok=2048, n_q=16) for b in (2, 4)}
    for b in (2, 4):
        say(f"quality {b}-bit: keys {r[b]['keys_only']} values {r[b]['values_only']} joint {r[b]['joint']} "
            f"entropy {r[b]['softmax_entropy']} (effective tokens {r[b]['effective_tokens']})")
    for b in (2, 4):
        k, v, j = r[b]["keys_only"], r[b]["values_only"], r[b]["joint"]
        assert k["adaptive"] < k["hadamard"] < k["identity"]
        assert v["rotated"] < 0.5 * v["stored"]
        assert j["adaptive"] < j["identity"]
        assert 3.0 < r[b]["softmax_entropy"] < 7.5  # between ~20 and ~1800 of 2048 tokens attended
    # Through a transform that spreads the outlier channels the keys' error is rounding error,
    # and two more bits cut it by well over half; with the identity it is the clipping of the
    # outlier channels at 2 x RMS, which does not depend on the width.
    for t in ("hadamard", "T_k", "adaptive"):
        assert r[4]["keys_only"][t] < 0.5 * r[2]["keys_only"][t]
    e2, e4 = r[2]["keys_only"]["identity"], r[4]["keys_only"]["identity"]
    assert abs(e4 - e2) < 0.25 * e2
    assert r[4]["values_only"]["rotated"] < 0.5 * r[2]["values_only"]["rotated"]
