"""GPU parity of the query pairing and the decode attention over the packed
cache (through the C ABI) against the CPU oracle, on the same seeded inputs.

Caches are written on the CPU (random codes and fp16 steps, or the oracle's
own quantizer on synthetic keys and values) and copied to the GPU: no oracle
input comes from the GPU path.

Bars:
  * paired queries: bit-exact (both sides sum exact products in fp64 in the
    same order, then round to fp32 and bf16);
  * attention output: |o_gpu - o_ref| <= ATT_TOL * max |v^| over the
    sequence's values, per (sequence, query head).  The GPU sums the scores
    in fp32 on MFMA (with the code operand's constant part subtracted after
    the product), takes exp2 in fp32 and sums p * v in fp32; the oracle works
    in fp64.
"""
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ATT_TOL = 2e-5
D = 128


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env(oracle_mod, synth_mod):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import bit_kv_cache_rope_amd as bk
    bk.library()
    os.environ.setdefault("WUSHKV_ORACLE_THREADS", "all")
    return dict(torch=torch, bk=bk, oracle=oracle_mod, synth=synth_mod)


def to_dev(env, a):
    torch = env["torch"]
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_u16(t):
    return t.detach().cpu().view(dtype=__import__("torch").int16).numpy().view(np.uint16)


def bf16_bits(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def random_cache(rng, rows, H, bits):
    codes = rng.integers(0, 256, (rows, H, 16 * bits), dtype=np.uint8)
    steps = (np.abs(rng.standard_normal((rows, H))) * 0.05 + 0.02).astype(np.float16).view(np.uint16)
    return dict(codes=codes, scales=steps)


def dev_cache(env, c):
    bk, torch = env["bk"], env["torch"]
    z = c.get("zeros")
    return bk.PackedCache(to_dev(env, c["codes"]), to_dev(env, c["scales"]).view(torch.float16),
                          None if z is None else to_dev(env, z).view(torch.float16))


def value_max(v, bits, row0, lens, n_rows, H):
    """max |v^| over each sequence's present rows, per (sequence, KV head)."""
    L = 1 << bits
    out = np.zeros((len(lens), H))
    for b, (r0, n) in enumerate(zip(row0, lens)):
        r = np.arange(r0, r0 + max(n, 0))
        r = r[(r >= 0) & (r < n_rows)]
        if r.size == 0:
            continue
        step = v["scales"][r].view(np.float16).astype(np.float64)  # [n][H]
        out[b] = (step * (L - 1) / 2).max(axis=0)  # |(q - m) step| <= m step
    return out


def random_affine_cache(rng, rows, H, bits):
    """Random codes with four fp16 steps and zeros per record (percentile-clipped affine)."""
    codes = rng.integers(0, 256, (rows, H, 16 * bits), dtype=np.uint8)
    steps = (np.abs(rng.standard_normal((rows, H, 4))) * 0.05 + 0.02).astype(np.float16).view(np.uint16)
    zeros = (rng.standard_normal((rows, H, 4)) * 0.2).astype(np.float16).view(np.uint16)
    return dict(codes=codes, scales=steps, zeros=zeros)


def value_max_affine(v, bits, row0, lens, n_rows, H):
    """max |z + q s| over each sequence's present rows, per (sequence, KV head)."""
    L = 1 << bits
    out = np.zeros((len(lens), H))
    for b, (r0, n) in enumerate(zip(row0, lens)):
        r = np.arange(r0, r0 + max(n, 0))
        r = r[(r >= 0) & (r < n_rows)]
        if r.size == 0:
            continue
        s = v["scales"][r].view(np.float16).astype(np.float64)  # [n][H][4]
        z = v["zeros"][r].view(np.float16).astype(np.float64)
        out[b] = np.maximum(np.abs(z), np.abs(z + (L - 1) * s)).max(axis=(0, 2))
    return out


def run_attention(env, qp_bits, k, v, Hkv, bits, row0, lens, scale, max_len=None, n_rows=None, quant=None):
    bk, torch = env["bk"], env["torch"]
    max_len = int(max(lens)) if max_len is None else max_len
    kc, vc = dev_cache(env, k), dev_cache(env, v)
    out = bk.wushkv_decode_attention(to_dev(env, qp_bits), kc, vc, Hkv, bits, quant or bk.sym(),
                                     to_dev(env, np.asarray(row0, np.int64)),
                                     to_dev(env, np.asarray(lens, np.int32)), max_len, scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_attention(env, got, ref, vmax, G, what):
    B, Hq = ref.shape[0], ref.shape[1]
    worst = 0.0
    for b in range(B):
        for hq in range(Hq):
            bound = ATT_TOL * vmax[b, hq // G]
            err = float(np.max(np.abs(got[b, hq].astype(np.float64) - ref[b, hq])))
            if bound == 0.0:
                assert err == 0.0, f"{what}: sequence {b} head {hq} should be 0"
                continue
            worst = max(worst, err / vmax[b, hq // G])
            assert err <= bound, f"{what}: sequence {b} head {hq}: error {err:.3e} > {bound:.3e}"
    say(f"{what}: worst error / max|v| = {worst:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pair_queries_bit_exact(env, dtype):
    synth, oracle, bk = env["synth"], env["oracle"], env["bk"]
    w = synth.WORKLOADS["decode_append"]
    _, Tinv = synth.transform(w, 3)
    rng = np.random.default_rng(21)
    for N, Hq in ((5, 32), (1, 8), (37, 64)):
        say(f"pair_queries dtype={dtype} N={N} Hq={Hq}")
        Q = (rng.standard_normal((N, Hq, D)) * 2.0).astype(np.float32)
        Qd = bf16_bits(Q) if dtype == "bf16" else Q
        got = host_u16(bk.wushkv_pair_queries(to_dev(env, Qd), bk.Transform(Tinv)))
        np.testing.assert_array_equal(got, oracle.pair_queries(Qd, Tinv))


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_attention_matches_oracle(env, bits, G):
    oracle = env["oracle"]
    rng = np.random.default_rng(100 * bits + G)
    Hkv = 2
    Hq = G * Hkv
    # empty, one token, a partial tile, exactly one split, several splits with
    # a ragged tail, rows running past the cache, rows starting below 0
    lens = np.array([0, 1, 17, 1024, 2500, 512, 40])
    row0 = np.array([5, 9, 100, 200, 1300, 3900, -25])
    rows = 4000
    say(f"attention bits={bits} G={G} lens={lens.tolist()}")
    k, v = random_cache(rng, rows, Hkv, bits), random_cache(rng, rows, Hkv, bits)
    # queries scaled so that the softmax ranges from flat to sharply peaked
    qmag = np.array([0.5, 2.0, 8.0, 30.0, 4.0, 1.0, 3.0])[:, None, None]
    qp = bf16_bits(rng.standard_normal((len(lens), Hq, D)) * qmag)
    scale = 1.0 / np.sqrt(D)
    got = run_attention(env, qp, k, v, Hkv, bits, row0, lens, scale)
    ref = oracle.decode_attention(qp, k, v, bits, row0, lens, scale)
    check_attention(env, got, ref, value_max(v, bits, row0, lens, rows, Hkv), G, f"bits={bits} G={G}")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_attention_odd_kv_heads_and_split_edges(env, bits):
    """Three KV heads (the block map spreads heads and splits over the XCDs
    modulo the head count) with two query heads each; lengths one past, at and
    one short of split multiples (2048, 4096) and of round multiples (256,
    512)."""
    oracle = env["oracle"]
    rng = np.random.default_rng(900 + bits)
    Hkv, G = 3, 2
    lens = np.array([2049, 4096, 2047, 257, 512, 511, 4097])
    row0 = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rows = int(lens.sum())
    say(f"attention odd heads bits={bits} lens={lens.tolist()}")
    k, v = random_cache(rng, rows, Hkv, bits), random_cache(rng, rows, Hkv, bits)
    qp = bf16_bits(rng.standard_normal((len(lens), Hkv * G, D)) * 2.0)
    scale = 1.0 / np.sqrt(D)
    got = run_attention(env, qp, k, v, Hkv, bits, row0, lens, scale)
    ref = oracle.decode_attention(qp, k, v, bits, row0, lens, scale)
    check_attention(env, got, ref, value_max(v, bits, row0, lens, rows, Hkv), G, f"odd heads bits={bits}")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_attention_query_dynamic_range(env, bits):
    """Paired queries whose elements span many binades, against the oracle's
    exact scores: the symmetric-cache kernel holds the query in 20-bit fixed
    point relative to its largest element (exact within 2^-11 of it, rounded to
    2^-19 of it below), so small elements beside a large one, a query of
    bf16-tiny values (the scale exponent at its clamp) and a large query (a
    peaked softmax) are the cases where that representation shows."""
    oracle = env["oracle"]
    rng = np.random.default_rng(1300 + bits)
    Hkv, G = 2, 4
    lens = np.array([1500, 700, 2100, 64])
    row0 = np.array([0, 1600, 2400, 4600])
    rows = 4700
    k, v = random_cache(rng, rows, Hkv, bits), random_cache(rng, rows, Hkv, bits)
    B, Hq = len(lens), Hkv * G
    q = np.zeros((B, Hq, D))
    sign = lambda shape: np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    for b in range(B):
        base = b % 2  # the two KV heads see the patterns in turn
        pats = []
        pats.append(rng.standard_normal(D) * 3.0)                                     # ordinary
        x = sign(D) * 8.0 * 10.0 ** rng.uniform(-7, -1, D); x[rng.integers(D)] = 8.0   # one large, the rest small
        pats.append(x)
        x = sign(D) * 1e-5; x[rng.integers(D)] = -20.0                                 # one large, the rest tiny
        pats.append(x)
        pats.append(sign(D) * 2.0)                                                     # equal magnitudes
        pats.append(sign(D) * 16.0 * 2.0 ** -rng.uniform(0, 30, D))                    # 30 binades
        pats.append(rng.standard_normal(D) * 1e-35)                                    # bf16-tiny values
        pats.append(rng.standard_normal(D) * 40.0)                                     # large: a peaked softmax
        x = np.zeros(D); x[rng.integers(D, size=3)] = rng.standard_normal(3) * 5.0     # three nonzero entries
        pats.append(x)
        for hq in range(Hq):
            q[b, hq] = pats[(hq + 4 * base) % len(pats)]
    qp = bf16_bits(q)
    say(f"attention query dynamic range bits={bits}")
    scale = 1.0 / np.sqrt(D)
    got = run_attention(env, qp, k, v, Hkv, bits, row0, lens, scale)
    ref = oracle.decode_attention(qp, k, v, bits, row0, lens, scale)
    check_attention(env, got, ref, value_max(v, bits, row0, lens, rows, Hkv), G, f"query dynamic range bits={bits}")


def test_attention_edge_cases(env):
    oracle = env["oracle"]
    rng = np.random.default_rng(31)
    bits, Hkv, G, rows = 2, 1, 4, 3000
    k, v = random_cache(rng, rows, Hkv, bits), random_cache(rng, rows, Hkv, bits)
    qp = bf16_bits(rng.standard_normal((4, G, D)) * 4.0)
    # every row absent; lengths beyond max_seq_len (truncated to it); a zero query
    row0 = np.array([rows + 10, 0, 500, 7])
    lens = np.array([50, 2900, 2100, 64])
    qp[3] = 0
    say("attention edge cases")
    got = run_attention(env, qp, k, v, Hkv, bits, row0, lens, 0.2, max_len=2048)
    ref = oracle.decode_attention(qp, k, v, bits, row0, np.minimum(lens, 2048), 0.2)
    np.testing.assert_array_equal(got[0], 0.0)
    check_attention(env, got, ref, value_max(v, bits, row0, np.minimum(lens, 2048), rows, Hkv), G, "edge cases")
    # no sequences: a no-op
    bk, torch = env["bk"], env["torch"]
    e = torch.empty((0, G, D), dtype=torch.bfloat16, device="cuda")
    out = bk.wushkv_decode_attention(e, dev_cache(env, k), dev_cache(env, v), Hkv, bits, bk.sym(),
                                     torch.empty(0, dtype=torch.int64, device="cuda"),
                                     torch.empty(0, dtype=torch.int32, device="cuda"), 0, 0.1)
    assert out.shape == (0, G, D)


def test_attention_on_quantized_synthetic_cache(env):
    """Keys and values written by the oracle's quantizer from the synthetic
    decode workload (keys through RoPE and the transform), queries paired on
    the GPU, attention on the GPU; against the oracle's pairing and attention."""
    synth, oracle, bk = env["synth"], env["oracle"], env["bk"]
    w = synth.WORKLOADS["decode_append"]
    T, Tinv = synth.transform(w, 0)
    Hkv, G, bits = w.heads, 4, 2
    lens = np.array([1500, 3000, 700])
    N = int(lens.sum())
    q = oracle.sym(2.0)
    K = synth.kv(w, 0, "K", 0, N)
    V = synth.kv(w, 0, "V", 0, N)
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in lens])
    say(f"synthetic cache N={N}")
    k = oracle.quantize_keys(K, pos, T, w.theta, bits, q)
    v = oracle.quantize_values(V, bits, q)
    row0 = np.concatenate([[0], np.cumsum(lens)[:-1]])
    Q = bf16_bits(synth_queries(len(lens), Hkv * G))
    qp_gpu = bk.wushkv_pair_queries(to_dev(env, Q), bk.Transform(Tinv))
    qp_ref = oracle.pair_queries(Q, Tinv)
    np.testing.assert_array_equal(host_u16(qp_gpu), qp_ref)
    scale = 1.0 / np.sqrt(D)
    got = run_attention(env, qp_ref, k, v, Hkv, bits, row0, lens, scale)
    ref = oracle.decode_attention(qp_ref, k, v, bits, row0, lens, scale)
    check_attention(env, got, ref, value_max(v, bits, row0, lens, N, Hkv), G, "synthetic cache")


def synth_queries(B, Hq):
    rng = np.random.default_rng(41)
    return rng.standard_normal((B, Hq, D)) * 3.0


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_attention_decode_batch_full_size_sampled(env, bits):
    """The benchmark's launch: 64 sequences with the decode workload's lengths
    (position + 1, up to 32768), 32 query heads over 8 KV heads, caches of
    64 x 32768 rows at 2, 3 and 4 bits; the oracle checks a sample of
    sequences."""
    synth, oracle = env["synth"], env["oracle"]
    w = synth.WORKLOADS["decode_append"]
    lens = synth.positions(w).astype(np.int64) + 1
    B, Hkv, G = len(lens), w.heads, 4
    rows = w.cache_rows
    rng = np.random.default_rng(51 + bits)
    k, v = random_cache(rng, rows, Hkv, bits), random_cache(rng, rows, Hkv, bits)
    row0 = np.arange(B, dtype=np.int64) * 32768
    qp = bf16_bits(rng.standard_normal((B, Hkv * G, D)) * 3.0)
    say(f"decode batch B={B} max len={int(lens.max())} bits={bits}")
    got = run_attention(env, qp, k, v, Hkv, bits, row0, lens, 1.0 / np.sqrt(D), max_len=32768)
    pick = np.array([int(np.argmax(lens)), int(np.argmin(lens)), int(np.argsort(lens)[B // 2])])
    ref = oracle.decode_attention(qp[pick], k, v, bits, row0[pick], lens[pick], 1.0 / np.sqrt(D))
    check_attention(env, got[pick], ref, value_max(v, bits, row0[pick], lens[pick], rows, Hkv), G, f"decode batch bits={bits}")


# ---------------------------------------------------------------------------------- affine caches

@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_affine_attention_matches_oracle(env, bits, G):
    """Percentile-clipped affine caches (four steps and zeros per record): the
    same sequences as the symmetric case, against the oracle's z + q s."""
    oracle, bk = env["oracle"], env["bk"]
    rng = np.random.default_rng(700 + 10 * bits + G)
    Hkv = 2
    Hq = G * Hkv
    lens = np.array([0, 1, 17, 1024, 2500, 512, 40])
    row0 = np.array([5, 9, 100, 200, 1300, 3900, -25])
    rows = 4000
    say(f"affine attention bits={bits} G={G}")
    k, v = random_affine_cache(rng, rows, Hkv, bits), random_affine_cache(rng, rows, Hkv, bits)
    qmag = np.array([0.5, 2.0, 8.0, 30.0, 4.0, 1.0, 3.0])[:, None, None]
    qp = bf16_bits(rng.standard_normal((len(lens), Hq, D)) * qmag)
    scale = 1.0 / np.sqrt(D)
    got = run_attention(env, qp, k, v, Hkv, bits, row0, lens, scale, quant=bk.affine(1.0, 99.0))
    ref = oracle.decode_attention(qp, k, v, bits, row0, lens, scale)
    check_attention(env, got, ref, value_max_affine(v, bits, row0, lens, rows, Hkv), G, f"affine bits={bits} G={G}")


def test_affine_attention_on_quantized_synthetic_cache(env):
    """An affine cache that the oracle's own quantizer wrote from synthetic keys
    (through RoPE and the workload's transform) and values, read with queries
    paired through the inverse transform; also at general percentiles."""
    s, oracle, bk = env["synth"], env["oracle"], env["bk"]
    w = s.WORKLOADS["affine_pct"]
    n, H, G = 3000, w.heads, 4
    K, V = s.kv(w, 0, "K", 0, n), s.kv(w, 0, "V", 0, n)
    pos = s.positions(w, 0, n)
    T, Ti = s.transform(w, 0)
    rng = np.random.default_rng(771)
    Q = (rng.standard_normal((3, H * G, D)) * 0.3).astype(np.float32)
    qp = oracle.pair_queries(Q, Ti)
    row0, lens = np.array([0, 700, 2999]), np.array([3000, 1500, 1])
    for plo, phi, bits in ((1.0, 99.0, 2), (5.0, 95.0, 4)):
        say(f"affine synthetic cache {plo}/{phi} {bits}-bit")
        q = oracle.affine(plo, phi)
        k = oracle.quantize_keys(K, pos, T, w.theta, bits, q)
        v = oracle.quantize_values(V, bits, q)
        got = run_attention(env, qp, k, v, H, bits, row0, lens, 0.1, quant=bk.affine(plo, phi))
        ref = oracle.decode_attention(qp, k, v, bits, row0, lens, 0.1)
        check_attention(env, got, ref, value_max_affine(v, bits, row0, lens, n, H), G, f"affine synthetic {bits}-bit")
