"""Pins for the oracle's query pairing and decode attention over the packed
cache.  Each test ties the oracle to something other than itself: closed forms
of signed-permutation transforms, exact rational sums, the textbook special
cases of softmax attention, and torch's own scaled-dot-product attention in
fp64 on the CPU.

Page references: P1 = ai4snews summary "WUSH-KV cuts 2-bit KV-cache perplexity
from OSCAR's 13.74 to 10.51 ..." (method paragraph: the key transform accounts
for the query heads that read the cached keys; deployment paragraph: keys are
cached in the transformed basis, the value transform is folded into the
weights).
"""
from fractions import Fraction as Fr

import numpy as np
import pytest
import torch

D = 128


def bf16_bits_of(x):
    """float32 -> bf16 bits by round-to-nearest-even (torch's cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_value(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def unpack_codes(rec, bits):
    """LSB-first bit stream -> codes, written out with numpy's bit unpacking."""
    b = np.unpackbits(np.asarray(rec, np.uint8), bitorder="little").reshape(D, bits)
    return (b * (1 << np.arange(bits))).sum(axis=1)


def dequant(rec, step_bits, bits):
    q = unpack_codes(rec, bits).astype(np.float64)
    step = float(np.array([step_bits], np.uint16).view(np.float16)[0])
    return (q - ((1 << bits) - 1) / 2.0) * step


def signed_perm(rng, H):
    """[H][128][128] signed permutation matrices times powers of two (exact in
    bf16), with permutations that are not their own inverse."""
    T = np.zeros((H, D, D), np.float32)
    perms, signs = [], []
    for h in range(H):
        p = np.roll(rng.permutation(D), 1)
        s = rng.choice([-1.0, 1.0], D) * 2.0 ** rng.integers(-2, 3, D)
        T[h, np.arange(D), p] = s
        perms.append(p)
        signs.append(s)
    return T, perms, signs


def random_cache(rng, rows, H, bits):
    codes = rng.integers(0, 256, (rows, H, 16 * bits), dtype=np.uint8)
    steps = np.abs(rng.standard_normal((rows, H)) * 0.05 + 0.1).astype(np.float16).view(np.uint16)
    return dict(codes=codes, scales=steps)


# ------------------------------------------------------------------ pairing (P1 method paragraph)

def test_pairing_is_the_transpose_closed_form(oracle_mod):
    rng = np.random.default_rng(11)
    Hkv, G, N = 2, 3, 4
    T, perms, signs = signed_perm(rng, Hkv)
    q = bf16_bits_of(rng.standard_normal((N, Hkv * G, D)))
    got = oracle_mod.pair_queries(q, T)
    qv = bf16_value(q)
    for n in range(N):
        for hq in range(Hkv * G):
            h = hq // G
            want = np.zeros(D, np.float32)
            # T[r][p[r]] = s[r]: q'_{p[r]} = s[r] * q_r
            want[perms[h]] = signs[h] * qv[n, hq]
            np.testing.assert_array_equal(bf16_value(got[n, hq]), want)


def test_pairing_rounds_the_exact_sum_once(oracle_mod):
    rng = np.random.default_rng(12)
    Tinv = rng.standard_normal((1, D, D)).astype(np.float32)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    got = oracle_mod.pair_queries(q, Tinv)[0, 0]
    Tb = bf16_value(bf16_bits_of(Tinv[0]))
    for j in range(0, D, 9):
        exact = sum(Fr(float(Tb[r, j])) * Fr(float(q[0, 0, r])) for r in range(D))
        f32 = np.float32(float(exact))  # nearest double; the sum is far from a double tie
        assert got[j] == bf16_bits_of(np.array([f32]))[0]


# ------------------------------------------------------------------ attention (P1 deployment paragraph)

def test_single_token_returns_its_value(oracle_mod):
    rng = np.random.default_rng(13)
    for bits in (2, 3, 4):
        k, v = random_cache(rng, 5, 2, bits), random_cache(rng, 5, 2, bits)
        qp = bf16_bits_of(rng.standard_normal((1, 4, D)))
        out = oracle_mod.decode_attention(qp, k, v, bits, np.array([3]), np.array([1]), 0.3)
        for hq in range(4):
            want = dequant(v["codes"][3, hq // 2], v["scales"][3, hq // 2], bits).astype(np.float32)
            np.testing.assert_array_equal(out[0, hq], want)


def test_zero_query_gives_the_mean(oracle_mod):
    rng = np.random.default_rng(14)
    bits, rows = 2, 40
    k, v = random_cache(rng, rows, 1, bits), random_cache(rng, rows, 1, bits)
    qp = np.zeros((1, 1, D), np.uint16)
    out = oracle_mod.decode_attention(qp, k, v, bits, np.array([5]), np.array([30]), 1.0)
    vals = np.stack([dequant(v["codes"][r, 0], v["scales"][r, 0], bits) for r in range(5, 35)])
    np.testing.assert_allclose(out[0, 0], vals.mean(axis=0).astype(np.float32), rtol=0, atol=1e-6)


def test_large_scale_picks_the_best_key(oracle_mod):
    rng = np.random.default_rng(15)
    bits, rows = 4, 64
    k, v = random_cache(rng, rows, 1, bits), random_cache(rng, rows, 1, bits)
    qp = bf16_bits_of(rng.standard_normal((1, 1, D)))
    qv = bf16_value(qp[0, 0]).astype(np.float64)
    s = np.array([qv @ dequant(k["codes"][r, 0], k["scales"][r, 0], bits) for r in range(rows)])
    best = int(np.argmax(s))
    assert np.sort(s)[-1] - np.sort(s)[-2] > 1e-3
    out = oracle_mod.decode_attention(qp, k, v, bits, np.array([0]), np.array([rows]), 1e6)
    want = dequant(v["codes"][best, 0], v["scales"][best, 0], bits).astype(np.float32)
    np.testing.assert_array_equal(out[0, 0], want)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_paired_attention_is_attention_on_the_read_path_keys(oracle_mod, bits):
    """softmax(q'.y^ s) v^ with q' = T~inv^T q equals torch's attention of q
    over k^ = T~inv y^ (exact here: signed-permutation transforms)."""
    rng = np.random.default_rng(16 + bits)
    Hkv, G, rows = 2, 4, 300
    Hq = Hkv * G
    T, _, _ = signed_perm(rng, Hkv)
    k, v = random_cache(rng, rows, Hkv, bits), random_cache(rng, rows, Hkv, bits)
    q = bf16_bits_of(rng.standard_normal((3, Hq, D)) * 0.5)
    row0, lens, scale = np.array([0, 100, 7]), np.array([100, 200, 1]), 0.125
    out = oracle_mod.decode_attention(oracle_mod.pair_queries(q, T), k, v, bits, row0, lens, scale)
    qv = bf16_value(q).astype(np.float64)
    for b in range(3):
        r = np.arange(row0[b], row0[b] + lens[b])
        for hq in range(Hq):
            h = hq // G
            Y = np.stack([dequant(k["codes"][i, h], k["scales"][i, h], bits) for i in r])
            V = np.stack([dequant(v["codes"][i, h], v["scales"][i, h], bits) for i in r])
            Kh = Y @ T[h].astype(np.float64).T  # rows k^_n = T~inv y^_n
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qv[b, hq][None, None, None]), torch.from_numpy(Kh[None, None]),
                torch.from_numpy(V[None, None]), scale=scale)[0, 0, 0].numpy()
            np.testing.assert_allclose(out[b, hq], ref.astype(np.float32), rtol=2e-7, atol=1e-7)


def test_absent_rows_and_empty_sequences(oracle_mod):
    rng = np.random.default_rng(17)
    bits, rows = 2, 50
    k, v = random_cache(rng, rows, 1, bits), random_cache(rng, rows, 1, bits)
    qp = bf16_bits_of(rng.standard_normal((3, 1, D)))
    # rows 40..59 of which 50..59 lie past the cache; rows -5..4 of which -5..-1 do
    out = oracle_mod.decode_attention(qp, k, v, bits, np.array([40, -5, 3]), np.array([20, 10, 0]), 0.2)
    cut = oracle_mod.decode_attention(qp[:2], k, v, bits, np.array([40, 0]), np.array([10, 5]), 0.2)
    np.testing.assert_array_equal(out[:2], cut)
    np.testing.assert_array_equal(out[2], np.zeros((1, D), np.float32))


# ------------------------------------------------------------------ affine caches (P1 end-to-end paragraph)

def random_affine_cache(rng, rows, H, bits):
    """Random codes with four fp16 steps (positive) and zeros per record."""
    codes = rng.integers(0, 256, (rows, H, 16 * bits), dtype=np.uint8)
    steps = np.abs(rng.standard_normal((rows, H, 4)) * 0.05 + 0.1).astype(np.float16).view(np.uint16)
    zeros = (rng.standard_normal((rows, H, 4)) * 0.3).astype(np.float16).view(np.uint16)
    return dict(codes=codes, scales=steps, zeros=zeros)


def dequant_affine(rec, steps, zeros, bits):
    """z_g + q s_g per 32-channel group g, from the fp16 bit patterns."""
    q = unpack_codes(rec, bits).astype(np.float64)
    s = np.asarray(steps, np.uint16).view(np.float16).astype(np.float64)
    z = np.asarray(zeros, np.uint16).view(np.float16).astype(np.float64)
    g = np.arange(D) // 32
    return z[g] + q * s[g]


def test_affine_single_token_returns_its_value(oracle_mod):
    rng = np.random.default_rng(23)
    for bits in (2, 3, 4):
        k, v = random_affine_cache(rng, 5, 2, bits), random_affine_cache(rng, 5, 2, bits)
        qp = bf16_bits_of(rng.standard_normal((1, 4, D)))
        out = oracle_mod.decode_attention(qp, k, v, bits, np.array([2]), np.array([1]), 0.3)
        for hq in range(4):
            h = hq // 2
            want = dequant_affine(v["codes"][2, h], v["scales"][2, h], v["zeros"][2, h], bits).astype(np.float32)
            np.testing.assert_array_equal(out[0, hq], want)


def test_affine_zero_query_gives_the_mean(oracle_mod):
    rng = np.random.default_rng(24)
    bits, rows = 3, 40
    k, v = random_affine_cache(rng, rows, 1, bits), random_affine_cache(rng, rows, 1, bits)
    qp = np.zeros((1, 1, D), np.uint16)
    out = oracle_mod.decode_attention(qp, k, v, bits, np.array([4]), np.array([30]), 1.0)
    vals = np.stack([dequant_affine(v["codes"][r, 0], v["scales"][r, 0], v["zeros"][r, 0], bits)
                     for r in range(4, 34)])
    np.testing.assert_allclose(out[0, 0], vals.mean(axis=0).astype(np.float32), rtol=0, atol=1e-6)


@pytest.mark.parametrize("bits", [2, 4])
def test_affine_attention_is_attention_on_the_dequantized_cache(oracle_mod, bits):
    """Affine keys and values: torch's fp64 attention of q over k^ = T~inv y^ and v^,
    both dequantized per 32-channel group as z + q s."""
    rng = np.random.default_rng(26 + bits)
    Hkv, G, rows = 2, 4, 200
    Hq = Hkv * G
    T, _, _ = signed_perm(rng, Hkv)
    k, v = random_affine_cache(rng, rows, Hkv, bits), random_affine_cache(rng, rows, Hkv, bits)
    q = bf16_bits_of(rng.standard_normal((2, Hq, D)) * 0.5)
    row0, lens, scale = np.array([0, 50]), np.array([120, 150]), 0.125
    out = oracle_mod.decode_attention(oracle_mod.pair_queries(q, T), k, v, bits, row0, lens, scale)
    qv = bf16_value(q).astype(np.float64)
    for b in range(2):
        r = np.arange(row0[b], row0[b] + lens[b])
        for hq in range(Hq):
            h = hq // G
            Y = np.stack([dequant_affine(k["codes"][i, h], k["scales"][i, h], k["zeros"][i, h], bits) for i in r])
            V = np.stack([dequant_affine(v["codes"][i, h], v["scales"][i, h], v["zeros"][i, h], bits) for i in r])
            Kh = Y @ T[h].astype(np.float64).T
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qv[b, hq][None, None, None]), torch.from_numpy(Kh[None, None]),
                torch.from_numpy(V[None, None]), scale=scale)[0, 0, 0].numpy()
            np.testing.assert_allclose(out[b, hq], ref.astype(np.float32), rtol=2e-7, atol=1e-7)


def test_affine_and_symmetric_caches_do_not_mix(oracle_mod):
    rng = np.random.default_rng(27)
    k = random_affine_cache(rng, 4, 1, 2)
    v = random_cache(rng, 4, 1, 2)
    with pytest.raises(ValueError):
        oracle_mod.decode_attention(np.zeros((1, 1, D), np.uint16), k, v, 2, np.array([0]), np.array([4]), 1.0)


@pytest.mark.parametrize("bits", [2, 4])
def test_paired_attention_gap_for_a_general_transform(oracle_mod, synth_mod, bits):
    """A general T_k (the decode workload's: an orthogonal factor times a
    log-normal diagonal) makes the bf16 rounding of the paired query (R34)
    inexact.  Against fp64 attention of the query itself over the read path's
    keys k^ = T~inv y^, the rounding of q' = T~inv^T q to fp32 and then bf16
    (relative error at most 2^-9 + 2^-24 per element) moves each score by at
    most B = scale * (2^-9 + 2^-24) * max_n sum_j |q'_j y^_nj|, so every
    softmax weight by a factor within exp(+-2B) and the output by at most
    (exp(2B) - 1) max|v^|.  The test checks the oracle's output against that
    bound and reports the gap it finds."""
    w = synth_mod.WORKLOADS["decode_append"]
    _, Tinv = synth_mod.transform(w, 5)
    Tb = bf16_value(bf16_bits_of(Tinv)).astype(np.float64)  # T~inv, the read path's operand
    rng = np.random.default_rng(60 + bits)
    Hkv, G, rows = 2, 4, 600
    Hq = Hkv * G
    k, v = random_cache(rng, rows, Hkv, bits), random_cache(rng, rows, Hkv, bits)
    q = bf16_bits_of(rng.standard_normal((2, Hq, D)) * 3.0)
    row0, lens, scale = np.array([0, 250]), np.array([250, 350]), 1.0 / np.sqrt(D)
    out = oracle_mod.decode_attention(oracle_mod.pair_queries(q, Tinv[:Hkv]), k, v, bits, row0, lens, scale)
    qv = bf16_value(q).astype(np.float64)
    worst = 0.0
    for b in range(2):
        r = np.arange(row0[b], row0[b] + lens[b])
        for hq in range(Hq):
            h = hq // G
            Y = np.stack([dequant(k["codes"][i, h], k["scales"][i, h], bits) for i in r])
            V = np.stack([dequant(v["codes"][i, h], v["scales"][i, h], bits) for i in r])
            qe = Tb[h].T @ qv[b, hq]              # the exact paired query
            s = (Y @ qe) * scale                  # = q . (T~inv y^) * scale
            p = np.exp(s - s.max())
            ref = (p / p.sum()) @ V
            B = scale * (2.0 ** -9 + 2.0 ** -24) * np.max(np.abs(Y) @ np.abs(qe))
            gap = np.max(np.abs(out[b, hq].astype(np.float64) - ref))
            vmax = np.max(np.abs(V))
            assert gap <= np.expm1(2 * B) * vmax + 1e-6 * vmax, (b, hq, gap, B)
            worst = max(worst, gap / vmax)
    print(f"[case] paired-query rounding, general T_k, {bits}-bit: worst gap / max|v| = {worst:.2e}")
    assert worst > 0.0  # the rounding is visible for this transform
