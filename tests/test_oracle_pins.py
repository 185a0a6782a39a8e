"""Pins for the CPU oracle: each test ties an oracle function to something other
than the oracle itself -- hand-derived bytes, exact rational brute force,
high-precision library evaluation, closed forms and invariants.

Page references: P1 = ai4snews summary "WUSH-KV cuts 2-bit KV-cache perplexity
from OSCAR's 13.74 to 10.51 ..."; P2 = cere-bro post "WUSH-KV: 2-bit KV-Cache
Quantization with Data-Adaptive Transforms"; P3 = the arXiv abstract.
"""
import json
import os
from fractions import Fraction as Fr

import mpmath
import numpy as np
import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def f16val(h):
    return float(np.array([h], dtype=np.uint16).view(np.float16)[0])


def nearest_even(x, levels):
    """Exact argmin_q |x - levels[q]| over Fractions; ties go to the even q."""
    xf = Fr(float(x))
    d = [abs(xf - lv) for lv in levels]
    best = min(d)
    cands = [q for q, v in enumerate(d) if v == best]
    ev = [q for q in cands if q % 2 == 0]
    assert len(cands) <= 2
    return ev[0] if ev else cands[0]


# ---------------------------------------------------------------- packing (P1 headline: 2-bit cache)

def test_pack_hand_bytes(oracle_mod):
    for case in GOLD["pack"]:
        q = np.zeros(128, np.uint8)
        pre = case["codes_prefix"]
        q[:len(pre)] = pre
        rec = oracle_mod.pack(q, case["bits"])
        exp = bytes.fromhex(case["bytes_prefix_hex"])
        assert rec[:len(exp)].tobytes() == exp, case["work"]
        assert not rec[len(exp):].any()
        assert rec.size == 16 * case["bits"]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_is_lsb_first_bitstream(oracle_mod, bits):
    """Reduction to numpy.packbits(bitorder='little') on the stream whose bit
    b*j + t is bit t of code j."""
    rng = np.random.default_rng(bits)
    for _ in range(50):
        q = rng.integers(0, 1 << bits, 128).astype(np.uint8)
        stream = ((q[:, None] >> np.arange(bits)[None, :]) & 1).astype(np.uint8).reshape(-1)
        ref = np.packbits(stream, bitorder="little")
        assert np.array_equal(oracle_mod.pack(q, bits), ref)
        assert np.array_equal(oracle_mod.unpack(ref, bits), q)


# ---------------------------------------------------------------- number formats

def test_bf16_rounding_matches_torch(oracle_mod):
    import torch
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(-8, 8, 200000)
    # values at, and one fp32 ulp either side of, bf16 rounding midpoints
    base = (rng.integers(0, 1 << 15, 20000).astype(np.uint32) << 16) | 0x8000
    mids = base.view(np.float32)
    mids = mids[np.isfinite(mids)]
    near = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))])
    near = near[np.isfinite(near)]
    for arr in (x.astype(np.float32), near.astype(np.float32)):
        ref = torch.from_numpy(arr).to(torch.bfloat16).to(torch.float32).numpy()
        got = oracle_mod.round_bf16(arr)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_f16_conversion_matches_numpy(oracle_mod):
    rng = np.random.default_rng(2)
    allh = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    fin = np.isfinite(allh.view(np.float16))
    vals = allh[fin].view(np.float16).astype(np.float32)
    # decode of every finite fp16 pattern
    dec = np.array([oracle_mod.f16_to_f32(int(h)) for h in allh[fin][::7]], dtype=np.float32)
    assert np.array_equal(dec.view(np.uint32), vals[::7].view(np.uint32))
    # encode at fp16 values, at midpoints between neighbours, and 1-2 fp32 ulp around them
    pos = np.sort(vals[vals >= 0])
    mids = ((pos[:-1].astype(np.float64) + pos[1:].astype(np.float64)) / 2).astype(np.float32)
    cand = [pos, mids]
    for k in (1, 2):
        up, dn = mids.copy(), mids.copy()
        for _ in range(k):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(-np.inf))
        cand += [up, dn]
    cand.append(np.abs(rng.standard_normal(300000).astype(np.float32)) * np.float32(2.0) ** rng.integers(-30, 17, 300000).astype(np.float32))
    x = np.concatenate(cand).astype(np.float32)
    x = np.concatenate([x, -x])
    inrange = np.abs(x) < 65520.0
    got = oracle_mod.f32_to_f16_bits(x)
    ref = x[inrange].astype(np.float16).view(np.uint16)
    assert np.array_equal(got[inrange], ref)
    # beyond the fp16 range: saturate (numpy would give inf)
    assert np.all(got[~inrange] & 0x7FFF == 0x7BFF)


# ---------------------------------------------------------------- RoPE (P1 deployment: transform after RoPE)

@pytest.mark.parametrize("theta", [1e6, 1e4, 5e5])
def test_omega_against_high_precision(oracle_mod, theta):
    mpmath.mp.dps = 60
    for i in range(64):
        ref = np.float32(float(mpmath.mpf(theta) ** (-mpmath.mpf(2 * i) / 128)))
        assert np.float32(oracle_mod.omega(theta, i)) == ref, i
    if theta == 1e6:
        assert oracle_mod.omega(theta, 0) == 1.0
        assert np.float32(oracle_mod.omega(theta, 32)) == np.float32(1e-3)


def test_cos_sin_against_high_precision(oracle_mod):
    mpmath.mp.dps = 60
    rng = np.random.default_rng(3)
    pos = np.concatenate([[0, 1, 2, 255, 1023, 1024, 32767, 131071, (1 << 24) - 1],
                          rng.integers(0, 1 << 24, 40), rng.integers(0, 32768, 40)]).astype(np.int32)
    cs = oracle_mod.cos_sin(1e6, pos)
    assert cs[0, :, 0].tolist() == [1.0] * 64 and cs[0, :, 1].tolist() == [0.0] * 64
    bad = 0
    for t, p in enumerate(pos):
        for i in range(64):
            ang = mpmath.mpf(int(p)) * mpmath.mpf(float(np.float32(oracle_mod.omega(1e6, i))))
            for k, f in enumerate((mpmath.cos, mpmath.sin)):
                v = f(ang)
                ref = np.float32(float(v))
                if cs[t, i, k] != ref:
                    bad += 1
    assert bad == 0


def _rot_ref(k, pos, theta):
    """Rotate-half RoPE in fp64 from its textbook form (pairs i, i+64)."""
    i = np.arange(64)
    w = np.float64(np.float32(np.power(np.float64(theta), -2.0 * i / 128.0)))
    c, s = np.cos(pos * w), np.sin(pos * w)
    k = k.astype(np.float64)
    return np.concatenate([k[:64] * c - k[64:] * s, k[64:] * c + k[:64] * s])


def test_rope_properties(oracle_mod):
    rng = np.random.default_rng(4)
    for trial in range(200):
        k = (rng.standard_normal(128) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        p = int(rng.integers(0, 1 << 20))
        x = oracle_mod.rope(k, p, 1e6)
        if trial == 0:
            assert np.array_equal(oracle_mod.rope(k, 0, 1e6), k)  # pos 0 is the identity
        ref = _rot_ref(k, p, 1e6)
        scale = np.abs(k).max()
        assert np.max(np.abs(x - ref)) <= 2e-6 * scale
        assert abs(np.linalg.norm(x.astype(np.float64)) - np.linalg.norm(k.astype(np.float64))) <= 1e-6 * np.linalg.norm(k)
    # relative position: <R_m q, R_n k> = <R_{m-n} q, k>
    for _ in range(50):
        q = rng.standard_normal(128).astype(np.float32)
        k = rng.standard_normal(128).astype(np.float32)
        m, n = sorted(rng.integers(0, 30000, 2))[::-1]
        a = np.dot(oracle_mod.rope(q, int(m), 1e6).astype(np.float64), oracle_mod.rope(k, int(n), 1e6))
        b = np.dot(oracle_mod.rope(q, int(m - n), 1e6).astype(np.float64), k.astype(np.float64))
        assert abs(a - b) <= 1e-5 * np.linalg.norm(q) * np.linalg.norm(k)


# ---------------------------------------------------------------- key transform (P1 method: general invertible T_k)

def _keys(oracle_mod, K, pos, T, bits=2, q=None, theta=1e6):
    q = q or oracle_mod.sym()
    return oracle_mod.quantize_keys(K, pos, T, theta, bits, q, want_y=True, threads=2)


def test_transform_special_cases_exact(oracle_mod):
    rng = np.random.default_rng(5)
    N, H = 16, 2
    K = rng.standard_normal((N, H, 128)).astype(np.float32) * 3
    pos = np.zeros(N, np.int32)  # RoPE is the identity at position 0
    xt = oracle_mod.round_bf16(K)
    eye = np.stack([np.eye(128, dtype=np.float32)] * H)
    assert np.array_equal(_keys(oracle_mod, K, pos, eye)["y"], xt)
    perm = rng.permutation(128)
    P = np.zeros((128, 128), np.float32)
    P[np.arange(128), perm] = 1.0  # y_r = x_perm[r]
    y = _keys(oracle_mod, K, pos, np.stack([P] * H))["y"]
    assert np.array_equal(y, xt[:, :, perm])
    d = (2.0 ** rng.integers(-4, 5, 128) * rng.choice([-1, 1], 128)).astype(np.float32)
    y = _keys(oracle_mod, K, pos, np.stack([np.diag(d)] * H))["y"]
    assert np.array_equal(y, xt * d)


def test_transform_matches_fp64_matmul(oracle_mod, synth_mod):
    w = synth_mod.WORKLOADS["tiny"]
    T, _ = synth_mod.transform(w, 0)
    K = synth_mod.kv(w, 0, "K", 0, 64)
    pos = synth_mod.positions(w, 0, 64)
    y = _keys(oracle_mod, K, pos, T)["y"]
    Tt = oracle_mod.round_bf16(T).astype(np.float64)
    for n in range(64):
        x = oracle_mod.round_bf16(np.stack([oracle_mod.rope(K[n, h], pos[n], 1e6) for h in range(2)]))
        for h in range(2):
            ref = Tt[h] @ x[h].astype(np.float64)
            ulp = np.spacing(np.abs(ref).astype(np.float32))
            assert np.all(np.abs(y[n, h] - ref) <= ulp)


def test_identity_transform_reduces_to_plain_quantizer(oracle_mod, synth_mod):
    """Keys with T = I quantize exactly like values fed bf16(RoPE(K))."""
    w = synth_mod.WORKLOADS["qwen3_8b_prefill"]
    K = synth_mod.kv(w, 0, "K", 1000, 64)
    pos = synth_mod.positions(w, 1000, 64)
    H = K.shape[1]
    eye = np.stack([np.eye(128, dtype=np.float32)] * H)
    for bits, q in ((2, oracle_mod.sym()), (3, oracle_mod.sym()), (2, oracle_mod.affine())):
        rk = oracle_mod.quantize_keys(K, pos, eye, 1e6, bits, q, threads=2)
        Kf = synth_mod.bf16_bits_to_f32(K)
        X = np.stack([[oracle_mod.rope(Kf[n, h], pos[n], 1e6) for h in range(H)] for n in range(64)])
        rv = oracle_mod.quantize_values(oracle_mod.round_bf16(X), bits, q, threads=2)
        for key in ("codes", "scales", "zeros"):
            if rk[key] is not None:
                assert np.array_equal(rk[key], rv[key])


def test_query_pairing_preserves_qk(oracle_mod, synth_mod):
    """(T~^{-T} q) . (T~ x~) = q . x~ before quantization (P1 method paragraph:
    the key transform is built with the query heads that read the keys in view)."""
    w = synth_mod.WORKLOADS["qwen3_8b_prefill"]
    T, _ = synth_mod.transform(w, 0)
    rng = np.random.default_rng(6)
    for h in range(4):
        Tt = oracle_mod.round_bf16(T[h]).astype(np.float64)
        cond = np.linalg.cond(Tt)
        for _ in range(20):
            x = oracle_mod.round_bf16(rng.standard_normal(128).astype(np.float32) * 5).astype(np.float64)
            q = rng.standard_normal(128)
            qp = oracle_mod.query_pair(T[h], q)
            y = oracle_mod.transform_f64(T[h], x)
            assert abs(qp @ y - q @ x) <= 1e-12 * np.linalg.norm(q) * np.linalg.norm(x) * cond
            ref = np.linalg.solve(Tt.T, q)
            assert np.max(np.abs(qp - ref)) <= 1e-10 * np.max(np.abs(ref)) * cond
            assert np.array_equal(y, y)  # finite


# ---------------------------------------------------------------- symmetric quantizer (P3: clipped quantizers)

def _sym_levels(delta, bits):
    L = 1 << bits
    return [(Fr(q) - Fr(L - 1, 2)) * Fr(delta) for q in range(L)]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_sym_codes_brute_force(oracle_mod, bits):
    rng = np.random.default_rng(10 + bits)
    L = 1 << bits
    for trial in range(300):
        kind = trial % 3
        if kind == 0:
            y = rng.standard_normal(128)
        elif kind == 1:
            y = rng.standard_t(3, 128) * np.exp(rng.standard_normal(128))
        else:
            y = rng.standard_normal(128)
            y[rng.integers(0, 128, 4)] *= 20
        y = (y * 10.0 ** rng.uniform(-6, 4)).astype(np.float32)
        q, sc = oracle_mod.sym_quantize(y, bits)
        lv = _sym_levels(f16val(sc), bits)
        assert all(q[j] == nearest_even(y[j], lv) for j in range(128))
    # ties: entries placed exactly on midpoints (fixed point on the step)
    for trial in range(100):
        y = (rng.standard_normal(128) * 3).astype(np.float32)
        for _ in range(20):
            _, sc = oracle_mod.sym_quantize(y, bits)
            d = f16val(sc)
            ks = rng.integers(0, L - 1, 16)
            y2 = y.copy()
            y2[:16] = ((ks + 1 - L // 2) * d).astype(np.float32)
            _, sc2 = oracle_mod.sym_quantize(y2, bits)
            y = y2
            if sc2 == sc:
                break
        q, sc = oracle_mod.sym_quantize(y, bits)
        lv = _sym_levels(f16val(sc), bits)
        assert all(q[j] == nearest_even(y[j], lv) for j in range(128))


@pytest.mark.parametrize("bits,a,code", [(2, 0.75, 2), (3, 1.75, 5), (4, 3.75, 11)])
def test_sym_scale_closed_form_exact(oracle_mod, bits, a, code):
    """Constant vector a: RMS = |a|, C = 2|a|, step 2C/(2^b-1) = 1 exactly.
    a/step = (L-1)/4 lies between levels; the nearest level is (L-1)/4 rounded
    to the half-integer grid, i.e. code m + 0.5 (resp. its mirror for -a)."""
    L = 1 << bits
    for sgn in (1, -1):
        q, sc = oracle_mod.sym_quantize(np.full(128, sgn * a, np.float32), bits)
        assert sc == 0x3C00
        assert np.all(q == (code if sgn > 0 else L - 1 - code))


def test_sym_scale_within_rounding_bound(oracle_mod):
    """Step within half an fp16 ulp (plus the fp32 sequence error) of
    2 * alpha * RMS / (2^b - 1) evaluated exactly."""
    rng = np.random.default_rng(20)
    mpmath.mp.dps = 40
    for trial in range(400):
        bits = int(rng.integers(2, 5))
        alpha = float(np.float32(rng.choice([2.0, 1.5, 3.0])))
        y = (rng.standard_normal(128) * 10.0 ** rng.uniform(-4, 3)).astype(np.float32)
        if trial % 5 == 0:
            y = np.zeros(128, np.float32)
            y[rng.integers(0, 128)] = np.float32(rng.uniform(0.1, 100))  # one-hot
        _, sc = oracle_mod.sym_quantize(y, bits, alpha)
        ms = sum(mpmath.mpf(float(v)) ** 2 for v in y) / 128
        exact = 2 * alpha * mpmath.sqrt(ms) / ((1 << bits) - 1)
        got = f16val(sc)
        ulp16 = float(np.spacing(np.float16(got)))
        assert abs(got - float(exact)) <= 0.5 * ulp16 + 1e-6 * float(exact)


def golden_vector(spec):
    """128 fp32 values from a golden case's spec: {"fill", "set": [[index, hex]]}
    or {"runs": [[[hex, ...], repeat], ...]} (hex = the fp32 bit pattern)."""
    h = lambda x: np.array([int(x, 16)], np.uint32).view(np.float32)[0]
    if "runs" in spec:
        y = np.array([h(x) for run, rep in spec["runs"] for _ in range(rep) for x in run], np.float32)
    else:
        y = np.full(128, h(spec["fill"]), np.float32)
        for i, x in spec.get("set", []):
            y[i] = h(x)
    assert y.shape == (128,)
    return y


def test_golden_pairwise_sum(oracle_mod):
    """The contiguous pairwise fp32 tree of the RMS (the reading of 'clip =
    2.0*RMS per 128-vector'), worked by hand on a vector where it differs from
    a sequential sum, a stride-64 butterfly and the exactly rounded sum."""
    for case in GOLD["pairwise_sum"]:
        t = golden_vector(case["terms_f32_hex"])
        got = np.array([oracle_mod.pairwise_sum(t)], np.float32).view(np.uint32)[0]
        assert got == int(case["S_hex"], 16), case["work"]
        assert all(int(v, 16) != got for v in case["other_orders_hex"].values())


def test_golden_sym_cases(oracle_mod):
    for case in GOLD["sym"]:
        y = np.zeros(128, np.float32)
        if "y_f32_hex" in case:
            y = golden_vector(case["y_f32_hex"])
        elif case["y_pattern"].startswith("alternating"):
            y[0::2], y[1::2] = 1.0, -1.0
        elif case["y_pattern"].startswith("y[0] = 2"):
            y[0], y[1] = 2.0, -2.0
        q, sc = oracle_mod.sym_quantize(y, case["bits"], case["alpha"])
        assert sc == int(case["scale_f16_hex"], 16), case["work"]
        rec = oracle_mod.pack(q, case["bits"])
        if "record_hex" in case:
            assert rec.tobytes().hex() == case["record_hex"]
        else:
            assert rec.tobytes().hex() == case["record_hex_each_byte"] * (16 * case["bits"])
        if "delta" in case:
            assert f16val(sc) == case["delta"]


# ---------------------------------------------------------------- affine percentile quantizer (P1 end-to-end)

def test_percentile_matches_numpy(oracle_mod):
    rng = np.random.default_rng(30)
    for trial in range(500):
        x = (rng.standard_normal(32) * np.exp(rng.standard_normal())).astype(np.float32)
        if trial % 4 == 0:
            x[rng.integers(0, 32, 8)] = x[0]  # duplicates
        s = np.sort(x)
        for p in (0.0, 1.0, 2.5, 50.0, 97.0, 99.0, 100.0):
            got = oracle_mod.percentile32(s, p)
            ref = np.percentile(s.astype(np.float64), p, method="linear")
            # fp32 interpolation: within 2 ulp of the larger bracketing order statistic
            i = min(int(np.floor(31 * p / 100)), 30)
            mag = np.float32(max(abs(s[i]), abs(s[i + 1]), abs(ref)))
            assert abs(got - ref) <= 2 * float(np.spacing(mag))
        assert oracle_mod.percentile32(s, 0.0) == s[0]
        assert oracle_mod.percentile32(s, 100.0) == s[31]


def _affine_levels(s, z, bits):
    return [Fr(z) + q * Fr(s) for q in range(1 << bits)]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_affine_brute_force(oracle_mod, bits):
    rng = np.random.default_rng(40 + bits)
    for trial in range(400):
        x = (rng.standard_normal(32) * np.exp(rng.standard_normal()) + rng.standard_normal()).astype(np.float32)
        if trial % 5 == 0:
            x[rng.integers(0, 32, 6)] = np.float32(-0.0) if trial % 2 else np.float32(0.0)
        q, sh, zh = oracle_mod.affine_quantize_group(x, bits)
        s, z = f16val(sh), f16val(zh)
        # the stored zero and step are the fp16 roundings of the percentiles' values
        lo = np.percentile(x.astype(np.float64), 1.0, method="linear")
        hi = np.percentile(x.astype(np.float64), 99.0, method="linear")
        assert abs(z - lo) <= float(np.spacing(np.float16(abs(lo)))) + 1e-6 * abs(lo) + 1e-7
        assert abs(s - (hi - lo) / ((1 << bits) - 1)) <= float(np.spacing(np.float16(s))) + 1e-6 * (hi - lo) + 1e-7
        if s == 0.0:
            assert np.all(q == 0)
            continue
        lv = _affine_levels(s, z, bits)
        assert all(q[j] == nearest_even(x[j], lv) for j in range(32))
    # ties: extremes pinned (s0 = s1 = A, s30 = s31 = B), middle entries on midpoints
    L = 1 << bits
    for trial in range(200):
        A = float(np.float16(rng.uniform(-8, 0)))
        B = float(np.float16(A + rng.uniform(0.5, 16)))
        x = np.full(32, (A + B) / 2, np.float32)
        x[:2], x[2:4] = A, B
        _, sh, zh = oracle_mod.affine_quantize_group(x, bits)
        s, z = f16val(sh), f16val(zh)
        ks = rng.integers(0, L - 1, 28)
        mids = z + (ks + 0.5) * s
        keep = (mids > A) & (mids < B) & (mids == mids.astype(np.float32))
        x[4:][keep] = mids[keep]
        q, sh2, zh2 = oracle_mod.affine_quantize_group(x, bits)
        assert (sh2, zh2) == (sh, zh)
        lv = _affine_levels(s, z, bits)
        assert all(q[j] == nearest_even(x[j], lv) for j in range(32))


def test_golden_affine_case(oracle_mod):
    for case in GOLD["affine"]:
        x = np.array(case["x"], np.float32)
        q, sh, zh = oracle_mod.affine_quantize_group(x, case["bits"], case["p_lo"], case["p_hi"])
        assert sh == int(case["scale_f16_hex"], 16) and zh == int(case["zero_f16_hex"], 16), case["work"]
        assert q.tolist() == case["codes"]
        codes = np.zeros(128, np.uint8)
        codes[:32] = q
        assert oracle_mod.pack(codes, case["bits"])[:8].tobytes().hex() == case["record_hex"]


# ---------------------------------------------------------------- read path

def test_golden_dequant_cases(oracle_mod):
    for case in GOLD["dequant"]:
        bits = case["bits"]
        q = np.full(128, case["code"], np.uint8)
        rec = oracle_mod.pack(q, bits)[None, None, :]
        if "zero_f16_hex" in case:
            sc = np.full((1, 1, 4), int(case["scale_f16_hex"], 16), np.uint16)
            zr = np.full((1, 1, 4), int(case["zero_f16_hex"], 16), np.uint16)
            out = oracle_mod.dequantize(rec, sc, zr, 1, 1, bits, oracle_mod.affine())
        else:
            sc = np.full((1, 1), int(case["scale_f16_hex"], 16), np.uint16)
            out = oracle_mod.dequantize(rec, sc, None, 1, 1, bits, oracle_mod.sym())
        assert np.all(out == case["value"]), case["work"]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_dequant_exact_and_error_bound(oracle_mod, bits):
    rng = np.random.default_rng(50 + bits)
    N, H = 32, 2
    V = (rng.standard_normal((N, H, 128)) * 4).astype(np.float32)
    for q in (oracle_mod.sym(), oracle_mod.affine()):
        r = oracle_mod.quantize_values(V, bits, q)
        out = oracle_mod.dequantize(r["codes"], r["scales"], r["zeros"], N, H, bits, q)
        L = 1 << bits
        for n in range(0, N, 7):
            for h in range(H):
                codes = oracle_mod.unpack(r["codes"][n, h], bits)
                for j in range(0, 128, 5):
                    if q.kind == 0:
                        d = f16val(r["scales"][n, h])
                        exact = (Fr(int(codes[j])) - Fr(L - 1, 2)) * Fr(d)
                        assert Fr(float(out[n, h, j])) == exact
                        if abs(V[n, h, j]) <= (L - 1) / 2 * d:
                            assert abs(Fr(float(V[n, h, j])) - exact) <= Fr(d) / 2
                    else:
                        g = j // 32
                        s, z = f16val(r["scales"][n, h, g]), f16val(r["zeros"][n, h, g])
                        exact = Fr(z) + int(codes[j]) * Fr(s)
                        got = Fr(float(out[n, h, j]))
                        ulp = Fr(float(np.spacing(np.float32(abs(float(exact))))))
                        assert abs(got - exact) <= ulp / 2
                        if z <= V[n, h, j] <= z + (L - 1) * s:
                            assert abs(Fr(float(V[n, h, j])) - exact) <= Fr(s) / 2 + ulp


def test_dequant_inverse_transform_matches_fp64(oracle_mod, synth_mod):
    w = synth_mod.WORKLOADS["tiny"]
    _, Ti = synth_mod.transform(w, 0)
    rng = np.random.default_rng(60)
    N, H = 8, 2
    V = (rng.standard_normal((N, H, 128)) * 2).astype(np.float32)
    for bits, q in ((3, oracle_mod.sym()), (2, oracle_mod.affine())):
        r = oracle_mod.quantize_values(V, bits, q)
        plain = oracle_mod.dequantize(r["codes"], r["scales"], r["zeros"], N, H, bits, q)
        k = oracle_mod.dequantize(r["codes"], r["scales"], r["zeros"], N, H, bits, q, Tinv=Ti)
        Tt = oracle_mod.round_bf16(Ti).astype(np.float64)
        for n in range(N):
            for h in range(H):
                ref = Tt[h] @ plain[n, h].astype(np.float64)
                assert np.all(np.abs(k[n, h] - ref) <= np.spacing(np.abs(ref).astype(np.float32)))


def test_slot_placement(oracle_mod):
    rng = np.random.default_rng(70)
    N, H, rows = 24, 3, 100
    V = rng.standard_normal((N, H, 128)).astype(np.float32)
    slots = rng.choice(rows, N, replace=False).astype(np.int64)
    dense = oracle_mod.quantize_values(V, 2, oracle_mod.sym())
    sl = oracle_mod.quantize_values(V, 2, oracle_mod.sym(), slots=slots, rows=rows)
    assert np.array_equal(sl["codes"][slots], dense["codes"])
    assert np.array_equal(sl["scales"][slots], dense["scales"])
    untouched = np.setdiff1d(np.arange(rows), slots)
    assert not sl["codes"][untouched].any()
    back = oracle_mod.dequantize(sl["codes"], sl["scales"], None, N, H, 2, oracle_mod.sym(), slots=slots)
    ref = oracle_mod.dequantize(dense["codes"], dense["scales"], None, N, H, 2, oracle_mod.sym())
    assert np.array_equal(back, ref)


def test_zero_and_empty(oracle_mod):
    V = np.zeros((3, 2, 128), np.float32)
    r = oracle_mod.quantize_values(V, 2, oracle_mod.sym())
    assert np.all(r["codes"] == 0xAA) and not r["scales"].any()
    r = oracle_mod.quantize_values(V, 4, oracle_mod.affine())
    assert not r["codes"].any() and not r["scales"].any()
    e = oracle_mod.quantize_values(np.zeros((0, 2, 128), np.float32), 2, oracle_mod.sym())
    assert e["codes"].shape[0] == 0
