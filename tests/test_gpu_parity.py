"""GPU parity: libwushkv (through the C ABI) against the CPU oracle on the same
seeded inputs.

Bars (the numerical contract of the write/read path):
  * cos/sin, RoPE operands, the quantizer fed a given fp32 tensor, packing,
    values end to end, plain dequantization: bit-exact;
  * transform y = T~ bf16(RoPE(k)): max |y_gpu - y_ref| <= 1e-5 * max |y_ref| per
    128-vector (fp32 accumulation on MFMA against an fp64 sum);
  * keys end to end: codes may differ only where the GPU's and the oracle's y
    fall on different sides of a decision midpoint, or where the step / zero
    crosses an fp16 rounding boundary; mismatches <= 1e-5 of elements;
  * dequantization through T_k^-1: within 1e-5 * max |k^_ref| per vector.
"""
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

TRANSFORM_TOL = 1e-5
MISMATCH_RATE = 1e-5


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


def oracle_q(env, q):
    o = env["oracle"]
    return o.sym(q.clip_alpha) if q.kind == 0 else o.affine(q.p_lo, q.p_hi)


def run_keys(env, K, pos, T, bits, q, theta=1e6, max_pos=1 << 17, slots=None, rows=None):
    bk = env["bk"]
    torch = env["torch"]
    N, H = K.shape[0], K.shape[1]
    rows = rows if rows is not None else N
    rope = bk.Rope(theta, max_pos)
    tk = bk.Transform(T)
    out = bk.alloc_packed(rows, H, bits, q)
    if slots is not None:
        out = out.with_slots(to_dev(env, slots))
    bk.wushkv_quantize_keys(to_dev(env, K), to_dev(env, pos), rope, tk, bits, q, out)
    torch.cuda.synchronize()
    return out


def run_values(env, V, bits, q, slots=None, rows=None):
    bk = env["bk"]
    N, H = V.shape[0], V.shape[1]
    rows = rows if rows is not None else N
    out = bk.alloc_packed(rows, H, bits, q)
    if slots is not None:
        out = out.with_slots(to_dev(env, slots))
    bk.wushkv_quantize_values(to_dev(env, V), bits, q, out)
    env["torch"].cuda.synchronize()
    return out


def dev_packed(env, h):
    """A GPU cache holding the records of an oracle result (codes, scales, zeros)."""
    torch, bk = env["torch"], env["bk"]
    f16 = lambda a: None if a is None else to_dev(env, np.ascontiguousarray(a, np.uint16)).view(torch.float16)
    return bk.PackedCache(to_dev(env, np.ascontiguousarray(h["codes"])), f16(h["scales"]), f16(h["zeros"]))


def packed_host(p):
    return dict(codes=p.codes.cpu().numpy(), scales=host_u16(p.scales),
                zeros=None if p.zeros is None else host_u16(p.zeros))


def assert_same_packed(g, r, what):
    for k in ("codes", "scales", "zeros"):
        if r[k] is None:
            continue
        bad = np.argwhere(g[k] != r[k])
        assert bad.size == 0, f"{what}: {k} differ at {bad[:5].tolist()} (total {len(bad)})"


def f16(bits_u16):
    return bits_u16.view(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------------- cos / sin

def test_cos_sin_exhaustive(env):
    bk, torch, o = env["bk"], env["torch"], env["oracle"]
    n = 1 << 17
    say(f"cos/sin exhaustive theta=1e6 pos < {n}")
    rope = bk.Rope(1e6, n)
    pos = np.arange(n, dtype=np.int32)
    cs = bk.wushkv_debug_rope_cos_sin(rope, to_dev(env, pos)).cpu().numpy()
    ref = o.cos_sin(1e6, pos)
    bad = np.argwhere(cs.view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, f"cos/sin differ at {bad[:5].tolist()} ({len(bad)})"
    say("cos/sin sampled theta=1e6 pos < 2^24 and theta=1e4")
    rng = np.random.default_rng(7)
    for theta, mp in ((1e6, 1 << 24), (1e4, 1 << 20)):
        rope = bk.Rope(theta, mp)
        pos = np.concatenate([[0, mp - 1], rng.integers(0, mp, 40000)]).astype(np.int32)
        cs = bk.wushkv_debug_rope_cos_sin(rope, to_dev(env, pos)).cpu().numpy()
        ref = o.cos_sin(theta, pos)
        assert np.array_equal(cs.view(np.uint32), ref.view(np.uint32)), theta


# ---------------------------------------------------------------------------------- transform

def test_sqrt_and_step_division_exhaustive(env):
    """The fp32 square root and the division by 2^b - 1 that the step computation uses,
    compiled as in the kernels, are correctly rounded for every one of the 2^32 fp32
    inputs on this device (checked exactly on the device: sqrt against the squares of
    the neighbouring fp32 midpoints, the divisions against the rounded fp64 quotient)."""
    say("exhaustive sqrt and division by 3, 7, 15 over 2^32 inputs")
    counts = env["bk"].wushkv_debug_check_arith()
    say(f"  mismatches [sqrt, /3, /7, /15] = {counts}")
    assert counts == [0, 0, 0, 0]


def _y_gpu(env, K, pos, T, theta=1e6):
    bk = env["bk"]
    rope = bk.Rope(theta, 1 << 17)
    tk = bk.Transform(T)
    y = bk.wushkv_debug_rope_transform(to_dev(env, K), to_dev(env, pos), rope, tk)
    env["torch"].cuda.synchronize()
    return y.cpu().numpy()


def _y_ref(env, K, pos, T, theta=1e6):
    return env["oracle"].quantize_keys(K, pos, T, theta, 2, env["oracle"].sym(), want_y=True)["y"]


@pytest.mark.parametrize("name,n", [("tiny", 256), ("qwen3_8b_prefill", 4096), ("qwen3_8b_prefill", 1000),
                                    ("affine_pct", 33)])
def test_transform_within_tolerance(env, name, n):
    s = env["synth"]
    w = s.WORKLOADS[name]
    say(f"transform {name} n={n}")
    K = s.kv(w, 0, "K", 0, n)
    pos = s.positions(w, 0, n)
    T, _ = s.transform(w, 0)
    yg, yr = _y_gpu(env, K, pos, T), _y_ref(env, K, pos, T)
    err = np.abs(yg - yr).max(axis=2)
    ref = np.abs(yr).max(axis=2)
    rel = err / np.maximum(ref, 1e-30)
    say(f"  max rel err {rel.max():.3e}")
    assert np.all(err <= TRANSFORM_TOL * ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_transform_exact_special_cases(env, dtype):
    """Identity, permutation and signed powers of two are exact in fp32, so the
    GPU's y must equal the oracle's bit for bit -- which also pins RoPE and the
    bf16 operand rounding exactly."""
    s = env["synth"]
    w = s.WORKLOADS["qwen3_8b_prefill"]
    n = 2048
    K = s.kv(w, 0, "K", 5000, n, dtype=dtype)
    pos = np.random.default_rng(3).integers(0, 1 << 17, n).astype(np.int32)
    rng = np.random.default_rng(11)
    H = K.shape[1]
    Ts = {"identity": np.stack([np.eye(128, dtype=np.float32)] * H)}
    P = np.zeros((H, 128, 128), np.float32)
    for h in range(H):
        P[h, np.arange(128), rng.permutation(128)] = 1.0
    Ts["permutation"] = P
    Ts["diag"] = np.stack([np.diag((2.0 ** rng.integers(-3, 4, 128) * rng.choice([-1, 1], 128)).astype(np.float32))
                           for _ in range(H)])
    for tn, T in Ts.items():
        say(f"exact transform {tn} {dtype}")
        yg, yr = _y_gpu(env, K, pos, T), _y_ref(env, K, pos, T)
        bad = np.argwhere(yg.view(np.uint32) != yr.view(np.uint32))
        assert bad.size == 0, f"{tn}: differ at {bad[:5].tolist()} ({len(bad)})"


def hadamard128():
    H = np.array([[1.0]])
    while H.shape[0] < 128:
        H = np.block([[H, H], [H, -H]])
    return H


def structured_transforms(H_heads, rng):
    """Hadamard / 8 (entries +-1/8, exact in bf16; its inverse is Hadamard / 16)
    and a block-diagonal transform of four random 32 x 32 blocks, per head,
    with their inverses."""
    Hd = hadamard128()
    had = np.stack([Hd / 8.0] * H_heads).astype(np.float32)
    had_inv = np.stack([Hd / 16.0] * H_heads).astype(np.float32)
    blk = np.zeros((H_heads, 128, 128))
    for h in range(H_heads):
        for b in range(4):
            blk[h, 32 * b:32 * b + 32, 32 * b:32 * b + 32] = rng.standard_normal((32, 32)) / np.sqrt(32) + 2 * np.eye(32)
    return {"hadamard": (had, had_inv),
            "block_diagonal": (blk.astype(np.float32), np.linalg.inv(blk).astype(np.float32))}


@pytest.mark.parametrize("tname", ["hadamard", "block_diagonal"])
def test_structured_transforms(env, tname):
    """Structured transforms go through the same dense path: the transform
    within tolerance, keys end to end by the same rule, the read path through
    their inverses within tolerance, on caches the oracle wrote."""
    s, o, bk, torch = env["synth"], env["oracle"], env["bk"], env["torch"]
    w = s.WORKLOADS["qwen3_8b_prefill"]
    n = 4096
    K = s.kv(w, 0, "K", 0, n)
    pos = s.positions(w, 0, n)
    T, Ti = structured_transforms(w.heads, np.random.default_rng(77))[tname]
    say(f"structured transform {tname}")
    yg, yr = _y_gpu(env, K, pos, T), _y_ref(env, K, pos, T)
    assert np.all(np.abs(yg - yr).max(axis=2) <= TRANSFORM_TOL * np.abs(yr).max(axis=2))
    q = bk.sym(2.0)
    account_keys(env, K, pos, T, 2, q, f"{tname} keys")
    rk = o.quantize_keys(K, pos, T, w.theta, 2, o.sym())
    ref = o.dequantize(rk["codes"], rk["scales"], None, n, w.heads, 2, o.sym(), Tinv=Ti)
    got = bk.wushkv_dequantize(dev_packed(env, rk), n, w.heads, 2, q, T_k_inv=bk.Transform(Ti),
                               out_dtype=torch.float32).cpu().numpy()
    assert np.all(np.abs(got - ref).max(axis=2) <= TRANSFORM_TOL * np.abs(ref).max(axis=2))


# ---------------------------------------------------------------------------------- quantizer + packing

QUANTS = [("sym", 2), ("sym", 3), ("sym", 4), ("affine", 2), ("affine", 3), ("affine", 4)]


def _bkq(env, kind):
    return env["bk"].sym(2.0) if kind == "sym" else env["bk"].affine(1.0, 99.0)


@pytest.mark.parametrize("kind,bits", QUANTS)
def test_quantizer_bit_exact_on_same_fp32_tensor(env, kind, bits):
    """Both sides quantize the oracle's fp32 transformed keys."""
    s, o = env["synth"], env["oracle"]
    w = s.WORKLOADS["qwen3_8b_prefill"]
    n = 3000
    K = s.kv(w, 0, "K", 0, n)
    pos = s.positions(w, 0, n)
    T, _ = s.transform(w, 0)
    y = _y_ref(env, K, pos, T)
    q = _bkq(env, kind)
    say(f"quantizer on oracle y: {kind} {bits}-bit n={n}")
    g = packed_host(run_values(env, y, bits, q))
    r = o.quantize_values(y, bits, oracle_q(env, q))
    assert_same_packed(g, r, f"{kind}{bits}")


@pytest.mark.parametrize("name,n,kind,bits", [
    ("tiny", 256, "sym", 2), ("qwen3_8b_prefill", 32768, "sym", 2), ("qwen3_8b_prefill", 777, "sym", 3),
    ("qwen3_32b_full", 8192, "sym", 3), ("qwen3_32b_full", 8192, "sym", 4), ("affine_pct", 8192, "affine", 2),
    ("affine_pct", 1001, "affine", 3), ("affine_pct", 513, "affine", 4), ("decode_append", 64, "sym", 2)])
def test_values_bit_exact(env, name, n, kind, bits):
    s, o = env["synth"], env["oracle"]
    w = s.WORKLOADS[name]
    V = s.kv(w, 0, "V", 0, n)
    q = _bkq(env, kind)
    say(f"values {name} n={n} {kind} {bits}-bit")
    g = packed_host(run_values(env, V, bits, q))
    r = o.quantize_values(V, bits, oracle_q(env, q))
    assert_same_packed(g, r, f"values {name}")


def test_values_strided_and_slots(env):
    """A token stride larger than H*128 (a slice of a fused tensor) and slot-addressed rows."""
    s, o, torch, bk = env["synth"], env["oracle"], env["torch"], env["bk"]
    w = s.WORKLOADS["decode_append"]
    V = s.kv(w, 0, "V")
    slots = s.slots(w)
    rows = int(slots.max()) + 1
    q = bk.sym(2.0)
    say("values strided + slots")
    big = torch.zeros((V.shape[0], 3, 8, 128), dtype=torch.bfloat16, device="cuda")
    big[:, 1] = to_dev(env, V)
    view = big[:, 1]
    out = bk.alloc_packed(rows, 8, 2, q).with_slots(to_dev(env, slots))
    bk.wushkv_quantize_values(view, 2, q, out)
    torch.cuda.synchronize()
    r = o.quantize_values(V, 2, oracle_q(env, q))
    sl = torch.from_numpy(slots).cuda()
    assert np.array_equal(out.codes[sl].cpu().numpy(), r["codes"])
    assert np.array_equal(host_u16(out.scales[sl]), r["scales"])
    mask = torch.ones(rows, dtype=torch.bool, device="cuda")
    mask[sl] = False
    assert int(out.codes[mask].count_nonzero()) == 0


# ---------------------------------------------------------------------------------- general percentiles

PERCENTILES = [(5.0, 95.0), (10.0, 90.0), (25.0, 75.0), (50.0, 50.0), (2.0, 90.0), (4.0, 99.5)]


@pytest.mark.parametrize("p_lo,p_hi", PERCENTILES)
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_values_general_percentiles_bit_exact(env, p_lo, p_hi, bits):
    """Percentiles that need order statistics other than the two extremes at each
    end (the kernels sort each 32-group in registers): bit-exact against the
    oracle, bf16 and fp32, with a ragged tail; 50/50 gives a zero step (code 0)."""
    s, o, bk = env["synth"], env["oracle"], env["bk"]
    w = s.WORKLOADS["affine_pct"]
    q = bk.affine(p_lo, p_hi)
    say(f"values percentiles {p_lo}/{p_hi} {bits}-bit")
    for dtype, n in (("bf16", 1999), ("f32", 300)):
        V = s.kv(w, 0, "V", 0, n, dtype=dtype)
        g = packed_host(run_values(env, V, bits, q))
        assert_same_packed(g, o.quantize_values(V, bits, o.affine(p_lo, p_hi)), f"values {p_lo}/{p_hi} {dtype}")


@pytest.mark.parametrize("p_lo,p_hi", [(5.0, 95.0), (10.0, 90.0), (2.0, 90.0)])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_keys_general_percentiles(env, p_lo, p_hi, bits):
    """Keys at general percentiles, end to end by the attribution rule, through the
    two-head and one-head kernels (8192 and 1000 tokens) and fp32 input."""
    s, bk = env["synth"], env["bk"]
    w = s.WORKLOADS["affine_pct"]
    q = bk.affine(p_lo, p_hi)
    T, _ = s.transform(w, 0)
    for dtype, n in (("bf16", 8192), ("bf16", 1000), ("f32", 700)):
        say(f"keys percentiles {p_lo}/{p_hi} {bits}-bit {dtype} n={n}")
        K = s.kv(w, 0, "K", 0, n, dtype=dtype)
        pos = s.positions(w, 0, n)
        account_keys(env, K, pos, T, bits, q, f"keys {p_lo}/{p_hi} {bits}-bit {dtype}")


def test_general_percentiles_read_path_and_fused_call(env):
    """A general-percentile cache read back plain (bit-exact against the oracle's
    dequantization of the oracle's records, written by the library) and the fused
    K+V call at the same quantizer (the separate calls' bytes)."""
    s, o, bk, torch = env["synth"], env["oracle"], env["bk"], env["torch"]
    w = s.WORKLOADS["affine_pct"]
    n, bits = 777, 3
    q = bk.affine(5.0, 95.0)
    V = s.kv(w, 0, "V", 0, n)
    K = s.kv(w, 0, "K", 0, n)
    pos = s.positions(w, 0, n)
    T, _ = s.transform(w, 0)
    say("general percentiles: read path and fused call")
    pv = run_values(env, V, bits, q)
    r = o.quantize_values(V, bits, o.affine(5.0, 95.0))
    back = bk.wushkv_dequantize(pv, n, w.heads, bits, q, out_dtype=torch.float32).cpu().numpy()
    ref = o.dequantize(r["codes"], r["scales"], r["zeros"], n, w.heads, bits, o.affine(5.0, 95.0))
    assert np.array_equal(back.view(np.uint32), ref.view(np.uint32))
    rope, tk = bk.Rope(w.theta, 1 << 17), bk.Transform(T)
    kc, vc = bk.alloc_packed(n, w.heads, bits, q), bk.alloc_packed(n, w.heads, bits, q)
    bk.wushkv_quantize_kv(to_dev(env, K), to_dev(env, V), to_dev(env, pos), rope, tk, bits, q, kc, vc)
    torch.cuda.synchronize()
    assert_same_packed(packed_host(vc), packed_host(pv), "fused values")
    assert_same_packed(packed_host(kc), packed_host(run_keys(env, K, pos, T, bits, q)), "fused keys")


# ---------------------------------------------------------------------------------- keys end to end

def fp16_boundary_abs(x):
    """Distance of x (fp64) to the nearest fp16 rounding midpoint (absolute)."""
    x = np.abs(np.asarray(x, np.float64))
    h = x.astype(np.float16)
    hv = h.astype(np.float64)
    up = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h, np.float16(0)).astype(np.float64)
    return np.minimum(np.abs((hv + up) / 2 - x), np.abs((hv + dn) / 2 - x))


def unpack_codes(codes, bits):
    """[..., 16*bits] LSB-first records -> [..., 128] codes (numpy.unpackbits)."""
    b = np.unpackbits(codes, axis=-1, bitorder="little").reshape(codes.shape[:-1] + (128, bits))
    return (b.astype(np.uint8) << np.arange(bits, dtype=np.uint8)).sum(axis=-1).astype(np.uint8)


# End-to-end key codes may differ from the oracle's only where a value lies
# within NEAR * step of a rounding boundary: a level midpoint (for a code), or
# an fp16 rounding midpoint (for the step or zero that the code is read with).
NEAR = 1e-6


def account_keys(env, K, pos, T, bits, q, what, g=None, y_gpu=None):
    """Compare GPU keys with the oracle and attribute every mismatch.  `g`: the
    GPU's packed rows for exactly these tokens (else the keys are run here);
    `y_gpu`: the GPU's transformed keys that produced them (else those of the
    dense path through T).

    A code may differ only if (a) the oracle's y lies within NEAR * step of the
    level midpoint that separates the two codes and the GPU's y lies on the
    other side of it, or (b) its vector's step (symmetric) or its group's step
    or zero (affine) differs, which is allowed only where the oracle's value
    before the fp16 rounding lies within NEAR * step of an fp16 rounding
    midpoint (for the zero, within NEAR * max(step, |zero|): the scale of the quantity
    rounded).  Returns (mismatches, elements, worst distance / scale)."""
    o = env["oracle"]
    if g is None:
        g = packed_host(run_keys(env, K, pos, T, bits, q))
    r = o.quantize_keys(K, pos, T, 1e6, bits, oracle_q(env, q), want_y=True)
    yr = r["y"].astype(np.float64)
    yg = (_y_gpu(env, K, pos, T) if y_gpu is None else y_gpu).astype(np.float64)
    gq, rq = unpack_codes(g["codes"], bits), unpack_codes(r["codes"], bits)
    mism = gq != rq
    L = 1 << bits
    worst = 0.0

    def code_excused(n, h, j, mids, step):
        lo, hi = sorted((yg[n, h, j], yr[n, h, j]))
        between = mids[(mids >= lo) & (mids <= hi)]
        assert between.size, f"{what}: code {(n, h, j)} differs with no midpoint between the two y"
        return np.abs(between - yr[n, h, j]).min() / step

    if q.kind == 0:
        sc_diff = g["scales"] != r["scales"]
        # the step before its fp16 rounding, from the oracle's y
        exact = 2 * q.clip_alpha * np.sqrt((yr ** 2).mean(axis=2)) / (L - 1)
        for n, h in np.argwhere(sc_diff):
            d = fp16_boundary_abs(exact[n, h]) / exact[n, h]
            worst = max(worst, d)
            assert d <= NEAR, f"{what}: step of {(n, h)} differs, {d:.2e} x step from an fp16 boundary"
        step = f16(r["scales"])
        for n, h, j in np.argwhere(~sc_diff[..., None] & mism):
            d = code_excused(n, h, j, (np.arange(L - 1) + 1 - L // 2) * step[n, h], step[n, h])
            worst = max(worst, d)
            assert d <= NEAR, f"{what}: code {(n, h, j)} differs, {d:.2e} x step from its midpoint"
    else:
        gs = g["scales"] != r["scales"]
        gz = g["zeros"] != r["zeros"]
        sc_diff = gs | gz
        for n, h, gi in np.argwhere(sc_diff):
            grp_r = np.sort(r["y"][n, h, 32 * gi:32 * gi + 32].astype(np.float32))
            lo = np.float32(o.percentile32(grp_r, q.p_lo))
            hi = np.float32(o.percentile32(grp_r, q.p_hi))
            st = float(np.float32(np.float32(hi - lo) / np.float32(L - 1)))
            # the scale of each rounded quantity: the step for the step, and for the zero
            # the larger of the step and the zero's own magnitude
            for differs, val, sc in ((gs[n, h, gi], st, abs(st)), (gz[n, h, gi], float(lo), max(abs(st), abs(float(lo))))):
                if differs:
                    d = float(fp16_boundary_abs(val)) / max(sc, 1e-30)
                    worst = max(worst, d)
                    assert d <= NEAR, f"{what}: step/zero of {(n, h, gi)} differs, {d:.2e} x step from an fp16 boundary"
        s_, z_ = f16(r["scales"]), f16(r["zeros"])
        for n, h, j in np.argwhere(np.repeat(~sc_diff, 32, axis=2) & mism):
            gi = j // 32
            d = code_excused(n, h, j, z_[n, h, gi] + (np.arange(L - 1) + 0.5) * s_[n, h, gi], s_[n, h, gi])
            worst = max(worst, d)
            assert d <= NEAR, f"{what}: code {(n, h, j)} differs, {d:.2e} x step from its midpoint"
    say(f"  {what}: code mismatches {int(mism.sum())}/{mism.size} (rate {mism.mean():.2e}), "
        f"scale diffs {int(sc_diff.sum())}, worst distance {worst:.2e} x step")
    return int(mism.sum()), mism.size, worst


@pytest.mark.parametrize("name,n,kind,bits", [
    ("tiny", 256, "sym", 2), ("qwen3_8b_prefill", 32768, "sym", 2), ("qwen3_32b_full", 8192, "sym", 3),
    ("qwen3_32b_full", 8192, "sym", 4), ("affine_pct", 16384, "affine", 2), ("affine_pct", 999, "affine", 3)])
def test_keys_end_to_end(env, name, n, kind, bits):
    s = env["synth"]
    w = s.WORKLOADS[name]
    K = s.kv(w, 0, "K", 0, n)
    pos = s.positions(w, 0, n)
    T, _ = s.transform(w, 0)
    say(f"keys {name} n={n} {kind} {bits}-bit")
    m, tot, _ = account_keys(env, K, pos, T, bits, _bkq(env, kind), f"keys {name}")
    if tot >= 1_000_000:
        assert m <= MISMATCH_RATE * tot


@pytest.mark.parametrize("name,n,dtype,hg", [
    ("qwen3_8b_prefill", 8192, "bf16", 4), ("qwen3_8b_prefill", 8192, "f32", 2),
    ("tiny", 16384, "bf16", 2), ("qwen3_8b_prefill", 1000, "bf16", 1)])
def test_keys_head_group_sizes(env, name, n, dtype, hg):
    """The key kernel runs 4, 2 or 1 heads per block (chosen from the tile count,
    the head count and the input type): each variant, end to end and through the
    exact permutation transform (y bit-exact)."""
    s = env["synth"]
    w = s.WORKLOADS[name]
    K = s.kv(w, 0, "K", 0, n, dtype=dtype)
    pos = s.positions(w, 0, n) if name != "tiny" else np.arange(n, dtype=np.int32)
    T, _ = s.transform(w, 0)
    H = K.shape[1]
    say(f"keys head groups {name} n={n} {dtype} (heads per block {hg})")
    for kind, bits in (("sym", 2), ("sym", 3), ("affine", 2)):
        account_keys(env, K, pos, T, bits, _bkq(env, kind), f"keys {name} {dtype} {kind} {bits}")
    P = np.zeros((H, 128, 128), np.float32)
    rng = np.random.default_rng(17)
    for hh in range(H):
        P[hh, np.arange(128), rng.permutation(128)] = 1.0
    yg, yr = _y_gpu(env, K, pos, P), _y_ref(env, K, pos, P)
    bad = np.argwhere(yg.view(np.uint32) != yr.view(np.uint32))
    assert bad.size == 0, f"permutation y differ at {bad[:5].tolist()} ({len(bad)})"


FULL_CASES = [("qwen3_32b_full", 0, "sym", 3), ("qwen3_32b_full", 63, "sym", 4),
              ("affine_pct", 0, "affine", 2), ("affine_pct", 35, "affine", 2)]


@pytest.mark.parametrize("name,layer,kind,bits", FULL_CASES)
def test_full_size_sampled(env, name, layer, kind, bits):
    """A whole layer at the workload's full token count (131072 or 262144
    tokens x 8 heads), launched exactly as a caller would; the oracle checks a
    seeded sample: the first and last 32-token tiles and 1024 random tokens.
    Keys by the end-to-end rule, values bit-exact, then the read path on the
    same cache (values bit-exact, keys through T_k^-1 within tolerance)."""
    s, o, bk, torch = env["synth"], env["oracle"], env["bk"], env["torch"]
    w = s.WORKLOADS[name]
    N, H = w.tokens, w.heads
    q = _bkq(env, kind)
    say(f"full-size {name} layer {layer} {kind} {bits}-bit N={N}")
    K = s.kv(w, layer, "K")
    V = s.kv(w, layer, "V")
    pos = s.positions(w)
    T, Ti = s.transform(w, layer)
    pk = run_keys(env, K, pos, T, bits, q)
    pv = run_values(env, V, bits, q)
    rng = np.random.default_rng(7000 + 100 * w.index + layer)
    idx = np.unique(np.concatenate([np.arange(32), np.arange(N - 32, N),
                                    rng.choice(N, 1024, replace=False)]))
    it = torch.from_numpy(idx).cuda()

    def rows(p):
        return dict(codes=p.codes[it].cpu().numpy(), scales=host_u16(p.scales[it]),
                    zeros=None if p.zeros is None else host_u16(p.zeros[it]))

    gk, gv = rows(pk), rows(pv)
    account_keys(env, K[idx], pos[idx], T, bits, q, f"full {name} keys", g=gk)
    rv = o.quantize_values(V[idx], bits, oracle_q(env, q))
    assert_same_packed(gv, rv, f"full {name} values")
    # read path over the whole cache, checked on the sample: the sampled rows
    # first take the oracle's own records, so that the read path's input there
    # comes from the oracle
    rk = o.quantize_keys(K[idx], pos[idx], T, w.theta, bits, oracle_q(env, q))
    for pc, r in ((pk, rk), (pv, rv)):
        hc = dev_packed(env, r)
        pc.codes[it] = hc.codes
        pc.scales[it] = hc.scales
        if pc.zeros is not None:
            pc.zeros[it] = hc.zeros
    outv = bk.wushkv_dequantize(pv, N, H, bits, q, out_dtype=torch.float32)[it].cpu().numpy()
    refv = o.dequantize(rv["codes"], rv["scales"], rv["zeros"], len(idx), H, bits, oracle_q(env, q))
    assert np.array_equal(outv.view(np.uint32), refv.view(np.uint32))
    outk = bk.wushkv_dequantize(pk, N, H, bits, q, T_k_inv=bk.Transform(Ti),
                                out_dtype=torch.float32)[it].cpu().numpy()
    refk = o.dequantize(rk["codes"], rk["scales"], rk["zeros"], len(idx), H, bits, oracle_q(env, q), Tinv=Ti)
    err = np.abs(outk - refk).max(axis=2)
    assert np.all(err <= TRANSFORM_TOL * np.abs(refk).max(axis=2))


def test_keys_identity_equals_values_of_rope(env):
    """With T = I the key path reduces to the plain quantizer on bf16(RoPE(K)) -- bit-exact."""
    s, o = env["synth"], env["oracle"]
    w = s.WORKLOADS["qwen3_8b_prefill"]
    n = 4096
    K = s.kv(w, 0, "K", 100, n)
    pos = s.positions(w, 100, n)
    eye = np.stack([np.eye(128, dtype=np.float32)] * 8)
    for kind, bits in (("sym", 2), ("affine", 2), ("sym", 4)):
        q = _bkq(env, kind)
        say(f"keys identity {kind} {bits}")
        g = packed_host(run_keys(env, K, pos, eye, bits, q))
        r = o.quantize_keys(K, pos, eye, 1e6, bits, oracle_q(env, q))
        assert_same_packed(g, r, "identity keys")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_symmetric_values_signed_zeros(env, dtype, bits):
    """Symmetric values with zeros of both signs: a zero is a tie between the
    two middle levels and takes the even code 2^(b-1) whatever its sign; whole
    zero vectors (a zero step) too.  Records and steps bit-exact against the
    oracle, in the value kernel and in the fused append."""
    o, bk, torch = env["oracle"], env["bk"], env["torch"]
    rng = np.random.default_rng(90 + bits)
    N, H = 67, 3
    V = rng.standard_normal((N, H, 128)).astype(np.float32)
    z = rng.random((N, H, 128)) < 0.3
    V[z] = np.where(rng.random(z.sum()) < 0.5, -0.0, 0.0)
    V[5] = -0.0                      # zero vectors: step 0
    V[6, 1] = 0.0
    V[7, 2] = np.where(np.arange(128) % 2, -0.0, 0.0)
    Vd = (V.view(np.uint32) >> 16).astype(np.uint16) if dtype == "bf16" else V  # bf16 bits by truncation, zeros keep their signs
    q = bk.sym(2.0)
    say(f"symmetric values with signed zeros, {bits}-bit, {dtype}")
    ref = o.quantize_values(Vd, bits, oracle_q(env, q))
    assert_same_packed(packed_host(run_values(env, Vd, bits, q)), ref, f"signed zeros {bits}-bit {dtype} values")
    # the fused append: keys of the same tokens (identity transform, position 0)
    K = Vd.copy()
    kc, vc = bk.alloc_packed(N, H, bits, q), bk.alloc_packed(N, H, bits, q)
    bk.wushkv_quantize_kv(to_dev(env, K), to_dev(env, Vd), to_dev(env, np.zeros(N, np.int32)), bk.Rope(1e6, 1 << 10),
                          bk.Transform(np.stack([np.eye(128, dtype=np.float32)] * H)), bits, q, kc, vc)
    torch.cuda.synchronize()
    assert_same_packed(packed_host(vc), ref, f"signed zeros {bits}-bit {dtype} fused append values")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("p", [(1.0, 99.0), (2.0, 98.0), (0.0, 100.0), (0.0, 99.0)])
@pytest.mark.parametrize("bits", [2, 4])
def test_affine_values_signed_zero_order_statistics(env, dtype, p, bits):
    """Percentile-clipped values whose smallest or largest order statistics tie
    between -0 and +0 (the oracle sorts by IEEE totalOrder, -0 below +0):
    groups of positive values with both zeros among the two smallest, negative
    values with both among the two largest, only zeros of both signs, a lone
    -0 below positives, zeros in the middle.  Interpolating percentiles
    (1st/99th, 2nd/98th) take the kernels' float selection, percentiles taken
    as an order statistic (0th/100th, 0th with the 99th) their totalOrder
    selection; records, steps and zeros bit-exact against the oracle."""
    o, bk = env["oracle"], env["bk"]
    rng = np.random.default_rng(int(10 * p[0] + p[1]) + 7 * bits)
    N, H = 41, 3
    V = rng.standard_normal((N, H, 4, 32)).astype(np.float32)
    for n in range(N):
        for h in range(H):
            for gi in range(4):
                x = V[n, h, gi]
                kind = (n * H * 4 + h * 4 + gi) % 6
                i, j = rng.choice(32, 2, replace=False)
                if kind == 0:
                    x[:] = np.abs(x) + 0.5
                    x[i], x[j] = -0.0, 0.0
                elif kind == 1:
                    x[:] = -np.abs(x) - 0.5
                    x[i], x[j] = 0.0, -0.0
                elif kind == 2:
                    x[:] = np.where(rng.random(32) < 0.5, -0.0, 0.0)
                elif kind == 3:
                    x[:] = np.abs(x) + 0.25
                    x[i] = -0.0
                elif kind == 4:
                    x[rng.choice(32, 6, replace=False)] = np.where(rng.random(6) < 0.5, -0.0, 0.0)
                else:
                    x[:] = np.abs(x)
                    x[rng.choice(32, 3, replace=False)] = [-0.0, 0.0, -0.0]
    V = V.reshape(N, H, 128)
    Vd = (V.view(np.uint32) >> 16).astype(np.uint16) if dtype == "bf16" else V  # bf16: truncation keeps the zeros' signs
    q = bk.affine(*p)
    say(f"affine values with signed zeros, p={p}, {bits}-bit, {dtype}")
    got = packed_host(run_values(env, Vd, bits, q))
    ref = o.quantize_values(Vd, bits, oracle_q(env, q))
    assert_same_packed(got, ref, f"signed zeros p={p} {bits}-bit {dtype}")


def test_keys_exact_zero_outputs(env):
    """Transformed keys that are exactly zero (cancellation and zero channels)
    must come out as +0 from the MFMA and take code L/2 like the oracle's: at
    position 0 RoPE is the identity, channels i + 64 copy channels i, and rows
    r < 64 of T are e_r - e_(r+64) (T = [[I, -I], [0, I]] is invertible)."""
    o = env["oracle"]
    rng = np.random.default_rng(23)
    n, H = 1000, 8
    half = rng.integers(-8, 9, size=(n, H, 64)).astype(np.float32)
    half[rng.random((n, H, 64)) < 0.3] = 0.0  # zero channels: signed-zero products
    K32 = np.concatenate([half, half], axis=2)
    K32[:, :, 5] = -0.0                        # negative zeros in both halves
    K32[:, :, 69] = -0.0
    Kb = (K32.view(np.uint32) >> 16).astype(np.uint16)  # exact: small integers
    pos = np.zeros(n, np.int32)
    T1 = np.eye(128, dtype=np.float32)
    T1[np.arange(64), np.arange(64) + 64] = -1.0
    T = np.stack([T1] * H)
    say("exact-zero transformed keys: y bits")
    yg = _y_gpu(env, Kb, pos, T)
    zeros = (yg.view(np.uint32) & 0x7FFFFFFF) == 0
    assert zeros[:, :, :64].all()
    assert not (yg.view(np.uint32) == 0x80000000).any(), "an MFMA output is -0"
    for kind, bits in (("sym", 2), ("sym", 3), ("affine", 2)):
        q = _bkq(env, kind)
        say(f"exact-zero transformed keys: codes {kind} {bits}")
        g = packed_host(run_keys(env, Kb, pos, T, bits, q))
        r = o.quantize_keys(Kb, pos, T, 1e6, bits, oracle_q(env, q))
        assert_same_packed(g, r, "exact-zero keys")


def test_decode_append_slots(env):
    s, o, bk, torch = env["synth"], env["oracle"], env["bk"], env["torch"]
    w = s.WORKLOADS["decode_append"]
    slots = s.slots(w)
    rows = 64 * 32768
    pos = s.positions(w)
    q = bk.sym(2.0)
    for layer in (0, 17, 35):
        say(f"decode append layer {layer}")
        K = s.kv(w, layer, "K")
        V = s.kv(w, layer, "V")
        T, _ = s.transform(w, layer)
        pk = run_keys(env, K, pos, T, 2, q, slots=slots, rows=rows)
        pv = run_values(env, V, 2, q, slots=slots, rows=rows)
        sl = torch.from_numpy(slots).cuda()
        rv = o.quantize_values(V, 2, o.sym())
        assert_same_packed(packed_host(bk.PackedCache(pv.codes[sl], pv.scales[sl])), rv, "decode values")
        account_keys(env, K, pos, T, 2, q, f"decode keys layer {layer}",
                     g=packed_host(bk.PackedCache(pk.codes[sl], pk.scales[sl])))
        # nothing is written outside the slot rows
        mask = torch.ones(rows, dtype=torch.bool, device="cuda")
        mask[sl] = False
        for p in (pk, pv):
            assert int(p.codes[mask].count_nonzero()) == 0 and int(p.scales[mask].count_nonzero()) == 0


def test_chunked_append_16_tokens(env):
    """Appends of 16 consecutive tokens per sequence (64 sequences at the
    decode workload's positions, clipped so that the chunk stays in its
    sequence's 32768 rows), keys and values into 64 x 32768-row caches through
    slots; the rows written are compared with the oracle's records."""
    s, o, bk, torch = env["synth"], env["oracle"], env["bk"], env["torch"]
    w = s.WORKLOADS["decode_append"]
    B, C, rows = 64, 16, 64 * 32768
    base = np.minimum(s.positions(w), 32768 - C)
    pos = (base[:, None] + np.arange(C)).reshape(-1).astype(np.int32)
    slots = (np.arange(B)[:, None] * 32768 + base[:, None] + np.arange(C)).reshape(-1).astype(np.int64)
    N = B * C
    q = bk.sym(2.0)
    for layer in (0, 35):
        say(f"chunked append layer {layer}")
        K = s.kv(w, layer, "K", 0, N)
        V = s.kv(w, layer, "V", 0, N)
        T, _ = s.transform(w, layer)
        pk = run_keys(env, K, pos, T, 2, q, slots=slots, rows=rows)
        pv = run_values(env, V, 2, q, slots=slots, rows=rows)
        sl = torch.from_numpy(slots).cuda()
        rv = o.quantize_values(V, 2, o.sym())
        assert_same_packed(packed_host(bk.PackedCache(pv.codes[sl], pv.scales[sl])), rv, "chunked values")
        account_keys(env, K, pos, T, 2, q, "chunked keys",
                     g=packed_host(bk.PackedCache(pk.codes[sl], pk.scales[sl])))
        assert int(pv.codes.count_nonzero()) <= N * 8 * 32


def test_decode_layers_in_a_graph(env):
    """Three layers' decode K and V calls captured once in a HIP graph
    (torch.cuda.CUDAGraph on a created stream) and replayed three times, with
    eager work and synchronizations between the replays: every replay writes
    exactly what the same calls write eagerly, and the first replay's rows are
    checked against the oracle (values bit-exact, keys by the end-to-end rule)."""
    s, o, bk, torch = env["synth"], env["oracle"], env["bk"], env["torch"]
    w = s.WORKLOADS["decode_append"]
    rows = 64 * 32768
    slots = torch.from_numpy(s.slots(w)).cuda()
    pos = torch.from_numpy(s.positions(w)).cuda()
    q = bk.sym(2.0)
    rope = bk.Rope(w.theta, 1 << 15)
    layers = []
    for layer in range(3):
        T, _ = s.transform(w, layer)
        layers.append(dict(K=to_dev(env, s.kv(w, layer, "K")), V=to_dev(env, s.kv(w, layer, "V")),
                           tk=bk.Transform(T), kc=bk.alloc_packed(rows, w.heads, 2, q).with_slots(slots),
                           vc=bk.alloc_packed(rows, w.heads, 2, q).with_slots(slots)))
    st = torch.cuda.Stream()
    calls = []
    for L in layers:
        calls.append(bk.prepare_quantize_keys(L["K"], pos, rope, L["tk"], 2, q, L["kc"], stream=st))
        calls.append(bk.prepare_quantize_values(L["V"], 2, q, L["vc"], stream=st))
    with torch.cuda.stream(st):
        for c in calls:  # eager once (also caches the launch shapes)
            c()
    torch.cuda.synchronize()
    want = [(L["kc"].codes[slots].clone(), L["kc"].scales[slots].clone(), L["vc"].codes[slots].clone(),
             L["vc"].scales[slots].clone()) for L in layers]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for c in calls:
            c()
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"graph replay {rep}")
        for L in layers:  # clear the rows with eager work between the replays
            L["kc"].codes[slots] = 0
            L["vc"].codes[slots] = 0
            L["kc"].scales[slots] = 0
            L["vc"].scales[slots] = 0
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for L, (kc, ks, vc, vs) in zip(layers, want):
            assert torch.equal(L["kc"].codes[slots], kc) and torch.equal(L["kc"].scales[slots], ks)
            assert torch.equal(L["vc"].codes[slots], vc) and torch.equal(L["vc"].scales[slots], vs)
        if rep == 0:
            for layer, L in enumerate(layers):
                rv = o.quantize_values(s.kv(w, layer, "V"), 2, o.sym())
                assert_same_packed(packed_host(bk.PackedCache(L["vc"].codes[slots], L["vc"].scales[slots])), rv,
                                   f"graph replay values layer {layer}")
                T, _ = s.transform(w, layer)
                account_keys(env, s.kv(w, layer, "K"), s.positions(w), T, 2, q, f"graph replay keys layer {layer}",
                             g=packed_host(bk.PackedCache(L["kc"].codes[slots], L["kc"].scales[slots])))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_symmetric_ties_take_the_even_code(env, bits):
    """Inputs exactly on level midpoints (j * step, |j| < 2^(b-1)): the nearest-
    level rule sends each tie to the even code; GPU and oracle must agree bit
    for bit.  The 24 tie channels of each vector are re-placed on the step
    that the vector ends up with until the step stops moving."""
    o, bk = env["oracle"], env["bk"]
    rng = np.random.default_rng(40 + bits)
    half = 1 << (bits - 1)
    N, H = 1024, 8
    V = (rng.standard_normal((N, H, 128)) * np.exp(rng.standard_normal((1, H, 1)))).astype(np.float32)
    j = rng.integers(-(half - 1), half, size=(N, H, 24)).astype(np.float32)
    for _ in range(8):
        step = o.quantize_values(V, bits, o.sym())["scales"].view(np.float16).astype(np.float32)
        V[:, :, :24] = j * step[..., None]
    r = o.quantize_values(V, bits, o.sym())
    step = r["scales"].view(np.float16).astype(np.float32)
    on_mid = np.all(V[:, :, :24] == j * step[..., None], axis=2) & (step > 0)
    say(f"ties {bits}-bit: {on_mid.mean():.3f} of vectors have all 24 ties on their step")
    assert on_mid.mean() > 0.5
    g = packed_host(run_values(env, V, bits, bk.sym(2.0)))
    assert_same_packed(g, r, f"ties {bits}-bit")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_affine_ties_take_the_even_code(env, bits):
    """Affine groups with six channels exactly on midpoints zero + (k + 1/2) step
    (placed among the middle ranks, re-placed until the group's zero and step
    stop moving): GPU and oracle agree bit for bit."""
    o, bk = env["oracle"], env["bk"]
    L = 1 << bits
    rng = np.random.default_rng(60 + bits)
    N, H = 1024, 8
    V = rng.standard_normal((N, H, 128)).astype(np.float32)
    G = V.reshape(N, H, 4, 32)
    k = rng.integers(0, L - 1, size=(N, H, 4, 6)).astype(np.float32) + 0.5
    for _ in range(6):
        r = o.quantize_values(V, bits, o.affine(1.0, 99.0))
        sc = r["scales"].view(np.float16).astype(np.float32).reshape(N, H, 4)
        zr = r["zeros"].view(np.float16).astype(np.float32).reshape(N, H, 4)
        mid = np.argsort(G, axis=3)[..., 8:14]
        np.put_along_axis(G, mid, (zr[..., None] + k * sc[..., None]).astype(np.float32), axis=3)
    r = o.quantize_values(V, bits, o.affine(1.0, 99.0))
    sc = r["scales"].view(np.float16).astype(np.float64).reshape(N, H, 4)
    zr = r["zeros"].view(np.float16).astype(np.float64).reshape(N, H, 4)
    on_mid = np.all(np.take_along_axis(G, mid, axis=3) == zr[..., None] + k * sc[..., None], axis=3)
    say(f"affine ties {bits}-bit: {on_mid.mean():.3f} of groups have all 6 ties exact")
    assert on_mid.mean() > 0.9
    g = packed_host(run_values(env, V, bits, bk.affine(1.0, 99.0)))
    assert_same_packed(g, r, f"affine ties {bits}-bit")


def _bf16_vectors_with_step(o, bits, N, H, seed, step=0.375):
    """bf16-exact 128-vectors built so that the symmetric quantizer's fp16 step
    comes out as `step` for most of them: 24 channels sit on midpoints j * step
    (|j| < 2^(b-1); j * step has at most 5 significant bits, so it is exact in
    bf16), 100 are random and 4 bring the sum of squares to the value that
    gives that step."""
    rng = np.random.default_rng(seed + bits)
    L = 1 << bits
    half = L // 2
    S_t = 128 * (step * (L - 1) / 4.0) ** 2  # alpha = 2: C = 2 rms, step = 2C / (L - 1)
    y = np.zeros((N, H, 128))
    perm = np.argsort(rng.random((N, H, 128)), axis=2)
    j = rng.integers(-(half - 1), half, size=(N, H, 24))
    np.put_along_axis(y, perm[..., :24], j * step, axis=2)
    S_ties = ((j * step) ** 2).sum(axis=2)
    sig = np.sqrt(np.maximum(0.85 * S_t - S_ties, 0) / 100)[..., None]
    r = o.round_bf16((rng.standard_normal((N, H, 100)) * sig).astype(np.float32)).astype(np.float64)
    np.put_along_axis(y, perm[..., 24:124], r, axis=2)
    adj = np.sqrt(np.maximum(S_t - S_ties - (r ** 2).sum(axis=2), 0) / 4)[..., None]
    adj = adj * np.sign(rng.standard_normal((N, H, 4)))
    np.put_along_axis(y, perm[..., 124:], o.round_bf16(adj.astype(np.float32)).astype(np.float64), axis=2)
    y = y.astype(np.float32)
    assert np.array_equal(o.round_bf16(y), y)
    return y


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_key_ties_take_the_even_code(env, bits):
    """The key kernel on exact ties: position 0 (RoPE is the identity) and the
    identity transform give y = the bf16 input, whose tie channels sit on
    midpoints of the step most vectors end up with."""
    o, bk = env["oracle"], env["bk"]
    N, H = 4096, 8
    y = _bf16_vectors_with_step(o, bits, N, H, seed=7)
    K = (y.view(np.uint32) >> 16).astype(np.uint16)
    pos = np.zeros(N, dtype=np.int32)
    T = np.stack([np.eye(128, dtype=np.float32)] * H)
    r = o.quantize_keys(K, pos, T, 1e6, bits, o.sym())
    hit = (r["scales"].view(np.float16).astype(np.float32) == 0.375).mean()
    say(f"key ties {bits}-bit: step on target for {hit:.3f} of vectors")
    assert hit > 0.5
    g = packed_host(run_keys(env, K, pos, T, bits, bk.sym(2.0)))
    assert_same_packed(g, r, f"key ties {bits}-bit")


# ---------------------------------------------------------------------------------- read path

@pytest.mark.parametrize("kind,bits", QUANTS)
def test_dequant_plain_bit_exact(env, kind, bits):
    s, o, bk, torch = env["synth"], env["oracle"], env["bk"], env["torch"]
    w = s.WORKLOADS["affine_pct" if kind == "affine" else "qwen3_32b_full"]
    n = 2049
    V = s.kv(w, 0, "V", 0, n)
    q = _bkq(env, kind)
    say(f"dequant plain {kind} {bits}")
    h = o.quantize_values(V, bits, oracle_q(env, q))
    p = dev_packed(env, h)
    ref = o.dequantize(h["codes"], h["scales"], h["zeros"], n, V.shape[1], bits, oracle_q(env, q))
    out32 = bk.wushkv_dequantize(p, n, V.shape[1], bits, q, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(out32.view(np.uint32), ref.view(np.uint32))
    out16 = bk.wushkv_dequantize(p, n, V.shape[1], bits, q, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.array_equal(out16.view(np.uint32), o.round_bf16(ref).view(np.uint32))


@pytest.mark.parametrize("n", [1025, 4100])
@pytest.mark.parametrize("kind,bits", QUANTS)
def test_dequant_inverse_transform(env, kind, bits, n):
    """Keys read back through T_k^-1, fp32 and bf16 out.  8 heads x 1025
    tokens launch one head per block; 4100 tokens (a ragged last tile) launch
    the four-head blocks (or the two-head blocks of the variants that take
    those)."""
    s, o, bk, torch = env["synth"], env["oracle"], env["bk"], env["torch"]
    w = s.WORKLOADS["affine_pct" if kind == "affine" else "qwen3_32b_full"]
    K = s.kv(w, 0, "K", 0, n)
    pos = s.positions(w, 0, n)
    T, Ti = s.transform(w, 0)
    q = _bkq(env, kind)
    say(f"dequant through T^-1 {kind} {bits} n={n}")
    h = o.quantize_keys(K, pos, T, w.theta, bits, oracle_q(env, q))
    p = dev_packed(env, h)
    ref = o.dequantize(h["codes"], h["scales"], h["zeros"], n, K.shape[1], bits, oracle_q(env, q), Tinv=Ti)
    g = bk.wushkv_dequantize(p, n, K.shape[1], bits, q, T_k_inv=bk.Transform(Ti), out_dtype=torch.float32)
    g = g.cpu().numpy()
    err = np.abs(g - ref).max(axis=2)
    mag = np.abs(ref).max(axis=2)
    say(f"  max rel err {(err / np.maximum(mag, 1e-30)).max():.3e}")
    assert np.all(err <= TRANSFORM_TOL * mag)
    g16 = bk.wushkv_dequantize(p, n, K.shape[1], bits, q, T_k_inv=bk.Transform(Ti), out_dtype=torch.bfloat16)
    g16 = g16.float().cpu().numpy()
    assert np.all(np.abs(g16 - ref) <= np.abs(ref) * 2.0 ** -8 + TRANSFORM_TOL * mag[..., None])


@pytest.mark.parametrize("kind,bits", [("sym", 2), ("sym", 3), ("sym", 4), ("affine", 2)])
def test_dequant_through_slots_with_missing_rows(env, kind, bits):
    """Reads through cache rows: rows in range decode their record; -1 and rows
    past the cache read as +0 (plain: bit-exact; through T_k^-1: within the
    transform tolerance, exact zeros for missing rows).  Also a cache of zero
    rows."""
    s, o, bk, torch = env["synth"], env["oracle"], env["bk"], env["torch"]
    w = s.WORKLOADS["affine_pct" if kind == "affine" else "qwen3_32b_full"]
    rows, n = 700, 613
    V = s.kv(w, 0, "V", 0, rows)
    H = V.shape[1]
    q = _bkq(env, kind)
    say(f"dequant through slots {kind} {bits}")
    h = o.quantize_values(V, bits, oracle_q(env, q))
    p = dev_packed(env, h)
    rng = np.random.default_rng(5)
    slots = rng.integers(0, rows, n).astype(np.int64)
    slots[rng.choice(n, 40, replace=False)] = -1
    slots[rng.choice(n, 40, replace=False)] = rows + rng.integers(0, 50, 40)
    ok = (slots >= 0) & (slots < rows)
    src = np.where(ok, slots, 0)
    g = lambda a: None if a is None else a[src]
    ref = o.dequantize(g(h["codes"]), g(h["scales"]), g(h["zeros"]), n, H, bits, oracle_q(env, q))
    ref[~ok] = 0.0
    ps = p.with_slots(to_dev(env, slots))
    out32 = bk.wushkv_dequantize(ps, n, H, bits, q, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(out32.view(np.uint32), ref.view(np.uint32))
    out16 = bk.wushkv_dequantize(ps, n, H, bits, q, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.array_equal(out16.view(np.uint32), o.round_bf16(ref).view(np.uint32))
    T, Ti = s.transform(w, 0)
    refk = o.dequantize(g(h["codes"]), g(h["scales"]), g(h["zeros"]), n, H, bits, oracle_q(env, q), Tinv=Ti)
    gk = bk.wushkv_dequantize(ps, n, H, bits, q, T_k_inv=bk.Transform(Ti), out_dtype=torch.float32).cpu().numpy()
    assert np.all(gk[~ok].view(np.uint32) == 0)
    err = np.abs(gk[ok] - refk[ok]).max(axis=2)
    mag = np.abs(refk[ok]).max(axis=2)
    assert np.all(err <= TRANSFORM_TOL * mag)
    # a cache with no rows: every read is +0
    empty = bk.PackedCache(p.codes[:0], p.scales[:0], None if p.zeros is None else p.zeros[:0], to_dev(env, slots))
    for Tk in (None, bk.Transform(Ti)):
        z = bk.wushkv_dequantize(empty, n, H, bits, q, T_k_inv=Tk, out_dtype=torch.float32).cpu().numpy()
        assert np.all(z.view(np.uint32) == 0)


def test_time_next_launch(env):
    """The timing call: the kernel-recorded events bracket the kernel alone, so
    they read less than events recorded around the call, and the setting is
    used by one launch only."""
    s, bk, torch = env["synth"], env["bk"], env["torch"]
    w = s.WORKLOADS["qwen3_8b_prefill"]
    n = 8192
    V = to_dev(env, s.kv(w, 0, "V", 0, n))
    q = bk.sym(2.0)
    out = bk.alloc_packed(n, w.heads, 2, q)
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record(st)
    torch.cuda.synchronize()
    say("timing events")
    for _ in range(3):
        ev[0].record(st)
        bk.wushkv_debug_time_next_launch(ev[1], ev[2])
        bk.wushkv_quantize_values(V, 2, q, out)
        ev[3].record(st)
        torch.cuda.synchronize()
        inner, outer = ev[1].elapsed_time(ev[2]), ev[0].elapsed_time(ev[3])
        assert 0.0 < inner <= outer
    # consumed: a second launch leaves the events where they were
    before = ev[1].elapsed_time(ev[2])
    bk.wushkv_quantize_values(V, 2, q, out)
    torch.cuda.synchronize()
    assert ev[1].elapsed_time(ev[2]) == before
    with pytest.raises(ValueError):
        bk.wushkv_debug_time_next_launch(torch.cuda.Event(enable_timing=True), None)


# ---------------------------------------------------------------------------------- edges

@pytest.mark.parametrize("n", [0, 1, 31, 33, 65])
def test_ragged_and_empty(env, n):
    s, o, bk, torch = env["synth"], env["oracle"], env["bk"], env["torch"]
    w = s.WORKLOADS["qwen3_8b_prefill"]
    K = s.kv(w, 0, "K", 0, max(n, 1))[:n]
    V = s.kv(w, 0, "V", 0, max(n, 1))[:n]
    pos = s.positions(w, 0, max(n, 1))[:n]
    T, _ = s.transform(w, 0)
    q = bk.sym(2.0)
    say(f"ragged n={n}")
    pk = run_keys(env, K, pos, T, 2, q, rows=max(n, 1))
    pv = run_values(env, V, 2, q, rows=max(n, 1))
    if n == 0:
        assert int(pk.codes.count_nonzero()) == 0 and int(pv.codes.count_nonzero()) == 0
        return
    rv = o.quantize_values(V, 2, o.sym())
    assert np.array_equal(pv.codes.cpu().numpy(), rv["codes"])
    assert np.array_equal(host_u16(pv.scales), rv["scales"])
    account_keys(env, K, pos, T, 2, q, f"ragged keys n={n}", g=packed_host(pk))


def test_deterministic(env):
    s, bk = env["synth"], env["bk"]
    w = s.WORKLOADS["qwen3_8b_prefill"]
    n = 8192
    K = s.kv(w, 0, "K", 0, n)
    pos = s.positions(w, 0, n)
    T, _ = s.transform(w, 0)
    say("determinism")
    a = packed_host(run_keys(env, K, pos, T, 2, bk.sym()))
    b = packed_host(run_keys(env, K, pos, T, 2, bk.sym()))
    c = packed_host(run_keys(env, K, pos, T, 2, bk.sym()))
    assert_same_packed(a, b, "run 2")
    assert_same_packed(a, c, "run 3")


@pytest.mark.parametrize("H", [3, 5])
def test_odd_head_count_strided_slots(env, H):
    """Head counts that are not powers of two (exact division by H on the GPU),
    a token stride larger than H*128 and scattered slot rows."""
    o, bk, torch = env["oracle"], env["bk"], env["torch"]
    rng = np.random.default_rng(100 + H)
    N, rows = 1000, 5000
    V = (rng.standard_normal((N, H, 128)) * np.exp(rng.standard_normal((1, H, 128)))).astype(np.float32)
    K = (rng.standard_normal((N, H, 128)) * 3).astype(np.float32)
    pos = rng.integers(0, 1 << 16, N).astype(np.int32)
    slots = rng.choice(rows, N, replace=False).astype(np.int64)
    T = np.stack([np.eye(128, dtype=np.float32)[rng.permutation(128)] * 2.0 for _ in range(H)])
    say(f"odd heads H={H}")
    big = torch.zeros((N, H + 1, 128), dtype=torch.float32, device="cuda")
    big[:, :H] = to_dev(env, V)
    for kind, bits in (("sym", 3), ("affine", 2)):
        q = _bkq(env, kind)
        out = bk.alloc_packed(rows, H, bits, q).with_slots(to_dev(env, slots))
        bk.wushkv_quantize_values(big[:, :H], bits, q, out)
        torch.cuda.synchronize()
        r = o.quantize_values(V, bits, oracle_q(env, q))
        sl = torch.from_numpy(slots).cuda()
        g = packed_host(bk.PackedCache(out.codes[sl], out.scales[sl], None if out.zeros is None else out.zeros[sl]))
        assert_same_packed(g, r, f"values H={H} {kind}")
        # keys through a permutation-times-two transform are exact: bit-exact against the oracle
        pk = run_keys(env, K, pos, T, bits, q, slots=slots, rows=rows)
        rk = o.quantize_keys(K, pos, T, 1e6, bits, oracle_q(env, q))
        gk = packed_host(bk.PackedCache(pk.codes[sl], pk.scales[sl], None if pk.zeros is None else pk.zeros[sl]))
        assert_same_packed(gk, rk, f"keys H={H} {kind}")
        back = bk.wushkv_dequantize(out, N, H, bits, q, out_dtype=torch.float32).cpu().numpy()
        ref = o.dequantize(r["codes"], r["scales"], r["zeros"], N, H, bits, oracle_q(env, q))
        assert np.array_equal(back.view(np.uint32), ref.view(np.uint32))
