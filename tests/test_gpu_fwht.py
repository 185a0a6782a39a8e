"""GPU checks of the structured key path: Transform.hadamard (wushkv_transform_create_hadamard),
whose keys go through an in-register fast Walsh-Hadamard transform instead of the dense
MFMA product, against the oracle's definition with the dense matrix T = H_128 / 8.

* Exact cases: keys at position 0 (RoPE is the identity there) that are small integers
  make every partial sum of the transform exact in fp32, so y and the records must equal
  the oracle's bit for bit -- which pins the butterflies' signs and the output row order.
* Realistic keys: y within the dense path's transform tolerance, and keys end to end with
  every code mismatch attributed as for the dense path (symmetric 2/3/4 bits, both affine
  kinds), at the full benchmark layer for 2 bits.
* Slot rows with missing rows, a token stride above H * 128, fp32 input, odd head counts
  (one head group of 3 or 5 heads, two of 6 for 12), ragged and empty calls.
* The fused K+V append takes the handle's dense copy: its bytes equal those of a dense
  handle made from the same matrix.
"""
import numpy as np
import pytest

from test_gpu_parity import (TRANSFORM_TOL, _bkq, account_keys, assert_same_packed, env, hadamard128,  # noqa: F401
                             host_u16, oracle_q, packed_host, say, to_dev)

pytestmark = pytest.mark.gpu


def had(H):
    return np.stack([hadamard128() / 8.0] * H).astype(np.float32)


def y_fwht(env, K, pos, theta=1e6, max_pos=1 << 17):
    bk = env["bk"]
    y = bk.wushkv_debug_rope_transform(to_dev(env, K), to_dev(env, pos), bk.Rope(theta, max_pos),
                                       bk.Transform.hadamard(K.shape[1]))
    env["torch"].cuda.synchronize()
    return y.cpu().numpy()


def run_fwht(env, K, pos, bits, q, slots=None, rows=None, theta=1e6, max_pos=1 << 17, Kdev=None):
    bk = env["bk"]
    N, H = K.shape[0], K.shape[1]
    out = bk.alloc_packed(rows if rows is not None else N, H, bits, q)
    if slots is not None:
        out = out.with_slots(to_dev(env, slots))
    bk.wushkv_quantize_keys(to_dev(env, K) if Kdev is None else Kdev, to_dev(env, pos), bk.Rope(theta, max_pos),
                            bk.Transform.hadamard(H), bits, q, out)
    env["torch"].cuda.synchronize()
    return out


def int_keys(rng, N, H):
    """bf16 bit patterns of integers in [-64, 64]."""
    v = rng.integers(-64, 65, (N, H, 128)).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("H,N", [(8, 100), (3, 37), (12, 50)])
def test_fwht_exact_on_integer_keys(env, H, N):
    o, bk = env["oracle"], env["bk"]
    rng = np.random.default_rng(500 + H)
    K = int_keys(rng, N, H)
    pos = np.zeros(N, np.int32)
    say(f"fwht exact H={H} N={N}")
    yg = y_fwht(env, K, pos)
    yr = o.quantize_keys(K, pos, had(H), 1e6, 2, o.sym(), want_y=True)["y"]
    bad = np.argwhere(yg.view(np.uint32) != yr.view(np.uint32))
    assert bad.size == 0, f"y differs at {bad[:5].tolist()} ({len(bad)})"
    for kind, bits in (("sym", 2), ("sym", 3), ("sym", 4), ("affine", 2)):
        q = _bkq(env, kind)
        g = packed_host(run_fwht(env, K, pos, bits, q))
        r = o.quantize_keys(K, pos, had(H), 1e6, bits, oracle_q(env, q))
        assert_same_packed(g, r, f"fwht exact {kind} {bits}-bit H={H}")


@pytest.mark.parametrize("name,n,dtype", [("qwen3_8b_prefill", 4096, "bf16"), ("qwen3_8b_prefill", 1000, "f32"),
                                          ("tiny", 256, "bf16"), ("qwen3_32b_full", 17, "bf16")])
def test_fwht_transform_within_tolerance(env, name, n, dtype):
    s, o = env["synth"], env["oracle"]
    w = s.WORKLOADS[name]
    K = s.kv(w, 0, "K", 0, n, dtype=dtype)
    pos = s.positions(w, 0, n)
    say(f"fwht transform {name} n={n} {dtype}")
    yg = y_fwht(env, K, pos)
    yr = o.quantize_keys(K, pos, had(w.heads), w.theta, 2, o.sym(), want_y=True)["y"]
    err, ref = np.abs(yg - yr).max(axis=2), np.abs(yr).max(axis=2)
    say(f"  max rel err {(err / np.maximum(ref, 1e-30)).max():.3e}")
    assert np.all(err <= TRANSFORM_TOL * ref)


@pytest.mark.parametrize("name,n,kind,bits", [
    ("qwen3_8b_prefill", 32768, "sym", 2), ("qwen3_32b_full", 8192, "sym", 3), ("qwen3_32b_full", 8192, "sym", 4),
    ("affine_pct", 16384, "affine", 2), ("affine_pct", 999, "affine", 4), ("qwen3_8b_prefill", 4096, "pct5", 2)])
def test_fwht_keys_end_to_end(env, name, n, kind, bits):
    s, bk = env["synth"], env["bk"]
    w = s.WORKLOADS[name]
    K = s.kv(w, 0, "K", 0, n)
    pos = s.positions(w, 0, n)
    q = bk.affine(5.0, 95.0) if kind == "pct5" else _bkq(env, kind)
    say(f"fwht keys {name} n={n} {kind} {bits}-bit")
    g = packed_host(run_fwht(env, K, pos, bits, q))
    account_keys(env, K, pos, had(w.heads), bits, q, f"fwht keys {name}", g=g, y_gpu=y_fwht(env, K, pos))


@pytest.mark.parametrize("H", [3, 5, 12])
def test_fwht_slots_strided_missing_rows(env, H):
    o, bk, torch = env["oracle"], env["bk"], env["torch"]
    rng = np.random.default_rng(900 + H)
    N, rows = 700, 3000
    K = (rng.standard_normal((N, H, 128)) * np.exp(rng.standard_normal((1, H, 128)))).astype(np.float32)
    pos = rng.integers(0, 1 << 16, N).astype(np.int32)
    slots = rng.choice(rows, N, replace=False).astype(np.int64)
    slots[::7] = -1           # no store
    slots[3::11] = rows + 5   # past the cache: no store
    big = torch.zeros((N, H + 2, 128), dtype=torch.float32, device="cuda")
    big[:, :H] = to_dev(env, K)
    say(f"fwht slots H={H}")
    for kind, bits in (("sym", 2), ("sym", 3), ("affine", 2)):
        q = _bkq(env, kind)
        out = run_fwht(env, K, pos, bits, q, slots=slots, rows=rows, Kdev=big[:, :H])
        ok = (slots >= 0) & (slots < rows)
        sl = torch.from_numpy(slots[ok]).cuda()
        g = packed_host(bk.PackedCache(out.codes[sl], out.scales[sl], None if out.zeros is None else out.zeros[sl]))
        sub = np.flatnonzero(ok)
        account_keys(env, K[sub], pos[sub], had(H), bits, q, f"fwht slots H={H} {kind}", g=g,
                     y_gpu=y_fwht(env, K[sub], pos[sub]))
        # rows no token was stored to stay zero
        untouched = np.setdiff1d(np.arange(rows), slots[ok])
        assert int(out.codes[torch.from_numpy(untouched).cuda()].count_nonzero()) == 0


@pytest.mark.parametrize("n", [0, 1, 15, 17])
def test_fwht_ragged_and_empty(env, n):
    s, bk = env["synth"], env["bk"]
    w = s.WORKLOADS["qwen3_8b_prefill"]
    K = s.kv(w, 0, "K", 0, max(n, 1))[:n]
    pos = s.positions(w, 0, max(n, 1))[:n]
    q = bk.sym(2.0)
    say(f"fwht ragged n={n}")
    out = run_fwht(env, K, pos, 2, q, rows=max(n, 1))
    if n == 0:
        assert int(out.codes.count_nonzero()) == 0
        return
    account_keys(env, K, pos, had(w.heads), 2, q, f"fwht ragged n={n}", g=packed_host(out), y_gpu=y_fwht(env, K, pos))


def test_fused_append_takes_the_dense_copy(env):
    s, bk, torch = env["synth"], env["bk"], env["torch"]
    w = s.WORKLOADS["qwen3_8b_prefill"]
    n = 64
    K, V = s.kv(w, 0, "K", 0, n), s.kv(w, 0, "V", 0, n)
    pos = s.positions(w, 0, n)
    q = bk.sym(2.0)
    rope = bk.Rope(w.theta, 1 << 17)
    say("fused append with the Hadamard handle")
    outs = []
    for tk in (bk.Transform.hadamard(w.heads), bk.Transform(had(w.heads))):
        kc, vc = bk.alloc_packed(n, w.heads, 2, q), bk.alloc_packed(n, w.heads, 2, q)
        bk.wushkv_quantize_kv(to_dev(env, K), to_dev(env, V), to_dev(env, pos), rope, tk, 2, q, kc, vc)
        torch.cuda.synchronize()
        outs.append((packed_host(kc), packed_host(vc)))
    assert_same_packed(outs[0][0], outs[1][0], "fused keys")
    assert_same_packed(outs[0][1], outs[1][1], "fused values")
