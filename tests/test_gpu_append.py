"""GPU parity of the fused key + value call (wushkv_quantize_kv) against the CPU
oracle, through the C ABI.

The fused kernel must write exactly the records that the oracle defines (values
bit-exact; keys by the end-to-end rule of test_gpu_parity.account_keys) and
exactly the bytes of the separate key and value calls, on the append shapes it
is built for: decode steps (one token per sequence per layer, all 36 layers of
the decode workload), 16-token chunks, ragged and single-token calls, fp32
inputs, every quantizer and width, strided inputs and slot-addressed caches with
skipped rows, and replays of a 36-layer HIP graph.
"""
import numpy as np
import pytest

from test_gpu_parity import (_bkq, account_keys, assert_same_packed, env, host_u16, oracle_q,  # noqa: F401
                             packed_host, run_keys, run_values, say, to_dev)

pytestmark = pytest.mark.gpu


def run_kv(env, K, V, pos, T, bits, q, slots=None, rows=None, theta=1e6, max_pos=1 << 17, Kd=None, Vd=None):
    bk, torch = env["bk"], env["torch"]
    N, H = K.shape[0], K.shape[1]
    rows = rows if rows is not None else max(N, 1)
    rope, tk = bk.Rope(theta, max_pos), bk.Transform(T)
    kc, vc = bk.alloc_packed(rows, H, bits, q), bk.alloc_packed(rows, H, bits, q)
    if slots is not None:
        sd = to_dev(env, slots)
        kc, vc = kc.with_slots(sd), vc.with_slots(sd)
    bk.wushkv_quantize_kv(to_dev(env, K) if Kd is None else Kd, to_dev(env, V) if Vd is None else Vd,
                          to_dev(env, pos), rope, tk, bits, q, kc, vc)
    torch.cuda.synchronize()
    return kc, vc


def rows_of(env, p, idx):
    """Host records of cache rows idx (None: all rows)."""
    bk, torch = env["bk"], env["torch"]
    if idx is None:
        return packed_host(p)
    it = torch.from_numpy(np.asarray(idx, np.int64)).cuda()
    return packed_host(bk.PackedCache(p.codes[it], p.scales[it], None if p.zeros is None else p.zeros[it]))


CASES = [
    ("decode_append", 64, "bf16", "sym", 2, True),
    ("qwen3_8b_prefill", 1, "bf16", "sym", 2, False),
    ("qwen3_8b_prefill", 13, "bf16", "sym", 2, False),
    ("qwen3_8b_prefill", 1000, "bf16", "sym", 3, False),
    ("qwen3_8b_prefill", 257, "bf16", "sym", 4, True),
    ("tiny", 256, "f32", "sym", 2, False),
    ("tiny", 77, "f32", "affine", 3, False),
    ("affine_pct", 512, "bf16", "affine", 2, False),
    ("affine_pct", 9, "bf16", "affine", 4, True),
]


@pytest.mark.parametrize("name,n,dtype,kind,bits,use_slots", CASES)
def test_fused_matches_oracle_and_separate_calls(env, name, n, dtype, kind, bits, use_slots):
    s, o, bk = env["synth"], env["oracle"], env["bk"]
    w = s.WORKLOADS[name]
    K = s.kv(w, 0, "K", 0, n, dtype=dtype)
    V = s.kv(w, 0, "V", 0, n, dtype=dtype)
    pos = s.positions(w, 0, n) if name != "tiny" else np.arange(n, dtype=np.int32)
    T, _ = s.transform(w, 0)
    q = _bkq(env, kind)
    rows, slots, idx = None, None, None
    if use_slots:
        rows = 4 * n + 7
        slots = np.random.default_rng(900 + n).choice(rows, n, replace=False).astype(np.int64)
        idx = slots
    say(f"fused {name} n={n} {dtype} {kind} {bits}-bit slots={use_slots}")
    kc, vc = run_kv(env, K, V, pos, T, bits, q, slots=slots, rows=rows)
    gk, gv = rows_of(env, kc, idx), rows_of(env, vc, idx)
    assert_same_packed(gv, o.quantize_values(V, bits, oracle_q(env, q)), "fused values vs oracle")
    account_keys(env, K, pos, T, bits, q, f"fused keys {name} n={n}", g=gk)
    # the separate calls write the same bytes (same MFMA sequence, same statistic)
    sk = rows_of(env, run_keys(env, K, pos, T, bits, q, slots=slots, rows=rows), idx)
    sv = rows_of(env, run_values(env, V, bits, q, slots=slots, rows=rows), idx)
    assert_same_packed(gk, sk, "fused keys vs the key call")
    assert_same_packed(gv, sv, "fused values vs the value call")


def test_fused_decode_all_layers(env):
    """The decode workload's 36 layers (64 sequences, one token each, slot rows
    b * 32768 + pos_b): one fused call per layer into shared 2M-row caches; every
    layer's rows against the oracle (values bit-exact, keys attributed), and
    nothing written outside the slot rows."""
    s, o, bk, torch = env["synth"], env["oracle"], env["bk"], env["torch"]
    w = s.WORKLOADS["decode_append"]
    rows = 64 * 32768
    slots = s.slots(w)
    pos = s.positions(w)
    q = bk.sym(2.0)
    rope = bk.Rope(w.theta, 1 << 15)
    sd, pd = to_dev(env, slots), to_dev(env, pos)
    kc = bk.alloc_packed(rows, w.heads, 2, q).with_slots(sd)
    vc = bk.alloc_packed(rows, w.heads, 2, q).with_slots(sd)
    worst, mism = 0.0, 0
    for layer in range(w.layers):
        K, V = s.kv(w, layer, "K"), s.kv(w, layer, "V")
        T, _ = s.transform(w, layer)
        bk.wushkv_quantize_kv(to_dev(env, K), to_dev(env, V), pd, rope, bk.Transform(T), 2, q, kc, vc)
        torch.cuda.synchronize()
        assert_same_packed(rows_of(env, vc, slots), o.quantize_values(V, 2, o.sym()), f"decode values layer {layer}")
        m, _, wd = account_keys(env, K, pos, T, 2, q, f"decode keys layer {layer}", g=rows_of(env, kc, slots))
        worst, mism = max(worst, wd), mism + m
    say(f"36 layers: key code mismatches {mism}, worst distance {worst:.2e} x step")
    mask = torch.ones(rows, dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(slots).cuda()] = False
    for p in (kc, vc):
        assert int(p.codes[mask].count_nonzero()) == 0 and int(p.scales[mask].count_nonzero()) == 0


def test_fused_chunked_append_16_tokens(env):
    """16 consecutive tokens per sequence for 64 sequences, into 64 x 32768-row
    caches through slots, two layers."""
    s, o, bk = env["synth"], env["oracle"], env["bk"]
    w = s.WORKLOADS["decode_append"]
    B, C, rows = 64, 16, 64 * 32768
    base = np.minimum(s.positions(w), 32768 - C)
    pos = (base[:, None] + np.arange(C)).reshape(-1).astype(np.int32)
    slots = (np.arange(B)[:, None] * 32768 + base[:, None] + np.arange(C)).reshape(-1).astype(np.int64)
    N = B * C
    q = bk.sym(2.0)
    for layer in (0, 35):
        say(f"fused chunked append layer {layer}")
        K, V = s.kv(w, layer, "K", 0, N), s.kv(w, layer, "V", 0, N)
        T, _ = s.transform(w, layer)
        kc, vc = run_kv(env, K, V, pos, T, 2, q, slots=slots, rows=rows, theta=w.theta, max_pos=1 << 15)
        assert_same_packed(rows_of(env, vc, slots), o.quantize_values(V, 2, o.sym()), "chunked values")
        account_keys(env, K, pos, T, 2, q, "fused chunked keys", g=rows_of(env, kc, slots))


def test_fused_strided_inputs_and_skipped_rows(env):
    """K and V as slices of wider tensors (token strides above H * 128, different
    for K and V), 5 heads, and slots with -1 and rows past the cache's end: those
    tokens write nothing, the others match the oracle."""
    o, bk, torch = env["oracle"], env["bk"], env["torch"]
    rng = np.random.default_rng(321)
    N, H, rows = 45, 5, 300
    K = (rng.standard_normal((N, H, 128)) * 2).astype(np.float32)
    V = (rng.standard_normal((N, H, 128)) * np.exp(rng.standard_normal((1, H, 128)))).astype(np.float32)
    pos = rng.integers(0, 1 << 16, N).astype(np.int32)
    slots = rng.choice(rows, N, replace=False).astype(np.int64)
    slots[::7] = -1
    slots[3::11] = rows + 5
    T = np.stack([np.linalg.qr(rng.standard_normal((128, 128)))[0].astype(np.float32) * 1.5 for _ in range(H)])
    Kb = torch.zeros((N, H + 2, 128), dtype=torch.float32, device="cuda")
    Vb = torch.zeros((N, H + 1, 128), dtype=torch.float32, device="cuda")
    Kb[:, 1:H + 1] = to_dev(env, K)
    Vb[:, :H] = to_dev(env, V)
    live = (slots >= 0) & (slots < rows)
    say("fused strided inputs, skipped rows")
    for kind, bits in (("sym", 2), ("sym", 4), ("affine", 3)):
        q = _bkq(env, kind)
        kc, vc = run_kv(env, K, V, pos, T, bits, q, slots=slots, rows=rows, Kd=Kb[:, 1:H + 1], Vd=Vb[:, :H])
        rv = o.quantize_values(V[live], bits, oracle_q(env, q))
        assert_same_packed(rows_of(env, vc, slots[live]), rv, f"strided values {kind} {bits}")
        account_keys(env, K[live], pos[live], T, bits, q, f"strided keys {kind} {bits}",
                     g=rows_of(env, kc, slots[live]))
        mask = torch.ones(rows, dtype=torch.bool, device="cuda")
        mask[torch.from_numpy(slots[live]).cuda()] = False
        for p in (kc, vc):
            assert int(p.codes[mask].count_nonzero()) == 0 and int(p.scales[mask].count_nonzero()) == 0


def test_fused_empty_call(env):
    s, bk = env["synth"], env["bk"]
    w = s.WORKLOADS["qwen3_8b_prefill"]
    K = s.kv(w, 0, "K", 0, 1)[:0]
    V = s.kv(w, 0, "V", 0, 1)[:0]
    T, _ = s.transform(w, 0)
    kc, vc = run_kv(env, K, V, np.zeros(0, np.int32), T, 2, bk.sym(2.0), rows=1)
    assert int(kc.codes.count_nonzero()) == 0 and int(vc.codes.count_nonzero()) == 0


def test_fused_decode_graph_36_layers(env):
    """The decode step as one HIP graph of 36 fused calls (one kernel node per
    layer), replayed three times with eager clearing and synchronizations in
    between: every replay writes exactly the eager bytes, and the first replay's
    records of every layer are checked against the oracle."""
    s, o, bk, torch = env["synth"], env["oracle"], env["bk"], env["torch"]
    w = s.WORKLOADS["decode_append"]
    B = 64
    slots = torch.from_numpy(np.random.default_rng(5).permutation(B).astype(np.int64)).cuda()
    pos_h = s.positions(w)
    pos = to_dev(env, pos_h)
    q = bk.sym(2.0)
    rope = bk.Rope(w.theta, 1 << 15)
    layers = []
    for layer in range(w.layers):
        T, _ = s.transform(w, layer)
        layers.append(dict(K=to_dev(env, s.kv(w, layer, "K")), V=to_dev(env, s.kv(w, layer, "V")),
                           tk=bk.Transform(T), kc=bk.alloc_packed(B, w.heads, 2, q).with_slots(slots),
                           vc=bk.alloc_packed(B, w.heads, 2, q).with_slots(slots)))
    st = torch.cuda.Stream()
    calls = [bk.prepare_quantize_kv(L["K"], L["V"], pos, rope, L["tk"], 2, q, L["kc"], L["vc"], stream=st)
             for L in layers]
    with torch.cuda.stream(st):
        for c in calls:
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
        say(f"fused graph replay {rep}")
        for L in layers:
            for p in (L["kc"], L["vc"]):
                p.codes.zero_()
                p.scales.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for L, (kcd, ksc, vcd, vsc) in zip(layers, want):
            assert torch.equal(L["kc"].codes[slots], kcd) and torch.equal(L["kc"].scales[slots], ksc)
            assert torch.equal(L["vc"].codes[slots], vcd) and torch.equal(L["vc"].scales[slots], vsc)
        if rep == 0:
            sl = slots.cpu().numpy()
            for layer, L in enumerate(layers):
                rv = o.quantize_values(s.kv(w, layer, "V"), 2, o.sym())
                assert_same_packed(rows_of(env, L["vc"], sl), rv, f"graph values layer {layer}")
                T, _ = s.transform(w, layer)
                account_keys(env, s.kv(w, layer, "K"), pos_h, T, 2, q, f"graph keys layer {layer}",
                             g=rows_of(env, L["kc"], sl))
