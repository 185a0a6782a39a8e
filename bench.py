"""Benchmark: WUSH-KV cache write path (K+V into the 2-bit cache) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: the Qwen3-8B-shaped single-layer prefill -- 32768 tokens x 8 KV
heads x 128, bf16 keys and values (seeded synthetic: per-channel LogNormal(0,1)
scales times Student-t(3) noise), per-head general invertible T_k, RoPE theta
1e6, 2-bit RMS-clipped symmetric codes with one fp16 step per (token, head).

One step = wushkv_quantize_keys (RoPE -> bf16 -> T_k on MFMA -> quantize ->
pack) + wushkv_quantize_values (quantize -> pack) over the whole layer.  Inputs
are resident in HBM before timing; the step cycles through enough input/output
sets (> 2x the 256 MB MALL) that no set is re-read from the MALL.

Prints one JSON line.  `value` is K+V tokens/s of the whole step, from K
steps launched back to back between two synchronizations, each step's keys on
the launch stream and its values on a second stream (they are independent, so
the GPU may run them side by side; `--one-stream` serializes them).  Both are
streams of their own, not the null stream: work on the null stream and on the
first stream created after it was seen to run one after the other;
`roofline` is for
the key kernel (algorithmic bytes per launch / its mean duration, from a pair
of HIP events that each key kernel records at its own start and end on the
launch stream, in a second pass over the same K steps); `cpu_baseline` is the
CPU oracle as it stands, single-threaded, on the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "K+V tokens/s into 2-bit cache; achieved HBM GB/s and MFMA % of peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MALL_BYTES = 256 << 20
D = 128
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "keys_qwen3_8b_prefill_traffic.md")
KEY_KERNEL_SOURCES = [os.path.join(ROOT, "bit_kv_cache_rope_amd", "csrc", f)
                      for f in ("keys.hip", "device_common.h")]


def key_bytes_per_token(H: int, bits: int) -> int:
    """Algorithmic bytes of the key kernel per token: bf16 K in, int32 position,
    packed codes and fp16 steps out."""
    return H * D * 2 + 4 + H * 16 * bits + H * 2


def value_bytes_per_token(H: int, bits: int) -> int:
    return H * D * 2 + H * 16 * bits + H * 2


def key_kernel_sha() -> str:
    h = hashlib.sha256()
    for p in KEY_KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per key-kernel launch from the committed rocprofv3 counter
    summary, or None if absent or taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    m = re.search(r"^bench-traffic: (\{.*\})\s*$", open(TRAFFIC_FILE).read(), re.M)
    if not m:
        return None
    t = json.loads(m.group(1))
    if t.get("source_sha") != key_kernel_sha():
        return None
    return t


def cpu_baseline(w, synth, seconds_hint: float = 20.0) -> dict:
    import oracle
    oracle.build()
    n = w.tokens
    K = synth.kv(w, 0, "K", 0, n)
    V = synth.kv(w, 0, "V", 0, n)
    pos = synth.positions(w, 0, n)
    T, _ = synth.transform(w, 0)
    reps = 0
    t0 = time.perf_counter()
    while True:  # whole layers until about seconds_hint of CPU work (at least two)
        oracle.quantize_keys(K, pos, T, w.theta, 2, oracle.sym(w.clip_alpha), threads=1)
        oracle.quantize_values(V, 2, oracle.sym(w.clip_alpha), threads=1)
        reps += 1
        dt = time.perf_counter() - t0
        if reps >= 2 and dt >= seconds_hint * 0.6:
            break
    return {"value": reps * n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} passes over one full layer of the workload ({n} tokens x {w.heads} heads, "
                      f"K and V), single-threaded, {dt:.1f} s"}


def quality_report(torch, synth, bk, dev, layers=4, n_tok=4096, n_q=64, q_scale=0.4, bits=2) -> dict:
    """Attention-output error of the quantized cache, per transform: identity,
    Hadamard / 8 and the workload's T_k (keys through the transform and paired
    queries, values plain, 2-bit symmetric) against fp32 attention over the
    unquantized bf16 keys after RoPE and bf16 values, on synthetic
    Qwen3-8B-shaped layers.  Error = |o - o_ref|^2 / |o_ref|^2 per layer
    (all query heads), geometric mean over the layers.  Queries are N(0, 1) x
    q_scale: 0.4 puts the scores' spread at about 2 (a softmax that is neither
    flat nor one-hot on these keys)."""
    w = synth.WORKLOADS["qwen3_8b_prefill"]
    H, G = w.heads, 4
    q = bk.sym(w.clip_alpha)
    rope = bk.Rope(w.theta, 1 << 17)
    Hd = np.array([[1.0]])
    while Hd.shape[0] < D:
        Hd = np.block([[Hd, Hd], [Hd, -Hd]])
    eye = bk.Transform(np.stack([np.eye(D, dtype=np.float32)] * H))
    pos = torch.from_numpy(synth.positions(w, 0, n_tok)).to(dev)
    errs = {"identity": [], "hadamard": [], "T_k": []}
    for layer in range(layers):
        K = torch.from_numpy(synth.kv(w, layer, "K", 0, n_tok).view(np.int16)).to(dev).view(torch.bfloat16)
        V = torch.from_numpy(synth.kv(w, layer, "V", 0, n_tok).view(np.int16)).to(dev).view(torch.bfloat16)
        X = bk.wushkv_debug_rope_transform(K, pos, rope, eye)  # bf16(RoPE(k)), exact in fp32
        T, Ti = synth.transform(w, layer)
        g = torch.Generator(device=dev)
        g.manual_seed(1000 + layer)
        Q = torch.randn((n_q, H * G, D), device=dev, generator=g) * q_scale
        Qb = Q.to(torch.bfloat16)
        scale = 1.0 / np.sqrt(D)
        # fp32 reference: query head hq reads KV head hq // G
        Xh = X.permute(1, 0, 2).contiguous()                  # [H][N][128]
        Vh = V.float().permute(1, 0, 2).contiguous()          # [H][N][128]
        Qh = Qb.float().view(n_q, H, G, D).permute(1, 0, 2, 3).reshape(H, n_q * G, D).contiguous()
        sc = torch.matmul(Qh, Xh.transpose(1, 2).contiguous()) * scale
        ref = torch.matmul(torch.softmax(sc, dim=-1), Vh)      # [H][n_q G][128]
        ref = ref.view(H, n_q, G, D).permute(1, 0, 2, 3).reshape(n_q, H * G, D)
        vc = bk.alloc_packed(n_tok, H, bits, q, dev)
        bk.wushkv_quantize_values(V, bits, q, vc)
        row0 = torch.zeros(n_q, dtype=torch.int64, device=dev)
        lens = torch.full((n_q,), n_tok, dtype=torch.int32, device=dev)
        for name, (Tm, Tim) in (("identity", (np.stack([np.eye(D, dtype=np.float32)] * H),) * 2),
                                ("hadamard", (np.stack([Hd / 8.0] * H).astype(np.float32),
                                              np.stack([Hd / 16.0] * H).astype(np.float32))),
                                ("T_k", (T, Ti))):
            kc = bk.alloc_packed(n_tok, H, bits, q, dev)
            bk.wushkv_quantize_keys(K, pos, rope, bk.Transform(Tm), bits, q, kc)
            qp = bk.wushkv_pair_queries(Qb, bk.Transform(Tim))
            o = bk.wushkv_decode_attention(qp, kc, vc, H, bits, q, row0, lens, n_tok, scale)
            errs[name].append(float(((o - ref) ** 2).sum() / (ref ** 2).sum()))
    torch.cuda.synchronize()
    return {k: {"geomean": float(np.exp(np.mean(np.log(v)))), "per_layer": [round(x, 6) for x in v]}
            for k, v in errs.items()} | {"layers": layers, "tokens": n_tok, "queries": n_q, "bits": bits,
                                         "query_scale": q_scale,
                                         "note": "synthetic heavy-tailed keys and values; no model weights"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=4000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--one-stream", action="store_true",
                    help="issue keys and values of the throughput pass on one stream")
    ap.add_argument("--light", action="store_true",
                    help="few repetitions in the sections beside the throughput pass (for counter runs)")
    ap.add_argument("--quality", action="store_true",
                    help="also report the attention-output error of the quantized cache per key transform")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the cache write path shards by KV head, token range or layer "
              "with no exchange between GPUs; bench.py times one MI355X only.", file=sys.stderr)
        return 2

    import torch
    import synth
    import bit_kv_cache_rope_amd as bk

    w = synth.WORKLOADS["qwen3_8b_prefill"]
    N, H, bits = w.tokens, w.heads, 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q = bk.sym(w.clip_alpha)

    K = synth.kv(w, 0, "K")
    V = synth.kv(w, 0, "V")
    pos = synth.positions(w)
    T, _ = synth.transform(w, 0)
    rope = bk.Rope(w.theta, 1 << 17)
    tk = bk.Transform(T)

    def dev_bf16(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    set_bytes = N * (key_bytes_per_token(H, bits) + value_bytes_per_token(H, bits))
    n_sets = max(2, -(-2 * MALL_BYTES // set_bytes) + 1)
    Kd, Vd = dev_bf16(K), dev_bf16(V)
    sets = []
    for i in range(n_sets):
        sets.append(dict(K=Kd.clone(), V=Vd.clone(), pos=torch.from_numpy(pos).to(dev),
                         ko=bk.alloc_packed(N, H, bits, q, dev), vo=bk.alloc_packed(N, H, bits, q, dev)))
    del Kd, Vd
    stream = torch.cuda.Stream()  # the launch stream (default priority, like every stream here)
    vstream = stream if args.one_stream else torch.cuda.Stream()
    # launches with their arguments marshalled once, so the host stays ahead of the GPU
    calls = [(bk.prepare_quantize_keys(s["K"], s["pos"], rope, tk, bits, q, s["ko"], stream=stream),
              bk.prepare_quantize_values(s["V"], bits, q, s["vo"], stream=stream)) for s in sets]
    # the throughput pass issues each step's values on their own stream: keys and
    # values of a step are independent, so the GPU may run one beside the other
    tcalls = [(k, bk.prepare_quantize_values(s["V"], bits, q, s["vo"], stream=vstream))
              for (k, _), s in zip(calls, sets)]

    def step(i):
        kcall, vcall = calls[i % n_sets]
        kcall()
        vcall()

    def new_events(n, k):
        """n groups of k timing events, recorded once on the launch stream so
        that they exist."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(k)] for _ in range(n)]
        for g in ev:
            for e in g:
                e.record(stream)
        torch.cuda.synchronize()
        return ev

    for i in range(min(args.warmup, 10)):
        step(i)
    # Warm-up: W steps of the throughput pass.  The chip takes some 0.1 s of
    # load to reach its sustained clocks (a 200-step pass right after a short
    # warm-up ran 20% slower than the same pass repeated).
    for i in range(args.warmup):
        kcall, vcall = tcalls[i % n_sets]
        kcall()
        vcall()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps, {n_sets} buffer sets)", file=sys.stderr, flush=True)

    # Throughput: K steps back to back (keys on the launch stream, values on a
    # second one), bracketed by device-wide synchronizations only.
    t0 = time.perf_counter()
    for i in range(args.steps):
        kcall, vcall = tcalls[i % n_sets]
        kcall()
        vcall()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps in {elapsed:.3f} s", file=sys.stderr, flush=True)
    # Per-kernel durations: the same K steps again on the launch stream, each
    # kernel recording a pair of HIP events at its own start and end
    # (hipExtLaunchKernel through wushkv_debug_time_next_launch), so the figure
    # is the kernel's duration without its dispatch latency.  (Events recorded
    # around a launch read 3-4 us more.)
    evs = new_events(args.steps, 4)
    for i in range(args.steps):
        kcall, vcall = calls[i % n_sets]
        bk.wushkv_debug_time_next_launch(evs[i][0], evs[i][1])
        kcall()
        bk.wushkv_debug_time_next_launch(evs[i][2], evs[i][3])
        vcall()
    torch.cuda.synchronize()
    key_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    val_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])

    if args.copy_probe:
        a = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    # achievable device-copy rate on this chip, same run: 256 MiB read + 256 MiB written per
    # copy (beyond the MALL), timed with events on the launch stream
    ca = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    cb = torch.empty_like(ca)
    with torch.cuda.stream(stream):
        for _ in range(3):
            cb.copy_(ca)
        ce = new_events(1, 2)[0]
        n_copy = 2 if args.light else 20
        ce[0].record(stream)
        for _ in range(n_copy):
            cb.copy_(ca)
        ce[1].record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * (256 << 20) * n_copy / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e9
    del ca, cb

    # ---- read path on the same data (keys back through T_k^-1, values plain), reported alongside
    _, Ti = synth.transform(w, 0)
    tki = bk.Transform(Ti)
    # one output pair per buffer set, so that the written bytes (2 x 64 MiB per
    # set) are not served from the MALL
    outs = [(torch.empty((N, H, D), dtype=torch.bfloat16, device=dev),
             torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)) for _ in sets]
    rcalls = [(bk.prepare_dequantize(s["ko"], N, H, bits, q, ok, T_k_inv=tki, stream=stream),
               bk.prepare_dequantize(s["vo"], N, H, bits, q, ov, stream=stream)) for s, (ok, ov) in zip(sets, outs)]
    rd = new_events(50, 4)
    for i in range(60):
        kc, vc = rcalls[i % n_sets]
        e = rd[i - 10] if i >= 10 else None
        if e:
            bk.wushkv_debug_time_next_launch(e[0], e[1])
        kc()
        if e:
            bk.wushkv_debug_time_next_launch(e[2], e[3])
        vc()
    torch.cuda.synchronize()
    rk_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in rd]))
    rv_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in rd]))

    # ---- decode append (64 sequences x 1 token, into 64 x 32768-row caches), reported alongside:
    # a layer's K and V calls back to back on the two streams, and each kernel's own duration
    wd = synth.WORKLOADS["decode_append"]
    dn = wd.tokens
    drows = 64 * 32768
    dslots = torch.from_numpy(synth.slots(wd)).to(dev)
    dpos = torch.from_numpy(synth.positions(wd)).to(dev)
    dK, dV = dev_bf16(synth.kv(wd, 0, "K")), dev_bf16(synth.kv(wd, 0, "V"))
    dT, _ = synth.transform(wd, 0)
    dtk = bk.Transform(dT)
    dkc = bk.alloc_packed(drows, H, bits, q, dev).with_slots(dslots)
    dvc = bk.alloc_packed(drows, H, bits, q, dev).with_slots(dslots)
    dk = bk.prepare_quantize_keys(dK, dpos, rope, dtk, bits, q, dkc, stream=stream)
    dv = bk.prepare_quantize_values(dV, bits, q, dvc, stream=vstream)
    rep = 1 if args.light else 10  # repetition scale of the sections beside the throughput pass
    for _ in range(20 * rep):
        dk()
        dv()
    torch.cuda.synchronize()
    n_dec = 36 * 2 * rep
    t0 = time.perf_counter()
    for _ in range(n_dec):
        dk()
        dv()
    torch.cuda.synchronize()
    dec_layer_us = (time.perf_counter() - t0) / n_dec * 1e6
    dev_ev = new_events(5 * rep, 4)
    for e in dev_ev:
        bk.wushkv_debug_time_next_launch(e[0], e[1])
        dk()
        bk.wushkv_debug_time_next_launch(e[2], e[3])
        bk.prepare_quantize_values(dV, bits, q, dvc, stream=stream)()
    torch.cuda.synchronize()
    dec_k_us = float(np.mean([e[0].elapsed_time(e[1]) for e in dev_ev])) * 1e3
    dec_v_us = float(np.mean([e[2].elapsed_time(e[3]) for e in dev_ev])) * 1e3
    # 36 layers' decode K and V calls (one token per sequence) captured in one HIP graph and
    # replayed: one launch per decode step for all layers (same inputs and caches for every
    # layer here; each layer's kernels do the same work).  All on one stream (keys and values
    # forked onto two streams and joined per layer inside the graph ran 423 against 319 us).
    gst = torch.cuda.Stream()
    gk = bk.prepare_quantize_keys(dK, dpos, rope, dtk, bits, q, dkc, stream=gst)
    gv = bk.prepare_quantize_values(dV, bits, q, dvc, stream=gst)
    gk()
    gv()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gst):
        for _ in range(36):
            gk()
            gv()
    for _ in range(2 * rep):
        graph.replay()
    torch.cuda.synchronize()
    n_rep = 10 * rep
    t0 = time.perf_counter()
    for _ in range(n_rep):
        graph.replay()
    torch.cuda.synchronize()
    graph_step_us = (time.perf_counter() - t0) / n_rep * 1e6
    # 16-token chunks: 64 sequences append 16 consecutive positions each (1024 tokens per layer call)
    cbase = np.minimum(synth.positions(wd), 32768 - 16)
    cpos = torch.from_numpy((cbase[:, None] + np.arange(16)).reshape(-1).astype(np.int32)).to(dev)
    cslots = torch.from_numpy((np.arange(dn)[:, None] * 32768 + cbase[:, None] + np.arange(16)).reshape(-1)).to(dev)
    cK = dev_bf16(synth.kv(wd, 0, "K", 0, 16 * dn))
    cV = dev_bf16(synth.kv(wd, 0, "V", 0, 16 * dn))
    ck = bk.prepare_quantize_keys(cK, cpos, rope, dtk, bits, q, dkc.with_slots(cslots), stream=stream)
    cv = bk.prepare_quantize_values(cV, bits, q, dvc.with_slots(cslots), stream=vstream)
    for _ in range(20 * rep):
        ck()
        cv()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_dec):
        ck()
        cv()
    torch.cuda.synchronize()
    chunk_layer_us = (time.perf_counter() - t0) / n_dec * 1e6

    # ---- one GPU's share under 8-way KV-head parallelism: the benchmark layer's tokens for a
    # single KV head (keys and values of 32768 tokens x 1 head, 18 MB), kernel-recorded events
    Kh = sets[0]["K"][:, :1].contiguous()
    Vh = sets[0]["V"][:, :1].contiguous()
    tk1 = bk.Transform(T[:1])
    ko1, vo1 = bk.alloc_packed(N, 1, bits, q, dev), bk.alloc_packed(N, 1, bits, q, dev)
    k1c = bk.prepare_quantize_keys(Kh, sets[0]["pos"], rope, tk1, bits, q, ko1, stream=stream)
    v1c = bk.prepare_quantize_values(Vh, bits, q, vo1, stream=stream)
    rep1 = 1 if args.light else 10
    for _ in range(20 * rep1):
        k1c()
        v1c()
    torch.cuda.synchronize()
    ev1 = new_events(5 * rep1, 4)
    for e in ev1:
        bk.wushkv_debug_time_next_launch(e[0], e[1])
        k1c()
        bk.wushkv_debug_time_next_launch(e[2], e[3])
        v1c()
    torch.cuda.synchronize()
    h1_k_us = float(np.mean([e[0].elapsed_time(e[1]) for e in ev1])) * 1e3
    h1_v_us = float(np.mean([e[2].elapsed_time(e[3]) for e in ev1])) * 1e3
    h1_bytes = N * (key_bytes_per_token(1, bits) + value_bytes_per_token(1, bits)) + D * D * 2

    # ---- structured key transforms through the same dense path (Hadamard / 8; four 32 x 32
    # blocks on the diagonal): the key kernel's time on the benchmark layer, one buffer set
    Hd = np.array([[1.0]])
    while Hd.shape[0] < D:
        Hd = np.block([[Hd, Hd], [Hd, -Hd]])
    blk = np.zeros((H, D, D), np.float32)
    brng = np.random.default_rng(77)
    for hh in range(H):
        for bb in range(4):
            blk[hh, 32 * bb:32 * bb + 32, 32 * bb:32 * bb + 32] = brng.standard_normal((32, 32)) / np.sqrt(32) + 2 * np.eye(32)
    struct_us = {}
    for tname, Tm in (("dense", T), ("hadamard", np.stack([Hd / 8.0] * H).astype(np.float32)),
                      ("block_diagonal", blk)):
        th = bk.Transform(Tm)
        call = bk.prepare_quantize_keys(sets[0]["K"], sets[0]["pos"], rope, th, bits, q, sets[0]["ko"], stream=stream)
        for _ in range(20 * rep):
            call()
        tev = new_events(5 * rep, 2)
        for e in tev:
            bk.wushkv_debug_time_next_launch(e[0], e[1])
            call()
        torch.cuda.synchronize()
        struct_us[tname] = round(float(np.mean([e[0].elapsed_time(e[1]) for e in tev])) * 1e3, 2)
        del th

    # ---- decode attention over the packed caches (64 sequences of the decode workload's lengths,
    # 32 query heads over 8 KV heads), reported alongside: the caches hold random codes and steps
    att_q = 32
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    for c in (dkc, dvc):
        c.codes.copy_(torch.randint(0, 256, c.codes.shape, dtype=torch.uint8, device=dev, generator=g))
        c.scales.copy_((torch.rand(c.scales.shape, device=dev, generator=g) * 0.05 + 0.02).to(torch.float16))
    att_len = synth.positions(wd).astype(np.int64) + 1
    att_lens = torch.from_numpy(att_len.astype(np.int32)).to(dev)
    att_row0 = torch.arange(dn, dtype=torch.int64, device=dev) * 32768
    _, dTi = synth.transform(wd, 0)
    dtki = bk.Transform(dTi)
    att_Q = (torch.randn((dn, att_q, D), device=dev, generator=g) * 3.0).to(torch.bfloat16)
    att_qp = torch.empty((dn, att_q, D), dtype=torch.bfloat16, device=dev)
    att_ws = torch.empty(bk.wushkv_decode_attention_workspace(dn, att_q, H, 32768) // 4, dtype=torch.float32,
                         device=dev)
    att_out = torch.empty((dn, att_q, D), dtype=torch.float32, device=dev)
    att = bk.prepare_decode_attention(att_qp, dkc, dvc, H, bits, q, att_row0, att_lens, 32768, 1.0 / np.sqrt(D),
                                      att_ws, att_out, stream=stream)
    with torch.cuda.stream(stream):
        for _ in range(2 * rep):
            bk.wushkv_pair_queries(att_Q, dtki, out=att_qp, stream=stream)
            att()
    torch.cuda.synchronize()
    att_ev = new_events(5 * rep, 6)
    for e in att_ev:
        bk.wushkv_debug_time_next_launch(e[0], e[1])
        bk.wushkv_pair_queries(att_Q, dtki, out=att_qp, stream=stream)
        e[4].record(stream)
        bk.wushkv_debug_time_next_launch(e[2], e[3])
        att()
        e[5].record(stream)
    torch.cuda.synchronize()
    att_pair_us = float(np.mean([e[0].elapsed_time(e[1]) for e in att_ev])) * 1e3
    att_kernel_us = float(np.mean([e[2].elapsed_time(e[3]) for e in att_ev])) * 1e3
    att_call_us = float(np.mean([e[4].elapsed_time(e[5]) for e in att_ev])) * 1e3
    att_bytes = int(att_len.sum()) * H * 2 * (16 * bits + 2) + dn * att_q * D * 2 + dn * 2 * 12
    att_flops = 4.0 * int(att_len.sum()) * att_q * D

    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = N * args.steps / elapsed
    kb = N * key_bytes_per_token(H, bits) + H * D * D * 2  # + T~ read once per launch
    vb = N * value_bytes_per_token(H, bits)
    key_us = float(key_ms.mean()) * 1e3
    val_us = float(val_ms.mean()) * 1e3
    achieved = kb / (key_us * 1e-6) / 1e9
    key_flops = 2.0 * N * H * D * D
    traffic = read_traffic()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else round(
                    (traffic["fetch_bytes_per_launch"] + traffic["write_bytes_per_launch"]) / 1e6, 3)}
    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_prefill_layer", "tokens": N, "kv_heads": H, "head_dim": D,
                   "bits": bits, "quantizer": "symmetric, clip 2.0 x RMS, fp16 step per token-head",
                   "kv_dtype": "bf16", "rope_theta": w.theta, "buffer_sets": n_sets,
                   "streams": 1 if args.one_stream else 2},
        "roofline": roofline,
        "achievable_copy": {"gbs": round(copy_gbs, 1), "keys_frac": round(achieved / copy_gbs, 4),
                            "step_frac": round((kb + vb) / (ms_per_step * 1e-3) / 1e9 / copy_gbs, 4),
                            "note": "device-to-device copy of 256 MiB (read + write) in the same run"},
        "kernels": {
            "keys_us": round(key_us, 2), "values_us": round(val_us, 2),
            "keys_us_p10_p50_p90": [round(float(np.percentile(key_ms, x)) * 1e3, 2) for x in (10, 50, 90)],
            "values_us_p10_p50_p90": [round(float(np.percentile(val_ms, x)) * 1e3, 2) for x in (10, 50, 90)],
            "keys_algorithmic_bytes": kb, "values_algorithmic_bytes": vb,
            "values_gbs": round(vb / (val_us * 1e-6) / 1e9, 1),
            "step_gbs": round((kb + vb) / (ms_per_step * 1e-3) / 1e9, 1),
            "keys_mfma_tflops": round(key_flops / (key_us * 1e-6) / 1e12, 2),
            "keys_mfma_frac": round(key_flops / (key_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic_note": None if traffic is None else "roofline.traffic in MB per key launch (FETCH+WRITE)",
        },
        "read_path": {
            "keys_through_T_inv_us": round(rk_ms * 1e3, 2), "values_us": round(rv_ms * 1e3, 2),
            "tokens_per_s": round(N / ((rk_ms + rv_ms) * 1e-3), 1),
            "keys_gbs": round((N * (H * 16 * bits + H * 2 + H * D * 2) + H * D * D * 2) / (rk_ms * 1e-3) / 1e9, 1),
            "out_dtype": "bf16",
        },
        "decode_append": {
            "tokens_per_layer": dn, "cache_rows": drows, "layer_us": round(dec_layer_us, 2),
            "keys_kernel_us": round(dec_k_us, 2), "values_kernel_us": round(dec_v_us, 2),
            "note": "one layer's K and V calls back to back, keys and values on two streams",
            "graph_36_layers_us": round(graph_step_us, 2),
            "graph_note": "36 layers' K and V calls in one HIP graph on one stream, replayed back to back",
            "chunk16_tokens_per_layer": 16 * dn, "chunk16_layer_us": round(chunk_layer_us, 2),
            "chunk16_tokens_per_s": round(16 * dn / (chunk_layer_us * 1e-6), 1),
        },
        "one_kv_head_share": {"tokens": N, "kv_heads": 1, "keys_us": round(h1_k_us, 2), "values_us": round(h1_v_us, 2),
                              "gbs": round(h1_bytes / ((h1_k_us + h1_v_us) * 1e-6) / 1e9, 1),
                              "note": "one GPU's share under 8-way KV-head parallelism; keys then values on one stream"},
        "structured_transforms_keys_us": dict(struct_us, note="key kernel on the benchmark layer, one buffer set"),
        "decode_attention": {
            "sequences": dn, "q_heads": att_q, "kv_heads": H, "bits": bits,
            "cached_tokens": int(att_len.sum()), "max_len": int(att_len.max()),
            "pair_queries_us": round(att_pair_us, 2), "attention_kernel_us": round(att_kernel_us, 2),
            "call_us": round(att_call_us, 2), "algorithmic_bytes": att_bytes,
            "attention_gbs": round(att_bytes / (att_kernel_us * 1e-6) / 1e9, 1),
            "attention_hbm_frac": round(att_bytes / (att_kernel_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(att_flops / (att_kernel_us * 1e-6) / 1e12, 2),
            "note": "packed 2-bit K and V read once; call_us = attention and split combine launched back to back",
        },
    }
    if args.quality:
        out["quality"] = {f"{b}bit": quality_report(torch, synth, bk, dev, bits=b) for b in (2, 4)}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle (single thread, one layer)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, synth)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
