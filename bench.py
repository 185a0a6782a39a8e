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
                      for f in ("keys.hip", "key_codes.h", "device_common.h")]


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


def host_cpu() -> dict:
    """Host cores visible to this process and the CPU model (/proc/cpuinfo)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"host_cores": cores, "cpu_model": model}


def cpu_baseline(w, synth, seconds_hint: float = 6.0) -> dict:
    """The CPU oracle as it stands, timed on this host: the benchmark layer
    single-threaded (the headline figure) and with all the process's cores
    (at most 16 threads), plus single-threaded slices of the other workloads
    (layer 0, first 8192 tokens; the decode workload's 64 tokens)."""
    import oracle
    oracle.build()
    hc = host_cpu()
    n = w.tokens
    K = synth.kv(w, 0, "K", 0, n)
    V = synth.kv(w, 0, "V", 0, n)
    pos = synth.positions(w, 0, n)
    T, _ = synth.transform(w, 0)

    def layer_rate(threads, min_reps):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.quantize_keys(K, pos, T, w.theta, 2, oracle.sym(w.clip_alpha), threads=threads)
            oracle.quantize_values(V, 2, oracle.sym(w.clip_alpha), threads=threads)
            reps += 1
            dt = time.perf_counter() - t0
            if reps >= min_reps and dt >= seconds_hint * 0.5:
                return reps, dt

    reps, dt = layer_rate(1, 1)
    all_threads = max(1, min(16, hc["host_cores"]))
    reps_n, dt_n = layer_rate(all_threads, 2)
    slices = {}
    for name, bits in (("decode_append", 2), ("qwen3_32b_full", 3), ("qwen3_32b_full", 4), ("affine_pct", 2)):
        ws = synth.WORKLOADS[name]
        ns = min(8192, ws.tokens)
        Ks, Vs = synth.kv(ws, 0, "K", 0, ns), synth.kv(ws, 0, "V", 0, ns)
        ps = synth.positions(ws, 0, ns)
        Ts, _ = synth.transform(ws, 0)
        qz = oracle.sym(ws.clip_alpha) if ws.quant == "sym" else oracle.affine(ws.p_lo, ws.p_hi)
        t0 = time.perf_counter()
        oracle.quantize_keys(Ks, ps, Ts, ws.theta, bits, qz, threads=1)
        oracle.quantize_values(Vs, bits, qz, threads=1)
        slices[f"{name}_{bits}bit"] = {"tokens": ns, "tokens_per_s": round(ns / (time.perf_counter() - t0), 1)}
    return {"value": reps * n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} pass(es) over one full layer of the workload ({n} tokens x {w.heads} heads, "
                      f"K and V), single-threaded, {dt:.1f} s",
            "host_cores": hc["host_cores"], "cpu_model": hc["cpu_model"],
            "all_cores": {"value": round(reps_n * n / dt_n, 1), "unit": "tokens/s", "threads": all_threads,
                          "sample": f"{reps_n} passes over the same layer, {dt_n:.1f} s"},
            "other_workloads_single_thread": slices}


def kernel_us(torch, bk, stream, call, reps: int, warm: int = 3) -> float:
    """Mean duration in us of the kernel `call` launches, from the pair of HIP
    events that the kernel itself records at its start and end
    (wushkv_debug_time_next_launch), so dispatch latency is excluded."""
    for _ in range(warm):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    for e0, e1 in ev:
        bk.wushkv_debug_time_next_launch(e0, e1)
        call()
    torch.cuda.synchronize()
    return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3


def other_workloads(torch, synth, bk, dev, stream, rope, light=False) -> dict:
    """Kernel times of the other workloads at their full per-layer sizes (layer
    0), as fractions of the 8 TB/s roofline of their algorithmic bytes: the tiny
    workload (launch-bound), the Qwen3-32B-shaped layer at 3 and 4 bits with the
    read back through T_k^-1, and the percentile-affine layer (16 x 16384
    tokens) with its read back.  Read-path outputs are bf16."""
    reps = 2 if light else 10
    res = {}

    def dev_t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    for name, bits_list in (("tiny", (2,)), ("qwen3_32b_full", (3, 4)), ("affine_pct", (2,))):
        w = synth.WORKLOADS[name]
        N, H = w.tokens, w.heads
        q = bk.sym(w.clip_alpha) if w.quant == "sym" else bk.affine(w.p_lo, w.p_hi)
        K, V = dev_t(synth.kv(w, 0, "K")), dev_t(synth.kv(w, 0, "V"))
        pos = torch.from_numpy(synth.positions(w)).to(dev)
        T, Ti = synth.transform(w, 0)
        tk, tki = bk.Transform(T), bk.Transform(Ti)
        esz = 4 if w.dtype == "f32" else 2
        nsc = 1 if w.quant == "sym" else 8  # fp16 step (sym) or 4 steps + 4 zeros (affine) per vector
        for bits in bits_list:
            ko, vo = bk.alloc_packed(N, H, bits, q, dev), bk.alloc_packed(N, H, bits, q, dev)
            kc = bk.prepare_quantize_keys(K, pos, rope, tk, bits, q, ko, stream=stream)
            vc = bk.prepare_quantize_values(V, bits, q, vo, stream=stream)
            rec = N * H * (16 * bits + 2 * nsc)
            kb = N * H * D * esz + 4 * N + rec + H * D * D * 2
            vb = N * H * D * esz + rec
            k_us, v_us = kernel_us(torch, bk, stream, kc, reps), kernel_us(torch, bk, stream, vc, reps)
            ent = {"tokens": N, "kv_heads": H, "bits": bits, "quantizer": w.quant,
                   "keys_us": round(k_us, 2), "values_us": round(v_us, 2),
                   "keys_hbm_frac": round(kb / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "values_hbm_frac": round(vb / (v_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "tokens_per_s": round(N / ((k_us + v_us) * 1e-6), 1)}
            if w.round_trip:
                ok = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)
                ov = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)
                rk = bk.prepare_dequantize(ko, N, H, bits, q, ok, T_k_inv=tki, stream=stream)
                rv = bk.prepare_dequantize(vo, N, H, bits, q, ov, stream=stream)
                rk_us, rv_us = kernel_us(torch, bk, stream, rk, reps), kernel_us(torch, bk, stream, rv, reps)
                rb = rec + N * H * D * 2
                ent.update({"read_keys_T_inv_us": round(rk_us, 2), "read_values_us": round(rv_us, 2),
                            "read_keys_hbm_frac": round((rb + H * D * D * 2) / (rk_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                            "read_values_hbm_frac": round(rb / (rv_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
                del ok, ov
            res[f"{name}_{bits}bit"] = ent
            del ko, vo
        del K, V, tk, tki
        torch.cuda.empty_cache()
    res["note"] = ("layer 0 at full size; kernel-recorded events; fractions of 8 TB/s of algorithmic bytes "
                   "(inputs in, packed records and fp16 steps/zeros out, T~ once per launch; reads: records in, "
                   "bf16 out)")
    return res


def kernel_label(name: str) -> str:
    """Short kernel name: namespaces and the argument list dropped, template arguments kept."""
    name = name.replace("void ", "").replace("wushkv::(anonymous namespace)::", "").replace("wushkv::", "")
    return re.sub(r"\((?:[^()]|\([^()]*\))*\)$", "", name).strip()


def summarize_pmc(dirs, pattern: str) -> str:
    """Markdown table of rocprofv3 counter collections (one directory per --pmc pass,
    each holding run_counter_collection.csv): per kernel and grid size, the mean of
    each counter over its dispatches."""
    import csv
    from collections import defaultdict
    acc = defaultdict(lambda: defaultdict(list))
    counters = []
    for d in dirs:
        with open(os.path.join(d, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                k = (kernel_label(r["Kernel_Name"]), int(r["Grid_Size"]))
                if not re.search(pattern, k[0]):
                    continue
                c = r["Counter_Name"]
                if c not in counters:
                    counters.append(c)
                acc[k][c].append(float(r["Counter_Value"]))
    lines = ["| kernel | grid | dispatches | " + " | ".join(counters) + " |",
             "|---|---|---|" + "---|" * len(counters)]
    for (name, grid), m in sorted(acc.items()):
        n = max(len(v) for v in m.values())
        vals = [f"{np.mean(m[c]):.4g}" if c in m else "" for c in counters]
        lines.append(f"| {name} | {grid} | {n} | " + " | ".join(vals) + " |")
    return "\n".join(lines)


def summarize_trace(d: str, pattern: str, part: str | None = None) -> str:
    """Markdown table of a rocprofv3 --kernel-trace run (run_kernel_trace.csv): per kernel
    and grid size, the number of dispatches and their mean, min and max duration.
    `part` = "a:b" keeps dispatches a .. b-1 of each kernel and grid in start order."""
    import csv
    from collections import defaultdict
    acc = defaultdict(list)
    with open(os.path.join(d, "run_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            name = kernel_label(r["Kernel_Name"])
            if re.search(pattern, name):
                acc[(name, int(r["Grid_Size_X"]))].append(
                    (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    lines = ["| kernel | grid | calls | average us | min us | max us |", "|---|---|---|---|---|---|"]
    for (name, grid), sv in sorted(acc.items()):
        v = [x[1] for x in sorted(sv)]
        if part:
            a, b = (int(x) if x else None for x in part.split(":"))
            v = v[a:b]
        if not v:
            continue
        lines.append(f"| {name} | {grid} | {len(v)} | {np.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(lines)


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
                    help="attention-output error over 4 layers at 2 and 4 bits (default: 1 layer, 2 bits)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="print a table of rocprofv3 --pmc output directories and exit (no GPU)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a table of a rocprofv3 --kernel-trace output directory and exit (no GPU)")
    ap.add_argument("--trace-slice", metavar="A:B",
                    help="with --summarize-trace: dispatches A .. B-1 of each kernel, in start order")
    ap.add_argument("--kernels", default=".",
                    help="regular expression selecting the kernels the summaries list")
    args = ap.parse_args()
    if args.summarize_pmc or args.summarize_trace:
        if args.summarize_pmc:
            print(summarize_pmc(args.summarize_pmc, args.kernels))
        if args.summarize_trace:
            print(summarize_trace(args.summarize_trace, args.kernels, args.trace_slice))
        return 0
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

    for i in range(10):
        step(i)
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

    # ---- decode append (64 sequences x 1 token per layer, into 64 x 32768-row caches through
    # slots), reported alongside: the 36 layers each with their own K, V and T~ (the caches are
    # shared); the fused K+V call (one kernel per layer) and, for comparison, the separate calls
    wd = synth.WORKLOADS["decode_append"]
    dn = wd.tokens
    drows = 64 * 32768
    dslots = torch.from_numpy(synth.slots(wd)).to(dev)
    dpos = torch.from_numpy(synth.positions(wd)).to(dev)
    dkc = bk.alloc_packed(drows, H, bits, q, dev).with_slots(dslots)
    dvc = bk.alloc_packed(drows, H, bits, q, dev).with_slots(dslots)
    dlayers = [dict(K=dev_bf16(synth.kv(wd, layer, "K")), V=dev_bf16(synth.kv(wd, layer, "V")),
                    tk=bk.Transform(synth.transform(wd, layer)[0])) for layer in range(wd.layers)]
    fused = [bk.prepare_quantize_kv(L["K"], L["V"], dpos, rope, L["tk"], bits, q, dkc, dvc, stream=stream)
             for L in dlayers]
    sep = [(bk.prepare_quantize_keys(L["K"], dpos, rope, L["tk"], bits, q, dkc, stream=stream),
            bk.prepare_quantize_values(L["V"], bits, q, dvc, stream=stream)) for L in dlayers]
    rep = 1 if args.light else 10  # repetition scale of the sections beside the throughput pass

    def host_rate(fns, n):
        """Wall time per call of the calls `fns` issued back to back, n rounds."""
        for _ in range(2):
            for f in fns:
                f()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            for f in fns:
                f()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / (n * len(fns)) * 1e6

    dec_fused_layer_us = host_rate(fused, 2 * rep)
    dec_sep_layer_us = host_rate([lambda k=k, v=v: (k(), v()) for k, v in sep], 2 * rep)
    # each kernel's own duration (events at its start and end), over the 36 layers
    fev = new_events(wd.layers * rep, 2)
    for i, e in enumerate(fev):
        bk.wushkv_debug_time_next_launch(e[0], e[1])
        fused[i % wd.layers]()
    sev = new_events(wd.layers * rep, 4)
    for i, e in enumerate(sev):
        k, v = sep[i % wd.layers]
        bk.wushkv_debug_time_next_launch(e[0], e[1])
        k()
        bk.wushkv_debug_time_next_launch(e[2], e[3])
        v()
    torch.cuda.synchronize()
    fk = np.array([e[0].elapsed_time(e[1]) for e in fev]) * 1e3
    dec_fused_kernel_us = float(np.median(fk))
    dec_k_us = float(np.median([e[0].elapsed_time(e[1]) for e in sev])) * 1e3
    dec_v_us = float(np.median([e[2].elapsed_time(e[3]) for e in sev])) * 1e3

    # one decode step as one HIP graph: the 36 layers' calls captured on one stream and replayed
    # back to back (the layer inputs, 18 MB, stay in the caches across replays)
    def graph_us(make):
        """Wall time per replay of one graph of the calls make(stream) issues."""
        gst = torch.cuda.Stream()
        fns = make(gst)
        for f in fns:
            f()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gst):
            for f in fns:
                f()
        for _ in range(2 * rep):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10 * rep):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / (10 * rep) * 1e6

    def fused_calls(st):
        return [bk.prepare_quantize_kv(L["K"], L["V"], dpos, rope, L["tk"], bits, q, dkc, dvc, stream=st)
                for L in dlayers]

    def separate_calls(st):
        out = []
        for L in dlayers:
            out.append(bk.prepare_quantize_keys(L["K"], dpos, rope, L["tk"], bits, q, dkc, stream=st))
            out.append(bk.prepare_quantize_values(L["V"], bits, q, dvc, stream=st))
        return out

    graph_step_us = graph_us(fused_calls)
    graph_sep_us = graph_us(separate_calls)
    # 16-token chunks: 64 sequences append 16 consecutive positions each (1024 tokens per layer call)
    cbase = np.minimum(synth.positions(wd), 32768 - 16)
    cpos = torch.from_numpy((cbase[:, None] + np.arange(16)).reshape(-1).astype(np.int32)).to(dev)
    cslots = torch.from_numpy((np.arange(dn)[:, None] * 32768 + cbase[:, None] + np.arange(16)).reshape(-1)).to(dev)
    cK = dev_bf16(synth.kv(wd, 0, "K", 0, 16 * dn))
    cV = dev_bf16(synth.kv(wd, 0, "V", 0, 16 * dn))
    ckc, cvc = dkc.with_slots(cslots), dvc.with_slots(cslots)
    cf = bk.prepare_quantize_kv(cK, cV, cpos, rope, dlayers[0]["tk"], bits, q, ckc, cvc, stream=stream)
    ck = bk.prepare_quantize_keys(cK, cpos, rope, dlayers[0]["tk"], bits, q, ckc, stream=stream)
    cv = bk.prepare_quantize_values(cV, bits, q, cvc, stream=stream)
    chunk_layer_us = host_rate([cf], 36 * rep)
    chunk_sep_layer_us = host_rate([lambda: (ck(), cv())], 36 * rep)

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

    # ---- structured key transforms (Hadamard / 8; four 32 x 32 blocks on the diagonal): the key
    # kernel's time on the benchmark layer, one buffer set, through the dense MFMA path, and
    # Hadamard / 8 also through the in-register fast Walsh-Hadamard path (Transform.hadamard)
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
                      ("block_diagonal", blk), ("hadamard_fwht", None)):
        th = bk.Transform(Tm) if Tm is not None else bk.Transform.hadamard(H)
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
    # the same batch over percentile-clipped affine caches (the same codes, four steps and four
    # zeros per record)
    rows_all = dkc.codes.shape[0]
    aff = [bk.PackedCache(c.codes, (torch.rand((rows_all, H, 4), device=dev, generator=g) * 0.05 + 0.02).to(torch.float16),
                          (torch.randn((rows_all, H, 4), device=dev, generator=g) * 0.2).to(torch.float16))
           for c in (dkc, dvc)]
    att_aff = bk.prepare_decode_attention(att_qp, aff[0], aff[1], H, bits, bk.affine(), att_row0, att_lens, 32768,
                                          1.0 / np.sqrt(D), att_ws, att_out, stream=stream)
    with torch.cuda.stream(stream):
        for _ in range(2 * rep):
            att_aff()
    torch.cuda.synchronize()
    aff_ev = new_events(5 * rep, 2)
    for e in aff_ev:
        bk.wushkv_debug_time_next_launch(e[0], e[1])
        att_aff()
    torch.cuda.synchronize()
    aff_kernel_us = float(np.mean([e[0].elapsed_time(e[1]) for e in aff_ev])) * 1e3
    aff_bytes = int(att_len.sum()) * H * 2 * (16 * bits + 16) + dn * att_q * D * 2 + dn * 2 * 12
    del aff, att_aff
    # the same batch over 3- and 4-bit symmetric caches (random codes and steps)
    width = {}
    for wb in (3, 4):
        wc = [bk.PackedCache(torch.randint(0, 256, (rows_all, H, 16 * wb), dtype=torch.uint8, device=dev, generator=g),
                             (torch.rand((rows_all, H), device=dev, generator=g) * 0.05 + 0.02).to(torch.float16))
              for _ in range(2)]
        att_w = bk.prepare_decode_attention(att_qp, wc[0], wc[1], H, wb, q, att_row0, att_lens, 32768,
                                            1.0 / np.sqrt(D), att_ws, att_out, stream=stream)
        with torch.cuda.stream(stream):
            for _ in range(2 * rep):
                att_w()
        torch.cuda.synchronize()
        w_ev = new_events(5 * rep, 2)
        for e in w_ev:
            bk.wushkv_debug_time_next_launch(e[0], e[1])
            att_w()
        torch.cuda.synchronize()
        w_us = float(np.mean([e[0].elapsed_time(e[1]) for e in w_ev])) * 1e3
        w_bytes = int(att_len.sum()) * H * 2 * (16 * wb + 2) + dn * att_q * D * 2 + dn * 2 * 12
        width[wb] = (round(w_us, 2), w_bytes, round(w_bytes / (w_us * 1e-6) / 8e12, 4))
        del wc, att_w

    # ---- the other workloads' kernels, each against the HBM roofline (kernel-recorded events,
    # one buffer set: every input is at least 256 MiB, beyond the MALL).
    other = other_workloads(torch, synth, bk, dev, stream, rope, light=args.light)

    # ---- throughput (the headline): W warm-up steps of the throughput pass, then K steps.
    # It runs after the sections above, so the chip is already at its sustained clocks (it
    # takes about 0.1 s of load to get there: a 200-step pass right after a short warm-up ran
    # 20% slower than the same pass repeated) even when W is small.
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
            "tokens_per_layer": dn, "layers": wd.layers, "cache_rows": drows,
            "fused_kernel_us": round(dec_fused_kernel_us, 2),
            "fused_kernel_us_p10_p90": [round(float(np.percentile(fk, 10)), 2), round(float(np.percentile(fk, 90)), 2)],
            "fused_layer_call_us": round(dec_fused_layer_us, 2),
            "graph_36_layers_us": round(graph_step_us, 2),
            "graph_note": "one decode step: the 36 layers' fused K+V calls (one kernel each) in one HIP graph, "
                          "replayed back to back",
            "separate_keys_kernel_us": round(dec_k_us, 2), "separate_values_kernel_us": round(dec_v_us, 2),
            "separate_layer_call_us": round(dec_sep_layer_us, 2),
            "graph_36_layers_separate_us": round(graph_sep_us, 2),
            "chunk16_tokens_per_layer": 16 * dn, "chunk16_layer_us": round(chunk_layer_us, 2),
            "chunk16_separate_layer_us": round(chunk_sep_layer_us, 2),
            "chunk16_tokens_per_s": round(16 * dn / (chunk_layer_us * 1e-6), 1),
            "note": "per layer: 36 distinct layers (K, V, T~ each); layer_call_us are wall time per call "
                    "issued back to back on one stream; kernel_us from events at the kernel's start and end",
        },
        "one_kv_head_share": {"tokens": N, "kv_heads": 1, "keys_us": round(h1_k_us, 2), "values_us": round(h1_v_us, 2),
                              "gbs": round(h1_bytes / ((h1_k_us + h1_v_us) * 1e-6) / 1e9, 1),
                              "note": "one GPU's share under 8-way KV-head parallelism; keys then values on one stream"},
        "structured_transforms_keys_us": dict(struct_us, note="key kernel on the benchmark layer, one buffer set; "
                                              "hadamard: H/8 through the dense MFMA path, hadamard_fwht: the same "
                                              "transform as an in-register fast Walsh-Hadamard transform"),
        "decode_attention": {
            "sequences": dn, "q_heads": att_q, "kv_heads": H, "bits": bits,
            "cached_tokens": int(att_len.sum()), "max_len": int(att_len.max()),
            "pair_queries_us": round(att_pair_us, 2), "attention_kernel_us": round(att_kernel_us, 2),
            "call_us": round(att_call_us, 2), "algorithmic_bytes": att_bytes,
            "attention_gbs": round(att_bytes / (att_kernel_us * 1e-6) / 1e9, 1),
            "attention_hbm_frac": round(att_bytes / (att_kernel_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(att_flops / (att_kernel_us * 1e-6) / 1e12, 2),
            "note": "packed 2-bit K and V read once; call_us = attention and split combine launched back to back",
            "affine_attention_kernel_us": round(aff_kernel_us, 2),
            "affine_algorithmic_bytes": aff_bytes,
            "affine_attention_hbm_frac": round(aff_bytes / (aff_kernel_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "affine_note": "the same batch and codes as affine caches (four fp16 steps and zeros per record)",
            "symmetric_widths": {f"{wb}bit": {"attention_kernel_us": v[0], "algorithmic_bytes": v[1], "attention_hbm_frac": v[2]}
                                 for wb, v in width.items()},
        },
        "other_workloads": other,
    }
    # attention-output error of the quantized cache per key transform: a light pass by default
    # (one layer, 2-bit), four layers at 2 and 4 bits with --quality
    from bit_kv_cache_rope_amd import quality
    if args.quality:
        out["quality"] = {f"{b}bit": quality.quality_report(synth, dev, bits=b, layers=4) for b in (2, 4)}
    else:
        out["quality"] = {"2bit": quality.quality_report(synth, dev, bits=2, layers=1, n_tok=2048, n_q=16)}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle (single thread, one layer)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, synth)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
