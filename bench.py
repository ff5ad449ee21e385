"""Verify-step benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4|3] [--single] [--no-cpu-baseline]
                    [--soak SECONDS]

A step is one pass of the whole verify path over one batch of synthetic input:
64 layers of 8-bit (the long-context pack, the headline) or 4-bit affine
group-quantized projections of 27B-like shape, multi-row attention over a bf16
KV cache on every fourth layer, the float32 lm_head and exact acceptance over
the vocabulary (logits mode). The step is captured once into a HIP graph and
replayed; inputs are resident in HBM when timing starts.

Printed (one JSON line), for the headline step (8-bit, M = 8, KV at 128k):
verify-step HBM GB/s over the step's algorithmic bytes (weights once + K/V once
per attention layer + the logit rows), its fraction of the 8 TB/s peak, ms per
step, cost(M)/cost(M=1) of the 64-layer stack for M = 1..16, a roofline record
of the dominant kernel (the skinny QMM, timed per launch with HIP events on its
stream), the acceptance call's µs, and the CPU oracle timed on a bounded sample
of the same workload. The same record for the 4-bit step (M = 4, KV at 16k) is
nested under "other_configs" (unless --single), with per-call records of the
multi-row attention at 8k and 32k context for M = 1..8 and the streaming-read
ceiling of the HBM.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "verify-step HBM GB/s (% of peak) and cost(M=8)/cost(M=1) at 27B shapes"

CONFIGS = {
    3: dict(bits=4, lm_bits=4, M=4, ctx=16384, temperature=0.7, top_k=0, top_p=0.95,
            workload="27B-shaped dense verify step: 64 layers 4-bit g64 (hidden 5120, MLP 17408, q/k/v/o, "
                     "gate/up/down), attention on 16 layers over bf16 KV at 16k context (Hq 24, Hkv 4, D 256), "
                     "M=4 rows (K=3 drafts), lm_head 248320 fp32 logits, exact acceptance T=0.7 top-p 0.95"),
    4: dict(bits=8, lm_bits=8, M=8, ctx=131072, temperature=1.0, top_k=20, top_p=0.95,
            workload="27B-shaped dense verify step, 8-bit pack: 64 layers 8-bit g64, attention on 16 layers over "
                     "bf16 KV at 128k context, M=8 rows (K=7 drafts), lm_head 248320 fp32 logits, exact acceptance "
                     "T=1.0 top-k 20 + top-p 0.95"),
}


# The profiled commands whose CSV output --summarize-profiles reads (run from the
# repository root on one MI355X, output under <out>).
PROFILE_CMDS = {
    "kt": "rocprofv3 --kernel-trace --stats -f csv -d <out>/kt -o kt -- python3 bench.py --config {config} --single "
          "--steps 5 --warmup 1 --no-ratio --no-cpu-baseline --no-next --no-extras > <out>/kt.out",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d <out>/fetch -o fetch -- python3 bench.py --config {config} "
             "--single --steps 1 --warmup 0 --layers 8 --no-ratio --no-cpu-baseline --no-next --no-extras "
             "--copy-calibration",
    "write": "rocprofv3 --pmc WRITE_SIZE -f csv -d <out>/write -o write -- python3 bench.py --config {config} "
             "--single --steps 1 --warmup 0 --layers 8 --no-ratio --no-cpu-baseline --no-next --no-extras "
             "--copy-calibration",
    "attn_fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d <out>/fetch -o fetch -- python3 bench.py --attn-counters "
                  "--copy-calibration",
    "attn_write": "rocprofv3 --pmc WRITE_SIZE -f csv -d <out>/write -o write -- python3 bench.py --attn-counters "
                  "--copy-calibration",
    "curve_fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d <out>/fetch -o fetch -- python3 bench.py "
                   "--qmm-curve-counters {bits} --copy-calibration",
    "curve_write": "rocprofv3 --pmc WRITE_SIZE -f csv -d <out>/write -o write -- python3 bench.py "
                   "--qmm-curve-counters {bits} --copy-calibration",
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_weights(cfg, torch, seed: int, T_cap: int):
    """Synthetic weights on the device: uniform code words, scales N(0.02, 0.005), biases N(0, 0.01),
    generated row-major and packed into the tiled layout one matrix at a time; KV caches N(0, 1)."""
    from speculative_decoding_verify_vq_amd.stack import QPack, StackWeights
    from synth import bf16_normal_torch, random_words_torch
    dev = torch.device("cuda")
    w = StackWeights()
    sh = cfg.shapes()

    def pack(N, K, bits, s):
        wq = random_words_torch(N * K * bits // 32, s, dev)
        sc = bf16_normal_torch((N, K // 64), 0.02, 0.005, s + 100000, dev)
        bi = bf16_normal_torch((N, K // 64), 0.0, 0.01, s + 200000, dev)
        p = QPack.from_rows(wq, sc, bi, bits, N, K)
        torch.cuda.synchronize()
        del wq, sc, bi
        return p

    s = seed
    for li in range(cfg.layers):
        lay = {}
        for name in ("qkv", "o", "gate_up", "down"):
            N, K = sh[name]
            s += 1
            lay[name] = pack(N, K, cfg.bits, s)
        w.layers.append(lay)
    N, K = sh["lm_head"]
    w.lm_head = pack(N, K, cfg.lm_bits, seed + 7)
    for a in range(cfg.n_attn):
        w.k_cache.append(bf16_normal_torch((cfg.Hkv, T_cap, cfg.D), 0.0, 1.0, seed + 300000 + a, dev))
        w.v_cache.append(bf16_normal_torch((cfg.Hkv, T_cap, cfg.D), 0.0, 1.0, seed + 400000 + a, dev))
    torch.cuda.synchronize()
    return w


def capture(torch, fn):
    """Warm up fn once on a side stream, then capture it into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, steps: int, warmup: int) -> float:
    """ms per replay over exactly `steps` replays after `warmup` untimed ones."""
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def replay_times(torch, g, n: int) -> list:
    """ms of each of n back-to-back replays (an event between consecutive replays,
    no synchronisation inside the run)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record()
    for i in range(n):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]


def percentiles(xs, ps=(10, 50, 90, 99)) -> dict:
    a = np.sort(np.asarray(xs, dtype=np.float64))
    return {f"p{p}": round(float(np.percentile(a, p)), 4) for p in ps}


def soak(torch, g, seconds: float, step_bytes: float) -> dict:
    """Replays the step back to back for `seconds`, in windows of about one
    second, each timed replay by replay; returns the per-window median and p99
    and the drift of the median from the first window to the last."""
    t_end = time.time() + seconds
    windows = []
    n = max(1, int(1000.0 / max(replay_times(torch, g, 5)[-1], 1e-3)))
    while time.time() < t_end:
        ts = replay_times(torch, g, n)
        windows.append({"t_s": round(seconds - (t_end - time.time()), 1), **percentiles(ts, (50, 99))})
        if len(windows) % 10 == 0:
            log(f"soak {windows[-1]['t_s']:.0f} s: median {windows[-1]['p50']:.3f} ms, p99 {windows[-1]['p99']:.3f} ms")
    p50 = [w["p50"] for w in windows]
    return {"seconds": round(seconds, 1), "replays": n * len(windows), "windows": len(windows),
            "median_ms_first": p50[0], "median_ms_last": p50[-1], "median_ms_max": max(p50),
            "p99_ms_max": max(w["p99"] for w in windows),
            "drift_pct": round(100.0 * (p50[-1] - p50[0]) / p50[0], 2),
            "GBs_at_median_last": round(step_bytes / (p50[-1] * 1e-3) / 1e9, 1),
            "series": windows}


def qmm_roofline(torch, stack, reps: int = 5) -> dict:
    """Average duration of the skinny-QMM launches of the verify step.

    The QMM launches of each projection kind (the 64 qkv, o, gate_up and down
    launches of the step with their fused prologues and epilogues, and the
    lm_head launch repeated 16 times) are captured into a graph of their own,
    with the step's buffers and launch configuration; each graph is replayed
    `reps` times between two HIP events on the stream it runs on. The per-kind
    durations are weighted by the step's launch counts. Algorithmic bytes per
    launch: packed codes, scales, biases, activations in, outputs (and the
    residual read of the residual epilogue)."""
    from speculative_decoding_verify_vq_amd import vq
    from speculative_decoding_verify_vq_amd.stack import qmm_algorithmic_bytes
    cfg = stack.cfg
    L = stack.w.layers
    kinds = {
        "qkv": (lambda p: stack._qmm(stack.h, p, stack.qkv, norm=True), [l["qkv"] for l in L], 2),
        "o": (lambda p: stack._qmm(stack.qkv[:, : cfg.q_width], p, stack.h, epilogue=vq.VQ_EPI_RESIDUAL,
                                   y_sumsq=stack.ss), [l["o"] for l in L], 4),
        "gate_up": (lambda p: stack._qmm(stack.h, p, stack.act, norm=True, epilogue=vq.VQ_EPI_SWIGLU),
                    [l["gate_up"] for l in L], 1),
        "down": (lambda p: stack._qmm(stack.act, p, stack.h, epilogue=vq.VQ_EPI_RESIDUAL, y_sumsq=stack.ss),
                 [l["down"] for l in L], 4),
        "lm_head": (lambda p: stack._qmm(stack.h, p, stack.logits[0], norm=True), [stack.w.lm_head] * 16, 4),
    }
    counts = {name: len(L) for name in ("qkv", "o", "gate_up", "down")}
    counts["lm_head"] = 1
    per_kind = {}
    tot_ms = tot_bytes = 0.0
    for name, (fn, packs, out_bytes) in kinds.items():
        g = capture(torch, lambda: [fn(p) for p in packs])
        ms = time_graph(torch, g, reps, 1) / len(packs)
        del g
        nb = qmm_algorithmic_bytes(cfg.M, packs[0].N, packs[0].K, packs[0].bits, out_bytes=out_bytes)
        per_kind[name] = {"us": round(ms * 1e3, 2), "GBs": round(nb / (ms * 1e-3) / 1e9, 1)}
        tot_ms += counts[name] * ms
        tot_bytes += counts[name] * nb
    n = sum(counts.values())
    avg_ms, avg_bytes = tot_ms / n, tot_bytes / n
    return {"avg_ms": avg_ms, "avg_bytes": avg_bytes, "launches": n, "per_kind": per_kind,
            "achieved_GBs": avg_bytes / (avg_ms * 1e-3) / 1e9}


def qmm_cost_curve(torch, bits: int, N: int = 17408, K: int = 5120,
                   Ms=(1, 2, 3, 4, 6, 8, 12, 16)) -> dict:
    """µs per skinny-QMM launch at each verify width M for one dense projection
    of the shape the pages tabulate, (M, 5120) x (17408, 5120)^T (page
    "Speculative decoding and MTP on Apple silicon", Facts), on the tiled pack
    with the store epilogue (bf16 out): the launches of each M are captured into
    one graph that rotates over distinct weights totalling at least 2 GiB, so
    every weight byte comes from HBM. Returns µs, GB/s and cost(M)/cost(M=1)."""
    from speculative_decoding_verify_vq_amd import vq
    from speculative_decoding_verify_vq_amd.stack import QPack, qmm_algorithmic_bytes
    from synth import bf16_normal_torch, random_words_torch
    dev = torch.device("cuda")
    one = QPack(torch.empty(0), N, K, bits).nbytes()
    n = max(8, -(-(2 << 30) // one))
    packs = []
    for i in range(n):
        wq = random_words_torch(N * K * bits // 32, 700 + i, dev)
        sc = bf16_normal_torch((N, K // 64), 0.02, 0.005, 800 + i, dev)
        bi = bf16_normal_torch((N, K // 64), 0.0, 0.01, 900 + i, dev)
        packs.append(QPack.from_rows(wq, sc, bi, bits, N, K))
        del wq, sc, bi
    torch.cuda.synchronize()
    ws = torch.zeros(max(vq.qmm_packed_workspace_bytes(bits, m, N, K) for m in Ms) + 256, dtype=torch.uint8,
                     device=dev)
    wsv = ws[(-ws.data_ptr()) % 256:]
    res = {}
    for m in Ms:
        x = torch.randn((m, K), device=dev).to(torch.bfloat16)
        y = torch.empty((m, N), device=dev, dtype=torch.bfloat16)
        g = capture(torch, lambda: [vq.qmm_packed(x, p.packed, bits, N, K, out=y, workspace=wsv) for p in packs])
        us = 1e3 * time_graph(torch, g, 5, 1) / n
        del g
        res[str(m)] = {"us": round(us, 2),
                       "GBs": round(qmm_algorithmic_bytes(m, N, K, bits) / (us * 1e-6) / 1e9, 1)}
    base = res[str(Ms[0])]["us"]
    for v in res.values():
        v["cost_ratio"] = round(v["us"] / base, 4)
    del packs, ws
    torch.cuda.empty_cache()
    return {"shape": f"(M, {K}) x ({N}, {K})^T, {bits}-bit g64, tiled pack, bf16 out", "per_M": res}


CURVE_MS = (1, 2, 3, 4, 6, 8, 12, 16)
CURVE_PACKS = 8


def qmm_curve_counter_run(torch, bits: int, N: int = 17408, K: int = 5120) -> None:
    """For hardware counters: CURVE_PACKS distinct (N, K) weights, then for each
    verify width M in CURVE_MS one eager launch on each weight, in that order
    (the dispatch order is what the counter summary relies on)."""
    from speculative_decoding_verify_vq_amd import vq
    from speculative_decoding_verify_vq_amd.stack import QPack
    from synth import bf16_normal_torch, random_words_torch
    dev = torch.device("cuda")
    packs = []
    for i in range(CURVE_PACKS):
        wq = random_words_torch(N * K * bits // 32, 700 + i, dev)
        sc = bf16_normal_torch((N, K // 64), 0.02, 0.005, 800 + i, dev)
        bi = bf16_normal_torch((N, K // 64), 0.0, 0.01, 900 + i, dev)
        packs.append(QPack.from_rows(wq, sc, bi, bits, N, K))
        del wq, sc, bi
    ws = torch.zeros(max(vq.qmm_packed_workspace_bytes(bits, m, N, K) for m in CURVE_MS) + 256,
                     dtype=torch.uint8, device=dev)
    wsv = ws[(-ws.data_ptr()) % 256:]
    torch.cuda.synchronize()
    for m in CURVE_MS:
        x = torch.randn((m, K), device=dev).to(torch.bfloat16)
        y = torch.empty((m, N), device=dev, dtype=torch.bfloat16)
        torch.cuda.synchronize()
        for p in packs:
            vq.qmm_packed(x, p.packed, bits, N, K, out=y, workspace=wsv)
        torch.cuda.synchronize()
    log(f"counter run: {len(CURVE_MS)} widths x {CURVE_PACKS} launches of ({N}, {K}) {bits}-bit")


def summarize_curve_counters(prof_dir: str, out_dir: str, bits: int, cmd_fetch: str, cmd_write: str,
                             N: int = 17408, K: int = 5120) -> None:
    """HBM bytes per launch of one (M, K) x (N, K)^T projection at every verify
    width, from FETCH_SIZE / WRITE_SIZE passes of qmm_curve_counter_run (the
    QMM dispatches in order: CURVE_PACKS per width), scaled by the 1 GiB copy."""
    from speculative_decoding_verify_vq_amd.stack import qmm_algorithmic_bytes
    per = {}
    scale = {}
    for ctr, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        rows = [r for r in _read_csv(os.path.join(prof_dir, sub), "_counter_collection.csv")
                if r["Counter_Name"] == ctr]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        scale[ctr] = (1 << 20) / max(copies)
        q = [float(r["Counter_Value"]) for r in rows if "qmm_kernel<" in r["Kernel_Name"]]
        if len(q) != len(CURVE_MS) * CURVE_PACKS:
            raise RuntimeError(f"{ctr}: expected {len(CURVE_MS) * CURVE_PACKS} QMM dispatches, found {len(q)}")
        for i, m in enumerate(CURVE_MS):
            v = q[i * CURVE_PACKS:(i + 1) * CURVE_PACKS]
            per.setdefault(m, {})[ctr] = sum(v) / len(v)
    md = [f"# HBM traffic of one (M, {K}) x ({N}, {K})^T projection, {bits}-bit g64, at every verify width", "",
          "Two counter passes of the same command (8 distinct weights, one eager launch on each per width, plus a "
          "1 GiB device copy for scaling):", "", f"    {cmd_fetch}", f"    {cmd_write}", "",
          f"Scaling: fetch counts x {scale['FETCH_SIZE']:.5f}, write counts x {scale['WRITE_SIZE']:.5f} (the copy "
          "reads and writes 1048576 KiB).", "",
          "| M | FETCH_SIZE KiB (raw) | WRITE_SIZE KiB (raw) | HBM bytes (scaled) | algorithmic bytes | ratio | "
          "HBM bytes / HBM bytes at M=1 |", "|---|---|---|---|---|---|---|"]
    base = None
    for m in CURVE_MS:
        f, w = per[m]["FETCH_SIZE"], per[m]["WRITE_SIZE"]
        hbm = 1024 * (f * scale["FETCH_SIZE"] + w * scale["WRITE_SIZE"])
        alg = qmm_algorithmic_bytes(m, N, K, bits)
        base = base or hbm
        md.append(f"| {m} | {f:.1f} | {w:.1f} | {int(hbm)} | {alg} | {hbm / alg:.3f} | {hbm / base:.3f} |")
    md += ["", "The weight stream is read once per launch whatever M is: the bytes grow only by the activations, "
               "the outputs and the split-K partials of the extra rows."]
    with open(os.path.join(out_dir, f"qmm_traffic_by_M_{bits}bit.md"), "w") as f:
        f.write("\n".join(md) + "\n")


def _time_calls(torch, fns, reps: int = 5) -> float:
    """µs per call of the callables `fns` (one each), captured into one graph and
    replayed `reps` times after one warm-up replay."""
    g = capture(torch, lambda: [f() for f in fns])
    ms = time_graph(torch, g, reps, 1)
    del g
    return 1e3 * ms / len(fns)


def next_rows(torch, stack, w, single_ms: float) -> dict:
    """Measurements of the rows after the hot path, at 27B attention heads
    (Hq 24, Hkv 4, D 256): tree-mask against causal attention at 16k context and
    16 drafted rows; 8-bit against bf16 KV at 128k context and 8 rows; the verify
    step of 16 // M sequences of M rows (the step's context each) against one
    sequence. Every
    attention timing rotates over distinct caches of at least 2 GiB in total, so
    that the KV is read from HBM."""
    from speculative_decoding_verify_vq_amd import vq
    from speculative_decoding_verify_vq_amd.stack import DenseVerifyStack, StackConfig
    from synth import bf16_normal_torch, chain_masks, random_words_torch, tree_masks
    dev = torch.device("cuda")
    Hq, Hkv, D = 24, 4, 256
    res = {}

    def caches(n, T, seed):
        return [(bf16_normal_torch((Hkv, T, D), 0.0, 1.0, seed + 2 * i, dev),
                 bf16_normal_torch((Hkv, T, D), 0.0, 1.0, seed + 2 * i + 1, dev)) for i in range(n)]

    # tree verify: 16 nodes at 16k
    M, T = 16, 16384 + 16
    kv = caches(32, T, 900)
    q = bf16_normal_torch((M, Hq, D), 0.0, 1.0, 950, dev)
    tm = torch.from_numpy(tree_masks(3, M).view(np.int32)).to(dev)
    cm = torch.from_numpy(chain_masks(M).view(np.int32)).to(dev)
    out = torch.empty_like(q)
    nb = 4 * Hkv * T * D + 4 * M * Hq * D
    us_c = _time_calls(torch, [lambda k=k, v=v: vq.multirow_attn(q, k, v, T, 1 / 16, out=out) for k, v in kv])
    us_t = _time_calls(torch, [lambda k=k, v=v: vq.multirow_attn(q, k, v, T, 1 / 16, out=out, tree_mask=tm)
                               for k, v in kv])
    us_ch = _time_calls(torch, [lambda k=k, v=v: vq.multirow_attn(q, k, v, T, 1 / 16, out=out, tree_mask=cm)
                                for k, v in kv])
    res["tree_attention"] = {"shape": "Hq 24, Hkv 4, D 256, 16384 committed + 16 tree nodes (random tree)",
                             "causal_us": round(us_c, 2), "tree_us": round(us_t, 2), "chain_mask_us": round(us_ch, 2),
                             "tree_GBs": round(nb / us_t / 1e3, 1)}
    del kv
    torch.cuda.empty_cache()

    # 8-bit KV: 8 rows at 128k
    M, T = 8, 131072 + 8
    q = bf16_normal_torch((M, Hq, D), 0.0, 1.0, 960, dev)
    out = torch.empty_like(q)
    kv = caches(4, T, 1000)
    nb16 = 4 * Hkv * T * D + 4 * M * Hq * D
    us16 = _time_calls(torch, [lambda k=k, v=v: vq.multirow_attn(q, k, v, T, 1 / 16, out=out) for k, v in kv])
    del kv
    torch.cuda.empty_cache()

    def kv8(seed):
        codes = random_words_torch(Hkv * T * D // 4, seed, dev).view(torch.uint8).view(Hkv, T, D)
        s_ = bf16_normal_torch((Hkv, T, D // 64), 0.02, 0.005, seed + 1, dev).view(torch.int16).to(torch.int32)
        b_ = bf16_normal_torch((Hkv, T, D // 64), -2.5, 0.1, seed + 2, dev).view(torch.int16).to(torch.int32)
        return codes, (s_ & 0xFFFF) | (b_ << 16)

    kv = [(kv8(1100 + 10 * i), kv8(1105 + 10 * i)) for i in range(8)]
    nb8 = 2 * Hkv * T * (D + 4 * (D // 64)) + 4 * M * Hq * D
    us8 = _time_calls(torch, [lambda a=a, b=b: vq.multirow_attn_int8(q, a[0], a[1], b[0], b[1], T, 1 / 16, out=out)
                              for a, b in kv])
    res["int8_kv_attention"] = {"shape": "Hq 24, Hkv 4, D 256, 131072 committed + 8 rows",
                                "bf16_us": round(us16, 2), "bf16_GBs": round(nb16 / us16 / 1e3, 1),
                                "int8_us": round(us8, 2), "int8_GBs": round(nb8 / us8 / 1e3, 1),
                                "kv_bytes_ratio": round(nb8 / nb16, 4)}
    del kv
    torch.cuda.empty_cache()

    # 16 // M sequences of M rows in one step (own caches at the step's context
    # each; at most 16 rows share the weight pass) against one sequence
    B = max(1, 16 // stack.cfg.M)
    cfg = stack.cfg
    cb = StackConfig(**{**cfg.__dict__, "B": B})
    T_cap = cfg.ctx + 16
    wb = type(w)(layers=w.layers, lm_head=w.lm_head,
                 k_cache=[bf16_normal_torch((B, cfg.Hkv, T_cap, cfg.D), 0.0, 1.0, 1200 + a, dev)
                          for a in range(cfg.n_attn)],
                 v_cache=[bf16_normal_torch((B, cfg.Hkv, T_cap, cfg.D), 0.0, 1.0, 1300 + a, dev)
                          for a in range(cfg.n_attn)])
    st = DenseVerifyStack(cb, wb)
    K, V = cfg.M - 1, cfg.vocab
    h_in = torch.randn((B * cfg.M, cfg.hidden), device=dev).to(torch.bfloat16)
    dl = torch.randn((B, K, V), device=dev) * 2
    dr = torch.randint(0, V, (B, K), dtype=torch.int32, device=dev)
    un = torch.rand((B, K + 1), device=dev)
    g = capture(torch, lambda: st.step(h_in, dl, dr, un))
    ms_b = time_graph(torch, g, 5, 2)
    del g, st, wb
    torch.cuda.empty_cache()
    res["multi_sequence"] = {"sequences": B, "rows": B * cfg.M, "ms_per_step": round(ms_b, 4),
                             "single_sequence_ms": round(single_ms, 4),
                             "speedup_vs_sequential_steps": round(B * single_ms / ms_b, 3)}
    return res


ATTN_HEADS = (24, 4, 256)          # Hq, Hkv, D of the 27B-shaped attention layers
ATTN_CTXS = (8192, 32768)
ATTN_MS = (1, 2, 3, 4, 5, 6, 7, 8)


def attention_config2(torch) -> dict:
    """µs per multi-row attention call at the 27B heads (Hq 24, Hkv 4, D 256,
    scale 1/16) for 8k and 32k committed keys plus M = 1..8 drafted rows causal
    among themselves: GB/s over the call's algorithmic bytes (K and V once, q in,
    out) and cost(M)/cost(M=1). Every timing is a graph of calls rotating over
    distinct caches of at least 2 GiB in total, so the KV comes from HBM (page
    "Speculative decoding and MTP on Apple silicon", Facts: 8 query rows at 32k
    context, each KV tile read once rather than once per row)."""
    from speculative_decoding_verify_vq_amd import vq
    from synth import bf16_normal_torch
    dev = torch.device("cuda")
    Hq, Hkv, D = ATTN_HEADS
    out = {}
    for ctx in ATTN_CTXS:
        Tcap = ctx + max(ATTN_MS)
        per = 4 * Hkv * Tcap * D
        n = max(8, -(-(2 << 30) // per))
        kv = [(bf16_normal_torch((Hkv, Tcap, D), 0.0, 1.0, 5000 + 2 * i, dev),
               bf16_normal_torch((Hkv, Tcap, D), 0.0, 1.0, 5001 + 2 * i, dev)) for i in range(n)]
        rec = {}
        for M in ATTN_MS:
            T = ctx + M
            q = bf16_normal_torch((M, Hq, D), 0.0, 1.0, 5900 + M, dev)
            o = torch.empty_like(q)
            ws = torch.zeros(vq.attn_workspace_bytes(M, Hq, Hkv, D, T) + 256, dtype=torch.uint8, device=dev)
            wsv = ws[(-ws.data_ptr()) % 256:]
            us = _time_calls(torch, [lambda k=k, v=v: vq.multirow_attn(q, k, v, T, 1 / 16, out=o, workspace=wsv)
                                     for k, v in kv], reps=5)
            nb = 4 * Hkv * T * D + 4 * M * Hq * D
            rec[str(M)] = {"us": round(us, 2), "GBs": round(nb / us / 1e3, 1)}
        base = rec["1"]["us"]
        for v in rec.values():
            v["cost_ratio"] = round(v["us"] / base, 4)
        out[f"{ctx // 1024}k"] = rec
        del kv
        torch.cuda.empty_cache()
    return {"shape": "Hq 24, Hkv 4, D 256, bf16 KV, ctx committed keys + M causal drafted rows", "per_ctx": out}


ATTN_COUNTER_CACHES = 4


def attn_counter_run(torch) -> None:
    """For hardware counters: at 32k context, for M = 1..8 in order, one eager
    multi-row attention call on each of ATTN_COUNTER_CACHES distinct caches
    (the dispatch order is what the counter summary relies on)."""
    from speculative_decoding_verify_vq_amd import vq
    from synth import bf16_normal_torch
    dev = torch.device("cuda")
    Hq, Hkv, D = ATTN_HEADS
    ctx = 32768
    Tcap = ctx + max(ATTN_MS)
    kv = [(bf16_normal_torch((Hkv, Tcap, D), 0.0, 1.0, 6000 + 2 * i, dev),
           bf16_normal_torch((Hkv, Tcap, D), 0.0, 1.0, 6001 + 2 * i, dev)) for i in range(ATTN_COUNTER_CACHES)]
    ws = torch.zeros(vq.attn_workspace_bytes(max(ATTN_MS), Hq, Hkv, D, ctx + max(ATTN_MS)) + 256,
                     dtype=torch.uint8, device=dev)
    wsv = ws[(-ws.data_ptr()) % 256:]
    torch.cuda.synchronize()
    for M in ATTN_MS:
        q = bf16_normal_torch((M, Hq, D), 0.0, 1.0, 6900 + M, dev)
        o = torch.empty_like(q)
        torch.cuda.synchronize()
        for k, v in kv:
            vq.multirow_attn(q, k, v, ctx + M, 1 / 16, out=o, workspace=wsv)
        torch.cuda.synchronize()
    log(f"attention counter run: {len(ATTN_MS)} widths x {ATTN_COUNTER_CACHES} calls at 32k")


def summarize_attn_counters(prof_dir: str, out_dir: str, cmd_fetch: str, cmd_write: str) -> None:
    """HBM bytes per multi-row attention call at 32k context for M = 1..8 from
    the FETCH_SIZE / WRITE_SIZE passes of attn_counter_run (partial and combine
    kernels of each call summed), scaled by the 1 GiB copy."""
    Hq, Hkv, D = ATTN_HEADS
    ctx = 32768
    per, scale = {}, {}
    for ctr, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        rows = [r for r in _read_csv(os.path.join(prof_dir, sub), "_counter_collection.csv")
                if r["Counter_Name"] == ctr]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        scale[ctr] = (1 << 20) / max(copies)
        for kname in ("attn_partial_kernel", "attn_combine_kernel"):
            vals = [float(r["Counter_Value"]) for r in rows if kname in r["Kernel_Name"]]
            if len(vals) != len(ATTN_MS) * ATTN_COUNTER_CACHES:
                raise RuntimeError(f"{ctr}: expected {len(ATTN_MS) * ATTN_COUNTER_CACHES} {kname} dispatches, "
                                   f"found {len(vals)}")
            for i, M in enumerate(ATTN_MS):
                v = vals[i * ATTN_COUNTER_CACHES:(i + 1) * ATTN_COUNTER_CACHES]
                per.setdefault(M, {}).setdefault(ctr, 0.0)
                per[M][ctr] += sum(v) / len(v)
    md = ["# HBM traffic of one multi-row attention call at 32k context, M = 1..8", "",
          f"Hq {Hq}, Hkv {Hkv}, D {D}, bf16 KV, T = 32768 + M. Two counter passes of the same command "
          f"({ATTN_COUNTER_CACHES} distinct caches, one eager call on each per width, plus a 1 GiB device copy for "
          "scaling); the partial and combine kernels of a call are summed:", "",
          f"    {cmd_fetch}", f"    {cmd_write}", "",
          f"Scaling: fetch counts x {scale['FETCH_SIZE']:.5f}, write counts x {scale['WRITE_SIZE']:.5f} (the copy "
          "reads and writes 1048576 KiB).", "",
          "| M | FETCH_SIZE KiB (raw) | WRITE_SIZE KiB (raw) | HBM bytes (scaled) | algorithmic bytes | ratio | "
          "HBM bytes / HBM bytes at M=1 |", "|---|---|---|---|---|---|---|"]
    base = None
    for M in ATTN_MS:
        f, w = per[M]["FETCH_SIZE"], per[M]["WRITE_SIZE"]
        hbm = 1024 * (f * scale["FETCH_SIZE"] + w * scale["WRITE_SIZE"])
        alg = 4 * Hkv * (ctx + M) * D + 4 * M * Hq * D
        base = base or hbm
        md.append(f"| {M} | {f:.1f} | {w:.1f} | {int(hbm)} | {alg} | {hbm / alg:.3f} | {hbm / base:.3f} |")
    md += ["", "Each K/V byte is read once per call whatever M is: the bytes grow only by the queries, the outputs "
               "and the per-range partial results of the extra rows."]
    with open(os.path.join(out_dir, "attn_traffic_by_M_32k.md"), "w") as f:
        f.write("\n".join(md) + "\n")


def acceptance_us(torch, stack, draft_logits, drafts, uniforms, reps: int = 20) -> float:
    """µs per acceptance call of the step (logits mode over the step's own lm_head
    logits and the draft logits, the step's sampler settings), as a graph of one
    call replayed `reps` times."""
    from speculative_decoding_verify_vq_amd import vq
    cfg = stack.cfg

    def call():
        vq.spec_accept(stack.logits, draft_logits, drafts, uniforms, logits=True, temperature=cfg.temperature,
                       top_k=cfg.top_k, top_p=cfg.top_p, probs_out=stack.probs, out_tokens=stack.tokens,
                       out_n=stack.n_acc, workspace=stack._wsv("accept"))
    g = capture(torch, call)
    ms = time_graph(torch, g, reps, 2)
    del g
    return 1e3 * ms


def stream_ceiling(torch, nbytes: int = 1 << 30) -> dict:
    """The HBM streaming-read ceiling: vq_stream_read over a 1 GiB buffer (4x the
    256 MB Infinity Cache, so every byte comes from HBM), ordinary and
    non-temporal 16-byte loads, at several grid sizes; TB/s of the best grid."""
    from speculative_decoding_verify_vq_amd import vq
    dev = torch.device("cuda")
    src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).random_()
    grids = (1024, 2048, 4096, 8192, 16384, 32768)
    sink = torch.empty(4 * max(grids), dtype=torch.int32, device=dev)
    res = {}
    for nt in (False, True):
        best = None
        for wg in grids:
            ms = 1e-3 * _time_calls(torch, [lambda: vq.stream_read(src, sink, wg, nontemporal=nt)] * 4, reps=5)
            tbs = nbytes / (ms * 1e-3) / 1e12
            if best is None or tbs > best[0]:
                best = (tbs, wg)
        res["nontemporal" if nt else "ordinary"] = {"TBs": round(best[0], 3), "workgroups": best[1]}
    del src, sink
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "kernel": "vq_stream_read (include/vq_bench.h)", **res}


def qmm_traffic(avg_bytes: float, bits: int, M: int):
    """HBM bytes per QMM launch from the committed counter summary, if it was taken
    on the current kernel source and on this workload's weight width and verify
    rows (else None): FETCH_SIZE + WRITE_SIZE per dispatch, each scaled by what the
    counter reads for a copy of known size."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"qmm_traffic_{bits}bit_M{M}.json")
    src = os.path.join(ROOT, "speculative_decoding_verify_vq_amd", "csrc", "qmm.hip")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if rec.get("qmm_hip_sha256") != digest or rec.get("bits") != bits or rec.get("M") != M:
        return None
    return {"bytes_per_launch": rec["hbm_bytes_per_launch"],
            "ratio_to_algorithmic": round(rec["hbm_bytes_per_launch"] / avg_bytes, 3),
            "source": f"profiles/qmm_traffic_{bits}bit_M{M}.json"}


def copy_calibration(torch, nbytes: int = 1 << 30) -> None:
    """A plain device copy of known size (reads and writes nbytes), launched for
    hardware counters to be scaled against."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_baseline(cfg_id: int, cfg, step_bytes: float) -> dict:
    """The oracle timed on a bounded sample of the same workload on this host's cores:
    one layer's four projections (qkv, o, gate_up, down) at the step's M, one
    attention layer at the step's context (every row and query head; above 32k
    keys one KV head and its query heads), and one acceptance over the full
    vocabulary. Rate = algorithmic
    bytes of the sample / CPU seconds, in GB/s (the step time is extrapolated from
    the same bytes-per-second)."""
    import oracle.accept as oacc
    import oracle.attn as oattn
    import oracle.qmm as oqmm
    from synth import accept_logits, attn_inputs, qmm_activations, qmm_weights, uniforms24
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    M = cfg.M
    parts, secs, nbytes = [], 0.0, 0
    sh = cfg.shapes()
    for li, name in enumerate(("qkv", "o", "gate_up", "down")):
        N, K = sh[name]
        w = qmm_weights(1, N, K, cfg.bits, layer=li)
        x = qmm_activations(1, M, K, extra=li)
        t0 = time.perf_counter()
        oqmm.skinny_qmm(x, w["wq"], w["scales"], w["biases"], cfg.bits, 64, M, N, K)
        dt = time.perf_counter() - t0
        b = oqmm.algorithmic_bytes(M, N, K, cfg.bits)
        del w
        parts.append(f"{name} {N}x{K} ({dt:.2f} s)")
        secs += dt
        nbytes += b
    T = cfg.ctx + M
    # Long contexts: one KV head and its query heads, so the sample stays bounded.
    hkv = cfg.Hkv if T <= 32768 else 1
    hq = cfg.Hq // cfg.Hkv * hkv
    q, k, v = attn_inputs(2, M, hq, hkv, cfg.D, T)
    t0 = time.perf_counter()
    oattn.multirow_attention(q, k, v, M, hq, hkv, cfg.D, T, T, cfg.D ** -0.5)
    dt = time.perf_counter() - t0
    parts.append(f"attention {M} rows x {hq} heads ({hkv} KV) at T={T} ({dt:.2f} s)")
    secs += dt
    nbytes += 2 * hkv * T * cfg.D * 2  # K and V of the sampled KV heads, once
    K = M - 1
    pl, ql = accept_logits(cfg_id, K, cfg.vocab)
    P, Q = oacc.probs_f32(pl, cfg.temperature), oacc.probs_f32(ql, cfg.temperature)
    us = uniforms24(cfg_id, (K + 1,))
    t0 = time.perf_counter()
    oacc.spec_accept(P, Q, [1, 2, 3, 4, 5, 6, 7][:K], us, cfg.top_k, cfg.top_p)
    dt = time.perf_counter() - t0
    parts.append(f"one acceptance over V={cfg.vocab} ({dt:.2f} s)")
    secs += dt
    nbytes += (2 * K + 1) * cfg.vocab * 4
    rate = nbytes / secs / 1e9
    return {"value": round(rate, 4), "unit": "GB/s", "cores": cores, "blas_threads": blas_threads,
            "kind": "oracle",
            "sample": "; ".join(parts) + f"; {nbytes / 1e6:.1f} MB in {secs:.2f} s",
            "ms_per_step_extrapolated": round(step_bytes / (rate * 1e9) * 1e3, 1)}


# Projection kinds of the 4-bit M=4 step in the order their QMM launches first
# appear in a profiled bench run, with their bf16/float32 output bytes per
# element (as in qmm_roofline) and their launch counts in one step.
_PROFILE_KINDS = [("qkv", 2, 64), ("o", 4, 64), ("gate_up", 1, 64), ("down", 4, 64), ("lm_head", 4, 1)]


def _read_csv(directory: str, suffix: str) -> list:
    import csv
    import glob
    paths = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not paths:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    with open(paths[0], newline="") as f:
        return list(csv.DictReader(f))


def _qmm_launch_groups(rows: list, grid_key) -> list:
    """QMM dispatches grouped by (kernel, grid) in order of first appearance."""
    groups = {}
    for r in rows:
        if "qmm_kernel<" in r["Kernel_Name"]:
            key = (r["Kernel_Name"], grid_key(r))
            groups.setdefault(key, []).append(r)
    return list(groups.items())


def summarize_profiles(prof_dir: str, out_dir: str, cmd_kt: str, cmd_fetch: str, cmd_write: str,
                       config: int = 3) -> None:
    """Writes the committed profile summaries from a profiled run's CSV output:
    <prof_dir>/kt (rocprofv3 --kernel-trace --stats -f csv), <prof_dir>/fetch and
    <prof_dir>/write (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE -f csv, runs with
    --copy-calibration). Produces the kernel-trace table, the HBM traffic table
    and qmm_traffic.json (read by qmm_traffic above). A part whose CSV
    directories are missing is left as it is."""
    if os.path.isdir(os.path.join(prof_dir, "kt")):
        _summarize_trace(prof_dir, out_dir, cmd_kt, config)
    if os.path.isdir(os.path.join(prof_dir, "fetch")) and os.path.isdir(os.path.join(prof_dir, "write")):
        _summarize_traffic(prof_dir, out_dir, cmd_fetch, cmd_write, config)


def _summarize_trace(prof_dir: str, out_dir: str, cmd_kt: str, config: int = 3) -> None:
    c = CONFIGS[config]
    tag = f"{c['bits']}bit_M{c['M']}"
    ctx_k = c["ctx"] // 1024
    stats = _read_csv(os.path.join(prof_dir, "kt"), "_kernel_stats.csv")
    trace = _read_csv(os.path.join(prof_dir, "kt"), "_kernel_trace.csv")
    tot = sum(float(r["TotalDurationNs"]) for r in stats)
    lines = [f"{'kernel':64s} {'calls':>6s} {'total_us':>10s} {'avg_us':>8s} {'min_us':>8s} {'max_us':>8s} {'pct':>6s}"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:25]:
        name = r["Name"].replace("void ", "").replace("(anonymous namespace)::", "")
        lines.append(f"{name[:64]:64s} {int(r['Calls']):6d} {float(r['TotalDurationNs']) / 1e3:10.1f} "
                     f"{float(r['AverageNs']) / 1e3:8.2f} {float(r['MinNs']) / 1e3:8.2f} "
                     f"{float(r['MaxNs']) / 1e3:8.2f} {100 * float(r['TotalDurationNs']) / tot:6.2f}")
    groups = _qmm_launch_groups(trace, lambda r: (int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]),
                                                  int(r["Grid_Size_Y"])))
    if len(groups) != len(_PROFILE_KINDS):
        raise RuntimeError(f"expected {len(_PROFILE_KINDS)} QMM launch shapes, found {len(groups)}")
    shape_lines, trace_avg = [], {}
    for (kind, _, _), ((name, grid), rs) in zip(_PROFILE_KINDS, groups):
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]
        trace_avg[kind] = sum(d) / len(d)
        short = name.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0]
        shape_lines.append(f"  {kind:8s} {short:42s} wg={grid} calls={len(d):5d} avg_us={trace_avg[kind]:8.2f} "
                           f"min_us={min(d):8.2f}")
    n_step = sum(c for _, _, c in _PROFILE_KINDS)
    trace_weighted = sum(trace_avg[k] * c for k, _, c in _PROFILE_KINDS) / n_step
    bench_line = None
    for fn in ("kt.out",):
        path = os.path.join(prof_dir, fn)
        if os.path.exists(path):
            with open(path) as f:
                txt = [ln for ln in f.read().splitlines() if ln.startswith("{")]
            bench_line = json.loads(txt[-1]) if txt else None
    md = [f"# Kernel trace: verify step, {c['bits']}-bit g64, M={c['M']}, {ctx_k}k context", "",
          "Command (from the repository root, on one MI355X):", "", f"    {cmd_kt}", "",
          "Durations summed over every dispatch of the command (rocprofv3 kernel stats): weight packing, the eager",
          "warm-up pass, the graph capture, the step replays and the per-projection QMM graphs the bench times for",
          "its roofline record. `qmm_kernel<bits, MT, layout, epilogue, norm, chunked>`: layout 2 = tiled pack;",
          "epilogue 0 store, 1 residual, 2 SwiGLU; chunked = the workgroup walks the whole of K (no split).", "",
          "```", *lines, "", "qmm_kernel by projection (workgroups x, y; from the kernel trace):", *shape_lines, "```", "",
          f"Trace average per QMM launch, weighted by the step's launch counts (64 each, lm_head once): "
          f"{trace_weighted:.2f} us."]
    if bench_line:
        rf = bench_line["roofline"]
        pk = ", ".join(f"{k} {v['us']} us" for k, v in rf["per_kind"].items())
        md.append(f"The bench's own HIP-event timing in the same command (graph replays, per launch): {pk}; "
                  f"weighted the same way {rf['avg_launch_us']} us per launch.")
        md.append(f"Step: {bench_line['ms_per_step']} ms ({bench_line['value']} GB/s) under the profiler.")
    with open(os.path.join(out_dir, f"qmm_kernel_verify_step_{tag}.md"), "w") as f:
        f.write("\n".join(md) + "\n")



def _summarize_traffic(prof_dir: str, out_dir: str, cmd_fetch: str, cmd_write: str, config: int = 3) -> None:
    import hashlib
    from speculative_decoding_verify_vq_amd.stack import StackConfig, qmm_algorithmic_bytes
    c = CONFIGS[config]
    cfg = StackConfig(bits=c["bits"], lm_bits=c["lm_bits"], M=c["M"])
    tag = f"{cfg.bits}bit_M{cfg.M}"
    sh = cfg.shapes()
    n_step = sum(c for _, _, c in _PROFILE_KINDS)
    per = {}
    scale = {}
    for ctr, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        rows = _read_csv(os.path.join(prof_dir, sub), "_counter_collection.csv")
        rows = [r for r in rows if r["Counter_Name"] == ctr]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        scale[ctr] = (1 << 20) / max(copies)  # the 1 GiB copy reads and writes 1048576 KiB
        groups = _qmm_launch_groups(rows, lambda r: int(r["Grid_Size"]))
        if len(groups) != len(_PROFILE_KINDS):
            raise RuntimeError(f"{ctr}: expected {len(_PROFILE_KINDS)} QMM launch shapes, found {len(groups)}")
        for (kind, _, _), (_, rs) in zip(_PROFILE_KINDS, groups):
            v = [float(r["Counter_Value"]) for r in rs]
            per.setdefault(kind, {})[ctr] = (sum(v) / len(v), len(v))
    kinds = {}
    tot_hbm = tot_alg = 0.0
    for kind, out_b, cnt in _PROFILE_KINDS:
        N, K = sh[kind]
        alg = qmm_algorithmic_bytes(cfg.M, N, K, cfg.bits, out_bytes=out_b)
        fk, nd = per[kind]["FETCH_SIZE"]
        wk, _ = per[kind]["WRITE_SIZE"]
        hbm = 1024 * (fk * scale["FETCH_SIZE"] + wk * scale["WRITE_SIZE"])
        kinds[kind] = {"fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1), "dispatches": nd,
                       "hbm_bytes": int(hbm), "algorithmic_bytes": alg, "ratio": round(hbm / alg, 3)}
        tot_hbm += cnt * hbm
        tot_alg += cnt * alg
    src = os.path.join(ROOT, "speculative_decoding_verify_vq_amd", "csrc", "qmm.hip")
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    rec = {"kernel": "qmm_kernel (tiled pack; q|k|v with RMSNorm, o and down with the residual epilogue, gate|up "
                     "with RMSNorm and SwiGLU, lm_head with RMSNorm)",
           "workload": f"{cfg.bits}-bit g64 verify step, M={cfg.M} (hidden 5120, MLP 17408, lm_head 248320)",
           "bits": cfg.bits, "M": cfg.M,
           "qmm_hip_sha256": digest, "fetch_scale": round(scale["FETCH_SIZE"], 5),
           "write_scale": round(scale["WRITE_SIZE"], 5),
           "calibration": "__amd_rocclr_copyBuffer of a 1 GiB bf16 tensor (torch copy_): reads and writes 1048576 KiB",
           "per_kind": kinds, "step_launch_counts": {k: c for k, _, c in _PROFILE_KINDS},
           "hbm_bytes_per_launch": int(tot_hbm / n_step), "algorithmic_bytes_per_launch": int(tot_alg / n_step),
           "commands": [cmd_fetch, cmd_write]}
    with open(os.path.join(out_dir, f"qmm_traffic_{tag}.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    md = [f"# HBM traffic of the skinny QMM: verify step, {cfg.bits}-bit g64, M={cfg.M}", "",
          "Two counter passes of the same short command (8 layers, one step, plus a 1 GiB device copy for scaling):",
          "", f"    {cmd_fetch}", f"    {cmd_write}", "",
          f"Scaling: the 1 GiB copy (1048576 KiB read and written) reads FETCH_SIZE = "
          f"{(1 << 20) / scale['FETCH_SIZE']:.1f} KiB and WRITE_SIZE = {(1 << 20) / scale['WRITE_SIZE']:.1f} KiB, "
          f"so fetch counts are scaled by {scale['FETCH_SIZE']:.5f} and write counts by {scale['WRITE_SIZE']:.5f}.", "",
          "| projection | launches in step | FETCH_SIZE KiB (raw) | WRITE_SIZE KiB (raw) | HBM bytes (scaled) | "
          "algorithmic bytes | ratio |", "|---|---|---|---|---|---|---|"]
    for kind, _, cnt in _PROFILE_KINDS:
        r = kinds[kind]
        md.append(f"| {kind} | {cnt} | {r['fetch_kib_raw']} | {r['write_kib_raw']} | {r['hbm_bytes']} | "
                  f"{r['algorithmic_bytes']} | {r['ratio']} |")
    md += ["", f"Weighted by the step's launch counts: {rec['hbm_bytes_per_launch']} HBM bytes per launch against "
               f"{rec['algorithmic_bytes_per_launch']} algorithmic bytes "
               f"({rec['hbm_bytes_per_launch'] / rec['algorithmic_bytes_per_launch']:.3f}x).",
           "Algorithmic bytes include the residual read of the residual epilogue (o, down) and count SwiGLU's N/2 "
           "outputs (gate|up).",
           "The excess of the split projections is their float32 partials (written once, read once by the last "
           "workgroup of each column block) and the x slices re-read by every workgroup; the lm_head is not split.",
           "", f"qmm.hip sha256 at the time of the runs: {digest} (bench.py reports the traffic only while the source "
               "matches)."]
    with open(os.path.join(out_dir, f"qmm_traffic_{tag}.md"), "w") as f:
        f.write("\n".join(md) + "\n")


def run_config(torch, cfg_id: int, args, headline: bool) -> dict:
    """Builds the stack of one step configuration on the device, times the step
    and the measurements that go with it; returns the JSON record (the headline
    adds the next rows, the CPU baseline and the soak)."""
    from speculative_decoding_verify_vq_amd.stack import DenseVerifyStack, StackConfig
    from synth import accept_logits, uniforms24
    c = CONFIGS[cfg_id]
    cfg = StackConfig(layers=args.layers, bits=c["bits"], lm_bits=c["lm_bits"], M=c["M"], ctx=c["ctx"],
                      temperature=c["temperature"], top_k=c["top_k"], top_p=c["top_p"])
    T_cap = cfg.ctx + 16
    log(f"config {cfg_id}: generating weights and KV caches on the device")
    w = make_weights(cfg, torch, 1000 * cfg_id, T_cap)
    stack = DenseVerifyStack(cfg, w)
    dev = torch.device("cuda")
    M, K, V = cfg.M, cfg.M - 1, cfg.vocab
    h_in = (torch.randn((M, cfg.hidden), generator=torch.Generator(device=dev).manual_seed(5), device=dev)
            .to(torch.bfloat16))
    pl, ql = accept_logits(cfg_id, K, V)
    draft_logits = torch.from_numpy(ql[None]).to(dev)
    drafts = torch.tensor([[int(np.argmax(ql[i])) for i in range(K)]], dtype=torch.int32, device=dev)
    uniforms = torch.from_numpy(uniforms24(cfg_id, (1, K + 1))).to(dev)

    log("capturing the verify step")
    g = capture(torch, lambda: stack.step(h_in, draft_logits, drafts, uniforms))
    log(f"timing {args.steps} steps after {args.warmup} warmup")
    ms = time_graph(torch, g, args.steps, args.warmup)
    nbytes = stack.bytes_per_step()
    gbs = nbytes["total"] / (ms * 1e-3) / 1e9
    tok, n = stack.tokens.cpu().tolist(), int(stack.n_acc.item())
    log(f"step {ms:.3f} ms, {gbs:.1f} GB/s; tokens {tok} n_accepted {n}")
    dist = percentiles(replay_times(torch, g, args.steps))
    log(f"per-replay ms: {dist}")

    ratio = curve = None
    if not args.no_ratio:
        # cost(M) / cost(M=1) of the layer stack (weights once + attention of M
        # rows on the KV caches) over the verify widths of the dense-projection
        # workload, M = 1, 2, 3, 4, 6, 8, 12, 16.
        res = {}
        for m in (1, 2, 3, 4, 6, 8, 12, 16):
            cm = StackConfig(**{**cfg.__dict__, "M": m})
            st = DenseVerifyStack(cm, w)
            hm = torch.randn((m, cfg.hidden), device=dev).to(torch.bfloat16)
            gm = capture(torch, lambda: st.forward_hidden(hm))
            res[m] = time_graph(torch, gm, max(5, args.steps // 2), 2)
            del gm, st
        ratio = res[8] / res[1]
        curve = {str(m): {"ms": round(v, 4), "cost_ratio": round(v / res[1], 4)} for m, v in res.items()}
        log(f"{cfg.layers}-layer stack: M=1 {res[1]:.3f} ms, M=8 {res[8]:.3f} ms, ratio {ratio:.3f}; "
            f"{ {m: round(v / res[1], 3) for m, v in res.items()} }")

    roof = qmm_roofline(torch, stack)
    log(f"QMM per launch: {roof['avg_ms'] * 1e3:.1f} us, {roof['achieved_GBs']:.0f} GB/s; {roof['per_kind']}")
    traffic = qmm_traffic(roof["avg_bytes"], cfg.bits, cfg.M)
    acc_us = acceptance_us(torch, stack, draft_logits, drafts, uniforms)
    log(f"acceptance: {acc_us:.1f} us per call")

    nxt = cpu = soak_rec = None
    if headline and not args.no_next:
        log("measuring tree-mask attention, 8-bit KV attention and a multi-sequence step")
        nxt = next_rows(torch, stack, w, ms)
        log(f"next rows: {nxt}")
    if headline and not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(cfg_id, cfg, nbytes["total"])
    if headline and args.soak > 0:
        log(f"soak: replaying the step for {args.soak:.0f} s")
        soak_rec = soak(torch, g, args.soak, nbytes["total"])
        log(f"soak: median {soak_rec['median_ms_first']} -> {soak_rec['median_ms_last']} ms, "
            f"drift {soak_rec['drift_pct']}%, p99 max {soak_rec['p99_ms_max']} ms")
    rec = {
        "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": round(ms, 4), "step_ms_percentiles": dist,
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "config": {"workload": c["workload"], "layers": cfg.layers, "M": M, "ctx": cfg.ctx, "bits": cfg.bits,
                   "vocab": V, "bytes_per_step": nbytes},
        "cost_ratio_m8_m1": None if ratio is None else round(ratio, 4),
        "cost_curve": curve,
        "acceptance_us": round(acc_us, 2),
        "roofline": {"bound": "hbm", "achieved": round(roof["achieved_GBs"], 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(roof["achieved_GBs"] / PEAK_HBM_GBS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_launch"],
                     "traffic_detail": traffic,
                     "kernel": "qmm_kernel", "avg_launch_us": round(roof["avg_ms"] * 1e3, 2),
                     "avg_algorithmic_bytes": int(roof["avg_bytes"]), "launches_timed": roof["launches"],
                     "per_kind": roof["per_kind"],
                     "timing": "HIP events around replays of graphs holding the step's QMM launches, "
                               "per projection kind, weighted by the step's launch counts"},
    }
    if headline:
        rec.update({"cpu_baseline": cpu, "next_rows": nxt, "soak": soak_rec})
    del g, stack, w
    torch.cuda.empty_cache()
    return rec


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, choices=[3, 4],
                    help="the headline step configuration (default 4: 8-bit, M=8, KV at 128k)")
    ap.add_argument("--single", action="store_true", help="measure the headline configuration only")
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ratio", action="store_true", help="skip the cost(M)/cost(1) curves")
    ap.add_argument("--no-next", action="store_true", help="skip the tree / 8-bit KV / multi-sequence measurements")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-call attention records and the streaming-read ceiling")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="write the profiles/ summaries of the --config step from a profiled run's CSV output (kt/, "
                         "fetch/, write/ under DIR) and exit; needs no GPU")
    ap.add_argument("--qmm-curve-counters", type=int, default=0, metavar="BITS",
                    help="only the launches that the per-width counter summary reads (with --copy-calibration), "
                         "then exit")
    ap.add_argument("--summarize-curve-profiles", metavar="DIR", default=None,
                    help="write profiles/qmm_traffic_by_M_<bits>bit.md from fetch/ and write/ under DIR (no GPU)")
    ap.add_argument("--attn-counters", action="store_true",
                    help="only the attention calls that the 32k counter summary reads (with --copy-calibration)")
    ap.add_argument("--summarize-attn-profiles", metavar="DIR", default=None,
                    help="write profiles/attn_traffic_by_M_32k.md from fetch/ and write/ under DIR (no GPU)")
    ap.add_argument("--soak", type=float, default=0.0, metavar="SECONDS",
                    help="after the measurements, replay the step back to back for this long and report the "
                         "per-second median / p99 series (sustained-run check)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy first (for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.summarize_profiles:
        fmt = {"config": args.config}
        summarize_profiles(args.summarize_profiles, os.path.join(ROOT, "profiles"), PROFILE_CMDS["kt"].format(**fmt),
                           PROFILE_CMDS["fetch"].format(**fmt), PROFILE_CMDS["write"].format(**fmt), args.config)
        return 0
    if args.summarize_curve_profiles:
        b = args.qmm_curve_counters or 4
        summarize_curve_counters(args.summarize_curve_profiles, os.path.join(ROOT, "profiles"), b,
                                 PROFILE_CMDS["curve_fetch"].format(bits=b), PROFILE_CMDS["curve_write"].format(bits=b))
        return 0
    if args.summarize_attn_profiles:
        summarize_attn_counters(args.summarize_attn_profiles, os.path.join(ROOT, "profiles"),
                                PROFILE_CMDS["attn_fetch"], PROFILE_CMDS["attn_write"])
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the verify step; runs on more than one GPU are not "
              "supported by this library.", file=sys.stderr)
        return 2

    import torch
    from speculative_decoding_verify_vq_amd import vq  # noqa: F401  (fails loudly without the HIP library)

    if args.copy_calibration:
        copy_calibration(torch)
    if args.qmm_curve_counters:
        qmm_curve_counter_run(torch, args.qmm_curve_counters)
        return 0
    if args.attn_counters:
        attn_counter_run(torch)
        return 0

    head = run_config(torch, args.config, args, headline=True)
    others = {}
    if not args.single:
        other = 3 if args.config == 4 else 4
        others[str(other)] = run_config(torch, other, args, headline=False)

    curves = attn = ceiling = None
    if not args.no_ratio:
        curves = {f"{b}bit": qmm_cost_curve(torch, b) for b in (4, 8)}
        log("QMM cost(M)/cost(1) at (M,5120)x(17408,5120)^T: " + "; ".join(
            f"{k}: " + " ".join(f"{m}:{v['cost_ratio']}" for m, v in c["per_M"].items()) for k, c in curves.items()))
    if not args.no_extras:
        attn = attention_config2(torch)
        log(f"attention per call: {attn}")
        ceiling = stream_ceiling(torch)
        log(f"streaming-read ceiling: {ceiling}")

    out = {
        "metric": METRIC, "value": head["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "step_ms_percentiles": head["step_ms_percentiles"],
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": head["config"],
        "pct_of_peak": head["pct_of_peak"],
        "cost_ratio_m8_m1": head["cost_ratio_m8_m1"],
        "cost_curve": head["cost_curve"],
        "acceptance_us": head["acceptance_us"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "other_configs": others,
        "qmm_cost_curve": curves,
        "attention_per_call": attn,
        "stream_ceiling": ceiling,
        "next_rows": head["next_rows"],
        "soak": head["soak"],
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
