#!/usr/bin/env python3
"""Benchmark: Q4_0 x Q8_0 weight-streaming GEMV sweep on one MI355X.

A step is one pass of the whole hot path over one decode token's projections:
every matrix's fresh fp32 activation quantized to Q8_0 and every Q4_0 matrix
streamed once with its output written -- one launch at N=1 (the GEMV waves
quantize what they stream), a quantize launch and a GEMV launch at N >= 2.
Weights are synthetic, seeded, Qwen2.5-shaped; consecutive steps alternate
between seeded copies of the weight set so no step finds the previous step's
bytes in the 256 MB Infinity Cache.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload qwen2.5-1.5b|qwen2.5-7b|lm_head|gemv1536] [--n N]
  python bench.py --workload lm_head_q8|attn [...]
  python bench.py --workload chain [--chain-model 1.5b|7b] [--sync all|tagged|tree|counter]

gemv1536 is the single 1536x1536 GEMV: 405 seeded copies (537 MB, past the
Infinity Cache) as one sweep launch, plus each GEMV as its own launch
bracketed by events (latency-bound: ~1.3 MB per launch).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "Q4_0 GEMV weight-stream GB/s (% of 8 TB/s HBM peak) and implied tok/s at N=1"
# the sources the sweep kernel is compiled from (a PMC summary applies only to these)
KERNEL_SRCS = [os.path.join(ROOT, "q4_weight_streaming_amd", "csrc", f)
               for f in ("q4s_kernels.hip", "q4s_lane.h", "q4s_device.h", "q4s_internal.h")]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def workload_shapes(name: str):
    from q4_weight_streaming_amd import synth
    if name == "qwen2.5-1.5b":
        return synth.qwen25_1p5b(), 1, 2
    if name == "qwen2.5-7b":
        return synth.qwen25_7b(), 4, 1
    if name == "lm_head":
        return [synth.MatShape("lm_head", 151936, 1536)], 2, 4
    if name == "gemv1536":
        return [synth.MatShape(f"w{i}", 1536, 1536) for i in range(405)], 0, 1
    raise SystemExit(f"unknown workload {name}")


def make_copy(shapes, cfg: int, copy: int, n: int, dev, keep_host: bool, act_cfg: int | None = None):
    """One seeded copy of the weight set with its activations and outputs."""
    import numpy as np  # noqa: F401
    import torch

    from q4_weight_streaming_amd import _lib as q
    from q4_weight_streaming_amd import synth
    mats, host = [], []
    for m, s in enumerate(shapes):
        w = synth.q4_0_weights(s.rows, s.cols, synth.generator(cfg, m, copy, 0))
        x = synth.activation(n, s.cols, synth.generator(cfg if act_cfg is None else act_cfg, m, copy, 1),
                             outliers=0 if s.name == "lm_head" and len(shapes) == 1 else 8)
        wc = torch.from_numpy(w.reshape(-1)).to(dev)
        wp = q.repack_q4_0(wc, s.rows, s.cols)
        del wc
        mats.append({"w_packed": wp, "x": torch.from_numpy(x).to(dev),
                     "x_q8": torch.empty(q.q8_bytes(n, s.cols), dtype=torch.uint8, device=dev),
                     "y": torch.empty((n, s.rows), dtype=torch.float32, device=dev),
                     "rows": s.rows, "cols": s.cols})
        if keep_host:
            host.append((w, x))
    torch.cuda.synchronize()
    return mats, host


def time_steps(run_fns, steps: int, warmup: int, stream):
    """Average ms per step of run_fns[i % len] over `steps` steps, after `warmup`."""
    import torch
    for i in range(warmup):
        run_fns[i % len(run_fns)]()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        run_fns[i % len(run_fns)]()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_kernel(run_fns, steps: int, stream):
    """Average duration of each launch of run_fns, bracketed by events on its stream."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        run_fns[i % len(run_fns)]()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    d = sorted(a.elapsed_time(b) for a, b in ev)
    return sum(d) / len(d), d[len(d) // 2], d[0]


def traffic_from_profile(workload: str, n: int, launch_bytes: int):
    """HBM bytes per GEMV launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"sweep_{workload}_n{n}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash():
        return None
    return float(m_bytes.group(1))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_sweep_rate(host, shapes, budget_s: float):
    """Whole passes (quantize + GEMV of every matrix of copy 0) until `budget_s` seconds have
    been spent, or matrices of one pass if a pass alone exceeds it -> (GB/s, sample text)."""
    from oracle import oracle
    t0 = time.perf_counter()
    done_bytes, done, passes = 0, 0, 0
    n = host[0][1].shape[0]
    while True:
        for (w, x), s in zip(host, shapes):
            xq = oracle.quantize_q8_0(x)
            oracle.gemv(w, xq, s.rows, s.cols, n)
            done_bytes += s.q4_bytes
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        else:
            passes += 1
            if time.perf_counter() - t0 < budget_s:
                continue
        break
    dt = time.perf_counter() - t0
    return done_bytes / dt / 1e9, (f"{done} matrix products ({passes} whole passes over the {len(shapes)} "
                                   f"matrices of copy 0, {done_bytes} Q4_0 bytes), quantize + GEMV, {dt:.1f} s")


def cpu_baseline(host, shapes, n: int, budget_s: float):
    """The CPU oracle, as it stands, on a bounded sample of the same workload: on every host
    thread (OpenMP over output rows), then on one thread, each for about `budget_s` / 2 s."""
    from oracle import oracle
    oracle.build(force=False)
    threads = oracle.max_threads()
    rate, sample = _oracle_sweep_rate(host, shapes, budget_s / 2)
    oracle.set_threads(1)
    try:
        rate1, sample1 = _oracle_sweep_rate(host, shapes, budget_s / 2)
    finally:
        oracle.set_threads(threads)
    return {"value": round(rate, 3), "unit": "GB/s", "cores": threads, "kind": "oracle", "sample": sample,
            "cpu_model": cpu_model(), "visible_cpus": len(os.sched_getaffinity(0)),
            "single_thread": {"value": round(rate1, 3), "unit": "GB/s", "cores": 1, "sample": sample1}}


Q8_SRCS = [os.path.join(ROOT, "q4_weight_streaming_amd", "csrc", f)
            for f in ("q4s_q8w.hip", "q4s_lane.h", "q4s_device.h", "q4s_internal.h")]


def q8_kernel_hash() -> str:
    h = hashlib.sha256()
    for f in Q8_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_q8_profile(n: int):
    path = os.path.join(ROOT, "profiles", f"gemv_q8_0_lm_head_n{n}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != q8_kernel_hash():
        return None
    return float(m_bytes.group(1))


def run_q8_head(args, dev, stream) -> int:
    """The 8-bit output head: Q8_0 weights 151936 x 1536, quantize + Q8_0-weight GEMV per step,
    over 4 rotated seeded copies (992 MB, beyond every cache level)."""
    import torch

    from q4_weight_streaming_amd import _lib as q
    from q4_weight_streaming_amd import synth
    rows, cols, n, ncopies = 151936, 1536, args.n, 4
    log(f"generating {ncopies} copies of the Q8_0 lm_head {rows}x{cols}, n={n}")
    copies, host0 = [], None
    for c in range(ncopies):
        w = synth.q8_0_weights(rows, cols, synth.generator(5, 0, c, 0))
        x = synth.activation(n, cols, synth.generator(5, 0, c, 1), outliers=0)
        wc = torch.from_numpy(w.reshape(-1)).to(dev)
        copies.append({"wp": q.repack_q8_0(wc, rows, cols), "x": torch.from_numpy(x).to(dev),
                       "xq": torch.empty(q.q8_bytes(n, cols), dtype=torch.uint8, device=dev),
                       "y": torch.empty((n, rows), dtype=torch.float32, device=dev)})
        del wc
        if c == 0 and not args.no_cpu_baseline:
            host0 = (w, x)
    torch.cuda.synchronize()
    weight_bytes = q.q8_0_bytes(rows, cols)
    launch_bytes = weight_bytes + n * cols // 32 * 34 + 4 * n * rows

    def step(c):
        def f():
            if n == 1:  # one launch: the waves quantize the activation of the chunks they stream
                q.gemv_q8_0_f32(c["wp"], c["x"], rows, cols, out=c["y"], x_q8=c["xq"])
            else:
                q.quantize_q8_0(c["x"], out=c["xq"])
                q.gemv_q8_0(c["wp"], c["xq"], rows, cols, n, out=c["y"])
        return f

    def gemv_only(c):
        return lambda: q.gemv_q8_0(c["wp"], c["xq"], rows, cols, n, out=c["y"])

    if args.profile_only:
        for i in range(10):
            step(copies[i % ncopies])()
        for i in range(10):
            gemv_only(copies[i % ncopies])()
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        q.bench_copy(src, dst)
        torch.cuda.synchronize()
        log(f"profile run done: 10 Q8_0 steps and 10 GEMVs of {launch_bytes} algorithmic bytes, one 1 GiB copy")
        return 0

    ms = time_steps([step(c) for c in copies], args.steps, args.warmup, stream)
    log(f"step {ms * 1e3:.1f} us")
    k_b2b = time_steps([gemv_only(c) for c in copies], args.steps, args.warmup, stream)
    k_avg, k_med, k_min = time_kernel([gemv_only(c) for c in copies], args.steps, stream)
    log(f"GEMV launches back to back: {k_b2b * 1e3:.1f} us each; bracketed one by one: avg "
        f"{k_avg * 1e3:.1f} us, median {k_med * 1e3:.1f}, min {k_min * 1e3:.1f}")
    value = weight_bytes / (ms * 1e-3) / 1e9
    # the dominant kernel: at n = 1 the step's one launch, else the GEMV launch
    achieved = launch_bytes / ((ms if n == 1 else k_b2b) * 1e-3) / 1e9
    out = {
        "metric": "Q8_0 lm_head GEMV weight-stream GB/s (% of 8 TB/s HBM peak)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic",
        "config": {"workload": f"Q8_0 lm_head {rows}x{cols} ({weight_bytes} B), N={n}, quantize + GEMV, "
                               f"{ncopies} rotated seeded copies", "n": n, "weight_bytes": weight_bytes,
                   "copies": ncopies, "launches_per_step": 1 if n == 1 else 2, "accumulate": "f32"},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "gemv_only": {"us_back_to_back": round(k_b2b * 1e3, 2), "us_bracketed_avg": round(k_avg * 1e3, 2),
                      "us_bracketed_median": round(k_med * 1e3, 2), "us_bracketed_min": round(k_min * 1e3, 2),
                      "weight_gb_s": round(weight_bytes / (k_b2b * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic_from_q8_profile(n),
                     "kernel": "k_gemv_q8_split<true> (the whole step)" if n == 1 else "k_gemv_q8",
                     "algorithmic_bytes_per_launch": launch_bytes},
    }
    if host0 is not None:
        from oracle import oracle
        oracle.build(force=False)
        w, x = host0
        t0 = time.perf_counter()
        done = 0
        while True:
            oracle.q8w_gemv(w, oracle.quantize_q8_0(x), rows, cols, n)
            done += 1
            if time.perf_counter() - t0 > args.cpu_budget:
                break
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(done * weight_bytes / dt / 1e9, 3), "unit": "GB/s",
                               "cores": oracle.max_threads(), "kind": "oracle",
                               "sample": f"{done} quantize + Q8_0-weight GEMV passes over copy 0 "
                                         f"({weight_bytes} B each), {dt:.1f} s"}
    print(json.dumps(out), flush=True)
    return 0


ATTN_SRCS = [os.path.join(ROOT, "q4_weight_streaming_amd", "csrc", f)
              for f in ("q4s_attn.hip", "q4s_device.h", "q4s_internal.h")]
CHAIN_SRCS = [os.path.join(ROOT, "q4_weight_streaming_amd", "csrc", f)
              for f in ("q4s_chain.hip", "q4s_chain.h", "q4s_lane.h", "q4s_device.h", "q4s_internal.h")]


def chain_kernel_hash() -> str:
    h = hashlib.sha256()
    for f in CHAIN_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def chain_traffic_from_profile(model: str, mode: str):
    """HBM bytes per chained step (its k_chain launch) from the committed summary, if taken on
    the current chain source and for this model and sync mode; else None."""
    path = os.path.join(ROOT, "profiles", "chain_decode_step.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
    m = re.search(rf"hbm_bytes_per_launch\[{re.escape(model)} {re.escape(mode)}\]:\s*([0-9]+)", text)
    if not m_hash or not m or m_hash.group(1) != chain_kernel_hash():
        return None
    return float(m.group(1))


def attn_traffic_from_profile(L: int):
    """HBM bytes (fetch + write) of the attention step's two kernels from the committed
    summary, if taken on the current attention source; else None."""
    path = os.path.join(ROOT, "profiles", f"attn_decode_l{L}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = hashlib.sha256()
    for f in ATTN_SRCS:
        h.update(open(f, "rb").read())
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
    if not m or m.group(1) != h.hexdigest()[:16]:
        return None
    mb = [float(v) for v in re.findall(r"\| `k_attn_\w+(?:<\d+>)?` \| ([0-9.]+) MB \| ([0-9.]+) MB \|", text)
          for v in v]
    return round(sum(mb) * 1e6) if mb else None


def run_attn(args, dev, stream) -> int:
    """Decode attention of one layer of the 1.5B model (12 query / 2 kv heads, head dim 128) at
    the 32768-position context, over 8 rotated seeded KV caches (512 MB, beyond every cache)."""
    import numpy as np
    import torch

    from q4_weight_streaming_amd import _lib as q
    L, n_q, n_kv, ncopies = args.context, 12, 2, 8
    if L % 64:
        raise SystemExit("--context must be a multiple of 64")
    log(f"generating {ncopies} KV caches, L={L}")
    copies, host0 = [], None
    for c in range(ncopies):
        rng = np.random.default_rng([2026, 9, c])
        qv = rng.standard_normal((n_q, 128), dtype=np.float32)
        k = rng.standard_normal((L, n_kv, 128), dtype=np.float32)
        v = rng.standard_normal((L, n_kv, 128), dtype=np.float32)
        # the cache layouts the kernel reads: keys [kv][L/64][128][64], values [kv][L][128]
        kb = np.ascontiguousarray(k.transpose(1, 0, 2).reshape(n_kv, L // 64, 64, 128).transpose(0, 1, 3, 2))
        vh = np.ascontiguousarray(v.transpose(1, 0, 2))
        copies.append({"q": torch.from_numpy(qv).to(dev), "kb": torch.from_numpy(kb).to(dev),
                       "v": torch.from_numpy(vh).to(dev),
                       "o": torch.empty((n_q, 128), dtype=torch.float32, device=dev),
                       "ws": torch.empty(q.attn_workspace_bytes(n_q, L), dtype=torch.uint8, device=dev)})
        if c == 0 and not args.no_cpu_baseline:
            host0 = (qv, k, v)
    torch.cuda.synchronize()
    kv_bytes = 2 * L * n_kv * 128 * 4
    launch_bytes = kv_bytes + 2 * n_q * 128 * 4

    def step(c):
        return lambda: q.attn_decode(c["q"], c["kb"], c["v"], L, workspace=c["ws"], out=c["o"])

    if args.profile_only:
        for i in range(10):
            step(copies[i % ncopies])()
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        q.bench_copy(src, dst)
        torch.cuda.synchronize()
        log(f"profile run done: 10 attention steps of {launch_bytes} algorithmic bytes, one 1 GiB copy")
        return 0

    ms = time_steps([step(c) for c in copies], args.steps, args.warmup, stream)
    log(f"attention step {ms * 1e3:.2f} us")
    achieved = launch_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "decode attention KV-stream GB/s (% of 8 TB/s HBM peak)",
        "value": round(kv_bytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"GQA decode attention, {n_q} query / {n_kv} kv heads x 128, L={L} fp32 KV "
                               f"({kv_bytes} B), split-KV partial + combine, {ncopies} rotated seeded caches",
                   "context": L, "kv_bytes": kv_bytes, "launches_per_step": 2},
        "pct_of_peak": round(100 * kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": attn_traffic_from_profile(L),
                     "kernel": "k_attn_partial + k_attn_combine", "algorithmic_bytes_per_launch": launch_bytes},
    }
    if host0 is not None:
        from oracle import oracle
        oracle.build(force=False)
        qv, k, v = host0
        t0 = time.perf_counter()
        done = 0
        while True:
            oracle.attn_decode(qv, k, v)
            done += 1
            if time.perf_counter() - t0 > args.cpu_budget:
                break
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(done * kv_bytes / dt / 1e9, 3), "unit": "GB/s",
                               "cores": oracle.max_threads(), "kind": "oracle",
                               "sample": f"{done} fp64 attention passes over KV cache 0 ({kv_bytes} B each), {dt:.1f} s"}
    print(json.dumps(out), flush=True)
    return 0


CHAIN_MODES = {"tagged": 2, "tree": 1, "counter": 0}


def run_chain(args, dev, stream) -> int:
    """The chained decode step (a token's layers as dependent phases in one launch) over the
    Qwen2.5-1.5B or -7B-shaped stack, each phase synchronisation mode, two rotated seeded
    weight copies; a phase timeline from the step's own clock marks."""
    import numpy as np
    import torch

    from q4_weight_streaming_amd import _lib as q
    from q4_weight_streaming_amd import synth
    model = args.chain_model
    L, E, D, F, V = (28, 1536, 256, 8960, 151936) if model == "1.5b" else (28, 3584, 512, 18944, 152064)
    shapes = [(E, E), (D, E), (D, E), (E, E), (F, E), (F, E), (E, F)] * L + [(V, E)]
    ncopies = 2
    log(f"generating {ncopies} copies of the {model} chain ({len(shapes)} matrices)")
    copies, host0 = [], None
    for c in range(ncopies):
        ws = [synth.q4_0_weights(r, cc, synth.generator(70 + c, m, 0, 0)) for m, (r, cc) in enumerate(shapes)]
        wp = [q.repack_q4_0(torch.from_numpy(w.reshape(-1)).to(dev), r, cc) for w, (r, cc) in zip(ws, shapes)]
        h0 = synth.activation(1, E, synth.generator(70 + c, 999, 0, 1))[0]
        copies.append({"wp": wp, "h0": torch.from_numpy(h0).to(dev),
                       "acts": torch.empty(q.chain_act_words(L, E, D, F, V), dtype=torch.int64, device=dev),
                       "logits": torch.empty(V, dtype=torch.float32, device=dev)})
        if c == 0 and not args.no_cpu_baseline:
            host0 = (ws, h0)
        del ws
    torch.cuda.synchronize()
    modes = list(CHAIN_MODES) if args.sync == "all" else [args.sync]
    if args.profile_only:
        # 10 steps of the first mode over the rotated copies, then a 1 GiB copy to calibrate counters
        chains = [q.Chain(L, E, D, F, V, c["wp"], c["h0"], c["acts"], c["logits"], sync_mode=CHAIN_MODES[modes[0]],
                          workgroups=args.chain_workgroups) for c in copies]
        for ch in chains:
            ch.set_cooperative(not args.chain_plain_launch)
        for i in range(10):
            chains[i % ncopies].run()
        for ch in chains:
            ch.check()
            ch.close()
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        q.bench_copy(src, dst)
        torch.cuda.synchronize()
        del chains, src, dst
        copies.clear()
        torch.cuda.empty_cache()
        log(f"profile run done: 10 chained steps ({modes[0]}), one 1 GiB copy")
        return 0
    results, chains_by_mode = {}, {}
    for mode in modes:
        chains = [q.Chain(L, E, D, F, V, c["wp"], c["h0"], c["acts"], c["logits"], sync_mode=CHAIN_MODES[mode],
                          workgroups=args.chain_workgroups) for c in copies]
        for ch in chains:
            ch.set_cooperative(not args.chain_plain_launch)
        ms = time_steps([ch.run for ch in chains], args.steps, args.warmup, stream)
        for ch in chains:
            ch.check()
        # phase timeline: the end of a phase is when its last workgroup finishes it
        tr = chains[0].set_trace(True)
        chains[0].run()
        chains[0].check()
        chains[0].set_trace(False)
        info = chains[0].info()
        t = tr.cpu().numpy().astype(np.float64)
        P, wg = info["n_phases"], info["workgroups"]
        ends = t[:P * wg].reshape(P, wg)
        start = t[P * wg:P * wg + wg].min()
        ready = t[2 * P * wg + wg:3 * P * wg + wg].reshape(P, wg)
        crit = ends.max(axis=1)
        dur = np.diff(np.concatenate([[start], crit])) / 100.0  # 100 MHz clock -> us
        names = ["qkv", "o", "gate_up", "down"]
        per = {name: round(float(np.median(dur[i:4 * L:4])), 2) for i, name in enumerate(names)}
        per["head"] = round(float(dur[-1]), 2)
        # per phase: how long after the previous phase's last workgroup the first tiles had
        # their activation (median over the phase's workgroups), medians over the layers
        wait = [float(np.median((ready[p][ready[p] > 0] - crit[p - 1]) / 100.0)) for p in range(1, P)]
        ready_us = {name: round(float(np.median(wait[i - 1::4] if i else wait[3:P - 2:4])), 2)
                    for i, name in enumerate(names)}   # (qkv: layers 1.. -- the head is phase P - 1)
        results[mode] = {"us_per_step": round(ms * 1e3, 1), "workgroups": wg, "phase_us_median": per,
                         "input_ready_after_us": ready_us}
        log(f"chain {model} {mode}: {ms * 1e3:.1f} us per step; phases (median us) {per}; "
            f"input ready after (median us) {ready_us}")
        chains_by_mode[mode] = chains
    packed = info["packed_bytes"]
    # release the chains and the device memory before the CPU baseline and the interpreter's exit
    # (nothing of the GPU work is left for teardown to free)
    for chs in chains_by_mode.values():
        for ch in chs:
            ch.close()
    chains_by_mode.clear()
    del chains, tr
    copies.clear()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    best = min(results, key=lambda m: results[m]["us_per_step"])
    us = results[best]["us_per_step"]
    achieved = packed / (us * 1e-6) / 1e9
    out = {
        "metric": "chained decode step: weight-stream GB/s (% of 8 TB/s HBM peak), step time",
        "value": round(achieved, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"Qwen2.5-{model}-shaped chained step: {L} layers x 4 dependent phases + head "
                               f"({P} phases, {len(shapes)} Q4_0 matrices, {packed} B), norm + Q8_0 prologues, "
                               f"residual epilogues, one cooperative launch, {ncopies} rotated seeded copies",
                   "sync": best, "modes": results},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": chain_traffic_from_profile(model, best),
                     "kernel": f"k_chain<{best}>",
                     "algorithmic_bytes_per_launch": packed},
    }
    if host0 is not None:
        from oracle import oracle
        oracle.build(force=False)
        ws, h0 = host0
        t0 = time.perf_counter()
        done = 0
        while True:
            oracle.chain_step(ws, E, D, F, V, h0)
            done += 1
            if time.perf_counter() - t0 > args.cpu_budget:
                break
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(done * packed / dt / 1e9, 3), "unit": "GB/s",
                               "cores": oracle.max_threads(), "kind": "oracle",
                               "sample": f"{done} fixed-order oracle chained steps over copy 0 ({packed} B each), "
                                         f"{dt:.1f} s"}
    print(json.dumps(out), flush=True)
    return 0


def timeline_summary(trace, n_tiles: int, waves: int, bin_us: float = 1.0) -> dict:
    """A traced launch (q4s_sweep_set_trace: per workgroup its start and its waves' ends on
    the 100 MHz clock) as when workgroups start and finish: the span, how fast the launch
    reaches its peak concurrency, when the last workgroup starts, how long the last 5% and
    the last workgroup take, and the number of workgroups running per bin."""
    import numpy as np
    t = trace.reshape(n_tiles, 9).astype(np.float64)
    start = t[:, 0]
    end = t[:, 1:1 + waves].max(axis=1)
    t0 = start.min()
    start, end = (start - t0) / 100.0, (end - t0) / 100.0      # us
    span = float(end.max())
    ev = np.concatenate([np.stack([start, np.ones_like(start)], 1), np.stack([end, -np.ones_like(end)], 1)])
    ev = ev[np.lexsort((ev[:, 1], ev[:, 0]))]
    conc = np.cumsum(ev[:, 1])
    peak = float(conc.max())
    ramp = float(ev[np.argmax(conc >= 0.9 * peak), 0])
    done = np.sort(end)
    edges = np.arange(0.0, span + bin_us, bin_us)
    running = [int(((start < b + bin_us) & (end > b)).sum()) for b in edges[:-1]]
    dur = end - start
    return {"span_us": round(span, 2), "workgroups": n_tiles, "peak_concurrent": int(peak),
            "ramp_to_90pct_us": round(ramp, 2), "last_start_us": round(float(start.max()), 2),
            "drain_after_last_start_us": round(span - float(start.max()), 2),
            "last_5pct_of_workgroups_us": round(span - float(done[int(0.95 * (n_tiles - 1))]), 2),
            "workgroup_us_median": round(float(np.median(dur)), 2), "workgroup_us_max": round(float(dur.max()), 2),
            "running_per_us": running}


def sweep_plans(shapes, copies, n: int, act_cfg: int, dev):
    """Sweeps of n activation rows over the weights of each copy, with fresh seeded activations."""
    import torch

    from q4_weight_streaming_amd import _lib as q
    from q4_weight_streaming_amd import synth
    plans, mats_all = [], []
    for c, m in enumerate(copies):
        mats_v = []
        for mi, (s, mm) in enumerate(zip(shapes, m)):
            x = synth.activation(n, s.cols, synth.generator(act_cfg, mi, c, 1),
                                 outliers=0 if s.name == "lm_head" and len(shapes) == 1 else 8)
            mats_v.append({"w_packed": mm["w_packed"], "x": torch.from_numpy(x).to(dev),
                           "x_q8": torch.empty(q.q8_bytes(n, s.cols), dtype=torch.uint8, device=dev),
                           "y": torch.empty((n, s.rows), dtype=torch.float32, device=dev),
                           "rows": s.rows, "cols": s.cols})
        plans.append(q.Sweep(mats_v, n))
        mats_all.append(mats_v)
    return plans, mats_all


def step_kernel_name(shapes, n: int, fused: bool) -> str:
    """The kernel that dominates a step (the whole step when it is one launch)."""
    if fused:
        split = n == 1 and all(s.cols <= 2048 for s in shapes)
        return ("k_sweep_split<true> (the whole step)" if split else "k_sweep_fused (the whole step)") if n == 1 \
            else f"k_sweep_fused<{n}> (the whole step)"
    if n == 1:
        return "k_sweep_one (GEMV launch of the sweep)"
    return (f"k_sweep<{n}>" if n <= 8 else "k_sweep_tiled") + " (GEMV launch of the sweep)"


def measure_plans(name, shapes, full, mats_all, n: int, args, stream):
    """Times the step (the full plans) and, when the step takes two launches, the GEMV launch
    alone over the quantized activations; returns the timings and the step's roofline."""
    from q4_weight_streaming_amd import _lib as q
    info = full[0].info()
    fused = bool(info["fused_quantize"])
    weight_bytes = info["weight_bytes"]
    launch_bytes = info["weight_bytes"] + info["act_bytes"] + info["out_bytes"]
    if fused:
        # one launch per step: fp32 activations read, Q8_0 bytes written, weights, y
        launch_bytes += sum(4 * n * s.cols for s in shapes)
    ms = time_steps([p.run for p in full], args.steps, args.warmup, stream)
    gemv = [q.Sweep([{k: v for k, v in mm.items() if k != "x"} for mm in m], n) for m in mats_all]
    k_b2b = time_steps([p.run for p in gemv], args.steps, args.warmup, stream)
    k_avg, k_med, k_min = time_kernel([p.run for p in gemv], args.steps, stream)
    dom_ms = ms if fused else k_b2b
    if not fused:  # the GEMV launch's bytes: Q8_0 activations read, no fp32 activations
        launch_bytes = info["weight_bytes"] + info["act_bytes"] + info["out_bytes"]
    achieved = launch_bytes / (dom_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(name, n, launch_bytes)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
            "kernel": step_kernel_name(shapes, n, fused), "algorithmic_bytes_per_launch": launch_bytes}
    gemv_only = {"us_back_to_back": round(k_b2b * 1e3, 2), "us_bracketed_avg": round(k_avg * 1e3, 2),
                 "us_bracketed_median": round(k_med * 1e3, 2), "us_bracketed_min": round(k_min * 1e3, 2),
                 "weight_gb_s": round(weight_bytes / (k_b2b * 1e-3) / 1e9, 1)}
    for p in gemv:
        p.close()
    return {"ms": ms, "fused": fused, "info": info, "weight_bytes": weight_bytes, "roofline": roof,
            "gemv_only": gemv_only}


def extra_workload(name: str, ns, args, dev, stream) -> dict:
    """A further configuration on the same line: the step at each row count in ns (the first
    is 1), as weight GB/s, % of peak and the step's roofline; t(n)/t(1) for n > 1."""
    import torch
    shapes, cfg, ncopies = workload_shapes(name)
    log(f"generating {ncopies} copies of {name} ({len(shapes)} matrices)")
    copies = []
    for c in range(ncopies):
        mats, _ = make_copy(shapes, cfg, c, 1, dev, keep_host=False)
        copies.append(mats)
    res, t1 = {}, None
    for n in ns:
        full, mats_all = sweep_plans(shapes, copies, n, cfg if n == 1 else 3, dev)
        r = measure_plans(name, shapes, full, mats_all, n, args, stream)
        for p in full:
            p.close()
        t1 = r["ms"] if n == 1 else t1
        gbs = r["weight_bytes"] / (r["ms"] * 1e-3) / 1e9
        e = {"ms_per_step": round(r["ms"], 5), "weight_gb_s": round(gbs, 1),
             "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2), "launches_per_step": 1 if r["fused"] else 2,
             "roofline": r["roofline"], "gemv_only_us": r["gemv_only"]["us_back_to_back"]}
        if n == 1 and name.startswith("qwen"):
            e["tok_s"] = round(1000.0 / r["ms"], 1)
        if n > 1 and t1:
            e["ratio_to_n1"] = round(r["ms"] / t1, 3)
        res[f"n{n}"] = e
        log(f"{name} n={n}: step {r['ms'] * 1e3:.1f} us, {gbs:.0f} GB/s, roofline frac {r['roofline']['frac']}")
        del full, mats_all
    res["workload"] = (f"{name}: {len(shapes)} Q4_0 matrices ({sum(s.q4_bytes for s in shapes)} B), "
                       f"{ncopies} rotated seeded copies, fresh seeded activations per matrix")
    del copies
    torch.cuda.empty_cache()
    return res


def run_sweep(args, dev, stream) -> int:
    import torch

    from q4_weight_streaming_amd import _lib as q
    shapes, cfg, ncopies = workload_shapes(args.workload)
    n = args.n
    log(f"generating {ncopies} copies of {args.workload} ({len(shapes)} matrices), n={n}")
    copies, host0 = [], None
    for c in range(ncopies):
        mats, host = make_copy(shapes, cfg, c, n, dev, keep_host=(c == 0 and not args.no_cpu_baseline))
        copies.append(mats)
        if c == 0:
            host0 = host
        log(f"copy {c} ready")
    full = [q.Sweep(m, n) for m in copies]                                 # quantize + GEMV

    if args.profile_only:
        info = full[0].info()
        gemv = [q.Sweep([{k: v for k, v in mm.items() if k != "x"} for mm in m], n) for m in copies]
        for i in range(10):
            full[i % ncopies].run()              # the step (quantized activations in place)
        for i in range(10):
            gemv[i % ncopies].run()
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        q.bench_copy(src, dst)
        torch.cuda.synchronize()
        log(f"profile run done: 10 steps and 10 GEMV-only sweeps ({info['weight_bytes']} weight bytes), "
            "one 1 GiB copy")
        return 0

    r = measure_plans(args.workload, shapes, full, copies, n, args, stream)
    ms, fused, info, weight_bytes = r["ms"], r["fused"], r["info"], r["weight_bytes"]
    log(f"step {ms * 1e3:.1f} us ({'one fused launch' if fused else 'quantize + GEMV launches'})")
    g = r["gemv_only"]
    log(f"GEMV-only launches back to back: {g['us_back_to_back']:.1f} us each; bracketed one by one: avg "
        f"{g['us_bracketed_avg']:.1f} us, median {g['us_bracketed_median']:.1f}, min {g['us_bracketed_min']:.1f}")

    value = weight_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"{args.workload} decode sweep, {len(shapes)} Q4_0 matrices "
                               f"({weight_bytes} B), N={n}, fresh Q8_0-quantized fp32 activation per "
                               f"matrix, {ncopies} rotated seeded copies",
                   "n": n, "matrices": len(shapes), "weight_bytes": weight_bytes, "copies": ncopies,
                   "launches_per_step": 1 if fused else 2, "quantize": "fused" if fused else "own launch",
                   "accumulate": "f32", "gemv_tiles": info["n_tiles"]},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "tok_s": round(1000.0 / ms, 1) if n == 1 and args.workload.startswith("qwen") else None,
        "gemv_only": g,
        "roofline": r["roofline"],
    }

    if args.timeline:
        # one traced step after the timed ones: when the step launch's workgroups start and finish
        waves = 8 if (n == 1 and all(sh.cols <= 2048 for sh in shapes)) else 4
        tr = full[0].set_trace(True)
        full[1 % ncopies].run()
        full[0].run()
        torch.cuda.synchronize()
        full[0].set_trace(False)
        tl = timeline_summary(tr.cpu().numpy(), info["n_tiles"], waves)
        out["timeline"] = tl
        log(f"timeline: span {tl['span_us']} us, peak {tl['peak_concurrent']} workgroups, ramp {tl['ramp_to_90pct_us']} us, "
            f"last start {tl['last_start_us']} us, drain {tl['drain_after_last_start_us']} us, "
            f"last 5% {tl['last_5pct_of_workgroups_us']} us, workgroup median {tl['workgroup_us_median']} us")

    if n == 1 and not args.no_verify_ratio:
        # the same weight copies stepped with several activation rows (multi-token verify)
        verify = {}
        for nv in sorted({int(v) for v in args.verify_n.split(",") if v}):
            plans, _ = sweep_plans(shapes, copies, nv, 3, dev)
            msv = time_steps([p.run for p in plans], args.steps, args.warmup, stream)
            verify[f"n{nv}"] = {"ms_per_step": round(msv, 5), "ratio_to_n1": round(msv / ms, 3),
                                "launches_per_step": 1 if plans[0].info()["fused_quantize"] else 2}
            log(f"n={nv} step {msv * 1e3:.1f} us, ratio {msv / ms:.3f}")
            for p in plans:
                p.close()
            del plans
        out["verify"] = verify

    if args.workload == "gemv1536":
        # each GEMV as its own launch over its quantized activation, bracketed by events on the stream
        m0 = copies[0]
        outs = [torch.empty((n, s.rows), dtype=torch.float32, device=dev) for s in shapes]
        fns = [lambda mm=mm, o=o: q.gemv_q4_0(mm["w_packed"], mm["x_q8"], mm["rows"], mm["cols"], n, out=o)
               for mm, o in zip(m0, outs)]
        for f in fns:
            f()
        torch.cuda.synchronize()
        s_avg, s_med, s_min = time_kernel(fns, len(fns), stream)
        per = shapes[0].rows * (shapes[0].cols // 32) * 18
        out["single_gemv"] = {"launches": len(fns), "us_bracketed_avg": round(s_avg * 1e3, 2),
                              "us_bracketed_median": round(s_med * 1e3, 2), "us_bracketed_min": round(s_min * 1e3, 2),
                              "weight_gb_s_at_median": round(per / (s_med * 1e-3) / 1e9, 1),
                              "note": "one 1536x1536 GEMV per launch; the bracket holds the dispatch latency"}
        log(f"single GEMV launch: median {s_med * 1e3:.2f} us, min {s_min * 1e3:.2f} us")

    if args.workload == "qwen2.5-1.5b" and n == 1 and not args.no_extra_configs:
        # the other configurations' pass bars on the same line: the lone head, the 7B stream at N = 1 and 8
        for p in full:
            p.close()
        del full, copies
        torch.cuda.empty_cache()
        out["lm_head"] = extra_workload("lm_head", [1], args, dev, stream)
        out["qwen2.5-7b"] = extra_workload("qwen2.5-7b", [1, 8], args, dev, stream)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(host0, shapes, n, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen2.5-1.5b",
                    choices=["qwen2.5-1.5b", "qwen2.5-7b", "lm_head", "gemv1536", "lm_head_q8", "attn", "chain"])
    ap.add_argument("--chain-model", default="1.5b", choices=["1.5b", "7b"], help="stack of --workload chain")
    ap.add_argument("--sync", default="all", choices=["all", *CHAIN_MODES], help="phase sync of --workload chain")
    ap.add_argument("--chain-workgroups", type=int, default=0, help="persistent workgroups (0: one per CU)")
    ap.add_argument("--chain-plain-launch", action="store_true",
                    help="launch the chained step without the cooperative-launch call (for the profiler)")
    ap.add_argument("--context", type=int, default=32768, help="KV positions for --workload attn")
    ap.add_argument("--n", type=int, default=1, help="activation rows per GEMV (1..24; 1..8 for lm_head_q8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify-ratio", action="store_true", help="skip the N=8 / N=1 step-cost ratio")
    ap.add_argument("--timeline", action="store_true",
                    help="add the step launch's per-workgroup timeline (one traced step) to the line")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="with the default workload, skip the lone-head and 7B lines")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work (half all-thread, half single)")
    ap.add_argument("--verify-n", default="2,4,8,16,24",
                    help="comma list of row counts for the step-cost curve t(N)/t(1)")
    ap.add_argument("--profile-only", action="store_true",
                    help="run a few GEMV-only sweeps plus a 1 GiB copy, for rocprofv3 counter runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU part)", file=sys.stderr)
        return 2
    if not 1 <= args.n <= (8 if args.workload == "lm_head_q8" else 24):
        raise SystemExit("--n must be in 1..24 (1..8 for lm_head_q8)")

    import torch

    from q4_weight_streaming_amd import _lib as q
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    q.lib()

    if args.workload == "lm_head_q8":
        return run_q8_head(args, dev, stream)
    if args.workload == "attn":
        return run_attn(args, dev, stream)
    if args.workload == "chain":
        return run_chain(args, dev, stream)
    return run_sweep(args, dev, stream)


if __name__ == "__main__":
    sys.exit(main())
