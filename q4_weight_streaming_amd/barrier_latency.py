"""Grid-barrier cost on this GPU: the per-barrier time of each q4s_bench_grid_barrier kind.

One persistent cooperative launch of n workgroups (256 threads each, all resident at
once) passes `phases` grid barriers; the per-barrier cost is (time with 2001 phases -
time with 1 phase) / 2000, over 10 timed launches each after 3 warm-up launches, HIP
events on the launch stream.  Every wait in the kernels is bounded, and the scratch
words are zeroed by each call.  Prints one line per (kind, workgroups) on stderr and a
JSON summary on stdout.

  python -m q4_weight_streaming_amd.barrier_latency [--wg 64,256,512,1024,2048] [--kinds 0,1,...,9]
"""
from __future__ import annotations

import argparse
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--wg", default="64,256,512,1024,2048")
    ap.add_argument("--kinds", default="0,1,2,3,4,5,6,7,8,9")
    ap.add_argument("--phases", type=int, default=2001)
    ap.add_argument("--reps", type=int, default=10)
    args = ap.parse_args()

    import torch

    from q4_weight_streaming_amd import _lib as q
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    max_wg = q.grid_barrier_max_workgroups()
    wgs = [w for w in (int(v) for v in args.wg.split(",")) if 1 <= w <= max_wg]
    scratch = torch.zeros(q.grid_barrier_scratch_bytes(max(wgs)) // 4 + 16, dtype=torch.int32, device=dev)

    def launch_ms(kind: int, n: int, phases: int) -> float:
        for _ in range(3):
            q.bench_grid_barrier(kind, n, phases, scratch)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.reps):
            q.bench_grid_barrier(kind, n, phases, scratch)
        b.record(stream)
        torch.cuda.synchronize()
        if int(scratch[1].item()) != 0:
            raise RuntimeError(f"kind {kind}, {n} workgroups: a workgroup gave up waiting")
        return a.elapsed_time(b) / args.reps

    rows = []
    for kind in (int(v) for v in args.kinds.split(",")):
        for n in wgs:
            t1 = launch_ms(kind, n, 1)
            tp = launch_ms(kind, n, args.phases)
            us = (tp - t1) * 1e3 / (args.phases - 1)
            rows.append({"kind": kind, "workgroups": n, "us_per_barrier": round(us, 3)})
            print(f"kind {kind} wg {n:5d}: {us:8.3f} us per barrier", file=sys.stderr, flush=True)
    print(json.dumps({"max_workgroups": max_wg, "barriers": rows}))
    return 0


if __name__ == "__main__":
    sys.exit(main())
