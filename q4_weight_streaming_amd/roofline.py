"""Achievable HBM read bandwidth on this GPU: the streaming-read microbenchmark.

One launch reads a buffer far larger than the 256 MB Infinity Cache with
16-byte loads, L loads in flight per thread, over a range of grid sizes; the
best rate is the practical ceiling the GEMV is compared with (the roofline
method of the minfer README, milestone M15: one launch over a large buffer,
several 16-byte loads in flight per thread).  A plain copy is timed as well.

  python -m q4_weight_streaming_amd.roofline [--gib 4] [--reps 5]
  python -m q4_weight_streaming_amd.roofline --sizes 131,868 [--reps 20] [--wg 2048,4096] [--lif 4,8]

--sizes times reads of the sizes the GEMV streams (MB, e.g. the 1.5B output head
and the whole 1.5B sweep) the way the benchmark times its steps: launches back to
back, four rotated buffers (past the Infinity Cache), over a small grid of loads
in flight and workgroups, and in the GEMV's own pattern (q4s_bench_read_units:
each wave streams one contiguous unit -- a 9216-byte chunk, a row group of 6 or
9 chunks -- with 1 KB wave loads).  The unit pattern is the reference: the
grid-stride kernel's loads in flight sit a power-of-two stride apart, which
some grid sizes serve far more slowly.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gib", type=float, default=4.0)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--sizes", default="", help="comma-separated MB: back-to-back reads of these sizes")
    ap.add_argument("--wg", default="2048,4096,8192,16384", help="workgroup counts for --sizes")
    ap.add_argument("--lif", default="4,8", help="loads in flight (1, 2, 4 or 8) for --sizes")
    args = ap.parse_args()
    if args.sizes:
        return by_size([int(v) for v in args.sizes.split(",")], max(args.reps, 10),
                       [int(v) for v in args.wg.split(",")], [int(v) for v in args.lif.split(",")])

    import torch

    from q4_weight_streaming_amd import _lib as q
    dev = torch.device("cuda:0")
    nbytes = int(args.gib * (1 << 30)) // 16 * 16
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(args.reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        ts.sort()
        return ts[len(ts) // 2]

    rows = []
    for lif in (1, 2, 4, 8):
        for blocks in (256, 512, 1024, 2048, 4096, 8192, 16384):
            t = timed(lambda: q.bench_read(buf, lif, blocks, sink))
            rows.append({"loads_in_flight": lif, "workgroups": blocks, "gb_s": round(nbytes / t / 1e9, 1)})
            print(f"read L={lif} wg={blocks:6d}: {nbytes / t / 1e9:8.1f} GB/s", file=sys.stderr, flush=True)
    half = nbytes // 2 // 16 * 16
    src, dst = buf[:half], buf[half:2 * half]
    t = timed(lambda: q.bench_copy(src, dst))
    copy = round(2 * half / t / 1e9, 1)
    print(f"copy: {copy} GB/s (read + write)", file=sys.stderr)
    best = max(rows, key=lambda r: r["gb_s"])
    print(json.dumps({"buffer_bytes": nbytes, "best_read": best, "copy_gb_s": copy, "sweep": rows}))
    return 0


def by_size(sizes_mb, reps, wgs, lifs) -> int:
    import torch

    from q4_weight_streaming_amd import _lib as q
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    out = []
    for mb in sizes_mb:
        n = mb * 1000 * 1000 // 16 * 16
        bufs = [torch.ones(n, dtype=torch.uint8, device=dev) for _ in range(4)]
        rows = []
        for lif in lifs:
            for blocks in wgs:
                for i in range(3):
                    q.bench_read(bufs[i % 4], lif, blocks, sink)
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for i in range(reps):
                    q.bench_read(bufs[i % 4], lif, blocks, sink)
                b.record(stream)
                torch.cuda.synchronize()
                us = a.elapsed_time(b) * 1e3 / reps
                rows.append({"loads_in_flight": lif, "workgroups": blocks, "us": round(us, 2),
                             "gb_s": round(n / us / 1e3, 1)})
                print(f"{mb} MB L={lif} wg={blocks:6d}: {us:7.1f} us {n / us / 1e3:8.1f} GB/s", file=sys.stderr,
                      flush=True)
        units = []
        for ub in (9216, 6 * 9216, 9 * 9216):
            nb = n // ub * ub
            for i in range(3):
                q.bench_read_units(bufs[i % 4], ub, sink)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(reps):
                q.bench_read_units(bufs[i % 4], ub, sink)
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / reps
            units.append({"unit_bytes": ub, "bytes_read": nb, "us": round(us, 2), "gb_s": round(nb / us / 1e3, 1)})
            print(f"{mb} MB units of {ub} B: {us:7.1f} us {nb / us / 1e3:8.1f} GB/s", file=sys.stderr, flush=True)
        best = max(rows, key=lambda r: r["gb_s"])
        out.append({"mb": mb, "bytes": n, "best": best, "grid": rows, "units": units,
                    "best_units": max(units, key=lambda r: r["gb_s"])})
        del bufs
    print(json.dumps({"back_to_back_reads": out}))
    return 0


if __name__ == "__main__":
    sys.exit(main())
