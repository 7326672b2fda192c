"""Benchmark of the batched sampler with support capture on one MI355X.

One step = one call of ``tsc_sample_with_mask`` over a whole batch: every row of the
B=256, V=151936 bfloat16 workload (0.125-grid Gaussian logits, per-row temperature U[0.6, 1.2],
top_k=1024, top_p=0.95, every row opted in, packed width 2048) is sampled and captured.
The logits are resident in HBM before timing starts; enough copies of them rotate (more than
512 MB in total) that the 256 MB Infinity Cache cannot serve a call's read from the previous
call. Prints one JSON line (rank 0).

``value`` is rows/s over the timed steps (wall clock, bracketed by device synchronizations).
``roofline`` prices the kernel against MI355X's 8 TB/s HBM with the algorithmic bytes of a
call: B*V*2 (one read of the logits) + sum over opt-in rows of min(L, W)*8 (ids + logprobs) +
R*8 (length + selected logprob) + B*5 (token + status), divided by the kernel's average
duration from HIP events on the stream the kernel runs on.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "sampled rows/s and achieved HBM GB/s (% of peak) at B=256, V=151936"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "top_support_capture_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(bytes_per_launch_alg: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_b256_v151936_bf16.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(wl, budget_s: float = 12.0) -> dict:
    import oracle
    rows, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and rows < wl.B:
        r = rows
        oracle.sample_row(oracle.decode_logits(wl.logits[r], wl.dtype), wl.temperature[r],
                          wl.top_k[r], wl.top_p[r], wl.min_p[r], int(wl.seeds[r]),
                          int(wl.positions[r]))
        rows += 1
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"first {rows} rows of the B={wl.B}, V={wl.V} bf16 batch, one process "
                      f"(numpy sort-based float64 oracle), {dt:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: rows are independent, so the sampler shards by "
              "rows with no communication; run it with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import top_support_capture_amd as tsc
    from workloads import make_workload
    from tests.gpu_helpers import device_inputs

    wl = make_workload(args.workload)
    dev = torch.device("cuda:0")
    d = device_inputs(wl)
    in_bytes = wl.B * wl.V * (2 if wl.dtype == "bf16" else 4)
    ncopies = max(1, -(-512 * 2**20 // in_bytes) + 1)
    copies = [d["logits"]] + [d["logits"].clone() for _ in range(ncopies - 1)]
    out = tsc.sample_with_mask(copies[0], d["temperature"], d["top_k"], d["top_p"], d["min_p"],
                               d["optin_rows"], d["seeds"], d["positions"], wl.W)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        tsc.sample_with_mask(copies[i % ncopies], d["temperature"], d["top_k"], d["top_p"],
                             d["min_p"], d["optin_rows"], d["seeds"], d["positions"], wl.W, out=out)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Timed region: K steps between device synchronizations (wall clock), with HIP events on the
    # launch stream around every call for the kernel's own average duration.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    durs_ms = np.array([a.elapsed_time(b) for a, b in ev])

    lengths = out.lengths.cpu().numpy().astype(np.int64)
    status = out.row_status.cpu().numpy()
    alg_bytes = in_bytes + int(np.minimum(lengths, wl.W).sum()) * 8 + wl.R * 8 + wl.B * 5
    avg_s = float(durs_ms.mean()) * 1e-3
    achieved = alg_bytes / avg_s / 1e9
    traffic = measured_traffic(alg_bytes)
    rows_per_s = wl.B * args.steps / wall
    line = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian logits on a 0.125 grid, cast to bfloat16)",
        "config": {"workload": wl.name, "B": wl.B, "V": wl.V, "logits": wl.dtype, "top_k": 1024,
                   "top_p": 0.95, "temperature": "U[0.6,1.2] per row", "R": wl.R, "W": wl.W,
                   "input_copies_rotated": ncopies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic},
        "kernel_ms": {"mean": float(durs_ms.mean()), "p10": float(np.percentile(durs_ms, 10)),
                      "p50": float(np.median(durs_ms)), "p90": float(np.percentile(durs_ms, 90))},
        "algorithmic_bytes_per_launch": alg_bytes,
        "rows_overflow": int(np.count_nonzero(status == 1)),
        "rows_not_ok": int(np.count_nonzero(status >= 2)),
        "mean_support": float(lengths.mean()),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
