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
R*8 (length + selected logprob) + B*5 (token + status), divided by the kernel's average launch
duration: HIP events on the launch stream around the K timed calls, over K.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same workload.

``--kernel csr`` times ``tsc_support_csr`` on a sampler call's capture, and the copy to pinned
host memory of the CSR payload (sized by the realized support) against that of the packed
[R, W] buffers (sized by the capacity).

``--kernel replay`` times ``tsc_replay_logprob`` instead: the supports and tokens a sampler call
captured on the workload, replayed on new logits (the workload's logits plus seeded N(0, 0.25^2)
noise, cast back to the same dtype); one step = one replay call over all captured rows.
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


# Kernels whose HBM traffic the counter summaries cover: name in the profiler's trace, prefix of
# the summary file.
TRAFFIC_KERNELS = {"sample": ("sample_fast_kernel", "traffic"),
                   "replay": ("replay_kernel", "traffic_replay")}


def traffic_path(wl, kernel: str = "sample") -> str:
    prefix = TRAFFIC_KERNELS[kernel][1]
    return os.path.join(ROOT, "profiles", f"{prefix}_{wl.name}.json")


def measured_traffic(wl, kernel: str = "sample"):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this workload and
    kernel, if it was taken on the current kernel sources; else None."""
    path = traffic_path(wl, kernel)
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("kernel_source_hash") != kernel_source_hash() or t.get("workload") != wl.name:
        return None
    return t.get("hbm_bytes_per_launch")


_CPU_WL = None


def _cpu_worker_init(index: int) -> None:
    global _CPU_WL
    from workloads import make_workload
    _CPU_WL = make_workload(index)


def _oracle_rows(args):
    """Worker: oracle.sample_row over rows start, start + step, ... of the batch (cycling) until
    the budget is spent; bf16 decoding is done once per row outside the clock."""
    start, step, budget_s = args
    import oracle
    wl = _CPU_WL
    decoded = {}
    rows, busy = 0, 0.0
    r = start
    while busy < budget_s:
        if r not in decoded:
            decoded[r] = oracle.decode_logits(wl.logits[r], wl.dtype)
        t = time.perf_counter()
        oracle.sample_row(decoded[r], wl.temperature[r], wl.top_k[r], wl.top_p[r], wl.min_p[r],
                          int(wl.seeds[r]), int(wl.positions[r]))
        busy += time.perf_counter() - t
        rows += 1
        r = (r + step) % wl.B
    return rows, busy


def cpu_baseline(wl, index: int, budget_s: float = 8.0, max_workers: int = 16) -> dict:
    """The CPU oracle (as it stands) on a bounded sample of the batch: one process alone, then one
    process per available core (at most ``max_workers``), each sampling rows for ``budget_s``
    seconds of its own time. ``value`` is the all-core rate (each worker's rows over its busy
    time, summed)."""
    import multiprocessing as mp
    global _CPU_WL
    _CPU_WL = wl
    n1, t1 = _oracle_rows((0, 1, budget_s / 2))
    ncores = max(1, min(len(os.sched_getaffinity(0)), max_workers))
    # Fresh interpreters (spawn): the workers inherit nothing from this process, which holds the
    # GPU; each rebuilds the seeded workload.
    ctx = mp.get_context("spawn")
    with ctx.Pool(ncores, initializer=_cpu_worker_init, initargs=(index,)) as pool:
        res = pool.map(_oracle_rows, [(w, ncores, budget_s) for w in range(ncores)])
    rate = sum(n / b for n, b in res)
    total = sum(n for n, _ in res)
    return {"value": rate, "unit": "rows/s", "cores": ncores, "kind": "oracle",
            "single_core_value": n1 / t1, "cpu_model": cpu_model(),
            "sample": f"{total} rows of the B={wl.B}, V={wl.V} {wl.dtype} batch (cycled) through "
                      f"oracle.sample_row, {ncores} worker processes x {budget_s:.0f} s each "
                      f"(one thread each), plus {n1} rows in one process for the 1-core rate; "
                      f"bf16 decoding done once per row outside the clock"}


def cpu_model() -> str:
    """The host CPU's model name as lscpu prints it (falling back to /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.strip().startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            return next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        return "unknown CPU"


def oracle_check(wl, got: dict) -> dict:
    """The timed call's outputs against the CPU oracle on every row of the batch (worker
    processes): mismatching rows, and the rows the oracle reports near a decision boundary, by
    kind (they are counted, and exempt only from what the boundary can change)."""
    from tests.oracle_pool import oracle_batch
    from tests.parity import compare
    t = time.perf_counter()
    ref = oracle_batch(wl)
    errs, stats = compare(got, ref, wl.optin_rows)
    return {"rows": stats["rows"], "rows_with_errors": len(errs), "errors": errs[:5],
            "race_flagged": stats["race_flagged"], "top_p_flagged": stats["top_p_flagged"],
            "min_p_flagged": stats["min_p_flagged"], "support_exempt": stats["support_exempt"],
            "overflow": stats["overflow"], "max_logprob_err": stats["max_lp_err"],
            "oracle_s": time.perf_counter() - t}


def copy_calibration(dev, nbytes: int, reps: int = 5) -> None:
    """A plain streaming kernel of known traffic for scaling the HBM counters: torch.neg over a
    bfloat16 buffer reads nbytes and writes nbytes once per launch."""
    import torch
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


# How the counter CSVs that --ingest-pmc reads are made (run from /tmp with TMPDIR=/tmp; R is the
# repository root, OUT a directory for the counter files).
def pmc_commands(index: int, kernel: str) -> list:
    """The commands that produce a counter summary (run from /tmp; R the repository root, OUT the
    directory the counter files go to)."""
    run = f'python3 "$R/bench.py" --workload {index} --kernel {kernel} --no-cpu-baseline --steps 20 --warmup 2 --copy-calibration'
    return [
        f'timeout -s KILL 180 rocprofv3 --pmc FETCH_SIZE --output-format csv -d "$OUT/fetch" -o fetch -- {run}',
        f'timeout -s KILL 180 rocprofv3 --pmc WRITE_SIZE --output-format csv -d "$OUT/write" -o write -- {run}',
        f'python3 bench.py --workload {index} --kernel {kernel} --ingest-pmc "$OUT/fetch/fetch_counter_collection.csv" '
        '"$OUT/write/write_counter_collection.csv" <JSON line of a bench run of the same kernel>',
    ]


def ingest_pmc(fetch_csv: str, write_csv: str, alg_bytes: int, copy_bytes: int,
               kernel: str = "sample") -> dict:
    """Per-launch HBM traffic of the sampler (or replay) kernel from two rocprofv3 --pmc counter
    CSVs (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled by what the same counter
    reads for the copy calibration kernel of known size."""
    kname = TRAFFIC_KERNELS[kernel][0]
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                key = (row["Kernel_Name"], row.get("Dispatch_Id", row.get("Correlation_Id")))
                vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
        out = {}
        for (name, _), v in vals.items():
            out.setdefault(name, []).append(v)
        return out

    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        k = per_kernel(path, counter)
        samp = [v for n, v in k.items() if kname in n]
        copy = [v for n, v in k.items() if "neg_kernel" in n]
        if not samp or not copy:
            raise SystemExit(f"{path}: no {kname} or calibration dispatches for {counter}")
        s_kib = statistics.median([x for v in samp for x in v])
        c_kib = statistics.median([x for v in copy for x in v])
        factor = copy_bytes / (c_kib * 1024.0)
        res[counter] = {"kernel_kib_median": s_kib, "copy_kib_median": c_kib,
                        "copy_known_bytes": copy_bytes, "scale": factor,
                        "kernel_bytes_scaled": s_kib * 1024.0 * factor,
                        "kernel_dispatches": sum(len(v) for v in samp)}
    total = res["FETCH_SIZE"]["kernel_bytes_scaled"] + res["WRITE_SIZE"]["kernel_bytes_scaled"]
    return {"counters": res, "hbm_bytes_per_launch": total,
            "algorithmic_bytes_per_launch": alg_bytes, "ratio_to_algorithmic": total / alg_bytes,
            "kernel_source_hash": kernel_source_hash()}


def param_summary(v):
    """A per-row parameter for the config record: its value when every row shares it, else its
    range."""
    import numpy as np
    v = np.asarray(v)
    one = lambda x: float(f"{x:.6g}") if isinstance(x, float) else x
    if np.all(v == v[0]):
        return one(v[0].item())
    return f"per row, {v.min().item():.4g}..{v.max().item():.4g}"


def replay_cpu_baseline(x_new, dtype, T, ids, lengths, tokens, budget_s: float = 10.0) -> dict:
    """The replay oracle (as it stands) on a bounded sample: rows in order, cycling."""
    import oracle
    decoded = {}
    rows, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        j = rows % len(tokens)
        if j not in decoded:
            decoded[j] = oracle.decode_logits(x_new[j], dtype)
        oracle.replay_row(decoded[j], T[j], ids[j, :lengths[j]], int(tokens[j]))
        rows += 1
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} rows (the captured rows of the batch, cycled) through "
                      f"oracle.replay_row in one process and one thread, {dt:.1f} s; decoding "
                      f"done once per row outside the clock"}


def bench_replay(args, wl) -> int:
    """Replay of the workload's captured supports on new logits (see the module docstring)."""
    import numpy as np
    import torch
    import top_support_capture_amd as tsc
    from tests.gpu_helpers import device_inputs, logits_tensor
    from workloads import perturbed_logits
    dev = torch.device("cuda:0")
    d = device_inputs(wl)
    cap = tsc.sample_with_mask(d["logits"], d["temperature"], d["top_k"], d["top_p"], d["min_p"],
                               d["optin_rows"], d["seeds"], d["positions"], wl.W,
                               return_logprobs=False, return_bits=True)
    torch.cuda.synchronize()
    rows = d["optin_rows"].long()
    N = rows.numel()
    x_new_host = perturbed_logits(wl.logits[wl.optin_rows], wl.dtype, seed=12345)
    esize = 2 if wl.dtype == "bf16" else 4
    in_bytes = N * wl.V * esize
    ncopies = max(1, -(-512 * 2**20 // in_bytes) + 1)
    x0 = logits_tensor(x_new_host, wl.dtype)
    copies = [x0] + [x0.clone() for _ in range(ncopies - 1)]
    T = d["temperature"][rows].contiguous()
    T = torch.where(T > 0, T, torch.ones_like(T))
    tokens = cap.tokens[rows].contiguous()
    status = cap.row_status[rows].contiguous()
    stream = torch.cuda.current_stream(dev)

    # One validated call through the binding, then the same library call with cached pointers,
    # so that the timed loop measures the kernel rather than Python.
    out = tsc.replay_logprob(copies[0], T, cap.packed_ids, cap.lengths, tokens, status,
                             cap.support_bits, return_logprobs=True, stream=stream)
    lib = tsc.library()
    dt = 1 if wl.dtype == "bf16" else 0
    W = cap.packed_ids.shape[1]
    tail = (dt, N, wl.V, wl.V, T.data_ptr(), cap.packed_ids.data_ptr(), cap.lengths.data_ptr(), W,
            status.data_ptr(), cap.support_bits.data_ptr(), cap.support_bits.shape[1],
            tokens.data_ptr(), out.selected_logprob.data_ptr())
    tail_end = (out.row_status.data_ptr(), stream.cuda_stream)

    def step(i, lp=False):
        assert lib.tsc_replay_logprob(copies[i % ncopies].data_ptr(), *tail,
                                      out.logprobs.data_ptr() if lp else None, *tail_end) == 0

    def timed(lp, steps):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            step(i, lp)
        ev1.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, ev0.elapsed_time(ev1) / steps

    # A counter run (--copy-calibration) times the selected-logprob mode alone, the mode the
    # roofline is quoted for, so that the counters cover that mode only.
    modes = (False,) if args.copy_calibration else (False, True)
    for i in range(args.warmup):
        step(i, modes[i % len(modes)])
    # The two modes (selected logprob only; with support logprobs) alternate in blocks, so that
    # clock and thermal drift fall on both alike; each mode's time is the median over its blocks.
    nblk = 10
    per = max(1, args.steps // nblk)
    blocks = {False: [], True: []}
    for _ in range(nblk):
        for lp in modes:
            blocks[lp].append(timed(lp, per))
    if args.copy_calibration:
        copy_calibration(dev, wl.B * wl.V * esize)
        blocks[True] = blocks[False]
    wall = sum(w for w, _ in blocks[False])
    avg_ms = float(np.median([m for _, m in blocks[False]]))
    avg_ms_lp = float(np.median([m for _, m in blocks[True]]))
    lengths = cap.lengths.cpu().numpy().astype(np.int64)
    st = status.cpu().numpy()
    packed = lengths[st == 0]
    nbits = int((st == 1).sum())
    members = cap.support_bits.cpu().numpy() if nbits else None
    bit_members = 0 if not nbits else int(sum(
        np.unpackbits(members[j], bitorder="little")[:wl.V].sum() for j in np.nonzero(st == 1)[0]))
    # Algorithmic bytes: packed rows read their ids and gather their logits; bitmask rows read
    # ceil(V / 8) mask bytes and gather their members; every row reads length, token and
    # temperature and writes its logprob and status.
    alg = int(packed.sum()) * (4 + esize) + nbits * ((wl.V + 7) // 8) + bit_members * esize + N * 17
    alg_lp = alg + int(lengths[st <= 1].sum()) * 4
    achieved = alg / (avg_ms * 1e-3) / 1e9
    rs = out.row_status.cpu().numpy()
    line = {
        "metric": "replayed rows/s and achieved GB/s (% of HBM peak), replay of captured supports",
        "value": N * nblk * per / wall, "unit": "rows/s", "n_gpus": 1, "steps": nblk * per,
        "warmup": args.warmup, "ms_per_step": wall / (nblk * per) * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (the workload's captures replayed on its logits plus seeded noise)",
        "config": {"workload": f"replay of {wl.name}", "N": N, "V": wl.V, "W": wl.W,
                   "rows_from_bitmask": nbits, "mean_support": float(lengths.mean()),
                   "outputs": "selected logprob"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": measured_traffic(wl, "replay")},
        "kernel_ms": {"mean": avg_ms, "with_support_logprobs": avg_ms_lp,
                      "timing": f"median over {nblk} blocks of {per} calls per mode, the two "
                                f"modes alternating block by block"},
        "algorithmic_bytes_per_launch": alg,
        "algorithmic_bytes_with_support_logprobs": alg_lp,
        "rows_not_ok": int(np.count_nonzero(rs != 0)),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        ids = cap.packed_ids.cpu().numpy()
        ok = np.nonzero(st == 0)[0]
        line["cpu_baseline"] = replay_cpu_baseline(
            x_new_host[ok], wl.dtype, T.cpu().numpy()[ok], ids[ok], lengths[ok],
            tokens.cpu().numpy()[ok])
    print(json.dumps(line), flush=True)
    return 0


def bench_csr(args, wl) -> int:
    """The support CSR of a sampler call's capture (see the module docstring)."""
    import numpy as np
    import torch
    import top_support_capture_amd as tsc
    from tests.gpu_helpers import device_inputs
    dev = torch.device("cuda:0")
    d = device_inputs(wl)
    cap = tsc.sample_with_mask(d["logits"], d["temperature"], d["top_k"], d["top_p"], d["min_p"],
                               d["optin_rows"], d["seeds"], d["positions"], wl.W)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    R, W = cap.packed_ids.shape
    csr = tsc.support_csr(cap, stream=stream)
    lib = tsc.library()
    args_c = (cap.lengths.data_ptr(), cap.packed_ids.data_ptr(), cap.logprobs.data_ptr(), R, W,
              csr.offsets.data_ptr(), csr.ids.data_ptr(), csr.logprobs.data_ptr(), R * W,
              stream.cuda_stream)

    def step():
        assert lib.tsc_support_csr(*args_c) == 0

    for _ in range(args.warmup):
        step()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms = ev0.elapsed_time(ev1) / args.steps
    total = int(csr.offsets[-1].item())
    alg = R * 4 + total * 8 + (R + 1) * 8 + total * 8

    # Host copies: the packed buffers whole, against the offsets then the realized payload.
    host_ids = torch.empty(R * W, dtype=torch.int32, pin_memory=True)
    host_lps = torch.empty(R * W, dtype=torch.float32, pin_memory=True)
    host_off = torch.empty(R + 1, dtype=torch.int64, pin_memory=True)

    def copy_ms(fn, reps=50):
        fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / reps * 1e3

    def packed_copy():
        host_ids.copy_(cap.packed_ids.view(-1), non_blocking=True)
        host_lps.copy_(cap.logprobs.view(-1), non_blocking=True)

    def csr_copy():
        host_off.copy_(csr.offsets, non_blocking=True)
        torch.cuda.synchronize()
        n = int(host_off[-1])
        host_ids[:n].copy_(csr.ids[:n], non_blocking=True)
        host_lps[:n].copy_(csr.logprobs[:n], non_blocking=True)

    line = {
        "metric": "support CSR: kernel time and host-copy bytes, realized support vs capacity",
        "value": alg / (avg_ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32+f32",
        "data": f"synthetic (a sampler call's capture of {wl.name})",
        "config": {"workload": f"CSR of the capture of {wl.name}", "R": R, "W": W,
                   "entries": total},
        "roofline": {"bound": "hbm", "achieved": alg / (avg_ms * 1e-3) / 1e9,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": alg / (avg_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, "traffic": None},
        "kernel_ms": {"mean": avg_ms},
        "algorithmic_bytes_per_launch": alg,
        "host_copy": {"packed_bytes": R * W * 8, "csr_bytes": total * 8 + (R + 1) * 8,
                      "packed_ms": copy_ms(packed_copy), "csr_ms_incl_offsets_sync": copy_ms(csr_copy)},
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    # About 45 ms of untimed calls: long enough for the GPU clocks to reach their sustained level
    # (20 warmup calls leave the timed region ~6% slower than the steady state).
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel", choices=["sample", "replay", "csr"], default="sample",
                    help="time the sampler (default), the replay of its captures or their CSR")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run the known-size copy kernel that scales the HBM counters")
    ap.add_argument("--ingest-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "BENCH_LINE"),
                    help="write the traffic summary from two rocprofv3 --pmc counter CSVs and "
                         "the JSON line of a bench run of the same kernel")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: rows are independent, so the sampler shards by "
              "rows with no communication; run it with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    from workloads import make_workload
    if not args.ingest_pmc:
        import torch
        import top_support_capture_amd as tsc
        from tests.gpu_helpers import device_inputs

    wl = make_workload(args.workload)
    in_bytes = wl.B * wl.V * (2 if wl.dtype == "bf16" else 4)
    if args.ingest_pmc:
        if args.kernel not in TRAFFIC_KERNELS:
            raise SystemExit(f"no counter summary for --kernel {args.kernel}")
        with open(args.ingest_pmc[2]) as f:  # the last JSON line (a profiler may print after it)
            bench_line = json.loads([l for l in f.read().splitlines() if l.startswith("{")][-1])
        alg = int(bench_line["algorithmic_bytes_per_launch"])
        wname = wl.name if args.kernel == "sample" else f"{args.kernel} of {wl.name}"
        if bench_line["config"].get("workload") != wname:
            raise SystemExit(f"the bench line is of {bench_line['config'].get('workload')}, "
                             f"not of {wname}")
        t = {"workload": wl.name, "kernel": args.kernel,
             "commands": pmc_commands(args.workload, args.kernel),
             **ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], alg, in_bytes, args.kernel)}
        path = traffic_path(wl, args.kernel)
        with open(path, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return 0
    if args.kernel == "replay":
        return bench_replay(args, wl)
    if args.kernel == "csr":
        return bench_csr(args, wl)
    dev = torch.device("cuda:0")
    d = device_inputs(wl)
    ncopies = max(1, -(-512 * 2**20 // in_bytes) + 1)
    copies = [d["logits"]] + [d["logits"].clone() for _ in range(ncopies - 1)]
    stream = torch.cuda.current_stream(dev)
    call = tsc.prepare(copies[0], d["temperature"], d["top_k"], d["top_p"], d["min_p"],
                       d["optin_rows"], d["seeds"], d["positions"], wl.W, stream=stream)
    out = call.out

    def step(i):
        call(copies[i % ncopies], check=False)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Timed region: K back-to-back steps between device synchronizations (wall clock), bracketed
    # by two HIP events on the launch stream: their elapsed time over K is the kernel's average
    # launch duration (consecutive launches overlap their dispatch with the previous kernel's
    # tail, as in any stream of calls).
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms = ev0.elapsed_time(ev1) / args.steps
    # Outside the timed region: events around single calls, for the spread of one launch's
    # duration (each includes the dispatch of that call alone).
    nsolo = min(args.steps, 50)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nsolo)]
    for i in range(nsolo):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    durs_ms = np.array([a.elapsed_time(b) for a, b in evs])
    # Library references on the same rotating copies, timed the same way, for context: a plain
    # one-pass row maximum (torch.amax; it reads the bytes the sampler must read and does nothing
    # else) and a device copy of the logits (torch copy_, which reads and writes them once: its
    # rate is the streaming bandwidth this machine reaches).
    refs = None
    if not args.copy_calibration:
        amax_out = torch.empty(wl.B, dtype=copies[0].dtype, device=dev)
        dst = torch.empty_like(copies[0])

        def ref_ms(fn, reps=500):
            for i in range(200):
                fn(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(reps):
                fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        amax_ms = ref_ms(lambda i: torch.amax(copies[i % ncopies], dim=1, out=amax_out))
        copy_ms = ref_ms(lambda i: dst.copy_(copies[i % ncopies]))
        refs = {"torch.amax rows": {"ms": amax_ms, "read GB/s": in_bytes / (amax_ms * 1e-3) / 1e9},
                "torch copy_": {"ms": copy_ms,
                                "read+write GB/s": 2 * in_bytes / (copy_ms * 1e-3) / 1e9}}
    if args.copy_calibration:
        copy_calibration(dev, in_bytes)

    lengths = out.lengths.cpu().numpy().astype(np.int64)
    status = out.row_status.cpu().numpy()
    alg_bytes = in_bytes + int(np.minimum(lengths, wl.W).sum()) * 8 + wl.R * 8 + wl.B * 5
    avg_s = avg_ms * 1e-3
    achieved = alg_bytes / avg_s / 1e9
    traffic = measured_traffic(wl)
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
        "dtype": wl.dtype,
        "data": ("synthetic (seeded Gaussian logits on a 0.125 grid, cast to bfloat16)"
                 if args.workload == 3 else f"synthetic (seeded workload {wl.name})"),
        "config": {"workload": wl.name, "B": wl.B, "V": wl.V, "logits": wl.dtype,
                   "top_k": param_summary(wl.top_k), "top_p": param_summary(wl.top_p),
                   "min_p": param_summary(wl.min_p),
                   "temperature": param_summary(wl.temperature), "R": wl.R, "W": wl.W,
                   "input_copies_rotated": ncopies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic},
        "kernel_ms": {"mean": avg_ms, "single_call_p10": float(np.percentile(durs_ms, 10)),
                      "single_call_p50": float(np.median(durs_ms)),
                      "single_call_p90": float(np.percentile(durs_ms, 90))},
        "algorithmic_bytes_per_launch": alg_bytes,
        "library_references": refs,
        "rows_overflow": int(np.count_nonzero(status == 1)),
        "rows_not_ok": int(np.count_nonzero(status >= 2)),
        "mean_support": float(lengths.mean()),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        from tests.parity import to_numpy_outputs
        line["oracle_check"] = oracle_check(wl, to_numpy_outputs(out))
        line["cpu_baseline"] = cpu_baseline(wl, args.workload)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
