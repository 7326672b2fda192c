"""The oracle over many rows in worker processes (test infrastructure).

Rows are independent, so they are sampled by ``oracle.sample_row`` in a pool of freshly started
interpreters (the spawn start method: a worker never inherits a parent's GPU state) and then
assembled by ``oracle.sample_with_mask`` exactly as if it had sampled them itself."""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

import oracle


def _rows_job(args):
    logits, dtype, T, k, p, mpv, seeds, pos, rows = args
    out = {}
    for i, r in enumerate(rows):
        out[int(r)] = oracle.sample_row(oracle.decode_logits(logits[i], dtype), T[i], k[i], p[i],
                                        mpv[i], int(seeds[i]), int(pos[i]))
    return out


def workers() -> int:
    # At most 16 workers, whatever os.cpu_count() reports: the host's CPUs are shared.
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_batch(wl, W=None, rows=None, bits_ld=None, nproc=None):
    """``oracle.sample_with_mask`` of a workload, its rows sampled in parallel."""
    rows = np.arange(wl.B) if rows is None else np.asarray(rows, np.int64)
    nproc = workers() if nproc is None else nproc
    parts = [p for p in np.array_split(rows, max(1, min(len(rows), 4 * nproc))) if p.size]
    jobs = [(wl.logits[p], wl.dtype, wl.temperature[p], wl.top_k[p], wl.top_p[p], wl.min_p[p],
             wl.seeds[p], wl.positions[p], p) for p in parts]
    results = {}
    with mp.get_context("spawn").Pool(nproc) as pool:
        for d in pool.imap_unordered(_rows_job, jobs):
            results.update(d)
    return oracle.sample_with_mask(wl.logits, wl.dtype, wl.temperature, wl.top_k, wl.top_p,
                                   wl.min_p, wl.optin_rows, wl.seeds, wl.positions,
                                   wl.W if W is None else W, rows=rows, bits_ld=bits_ld,
                                   row_results=results)
