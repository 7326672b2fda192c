"""Host logic of bench.py (no GPU): the one-GPU guard, the config record, the HBM-counter
ingestion and the kernel source hash."""
import csv
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_param_summary():
    assert bench.param_summary(np.full(4, 1024, np.int32)) == 1024
    assert bench.param_summary(np.full(3, 0.95, np.float32)) == 0.95
    assert bench.param_summary(np.array([0.5, 1.5, 1.0], np.float32)) == "per row, 0.5..1.5"


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_ingest_pmc_scales_by_the_copy_kernel(tmp_path):
    # The copy of 1 MiB reads half its bytes on FETCH_SIZE (scale 2) and all on WRITE_SIZE.
    copy_bytes = 2**20
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    samp = "void tsc::sample_fast_kernel<1, false>(tsc::SampleArgs)"
    neg = "void at::native::neg_kernel_cuda(...)"
    _counter_csv(fetch, "FETCH_SIZE", [(samp, 600.0), (samp, 600.0), (neg, 512.0)])
    _counter_csv(write, "WRITE_SIZE", [(samp, 10.0), (neg, 1024.0)])
    t = bench.ingest_pmc(str(fetch), str(write), alg_bytes=1_200_000, copy_bytes=copy_bytes)
    f, w = t["counters"]["FETCH_SIZE"], t["counters"]["WRITE_SIZE"]
    assert f["scale"] == 2.0 and w["scale"] == 1.0
    assert f["kernel_bytes_scaled"] == 600.0 * 1024 * 2
    assert w["kernel_bytes_scaled"] == 10.0 * 1024
    assert t["hbm_bytes_per_launch"] == 600.0 * 1024 * 2 + 10.0 * 1024
    assert t["kernel_source_hash"] == bench.kernel_source_hash()


def test_ingest_pmc_of_the_replay_counts_replay_dispatches_only(tmp_path):
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    samp = "void tsc::sample_fast_kernel<1, false>(tsc::SampleArgs)"
    rep = "void tsc::replay_kernel<1, false>(tsc::ReplayArgs)"
    neg = "void at::native::neg_kernel_cuda(...)"
    _counter_csv(fetch, "FETCH_SIZE", [(samp, 9000.0), (rep, 100.0), (rep, 100.0), (neg, 512.0)])
    _counter_csv(write, "WRITE_SIZE", [(samp, 90.0), (rep, 1.0), (neg, 1024.0)])
    t = bench.ingest_pmc(str(fetch), str(write), alg_bytes=200_000, copy_bytes=2**20,
                         kernel="replay")
    assert t["counters"]["FETCH_SIZE"]["kernel_dispatches"] == 2
    assert t["hbm_bytes_per_launch"] == 100.0 * 1024 * 2 + 1.0 * 1024
    import types
    wl = types.SimpleNamespace(B=256, V=151936, dtype="bf16", name="w")
    assert bench.traffic_path(wl, "replay") != bench.traffic_path(wl)


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()


def test_traffic_summary_is_keyed_by_workload_and_sources(tmp_path, monkeypatch):
    # A counter summary counts only for the workload it was taken on, and only while the kernel
    # sources hash to what it records.
    import json
    import types
    h = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: h)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    wl = types.SimpleNamespace(B=256, V=151936, dtype="bf16", name="b256_v151936_bf16_grid")
    other = types.SimpleNamespace(B=256, V=151936, dtype="bf16", name="another")
    assert bench.measured_traffic(wl) is None  # no summary
    with open(bench.traffic_path(wl), "w") as f:
        json.dump({"workload": wl.name, "kernel_source_hash": h, "hbm_bytes_per_launch": 123.0}, f)
    assert bench.measured_traffic(wl) == 123.0
    assert bench.measured_traffic(other) is None
    with open(bench.traffic_path(wl), "w") as f:
        json.dump({"workload": wl.name, "kernel_source_hash": "0" * 16,
                   "hbm_bytes_per_launch": 123.0}, f)
    assert bench.measured_traffic(wl) is None


def test_cpu_model_is_named():
    import bench
    assert bench.cpu_model().strip() not in ("", "unknown CPU")


def test_oracle_check_counts_the_boundary_reports():
    # The oracle's own outputs for workload 1 pass the bench's check; a wrong token is counted.
    import numpy as np
    import oracle
    import bench
    from workloads import make_workload
    wl = make_workload(1)
    ref = oracle.sample_with_mask(wl.logits, wl.dtype, wl.temperature, wl.top_k, wl.top_p,
                                  wl.min_p, wl.optin_rows, wl.seeds, wl.positions, wl.W)
    got = {"tokens": ref.tokens.copy(), "row_status": ref.row_status.copy(),
           "packed_ids": ref.packed_ids.copy(), "lengths": ref.lengths.copy(),
           "logprobs": ref.logprobs.copy(), "selected_logprob": ref.selected_logprob.copy()}
    chk = bench.oracle_check(wl, got)
    assert chk["rows"] == wl.B and chk["rows_with_errors"] == 0
    for key in ("race_flagged", "top_p_flagged", "min_p_flagged", "overflow"):
        assert chk[key] >= 0
    got["tokens"][0] = (got["tokens"][0] + 1) % wl.V
    assert bench.oracle_check(wl, got)["rows_with_errors"] >= 1
