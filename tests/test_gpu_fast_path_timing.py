"""Every row of the benchmark batches stays on a single-read path (needs an MI355X).

Which path serves a row is invisible in its results: a row the single-read paths cannot decide
exactly runs the general multi-pass path and returns the same outputs, only more slowly (a few
hundred microseconds on one CU for these vocabularies). A cutoff that came out above the k-th
value, or a capacity that stopped fitting these rows, would therefore pass every parity test.
The launch time shows it: the bounds below are about three times the measured times of these
batches and far below a batch with even one general-path row.

Every case prints its name before touching the GPU, so a fault names the case that caused it.
"""
import pytest
import torch

from tests.gpu_helpers import device_inputs, log
from workloads import make_workload

pytestmark = pytest.mark.gpu

# (workload, bound in microseconds): measured 16, 21, 33, 109 and 119 us.
CASES = [(2, 60.0), (3, 70.0), (4, 100.0), (5, 300.0), (6, 300.0)]


@pytest.mark.parametrize("index,bound_us", CASES)
def test_batch_time_has_no_general_path_row(index, bound_us):
    import top_support_capture_amd as tsc
    wl = make_workload(index)
    log(f"case launch time workload {index} {wl.name}: bound {bound_us} us")
    d = device_inputs(wl)
    stream = torch.cuda.current_stream()
    call = tsc.prepare(d["logits"], d["temperature"], d["top_k"], d["top_p"], d["min_p"],
                       d["optin_rows"], d["seeds"], d["positions"], wl.W, stream=stream)
    for _ in range(20):
        call(d["logits"], check=False)
    torch.cuda.synchronize()
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(20):
            call(d["logits"], check=False)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / 20 * 1000.0)
    t = sorted(times)[len(times) // 2]
    log(f"  median {t:.1f} us per launch")
    assert t < bound_us, f"{wl.name}: {t:.1f} us per launch, bound {bound_us} us"
