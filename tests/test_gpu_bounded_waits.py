"""The waits between the waves of a row's workgroup are bounded (needs an MI355X).

The host sets a wait limit of one sleep, so that waits which are not satisfied at once give up:
every kernel must still finish, every row must come back either exactly as the oracle says or
with the ABORTED status (token -1, length 0, NaN selected logprob), and the next call with the
default limit must match the oracle again. Nothing here faults or hangs the GPU: the condition is
the kernel's own bounded wait, forced from the host.
"""
import numpy as np
import pytest

from tests.gpu_helpers import log, run_gpu
from tests.oracle_pool import oracle_batch
from tests.parity import compare
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("index,W", [(3, None), (4, 8192)])
def test_waits_give_up_with_aborted_rows_and_recover(index, W):
    import top_support_capture_amd as tsc
    wl = make_workload(index, W=W) if W is not None else make_workload(index)
    ref = oracle_batch(wl)
    log(f"case bounded waits workload {index} W={wl.W}: limit 1")
    prev = tsc.set_wait_limit(1)
    try:
        got = run_gpu(wl, bits=True)
    finally:
        tsc.set_wait_limit(prev)
    st = got["row_status"]
    aborted = st == tsc.ROW_ABORTED
    log(f"  {int(aborted.sum())} of {wl.B} rows aborted")
    assert aborted.any()
    assert np.all(got["tokens"][aborted] == -1)
    slot_of = {int(r): j for j, r in enumerate(wl.optin_rows)}
    for r in np.nonzero(aborted)[0]:
        j = slot_of[int(r)]
        assert got["lengths"][j] == 0 and np.isnan(got["selected_logprob"][j])
    done = np.nonzero(~aborted)[0]
    errs, _ = compare(got, ref, wl.optin_rows, rows=done)
    assert errs == [], errs[:10]
    log(f"case bounded waits workload {index}: default limit again")
    again = run_gpu(wl)
    errs, stats = compare(again, ref, wl.optin_rows)
    assert errs == [] and not np.any(again["row_status"] == tsc.ROW_ABORTED), errs[:10]
