"""Debug poison (needs an MI355X): with tsc_set_debug_poison on, packed slots past each length
hold id -1 and logprob NaN while every other output equals an unpoisoned call's, and the
library's own readers of a capture (support CSR, replay) return the same results from the
poisoned buffers: they never read past a length.

Every case prints its name before touching the GPU, so a fault names the case that caused it.
"""
import numpy as np
import pytest

from tests.gpu_helpers import log, run_gpu
from tests.test_gpu_csr import run_csr
from tests.test_gpu_replay import run_replay
from workloads import make_workload, perturbed_logits

pytestmark = pytest.mark.gpu


def _same(a, b):
    np.testing.assert_array_equal(np.asarray(a), np.asarray(b))


@pytest.mark.parametrize("index,W", [(3, 2048), (2, 64), (5, 64)])
def test_poisoned_capture_and_its_readers(index, W):
    import top_support_capture_amd as tsc
    wl = make_workload(index, W=W)
    log(f"case debug poison: workload {index} W={W}")
    clean = run_gpu(wl)
    prev = tsc.set_debug_poison(True)
    try:
        poisoned = run_gpu(wl)
    finally:
        tsc.set_debug_poison(prev)

    # The capture: entries up to each length and every other output unchanged, the rest poisoned.
    L = clean["lengths"]
    for key in ("tokens", "row_status", "lengths", "selected_logprob"):
        _same(poisoned[key], clean[key])
    past = np.arange(W)[None, :] >= np.clip(L, 0, W)[:, None]
    assert past.any(), "no slot shorter than W: nothing was poisoned"
    assert (poisoned["packed_ids"][past] == -1).all()
    assert np.isnan(poisoned["logprobs"][past]).all()
    _same(poisoned["packed_ids"][~past], clean["packed_ids"][~past])
    _same(poisoned["logprobs"][~past], clean["logprobs"][~past])
    log(f"  {int(past.sum())} poisoned entries in {int(past.any(1).sum())} of {len(L)} slots")

    # Support CSR of both captures.
    c0 = run_csr(L, clean["packed_ids"], clean["logprobs"])
    c1 = run_csr(L, poisoned["packed_ids"], poisoned["logprobs"])
    n = int(c0[0][-1])
    _same(c1[0], c0[0])
    _same(c1[1][:n], c0[1][:n])
    _same(c1[2][:n], c0[2][:n])

    # Replay of both captures on perturbed logits (overflowed slots have no bitmask here, so
    # both report them invalid alike).
    opt = wl.optin_rows
    x_new = perturbed_logits(wl.logits[opt], wl.dtype, seed=300 + index)
    T = wl.temperature[opt].copy()
    T[T == 0] = 1.0
    tok = clean["tokens"][opt]
    cs = clean["row_status"][opt]
    r0 = run_replay(x_new, wl.dtype, T, clean["packed_ids"], L, tok, cs)
    r1 = run_replay(x_new, wl.dtype, T, poisoned["packed_ids"], L, tok, cs)
    _same(r1[0], r0[0])
    _same(r1[2], r0[2])
    _same(r1[1][~past], r0[1][~past])
