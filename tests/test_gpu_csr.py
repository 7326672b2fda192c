"""Parity of the support CSR kernels (tsc_support_csr) with the CPU oracle (needs an MI355X).

Packed inputs are seeded synthetic arrays or the CPU oracle sampler's own capture, never the
library's output. Every case prints its name before touching the GPU."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import log
from workloads import make_workload

pytestmark = pytest.mark.gpu

SENTINEL = -77


def run_csr(lengths, packed, lps, cap=None):
    import top_support_capture_amd as tsc
    dev = "cuda:0"
    R, W = packed.shape
    cap = R * W if cap is None else cap
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)
    L, P = t(lengths, torch.int32), t(packed, torch.int32)
    LP = None if lps is None else t(lps, torch.float32)
    off = torch.full((R + 1,), SENTINEL, dtype=torch.int64, device=dev)
    ids = torch.full((max(cap, 1),), SENTINEL, dtype=torch.int32, device=dev)
    out_lp = torch.full((max(cap, 1),), float(SENTINEL), dtype=torch.float32, device=dev)
    lib = tsc.library()
    code = lib.tsc_support_csr(L.data_ptr(), P.data_ptr(), None if LP is None else LP.data_ptr(),
                               R, W, off.data_ptr(), ids.data_ptr(), out_lp.data_ptr(), cap,
                               torch.cuda.current_stream().cuda_stream)
    assert code == 0
    torch.cuda.synchronize()
    return off.cpu().numpy(), ids.cpu().numpy(), out_lp.cpu().numpy()


@pytest.mark.parametrize("R,W", [(0, 4), (1, 1), (7, 5), (256, 2048), (2048, 7), (2049, 7), (3000, 16),
                                 (5000, 3), (6, 8200), (3, 4097)])
def test_csr_synthetic(R, W):
    log(f"case csr synthetic R={R} W={W}")
    rng = np.random.default_rng(R * 31 + W)
    lengths = rng.integers(-2, W + 3, R).astype(np.int32)
    packed = rng.integers(0, 2**31 - 1, (R, W)).astype(np.int32)
    lps = rng.standard_normal((R, W)).astype(np.float32)
    off, ids, lp = run_csr(lengths, packed, lps)
    r_off, r_ids, r_lp = oracle.support_csr(lengths, packed, lps)
    assert np.array_equal(off, r_off)
    n = int(r_off[-1])
    assert np.array_equal(ids[:n], r_ids) and np.array_equal(lp[:n], r_lp)
    assert np.all(ids[n:] == SENTINEL)


def test_csr_capacity_and_selected_mode():
    log("case csr capacity bound, no logprobs")
    rng = np.random.default_rng(3)
    R, W = 40, 64
    lengths = rng.integers(0, W + 1, R).astype(np.int32)
    packed = rng.integers(0, 1000, (R, W)).astype(np.int32)
    r_off, r_ids, _ = oracle.support_csr(lengths, packed)
    cap = int(r_off[-1]) // 2
    off, ids, lp = run_csr(lengths, packed, None, cap=cap)
    assert np.array_equal(off, r_off)  # offsets are complete even when the payload is cut
    assert np.array_equal(ids[:cap], r_ids[:cap])
    assert np.all(lp == SENTINEL)       # no logprobs given: none written


def test_csr_long_slots_cut_by_capacity():
    # Slots on either side of the length from which the copy uses nontemporal stores, with the
    # capacity ending inside a long one.
    log("case csr long slots, capacity inside a long slot")
    rng = np.random.default_rng(11)
    R, W = 5, 6000
    lengths = np.array([6000, 4095, 4096, 0, 5000], np.int32)
    packed = rng.integers(0, 2**31 - 1, (R, W)).astype(np.int32)
    lps = rng.standard_normal((R, W)).astype(np.float32)
    r_off, r_ids, r_lp = oracle.support_csr(lengths, packed, lps)
    cap = int(r_off[3]) - 1000  # inside the third slot (4096 entries)
    off, ids, lp = run_csr(lengths, packed, lps, cap=cap)
    assert np.array_equal(off, r_off)
    assert np.array_equal(ids[:cap], r_ids[:cap]) and np.array_equal(lp[:cap], r_lp[:cap])


def test_csr_of_an_oracle_capture():
    wl = make_workload(3)
    log("case csr of the oracle capture of workload 3")
    ref = oracle.sample_with_mask(wl.logits, wl.dtype, wl.temperature, wl.top_k, wl.top_p,
                                  wl.min_p, wl.optin_rows, wl.seeds, wl.positions, wl.W)
    packed = np.where(ref.packed_ids < 0, 0, ref.packed_ids).astype(np.int32)
    lps = np.nan_to_num(ref.logprobs, nan=0.0)
    off, ids, lp = run_csr(ref.lengths, packed, lps)
    r_off, r_ids, r_lp = oracle.support_csr(ref.lengths, packed, lps)
    n = int(r_off[-1])
    assert n == int(ref.lengths.sum()) and np.array_equal(off, r_off)
    assert np.array_equal(ids[:n], r_ids) and np.array_equal(lp[:n], r_lp)


def test_csr_binding_round_trip():
    # The binding's host copy is sized by offsets[R] and equals the packed prefixes.
    import top_support_capture_amd as tsc
    from tests.gpu_helpers import device_inputs
    wl = make_workload(2)
    log("case csr binding round trip, workload 2")
    d = device_inputs(wl)
    out = tsc.sample_with_mask(d["logits"], d["temperature"], d["top_k"], d["top_p"], d["min_p"],
                               d["optin_rows"], d["seeds"], d["positions"], wl.W)
    off, ids, lps = tsc.csr_to_host(tsc.support_csr(out))
    L = out.lengths.cpu().numpy()
    P = out.packed_ids.cpu().numpy()
    LP = out.logprobs.cpu().numpy()
    assert off[-1] == L.sum() and ids.size == L.sum()
    for j in range(len(L)):
        assert np.array_equal(ids[off[j]:off[j + 1]], P[j, :L[j]])
        assert np.array_equal(lps[off[j]:off[j + 1]], LP[j, :L[j]])
