"""The CPU oracle against its pins (no GPU): the pages' worked tie example, an exhaustive
per-token brute force on tiny vocabularies, library special cases, Philox against numpy, the
race distribution and output invariants; plus mutation checks showing the pins catch plausible
oracle mistakes."""
import inspect
import math

import numpy as np
import pytest

import oracle
from oracle import philox as ophilox
from oracle import sampler as osampler
from tests import oracle_pins as pins
from tests.invariants import check_invariants
from workloads import make_workload


def test_tie_example_from_the_pages():
    assert pins.pin_tie_example(oracle.sample_row) == []


def test_brute_force_enumeration():
    assert pins.pin_brute_force(oracle.sample_row) == []


def test_library_special_cases():
    assert pins.pin_special_cases(oracle.sample_row) == []


def test_support_bitmask():
    assert pins.pin_support_bitmask(oracle.support_bitmask, oracle.sample_row) == []


def test_support_bitmask_pin_catches_planted_mistakes():
    src = inspect.getsource(osampler.support_bitmask)
    for old, new in (('bitorder="little"', 'bitorder="big"'),
                     ("keep[np.asarray(support, dtype=np.int64)] = True",
                      "keep[np.asarray(support, dtype=np.int64)[:-1]] = True")):
        assert src.count(old) == 1
        ns = dict(vars(osampler))
        exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
        assert pins.pin_support_bitmask(ns["support_bitmask"], oracle.sample_row), old


def test_replay():
    assert pins.pin_replay(oracle.replay_row, oracle.sample_row) == []


@pytest.mark.parametrize("old,new", [
    ("z = (xs - m) / T", "z = (xs - m)"),
    ("lse = np.log(np.sum(np.exp((x[np.unique(support)] - m) / T)))",
     "lse = np.log(np.sum(np.exp((x[np.isfinite(x)] - m) / T)))"),
    ("sel = (x[token] - m) / T - lse", "sel = (x[token] - m) / T + lse"),
    ("sel = -np.inf", "sel = (x[token] - m) / T - lse"),
])
def test_replay_pin_catches_planted_mistakes(old, new):
    import importlib
    oreplay = importlib.import_module("oracle.replay")
    src = inspect.getsource(oreplay.replay_row)
    assert src.count(old) == 1
    ns = dict(vars(oreplay))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    assert pins.pin_replay(ns["replay_row"], oracle.sample_row, cases=60), old


def test_replay_support_is_a_set():
    # R14: an id listed twice counts once in the normalizer.
    x = np.log(np.array([0.4, 0.2, 0.2, 0.1, 0.1]))
    r = oracle.replay_row(x, 1.0, np.array([0, 1, 1, 2]), 0)
    assert abs(r.selected_logprob - math.log(0.5)) < 1e-12
    assert np.allclose(r.logprobs, np.log([0.5, 0.25, 0.25, 0.25]), atol=1e-12)


def test_replay_batch_statuses():
    # Packed rows, an OVERFLOW row read from its bitmask, and the status rows.
    x = np.log(np.array([[0.4, 0.2, 0.2, 0.1, 0.1]] * 6, np.float32))
    x[3, 1] = np.nan
    ids = np.array([[0, 1, 2, 0], [0, 1, 2, 0], [0, 1, 0, 0], [0, 1, 2, 0], [0, 1, 2, 0],
                    [0, 1, 2, 0]], np.int32)
    lengths = np.array([3, 3, 2, 3, 0, 3], np.int32)
    cs = np.array([0, 0, 1, 0, 0, 3], np.int8)
    bits = np.zeros((6, 16), np.uint8)
    bits[2, 0] = 0b00111  # the full support {0, 1, 2} of the overflowing row
    T = np.array([1, 1, 1, 1, 1, 1], np.float32)
    tokens = np.array([0, 4, 1, 0, 0, 0], np.int32)
    sel, lps, st = oracle.replay(x, "f32", T, ids, lengths, tokens, cs, bits)
    assert st.tolist() == [0, 0, 0, 3, 4, 3]
    assert abs(sel[0] - math.log(0.5)) < 1e-6 and sel[1] == -np.inf
    assert abs(sel[2] - math.log(0.25)) < 1e-6
    assert np.allclose(lps[2, :2], [math.log(0.5), math.log(0.25)], atol=1e-6)
    assert np.isnan(sel[3:]).all()


def test_support_csr():
    assert pins.pin_support_csr(oracle.support_csr) == []


@pytest.mark.parametrize("old,new", [
    ("offsets[1:] = np.cumsum(n)", "offsets[1:] = np.cumsum(n) - n"),
    ("n = np.clip(np.asarray(lengths, dtype=np.int64), 0, W)", "n = np.asarray(lengths, dtype=np.int64)"),
    ("packed_ids[j, :n[j]] for j in range(R)", "packed_ids[j, 1:n[j] + 1] for j in range(R)"),
])
def test_support_csr_pin_catches_planted_mistakes(old, new):
    import importlib
    ocsr = importlib.import_module("oracle.csr")
    src = inspect.getsource(ocsr.support_csr)
    assert src.count(old) == 1
    ns = dict(vars(ocsr))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    try:
        fails = pins.pin_support_csr(ns["support_csr"])
    except Exception as e:  # a broken layout may also raise
        fails = [repr(e)]
    assert fails, old


def test_race_distribution():
    assert pins.pin_race_distribution(oracle.sample_row) == []


def test_philox_4x64_instance_matches_numpy():
    # numpy's Philox is Philox4x64-10; it increments the 256-bit counter before each block, so
    # the block it returns for state counter c is the bijection applied to c + 1.
    rng = np.random.default_rng(5)
    for _ in range(20):
        key = rng.integers(0, 2**63, 2, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
        ctr = rng.integers(0, 2**63, 4, dtype=np.uint64)
        ctr[0] = np.uint64(ctr[0] & np.uint64(0xFFFFFFFF))  # no carry out of word 0
        bg = np.random.Philox(key=key, counter=ctr)
        got = bg.random_raw(4)
        nxt = ctr.copy()
        nxt[0] += np.uint64(1)
        mine = ophilox.philox4(tuple(int(c) for c in nxt), tuple(int(k) for k in key), w=64)
        assert [int(v) for v in mine] == [int(v) for v in got]


def test_philox_4x64_pin_detects_a_wrong_constant(monkeypatch):
    bad = dict(ophilox.PARAMS)
    M0, M1, W0, W1 = bad[64]
    bad[64] = (M0, M1, W0 ^ 2, W1)
    monkeypatch.setattr(ophilox, "PARAMS", bad)
    bg = np.random.Philox(key=np.array([3, 4], np.uint64), counter=np.zeros(4, np.uint64))
    mine = ophilox.philox4((1, 0, 0, 0), (3, 4), w=64)
    assert [int(v) for v in mine] != [int(v) for v in bg.random_raw(4)]


def test_uniforms_open_interval_and_exact():
    u = oracle.token_uniforms(np.arange(4096), 0xDEADBEEF12345678, 2**40 + 3)
    assert u.min() > 0.0 and u.max() < 1.0
    assert np.all(u.astype(np.float32).astype(np.float64) == u)  # exact in float32
    # Distinct counters/words give distinct draws; position and seed both matter.
    assert np.unique(u).size > 4000
    assert not np.array_equal(u, oracle.token_uniforms(np.arange(4096), 0xDEADBEEF12345678, 3))
    assert not np.array_equal(u, oracle.token_uniforms(np.arange(4096), 0xDEADBEEF12345679, 2**40 + 3))


@pytest.mark.parametrize("index", [1, 2])
def test_invariants_on_workloads(index):
    wl = make_workload(index)
    res = oracle.sample_with_mask(wl.logits, wl.dtype, wl.temperature, wl.top_k, wl.top_p,
                                  wl.min_p, wl.optin_rows, wl.seeds, wl.positions, wl.W)
    xr = lambda r: oracle.decode_logits(wl.logits[r], wl.dtype)
    errs = check_invariants(res.tokens, res.row_status, res.packed_ids, res.logprobs,
                            res.lengths, res.selected_logprob, wl.optin_rows, wl.W, xr,
                            wl.temperature)
    assert errs == []
    assert np.all(res.row_status == 0)


def test_overflow_and_status_rows():
    rng = np.random.default_rng(3)
    V = 300
    x = (rng.standard_normal((6, V))).astype(np.float32)
    x[1, 5] = np.nan
    x[2, :] = -np.inf
    x[3, 7] = np.inf
    T = np.array([1.0, 1.0, 1.0, 1.0, -1.0, 0.0], np.float32)
    k = np.array([-1, 5, 5, 5, 5, 5], np.int32)
    p = np.ones(6, np.float32)
    mp = np.zeros(6, np.float32)
    opt = np.arange(6, dtype=np.int32)
    res = oracle.sample_with_mask(x, "f32", T, k, p, mp, opt, np.arange(6, dtype=np.uint64),
                                  np.zeros(6, np.uint64), 16)
    assert res.row_status.tolist() == [1, 3, 2, 3, 4, 0]
    assert res.lengths.tolist() == [16, 0, 0, 0, 0, 1]
    assert res.tokens[1:5].tolist() == [-1, -1, -1, -1]
    assert math.isnan(res.selected_logprob[1])
    # OVERFLOW: the packed prefix is the first W of the full order; logprobs use the full support.
    full = res.rows[0]
    assert full.L == V and res.packed_ids[0].tolist() == full.support[:16].tolist()
    # The bitmask is written for the OVERFLOW slot only; it holds every finite token of row 0.
    res_b = oracle.sample_with_mask(x, "f32", T, k, p, mp, opt, np.arange(6, dtype=np.uint64),
                                    np.zeros(6, np.uint64), 16, bits_ld=48)
    assert res_b.support_bits.shape == (6, 48)
    assert not res_b.support_bits[1:].any()
    assert np.unpackbits(res_b.support_bits[0], bitorder="little")[:V].all()
    assert not np.unpackbits(res_b.support_bits[0], bitorder="little")[V:].any()
    xr = lambda r: x[r].astype(np.float64)
    assert check_invariants(res.tokens, res.row_status, res.packed_ids, res.logprobs, res.lengths,
                            res.selected_logprob, opt, 16, xr, T) == []


def test_slot_validity():
    v = oracle.slot_validity(np.array([0, 2, 2, 1, 5, -1, 7, 3, 6, 8], np.int32), 8)
    assert v.tolist() == [True, True, False, False, True, False, True, False, False, False]
    # An out-of-range entry still raises the running maximum that later entries must exceed.
    v = oracle.slot_validity(np.array([1, 9, 5], np.int32), 8)
    assert v.tolist() == [True, False, False]
    assert oracle.slot_validity(np.array([1, 3, 7], np.int32), 8).all()


# ---- Mutation checks: plant a mistake in a copy of the oracle, on the CPU, and show a pin fails.

MUTATIONS = {
    "positional_topk_drops_ties": (
        "L = n if first_fail.size == 0 else int(starts[first_fail[0]])",
        "L = min(n if first_fail.size == 0 else int(starts[first_fail[0]]), k_eff)"),
    "topk_off_by_one": ("pass_k = starts < k_eff", "pass_k = starts <= k_eff"),
    "top_p_strict": ("C[starts] <= top_p * Z", "C[starts] < top_p * Z"),
    "top_p_inclusive_mass": ("C[starts] <= top_p * Z", "incl[starts] <= top_p * Z"),
    "ties_by_descending_id": ("np.lexsort((finite_ids, -xf))", "np.lexsort((-finite_ids, -xf))"),
    "logprob_over_full_mass": ("lp64 = scaled[:L] - np.log(Z_S)", "lp64 = scaled[:L] - np.log(Z)"),
    "min_p_direction": ("pass_m = scaled[starts] >= ln_min_p", "pass_m = scaled[starts] <= ln_min_p"),
    "race_noise_sign": ("score = scaled[:L] - np.log(-np.log(u))", "score = scaled[:L] + np.log(-np.log(u))"),
    "temperature_dropped": ("scaled = (s - s[0]) / T", "scaled = (s - s[0])"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    src = inspect.getsource(osampler.sample_row)
    assert src.count(old) == 1, f"mutation anchor for {name} not found in the oracle"
    ns = dict(vars(osampler))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["sample_row"]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    fn = _mutant(name)
    fails = pins.pin_tie_example(fn)
    if not fails:
        fails = pins.pin_brute_force(fn, max_v=4, full_grid_v=4, stop_after=1)
    if not fails:
        fails = pins.pin_special_cases(fn)
    if not fails:
        fails = pins.pin_race_distribution(fn, draws=3000)
    assert fails, f"no pin detects mutation {name}"


def test_first_tie_group_is_never_reported_as_near_a_boundary():
    x = np.array([1.0, 1.0, 0.5, -0.25, -2.0])
    for (p, mp) in ((0.0, 0.0), (1.0, 1.0), (0.0, 1.0)):
        r = oracle.sample_row(x, 1.0, -1, p, mp, 3, 0)
        assert r.support.tolist() == [0, 1] and not r.top_p_flag and not r.min_p_flag
    # A later group within the window still is.
    w = np.exp(np.array([0.0, -0.5]))
    r = oracle.sample_row(np.array([0.0, -0.5]), 1.0, -1, float(np.float32(w[0] / w.sum())), 0.0, 3, 0)
    assert r.top_p_flag
