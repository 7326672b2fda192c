"""Parity of the HIP library with the CPU oracle, through the C ABI (needs an MI355X).

Every case prints its name before touching the GPU, so a fault names the case that caused it.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import device_inputs, log, run_gpu
from tests.invariants import check_invariants
from tests.parity import compare, compare_bits
from workloads import Workload, f32_to_bf16_bits, make_workload

pytestmark = pytest.mark.gpu


def oracle_of(wl, W=None, rows=None, bits=False):
    bits_ld = (wl.V + 127) // 128 * 16 if bits else None
    return oracle.sample_with_mask(wl.logits, wl.dtype, wl.temperature, wl.top_k, wl.top_p,
                                   wl.min_p, wl.optin_rows, wl.seeds, wl.positions,
                                   wl.W if W is None else W, rows=rows, bits_ld=bits_ld)


def check_bits(wl, got, ref, rows=None, min_rows=1):
    errs, n = compare_bits(got, ref, wl.optin_rows, rows=rows)
    log(f"  {wl.name}: {n} overflow bitmask rows checked")
    assert errs == [], errs[:10]
    assert n >= min_rows, n


def check(wl, got, ref, W=None, rows=None, max_flagged_frac=0.05):
    W = wl.W if W is None else W
    errs, stats = compare(got, ref, wl.optin_rows, rows=rows)
    xr = lambda r: oracle.decode_logits(wl.logits[r], wl.dtype)
    errs += check_invariants(got["tokens"], got["row_status"], got["packed_ids"], got["logprobs"],
                             got["lengths"], got["selected_logprob"], wl.optin_rows, W, xr,
                             wl.temperature, rows=rows)
    log(f"  {wl.name}: {stats}")
    assert errs == [], errs[:10]
    assert stats["flagged"] <= max(2, max_flagged_frac * stats["rows"]), stats
    return stats


def make(name, rows, dtype="f32", T=1.0, k=-1, p=1.0, mp=0.0, optin=None, W=64, seeds=None,
         positions=None):
    """A workload from explicit float rows (``dtype`` bf16 rounds them to bfloat16)."""
    x = np.stack([np.asarray(r, dtype=np.float32) for r in rows])
    B = x.shape[0]
    full = lambda v, dt: np.asarray(v, dtype=dt) if np.ndim(v) else np.full(B, v, dtype=dt)
    logits = f32_to_bf16_bits(np.nan_to_num(x, nan=0.0, posinf=0.0, neginf=0.0)) if dtype == "bf16" else x
    if dtype == "bf16":  # keep the non-finite patterns exactly
        logits = logits.copy()
        logits[np.isnan(x)] = 0x7FC0
        logits[np.isposinf(x)] = 0x7F80
        logits[np.isneginf(x)] = 0xFF80
    opt = np.arange(B, dtype=np.int32) if optin is None else np.asarray(optin, np.int32)
    sd = (np.arange(B, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15)) if seeds is None else np.asarray(seeds, np.uint64)
    ps = (np.arange(B, dtype=np.uint64) + np.uint64(2**33 + 5)) if positions is None else np.asarray(positions, np.uint64)
    return Workload(name, dtype, logits, full(T, np.float32), full(k, np.int32), full(p, np.float32),
                    full(mp, np.float32), opt, sd, ps, W)


def test_tie_example_from_the_pages_on_256_rows():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tie_example.json")))
    B = g["batch_size"]
    for dtype in ("f32", "bf16"):
        log(f"case tie_example {dtype} B={B}")
        row = np.log(np.array(g["probs"], np.float32))
        wl = make("tie_example", [row] * B, dtype, k=g["top_k"], p=g["top_p"], W=8)
        got = run_gpu(wl)
        assert np.all(got["lengths"] == 3)
        assert np.all(got["packed_ids"][:, :3] == np.array(g["expected_support_ids"]))
        assert np.all(np.isin(got["tokens"], g["expected_support_ids"]))
        check(wl, got, oracle_of(wl))


@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_workload_parity_full(index):
    wl = make_workload(index)
    log(f"case workload {index} {wl.name} B={wl.B} V={wl.V} W={wl.W}")
    got = run_gpu(wl)
    check(wl, got, oracle_of(wl))


@pytest.mark.parametrize("index,W", [(2, 2), (3, 512), (4, 8192)])
def test_overflow_support_bitmasks(index, W):
    # Workload 2 (float32, general path) with W = 2, workload 3 (stash mode) with W = 512 and
    # workload 4 (compaction mode) at its own W: most captured rows overflow.
    wl = make_workload(index, W=W)
    log(f"case support bitmasks workload {index} W={W}")
    got = run_gpu(wl, bits=True)
    ref = oracle_of(wl, bits=True)
    check(wl, got, ref)
    check_bits(wl, got, ref, min_rows=len(wl.optin_rows) // 2)


def test_workload4_wide_packed_width():
    wl = make_workload(4, W=9216)  # the pages' own packed width for top_k=8192
    log(f"case workload 4 W=9216")
    got = run_gpu(wl)
    stats = check(wl, got, oracle_of(wl))
    assert stats["overflow"] == 0


def test_workload5_sampled_rows():
    wl = make_workload(5)
    log(f"case workload 5 {wl.name} B={wl.B} V={wl.V} (sampled oracle rows)")
    got = run_gpu(wl)
    rng = np.random.default_rng(11)
    greedy = np.nonzero(wl.temperature == 0)[0][:8]
    opt = rng.choice(wl.optin_rows, 24, replace=False)
    rest = rng.choice(wl.B, 16, replace=False)
    rows = np.unique(np.concatenate([greedy, opt, rest]))
    check(wl, got, oracle_of(wl, rows=rows), rows=rows)


def _edge_rows(rng, V):
    grid = np.round(rng.standard_normal(V) * 2) / 2  # heavy ties on a 0.5 grid
    flat = np.zeros(V)
    x = rng.standard_normal(V) * 3
    neg = x.copy(); neg[rng.choice(V, V // 3, replace=False)] = -np.inf
    allneg = np.full(V, -np.inf)
    nan = x.copy(); nan[V // 2] = np.nan
    pinf = x.copy(); pinf[1] = np.inf
    tiedmax = x.copy(); tiedmax[[3, 10, V - 1]] = x.max() + 1
    zeros = -np.abs(x) - 1; zeros[[4, 9]] = 0.0; zeros[7] = -0.0
    return dict(grid=grid, flat=flat, x=x, neg=neg, allneg=allneg, nan=nan, pinf=pinf,
                tiedmax=tiedmax, zeros=zeros)


EDGE_PARAMS = [
    # (label, row name, T, k, p, min_p)
    ("topk_ties", "grid", 1.0, 50, 1.0, 0.0),
    ("topp_ties", "grid", 1.0, -1, 0.6, 0.0),
    ("joint_ties", "grid", 0.8, 100, 0.7, 0.0),
    ("all_equal_k5", "flat", 1.0, 5, 1.0, 0.0),
    ("all_equal_p", "flat", 1.0, -1, 0.3, 0.0),
    ("neg_inf", "neg", 1.0, 20, 0.9, 0.0),
    ("all_neg_inf", "allneg", 1.0, 20, 0.9, 0.0),
    ("nan", "nan", 1.0, 20, 0.9, 0.0),
    ("pos_inf", "pinf", 1.0, 20, 0.9, 0.0),
    ("k1_tied_max", "tiedmax", 1.0, 1, 1.0, 0.0),
    ("k_ge_V", "x", 1.0, 10**6, 1.0, 0.0),
    ("k0", "x", 1.0, 0, 0.95, 0.0),
    ("k_neg", "x", 1.3, -5, 0.9, 0.0),
    ("p0", "x", 1.0, 40, 0.0, 0.0),
    ("p1", "x", 1.0, 40, 1.0, 0.0),
    ("minp1", "tiedmax", 1.0, -1, 1.0, 1.0),
    ("minp_half", "x", 0.7, -1, 1.0, 0.5),
    ("minp_joint", "x", 1.1, 200, 0.9, 0.05),
    ("tiny_T", "x", 1e-3, 30, 0.9, 0.0),
    ("flat_T", "x", 50.0, -1, 0.5, 0.0),
    ("greedy_tied", "tiedmax", 0.0, 7, 0.5, 0.0),
    ("greedy_neg", "neg", 0.0, -1, 1.0, 0.0),
    ("zero_ties", "zeros", 1.0, 2, 1.0, 0.0),
    ("bad_T", "x", -1.0, 5, 0.9, 0.0),
    ("nan_T", "x", float("nan"), 5, 0.9, 0.0),
    ("subnormal_T", "x", 1e-40, 5, 0.9, 0.0),
    ("bad_p", "x", 1.0, 5, 1.5, 0.0),
    ("bad_minp", "x", 1.0, 5, 0.9, -0.1),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_cases(dtype):
    rng = np.random.default_rng(123)
    V = 3001  # not a multiple of the vector width
    rows = _edge_rows(rng, V)
    names = [e[0] for e in EDGE_PARAMS]
    x = [rows[e[1]] for e in EDGE_PARAMS]
    cols = list(zip(*[e[2:] for e in EDGE_PARAMS]))
    wl = make(f"edge_{dtype}", x, dtype, T=np.array(cols[0]), k=np.array(cols[1]),
              p=np.array(cols[2]), mp=np.array(cols[3]), W=64)
    log(f"case edge cases {dtype}: {names}")
    got = run_gpu(wl)
    ref = oracle_of(wl)
    errs, stats = compare(got, ref, wl.optin_rows)
    assert errs == [], [(e, names[int(e.split()[1].rstrip(':'))]) if e.startswith("row") else e for e in errs]
    check(wl, got, ref, max_flagged_frac=0.2)


@pytest.mark.parametrize("V", [1, 2, 7, 8, 9, 1023, 1025])
def test_small_and_ragged_vocabularies(V):
    rng = np.random.default_rng(V)
    rows = [np.round(rng.standard_normal(V) * 4) / 4 for _ in range(6)]
    for dtype in ("f32", "bf16"):
        wl = make(f"ragged_V{V}_{dtype}", rows, dtype, T=np.array([1, .5, 2, 1, 0, 1]),
                  k=np.array([3, -1, 1, 5, 2, 100]), p=np.array([.9, .5, 1, 0, 1, .99]),
                  mp=np.array([0, .1, 0, 0, 0, .3]), W=4)
        log(f"case ragged V={V} {dtype}")
        check(wl, run_gpu(wl), oracle_of(wl), max_flagged_frac=0.5)


def test_unaligned_row_stride():
    wl = make_workload(2)
    log("case workload 2 with row stride V+1 (unaligned rows)")
    check(wl, run_gpu(wl, pad=1), oracle_of(wl))
    rng = np.random.default_rng(5)
    wlb = make("bf16_stride", [rng.standard_normal(5000) * 2 for _ in range(8)], "bf16", k=64, p=0.9)
    log("case bf16 rows with row stride V+3")
    check(wlb, run_gpu(wlb, pad=3), oracle_of(wlb))


def test_supports_wider_than_on_chip_buffer():
    rng = np.random.default_rng(9)
    V = 40000
    rows = [rng.standard_normal(V), np.zeros(V), np.round(rng.standard_normal(V)), rng.standard_normal(V)]
    for W in (16, 16384):
        wl = make(f"wide_W{W}", rows, "f32", k=np.array([-1, -1, -1, 30000]), p=1.0, W=W)
        log(f"case supports of {V} tokens, W={W}")
        got = run_gpu(wl)
        stats = check(wl, got, oracle_of(wl))
        assert stats["overflow"] == 4


def test_optin_subsets_and_invalid_slots():
    wl = make_workload(2)
    base = oracle_of(wl)
    for opt in ([], [5], list(range(wl.B)), [0, 3, 3, 2, 70, 10, -1, 63]):
        w2 = Workload(**{**wl.__dict__, "optin_rows": np.array(opt, np.int32)})
        log(f"case workload 2 optin={opt[:8]}")
        got = run_gpu(w2)
        ref = oracle_of(w2)
        assert np.array_equal(got["tokens"], base.tokens)  # capture never changes the draw
        errs, _ = compare(got, ref, w2.optin_rows)
        assert errs == []


def test_selected_mode_matches_support_mode():
    wl = make_workload(3)
    log("case workload 3 selected mode vs support mode")
    d = device_inputs(wl)
    sup = run_gpu(wl, inputs=d)
    sel = run_gpu(wl, inputs=d, return_logprobs=False)
    for key in ("tokens", "row_status", "lengths", "selected_logprob"):
        assert np.array_equal(sup[key], sel[key]), key
    for j, n in enumerate(sup["lengths"]):
        assert np.array_equal(sup["packed_ids"][j, :n], sel["packed_ids"][j, :n])


def test_repeated_calls_are_bit_identical():
    wl = make_workload(3)
    log("case workload 3 repeated")
    d = device_inputs(wl)
    a = run_gpu(wl, inputs=d)
    b = run_gpu(wl, inputs=d)
    for key in a:
        if a[key] is not None:
            assert a[key].tobytes() == b[key].tobytes() or key in ("packed_ids", "logprobs"), key
    for j, n in enumerate(a["lengths"]):
        assert a["packed_ids"][j, :n].tobytes() == b["packed_ids"][j, :n].tobytes()
        assert a["logprobs"][j, :n].tobytes() == b["logprobs"][j, :n].tobytes()


def _fast_rows(rng, V):
    """bf16-representable rows for the single-read path (V in its range, k small)."""
    grid = np.round(rng.standard_normal(V) * 2.5 * 8) / 8          # many ties, like workload 3
    gauss = rng.standard_normal(V) * 1.5
    neg = gauss.copy(); neg[rng.choice(V, V // 4, replace=False)] = -np.inf
    nan = gauss.copy(); nan[V - 3] = np.nan
    pinf = gauss.copy(); pinf[V // 3] = np.inf
    allneg = np.full(V, -np.inf)
    # Top values hidden away from the first load of every wave segment: the early cutoff is too
    # low, the stash overflows and the row must take the general path.
    seg = V // 16
    hidden = rng.standard_normal(V)
    for w in range(16):
        hidden[w * seg + 512:(w + 1) * seg] += 6.0
    # The first loads hold the row's largest values but fewer than k of them: cutoff too high,
    # fewer than k candidates, general path.
    front = rng.standard_normal(V) - 5.0
    for w in range(16):
        front[w * seg:w * seg + 16] = 8.0 + rng.standard_normal(16)
    # A support of more than 256 distinct keys within the histogram's key span (values spread
    # over six binades above a dense filler): the capture tables are too small, general path.
    spread = rng.uniform(1.0, 1.9, V)
    spread[rng.choice(V, 900, replace=False)] = np.geomspace(2.0, 60.0, 900)
    # A key span of several hundred bins between the cutoff and the maximum (spikes on a
    # geometric ladder above a coarse-grid bulk) that still has few distinct values: the wide
    # form of the bin scan, served by the single-read path.
    wide = np.round(rng.standard_normal(V) * 4) / 4
    wide[rng.choice(V, 40, replace=False)] = np.round(np.geomspace(8.0, 60.0, 40))
    # The maximum is zero, held by +0 and -0 tokens (they tie), over a negative bulk.
    zeros = -np.abs(rng.standard_normal(V)) - 0.5
    zpos = rng.choice(V, 12, replace=False)
    zeros[zpos[:6]] = 0.0
    zeros[zpos[6:]] = -0.0
    # A language-model-like head: a log-Zipf rank bonus on a random permutation over a Gaussian
    # bulk, so that top-p keeps a handful of tokens (drawn last: the rows above keep their draws).
    rank = rng.permutation(V).astype(np.float64) + 1.0
    zipf = rng.standard_normal(V) + 4.0 * (-1.2 * np.log(rank))
    return dict(grid=grid, gauss=gauss, neg=neg, nan=nan, pinf=pinf, allneg=allneg,
                hidden=hidden, front=front, spread=spread, wide=wide, zeros=zeros, zipf=zipf)


FAST_PARAMS = [
    # (label, row, T, k, p, min_p)
    ("grid_k1024_p95", "grid", 0.8, 1024, 0.95, 0.0),
    ("grid_k64_p1", "grid", 1.0, 64, 1.0, 0.0),
    ("grid_k1_ties", "grid", 1.0, 1, 1.0, 0.0),
    ("grid_k1536", "grid", 1.2, 1536, 0.9, 0.0),
    ("gauss_k300_p5", "gauss", 0.7, 300, 0.5, 0.0),
    ("gauss_k1000_p0", "gauss", 1.0, 1000, 0.0, 0.0),
    ("gauss_minp", "gauss", 1.0, 1200, 1.0, 0.2),
    ("gauss_minp_p", "gauss", 0.9, 800, 0.8, 0.05),
    ("neg_inf", "neg", 1.0, 500, 0.9, 0.0),
    ("nan_p", "nan", 1.0, 100, 0.9, 0.0),
    ("nan_nop", "nan", 1.0, 100, 1.0, 0.0),
    ("pos_inf", "pinf", 1.0, 100, 1.0, 0.0),
    ("all_neg_inf", "allneg", 1.0, 100, 0.9, 0.0),
    ("hidden_top", "hidden", 1.0, 1024, 0.95, 0.0),
    ("front_loaded", "front", 1.0, 1024, 1.0, 0.0),
    ("spread_keys", "spread", 5.0, 1000, 1.0, 0.0),
    ("wide_span", "wide", 12.0, 1024, 0.97, 0.0),
    ("wide_span_minp", "wide", 12.0, 1024, 1.0, 0.01),
    ("tiny_T", "gauss", 1e-3, 50, 0.9, 0.0),
    ("greedy", "grid", 0.0, 50, 0.9, 0.0),
    ("min_p_one", "grid", 1.0, 500, 0.9, 1.0),           # only the top tie group
    ("signed_zero_top_k1", "zeros", 1.0, 1, 1.0, 0.0),   # -0 and +0 tie at the maximum
    ("signed_zero_p0", "zeros", 0.7, 300, 0.0, 0.0),
    ("huge_T", "gauss", 1.0e30, 1024, 0.95, 0.0),        # every weight is 1: top-k decides
    ("top_p_zero_ties", "grid", 1.0, 1024, 0.0, 0.0),
    # top_k above 1536: stash mode with loads past the stash read again (top_k <= 4096), the
    # compaction mode above that; tiny_T above flags every load, overflows both and falls back
    ("compact_k4000_p9", "gauss", 1.0, 4000, 0.9, 0.0),
    ("compact_k8192_p1", "gauss", 1.0, 8192, 1.0, 0.0),
    ("compact_grid_k2000", "grid", 0.8, 2000, 0.95, 0.0),
    ("compact_minp", "gauss", 1.0, 3000, 1.0, 0.05),
    ("compact_minp_p", "wide", 12.0, 2500, 0.97, 0.01),
    ("compact_nan", "nan", 1.0, 2000, 0.9, 0.0),
    ("compact_pinf", "pinf", 1.0, 2000, 1.0, 0.0),
    ("compact_neg_inf", "neg", 1.0, 3000, 0.9, 0.0),
    ("compact_hidden_top", "hidden", 1.0, 4096, 0.95, 0.0),
    # A NaN or +inf logit with top_p < 1: the mass overflows or turns NaN; in stash mode
    # (top_k <= 4096) and in compaction mode (top_k above 4096), with and without min-p.
    ("pinf_p", "pinf", 1.0, 100, 0.9, 0.0),
    ("pinf_minp_p", "pinf", 0.8, 300, 0.8, 0.05),
    ("nan_minp_p", "nan", 1.2, 300, 0.8, 0.05),
    ("compact8k_nan_p", "nan", 1.0, 6000, 0.9, 0.0),
    ("compact8k_pinf_p", "pinf", 1.0, 6000, 0.9, 0.0),
    ("compact8k_pinf_minp", "pinf", 1.0, 8192, 0.95, 0.02),
    # top_k off (<= 0 or >= V) or above the compaction range: the row is served here when top-p
    # or min-p ends its support among the candidates, else by the general path.
    ("koff_zipf_p9", "zipf", 1.0, -1, 0.9, 0.0),
    ("koff_zipf_p99", "zipf", 1.4, 0, 0.99, 0.0),
    ("koff_zipf_minp", "zipf", 1.0, -1, 1.0, 0.05),
    ("koff_zipf_p_minp", "zipf", 0.7, -1, 0.95, 0.001),
    ("koff_grid_p5", "grid", 0.8, -1, 0.5, 0.0),
    ("koff_grid_p0", "grid", 1.0, -1, 0.0, 0.0),
    ("koff_gauss_minp", "gauss", 1.0, -1, 1.0, 0.3),
    ("koff_gauss_p9", "gauss", 1.0, -1, 0.9, 0.0),         # a wide support: general path
    ("koff_wide_minp_p", "wide", 12.0, -1, 0.97, 0.01),
    ("koff_nan_p", "nan", 1.0, -1, 0.9, 0.0),
    ("koff_pinf_p", "pinf", 1.0, -1, 0.9, 0.0),
    ("koff_allneg_p", "allneg", 1.0, -1, 0.9, 0.0),
    ("kgeV_grid_p7", "grid", 1.0, 10**6, 0.7, 0.0),
    ("kbig_zipf_p8", "zipf", 0.5, 20000, 0.8, 0.0),
    ("kbig_gauss_p", "gauss", 1.0, 12000, 0.5, 0.0),
    ("koff_nofilter", "zipf", 1.0, -1, 1.0, 0.0),          # every finite token: general path
]


@pytest.mark.parametrize("V", [32768, 151936, 262144])
def test_single_read_path_rows(V):
    rng = np.random.default_rng(77)
    rows = _fast_rows(rng, V)
    names = [e[0] for e in FAST_PARAMS]
    x = [rows[e[1]] for e in FAST_PARAMS]
    cols = list(zip(*[e[2:] for e in FAST_PARAMS]))
    for W in (2048, 16):
        wl = make(f"fast_V{V}_W{W}", x, "bf16", T=np.array(cols[0]), k=np.array(cols[1]),
                  p=np.array(cols[2]), mp=np.array(cols[3]), W=W)
        log(f"case single-read path V={V} W={W}: {names}")
        got = run_gpu(wl, bits=True)
        ref = oracle_of(wl, bits=True)
        errs, stats = compare(got, ref, wl.optin_rows)
        assert errs == [], [(e, names[int(e.split()[1].rstrip(':'))]) if e.startswith("row") else e for e in errs]
        check(wl, got, ref, max_flagged_frac=0.2)
        check_bits(wl, got, ref, min_rows=0 if W == 2048 else 10)


def test_empty_batch():
    # B = 0 (and a replay of N = 0 rows): no launch, empty outputs, no error.
    import torch
    import top_support_capture_amd as tsc
    log("case empty batch")
    dev = "cuda:0"
    e = lambda dt: torch.empty(0, dtype=dt, device=dev)
    x = torch.empty((0, 32768), dtype=torch.bfloat16, device=dev)
    out = tsc.sample_with_mask(x, e(torch.float32), e(torch.int32), e(torch.float32),
                               e(torch.float32), e(torch.int32), e(torch.int64), e(torch.int64), 16)
    torch.cuda.synchronize()
    assert out.tokens.numel() == 0 and out.packed_ids.shape == (0, 16)
    rep = tsc.replay_logprob(x, e(torch.float32), torch.empty((0, 16), dtype=torch.int32, device=dev),
                             e(torch.int32), e(torch.int32))
    torch.cuda.synchronize()
    assert rep.selected_logprob.numel() == 0 and rep.row_status.numel() == 0


@pytest.mark.parametrize("V", [16384, 32000, 100000])
def test_single_read_path_rows_f32(V):
    # The float32 single-read path (sorted candidates): the same row kinds and parameters as the
    # bfloat16 rows, as float32 values; rows it cannot decide take the general path.
    rng = np.random.default_rng(91 + V)
    rows = _fast_rows(rng, V)
    rows["gauss_fine"] = rng.standard_normal(V) * 1.7  # distinct float32 values (few ties)
    params = FAST_PARAMS + [("fine_k100_p9", "gauss_fine", 1.0, 100, 0.9, 0.0),
                            ("fine_k2048", "gauss_fine", 0.8, 2048, 0.97, 0.0),
                            ("fine_koff_minp", "gauss_fine", 0.5, -1, 1.0, 0.02)]
    names = [e[0] for e in params]
    x = [rows[e[1]] for e in params]
    cols = list(zip(*[e[2:] for e in params]))
    for W in (2048, 16):
        wl = make(f"fast_f32_V{V}_W{W}", x, "f32", T=np.array(cols[0]), k=np.array(cols[1]),
                  p=np.array(cols[2]), mp=np.array(cols[3]), W=W)
        log(f"case float32 single-read path V={V} W={W}: {names}")
        got = run_gpu(wl, bits=True)
        ref = oracle_of(wl, bits=True)
        errs, stats = compare(got, ref, wl.optin_rows)
        assert errs == [], [(e, names[int(e.split()[1].rstrip(':'))]) if e.startswith("row") else e for e in errs]
        check(wl, got, ref, max_flagged_frac=0.2)
        check_bits(wl, got, ref, min_rows=0 if W == 2048 else 10)
