"""More parity of the HIP library with the CPU oracle (needs an MI355X): every row of the mixed
1024-row workload, selected mode (no support logprobs) against the oracle on every path, and
single-read rows whose top-p boundary lies just outside the report window.

Every case prints its name before touching the GPU, so a fault names the case that caused it.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import device_inputs, log, run_gpu
from tests.invariants import check_invariants
from tests.oracle_pool import oracle_batch
from tests.parity import compare
from tests.test_gpu_parity import make
from workloads import f32_to_bf16_bits, make_workload

pytestmark = pytest.mark.gpu


def _check(wl, got, ref, W=None, max_flagged_frac=0.05):
    errs, stats = compare(got, ref, wl.optin_rows)
    xr = lambda r: oracle.decode_logits(wl.logits[r], wl.dtype)
    errs += check_invariants(got["tokens"], got["row_status"], got["packed_ids"], got["logprobs"],
                             got["lengths"], got["selected_logprob"], wl.optin_rows,
                             wl.W if W is None else W, xr, wl.temperature)
    log(f"  {wl.name}: {stats}")
    assert errs == [], errs[:10]
    assert stats["flagged"] <= max(2, max_flagged_frac * stats["rows"]), stats
    return stats


@pytest.mark.parametrize("index", [5, 6])
def test_workload_every_row(index):
    # The mixed 1024-row batch (top_k 1..4096, top_p, min_p, temperature per row, 10% greedy
    # rows) and the same recipe with top-k off: every row against the oracle, which samples its
    # rows in worker processes.
    wl = make_workload(index)
    log(f"case workload {index} {wl.name} B={wl.B} V={wl.V}: every row")
    got = run_gpu(wl)
    ref = oracle_batch(wl)
    stats = _check(wl, got, ref)
    assert stats["rows"] == wl.B


@pytest.mark.parametrize("index,W", [(2, None), (3, None), (4, 8192), (4, 9216), (5, None)])
def test_selected_mode_against_oracle(index, W):
    # logprobs == NULL: packed ids, lengths, tokens and the selected logprob, against the oracle,
    # on the general path (float32), stash mode, compaction mode (clamped and full width) and
    # the mixed batch; the support mode of the same inputs must agree with it too.
    wl = make_workload(index, W=W) if W is not None else make_workload(index)
    log(f"case selected mode workload {index} W={wl.W}")
    d = device_inputs(wl)
    sel = run_gpu(wl, inputs=d, return_logprobs=False)
    assert sel["logprobs"] is None
    ref = oracle_batch(wl)
    _check(wl, sel, ref)
    sup = run_gpu(wl, inputs=d)
    for key in ("tokens", "row_status", "lengths"):
        assert np.array_equal(sup[key], sel[key]), key
    assert np.array_equal(sup["selected_logprob"], sel["selected_logprob"], equal_nan=True)
    for j, n in enumerate(sup["lengths"]):
        assert np.array_equal(sup["packed_ids"][j, :n], sel["packed_ids"][j, :n])


@pytest.mark.parametrize("W", [1024, 4095, 4096])
def test_compaction_capture_widths(W):
    # Compaction-mode captures (top_k 8192) clamped to W on either side of the length from which
    # the copy-out uses nontemporal stores: every row against the oracle.
    wl = make_workload(4, W=W)
    log(f"case compaction capture width workload 4 W={W}")
    got = run_gpu(wl)
    ref = oracle_batch(wl)
    _check(wl, got, ref)
    assert (got["lengths"] == W).sum() >= wl.B // 2, "most rows should fill the capture"


def _group_masses(x64, T):
    """(first sorted position, C/Z) of every tie group of a finite row, in logit-descending order
    (input construction only: the expected outputs come from the oracle)."""
    s = np.sort(x64)[::-1]
    w = np.exp((s - s[0]) / T)
    C = np.concatenate(([0.0], np.cumsum(w)[:-1]))
    Z = w.sum()
    starts = np.concatenate(([0], np.nonzero(s[1:] != s[:-1])[0] + 1))
    return starts, C[starts] / Z


@pytest.mark.parametrize("V", [151936, 262144])
def test_top_p_boundary_just_outside_the_window(V):
    # Rows whose top-p threshold lies 1.5e-5 to 3e-5 (in C/Z) from a tie group's boundary: no
    # row is reported, so support, length, order, logprobs and token must all be exact. Stash
    # mode (top_k 1024) and compaction mode (top_k 6000), on bf16 rows with and without ties.
    rng = np.random.default_rng(V + 17)
    deltas = [1.5e-5, -1.5e-5, 2e-5, -2e-5, 3e-5, -3e-5]
    rows, Ts, ks, ps = [], [], [], []
    for kind, k in (("gauss", 1024), ("grid", 1024), ("gauss", 6000), ("grid", 6000)):
        for i, dlt in enumerate(deltas):
            x = rng.standard_normal(V) * 1.5
            if kind == "grid":
                x = np.round(x * 8) / 8
            x = oracle.decode_logits(f32_to_bf16_bits(np.asarray(x, np.float32)), "bf16")
            T = float(np.float32(rng.uniform(0.7, 1.3)))
            starts, cz = _group_masses(x, T)
            inside = np.nonzero((starts > 0) & (starts < k) & (cz > 0.01) & (cz < 0.99))[0]
            g = inside[rng.integers(len(inside))]
            p = np.float32(cz[g] + dlt)
            rows.append(x)
            Ts.append(T)
            ks.append(k)
            ps.append(float(p))
    wl = make(f"top_p_boundary_V{V}", rows, "bf16", T=np.array(Ts), k=np.array(ks),
              p=np.array(ps), W=8192)
    ref = oracle_batch(wl)
    flagged = [r for r in range(wl.B) if ref.rows[r].flagged]
    assert not flagged, flagged  # the construction keeps every row outside the windows
    log(f"case top-p boundary rows V={V}")
    got = run_gpu(wl)
    errs, stats = compare(got, ref, wl.optin_rows)
    assert errs == [], errs[:10]
    assert stats["flagged"] == 0 and stats["rows"] == wl.B


def _greedy_case(dtype, V):
    # Greedy rows (temperature 0) with the maximum planted where the one-read greedy pass keeps
    # its bookkeeping: twice in one thread's chunks (chunk c and c + 1024 are read by the same
    # thread), twice in one chunk, in neighbouring chunks (two threads), in the ragged tail, as
    # -0 / +0 ties; and rows that are NaN, +inf, all -inf or finite in one place only.
    kv = 8 if dtype == "bf16" else 4
    rng = np.random.default_rng(V + kv)
    base = np.round(rng.standard_normal(V) * 2 * 8) / 8  # bfloat16-exact values below 64
    rows, expect = [], []

    def plant(ids, value=64.0, first=None):
        r = base.copy()
        r[list(ids)] = value
        rows.append(r)
        expect.append(min(ids) if first is None else first)

    c = 777
    plant([c * kv + 5, (c + 1024) * kv + 1])
    plant([c * kv + 6, c * kv + 2])
    plant([(c + 1) * kv, c * kv + kv - 1])
    plant([V - 1])
    plant([3, V - 1])
    z = -np.abs(base) - 1
    r = z.copy(); r[100] = -0.0; r[50] = 0.0; rows.append(r); expect.append(50)
    r = z.copy(); r[30] = -0.0; r[60] = 0.0; rows.append(r); expect.append(30)
    r = base.copy(); r[V // 2] = np.nan; rows.append(r); expect.append(-1)
    r = base.copy(); r[V - 1] = np.nan; rows.append(r); expect.append(-1)
    r = base.copy(); r[11] = np.inf; rows.append(r); expect.append(-1)
    rows.append(np.full(V, -np.inf)); expect.append(-1)
    r = np.full(V, -np.inf); r[V - 2] = -3.5; rows.append(r); expect.append(V - 2)
    rows.append(base.copy()); expect.append(int(np.argmax(base)))
    B = len(rows)
    p = np.full(B, 0.9, np.float32)
    p[-1] = 1.5  # invalid parameters on a greedy row: INVALID_PARAM
    expect[-1] = -1
    wl = make(f"greedy_{dtype}_V{V}", rows, dtype, T=0.0, k=np.arange(B) - 3, p=p,
              mp=np.where(np.arange(B) % 3 == 0, 0.05, 0.0), optin=np.arange(0, B, 2), W=4)
    return wl, np.array(expect)


@pytest.mark.parametrize("dtype,V,pad", [("bf16", 262144, 0), ("bf16", 100003, 5),
                                         ("bf16", 50000, 3), ("f32", 131075, 1),
                                         ("f32", 32000, 0)])
def test_greedy_rows(dtype, V, pad):
    # pad 5 / 1 keeps 16-byte aligned rows with a ragged end (the one-read greedy pass); pad 3
    # leaves the rows unaligned, which the general path serves.
    wl, expect = _greedy_case(dtype, V)
    log(f"case greedy rows {dtype} V={V} row stride V+{pad}")
    got = run_gpu(wl, pad=pad)
    assert got["tokens"].tolist() == expect.tolist(), (got["tokens"], expect)
    _check(wl, got, oracle.sample_with_mask(wl.logits, wl.dtype, wl.temperature, wl.top_k,
                                            wl.top_p, wl.min_p, wl.optin_rows, wl.seeds,
                                            wl.positions, wl.W), max_flagged_frac=0.0)


def _random_case(seed):
    # One seeded case: dtype and V drawn across every path's range, rows of mixed shapes, and
    # per-row parameters drawn from the values each path treats specially.
    rng = np.random.default_rng(seed)
    dtype = ["f32", "bf16"][seed % 2]
    sizes = [1000, 8192, 16384, 32000, 50000, 131072] + ([151936, 262144] if dtype == "bf16" else [131076])
    V = int(rng.choice(sizes))
    B = int(rng.integers(4, 13))
    rows = []
    for _ in range(B):
        kind = rng.choice(7, p=[0.28, 0.28, 0.2, 0.14, 0.04, 0.03, 0.03])
        if kind == 0:
            x = rng.standard_normal(V) * rng.uniform(0.5, 3.0)
        elif kind == 1:
            x = rng.standard_normal(V) + 4.0 * np.log(1.0 / np.arange(1, V + 1) ** 1.2)[rng.permutation(V)]
        elif kind == 2:
            x = np.round(rng.standard_normal(V) * 4) / 4  # ties on a grid
        elif kind == 3:
            x = rng.standard_normal(V) * 2
            x[rng.choice(V, V // 4, replace=False)] = -np.inf
        elif kind == 4:
            x = rng.standard_normal(V)
            x[rng.integers(V)] = np.nan
        elif kind == 5:
            x = rng.standard_normal(V)
            x[rng.integers(V)] = np.inf
        else:
            x = np.full(V, -np.inf)
        rows.append(x)
    T = rng.choice([0.0, 0.5, 0.8, 1.0, 1.3, 2.0], B).astype(np.float32)
    k = rng.choice([-1, 0, 1, 2, 10, 50, 500, 1024, 3000, 5000, 8192, 10000], B).astype(np.int32)
    p = rng.choice([1.0, 0.99, 0.95, 0.9, 0.5, 0.0], B).astype(np.float32)
    mp = rng.choice([0.0, 0.0, 0.01, 0.05, 0.2], B).astype(np.float32)
    R = int(rng.integers(0, B + 1))
    opt = np.sort(rng.choice(B, R, replace=False)).astype(np.int32)
    W = int(rng.choice([1, 8, 64, 1024, 4096]))
    return make(f"sweep{seed}_{dtype}_V{V}", rows, dtype, T=T, k=k, p=p, mp=mp, optin=opt, W=W)


@pytest.mark.parametrize("seed", list(range(64)))
def test_random_parameter_sweep(seed):
    wl = _random_case(seed)
    log(f"case random sweep seed {seed}: {wl.name} B={wl.B} W={wl.W} R={wl.R}")
    got = run_gpu(wl)
    ref = oracle.sample_with_mask(wl.logits, wl.dtype, wl.temperature, wl.top_k, wl.top_p,
                                  wl.min_p, wl.optin_rows, wl.seeds, wl.positions, wl.W)
    _check(wl, got, ref, max_flagged_frac=0.5)


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("bf16", 262144), ("f32", 32000),
                                     ("f32", 131072)])
def test_min_p_floor_rows(dtype, V):
    # Rows with min_p > 0 on the single-read paths, whose cutoff rises to the min-p floor of the
    # sampled maximum: heavy-headed rows (a Zipf term: a handful of candidates instead of
    # thousands), Gaussian rows, rows of negative values only (the floor is negative and is
    # rounded down to a representable cutoff) and rows on a 1/8 grid (ties), crossed with min_p
    # from 1e-4 to 1, top_p 1 or 0.95, three temperatures and top_k: off, 64, 4096 (stash mode)
    # and 6000 (compaction mode) for bfloat16; off, 64, 2048 and 3000 (beyond the margin's range)
    # for float32. Every row against the oracle.
    rng = np.random.default_rng(V + 101)
    kset = [-1, 64, 4096, 6000] if dtype == "bf16" else [-1, 64, 2048, 3000]
    ranks = np.arange(1, V + 1, dtype=np.float64)
    rows, Ts, ks, ps, mps = [], [], [], [], []
    for kind in ("zipf", "gauss", "negative", "grid"):
        for i in range(12):
            x = rng.standard_normal(V)
            if kind == "zipf":
                x = x + 4.0 * np.log(ranks ** -1.2)[rng.permutation(V)]
            elif kind == "negative":
                x = x * 1.5 - 40.0
            elif kind == "grid":
                x = np.round(x * 1.5 * 8) / 8
            x = np.asarray(x, np.float32)
            rows.append(oracle.decode_logits(f32_to_bf16_bits(x), "bf16") if dtype == "bf16" else x)
            ks.append(kset[i % 4])
            mps.append([1e-4, 0.02, 0.1, 0.6, 1.0, 0.05][i % 6])
            Ts.append([0.4, 1.0, 2.0][i % 3])
            ps.append([1.0, 0.95][(i // 4) % 2])
    wl = make(f"min_p_floor_{dtype}_V{V}", rows, dtype, T=np.array(Ts), k=np.array(ks),
              p=np.array(ps), mp=np.array(mps), W=8192)
    log(f"case min-p floor rows {dtype} V={V}")
    got = run_gpu(wl)
    ref = oracle_batch(wl)
    stats = _check(wl, got, ref, max_flagged_frac=0.1)
    assert stats["rows"] == wl.B


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f32", 32000)])
def test_min_p_floor_extremes(dtype, V):
    # The min-p floor where its margin and rounding matter: temperatures of 1e-3 and 50, min_p
    # of 1e-30 and 0.999999, values near the float range limit, a row of equal values, rows
    # with -inf entries and rows whose maximum lies outside the sampled loads (the floor then
    # comes from a smaller sampled maximum). Some of these rows go to the general path; every
    # row must agree with the oracle either way.
    rng = np.random.default_rng(V + 202)
    big = 3.0e38 if dtype == "f32" else 3.3e38
    rows, Ts, ks, ps, mps = [], [], [], [], []

    def add(x, T, k, p, mp):
        x = np.asarray(x, np.float32)
        rows.append(oracle.decode_logits(f32_to_bf16_bits(x), "bf16") if dtype == "bf16" else x)
        Ts.append(T); ks.append(k); ps.append(p); mps.append(mp)

    for T in (1e-3, 50.0):
        for mp in (1e-30, 0.999999, 0.3):
            add(rng.standard_normal(V) * 2, T, 64, 1.0, mp)
            add(rng.standard_normal(V) * 2, T, -1, 0.9, mp)
    x = rng.standard_normal(V)
    x[rng.integers(V)] = big
    add(x, 1.0, 32, 1.0, 0.5)
    add(-x, 1.0, 32, 1.0, 0.5)
    add(np.full(V, 1.25), 1.0, 64, 1.0, 0.2)
    x = rng.standard_normal(V) * 3
    x[rng.choice(V, V // 3, replace=False)] = -np.inf
    add(x, 0.7, 128, 0.95, 0.05)
    add(x, 0.7, -1, 1.0, 0.01)
    for mp in (0.01, 0.2, 0.9):
        x = rng.standard_normal(V)
        x[V - 5] = 12.0  # the maximum in the last load of the last segment, far from the sample
        add(x, 1.0, 256, 1.0, mp)
        add(x - 30.0, 1.0, -1, 0.95, mp)
    wl = make(f"min_p_floor_extremes_{dtype}_V{V}", rows, dtype, T=np.array(Ts), k=np.array(ks),
              p=np.array(ps), mp=np.array(mps), W=2048)
    log(f"case min-p floor extremes {dtype} V={V}")
    got = run_gpu(wl)
    ref = oracle_batch(wl)
    stats = _check(wl, got, ref, max_flagged_frac=0.25)
    assert stats["rows"] == wl.B


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f32", 32000), ("bf16", 4000)])
def test_tiny_temperatures(dtype, V):
    # Temperatures of 1e-30 and 1e-12 with top-p, top-k and min-p: log2(e) / T is so large that
    # the stream's mass, summed against a rounded reference, loses its meaning; such top-p rows
    # must leave for the general path, whose weights use x - m directly. A float32 row at 1e-30
    # with top_p = 0.5 once came back with an empty support. The single-read paths and (V = 4000)
    # the general path, every row against the oracle.
    rng = np.random.default_rng(V + 303)
    rows, Ts, ks, ps, mps = [], [], [], [], []
    for T in (1e-30, 1e-12):
        for (k, p, mp) in ((8, 0.5, 0.0), (-1, 0.9, 0.0), (64, 1.0, 0.1), (-1, 1.0, 0.05),
                           (64, 0.95, 0.0), (4, 0.2, 0.3)):
            x = np.asarray(np.round(rng.standard_normal(V) * 16) / 16, np.float32)
            rows.append(oracle.decode_logits(f32_to_bf16_bits(x), "bf16") if dtype == "bf16" else x)
            Ts.append(T); ks.append(k); ps.append(p); mps.append(mp)
    wl = make(f"tiny_T_{dtype}_V{V}", rows, dtype, T=np.array(Ts, np.float32), k=np.array(ks),
              p=np.array(ps), mp=np.array(mps), W=64)
    log(f"case tiny temperatures {dtype} V={V}")
    got = run_gpu(wl)
    ref = oracle_batch(wl)
    stats = _check(wl, got, ref, max_flagged_frac=0.25)
    assert stats["rows"] == wl.B


@pytest.mark.parametrize("dtype,V,kind", [("bf16", 262152, "plain"), ("bf16", 400000, "plain"),
                                          ("f32", 200000, "plain"), ("bf16", 151936, "extreme"),
                                          ("f32", 32000, "extreme")])
def test_beyond_the_single_read_ranges(dtype, V, kind):
    # "plain": vocabularies past the single-read limits (bfloat16 above 262144, float32 above
    # 131072), served by the general path. "extreme": huge temperatures (1e20, 1e30: every
    # weight ~1) and logits of magnitude ~1e30 at ordinary temperatures (the stream's mass
    # reference is out of range for top-p rows). Every row against the oracle.
    rng = np.random.default_rng(V + 404)
    rows, Ts, ks, ps, mps = [], [], [], [], []

    def add(x, T, k, p, mp):
        x = np.asarray(x, np.float32)
        rows.append(oracle.decode_logits(f32_to_bf16_bits(x), "bf16") if dtype == "bf16" else x)
        Ts.append(T); ks.append(k); ps.append(p); mps.append(mp)

    if kind == "plain":
        for (k, p, mp) in ((64, 0.9, 0.0), (-1, 0.95, 0.0), (8192, 1.0, 0.0), (1000, 0.8, 0.05),
                           (1, 1.0, 0.0)):
            add(rng.standard_normal(V) * 2, float(rng.uniform(0.5, 1.5)), k, p, mp)
        add(np.round(rng.standard_normal(V) * 8) / 8, 1.0, 500, 0.9, 0.0)
    else:
        for T in (1e20, 1e30):
            for (k, p, mp) in ((64, 0.9, 0.0), (-1, 0.5, 0.0), (16, 1.0, 0.5)):
                add(rng.standard_normal(V), T, k, p, mp)
        for (k, p, mp) in ((64, 0.9, 0.0), (-1, 0.99, 0.0), (32, 1.0, 0.2)):
            add(rng.standard_normal(V) * 1e30, 1.0, k, p, mp)
            add(rng.standard_normal(V) * 1e30 + 1e31, 1.0, k, p, mp)
    wl = make(f"beyond_{kind}_{dtype}_V{V}", rows, dtype, T=np.array(Ts, np.float32),
              k=np.array(ks), p=np.array(ps), mp=np.array(mps), W=64)
    log(f"case beyond the single-read ranges {kind} {dtype} V={V}")
    got = run_gpu(wl)
    ref = oracle_batch(wl)
    stats = _check(wl, got, ref, max_flagged_frac=0.25)
    assert stats["rows"] == wl.B


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f32", 32000), ("bf16", 4000)])
def test_extreme_seeds_and_positions(dtype, V):
    # The race's generator at the ends of its 64-bit inputs: seeds and positions of 0, 2^32 - 1,
    # 2^32, 2^63 and 2^64 - 1 (every 32-bit half of the Philox key and counter at 0 and all
    # ones), on flat rows where the token is decided by the draws. Every row against the oracle.
    rng = np.random.default_rng(V + 505)
    edge = [0, 2**32 - 1, 2**32, 2**63, 2**64 - 1]
    seeds, positions, rows = [], [], []
    for s in edge:
        for q in edge:
            seeds.append(s)
            positions.append(q)
            x = np.asarray(np.round(rng.standard_normal(V) * 4) / 4, np.float32)
            rows.append(oracle.decode_logits(f32_to_bf16_bits(x), "bf16") if dtype == "bf16" else x)
    wl = make(f"extreme_seeds_{dtype}_V{V}", rows, dtype, T=1.0, k=256, p=0.95,
              seeds=np.array(seeds, np.uint64), positions=np.array(positions, np.uint64), W=64)
    log(f"case extreme seeds and positions {dtype} V={V}")
    got = run_gpu(wl)
    ref = oracle_batch(wl)
    stats = _check(wl, got, ref)
    assert stats["rows"] == wl.B


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f32", 32000)])
def test_min_p_floor_overflow_bitmasks(dtype, V):
    # Min-p floor rows whose support overflows a capture of width 16: the packed prefix and the
    # exact support bitmask, against the oracle, in stash mode, compaction mode and on the
    # float32 path.
    from tests.test_gpu_parity import check_bits
    rng = np.random.default_rng(V + 606)
    kset = [256, 4096, 6000] if dtype == "bf16" else [256, 2048, 3000]
    rows, Ts, ks, ps, mps = [], [], [], [], []
    for k in kset:
        for mp in (0.001, 0.01, 0.2):
            for T in (0.5, 1.0):
                x = np.asarray(rng.standard_normal(V) * 2, np.float32)
                rows.append(oracle.decode_logits(f32_to_bf16_bits(x), "bf16") if dtype == "bf16" else x)
                Ts.append(T); ks.append(k); ps.append(0.97); mps.append(mp)
    wl = make(f"min_p_floor_bits_{dtype}_V{V}", rows, dtype, T=np.array(Ts), k=np.array(ks),
              p=np.array(ps), mp=np.array(mps), W=16)
    log(f"case min-p floor overflow bitmasks {dtype} V={V}")
    got = run_gpu(wl, bits=True)
    ref = oracle_batch(wl, bits_ld=(wl.V + 127) // 128 * 16)
    _check(wl, got, ref, max_flagged_frac=0.1)
    check_bits(wl, got, ref, min_rows=6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_many_capture_slots_with_invalid_entries(dtype):
    # More capture slots than one workgroup's threads (R = 1100 > 1024), so that each row finds
    # its slot by the general lookup instead of the in-kernel scan, with duplicates, a descending
    # run and out-of-range rows among them (invalid slots: length 0, NaN selected logprob).
    rng = np.random.default_rng(707)
    B, V = 1100, 16384
    x = np.asarray(rng.standard_normal((B, V)) * 2, np.float32)
    rows = [oracle.decode_logits(f32_to_bf16_bits(r), "bf16") if dtype == "bf16" else r for r in x]
    opt = np.arange(B, dtype=np.int32)
    opt[100] = opt[99]            # a duplicate
    opt[500:510] = opt[500:510][::-1]  # a descending run
    opt[700] = B + 5              # out of range
    opt[701] = -3
    wl = make(f"many_slots_{dtype}", rows, dtype, T=np.asarray(rng.uniform(0.6, 1.2, B), np.float32),
              k=64, p=0.9, mp=0.0, optin=opt, W=32)
    log(f"case many capture slots {dtype} B={B} R={len(opt)}")
    got = run_gpu(wl)
    ref = oracle_batch(wl)
    assert int(np.sum(~ref.slot_valid)) >= 10
    stats = _check(wl, got, ref)
    assert stats["rows"] == wl.B


@pytest.mark.parametrize("V", [32768, 151936, 262144])
def test_negative_maximum_at_low_temperature(V):
    # Rows whose maximum is negative, at temperatures where -m / T exceeds float exp2's range
    # (e.g. m = -1.5, T = 0.01): the bin scan's unused slots once produced 0 * inf = NaN in the
    # support mass: a NaN logprob on a row of support 1 (top_p = 1), and with top_p < 1 no bin
    # qualified, d* = -1, and the pick's loop over d <= d* never ended. Stash mode, both stream
    # forms.
    rng = np.random.default_rng(V + 808)
    rows, Ts, ks, ps, mps = [], [], [], [], []
    for shift in (-6.0, -30.0):
        for (T, k, p, mp) in ((0.01, 64, 1.0, 0.0), (1e-3, 500, 1.0, 0.1), (0.01, 64, 0.9, 0.0),
                              (0.05, 1024, 0.95, 0.01), (1e-3, -1, 1.0, 0.5)):
            x = np.round((rng.standard_normal(V) + shift) * 16) / 16
            rows.append(oracle.decode_logits(f32_to_bf16_bits(np.asarray(x, np.float32)), "bf16"))
            Ts.append(T); ks.append(k); ps.append(p); mps.append(mp)
    wl = make(f"neg_max_low_T_V{V}", rows, "bf16", T=np.array(Ts, np.float32), k=np.array(ks),
              p=np.array(ps), mp=np.array(mps), W=64)
    log(f"case negative maximum at low temperature V={V}")
    got = run_gpu(wl)
    ref = oracle_batch(wl)
    stats = _check(wl, got, ref, max_flagged_frac=0.25)
    assert stats["rows"] == wl.B


@pytest.mark.parametrize("seed", list(range(1000, 1096)))
def test_random_parameter_sweep_wide(seed):
    # The random sweep's cases with wider parameter sets: temperatures from 1e-3 to 10, min_p
    # from 1e-4 to 1 and top_p from 0 to 0.999 (this combination found a NaN support mass and a
    # pick that never ended on rows with a negative maximum at a low temperature).
    wl = _random_case(seed)
    rng = np.random.default_rng(seed + 99991)
    B = wl.B
    wl.temperature[:] = rng.choice([0.0, 1e-3, 0.05, 0.5, 1.0, 2.0, 10.0], B).astype(np.float32)
    wl.min_p[:] = rng.choice([0.0, 0.0, 1e-4, 0.01, 0.1, 0.5, 1.0], B).astype(np.float32)
    wl.top_p[:] = rng.choice([1.0, 0.999, 0.95, 0.7, 0.3, 0.0], B).astype(np.float32)
    log(f"case wide random sweep seed {seed}: {wl.name} B={wl.B} W={wl.W} R={wl.R}")
    got = run_gpu(wl)
    ref = oracle_batch(wl)
    _check(wl, got, ref, max_flagged_frac=0.5)
