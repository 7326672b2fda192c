"""Parity of the replay kernel (tsc_replay_logprob) with the CPU oracle (needs an MI355X).

Supports and tokens always come from the CPU oracle's sampler, never from the library; both
sides then replay them on the same new logits. Every case prints its name before touching the
GPU."""
import functools
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import log, logits_tensor
from tests.parity import logprob_tol
from workloads import make_workload, perturbed_logits

pytestmark = pytest.mark.gpu

LP_TOL = 1e-5


def run_replay(logits, dtype, T, ids, lengths, tokens, cs=None, bits=None, return_logprobs=True,
               pad=0):
    import top_support_capture_amd as tsc
    dev = "cuda:0"
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)
    out = tsc.replay_logprob(logits_tensor(logits, dtype, pad=pad), t(T, torch.float32),
                             t(ids, torch.int32), t(lengths, torch.int32), t(tokens, torch.int32),
                             None if cs is None else t(cs, torch.int8),
                             None if bits is None else t(bits, torch.uint8),
                             return_logprobs=return_logprobs)
    torch.cuda.synchronize()
    return (out.selected_logprob.cpu().numpy(),
            None if out.logprobs is None else out.logprobs.cpu().numpy(),
            out.row_status.cpu().numpy())


def compare_replay(got, ref, lengths, rows=None):
    gs, gl, gst = got
    rs, rl, rst = ref
    todo = range(len(rs)) if rows is None else rows
    errs, worst, n = [], 0.0, 0
    for j in todo:
        if gst[j] != rst[j]:
            errs.append(f"row {j}: status {gst[j]} != {rst[j]}")
            continue
        if rst[j] != 0:
            if not np.isnan(gs[j]):
                errs.append(f"row {j}: logprob {gs[j]} on status {rst[j]}")
            continue
        if np.isinf(rs[j]) or np.isinf(gs[j]):
            if gs[j] != rs[j]:
                errs.append(f"row {j}: logprob {gs[j]} != {rs[j]}")
            n += 1
            continue
        worst = max(worst, abs(float(gs[j]) - float(rs[j])))
        if abs(float(gs[j]) - float(rs[j])) > float(logprob_tol(rs[j])):
            errs.append(f"row {j}: logprob {gs[j]} != {rs[j]}")
        m = int(lengths[j])
        if gl is not None and 1 <= m <= gl.shape[1]:
            a, b = gl[j, :m].astype(np.float64), rl[j, :m].astype(np.float64)
            fin = np.isfinite(b)
            if not np.array_equal(np.isfinite(a), fin) or np.any(np.abs(a[fin] - b[fin]) > logprob_tol(b[fin])):
                errs.append(f"row {j}: support logprobs differ (max {np.max(np.abs(a[fin] - b[fin]))})")
            if fin.any():
                worst = max(worst, float(np.max(np.abs(a[fin] - b[fin]))))
        n += 1
    return errs, n, worst


@functools.lru_cache(maxsize=None)
def captured(index, W):
    """The oracle sampler's capture of workload ``index``, one replay row per capture slot: the
    slot's sampling logits and temperature, packed ids, length, row status, token, and the
    bitmask of an overflowing slot."""
    wl = make_workload(index, W=W)
    bits_ld = (wl.V + 127) // 128 * 16
    ref = oracle.sample_with_mask(wl.logits, wl.dtype, wl.temperature, wl.top_k, wl.top_p,
                                  wl.min_p, wl.optin_rows, wl.seeds, wl.positions, W,
                                  bits_ld=bits_ld)
    rows = wl.optin_rows.astype(np.int64)
    ids = np.where(ref.packed_ids < 0, 0, ref.packed_ids).astype(np.int32)
    return (np.ascontiguousarray(wl.logits[rows]), wl.dtype, wl.temperature[rows].copy(), ids,
            ref.lengths.copy(), ref.row_status[rows].copy(), ref.tokens[rows].copy(),
            ref.support_bits, ref.selected_logprob.copy(), ref.logprobs.copy())


def test_tie_example_replay():
    log("case replay tie example")
    x = np.tile(np.log(np.array([0.4, 0.2, 0.2, 0.1, 0.1], np.float32)), (5, 1))
    ids = np.tile(np.array([0, 1, 2, 0], np.int32), (5, 1))
    lengths = np.full(5, 3, np.int32)
    tokens = np.arange(5, dtype=np.int32)
    T = np.ones(5, np.float32)
    for dtype in ("f32", "bf16"):
        xx = x if dtype == "f32" else (x.view(np.uint32) >> 16).astype(np.uint16)
        got = run_replay(xx, dtype, T, ids, lengths, tokens)
        ref = oracle.replay(xx, dtype, T, ids, lengths, tokens)
        errs, n, _ = compare_replay(got, ref, lengths)
        assert errs == [] and n == 5, errs
    sel = got[0]
    assert abs(sel[0] - math.log(0.5)) < 2e-2 and sel[3] == -np.inf and sel[4] == -np.inf


@pytest.mark.parametrize("index,W", [(3, 2048), (4, 8192), (2, 2)])
def test_replay_of_captured_workloads(index, W):
    # Workload 3: packed supports of ~1000; workload 4 at W = 8192: most rows overflowed, their
    # supports come from the bitmasks; workload 2 (float32) with W = 2: a mix of both.
    x, dtype, T, ids, lengths, status, tokens, bits, _, _ = captured(index, W)
    log(f"case replay workload {index} W={W}: {int((status == 1).sum())} overflowed rows")
    x_new = perturbed_logits(x, dtype, seed=100 + index)
    T = T.copy()
    T[T == 0] = 1.0  # greedy rows replay their width-1 support at T = 1
    got = run_replay(x_new, dtype, T, ids, lengths, tokens, status, bits)
    ref = oracle.replay(x_new, dtype, T, ids, lengths, tokens, status, bits)
    errs, n, worst = compare_replay(got, ref, lengths)
    log(f"  {n} rows compared, max |logprob error| {worst:.2e}")
    assert errs == [], errs[:10]
    assert n >= len(tokens) // 2


def test_replay_on_the_sampling_logits_reproduces_the_capture():
    # Replaying the oracle's capture on the very logits it was sampled from gives back the
    # oracle's own logprobs (the importance ratio of an unchanged policy is 1).
    x, dtype, T, ids, lengths, status, tokens, bits, sel, lps = captured(3, 2048)
    log("case replay on unchanged logits, workload 3")
    got = run_replay(x, dtype, T, ids, lengths, tokens, status, bits)
    ok = status == 0
    assert ok.sum() > 200
    assert np.all(got[2][ok] == 0)
    assert np.max(np.abs(got[0][ok] - sel[ok])) <= LP_TOL
    for j in np.nonzero(ok)[0]:
        m = lengths[j]
        assert np.max(np.abs(got[1][j, :m] - lps[j, :m])) <= LP_TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_replay_edge_cases(dtype):
    rng = np.random.default_rng(9)
    V, W = 1029, 8  # ragged: V % 8 = 5, so the last mask byte has bits past V
    N = 14
    x = rng.standard_normal((N, V)).astype(np.float32)
    ids = np.tile(np.array([5, 9, 1028, 0, 700, 3, 2, 1], np.int32), (N, 1))
    lengths = np.full(N, 5, np.int32)
    tokens = np.full(N, 9, np.int32)
    T = np.full(N, 0.8, np.float32)
    cs = np.zeros(N, np.int8)
    bits = np.zeros((N, (V + 7) // 8 + 3), np.uint8)
    T[1] = 0.0                      # invalid temperature
    T[2] = np.nan
    tokens[3] = V                   # token out of range
    tokens[4] = 4                   # token outside the support: -inf
    lengths[5] = 0                  # empty packed support
    lengths[6] = W + 1
    ids[7, 2] = V                   # an id out of range
    x[8, 700] = np.nan              # a non-finite support logit
    x[9, [5, 9, 1028, 0, 700]] = -np.inf  # every support logit -inf
    cs[10] = 3                      # capture status passed through
    cs[11] = 1                      # overflowed: support from the bitmask, junk past V ignored
    keep = np.zeros(V, bool)
    keep[[9, 17, 64, 65, 1000, 1027, 1028]] = True
    bits[11, :(V + 7) // 8] = np.packbits(keep, bitorder="little")
    bits[11, -4] |= 0xE0            # bits 1029..1031 of the last byte: past V
    bits[11, -3:] = 0xFF            # bytes past ceil(V / 8)
    cs[12] = 1                      # overflowed with an empty bitmask
    x[13, 9] = -np.inf              # the token's own logit is -inf: logprob -inf
    if dtype == "bf16":
        from workloads import f32_to_bf16_bits
        xx = f32_to_bf16_bits(np.nan_to_num(x, nan=0.0, neginf=0.0))
        xx[np.isnan(x)] = 0x7FC0
        xx[np.isneginf(x)] = 0xFF80
    else:
        xx = x
    log(f"case replay edge cases {dtype}")
    got = run_replay(xx, dtype, T, ids, lengths, tokens, cs, bits)
    ref = oracle.replay(xx, dtype, T, ids, lengths, tokens, cs, bits)
    errs, n, _ = compare_replay(got, ref, lengths)
    assert errs == [], errs
    assert got[2].tolist() == [0, 4, 4, 4, 0, 4, 4, 4, 3, 2, 3, 0, 4, 0]
    assert got[0][4] == -np.inf and got[0][13] == -np.inf and np.isfinite(got[0][11])
    # Without logprobs requested, the selected logprobs are the same.
    got2 = run_replay(xx, dtype, T, ids, lengths, tokens, cs, bits, return_logprobs=False)
    assert np.array_equal(got2[2], got[2])
    assert np.array_equal(np.nan_to_num(got2[0], nan=7.0), np.nan_to_num(got[0], nan=7.0))


def test_replay_large_vocabulary_gathers():
    # A vocabulary past the sampler's single-read range, with supports of 1 to 700 ids.
    rng = np.random.default_rng(21)
    N, V, W = 4, 600000, 700
    x = rng.standard_normal((N, V)).astype(np.float32)
    from workloads import f32_to_bf16_bits
    xx = f32_to_bf16_bits(x)
    ids = np.stack([rng.choice(V, W, replace=False) for _ in range(N)]).astype(np.int32)
    lengths = np.array([700, 1, 350, 699], np.int32)
    tokens = np.array([ids[0, 5], ids[1, 0], 17, ids[3, 698]], np.int32)
    T = np.array([1.0, 0.7, 1.3, 2.0], np.float32)
    log(f"case replay V={V}")
    got = run_replay(xx, "bf16", T, ids, lengths, tokens)
    ref = oracle.replay(xx, "bf16", T, ids, lengths, tokens)
    errs, n, _ = compare_replay(got, ref, lengths)
    assert errs == [] and n == N, errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,extra,pad", [(1029, 0, 0), (1029, 3, 0), (1029, 11, 0), (4096, 0, 0),
                                         (4096, 5, 0), (777, 7, 0), (1029, 15, 3), (1029, 3, 3)])
def test_replay_bitmask_strides(dtype, V, extra, pad):
    # Overflow rows whose supports come from bitmask rows of stride ceil(V / 8) + extra bytes:
    # some rows 16-byte aligned and some not, with a ragged last byte (V % 8 != 0), junk bits past
    # V and junk bytes past ceil(V / 8); densities from one member to every id. With pad, the
    # logits rows have stride V + pad, so that every row is 16-byte aligned despite a ragged V.
    rng = np.random.default_rng(V * 31 + extra)
    N = 12
    nb = (V + 7) // 8
    ld = nb + extra
    x = rng.standard_normal((N, V)).astype(np.float32) * 3.0
    density = [0.0005, 0.002, 0.01, 0.05, 0.2, 0.5, 0.9, 1.0, 0.03, 0.3, 0.001, 0.7]
    bits = rng.integers(0, 256, (N, ld), dtype=np.uint8)  # junk everywhere, then the masks
    tokens = np.zeros(N, np.int32)
    for j in range(N):
        keep = rng.random(V) < density[j]
        keep[rng.integers(V)] = True
        bits[j, :nb] = np.packbits(keep, bitorder="little")
        if V % 8:
            bits[j, nb - 1] |= np.uint8((0xFF << (V % 8)) & 0xFF)  # bits past V
        members = np.nonzero(keep)[0]
        tokens[j] = members[rng.integers(members.size)] if j % 3 else V - 1 - (j % 5)
    T = rng.uniform(0.5, 1.5, N).astype(np.float32)
    cs = np.ones(N, np.int8)
    member = lambda j: np.nonzero(np.unpackbits(bits[j, :nb], bitorder="little")[:V])[0]
    # Packed ids whose logprobs are asked for: the first and last members, an id outside the
    # support (when there is one), and the last id of the row (in a ragged last chunk if V % 8).
    ids = np.zeros((N, 4), np.int32)
    for j in range(N):
        mj = member(j)
        outside = np.setdiff1d(np.arange(V), mj)
        ids[j] = [mj[0], mj[-1], outside[0] if outside.size else mj[0], V - 1]
    lengths = np.full(N, 4, np.int32)
    x[2, member(2)[-1]] = np.nan                       # a NaN member: NONFINITE
    x[4, member(4)[0]] = np.inf                        # a +inf member: NONFINITE
    x[6, member(6)] = -np.inf                          # every member -inf: NO_SUPPORT
    x[3, np.setdiff1d(np.arange(V), member(3))] = np.nan  # NaN outside the support: ignored
    x[5, member(5)[::2]] = -np.inf                     # some members -inf
    if dtype == "bf16":
        from workloads import f32_to_bf16_bits
        xx = f32_to_bf16_bits(np.nan_to_num(x, nan=0.0, posinf=0.0, neginf=0.0))
        xx[np.isnan(x)] = 0x7FC0
        xx[np.isposinf(x)] = 0x7F80
        xx[np.isneginf(x)] = 0xFF80
    else:
        xx = x
    log(f"case replay bitmask strides {dtype} V={V} bits ld={ld} pad={pad}")
    got = run_replay(xx, dtype, T, ids, lengths, tokens, cs, bits, pad=pad)
    ref = oracle.replay(xx, dtype, T, ids, lengths, tokens, cs, bits)
    errs, n, _ = compare_replay(got, ref, lengths)
    assert errs == [] and n == int(np.sum(ref[2] == 0)) == N - 3, errs
    assert got[2][2] == 3 and got[2][4] == 3 and got[2][6] == 2 and got[2][3] == 0
    assert np.sum(np.isfinite(got[0])) >= 4


@pytest.mark.parametrize("V", [131072, 131080])
def test_replay_support_logprobs_staging_limits(V):
    # bfloat16 bitmask rows with support logprobs: at V = 131072 (16384 chunks, the most that are
    # staged in LDS) a sparse row is staged and a dense one (more member chunks than slots) is
    # not; at V = 131080 no row is. Both ways must agree with the oracle.
    rng = np.random.default_rng(V)
    N, W = 4, 64
    nb = (V + 7) // 8
    ld = (nb + 15) // 16 * 16
    from workloads import f32_to_bf16_bits
    xx = f32_to_bf16_bits(rng.standard_normal((N, V)).astype(np.float32) * 2.0)
    bits = np.zeros((N, ld), np.uint8)
    ids = np.zeros((N, W), np.int32)
    tokens = np.zeros(N, np.int32)
    for j, density in enumerate([0.002, 0.6, 0.05, 1.0]):
        keep = rng.random(V) < density
        keep[rng.integers(V)] = True
        bits[j, :nb] = np.packbits(keep, bitorder="little")
        mj = np.nonzero(keep)[0]
        ids[j] = rng.choice(mj, W) if mj.size < W else rng.choice(mj, W, replace=False)
        ids[j, -1] = np.setdiff1d(np.arange(V), mj)[0] if mj.size < V else mj[0]  # outside
        tokens[j] = mj[rng.integers(mj.size)]
    lengths = np.full(N, W, np.int32)
    T = np.array([1.0, 0.7, 1.3, 1.0], np.float32)
    cs = np.ones(N, np.int8)
    log(f"case replay staging limits V={V}")
    got = run_replay(xx, "bf16", T, ids, lengths, tokens, cs, bits)
    ref = oracle.replay(xx, "bf16", T, ids, lengths, tokens, cs, bits)
    errs, n, worst = compare_replay(got, ref, lengths)
    assert errs == [] and n == N, errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_replay_extreme_temperatures_and_magnitudes(dtype):
    # Temperatures from 1e-30 to 1e30 and logits of magnitude ~1e30, on packed and bitmask
    # supports: (x - m) / T and the support's log-sum-exp must stay finite where the oracle's
    # do. Supports and tokens are drawn here; both sides replay them.
    rng = np.random.default_rng(77)
    V, W = 3000, 48
    rows = []
    for T in (1e-30, 1e-12, 1.0, 1e20, 1e30):
        for scale in (1.0, 1e30):
            rows.append((T, scale))
    N = len(rows)
    x = np.zeros((N, V), np.float32)
    ids = np.zeros((N, W), np.int32)
    lengths = np.zeros(N, np.int32)
    tokens = np.zeros(N, np.int32)
    Ts = np.zeros(N, np.float32)
    cs = np.zeros(N, np.int8)
    bits = np.zeros((N, (V + 7) // 8), np.uint8)
    for j, (T, scale) in enumerate(rows):
        x[j] = (rng.standard_normal(V) * scale).astype(np.float32)
        Ts[j] = T
        L = int(rng.integers(1, W + 1))
        sup = rng.choice(V, L, replace=False).astype(np.int32)
        ids[j, :L] = sup
        lengths[j] = L
        tokens[j] = sup[int(rng.integers(L))]
        if j % 3 == 2:  # every third row overflowed: its support is a bitmask
            cs[j] = 1
            keep = np.zeros(V, bool)
            keep[rng.choice(V, 200, replace=False)] = True
            keep[tokens[j]] = True
            bits[j] = np.packbits(keep, bitorder="little")
    if dtype == "bf16":
        from workloads import f32_to_bf16_bits
        xx = f32_to_bf16_bits(x)
    else:
        xx = x
    log(f"case replay extreme temperatures and magnitudes {dtype}")
    got = run_replay(xx, dtype, Ts, ids, lengths, tokens, cs, bits)
    ref = oracle.replay(xx, dtype, Ts, ids, lengths, tokens, cs, bits)
    errs, n, _ = compare_replay(got, ref, lengths)
    assert errs == [], errs


@pytest.mark.parametrize("seed", list(range(48)))
def test_replay_random_sweep(seed):
    # Supports captured by the oracle sampler on random rows (scales, -inf entries, top-k, top-p,
    # min-p, widths 1..512), replayed on perturbed logits at temperatures from 1e-3 to 1e3.
    from tests.oracle_pool import oracle_batch
    from tests.test_gpu_parity import make
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    dtype = ["f32", "bf16"][seed % 2]
    V = int(rng.choice([1000, 8192, 32000, 131072, 151936] if dtype == "bf16" else [1000, 8192, 32000, 100000]))
    B = int(rng.integers(2, 9))
    rows = []
    for _ in range(B):
        x = rng.standard_normal(V) * float(rng.choice([0.3, 1.0, 3.0])) + float(rng.choice([0.0, -20.0]))
        if rng.integers(4) == 0:
            x[rng.choice(V, V // 5, replace=False)] = -np.inf
        x = np.asarray(x, np.float32)
        rows.append(oracle.decode_logits(f32_to_bf16_bits(x), "bf16") if dtype == "bf16" else x)
    T = rng.choice([0.3, 0.7, 1.0, 2.0], B).astype(np.float32)
    k = rng.choice([-1, 5, 100, 1000, 5000], B).astype(np.int32)
    p = rng.choice([1.0, 0.95, 0.8], B).astype(np.float32)
    mp = rng.choice([0.0, 0.0, 0.01, 0.1], B).astype(np.float32)
    W = int(rng.choice([1, 8, 64, 512]))
    wl = make(f"replay_sweep{seed}_{dtype}_V{V}", rows, dtype, T=T, k=k, p=p, mp=mp, W=W)
    ref = oracle_batch(wl, bits_ld=(V + 127) // 128 * 16)
    ids = np.where(ref.packed_ids < 0, 0, ref.packed_ids).astype(np.int32)
    newx = perturbed_logits(np.asarray(wl.logits), dtype, seed + 7,
                            sigma=float(rng.choice([0.0, 0.25, 2.0])))
    T2 = rng.choice([1e-3, 0.5, 1.0, 4.0, 1e3], B).astype(np.float32)
    cs = ref.row_status[wl.optin_rows].astype(np.int8)
    toks = ref.tokens[wl.optin_rows].astype(np.int32)
    xr = np.ascontiguousarray(newx[wl.optin_rows])
    log(f"case replay random sweep seed {seed}: {wl.name} B={B} W={W}")
    got = run_replay(xr, dtype, T2, ids, ref.lengths, toks, cs, ref.support_bits)
    exp = oracle.replay(xr, dtype, T2, ids, ref.lengths, toks, cs, ref.support_bits)
    errs, n, _ = compare_replay(got, exp, ref.lengths)
    assert errs == [], errs[:5]
