"""Pins for the CPU oracle: checks that tie it to the pages and to mathematics, not to itself.

Each ``pin_*`` function takes a row sampler with the signature of ``oracle.sample_row`` and
returns a list of failure descriptions (empty = pass). The oracle tests call them with the real
oracle; the mutation tests call them with deliberately broken copies of it, to show that a
plausible mistake in the oracle (a dropped tie, a strict inequality, a wrong normalizer, a
flipped sign) fails at least one pin.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

from oracle import token_uniforms

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f32(v):
    return float(np.float32(v))


def pin_tie_example(sample_row):
    """The pages' worked tie case (sglang PR #36630 summary, 'Key code' tie test): probabilities
    [0.4, 0.2, 0.2, 0.1, 0.1] with top_k=2 and top_p=0.45 keep ids {0, 1, 2}, more than top_k.
    Logits are the float32 logs of those probabilities, so equal probabilities have equal bits.
    The renormalized support is {0.4, 0.2, 0.2} / 0.8, so the logprobs are ln 1/2, ln 1/4, ln 1/4
    (closed form); the drawn token must lie in the support."""
    g = json.load(open(os.path.join(GOLDEN, "tie_example.json")))
    x = np.log(np.array(g["probs"], dtype=np.float32)).astype(np.float32).astype(np.float64)
    fails = []
    for seed in range(16):
        try:
            r = sample_row(x, 1.0, g["top_k"], g["top_p"], 0.0, seed, 0)
        except Exception as e:  # a broken oracle may raise
            return [f"tie example raised {e!r}"]
        if r.support.tolist() != g["expected_support_ids"]:
            fails.append(f"tie example support {r.support.tolist()}")
        want = np.array([math.log(0.5), math.log(0.25), math.log(0.25)])
        if r.L == 3 and np.max(np.abs(r.logprobs - want)) > 1e-6:
            fails.append(f"tie example logprobs {r.logprobs}")
        if r.token not in g["expected_support_ids"]:
            fails.append(f"tie example token {r.token}")
    return fails


def brute_force(x, T, k, p, min_p):
    """Per-token closed form of the joint filter, O(V^2), no sorting:
    i in S  <=>  x_i finite, #{j: x_j > x_i} < k_eff, sum_{x_j > x_i} w_j <= p * Z (if p < 1),
    and (x_i - max)/T >= ln(min_p) (if min_p > 0).
    Returns (support in (logit desc, id asc) order, near_boundary)."""
    T, p, min_p = _f32(T), _f32(p), _f32(min_p)
    V = len(x)
    F = [i for i in range(V) if x[i] > -math.inf]
    n = len(F)
    m = max(x[i] for i in F)
    k_eff = k if 1 <= k < n else n
    w = {i: math.exp((x[i] - m) / T) for i in F}
    Z = math.fsum(w.values())
    S, near = [], False
    for i in F:
        gt = [j for j in F if x[j] > x[i]]
        mass = math.fsum(w[j] for j in gt)
        ok = len(gt) < k_eff
        if p < 1.0:
            ok = ok and mass <= p * Z
            near |= abs(mass - p * Z) <= 1e-9 * Z
        if min_p > 0.0:
            lhs = (x[i] - m) / T
            ok = ok and lhs >= math.log(min_p)
            near |= abs(lhs - math.log(min_p)) <= 1e-9
        if ok:
            S.append(i)
    S.sort(key=lambda i: (-x[i], i))
    return S, near


def _check_against_brute(sample_row, x, T, k, p, mp, seed, pos):
    """Compare one oracle row with the brute force; returns a failure string or None."""
    S, near = brute_force(x, T, k, p, mp)
    try:
        r = sample_row(np.asarray(x, dtype=np.float64), T, k, p, mp, seed, pos)
    except Exception as e:
        return f"raised {e!r} for x={x} T={T} k={k} p={p} mp={mp}"
    if near:
        return None
    if r.support.tolist() != S:
        return f"support {r.support.tolist()} != {S} for x={x} T={T} k={k} p={p} mp={mp}"
    m = max(x[i] for i in S)
    lse = math.log(math.fsum(math.exp((x[i] - m) / _f32(T)) for i in S))
    want = np.array([(x[i] - m) / _f32(T) - lse for i in S])
    if np.max(np.abs(r.logprobs.astype(np.float64) - want)) > 2e-6:
        return f"logprobs {r.logprobs} != {want} for x={x}"
    u = token_uniforms(np.array(S), seed, pos)
    score = [(x[i] - m) / _f32(T) - math.log(-math.log(u[j])) for j, i in enumerate(S)]
    best = max(score)
    tok = min(i for j, i in enumerate(S) if score[j] == best)
    if r.token != tok:
        return f"token {r.token} != {tok} for x={x}"
    return None


LEVELS = (1.0, 0.0, -0.75, -math.inf)


def pin_brute_force(sample_row, max_v=6, full_grid_v=4, rng_seed=0, stop_after=None):
    """Exhaustive comparison over every logit vector of length <= max_v drawn from a 4-level grid
    (so every tie pattern and -inf exclusions occur), against the per-token closed form. Vectors
    with V <= full_grid_v run the whole parameter grid; longer ones a seeded sample of it."""
    ks = (-1, 0, 1, 2, 3, 5)
    ps = (0.0, 0.5, 0.8, 1.0)
    mps = (0.0, 0.3, 1.0)
    Ts = (0.5, 2.0)
    grid = list(itertools.product(ks, ps, mps, Ts))
    rng = np.random.default_rng(rng_seed)
    fails = []
    for V in range(1, max_v + 1):
        for x in itertools.product(LEVELS, repeat=V):
            if all(v == -math.inf for v in x):
                continue
            combos = grid if V <= full_grid_v else [grid[i] for i in rng.choice(len(grid), 3, replace=False)]
            for (k, p, mp, T) in combos:
                f = _check_against_brute(sample_row, list(x), T, k, p, mp, 7 + V, 3)
                if f:
                    fails.append(f)
                    if stop_after and len(fails) >= stop_after:
                        return fails
    return fails


def pin_special_cases(sample_row, rng_seed=1):
    """Cases that reduce to textbook or library routines."""
    from scipy.special import log_softmax
    rng = np.random.default_rng(rng_seed)
    fails = []
    for trial in range(4):
        V = 700
        x = (rng.standard_normal(V) * 2).astype(np.float32).astype(np.float64)
        x[rng.choice(V, 20, replace=False)] = -np.inf
        T = [0.7, 1.0, 1.9, 0.35][trial]
        F = np.nonzero(np.isfinite(x))[0]
        # No filter at all: the support is every finite token and logprobs are log_softmax(x/T).
        r = sample_row(x, T, -1, 1.0, 0.0, trial, 0)
        if sorted(r.support.tolist()) != F.tolist():
            fails.append("unfiltered support is not the finite set")
        else:
            ref = log_softmax(x[F] / _f32(T))
            got = np.empty(V)
            got[r.support] = r.logprobs
            if np.max(np.abs(got[F] - ref)) > 1e-5:
                fails.append("unfiltered logprobs differ from scipy log_softmax")
        # Distinct logits, top-k only: the set is numpy's top-k and does not depend on T.
        k = [1, 10, 64, 300][trial]
        xs = x[F]
        if np.unique(xs).size == xs.size:
            want = set(F[np.argsort(-xs, kind="stable")[:k]].tolist())
            for TT in (0.5, 1.0, 3.0):
                rr = sample_row(x, TT, k, 1.0, 0.0, trial, 0)
                if set(rr.support.tolist()) != want:
                    fails.append(f"top-{k} set differs from argsort at T={TT}")
        # top_p = 0 and min_p = 1 keep exactly the top tie group.
        xt = x.copy()
        top = np.max(xt[F])
        tied = rng.choice(F, 3, replace=False)
        xt[tied] = top
        want = sorted(np.nonzero(xt == top)[0].tolist())
        for (p, mp) in ((0.0, 0.0), (1.0, 1.0), (0.0, 1.0)):
            rr = sample_row(xt, T, -1, p, mp, trial, 0)
            if rr.support.tolist() != want:
                fails.append(f"top_p={p} min_p={mp} is not the top tie group")
        # Greedy: numpy's argmax (first index of the maximum), width 1, logprob 0.
        g = sample_row(xt, 0.0, 5, 0.9, 0.0, trial, 0)
        if g.token != int(np.argmax(np.where(np.isfinite(xt), xt, -np.inf))) or g.L != 1 or g.logprobs[0] != 0.0:
            fails.append("greedy row is not argmax / width 1 / logprob 0")
    return fails


def pin_race_distribution(sample_row, draws=6000):
    """The exponential race draws token i with probability w_i / sum(w) (chi-square, 3 dof)."""
    from scipy.stats import chisquare
    probs = np.array([0.4, 0.3, 0.2, 0.1])
    x = np.log(probs)
    counts = np.zeros(4)
    for s in range(draws):
        counts[sample_row(x, 1.0, -1, 1.0, 0.0, 10_000 + s, 17).token] += 1
    p = chisquare(counts, probs * draws).pvalue
    return [] if p > 1e-4 else [f"race frequencies {counts} reject w/Z (p={p:.2e})"]


def _int_mask_bytes(ids, nbytes):
    """Bytes of the integer sum(2^i for i in ids), least significant byte first: token i lands at
    bit i % 8 of byte i // 8 by positional notation, with no bit-packing routine involved."""
    v = 0
    for i in ids:
        v |= 1 << int(i)
    return list(v.to_bytes(nbytes, "little"))


def pin_support_bitmask(support_bitmask, sample_row, rng_seed=2, cases=300):
    """The bitmask of a support (vLLM article, "How it works" step 2: a bit-packed mask of
    ceil(V / 8) bytes per row). The pages' tie example keeps ids {0, 1, 2} of V = 5, so its mask
    is the single byte 0b111 = 7; random tiny rows compare the mask of the oracle's support with
    the integer image of the brute-force support, zero-padded."""
    fails = []
    g = json.load(open(os.path.join(GOLDEN, "tie_example.json")))
    x = np.log(np.array(g["probs"], dtype=np.float32)).astype(np.float32).astype(np.float64)
    r = sample_row(x, 1.0, g["top_k"], g["top_p"], 0.0, 0, 0)
    got = support_bitmask(r.support, len(x)).tolist()
    if got != [7]:
        fails.append(f"tie example mask {got} != [7]")
    rng = np.random.default_rng(rng_seed)
    for _ in range(cases):
        V = int(rng.integers(1, 40))
        xs = [float(v) for v in rng.choice(LEVELS, V)]
        if all(v == -math.inf for v in xs):
            continue
        k = int(rng.integers(0, V + 2))
        p = float(rng.choice([0.0, 0.3, 0.7, 1.0]))
        S, near = brute_force(xs, 1.0, k, p, 0.0)
        if near:
            continue
        nbytes = (V + 7) // 8 + int(rng.integers(0, 3))
        r = sample_row(np.array(xs), 1.0, k, p, 0.0, 0, 0)
        got = support_bitmask(r.support, V, nbytes).tolist()
        want = _int_mask_bytes(S, nbytes)
        if got != want:
            fails.append(f"mask {got} != {want} for x={xs} k={k} p={p}")
            break
    return fails


def pin_replay(replay_row, sample_row, rng_seed=4, cases=200):
    """The replay of a support under new logits (vLLM article, section "RL training side:
    computing pi_theta with the mask": the training logits masked to the support, then the
    log-softmax at the sampled token).
    - The pages' tie example replayed on its own logits gives the closed forms ln 1/2, ln 1/4,
      ln 1/4, and -inf for a token outside the support.
    - Random rows against the page's recipe run with a library routine: scipy's log_softmax of
      the logits divided by T with every token outside the support set to -inf.
    - Replaying the oracle sampler's own support on the same logits reproduces its logprobs.
    - Adding a constant to every logit changes nothing."""
    from scipy.special import log_softmax
    fails = []
    g = json.load(open(os.path.join(GOLDEN, "tie_example.json")))
    x = np.log(np.array(g["probs"], dtype=np.float32)).astype(np.float32).astype(np.float64)
    S = np.array(g["expected_support_ids"])
    want = {0: math.log(0.5), 1: math.log(0.25), 2: math.log(0.25), 3: -math.inf}
    for tok, w in want.items():
        r = replay_row(x, 1.0, S, tok)
        if not (r.selected_logprob == w or abs(r.selected_logprob - w) < 1e-7):
            fails.append(f"tie example replay token {tok}: {r.selected_logprob} != {w}")
    rng = np.random.default_rng(rng_seed)
    for _ in range(cases):
        V = int(rng.integers(2, 60))
        xs = np.round(rng.standard_normal(V) * 3, 2)
        T = float(np.float32(rng.choice([0.5, 1.0, 1.7])))
        n = int(rng.integers(1, V + 1))
        S = rng.choice(V, n, replace=False)
        tok = int(rng.integers(0, V))
        keep = np.zeros(V, bool)
        keep[S] = True
        ref = log_softmax(np.where(keep, xs / T, -np.inf))
        r = replay_row(xs, T, S, tok)
        if not np.allclose(r.logprobs, ref[S], rtol=0, atol=1e-12):
            fails.append(f"replay logprobs differ from log_softmax for x={xs.tolist()} S={S} T={T}")
            break
        if not (r.selected_logprob == ref[tok] or abs(r.selected_logprob - ref[tok]) < 1e-12):
            fails.append(f"replay token {tok}: {r.selected_logprob} != {ref[tok]}")
            break
        shifted = replay_row(xs + 7.25, T, S, tok)
        if not np.allclose(shifted.logprobs, r.logprobs, rtol=0, atol=1e-9):
            fails.append("replay is not shift invariant")
            break
        k = int(rng.integers(1, V + 1))
        sr = sample_row(xs, T, k, float(rng.choice([0.6, 1.0])), 0.0, 1, 0)
        rr = replay_row(xs, T, sr.support, sr.token)
        if (not np.allclose(rr.logprobs, sr.logprobs.astype(np.float64), rtol=0, atol=2e-6)
                or abs(rr.selected_logprob - float(sr.logprobs[list(sr.support).index(sr.token)])) > 2e-6):
            fails.append(f"replay of the sampler's own support differs for x={xs.tolist()}")
            break
    return fails


def pin_support_csr(support_csr, rng_seed=6, cases=100):
    """The CSR layout of packed supports (sglang PR #40986, "Limitations": a transfer sized by
    the realized support instead of the packed capacity). Checked by properties that hold for any
    layout of this kind: offsets start at 0 and step by each row's length (clamped to [0, W]),
    the payload has offsets[R] entries, and cutting the payload at the offsets gives back every
    row's packed prefix, ids and logprobs alike; a hand-made three-row case is written out."""
    fails = []
    ids = np.array([[7, 3, 9, 0], [1, 2, 0, 0], [5, 6, 8, 4]], np.int32)
    lps = np.array([[-0.5, -1, -2, 0], [-0.1, -3, 0, 0], [-1, -1, -1, -1]], np.float32)
    off, cid, clp = support_csr(np.array([3, 0, 4], np.int32), ids, lps)
    if off.tolist() != [0, 3, 3, 7] or cid.tolist() != [7, 3, 9, 5, 6, 8, 4]:
        fails.append(f"three-row CSR {off.tolist()} {cid.tolist()}")
    if clp is None or clp.tolist() != [-0.5, -1, -2, -1, -1, -1, -1]:
        fails.append(f"three-row CSR logprobs {clp}")
    rng = np.random.default_rng(rng_seed)
    for _ in range(cases):
        R, W = int(rng.integers(0, 9)), int(rng.integers(1, 12))
        lengths = rng.integers(-2, W + 3, R).astype(np.int32)
        packed = rng.integers(0, 1000, (R, W)).astype(np.int32)
        lp = rng.standard_normal((R, W)).astype(np.float32)
        off, cid, clp = support_csr(lengths, packed, lp)
        n = [min(max(int(x), 0), W) for x in lengths]
        if off[0] != 0 or any(off[j + 1] - off[j] != n[j] for j in range(R)):
            fails.append(f"offsets {off.tolist()} for lengths {lengths.tolist()} W={W}")
            break
        if cid.size != off[-1] or clp.size != off[-1]:
            fails.append("payload size differs from offsets[R]")
            break
        for j in range(R):
            if (cid[off[j]:off[j + 1]].tolist() != packed[j, :n[j]].tolist()
                    or clp[off[j]:off[j + 1]].tolist() != lp[j, :n[j]].tolist()):
                fails.append(f"row {j} of the payload differs")
                break
    return fails
