"""CPU oracle of the batched top-k / top-p / min-p sampler with support capture (test infrastructure).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check of the graft entry point and the CPU
baseline leg of the bench may import or call this package. The product path never does: it runs
entirely in the HIP library and fails loudly when that library is missing.

The method reaches an exactly defined result, so this file computes that definition directly,
one row at a time, in float64 on sorted data, with no blocking or fusion:

* sglang PR #36630 summary (prhub), "Implementation breakdown" items 2-3 and the "Key code" tie
  test: the sampler's support is S = {i | w[i] > 0} of the post-filter weights; top-k and top-p
  are evaluated jointly on the same (unrenormalized) distribution and their kept sets are
  intersected; both filters are thresholds, so every token tied with the cutoff value is kept and
  the support can exceed k; top-p keeps the sorted tokens whose probability mass strictly before
  them is at most top_p; min-p is applied after top-k and top-p; the sampled token's logprob is
  log(w[y] / sum(w)) from the same capture.
* vLLM "Sampling Mask / Distribution Replay" article, "How it works" steps 1-2: excluded tokens
  carry -inf logits and a token survives only when its logit is finite; logprobs are normalized
  over the truncated nucleus (processed logprobs).
* sglang PR #40986, "Design" and "Checks removed": the packed capture holds
  min(realized support, packed width) entries; a wider support gets OVERFLOW status; a greedy row
  is width 1, length 1.
* Gaudi cookbook "topk-subset-sampler", "The fix": the token is drawn with the exponential race.

Readings taken where the pages are silent or disagree (each is a documented choice):
  R1 ties are judged on the logit value (p_i = p_j exactly when x_i = x_j for T > 0); -0 ties +0;
     the support order is (logit descending, token id ascending);
  R2 membership is by predicate in exact arithmetic, never by floating-point underflow of w;
  R3 top-p: keep tie group g iff C(g) <= top_p * Z, C(g) the mass of tokens with strictly larger
     logit, Z the mass of all finite tokens; top_p >= 1 disables the filter;
  R4 top_k <= 0 or top_k >= |finite tokens| disables the filter; top_k = 1 keeps a tied maximum;
  R5 min-p keeps w >= min_p (w relative to the maximum, so w_max = 1), evaluated in the log domain
     as (x - max) / T >= ln(min_p); min_p = 0 disables it; it runs after top-k and top-p;
  R6 temperature 0 is greedy: the first index of the maximum, support of width 1, logprob 0;
     a temperature must be 0 or a normal positive finite float32;
  R7 the race uses Philox4x32-10 uniforms keyed by (seed, position, token id), see
     ``oracle.philox.token_uniforms``; score = (x - max)/T - ln(-ln u); ties go to the lowest id;
  R8 any NaN or +inf logit makes the row NONFINITE; a row with no finite logit is NO_SUPPORT;
     invalid parameters (negative / non-finite / subnormal temperature, top_p or min_p NaN or
     outside [0, 1]) make it INVALID_PARAM; such rows return token -1 and an empty capture;
  R9 capture slot j is valid iff 0 <= optin_rows[j] < B and optin_rows[j] exceeds every earlier
     entry (so valid slots name distinct rows, in ascending order); invalid slots get length 0
     and a NaN selected logprob;
  R10 logprobs are normalized over the full support even when the packed prefix is clamped;
  R11 the exact fallback for a support wider than the packed width is a bit-packed mask of
     ceil(V / 8) bytes per row (vLLM article, "How it works" step 2); the page does not fix the
     bit order: token i is bit i % 8 of byte i // 8 (least significant bit first), and the mask
     is written for OVERFLOW slots only.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from .philox import token_uniforms

ROW_OK, ROW_OVERFLOW, ROW_NO_SUPPORT, ROW_NONFINITE, ROW_INVALID_PARAM = 0, 1, 2, 3, 4

FLT_MIN = float(np.finfo(np.float32).tiny)

RACE_TIE_EPS = 1e-6   # top-two race scores closer than this (log domain) are reported, not failed
TOP_P_EPS = 1e-5      # |C(g)/Z - top_p| within this is reported, not failed
MIN_P_EPS = 1e-6      # |(x_g - max)/T - ln(min_p)| within this is reported, not failed


@dataclasses.dataclass
class RowResult:
    status: int
    token: int
    support: np.ndarray          # int64 ids in (logit desc, id asc) order; full support
    logprobs: np.ndarray         # float32, aligned with ``support``
    race_gap: float = np.inf     # top-1 minus top-2 race score (inf if |S| < 2)
    top_p_flag: bool = False
    min_p_flag: bool = False

    @property
    def L(self) -> int:
        return int(self.support.size)

    @property
    def flagged(self) -> bool:
        return self.top_p_flag or self.min_p_flag or self.race_gap <= RACE_TIE_EPS


def decode_logits(row, dtype: str) -> np.ndarray:
    """Exact float64 image of one logits row; ``row`` is float32 or raw bfloat16 bits (uint16)."""
    if dtype == "f32":
        return np.asarray(row, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(row, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def params_valid(T: float, top_p: float, min_p: float) -> bool:
    T, top_p, min_p = float(np.float32(T)), float(np.float32(top_p)), float(np.float32(min_p))
    if not np.isfinite(T) or T < 0.0 or (0.0 < T < FLT_MIN):
        return False
    if not (0.0 <= top_p <= 1.0):  # False for NaN
        return False
    if not (0.0 <= min_p <= 1.0):
        return False
    return True


def _empty(status: int) -> RowResult:
    return RowResult(status, -1, np.zeros(0, np.int64), np.zeros(0, np.float32))


def sample_row(x: np.ndarray, T: float, top_k: int, top_p: float, min_p: float,
               seed: int, position: int) -> RowResult:
    """Sample one row; ``x`` is the exact float64 logits row."""
    T = float(np.float32(T))
    top_p = float(np.float32(top_p))
    min_p = float(np.float32(min_p))
    top_k = int(top_k)
    if not params_valid(T, top_p, min_p):
        return _empty(ROW_INVALID_PARAM)
    if np.isnan(x).any() or np.isposinf(x).any():
        return _empty(ROW_NONFINITE)
    finite_ids = np.nonzero(x > -np.inf)[0]
    if finite_ids.size == 0:
        return _empty(ROW_NO_SUPPORT)

    xf = x[finite_ids]
    if T == 0.0:
        # Greedy (R6): first index of the maximum, a width-1 support with logprob 0.
        tok = int(finite_ids[np.argmax(xf)])
        return RowResult(ROW_OK, tok, np.array([tok], np.int64), np.zeros(1, np.float32))

    # Sort by (logit descending, id ascending) (R1). -0.0 and +0.0 compare equal in lexsort.
    order = np.lexsort((finite_ids, -xf))
    ids = finite_ids[order]
    s = xf[order]
    n = s.size

    # Unrenormalized weights relative to the maximum and their exclusive prefix (R3).
    scaled = (s - s[0]) / T
    w = np.exp(scaled)
    incl = np.cumsum(w)
    C = np.concatenate(([0.0], incl[:-1]))
    Z = incl[-1]

    # Tie groups: maximal runs of equal logits; a_g is each group's first sorted position.
    starts = np.concatenate(([0], np.nonzero(s[1:] != s[:-1])[0] + 1))
    k_eff = top_k if 1 <= top_k < n else n
    pass_k = starts < k_eff
    pass_p = np.ones(starts.size, bool) if top_p >= 1.0 else (C[starts] <= top_p * Z)
    if min_p > 0.0:
        ln_min_p = np.log(min_p)
        pass_m = scaled[starts] >= ln_min_p
    else:
        pass_m = np.ones(starts.size, bool)
    keep = pass_k & pass_p & pass_m
    # Every predicate is monotone along the sorted order, so the kept groups form a prefix.
    first_fail = np.nonzero(~keep)[0]
    L = n if first_fail.size == 0 else int(starts[first_fail[0]])
    assert L >= 1 and keep[: np.searchsorted(starts, L)].all()

    # Support mass and logprobs in the log domain (R2): lp = (x - max)/T - ln(Z_S).
    Z_S = np.sum(w[:L])
    lp64 = scaled[:L] - np.log(Z_S)
    lp = lp64.astype(np.float32)

    # Exponential race over the support (R7).
    u = token_uniforms(ids[:L], seed, position)
    score = scaled[:L] - np.log(-np.log(u))
    best = np.max(score)
    token = int(np.min(ids[:L][score == best]))
    if L >= 2:
        top2 = np.partition(score, L - 2)[L - 2:]
        race_gap = float(top2.max() - top2.min())
    else:
        race_gap = np.inf

    # Boundary reports (near-threshold rows are counted, not failed). The first tie group is
    # never near a boundary: no mass precedes it and its weight is exactly 1 in any arithmetic,
    # so top-p and min-p keep it exactly whatever the rounding.
    later = np.arange(starts.size) > 0
    top_p_flag = False
    if top_p < 1.0:
        cand = pass_k & pass_m & later
        top_p_flag = bool(np.any(np.abs(C[starts][cand] / Z - top_p) <= TOP_P_EPS))
    min_p_flag = False
    if min_p > 0.0:
        cand = pass_k & pass_p & later
        min_p_flag = bool(np.any(np.abs(scaled[starts][cand] - np.log(min_p)) <= MIN_P_EPS))

    return RowResult(ROW_OK, token, ids[:L].astype(np.int64), lp, race_gap, top_p_flag, min_p_flag)


def support_bitmask(support: np.ndarray, V: int, nbytes: Optional[int] = None) -> np.ndarray:
    """R11: the support as a bit-packed mask, token i at bit i % 8 of byte i // 8, zero-padded to
    ``nbytes`` bytes (default ceil(V / 8))."""
    keep = np.zeros(V, dtype=bool)
    keep[np.asarray(support, dtype=np.int64)] = True
    packed = np.packbits(keep, bitorder="little")
    n = packed.size if nbytes is None else int(nbytes)
    out = np.zeros(n, np.uint8)
    out[:packed.size] = packed
    return out


@dataclasses.dataclass
class BatchResult:
    tokens: np.ndarray            # int32 [B]
    row_status: np.ndarray        # int8 [B]; OVERFLOW only for captured rows
    packed_ids: np.ndarray        # int32 [R, W]; -1 past each length
    logprobs: np.ndarray          # float32 [R, W]; NaN past each length
    lengths: np.ndarray           # int32 [R]
    selected_logprob: np.ndarray  # float32 [R]
    slot_valid: np.ndarray        # bool [R]
    rows: List[RowResult]
    support_bits: Optional[np.ndarray] = None  # uint8 [R, bits_ld]; zero except OVERFLOW slots


def slot_validity(optin_rows: np.ndarray, B: int) -> np.ndarray:
    """R9: a capture slot is valid iff its row is in range and exceeds every earlier entry."""
    e = np.asarray(optin_rows, dtype=np.int64)
    ok = (e >= 0) & (e < B)
    if e.size > 1:
        ok[1:] &= e[1:] > np.maximum.accumulate(e)[:-1]
    return ok


def sample_with_mask(logits: np.ndarray, dtype: str, temperature, top_k, top_p, min_p,
                     optin_rows, seeds, positions, W: int,
                     rows: Optional[np.ndarray] = None,
                     bits_ld: Optional[int] = None,
                     row_results: Optional[dict] = None) -> BatchResult:
    """Oracle of the whole batched call.

    ``logits``: float32 [B, V] or uint16 [B, V] of bfloat16 bits. Returns every output of the
    library call plus the per-row diagnostics. With ``rows`` given, only those rows are sampled
    (the others keep token -1 / status -1 and empty captures): used for sampled checks at full
    size. With ``bits_ld`` the support of every OVERFLOW slot is also returned as a bitmask row
    of that many bytes (R11). ``row_results`` maps row index -> RowResult already computed by
    ``sample_row`` for that row (e.g. by worker processes); those rows are assembled, not
    sampled again."""
    B = logits.shape[0]
    R = len(optin_rows)
    tokens = np.full(B, -1, np.int32)
    status = np.full(B, -1, np.int8)
    packed = np.full((R, W), -1, np.int32)
    lps = np.full((R, W), np.nan, np.float32)
    lengths = np.zeros(R, np.int32)
    sel = np.full(R, np.nan, np.float32)
    V = logits.shape[1]
    bits = None if bits_ld is None else np.zeros((R, int(bits_ld)), np.uint8)
    valid = slot_validity(optin_rows, B)
    slot_of = {int(optin_rows[j]): j for j in range(R) if valid[j]}
    todo = range(B) if rows is None else [int(r) for r in rows]
    results: List[Optional[RowResult]] = [None] * B
    for r in todo:
        if row_results is not None and r in row_results:
            res = row_results[r]
        else:
            res = sample_row(decode_logits(logits[r], dtype), temperature[r], top_k[r], top_p[r],
                             min_p[r], int(seeds[r]), int(positions[r]))
        results[r] = res
        tokens[r] = res.token
        st = res.status
        j = slot_of.get(r)
        if j is not None and res.status == ROW_OK:
            n = min(res.L, W)
            packed[j, :n] = res.support[:n]
            lps[j, :n] = res.logprobs[:n]
            lengths[j] = n
            pos = int(np.nonzero(res.support == res.token)[0][0])
            sel[j] = res.logprobs[pos]
            if res.L > W:
                st = ROW_OVERFLOW
                if bits is not None:
                    bits[j] = support_bitmask(res.support, V, bits_ld)
        status[r] = st
    return BatchResult(tokens, status, packed, lps, lengths, sel, valid, results, bits)
