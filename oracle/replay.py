"""CPU oracle of the replay of a captured support under new logits (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by the tests, the graft smoke check and the bench's CPU
baseline leg, never by the product path.

vLLM "Sampling Mask / Distribution Replay" article, section "RL training side: computing pi_theta
with the mask": the training side restricts its own logits to the support the sampler returned
(every other token set to -inf) and takes the log-softmax at the sampled token, so that pi_theta
and pi_old are normalized over the same token set. The definition, written out in float64:

    lp(a) = z_a - ln sum_{i in S} exp(z_i),   z_i = (x_i - m) / T,   m = max_{i in S} x_i

Readings taken where the page is silent (each is a documented choice):
  R12 the page applies the mask to raw logits; pi_old is the sampler's processed logprob, which
      divides by the temperature first. The replay takes a per-row temperature T > 0 and divides
      by it (T = 1 is the page's recipe exactly); T <= 0, non-finite or subnormal is invalid
      (the page rejects replay for temperature <= 0);
  R13 a token outside S has logprob -inf (what the masked log-softmax gives); a support logit
      that is NaN or +inf makes the row NONFINITE, a support whose logits are all -inf makes it
      NO_SUPPORT, and both return NaN;
  R14 the support of a row is the set of its ids (the sampler writes distinct ids).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from .sampler import FLT_MIN, ROW_OK, ROW_NO_SUPPORT, ROW_NONFINITE, ROW_INVALID_PARAM


@dataclasses.dataclass
class ReplayRow:
    status: int
    selected_logprob: float     # float64; NaN unless status is OK
    logprobs: np.ndarray        # float64, aligned with the given ids; NaN unless OK


def replay_row(x: np.ndarray, T: float, support: np.ndarray, token: int) -> ReplayRow:
    """Masked log-softmax of row ``x`` (float64, decoded exactly) over ``support`` at ``token``,
    plus the logprob of every support id in the given order."""
    support = np.asarray(support, dtype=np.int64)
    V = x.size
    nan = lambda: ReplayRow(ROW_INVALID_PARAM, np.nan, np.full(support.size, np.nan))
    T = float(np.float32(T))
    if not (np.isfinite(T) and T >= FLT_MIN):
        return nan()
    if support.size == 0 or np.any(support < 0) or np.any(support >= V) or not (0 <= token < V):
        return nan()
    xs = x[support]
    if np.any(np.isnan(xs)) or np.any(xs == np.inf):
        return ReplayRow(ROW_NONFINITE, np.nan, np.full(support.size, np.nan))
    if np.all(xs == -np.inf):
        return ReplayRow(ROW_NO_SUPPORT, np.nan, np.full(support.size, np.nan))
    m = xs.max()
    z = (xs - m) / T
    lse = np.log(np.sum(np.exp((x[np.unique(support)] - m) / T)))  # R14: a set of ids
    lps = z - lse
    if np.any(support == token):
        sel = (x[token] - m) / T - lse
    else:
        sel = -np.inf
    return ReplayRow(ROW_OK, float(sel), lps)


def replay(logits: np.ndarray, dtype: str, temperature, packed_ids, lengths, tokens,
           capture_status: Optional[np.ndarray] = None,
           support_bits: Optional[np.ndarray] = None, rows=None):
    """Oracle of the batched replay call. Row j's support is its first lengths[j] packed ids, or,
    where capture_status[j] is OVERFLOW, the ids set in support_bits[j] (bit i % 8 of byte
    i // 8). Rows whose capture_status is 2 or more keep that status. Returns (selected logprob
    float32 [N], logprobs float32 [N, W] aligned with packed_ids, status int8 [N])."""
    from .sampler import decode_logits, ROW_OVERFLOW
    N, W = packed_ids.shape
    V = logits.shape[1]
    sel = np.full(N, np.nan, np.float32)
    lps = np.full((N, W), np.nan, np.float32)
    status = np.full(N, -1, np.int8)
    todo = range(N) if rows is None else [int(r) for r in rows]
    for j in todo:
        cs = ROW_OK if capture_status is None else int(capture_status[j])
        if cs >= 2:
            status[j] = cs
            continue
        n = int(lengths[j])
        if cs == ROW_OVERFLOW:
            if support_bits is None:
                status[j] = ROW_INVALID_PARAM
                continue
            keep = np.unpackbits(support_bits[j], bitorder="little")[:V].astype(bool)
            support = np.nonzero(keep)[0]
        else:
            if not (1 <= n <= W):
                status[j] = ROW_INVALID_PARAM
                continue
            support = packed_ids[j, :n]
        res = replay_row(decode_logits(logits[j], dtype), temperature[j], support, int(tokens[j]))
        status[j] = res.status
        sel[j] = res.selected_logprob
        if res.status == ROW_OK and 1 <= n <= W:
            ids = packed_ids[j, :n].astype(np.int64)
            if cs == ROW_OVERFLOW:  # the packed prefix of a wider support: its ids' logprobs
                pos = {int(i): k for k, i in enumerate(support)}
                lps[j, :n] = [res.logprobs[pos[int(i)]] if int(i) in pos else -np.inf for i in ids]
            else:
                lps[j, :n] = res.logprobs
    return sel, lps, status
