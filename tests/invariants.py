"""Output invariants of one sampler call; applied to the oracle and to the HIP library alike.

Sources: sglang PR #40986 ("Checks removed": 0 <= length <= packed width, greedy rows width 1;
"Correctness": the selected logprob equals the token's support logprob; "Testing": the sampled
token lies in its support) and sglang PR #36630 summary ("Implementation breakdown": the support
is every token with positive post-filter weight, ties at a cutoff are all kept).
"""
from __future__ import annotations

import numpy as np

OK, OVERFLOW, NO_SUPPORT, NONFINITE, INVALID = 0, 1, 2, 3, 4


def check_invariants(tokens, row_status, packed_ids, logprobs, lengths, selected_logprob,
                     optin_rows, W, x_rows, temperature, rows=None):
    """Return a list of violations. ``x_rows(r)`` gives the exact float64 logits of row r.
    ``rows`` restricts the per-row checks to a subset (sampled checks)."""
    errs = []
    B = len(tokens)
    R = len(optin_rows)
    lengths = np.asarray(lengths)
    if R and (lengths.min() < 0 or lengths.max() > W):
        errs.append("length outside [0, W]")
    check = set(range(B)) if rows is None else set(int(r) for r in rows)
    # A slot is valid iff its row is in range and exceeds every earlier entry (the boundary's
    # contract for optin_rows); an invalid slot has length 0 and a NaN selected logprob.
    slot, running = {}, None
    for j in range(R):
        e = int(optin_rows[j])
        if 0 <= e < B and (running is None or e > running):
            slot[e] = j
        elif lengths[j] != 0 or not np.isnan(selected_logprob[j]):
            errs.append(f"slot {j}: invalid slot with length {lengths[j]} and selected logprob "
                        f"{selected_logprob[j]}")
        running = e if running is None else max(running, e)
    for r in sorted(check):
        st = int(row_status[r])
        tok = int(tokens[r])
        x = x_rows(r)
        if st >= NO_SUPPORT:
            if tok != -1:
                errs.append(f"row {r}: status {st} but token {tok}")
            if r in slot and lengths[slot[r]] != 0:
                errs.append(f"row {r}: status {st} but capture length {lengths[slot[r]]}")
            continue
        if not (0 <= tok < x.size) or not np.isfinite(x[tok]):
            errs.append(f"row {r}: token {tok} is not a finite-logit id")
            continue
        if st == OVERFLOW and r not in slot:
            errs.append(f"row {r}: OVERFLOW without capture")
        if r not in slot:
            continue
        j = slot[r]
        n = int(lengths[j])
        ids = np.asarray(packed_ids[j, :n])
        lp = np.asarray(logprobs[j, :n], dtype=np.float32) if logprobs is not None else None
        if n < 1:
            errs.append(f"row {r}: captured OK row with length 0")
            continue
        if np.unique(ids).size != n or ids.min() < 0 or ids.max() >= x.size:
            errs.append(f"row {r}: packed ids not distinct valid ids")
            continue
        xs = x[ids]
        if np.any(np.diff(xs) > 0):
            errs.append(f"row {r}: packed ids not in logit-descending order")
        tie = np.nonzero(np.diff(xs) == 0)[0]
        if tie.size and np.any(ids[tie + 1] < ids[tie]):
            errs.append(f"row {r}: tied ids not ascending")
        if float(temperature[r]) == 0.0:
            if n != 1 or (lp is not None and lp[0] != 0.0) or ids[0] != tok:
                errs.append(f"row {r}: greedy capture is not [token] with logprob 0")
        if st == OK:
            # The full support is packed: the token is in it, no tie group is split at the edge
            # (a greedy row is width 1 by definition, so its tie check is skipped).
            if tok not in ids:
                errs.append(f"row {r}: token {tok} outside its support")
            edge = xs[-1] if float(temperature[r]) > 0.0 else -np.inf
            if edge > -np.inf and np.count_nonzero(x == edge) != np.count_nonzero(xs == edge):
                errs.append(f"row {r}: tie group split at the support edge")
            if edge > -np.inf and np.count_nonzero(x > edge) != np.count_nonzero(xs > edge):
                errs.append(f"row {r}: a token above the edge is missing")
            if lp is not None:
                if np.any(np.diff(lp.astype(np.float64)) > 0):
                    errs.append(f"row {r}: logprobs increase along the row")
                tot = np.sum(np.exp(lp.astype(np.float64)))
                if abs(tot - 1.0) > 1e-5:
                    errs.append(f"row {r}: sum exp(logprobs) = {tot!r}")
                pos = np.nonzero(ids == tok)[0][0]
                if np.float32(selected_logprob[j]).tobytes() != np.float32(lp[pos]).tobytes():
                    errs.append(f"row {r}: selected logprob != support logprob of the token")
        elif st == OVERFLOW and n != W:
            errs.append(f"row {r}: OVERFLOW with length {n} != W")
    return errs
