"""Comparison of a library call's outputs with the oracle's, element by element.

The bar: support ids, lengths and order bit-exact, tokens equal,
logprobs within 1e-5 absolute (or one float32 spacing at the value, where that is larger), except on rows the oracle reports as near a decision boundary
(top-p mass within 1e-5 of top_p, min-p within 1e-6, top-two race scores within 1e-6), which are
counted; each report exempts only the outputs it can change (see ``compare``).
"""
from __future__ import annotations

import numpy as np

from oracle.sampler import RACE_TIE_EPS

LOGPROB_ATOL = 1e-5


def logprob_tol(ref) -> np.ndarray:
    """The bound on a float32 logprob against the oracle's: 1e-5, or one float32 spacing at the
    reference value where that is larger (above 128 in magnitude, e.g. at temperatures near
    1e-3, float32 cannot hold a value to 1e-5, and a difference of 1e-7 in the float64 value
    before rounding can move it by one spacing)."""
    r = np.abs(np.asarray(ref, dtype=np.float32))
    return np.maximum(LOGPROB_ATOL, np.spacing(r).astype(np.float64))


def to_numpy_outputs(out) -> dict:
    """SampleOutput (torch) -> dict of numpy arrays."""
    return {
        "tokens": out.tokens.cpu().numpy(),
        "row_status": out.row_status.cpu().numpy(),
        "packed_ids": out.packed_ids.cpu().numpy(),
        "lengths": out.lengths.cpu().numpy(),
        "logprobs": None if out.logprobs is None else out.logprobs.cpu().numpy(),
        "selected_logprob": out.selected_logprob.cpu().numpy(),
        "support_bits": None if out.support_bits is None else out.support_bits.cpu().numpy(),
    }


BITS_SENTINEL = 0xA5  # what a bitmask row holds before the call; slots that do not overflow keep it


def compare_bits(got: dict, ref, optin_rows, rows=None):
    """Support bitmasks: bit-exact against the oracle on every OVERFLOW slot whose support is
    decided away from a filter boundary; every other valid slot's row left untouched. Returns
    (errors, number of bitmask rows checked)."""
    errs, n = [], 0
    bits = got["support_bits"]
    todo = None if rows is None else set(int(r) for r in rows)
    for j in range(len(optin_rows)):
        if not ref.slot_valid[j]:
            continue
        r = int(optin_rows[j])
        if todo is not None and r not in todo:
            continue
        res = ref.rows[r]
        if ref.row_status[r] == 1:
            if res.top_p_flag or res.min_p_flag:
                continue
            n += 1
            if not np.array_equal(bits[j], ref.support_bits[j]):
                diff = np.nonzero(np.unpackbits(bits[j] ^ ref.support_bits[j], bitorder="little"))[0]
                errs.append(f"slot {j} row {r}: bitmask differs at ids {diff[:8].tolist()} "
                            f"({diff.size} bits)")
        elif int(got["row_status"][r]) != 1 and not np.all(bits[j] == BITS_SENTINEL):
            errs.append(f"slot {j} row {r}: bitmask row written without OVERFLOW")
    return errs, n


def compare(got: dict, ref, optin_rows, rows=None):
    """Return (errors, stats). ``ref`` is an ``oracle.BatchResult``; ``rows`` limits the check
    to the rows the oracle computed.

    Each boundary report exempts only what it can change:
    * a race near-tie (top two scores within 1e-6) exempts the token alone; the support, its
      length, order and logprobs are still compared bit-exactly / within tolerance;
    * a top-p or min-p report (a tie group within the window of its filter's boundary) exempts
      the support (ids, length, logprobs, and an OK / OVERFLOW status that depends on the
      length); when the captured support still came out equal (and is not clamped), its
      logprobs, the token and the selected logprob are compared as usual.
    stats counts each kind of report apart ("race_flagged", "top_p_flagged", "min_p_flagged");
    "flagged" counts rows with any report."""
    errs = []
    stats = {"rows": 0, "flagged": 0, "race_flagged": 0, "top_p_flagged": 0, "min_p_flagged": 0,
             "support_exempt": 0, "overflow": 0, "exact_lp": 0, "lp_entries": 0,
             "max_lp_err": 0.0}
    B = len(got["tokens"])
    todo = range(B) if rows is None else [int(r) for r in rows]
    slot = {int(optin_rows[j]): j for j in range(len(optin_rows)) if ref.slot_valid[j]}
    for j in range(len(optin_rows)):
        if not ref.slot_valid[j]:
            if got["lengths"][j] != 0 or not np.isnan(got["selected_logprob"][j]):
                errs.append(f"invalid slot {j}: length {got['lengths'][j]}")
    for r in todo:
        rr = ref.rows[r]
        stats["rows"] += 1
        race_flag = rr.race_gap <= RACE_TIE_EPS
        support_flag = rr.top_p_flag or rr.min_p_flag
        stats["flagged"] += int(rr.flagged)
        stats["race_flagged"] += int(race_flag)
        stats["top_p_flagged"] += int(rr.top_p_flag)
        stats["min_p_flagged"] += int(rr.min_p_flag)
        gst, rst = int(got["row_status"][r]), int(ref.row_status[r])
        if gst != rst and not (support_flag and {gst, rst} == {0, 1}):
            errs.append(f"row {r}: status {gst} != {rst}")
            continue
        if rst == 1:
            stats["overflow"] += 1
        j = slot.get(r)
        # Whether this row's full support is known to equal the oracle's: for a captured row,
        # equal lengths and ids unless the packed prefix is clamped (OVERFLOW); for a row that
        # is not captured it is not visible.
        support_same = not support_flag
        if j is not None:
            n = int(ref.lengths[j])
            gn = int(got["lengths"][j])
            prefix_same = gn == n and np.array_equal(got["packed_ids"][j, :n], ref.packed_ids[j, :n])
            if support_flag:
                support_same = prefix_same and gst == rst != 1
                stats["support_exempt"] += int(not support_same)
            elif gn != n:
                errs.append(f"row {r}: length {gn} != {n} (L={rr.L})")
                continue
            elif not prefix_same:
                gi = got["packed_ids"][j, :n]
                bad = int(np.nonzero(gi != ref.packed_ids[j, :n])[0][0])
                errs.append(f"row {r}: packed ids differ first at {bad}: {gi[bad]} != "
                            f"{ref.packed_ids[j, bad]}")
                continue
            if support_same and got["logprobs"] is not None and n:
                d = np.abs(got["logprobs"][j, :n].astype(np.float64)
                           - ref.logprobs[j, :n].astype(np.float64))
                stats["max_lp_err"] = max(stats["max_lp_err"], float(d.max()))
                stats["exact_lp"] += int(np.count_nonzero(d == 0))
                stats["lp_entries"] += n
                tol = logprob_tol(np.where(np.isfinite(ref.logprobs[j, :n]), ref.logprobs[j, :n], 0.0))
                if np.any(d > tol) or not np.all(
                        np.isfinite(got["logprobs"][j, :n]) == np.isfinite(ref.logprobs[j, :n])):
                    errs.append(f"row {r}: logprob error {d.max():.3g}")
        elif support_flag:
            stats["support_exempt"] += 1
        if race_flag or not support_same:
            continue
        if int(got["tokens"][r]) != int(ref.tokens[r]):
            errs.append(f"row {r}: token {got['tokens'][r]} != {ref.tokens[r]} (gap {rr.race_gap:.3g})")
        if j is None:
            continue
        gs, rs = float(got["selected_logprob"][j]), float(ref.selected_logprob[j])
        if np.isnan(rs) or np.isnan(gs):
            if not (np.isnan(rs) and np.isnan(gs)):
                errs.append(f"row {r}: selected logprob {gs} vs {rs}")
        elif not abs(gs - rs) <= float(logprob_tol(rs if np.isfinite(rs) else 0.0)):
            errs.append(f"row {r}: selected logprob error {abs(gs - rs):.3g}")
    return errs, stats
