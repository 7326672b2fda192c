"""The parity harness itself fails on plausible GPU mistakes (no GPU: the oracle's own output
stands in for the library's, then is broken on purpose)."""
import copy
import json
import os

import numpy as np

import oracle
from tests.parity import BITS_SENTINEL, compare, compare_bits


def _tie_batch():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tie_example.json")))
    B = 8
    x = np.tile(np.log(np.array(g["probs"], np.float32)), (B, 1)).astype(np.float32)
    T = np.ones(B, np.float32)
    k = np.full(B, g["top_k"], np.int32)
    p = np.full(B, g["top_p"], np.float32)
    mp = np.zeros(B, np.float32)
    opt = np.arange(B, dtype=np.int32)
    ref = oracle.sample_with_mask(x, "f32", T, k, p, mp, opt, np.arange(B, dtype=np.uint64),
                                  np.zeros(B, np.uint64), 4)
    got = {"tokens": ref.tokens.copy(), "row_status": ref.row_status.copy(),
           "packed_ids": ref.packed_ids.copy(), "lengths": ref.lengths.copy(),
           "logprobs": ref.logprobs.copy(), "selected_logprob": ref.selected_logprob.copy()}
    return got, ref, opt


def test_identical_outputs_pass():
    got, ref, opt = _tie_batch()
    errs, stats = compare(got, ref, opt)
    assert errs == [] and stats["rows"] == 8


def test_dropped_tied_token_fails():
    got, ref, opt = _tie_batch()
    got["lengths"][3] = 2  # the tied id 2 is lost
    assert compare(got, ref, opt)[0]


def test_swapped_tie_order_fails():
    got, ref, opt = _tie_batch()
    got["packed_ids"][5, [1, 2]] = got["packed_ids"][5, [2, 1]]
    assert compare(got, ref, opt)[0]


def test_logprob_drift_fails_and_small_noise_passes():
    got, ref, opt = _tie_batch()
    got2 = copy.deepcopy(got)
    got["logprobs"][0, 1] += 2e-5
    assert compare(got, ref, opt)[0]
    got2["logprobs"][0, 1] += 2e-6
    got2["selected_logprob"][0] += 2e-6
    assert compare(got2, ref, opt)[0] == []


def test_wrong_token_and_status_fail():
    got, ref, opt = _tie_batch()
    got["tokens"][1] = 4
    assert compare(got, ref, opt)[0]
    got, ref, opt = _tie_batch()
    got["row_status"][2] = 1
    assert compare(got, ref, opt)[0]


def test_status_rows_compare_nan_selected_logprob_as_equal():
    x = np.array([[0.0, np.nan, 1.0], [0.5, 0.25, 0.0]], np.float32)
    one = np.ones(2, np.float32)
    ref = oracle.sample_with_mask(x, "f32", one, np.full(2, 2, np.int32), one, 0 * one,
                                  np.arange(2, dtype=np.int32), np.arange(2, dtype=np.uint64),
                                  np.zeros(2, np.uint64), 4)
    got = {"tokens": ref.tokens.copy(), "row_status": ref.row_status.copy(),
           "packed_ids": ref.packed_ids.copy(), "lengths": ref.lengths.copy(),
           "logprobs": ref.logprobs.copy(), "selected_logprob": ref.selected_logprob.copy()}
    assert ref.row_status.tolist() == [3, 0] and np.isnan(ref.selected_logprob[0])
    assert compare(got, ref, np.arange(2))[0] == []
    got["selected_logprob"][1] = np.nan
    assert compare(got, ref, np.arange(2))[0]


def _bits_batch():
    # The tie example with W = 2: support {0, 1, 2} overflows, bitmask byte 0b111.
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tie_example.json")))
    B = 4
    x = np.tile(np.log(np.array(g["probs"], np.float32)), (B, 1)).astype(np.float32)
    T = np.ones(B, np.float32)
    T[3] = 0.0  # greedy: width 1, never overflows
    k = np.full(B, g["top_k"], np.int32)
    p = np.full(B, g["top_p"], np.float32)
    opt = np.arange(B, dtype=np.int32)
    ref = oracle.sample_with_mask(x, "f32", T, k, p, np.zeros(B, np.float32), opt,
                                  np.arange(B, dtype=np.uint64), np.zeros(B, np.uint64), 2,
                                  bits_ld=16)
    bits = ref.support_bits.copy()
    bits[3] = BITS_SENTINEL
    got = {"row_status": ref.row_status.copy(), "support_bits": bits}
    return got, ref, opt


def test_bitmask_harness():
    got, ref, opt = _bits_batch()
    assert ref.support_bits[0, 0] == 7 and not ref.support_bits[0, 1:].any()
    errs, n = compare_bits(got, ref, opt)
    assert errs == [] and n == 3
    bad = copy.deepcopy(got)
    bad["support_bits"][1, 0] ^= 0x08  # an extra token
    assert compare_bits(bad, ref, opt)[0]
    bad = copy.deepcopy(got)
    bad["support_bits"][2, 0] = 3  # a dropped tied token
    assert compare_bits(bad, ref, opt)[0]
    bad = copy.deepcopy(got)
    bad["support_bits"][3, 5] = 0  # a row without OVERFLOW written
    assert compare_bits(bad, ref, opt)[0]


def test_race_report_exempts_only_the_token():
    got, ref, opt = _tie_batch()
    ref.rows[2].race_gap = 0.0  # the oracle reports a race near-tie on row 2
    got["tokens"][2] = (got["tokens"][2] + 1) % 3
    got["selected_logprob"][2] = got["logprobs"][2, (got["tokens"][2]) % 3]
    errs, stats = compare(got, ref, opt)
    assert errs == [] and stats["race_flagged"] == 1
    got["packed_ids"][2, [1, 2]] = got["packed_ids"][2, [2, 1]]  # its support is still checked
    assert compare(got, ref, opt)[0]
    got, ref, opt = _tie_batch()
    ref.rows[2].race_gap = 0.0
    got["logprobs"][2, 0] += 1e-3
    assert compare(got, ref, opt)[0]


def test_top_p_report_exempts_the_support_but_not_an_equal_supports_token():
    got, ref, opt = _tie_batch()
    ref.rows[4].top_p_flag = True
    got["lengths"][4] = 2  # a boundary group decided the other way: exempt
    errs, stats = compare(got, ref, opt)
    assert errs == [] and stats["top_p_flagged"] == 1 and stats["support_exempt"] == 1
    got, ref, opt = _tie_batch()
    ref.rows[4].top_p_flag = True
    got["tokens"][4] = [t for t in (0, 1, 2) if t != got["tokens"][4]][0]  # same support
    assert compare(got, ref, opt)[0]
    got, ref, opt = _tie_batch()
    ref.rows[4].min_p_flag = True
    got["logprobs"][4, 1] += 1e-3  # same support, wrong logprob
    assert compare(got, ref, opt)[0]
