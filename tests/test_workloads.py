"""The seeded input generator reproduces the recorded bytes of every workload (no GPU)."""
import json
import os

import numpy as np
import pytest

from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_workload

DIG = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                  "workload_digests.json")))


@pytest.mark.parametrize("index", [1, 2, 3, 4, 5, 6])
def test_workload_digest(index):
    wl = make_workload(index)
    d = DIG[str(index)]
    assert (wl.B, wl.V, wl.dtype, wl.R, wl.W) == (d["B"], d["V"], d["dtype"], d["R"], d["W"])
    assert wl.digest() == d["sha256"]


def test_workload_shapes_follow_the_recipe():
    wl = make_workload(3)
    x = bf16_bits_to_f32(wl.logits[:4])
    assert np.all(x * 8 == np.round(x * 8))  # the 0.125 grid survives the bfloat16 cast
    assert 0.6 <= wl.temperature.min() and wl.temperature.max() <= 1.2
    wl5 = make_workload(5)
    assert np.count_nonzero(wl5.temperature == 0) == 102 and wl5.R == 256
    assert np.all(np.diff(wl5.optin_rows) > 0)
    wl6 = make_workload(6)
    assert np.all(wl6.top_k == -1) and np.count_nonzero(wl6.min_p == 0) == wl6.B // 2


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38], np.float32)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0; 1 + 3*2^-8 -> 1 + 2^-6.
    assert bf16_bits_to_f32(f32_to_bf16_bits(x)).tolist()[:4] == [1.0, 1.0, 1.015625, -2.5]
