"""Pins of the oracle's input decode and of its race generator (no GPU).

* bfloat16 -> float64 (``oracle.sampler.decode_logits``): a bfloat16 value is the upper half of
  a binary32 value (1 sign bit, 8 exponent bits with bias 127, 7 fraction bits). Fixed patterns
  are checked against values written out from that format, and every one of the 65536 patterns
  against torch's CPU bfloat16 -> float32 conversion (an independent implementation).
* Philox4x32-10 (``oracle.philox.philox4`` with w = 32): the known-answer vectors that the
  generator's authors publish with their Random123 library (file ``kat_vectors``, lines
  ``philox4x32 10 <counter x4> <key x2> <output x4>``), for Salmon, Moraes, Dror and Shaw,
  "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11.
* The race uniform's bit mapping (``oracle.philox.token_uniforms``): counter (id / 4, 0,
  position lo, position hi), key (seed lo, seed hi), output word id % 4, u = (2 (word >> 9) + 1)
  / 2^24, checked on the all-zero known-answer block written out by hand.
Each pin is shown to fail on a planted mistake.
"""
import inspect

import numpy as np
import pytest

from oracle import philox as ophilox
from oracle import sampler as osampler

# (counter words, key words, output words), Random123 kat_vectors, Philox4x32 with 10 rounds.
PHILOX4X32_10_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]

# bfloat16 bit pattern -> exact value, from the format: sign, biased exponent, 7 fraction bits.
BF16_PATTERNS = [
    (0x3F80, 1.0),                      # exponent 127, fraction 0
    (0xBF80, -1.0),
    (0x0000, 0.0),
    (0x4000, 2.0),
    (0x4049, 3.140625),                 # 2 * (1 + 73/128)
    (0xC2F7, -123.5),                   # -(2^6) * (1 + 119/128)
    (0x3E00, 0.125),
    (0x0001, 2.0 ** -133),              # smallest subnormal: 2^-126 * 2^-7
    (0x007F, 127 * 2.0 ** -133),        # largest subnormal
    (0x0080, 2.0 ** -126),              # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),  # largest finite
    (0xFF7F, -(2.0 - 2.0 ** -7) * 2.0 ** 127),
    (0x7F80, np.inf),
    (0xFF80, -np.inf),
]


def pin_bf16_patterns(decode):
    fails = []
    for bits, want in BF16_PATTERNS:
        got = float(decode(np.array([bits], np.uint16), "bf16")[0])
        if got != want:
            fails.append(f"{bits:#06x}: {got!r} != {want!r}")
    neg0 = float(decode(np.array([0x8000], np.uint16), "bf16")[0])
    if not (neg0 == 0.0 and np.signbit(neg0)):
        fails.append(f"0x8000: {neg0!r} is not -0")
    for bits in (0x7FC0, 0xFFC0, 0x7F81):
        if not np.isnan(decode(np.array([bits], np.uint16), "bf16")[0]):
            fails.append(f"{bits:#06x} is not NaN")
    return fails


def test_bf16_decode_fixed_patterns():
    assert pin_bf16_patterns(osampler.decode_logits) == []


def test_bf16_decode_all_patterns_match_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = osampler.decode_logits(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().double().numpy()
    both_nan = np.isnan(mine) & np.isnan(ref)
    same = (mine == ref) & (np.signbit(mine) == np.signbit(ref))
    assert np.all(both_nan | same)
    assert both_nan.sum() == 2 * 127  # exponent all ones, fraction nonzero, either sign


@pytest.mark.parametrize("old,new", [
    ("<< np.uint32(16)", "<< np.uint32(15)"),
    ("astype(np.uint32) << np.uint32(16)", "astype(np.uint32) << np.uint32(16) | np.uint32(1)"),
    ("bits.view(np.float32)", "(bits & np.uint32(0x7FFFFFFF)).view(np.float32)"),
])
def test_bf16_pin_catches_planted_mistakes(old, new):
    src = inspect.getsource(osampler.decode_logits)
    assert src.count(old) == 1
    ns = dict(vars(osampler))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    assert pin_bf16_patterns(ns["decode_logits"])


def pin_philox4x32(philox4):
    fails = []
    for ctr, key, want in PHILOX4X32_10_KAT:
        got = tuple(int(v) for v in philox4(ctr, key, w=32, rounds=10))
        if got != want:
            fails.append(f"counter {ctr}: {[hex(v) for v in got]}")
    return fails


def test_philox4x32_10_known_answers():
    assert pin_philox4x32(ophilox.philox4) == []


@pytest.mark.parametrize("which,flip", [(0, 1), (1, 1 << 31), (2, 4), (3, 1 << 16)])
def test_philox4x32_pin_detects_a_wrong_constant(monkeypatch, which, flip):
    bad = dict(ophilox.PARAMS)
    consts = list(bad[32])
    consts[which] ^= flip
    bad[32] = tuple(consts)
    monkeypatch.setattr(ophilox, "PARAMS", bad)
    assert pin_philox4x32(ophilox.philox4)


def test_philox4x32_pin_detects_a_wrong_round_count():
    assert pin_philox4x32(lambda c, k, w, rounds: ophilox.philox4(c, k, w=w, rounds=rounds - 1))


def _u_of_word(word):
    return (2.0 * (word >> 9) + 1.0) / 2.0 ** 24


def pin_token_uniforms(token_uniforms):
    fails = []
    # Seed 0, position 0, ids 0..3: counter (0, 0, 0, 0), key (0, 0), words of the first vector.
    want = [_u_of_word(w) for w in PHILOX4X32_10_KAT[0][2]]
    got = token_uniforms(np.arange(4), 0, 0)
    if got.tolist() != want:
        fails.append(f"zero block: {got.tolist()}")
    # Word 0x6627E8D5 >> 9 = 0x3313F4, so u = (2 * 0x3313F4 + 1) / 2^24, written out.
    if got[0] != (2 * 0x3313F4 + 1) / 16777216.0:
        fails.append("zero block word 0")
    # Counter (id >> 2, 0, position lo, position hi), key (seed lo, seed hi), word id & 3, on
    # words of the generator pinned by the known answers above.
    seed, pos = 0x0123456789ABCDEF, 0xFEDCBA9876543210
    ids = np.array([0, 5, 6, 7, 4 * 0x1234 + 2, 4 * 0x3FFFFFFF + 3], np.int64)
    got = token_uniforms(ids, seed, pos)
    for i, u in zip(ids.tolist(), got.tolist()):
        words = ophilox.philox4((i >> 2, 0, pos & 0xFFFFFFFF, pos >> 32),
                                (seed & 0xFFFFFFFF, seed >> 32), w=32, rounds=10)
        if u != _u_of_word(int(words[i & 3])):
            fails.append(f"id {i}: {u}")
    return fails


def test_race_uniform_mapping():
    assert pin_token_uniforms(ophilox.token_uniforms) == []


@pytest.mark.parametrize("old,new", [
    ("(ids >> _U64(2), np.zeros_like(ids),", "(ids >> _U64(2), np.ones_like(ids),"),
    ("key = (seed & 0xFFFFFFFF, seed >> 32)", "key = (seed >> 32, seed & 0xFFFFFFFF)"),
    ("np.full_like(ids, position & 0xFFFFFFFF),\n           np.full_like(ids, position >> 32))",
     "np.full_like(ids, position >> 32),\n           np.full_like(ids, position & 0xFFFFFFFF))"),
    ("sel = (ids & _U64(3))", "sel = (ids >> _U64(30) & _U64(3))"),
    ("(words >> _U64(9))", "(words >> _U64(8))"),
    ("(2.0 * k + 1.0)", "(2.0 * k)"),
])
def test_race_uniform_pin_catches_planted_mistakes(old, new):
    src = inspect.getsource(ophilox.token_uniforms)
    assert src.count(old) == 1, old
    ns = dict(vars(ophilox))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    assert pin_token_uniforms(ns["token_uniforms"])
