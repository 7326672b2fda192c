"""Philox counter-based generator, written from its published definition (test infrastructure).

Reference: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random Numbers: As
Easy as 1, 2, 3", SC'11, section 4 (the Philox bijection). One round maps a counter of N=4 words
(X0, X1, X2, X3) under a round key (K0, K1) as follows, with (hi_a, lo_a) = M0 * X0 and
(hi_b, lo_b) = M1 * X2 taken as double-width products:

    X' = (hi_b ^ X1 ^ K0,  lo_b,  hi_a ^ X3 ^ K1,  lo_a)

and the key is bumped by the Weyl constants (W0, W1) modulo 2**w between rounds. Philox4xW-R
applies R rounds. The multipliers and Weyl constants below are the ones the paper gives for
w = 32 and w = 64.

This file is written once, generically over the word width w, so that the 4x64-10 instance can
be checked against ``numpy.random.Philox`` (an independent library implementation of
Philox4x64-10) and the 4x32-10 instance, which differs only in its constants, inherits that
check. It belongs to the CPU oracle and is test infrastructure only.
"""
from __future__ import annotations

import numpy as np

# (M0, M1, W0, W1) per word width, from the paper's Philox parameter table.
PARAMS = {
    32: (0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85),
    64: (0xD2E7470EE14C6C93, 0xCA5A826395121157, 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B),
}

_U64 = np.uint64
_M32 = _U64(0xFFFFFFFF)


def _mulhilo(a: np.ndarray, m: int, w: int):
    """Double-width product a*m split into (high word, low word), elementwise over uint64 arrays."""
    if w == 32:
        p = a * _U64(m)  # a < 2**32 and m < 2**32, so the product fits in 64 bits
        return p >> _U64(32), p & _M32
    # w == 64: schoolbook multiplication on 32-bit halves, every partial product below 2**64.
    a_lo, a_hi = a & _M32, a >> _U64(32)
    m_lo, m_hi = _U64(m & 0xFFFFFFFF), _U64(m >> 32)
    ll = a_lo * m_lo  # each partial product of two 32-bit halves fits in 64 bits
    lh = a_lo * m_hi
    hl = a_hi * m_lo
    hh = a_hi * m_hi
    mid = (ll >> _U64(32)) + (lh & _M32) + (hl & _M32)
    lo = (ll & _M32) | ((mid & _M32) << _U64(32))
    hi = hh + (lh >> _U64(32)) + (hl >> _U64(32)) + (mid >> _U64(32))
    return hi, lo


def philox4(counter, key, w: int = 32, rounds: int = 10):
    """Philox4xW-R. ``counter``: 4 arrays (or ints) of w-bit words; ``key``: 2 of them.

    Returns a tuple of 4 uint64 arrays holding the w-bit output words."""
    M0, M1, W0, W1 = PARAMS[w]
    mask = _U64((1 << w) - 1)
    x = [np.asarray(c, dtype=np.uint64) & mask for c in counter]
    k0, k1 = (np.asarray(k, dtype=np.uint64) & mask for k in key)
    with np.errstate(over="ignore"):  # key bumps and products wrap modulo 2**64 by design
        for r in range(rounds):
            if r:
                k0 = (k0 + _U64(W0)) & mask
                k1 = (k1 + _U64(W1)) & mask
            hi_a, lo_a = _mulhilo(x[0], M0, w)
            hi_b, lo_b = _mulhilo(x[2], M1, w)
            x = [(hi_b ^ x[1] ^ k0) & mask, lo_b & mask, (hi_a ^ x[3] ^ k1) & mask, lo_a & mask]
    return tuple(x)


def token_uniforms(token_ids, seed: int, position: int) -> np.ndarray:
    """Uniform variates in (0, 1) for the exponential race of one row (float64).

    Philox4x32-10 keyed by the row's 64-bit seed (low word, high word); the counter of token i is
    (i >> 2, 0, position low word, position high word) and the token takes output word i & 3.
    The uniform keeps the 23 high bits k of that word and centres it: u = (2k + 1) / 2**24, which
    lies strictly inside (0, 1) and is exact in float32 and float64."""
    ids = np.asarray(token_ids, dtype=np.uint64)
    seed = int(seed)
    position = int(position)
    key = (seed & 0xFFFFFFFF, seed >> 32)
    ctr = (ids >> _U64(2), np.zeros_like(ids), np.full_like(ids, position & 0xFFFFFFFF),
           np.full_like(ids, position >> 32))
    out = philox4(ctr, key, w=32, rounds=10)
    sel = (ids & _U64(3)).astype(np.int64)
    words = np.choose(sel, out)
    k = (words >> _U64(9)).astype(np.float64)
    return (2.0 * k + 1.0) / 16777216.0
