"""CPU oracle of the compressed (CSR) layout of captured supports (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by the tests, the graft smoke check and the bench's CPU
baseline leg, never by the product path.

sglang PR #40986, "Limitations": the packed [rows, width] capture buffer crosses to the host
whole every step, sized by its capacity rather than by the realized support. The CSR layout
holds the same entries back to back: row j's first lengths[j] packed ids (and logprobs) at
offsets[j] .. offsets[j + 1], with offsets the exclusive prefix sum of the lengths, so a copy can
be sized by offsets[R].

Reading (R15): a length outside [0, W] is clamped into it (the sampler writes only lengths in
range; a clamped length keeps the layout well-formed for any input).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def support_csr(lengths: np.ndarray, packed_ids: np.ndarray,
                logprobs: Optional[np.ndarray] = None
                ) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """(offsets int64 [R + 1], ids int32 [offsets[R]], logprobs float32 [offsets[R]] or None)."""
    R, W = packed_ids.shape
    n = np.clip(np.asarray(lengths, dtype=np.int64), 0, W)
    offsets = np.zeros(R + 1, np.int64)
    offsets[1:] = np.cumsum(n)
    ids = np.concatenate([packed_ids[j, :n[j]] for j in range(R)] or [np.zeros(0, np.int32)])
    lps = None
    if logprobs is not None:
        lps = np.concatenate([logprobs[j, :n[j]] for j in range(R)] or [np.zeros(0, np.float32)])
        lps = lps.astype(np.float32)
    return offsets, ids.astype(np.int32), lps
