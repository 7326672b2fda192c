"""CPU oracle of the batched sampler with support capture.

TEST INFRASTRUCTURE ONLY: imported by the tests, the graft smoke check and the bench's CPU
baseline leg, never by the product path. It shares no code with the HIP library.
"""
from .philox import philox4, token_uniforms  # noqa: F401
from .sampler import (  # noqa: F401
    ROW_OK, ROW_OVERFLOW, ROW_NO_SUPPORT, ROW_NONFINITE, ROW_INVALID_PARAM,
    RACE_TIE_EPS, TOP_P_EPS, MIN_P_EPS, RowResult, BatchResult,
    decode_logits, params_valid, sample_row, sample_with_mask, slot_validity, support_bitmask,
)
from .replay import ReplayRow, replay, replay_row  # noqa: F401
from .csr import support_csr  # noqa: F401
