"""MI355X-native batched top-k / top-p / min-p sampler with exact support capture.

Python binding of the C-ABI library ``libtsc.so`` (declared in ``include/tsc.h``). This module
only marshals arguments: it checks tensor devices and dtypes, allocates the output tensors with
PyTorch on the logits' device, and calls ``tsc_sample_with_mask`` on the current HIP stream.
Every step of the sampling runs in the library's HIP kernels; there is no fallback, and the
import fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch  # must come first: the library binds to the HIP runtime PyTorch has loaded

__all__ = ["sample_with_mask", "prepare", "PreparedSample", "SampleOutput", "workspace_size",
           "support_bits_ld", "replay_logprob", "ReplayOutput", "support_csr", "SupportCsr",
           "csr_to_host",
           "library", "LIB_PATH",
           "ROW_OK", "ROW_OVERFLOW", "ROW_NO_SUPPORT", "ROW_NONFINITE", "ROW_INVALID_PARAM",
           "ROW_ABORTED", "set_wait_limit", "set_debug_poison",
           "MAX_PACKED_WIDTH", "TscError"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtsc.so")

TSC_DTYPE_F32, TSC_DTYPE_BF16 = 0, 1
ROW_OK, ROW_OVERFLOW, ROW_NO_SUPPORT, ROW_NONFINITE, ROW_INVALID_PARAM, ROW_ABORTED = 0, 1, 2, 3, 4, 5
MAX_PACKED_WIDTH = 16384

_lib: Optional[ctypes.CDLL] = None


class TscError(RuntimeError):
    def __init__(self, code: int, name: str):
        super().__init__(f"tsc_sample_with_mask failed: {name} ({code})")
        self.code = code


def library() -> ctypes.CDLL:
    """Load ``libtsc.so`` (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m top_support_capture_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.tsc_sample_with_mask.argtypes = [P, I32, I64, I64, I64, P, P, P, P, P, I64, P, P, I32,
                                         P, P, P, P, P, P, P, SZ, P]
    lib.tsc_sample_with_mask.restype = I32
    lib.tsc_sample_with_mask_bits.argtypes = [P, I32, I64, I64, I64, P, P, P, P, P, I64, P, P,
                                              I32, P, P, P, P, P, P, P, I64, P, SZ, P]
    lib.tsc_sample_with_mask_bits.restype = I32
    lib.tsc_replay_logprob.argtypes = [P, I32, I64, I64, I64, P, P, P, I32, P, P, I64, P, P, P,
                                       P, P]
    lib.tsc_replay_logprob.restype = I32
    lib.tsc_support_csr.argtypes = [P, P, P, I64, I32, P, P, P, I64, P]
    lib.tsc_support_csr.restype = I32
    lib.tsc_support_bits_ld.argtypes = [I64]
    lib.tsc_support_bits_ld.restype = I64
    lib.tsc_workspace_size.argtypes = [I64, I64, I64, I32, I32]
    lib.tsc_workspace_size.restype = SZ
    lib.tsc_status_string.argtypes = [I32]
    lib.tsc_status_string.restype = ctypes.c_char_p
    lib.tsc_version.argtypes = []
    lib.tsc_version.restype = I32
    lib.tsc_set_wait_limit.argtypes = [ctypes.c_uint32]
    lib.tsc_set_wait_limit.restype = ctypes.c_uint32
    lib.tsc_set_debug_poison.argtypes = [ctypes.c_int32]
    lib.tsc_set_debug_poison.restype = ctypes.c_int32
    _lib = lib
    return lib


class SampleOutput(NamedTuple):
    tokens: torch.Tensor            # int32 [B]
    packed_ids: torch.Tensor        # int32 [R, W]
    lengths: torch.Tensor           # int32 [R]
    logprobs: Optional[torch.Tensor]  # float32 [R, W] (None in selected mode)
    selected_logprob: torch.Tensor  # float32 [R]
    row_status: torch.Tensor        # int8 [B]
    # uint8 [R, bits_ld]: the support bitmask of each OVERFLOW slot (bit i % 8 of byte i / 8);
    # rows of other slots are left as they were. None unless requested.
    support_bits: Optional[torch.Tensor] = None


def workspace_size(B: int, V: int, R: int, W: int, dtype: torch.dtype) -> int:
    dt = TSC_DTYPE_BF16 if dtype == torch.bfloat16 else TSC_DTYPE_F32
    return int(library().tsc_workspace_size(B, V, R, W, dt))


def set_wait_limit(sleeps: int) -> int:
    """Limit of the bounded waits between the waves of a row's workgroup (``tsc_set_wait_limit``):
    0 restores the default; a tiny value makes rows give up with ROW_ABORTED (for tests of that
    path). Returns the previous limit."""
    return int(library().tsc_set_wait_limit(int(sleeps)))


def set_debug_poison(on: bool) -> bool:
    """While on, every capturing call fills packed slots past each length with id -1 and
    logprob NaN (``tsc_set_debug_poison``), so that reads past a length stand out. Returns the
    previous setting."""
    return bool(library().tsc_set_debug_poison(1 if on else 0))


def support_bits_ld(V: int) -> int:
    """Smallest row stride in bytes of a support bitmask buffer for vocabulary size V."""
    return int(library().tsc_support_bits_ld(V))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor, name: str, dtype, n: int, dev) -> None:
    if t.device != dev or t.dtype != dtype or t.dim() != 1 or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape [{n}] on {dev}")


def _check_out(out: "SampleOutput", B: int, R: int, W: int, dev) -> None:
    Wc = max(int(W), 1)
    _check(out.tokens, "out.tokens", torch.int32, B, dev)
    _check(out.row_status, "out.row_status", torch.int8, B, dev)
    _check(out.lengths, "out.lengths", torch.int32, R, dev)
    _check(out.selected_logprob, "out.selected_logprob", torch.float32, R, dev)
    for name, t, dt in (("packed_ids", out.packed_ids, torch.int32),
                        ("logprobs", out.logprobs, torch.float32)):
        if t is None and name == "logprobs":
            continue
        if (t.device != dev or t.dtype != dt or tuple(t.shape) != (R, Wc)
                or not t.is_contiguous()):
            raise ValueError(f"out.{name} must be a contiguous {dt} tensor of shape [{R}, {Wc}] "
                             f"on {dev}")


class PreparedSample:
    """A validated argument set for repeated calls that differ only in the logits tensor (same
    shape, dtype, device and strides): each call is one library call with cached pointers."""

    def __init__(self, logits: torch.Tensor, temperature: torch.Tensor, top_k: torch.Tensor,
                 top_p: torch.Tensor, min_p: torch.Tensor, optin_rows: torch.Tensor,
                 seeds: torch.Tensor, positions: torch.Tensor, W: int,
                 return_logprobs: bool = True, out: Optional[SampleOutput] = None,
                 stream: Optional[torch.cuda.Stream] = None, return_bits: bool = False):
        self._lib = library()
        if logits.dim() != 2 or logits.stride(1) != 1:
            raise ValueError("logits must be [B, V] with unit column stride")
        if logits.dtype == torch.float32:
            dt = TSC_DTYPE_F32
        elif logits.dtype == torch.bfloat16:
            dt = TSC_DTYPE_BF16
        else:
            raise ValueError("logits must be float32 or bfloat16")
        dev = logits.device
        B, V = logits.shape
        ld = logits.stride(0) if B > 1 else V
        R = int(optin_rows.numel())
        _check(temperature, "temperature", torch.float32, B, dev)
        _check(top_k, "top_k", torch.int32, B, dev)
        _check(top_p, "top_p", torch.float32, B, dev)
        _check(min_p, "min_p", torch.float32, B, dev)
        _check(optin_rows, "optin_rows", torch.int32, R, dev)
        _check(seeds, "seeds", torch.int64, B, dev)
        _check(positions, "positions", torch.int64, B, dev)
        if out is None:
            Wc = max(int(W), 1)
            out = SampleOutput(
                tokens=torch.empty(B, dtype=torch.int32, device=dev),
                packed_ids=torch.empty((R, Wc), dtype=torch.int32, device=dev),
                lengths=torch.empty(R, dtype=torch.int32, device=dev),
                logprobs=(torch.empty((R, Wc), dtype=torch.float32, device=dev)
                          if return_logprobs else None),
                selected_logprob=torch.empty(R, dtype=torch.float32, device=dev),
                row_status=torch.empty(B, dtype=torch.int8, device=dev),
                support_bits=(torch.zeros((R, support_bits_ld(V)), dtype=torch.uint8, device=dev)
                              if return_bits else None))
        else:
            _check_out(out, B, R, W, dev)
            sb = out.support_bits
            if sb is not None and (sb.device != dev or sb.dtype != torch.uint8 or sb.dim() != 2
                                   or sb.shape[0] != R or sb.stride(1) != 1
                                   or (R > 1 and sb.stride(0) != sb.shape[1])):
                raise ValueError(f"out.support_bits must be a contiguous uint8 tensor [{R}, ld] "
                                 f"on {dev}")
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        self.out = out
        self._shape = (tuple(logits.shape), tuple(logits.stride()), logits.dtype, dev)
        # Keep the argument tensors alive as long as their pointers are cached.
        self._keep = (temperature, top_k, top_p, min_p, optin_rows, seeds, positions, s)
        self._tail = (
            dt, B, V, ld, temperature.data_ptr(), top_k.data_ptr(), top_p.data_ptr(),
            min_p.data_ptr(), _ptr(optin_rows) if R else None, R, seeds.data_ptr(),
            positions.data_ptr(), int(W), out.tokens.data_ptr(), out.row_status.data_ptr(),
            _ptr(out.packed_ids) if R else None,
            _ptr(out.logprobs) if (R and out.logprobs is not None) else None,
            _ptr(out.lengths) if R else None, _ptr(out.selected_logprob) if R else None,
            _ptr(out.support_bits) if (R and out.support_bits is not None) else None,
            int(out.support_bits.shape[1]) if out.support_bits is not None else 0,
            None, 0, s.cuda_stream)

    def __call__(self, logits: torch.Tensor, check: bool = True) -> SampleOutput:
        if check and (tuple(logits.shape), tuple(logits.stride()), logits.dtype,
                      logits.device) != self._shape:
            raise ValueError("logits must match the prepared shape, strides, dtype and device")
        code = self._lib.tsc_sample_with_mask_bits(logits.data_ptr(), *self._tail)
        if code != 0:
            raise TscError(code, self._lib.tsc_status_string(code).decode())
        return self.out


def prepare(logits: torch.Tensor, temperature: torch.Tensor, top_k: torch.Tensor,
            top_p: torch.Tensor, min_p: torch.Tensor, optin_rows: torch.Tensor,
            seeds: torch.Tensor, positions: torch.Tensor, W: int, return_logprobs: bool = True,
            out: Optional[SampleOutput] = None, stream: Optional[torch.cuda.Stream] = None,
            return_bits: bool = False) -> PreparedSample:
    """Validate the arguments once; the returned object samples a logits tensor per call."""
    return PreparedSample(logits, temperature, top_k, top_p, min_p, optin_rows, seeds, positions,
                          W, return_logprobs, out, stream, return_bits)


def sample_with_mask(logits: torch.Tensor, temperature: torch.Tensor, top_k: torch.Tensor,
                     top_p: torch.Tensor, min_p: torch.Tensor, optin_rows: torch.Tensor,
                     seeds: torch.Tensor, positions: torch.Tensor, W: int,
                     return_logprobs: bool = True, out: Optional[SampleOutput] = None,
                     stream: Optional[torch.cuda.Stream] = None,
                     return_bits: bool = False) -> SampleOutput:
    """Sample one token per row of ``logits`` [B, V] (float32 or bfloat16, unit column stride)
    and capture the support of the rows listed in ``optin_rows`` (int32, ascending).

    ``temperature``/``top_p``/``min_p`` are float32 [B], ``top_k`` int32 [B], ``seeds`` and
    ``positions`` int64 [B] holding the uint64 bit patterns. Outputs are allocated on the
    logits' device unless ``out`` supplies them. Runs asynchronously on ``stream`` (default: the
    current stream). With ``return_bits`` (or ``out.support_bits`` given) the support of every
    OVERFLOW slot is also written as a bitmask."""
    return PreparedSample(logits, temperature, top_k, top_p, min_p, optin_rows, seeds, positions,
                          W, return_logprobs, out, stream, return_bits)(logits, check=False)


class ReplayOutput(NamedTuple):
    selected_logprob: torch.Tensor     # float32 [N]
    logprobs: Optional[torch.Tensor]   # float32 [N, W] (None unless requested)
    row_status: torch.Tensor           # int8 [N]


def replay_logprob(logits: torch.Tensor, temperature: torch.Tensor, packed_ids: torch.Tensor,
                   lengths: torch.Tensor, tokens: torch.Tensor,
                   capture_status: Optional[torch.Tensor] = None,
                   support_bits: Optional[torch.Tensor] = None, return_logprobs: bool = False,
                   stream: Optional[torch.cuda.Stream] = None) -> ReplayOutput:
    """Log-probability of ``tokens`` under ``logits`` [N, V] normalized over each row's captured
    support: ``packed_ids`` [N, W] / ``lengths`` [N] (int32, as the sampler writes them), or,
    where ``capture_status`` (int8 [N]) is OVERFLOW, the row of ``support_bits`` (uint8 [N, ld]).
    ``temperature`` float32 [N] divides the logits first (1 = the plain masked log-softmax)."""
    lib = library()
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [N, V] with unit column stride")
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("logits must be float32 or bfloat16")
    dt = TSC_DTYPE_BF16 if logits.dtype == torch.bfloat16 else TSC_DTYPE_F32
    dev = logits.device
    N, V = logits.shape
    ld = logits.stride(0) if N > 1 else V
    _check(temperature, "temperature", torch.float32, N, dev)
    _check(lengths, "lengths", torch.int32, N, dev)
    _check(tokens, "tokens", torch.int32, N, dev)
    if (packed_ids.device != dev or packed_ids.dtype != torch.int32 or packed_ids.dim() != 2
            or packed_ids.shape[0] != N or not packed_ids.is_contiguous()):
        raise ValueError(f"packed_ids must be a contiguous int32 tensor [{N}, W] on {dev}")
    W = int(packed_ids.shape[1])
    if capture_status is not None:
        _check(capture_status, "capture_status", torch.int8, N, dev)
    bits_ld = 0
    if support_bits is not None:
        if (support_bits.device != dev or support_bits.dtype != torch.uint8
                or support_bits.dim() != 2 or support_bits.shape[0] != N
                or not support_bits.is_contiguous()):
            raise ValueError(f"support_bits must be a contiguous uint8 tensor [{N}, ld] on {dev}")
        bits_ld = int(support_bits.shape[1])
    out = ReplayOutput(torch.empty(N, dtype=torch.float32, device=dev),
                       torch.empty((N, W), dtype=torch.float32, device=dev)
                       if return_logprobs else None,
                       torch.empty(N, dtype=torch.int8, device=dev))
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    code = lib.tsc_replay_logprob(logits.data_ptr(), dt, N, V, ld, temperature.data_ptr(),
                                  packed_ids.data_ptr(), lengths.data_ptr(), W,
                                  _ptr(capture_status), _ptr(support_bits), bits_ld,
                                  tokens.data_ptr(), out.selected_logprob.data_ptr(),
                                  _ptr(out.logprobs), out.row_status.data_ptr(), s.cuda_stream)
    if code != 0:
        raise TscError(code, lib.tsc_status_string(code).decode())
    return out


class SupportCsr(NamedTuple):
    offsets: torch.Tensor              # int64 [R + 1]
    ids: torch.Tensor                  # int32 [cap]; the first offsets[R] entries are valid
    logprobs: Optional[torch.Tensor]   # float32 [cap] or None


def support_csr(out: SampleOutput, cap: Optional[int] = None,
                stream: Optional[torch.cuda.Stream] = None) -> SupportCsr:
    """The captured supports of ``out`` back to back on the device (asynchronous): slot j's ids
    (and logprobs) at offsets[j] .. offsets[j + 1]. ``cap`` (default R * W) bounds the payload."""
    lib = library()
    R, W = out.packed_ids.shape
    dev = out.packed_ids.device
    cap = R * W if cap is None else int(cap)
    csr = SupportCsr(torch.empty(R + 1, dtype=torch.int64, device=dev),
                     torch.empty(max(cap, 1), dtype=torch.int32, device=dev),
                     torch.empty(max(cap, 1), dtype=torch.float32, device=dev)
                     if out.logprobs is not None else None)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    code = lib.tsc_support_csr(_ptr(out.lengths), _ptr(out.packed_ids), _ptr(out.logprobs), R, W,
                               csr.offsets.data_ptr(), csr.ids.data_ptr(), _ptr(csr.logprobs),
                               cap, s.cuda_stream)
    if code != 0:
        raise TscError(code, lib.tsc_status_string(code).decode())
    return csr


def csr_to_host(csr: SupportCsr, stream: Optional[torch.cuda.Stream] = None):
    """Copy a support CSR to host memory sized by the realized support: the offsets first (one
    synchronization), then exactly offsets[R] ids and logprobs. Returns numpy arrays
    (offsets, ids, logprobs or None)."""
    offsets = csr.offsets.cpu()
    total = int(offsets[-1])
    ids = csr.ids[:total].cpu().numpy()
    lps = csr.logprobs[:total].cpu().numpy() if csr.logprobs is not None else None
    return offsets.numpy(), ids, lps
