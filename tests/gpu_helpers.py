"""Moving seeded workloads to the GPU and calling the library through its Python binding."""
from __future__ import annotations

import sys

import numpy as np
import torch

from tests.parity import to_numpy_outputs


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def logits_tensor(logits: np.ndarray, dtype: str, device="cuda:0", pad: int = 0) -> torch.Tensor:
    """[B, V] device tensor; ``pad`` extra columns give a row stride ld = V + pad."""
    B, V = logits.shape
    if dtype == "bf16":
        host = torch.from_numpy(np.ascontiguousarray(logits).view(np.int16)).view(torch.bfloat16)
    else:
        host = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32))
    if pad:
        full = torch.zeros((B, V + pad), dtype=host.dtype)
        full[:, :V] = host
        return full.to(device)[:, :V]
    return host.to(device)


def device_inputs(wl, device="cuda:0", pad: int = 0) -> dict:
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(device)
    return {
        "logits": logits_tensor(wl.logits, wl.dtype, device, pad),
        "temperature": t(wl.temperature.astype(np.float32), torch.float32),
        "top_k": t(wl.top_k.astype(np.int32), torch.int32),
        "top_p": t(wl.top_p.astype(np.float32), torch.float32),
        "min_p": t(wl.min_p.astype(np.float32), torch.float32),
        "optin_rows": t(wl.optin_rows.astype(np.int32), torch.int32),
        "seeds": torch.from_numpy(wl.seeds.astype(np.uint64).view(np.int64)).to(device),
        "positions": torch.from_numpy(wl.positions.astype(np.uint64).view(np.int64)).to(device),
    }


def run_gpu(wl, W=None, return_logprobs=True, pad=0, inputs=None, bits=False) -> dict:
    """One library call; with ``bits`` the support bitmask buffer is passed too, pre-filled with
    BITS_SENTINEL so that rows the call must not write can be checked."""
    import top_support_capture_amd as tsc
    from tests.parity import BITS_SENTINEL
    d = inputs if inputs is not None else device_inputs(wl, pad=pad)
    W = wl.W if W is None else W
    out = None
    if bits:
        dev = d["logits"].device
        B, V = d["logits"].shape
        R, Wc = int(d["optin_rows"].numel()), max(int(W), 1)
        out = tsc.SampleOutput(
            tokens=torch.empty(B, dtype=torch.int32, device=dev),
            packed_ids=torch.empty((R, Wc), dtype=torch.int32, device=dev),
            lengths=torch.empty(R, dtype=torch.int32, device=dev),
            logprobs=(torch.empty((R, Wc), dtype=torch.float32, device=dev)
                      if return_logprobs else None),
            selected_logprob=torch.empty(R, dtype=torch.float32, device=dev),
            row_status=torch.empty(B, dtype=torch.int8, device=dev),
            support_bits=torch.full((R, tsc.support_bits_ld(V)), BITS_SENTINEL,
                                    dtype=torch.uint8, device=dev))
    out = tsc.sample_with_mask(d["logits"], d["temperature"], d["top_k"], d["top_p"], d["min_p"],
                               d["optin_rows"], d["seeds"], d["positions"], W,
                               return_logprobs=return_logprobs, out=out)
    torch.cuda.synchronize()
    return to_numpy_outputs(out)
