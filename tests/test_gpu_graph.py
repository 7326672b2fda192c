"""The library's calls inside a captured HIP graph (needs an MI355X): the sampler, its bitmask
form, the replay and the CSR launch no allocation and no memset, so a graph of them replays
bit-identically. Each replay is checked against the eager result, with eager work and
synchronizations between replays. Every case prints its name before touching the GPU."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import device_inputs, log
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _outputs(out):
    return [t.cpu().numpy().copy() for t in out if t is not None]


def _defined(out):
    """The outputs a call defines: per-row arrays whole, packed rows up to their length, bitmask
    rows of OVERFLOW slots only (the API leaves the rest unspecified or untouched)."""
    o = {k: (None if v is None else v.cpu().numpy().copy()) for k, v in out._asdict().items()}
    L = o["lengths"]
    res = [o["tokens"], o["row_status"], L, np.nan_to_num(o["selected_logprob"], nan=1e9)]
    for j in range(len(L)):
        res.append(o["packed_ids"][j, :L[j]])
        if o["logprobs"] is not None:
            res.append(o["logprobs"][j, :L[j]])
    return res


@pytest.mark.parametrize("index,bits", [(3, False), (4, True), (2, False)])
def test_sampler_in_a_graph(index, bits):
    import top_support_capture_amd as tsc
    wl = make_workload(index)
    log(f"case graph capture of the sampler, workload {index}, bitmask {bits}")
    d = device_inputs(wl)
    call = tsc.prepare(d["logits"], d["temperature"], d["top_k"], d["top_p"], d["min_p"],
                       d["optin_rows"], d["seeds"], d["positions"], wl.W, return_bits=bits)
    call(d["logits"])  # first launch (sets the kernel attribute) outside the capture
    torch.cuda.synchronize()
    eager = _defined(call.out)
    status = call.out.row_status.cpu().numpy()[wl.optin_rows]
    eager_bits = call.out.support_bits.cpu().numpy()[status == 1] if bits else None
    csr = tsc.support_csr(call.out)
    torch.cuda.synchronize()
    eager_csr = _outputs(csr)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call2 = tsc.prepare(d["logits"], d["temperature"], d["top_k"], d["top_p"], d["min_p"],
                            d["optin_rows"], d["seeds"], d["positions"], wl.W, out=call.out,
                            stream=s, return_bits=bits)
        with torch.cuda.graph(g, stream=s):
            call2(d["logits"])
            tsc.support_csr(call.out, stream=s)  # writes csr-shaped outputs of its own
    torch.cuda.synchronize()
    for rep in range(3):
        for t in call.out:  # scribble over the outputs between replays
            if t is not None:
                t.fill_(7 if t.dtype != torch.float32 else 7.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _defined(call.out)
        assert len(got) == len(eager)
        for a, b in zip(got, eager):
            assert np.array_equal(a, b), rep
        if bits:
            assert np.array_equal(call.out.support_bits.cpu().numpy()[status == 1], eager_bits)
    # The CSR launched eagerly after a replay equals the eager CSR (its first offsets[R] entries).
    csr2 = tsc.support_csr(call.out)
    torch.cuda.synchronize()
    n = int(eager_csr[0][-1])
    got_csr = _outputs(csr2)
    assert np.array_equal(got_csr[0], eager_csr[0])
    for a, b in zip(got_csr[1:], eager_csr[1:]):
        assert np.array_equal(a[:n], b[:n])


def test_concurrent_streams():
    # Two batches sampled at the same time on two streams (the library keeps no per-call state)
    # give what each gives alone.
    import top_support_capture_amd as tsc
    log("case two streams at once: workloads 3 and 4")
    outs = {}
    calls = {}
    for index in (3, 4):
        wl = make_workload(index)
        d = device_inputs(wl)
        calls[index] = (wl, d)
        o = tsc.sample_with_mask(d["logits"], d["temperature"], d["top_k"], d["top_p"],
                                 d["min_p"], d["optin_rows"], d["seeds"], d["positions"], wl.W)
        torch.cuda.synchronize()
        outs[index] = _defined(o)
    s3, s4 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(5):
        res = {}
        for index, s in ((3, s3), (4, s4)):
            wl, d = calls[index]
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                res[index] = tsc.sample_with_mask(d["logits"], d["temperature"], d["top_k"],
                                                  d["top_p"], d["min_p"], d["optin_rows"],
                                                  d["seeds"], d["positions"], wl.W, stream=s)
        torch.cuda.synchronize()
        for index in (3, 4):
            got = _defined(res[index])
            assert len(got) == len(outs[index])
            for a, b in zip(got, outs[index]):
                assert np.array_equal(a, b)
