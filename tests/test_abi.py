"""The C-ABI library loads and exports every entry point the header declares; host-side
argument checks return their documented codes without touching the GPU (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsc.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tsc_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    import top_support_capture_amd as tsc
    return tsc.library()


def test_header_declares_the_entry_points():
    assert declared_functions() == ["tsc_replay_logprob", "tsc_sample_with_mask",
                                    "tsc_sample_with_mask_bits", "tsc_set_debug_poison",
                                    "tsc_set_wait_limit", "tsc_status_string",
                                    "tsc_support_bits_ld", "tsc_support_csr", "tsc_version",
                                    "tsc_workspace_size"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert lib.tsc_status_string(0) == b"TSC_OK"
    assert lib.tsc_status_string(3) == b"TSC_ERR_WORKSPACE"
    assert lib.tsc_status_string(99) == b"TSC_UNKNOWN_STATUS"
    assert lib.tsc_version() >= 100
    assert lib.tsc_workspace_size(256, 151936, 256, 2048, 1) == 0


def test_wait_limit_setting(lib):
    # Host-side state only: 0 restores the default (2^20 sleeps); the previous value is returned.
    import top_support_capture_amd as tsc
    prev = tsc.set_wait_limit(7)
    try:
        assert tsc.set_wait_limit(0) == 7
        assert tsc.set_wait_limit(0) == 1 << 20
    finally:
        tsc.set_wait_limit(prev)


def test_debug_poison_setting(lib):
    # Host-side state only: off by default, the previous setting is returned.
    import top_support_capture_amd as tsc
    prev = tsc.set_debug_poison(True)
    try:
        assert prev is False
        assert tsc.set_debug_poison(False) is True
        assert tsc.set_debug_poison(False) is False
    finally:
        tsc.set_debug_poison(prev)


def _call(lib, **kw):
    args = dict(logits=0x1000, dtype=1, B=4, V=100, ld=100, temperature=8, top_k=8, top_p=8,
                min_p=8, optin_rows=8, R=2, seeds=8, positions=8, W=16, tokens=8, row_status=8,
                packed_ids=8, logprobs=8, lengths=8, selected_logprob=8, workspace=None, wsb=0,
                stream=None)
    args.update(kw)
    return lib.tsc_sample_with_mask(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 1), (dict(B=-1), 1), (dict(V=0), 1), (dict(ld=99), 1), (dict(R=5), 1),
    (dict(R=-1), 1), (dict(W=0), 1), (dict(W=16385), 2), (dict(logits=0x1001), 1),
    (dict(logits=None), 1), (dict(seeds=None), 1), (dict(tokens=None), 1),
    (dict(optin_rows=None), 1), (dict(lengths=None), 1), (dict(B=0, R=0), 0),
])
def test_host_argument_checks(lib, kw, code):
    # Every case returns before any HIP call, so this runs without a GPU.
    assert _call(lib, **kw) == code


def _call_bits(lib, **kw):
    args = dict(logits=0x1000, dtype=1, B=4, V=100, ld=100, temperature=8, top_k=8, top_p=8,
                min_p=8, optin_rows=8, R=2, seeds=8, positions=8, W=16, tokens=8, row_status=8,
                packed_ids=8, logprobs=8, lengths=8, selected_logprob=8, support_bits=0x2000,
                bits_ld=16, workspace=None, wsb=0, stream=None)
    args.update(kw)
    return lib.tsc_sample_with_mask_bits(*args.values())


def test_support_bits_row_size(lib):
    # ceil(V / 8) bytes rounded up to 16.
    for V, ld in [(1, 16), (8, 16), (128, 16), (129, 32), (100, 16), (151936, 18992),
                  (129280, 16160), (262144, 32768), (32000, 4000), (0, 0)]:
        assert lib.tsc_support_bits_ld(V) == ld, V


@pytest.mark.parametrize("kw,code", [
    (dict(bits_ld=15), 1), (dict(bits_ld=8), 1), (dict(bits_ld=24), 1),
    (dict(support_bits=0x2008), 1), (dict(V=129, ld=129, bits_ld=16), 1),
    (dict(dtype=7), 1), (dict(W=0), 1), (dict(B=0, R=0), 0),
])
def test_bits_argument_checks(lib, kw, code):
    # Every case returns before any HIP call, so this runs without a GPU.
    assert _call_bits(lib, **kw) == code


def _call_replay(lib, **kw):
    args = dict(logits=0x1000, dtype=1, N=4, V=100, ld=100, temperature=8, packed_ids=8,
                lengths=8, W=16, capture_status=None, support_bits=None, bits_ld=0, tokens=8,
                selected_logprob=8, logprobs=None, row_status=8, stream=None)
    args.update(kw)
    return lib.tsc_replay_logprob(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), 1), (dict(N=-1), 1), (dict(V=0), 1), (dict(ld=50), 1), (dict(W=0), 1),
    (dict(W=16385), 2), (dict(logits=0x1001), 1), (dict(logits=None), 1),
    (dict(temperature=None), 1), (dict(packed_ids=None), 1), (dict(lengths=None), 1),
    (dict(tokens=None), 1), (dict(selected_logprob=None), 1), (dict(row_status=None), 1),
    (dict(support_bits=0x2000, bits_ld=12), 1), (dict(N=0), 0),
])
def test_replay_argument_checks(lib, kw, code):
    # Every case returns before any HIP call, so this runs without a GPU.
    assert _call_replay(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(R=-1), 1), (dict(W=0), 1), (dict(W=16385), 2), (dict(cap=-1), 1),
    (dict(offsets=None), 1), (dict(lengths=None), 1), (dict(packed_ids=None), 1),
    (dict(csr_ids=None), 1),
])
def test_csr_argument_checks(lib, kw, code):
    # Every case returns before any HIP call, so this runs without a GPU.
    args = dict(lengths=8, packed_ids=8, logprobs=None, R=4, W=16, offsets=8, csr_ids=8,
                csr_logprobs=None, cap=64, stream=None)
    args.update(kw)
    assert lib.tsc_support_csr(*args.values()) == code


def test_binding_rejects_bad_tensors():
    import torch
    import top_support_capture_amd as tsc
    x = torch.zeros((2, 8), dtype=torch.float16)
    z = torch.zeros(2)
    with pytest.raises(ValueError):
        tsc.sample_with_mask(x, z, z.int(), z, z, z.int(), z.long(), z.long(), 4)
