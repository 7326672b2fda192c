"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The host part of the C ABI (argument checks, host-side state, strings) is compiled with both
sanitizers on the host pass only (`-Xarch_host`; the kernels are compiled as usual and never
launched), and
`tests/host_abi_check.c` calls every entry point with invalid and boundary arguments, none of
which launches anything. Any sanitizer report fails the test. The oracle is plain Python and
numpy: it has no native code of its own to instrument.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm/bin"


def _tool(name):
    for cand in (os.path.join("/opt/rocm/bin", name), os.path.join(LLVM, name), shutil.which(name)):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip(f"{name} not found")


def test_host_abi_under_asan_and_ubsan(tmp_path):
    hipcc, clang = _tool("hipcc"), os.path.join(LLVM, "clang")
    if not os.path.exists(clang):
        pytest.skip("the ROCm clang is needed for the sanitizer runtimes")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "top_support_capture_amd", "csrc")]
    lib = tmp_path / "libtsc_hostsan.so"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([hipcc, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-fPIC", "-shared", *san, *inc, "-o", str(lib),
                    os.path.join(ROOT, "top_support_capture_amd", "csrc", "tsc_api.hip")],
                   check=True, capture_output=True, timeout=600)
    exe = tmp_path / "host_abi_check"
    subprocess.run([clang, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-g",
                    "-O1", *inc, os.path.join(ROOT, "tests", "host_abi_check.c"), str(lib),
                    f"-Wl,-rpath,{tmp_path}", "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=99",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=98")
    r = subprocess.run([str(exe)], env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "host ABI checks: 0 failure(s)" in r.stdout
