"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the library's host sources -- the C ABI's validation and dispatch
(abi.cpp) and the paged planner (paged_plan.cpp) -- for the host alone (no GPU
code is generated), with the sanitizers on and recovery off, links them with
tests/host/abi_fuzz.cpp (launcher stubs plus a seeded sweep of valid and
malformed arguments, plan-table bounds checks) and runs it.  Any out-of-bounds
access, leak, signed overflow or invalid shift in the host code fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "scaled_dot_product_bwd_amd", "csrc")


def _tool(name):
    for cand in (shutil.which(name), os.path.join("/opt/rocm/bin", name),
                 os.path.join("/opt/rocm/llvm/bin", name)):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    hipcc, clang = _tool("hipcc"), _tool("clang++")
    if not hipcc or not clang:
        pytest.skip("the ROCm toolchain is needed for the host sanitizer build")
    out = tmp_path_factory.mktemp("asan")
    flags = ["-x", "hip", "--offload-host-only", "-O1", "-g", "-std=c++17",
             "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address,undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in (os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "paged_plan.cpp"),
                os.path.join(ROOT, "tests", "host", "abi_fuzz.cpp")):
        obj = str(out / (os.path.basename(src) + ".o"))
        r = subprocess.run([hipcc] + flags + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(out / "abi_fuzz")
    r = subprocess.run([clang, "-fsanitize=address,undefined", "-o", exe] + objs,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


@pytest.mark.parametrize("seed", [1])
def test_abi_and_planner_are_sanitizer_clean(fuzz_binary, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([fuzz_binary, "1500", str(seed)], capture_output=True, text=True,
                       env=env, timeout=600)
    report = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
    assert "plans built" in r.stdout and "accepted by attn_bwd" in r.stdout, report
    print(r.stdout)
