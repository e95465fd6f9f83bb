"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

api.cpp (validation, workspace planning, launch sequencing) and hilbert.cpp (the
host Hilbert order) are compiled by g++ with -fsanitize=address,undefined into a
host-only library whose kernel launchers are stand-ins (tests/host/abi_host_stubs.cpp;
no test here reaches a launch or a device lookup), and tests/test_abi.py runs against that library in
a child process with the ASan runtime preloaded.  Any out-of-bounds access, use of
freed memory or undefined behaviour on those paths aborts the child.
"""

import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_quantized_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def sanitized_lib():
    asan = _gcc_runtime("libasan.so")
    if asan is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("no libasan or no HIP host runtime on this machine")
    d = tempfile.mkdtemp(prefix="sparge_asan_")
    out = os.path.join(d, "libsparge_asan.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           # device-side spellings the host compiler lacks (the static scratch of the
           # allocation-free entry point becomes ordinary host storage here)
           "-D__align__(n)=__attribute__((aligned(n)))", "-DHIP_SYMBOL(x)=((const void*)&(x))",
           "-x", "c++", os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "hilbert.cpp"),
           os.path.join(ROOT, "tests", "host", "abi_host_stubs.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out, asan


def test_sanitized_build_is_instrumented(sanitized_lib):
    lib, _ = sanitized_lib
    und = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_init" in und or "__asan_report_load8" in und
    assert "__ubsan_handle" in und


def test_abi_tests_pass_under_sanitizers(sanitized_lib):
    lib, asan = sanitized_lib
    env = dict(os.environ)
    env["SPARGE_LIB"] = lib
    prev = env.get("LD_PRELOAD")
    env["LD_PRELOAD"] = asan + (":" + prev if prev else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    log = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, log
    assert "AddressSanitizer" not in log and "runtime error" not in log, log
    assert " passed" in r.stdout
