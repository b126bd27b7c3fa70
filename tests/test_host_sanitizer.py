"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

librnnt is rebuilt into a temporary directory with the sanitizers on its host code only (each flag given to the
host compilation alone; the device code is built as usual and never runs here), and
``tests/c_abi/rnnt_host_check.c``, itself built with the same sanitizers, drives every host-only path of the C ABI:
validation and each refusal, the longest-first schedule and workspace layouts of random batches (its chunk
table checked to cover every node once), the refusals of the allocation-free call, the timing switches.  Any
sanitizer report, or a failed check, fails the test.  Leaks are reported except those inside the HIP runtime's
own initialisation.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rnn_transducer_loss_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
# host-side sanitizers: every flag follows -Xarch_host, so it applies to the host compilation only
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
HOST_SAN += "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer".split()


def _hipcc():
    for c in (os.path.join(ROCM, "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not available")


def _clang():
    c = os.path.join(ROCM, "llvm", "bin", "clang")
    if not os.path.exists(c):
        pytest.skip("ROCm clang not available")
    return c


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    lib = os.path.join(str(d), "librnnt.so")
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + HOST_SAN + [
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", lib,
           os.path.join(CSRC, "rnnt_api.cpp"), os.path.join(CSRC, "rnnt_kernels.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    exe = os.path.join(str(d), "rnnt_host_check")
    cmd = [_clang(), "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi", "rnnt_host_check.c"),
           "-o", exe, "-L", str(d), "-lrnnt", f"-Wl,-rpath,{d}", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{ROCM}/lib", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    supp = os.path.join(str(d), "lsan.supp")
    with open(supp, "w") as f:
        f.write("leak:libamdhip64\nleak:libhsa-runtime64\nleak:libhsakmt\nleak:libdrm\n")
    return exe, supp


def test_host_paths_clean_under_address_and_ub_sanitizers(sanitized):
    exe, supp = sanitized
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["LSAN_OPTIONS"] = f"suppressions={supp}"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = res.stdout + res.stderr
    print(out[-4000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out and "LeakSanitizer" not in out
    assert res.returncode == 0, out[-3000:]
    assert "host-check: ok" in res.stdout
