"""The C ABI used from C alone: ``tests/c_abi/rnnt_c_check.c`` includes only ``include/rnnt.h`` (and the HIP
runtime's C API for its own buffers), links ``librnnt.so`` and the C oracle, and checks a small batch against the
oracle.  On the CPU it is compiled and linked (every symbol it uses resolves); on the GPU it runs."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "rnn_transducer_loss_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(out_dir) -> str:
    exe = os.path.join(str(out_dir), "rnnt_c_check")
    cmd = ["gcc", "-std=c99", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), os.path.join(ROOT, "tests", "c_abi", "rnnt_c_check.c"),
           os.path.join(ROOT, "oracle", "rnnt_oracle.c"), "-o", exe, "-L", LIBDIR, "-lrnnt",
           f"-Wl,-rpath,{LIBDIR}", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return exe


def test_c_program_compiles_and_links(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "librnnt.so")):
        pytest.skip("librnnt.so is not built")
    assert os.path.exists(_build(tmp_path))


@pytest.mark.gpu
def test_c_program_matches_the_oracle(tmp_path):
    exe = _build(tmp_path)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr)
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    assert "c-abi: worst loss rel" in res.stdout
