"""The C ABI used from plain C99, without the Python binding: tests/c_abi/
df11_c_check.c is compiled against include/df11.h and linked with the built
library.  On the CPU it runs the host codec calls; on a GPU it also uploads
the unit and checks df11_decompress_block / _tensor bit for bit."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "df11_c_check.c")
LIBDIR = os.path.join(ROOT, "entropy_decoding_amd")
ROCM = "/opt/rocm"


def _build(tmp_path, gpu: bool):
    exe = str(tmp_path / ("df11_c_check_gpu" if gpu else "df11_c_check"))
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-I", os.path.join(ROOT, "include"), SRC,
           "-o", exe, "-L", LIBDIR, "-ldf11", f"-Wl,-rpath,{LIBDIR}"]
    if gpu:
        cmd += ["-DDF11_C_CHECK_GPU", "-D__HIP_PLATFORM_AMD__", "-I", f"{ROCM}/include",
                "-L", f"{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]
    else:
        cmd.insert(1, "-Werror")
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_c_program_host_calls(tmp_path):
    exe = _build(tmp_path, gpu=False)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "host:" in r.stdout


@pytest.mark.gpu
def test_c_program_decompresses_on_the_gpu(tmp_path):
    exe = _build(tmp_path, gpu=True)
    print("[gpu] C program: df11_decompress_block / _tensor", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bit-exact" in r.stdout and "window counts consistent" in r.stdout
