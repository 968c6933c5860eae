"""The C ABI used from C alone: tests/c_greedy_check.c allocates device memory
with the HIP runtime, calls spec_verify_greedy through include/spec_verify.h
on the null stream and checks the outputs against the greedy rule computed in
C (needs an MI355X; the program is compiled here with gcc, in seconds)."""

import os
import shutil
import subprocess

import pytest

import draft_token_verification_04_amd as sv
from gpu_helpers import note

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_plain_c_caller(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    libdir = os.path.dirname(sv.LIB_PATH)
    exe = tmp_path / "c_greedy_check"
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}",
                    os.path.join(HERE, "c_greedy_check.c"), "-o", str(exe),
                    f"-L{libdir}", "-lspecverify", f"-Wl,-rpath,{libdir}",
                    f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"], check=True)
    note("plain C caller: spec_verify_greedy B=16 K=5 V=3001")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 requests differ" in r.stdout
