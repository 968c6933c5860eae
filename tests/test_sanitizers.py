"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code (CPU only).

* The oracle (oracle/sv_oracle.c), built with gcc under both sanitizers, runs
  every pin that checks it (the fast battery plus the full-vocabulary margin
  recomputation) in a child process with the sanitizer runtime preloaded.
* The library's host code (argument checks, workspace layout, the scratch
  lookup, the tracer) is built with both sanitizers on the host side only
  (device code is built as usual), and the ABI tests that need no GPU run
  against that build.

Any report aborts the child, which fails the test.  Nothing here touches a GPU.
"""

import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child_env(preload, **extra):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env["LD_PRELOAD"] = preload
    env["OMP_NUM_THREADS"] = "4"
    env.update(extra)
    return env


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    rt = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("gcc has no AddressSanitizer runtime")
    so = tmp_path / "liborc_san.so"
    subprocess.run([gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fPIC", "-shared", "-fopenmp",
                    os.path.join(ROOT, "oracle", "sv_oracle.c"), "-o", str(so), "-lm"], check=True)
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import oracle, pins\n"
            "lib = oracle.load(%r)\n"
            "for p in pins.ALL_FAST: p(lib)\n"
            "pins.pin_margins_full_vocab(lib)\n"
            "print('sanitized oracle: every pin passed')\n") % (ROOT, HERE, str(so))
    r = subprocess.run([sys.executable, "-c", code], env=_child_env(rt), capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "every pin passed" in r.stdout


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    from draft_token_verification_04_amd import build as hb

    try:
        hb.hipcc()
    except RuntimeError:
        pytest.skip("no hipcc")
    llvm = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "lib", "clang")
    rts = [os.path.join(llvm, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
           for v in (os.listdir(llvm) if os.path.isdir(llvm) else [])]
    rts = [p for p in rts if os.path.exists(p)]
    if not rts:
        pytest.skip("no clang AddressSanitizer runtime")
    so = str(tmp_path / "libspecverify_san.so")
    # host side only: each sanitizer flag goes to the host compilation
    hb.build(so, extra=("-g",
                        "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-sanitize-recover=all",
                        "-Xarch_host", "-fno-omit-frame-pointer",
                        "-shared-libsan"))
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi.py"), "-q", "-s",
                        "-m", "not gpu", "-p", "no:cacheprovider", "-k", "not header and not stale"],
                       env=_child_env(rts[0], SPECVERIFY_LIB=so), cwd=ROOT, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-4000:]
    assert " passed" in r.stdout and "failed" not in r.stdout
