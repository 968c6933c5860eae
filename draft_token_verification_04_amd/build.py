"""Build libspecverify.so (the HIP library) in-tree for gfx950 with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libspecverify.so")
SOURCES = ["sv_api.hip", "sv_sample.hip", "sv_greedy.hip", "sv_commit.hip", "sv_lmhead.hip",
           "sv_ngram.hip", "sv_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libspecverify")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
        # no packed fp32 instructions (v_pk_*_f32) anywhere in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def source_digest(extra=()) -> str:
    """Hash of everything the library is built from: the kernel and API sources,
    the headers, and the compiler flags."""
    import hashlib

    h = hashlib.sha256()
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".hpp", ".h")):
                h.update(name.encode())
                with open(os.path.join(d, name), "rb") as f:
                    h.update(f.read())
    h.update(" ".join([*flags(), *extra, *SOURCES]).encode())
    return h.hexdigest()


def digest_path(out: str = LIB) -> str:
    return out + ".srchash"


def is_current(out: str = LIB) -> bool:
    """True when `out` exists and was built from the sources as they are now."""
    try:
        with open(digest_path(out)) as f:
            return os.path.exists(out) and f.read().strip() == source_digest()
    except OSError:
        return False


def build(out: str = LIB, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *flags(), *extra, *srcs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    if not extra:
        with open(digest_path(out), "w") as f:
            f.write(source_digest() + "\n")
    return out


if __name__ == "__main__":
    print(build())
