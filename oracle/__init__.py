"""CPU oracle for batched speculative-decoding verification (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import this package.  It wraps ``sv_oracle.c`` (plain C, fp64, scalar),
which shares no code with the HIP library.  See the header of ``sv_oracle.c``
for the passages each function follows and the readings it takes.

Arrays are numpy: logits are float32 or uint16 (bfloat16 bit patterns), token
and parent arrays int32, uniforms float32.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sv_oracle.c")
LIB = os.path.join(HERE, "libsv_oracle.so")

F32, BF16 = 0, 1

_lib = None


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP over requests)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-fopenmp", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.sv_oracle_sample.argtypes = [P, P, I, P, P, P, I, I, I, D, P, P, P, P, P, P, P, P, P, I]
    lib.sv_oracle_greedy.argtypes = [P, I, P, I, I, I, P, P, P, I]
    lib.sv_oracle_tree.argtypes = [P, I, P, P, I, I, I, P, P, P, P, I]
    lib.sv_oracle_row_stats.argtypes = [P, I, I, I, D, P, P, P]
    lib.sv_oracle_argmax.argtypes = [P, I, I, I, P]
    for f in (lib.sv_oracle_sample, lib.sv_oracle_greedy, lib.sv_oracle_tree,
              lib.sv_oracle_row_stats, lib.sv_oracle_argmax):
        f.restype = ctypes.c_int
    return lib


def load(path: str = LIB):
    """Load the compiled oracle (building it first if it is missing)."""
    global _lib
    if path == LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    lib = _bind(ctypes.CDLL(path))
    if path == LIB:
        _lib = lib
    return lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def verify_sample(target, draft, draft_tokens, u_accept, u_sample, T, threads=None, lib=None, lse=True):
    """Stochastic chain verification.  Returns a dict of numpy arrays:
    accept_len [B], tokens [B,K+1], lse_target [B,K+1], lse_draft [B,K] (left
    out with lse=False, which spares the rows no draw consumes),
    status [B], margin [B] (smallest consumed-draw margin), margin_accept [B]
    (smallest margin of the consumed acceptance draws, which alone decide
    accept_len; +inf when none), margin_sample [B] (the sample draw's margin),
    Z [B]."""
    lib = lib or load()
    B, K1, V = target.shape
    K = K1 - 1
    dt = _dt(target)
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft) if K > 0 else np.zeros((B, 0, V), target.dtype)
    if _dt(draft) != dt or draft.shape != (B, K, V):
        raise ValueError("draft logits must match the target dtype and be [B, K, V]")
    x = _c(draft_tokens, np.int32).reshape(B, K)
    ua = _c(u_accept, np.float32).reshape(B, K)
    us = _c(u_sample, np.float32).reshape(B, K + 1)
    out = dict(accept_len=np.empty(B, np.int32), tokens=np.empty((B, K + 1), np.int32),
               status=np.empty(B, np.int32), margin=np.empty(B), margin_accept=np.empty(B),
               margin_sample=np.empty(B), Z=np.empty(B))
    if lse:
        out.update(lse_target=np.empty((B, K + 1)), lse_draft=np.empty((B, K)))
    rc = lib.sv_oracle_sample(_ptr(target), _ptr(draft), dt, _ptr(x), _ptr(ua), _ptr(us), B, K, V,
                              float(T), _ptr(out["accept_len"]), _ptr(out["tokens"]),
                              _ptr(out.get("lse_target")), _ptr(out.get("lse_draft")), _ptr(out["status"]),
                              _ptr(out["margin"]), _ptr(out["margin_accept"]),
                              _ptr(out["margin_sample"]), _ptr(out["Z"]), threads or default_threads())
    if rc:
        raise ValueError("oracle rejected the arguments")
    return out


def verify_greedy(target, draft_tokens, threads=None, lib=None):
    """Greedy chain verification: accept_len [B], tokens [B,K+1], status [B]."""
    lib = lib or load()
    B, K1, V = target.shape
    K = K1 - 1
    target = np.ascontiguousarray(target)
    x = _c(draft_tokens, np.int32).reshape(B, K)
    out = dict(accept_len=np.empty(B, np.int32), tokens=np.empty((B, K + 1), np.int32),
               status=np.empty(B, np.int32))
    rc = lib.sv_oracle_greedy(_ptr(target), _dt(target), _ptr(x), B, K, V, _ptr(out["accept_len"]),
                              _ptr(out["tokens"]), _ptr(out["status"]), threads or default_threads())
    if rc:
        raise ValueError("oracle rejected the arguments")
    return out


def verify_tree(target, node_tokens, parents, threads=None, lib=None):
    """Greedy tree verification: accept_len [B], path [B,N], tokens [B,N], status [B]."""
    lib = lib or load()
    B, N, V = target.shape
    target = np.ascontiguousarray(target)
    tk = _c(node_tokens, np.int32).reshape(B, N)
    par = _c(parents, np.int32).reshape(B, N)
    out = dict(accept_len=np.empty(B, np.int32), path=np.empty((B, N), np.int32),
               tokens=np.empty((B, N), np.int32), status=np.empty(B, np.int32))
    rc = lib.sv_oracle_tree(_ptr(target), _dt(target), _ptr(tk), _ptr(par), B, N, V,
                            _ptr(out["accept_len"]), _ptr(out["path"]), _ptr(out["tokens"]),
                            _ptr(out["status"]), threads or default_threads())
    if rc:
        raise ValueError("oracle rejected the arguments")
    return out


def row_stats(logits, T, lib=None):
    """Per-row max m, normaliser s = sum exp((L-m)/T) and lse = m/T + log s."""
    lib = lib or load()
    a = np.ascontiguousarray(logits)
    V = a.shape[-1]
    rows = a.size // V
    m, s, lse = np.empty(rows), np.empty(rows), np.empty(rows)
    rc = lib.sv_oracle_row_stats(_ptr(a), _dt(a), rows, V, float(T), _ptr(m), _ptr(s), _ptr(lse))
    if rc:
        raise ValueError("oracle rejected the arguments")
    shp = a.shape[:-1]
    return m.reshape(shp), s.reshape(shp), lse.reshape(shp)


def argmax(logits, lib=None):
    """Lowest-index argmax of every row."""
    lib = lib or load()
    a = np.ascontiguousarray(logits)
    V = a.shape[-1]
    rows = a.size // V
    out = np.empty(rows, np.int32)
    if lib.sv_oracle_argmax(_ptr(a), _dt(a), rows, V, _ptr(out)):
        raise ValueError("oracle rejected the arguments")
    return out.reshape(a.shape[:-1])


def flagged(margin: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Requests that consumed a draw within eps of its decision boundary."""
    return np.asarray(margin) <= eps
