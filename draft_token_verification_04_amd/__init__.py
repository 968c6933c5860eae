"""Python binding of libspecverify (batched speculative-decoding verification
on MI355X).

Argument marshalling only: every step of verification runs in the HIP kernels
of ``libspecverify.so``; this module checks tensor shapes/dtypes/devices,
allocates outputs and workspace with PyTorch, and passes raw device pointers
and the current HIP stream through the C ABI declared in
``include/spec_verify.h``.  There is no CPU fallback: if the library is not
built, or no GPU is visible, calls raise.

Entry points (same names as the C ABI):

* ``spec_verify_sample(target, draft, draft_tokens, u_accept, u_sample, T)``
* ``spec_verify_greedy(target, draft_tokens)``
* ``spec_verify_tree(target, node_tokens, parents)``
* ``spec_verify_greedy_lmhead``, ``spec_verify_tree_lmhead`` and
  ``spec_verify_sample_lmhead``: the same from the target's hidden states and
  LM head (logits formed on the matrix cores, never written)
* ``spec_commit_tree_kv``, ``spec_ngram_candidates``, ``sv_read_probe``
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SPECVERIFY_LIB names another build of the library to load (the sanitizer
# build of the host code, for instance); by default the in-tree one.
LIB_PATH = os.environ.get("SPECVERIFY_LIB") or os.path.join(HERE, "libspecverify.so")

SV_OK, SV_ERR_INVALID_ARG, SV_ERR_UNSUPPORTED, SV_ERR_WORKSPACE, SV_ERR_HIP, SV_ERR_SCRATCH = range(6)
SV_NOALLOC_SCRATCH_BYTES = 8 << 20
SV_F32, SV_BF16 = 0, 1
SV_MAX_TREE_NODES = 2048
KERNELS = ("rowstats", "accept", "resid_mass", "resid_select", "argmax", "match", "tree",
           "skip_stats", "skip_argmax", "commit", "lmhead", "ngram_count", "ngram_emit",
           "skip_tree", "read_probe", "lmhead_stats", "lmhead_rows", "merge_parts")

EXPORTS = ("sv_sample_workspace_bytes", "sv_greedy_workspace_bytes", "spec_verify_sample",
           "spec_verify_greedy", "spec_verify_tree", "spec_commit_tree_kv", "sv_status_string",
           "sv_version", "sv_lmhead_workspace_bytes", "spec_verify_greedy_lmhead",
           "spec_verify_tree_lmhead", "sv_ngram_workspace_bytes", "spec_ngram_candidates",
           "sv_read_probe", "sv_read_probe_folds", "sv_trace_begin", "sv_trace_end", "sv_kernel_name",
           "sv_sample_lmhead_workspace_bytes", "spec_verify_sample_lmhead", "spec_verify_sample_noalloc")


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class KernelTime(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("ms", ctypes.c_float)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libspecverify.so and declare its signatures (no GPU needed)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.sv_sample_workspace_bytes.argtypes = [I, I, I, I]
    lib.sv_sample_workspace_bytes.restype = Z
    lib.sv_greedy_workspace_bytes.argtypes = [I, I, I, I]
    lib.sv_greedy_workspace_bytes.restype = Z
    lib.spec_verify_sample.argtypes = [P, P, P, P, P, I, I, I, I, ctypes.c_float, P, P, P, P, P, P, Z, P]
    lib.spec_verify_sample.restype = I
    lib.spec_verify_sample_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, ctypes.c_float, P, P, P, P, P, P]
    lib.spec_verify_sample_noalloc.restype = I
    lib.spec_verify_greedy.argtypes = [P, P, I, I, I, I, P, P, P, P, Z, P]
    lib.spec_verify_greedy.restype = I
    lib.spec_verify_tree.argtypes = [P, P, P, I, I, I, I, P, P, P, P, P, Z, P]
    lib.spec_verify_tree.restype = I
    lib.spec_commit_tree_kv.argtypes = [P, P, I, I, I, I, P, P, P, P, I, P, P]
    lib.spec_commit_tree_kv.restype = I
    lib.sv_ngram_workspace_bytes.argtypes = [I, I]
    lib.sv_ngram_workspace_bytes.restype = Z
    lib.spec_ngram_candidates.argtypes = [P, I, I, P, P, I, I, P, P, P, P, Z, P]
    lib.spec_ngram_candidates.restype = I
    lib.sv_lmhead_workspace_bytes.argtypes = [I, I]
    lib.sv_lmhead_workspace_bytes.restype = Z
    lib.spec_verify_greedy_lmhead.argtypes = [P, P, P, I, I, I, I, P, P, P, P, Z, P]
    lib.spec_verify_greedy_lmhead.restype = I
    lib.spec_verify_tree_lmhead.argtypes = [P, P, P, P, I, I, I, I, P, P, P, P, P, Z, P]
    lib.spec_verify_tree_lmhead.restype = I
    lib.sv_sample_lmhead_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.sv_sample_lmhead_workspace_bytes.restype = Z
    lib.spec_verify_sample_lmhead.argtypes = [P, P, P, P, P, P, I, I, I, I, I, ctypes.c_float, P, P, P, P,
                                              P, P, Z, P]
    lib.spec_verify_sample_lmhead.restype = I
    lib.sv_read_probe.argtypes = [P, Z, P, P]
    lib.sv_read_probe.restype = I
    lib.sv_read_probe_folds.argtypes = [Z]
    lib.sv_read_probe_folds.restype = Z
    lib.sv_status_string.argtypes = [I]
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.sv_version.argtypes = []
    lib.sv_version.restype = ctypes.c_char_p
    lib.sv_trace_begin.argtypes = [I, ctypes.c_uint]
    lib.sv_trace_begin.restype = I
    lib.sv_trace_end.argtypes = [ctypes.POINTER(KernelTime), I]
    lib.sv_trace_end.restype = I
    lib.sv_kernel_name.argtypes = [I]
    lib.sv_kernel_name.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load_library().sv_status_string(status).decode()
    except RuntimeError:
        return "unknown"


def version() -> str:
    return load_library().sv_version().decode()


# ---- helpers -------------------------------------------------------------------

def _torch():
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("specverify needs a ROCm GPU; none is visible")
    return torch


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _check(t, name, ndim=None, dtype=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(torch, device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _hold(torch, device, stream, *tensors):
    """The kernels of a call made with ``stream=`` run on that stream, while
    this binding allocates the workspace and outputs on the current one.  When
    the two differ, mark those blocks as in use on ``stream`` so the caching
    allocator hands none of them to another allocation before the call's
    kernels are done with it."""
    if stream is None or stream.cuda_stream == torch.cuda.current_stream(device).cuda_stream:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _workspace(torch, nbytes, device, workspace):
    if workspace is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    _check(workspace, "workspace", device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise SpecVerifyError(SV_ERR_WORKSPACE, "workspace")
    return workspace


# ---- entry points ----------------------------------------------------------------

def sample_workspace_bytes(B, K, V, dtype_code) -> int:
    return int(load_library().sv_sample_workspace_bytes(B, K, V, dtype_code))


def greedy_workspace_bytes(B, rows_per_req, V, dtype_code) -> int:
    return int(load_library().sv_greedy_workspace_bytes(B, rows_per_req, V, dtype_code))


def spec_verify_sample(target, draft, draft_tokens, u_accept, u_sample, temperature, *,
                       lse=True, status=True, workspace=None, stream=None):
    """Stochastic chain verification.

    target [B,K+1,V] and draft [B,K,V] logits (bf16 or f32, same dtype),
    draft_tokens [B,K] int32, u_accept [B,K] and u_sample [B,K+1] float32 in
    [0,1).  Returns a dict with ``accept_len`` [B], ``tokens`` [B,K+1] and,
    when requested, ``lse_target`` [B,K+1], ``lse_draft`` [B,K], ``status`` [B].
    With lse=False (and K <= 31) the library skips the rows of positions after
    a request's first rejection (same outputs, fewer bytes).
    """
    torch = _torch()
    lib = load_library()
    _check(target, "target", 3)
    dev = target.device
    B, K1, V = target.shape
    K = K1 - 1
    dt = _dtype_code(target)
    if K > 0:
        _check(draft, "draft", 3, target.dtype, dev)
        if tuple(draft.shape) != (B, K, V):
            raise ValueError(f"draft must be [{B},{K},{V}], got {tuple(draft.shape)}")
        _check(draft_tokens, "draft_tokens", 2, torch.int32, dev)
        _check(u_accept, "u_accept", 2, torch.float32, dev)
        if tuple(draft_tokens.shape) != (B, K) or tuple(u_accept.shape) != (B, K):
            raise ValueError("draft_tokens and u_accept must be [B, K]")
    _check(u_sample, "u_sample", 2, torch.float32, dev)
    if tuple(u_sample.shape) != (B, K + 1):
        raise ValueError("u_sample must be [B, K+1]")
    out = dict(accept_len=torch.empty(B, dtype=torch.int32, device=dev),
               tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev))
    if lse:
        out["lse_target"] = torch.empty((B, K + 1), dtype=torch.float32, device=dev)
        out["lse_draft"] = torch.empty((B, K), dtype=torch.float32, device=dev)
    if status:
        out["status"] = torch.empty(B, dtype=torch.int32, device=dev)
    nbytes = lib.sv_sample_workspace_bytes(B, K, V, dt)
    ws = _workspace(torch, nbytes, dev, workspace)
    with torch.cuda.device(dev):
        rc = lib.spec_verify_sample(
            _ptr(target), _ptr(draft if K > 0 else None), _ptr(draft_tokens if K > 0 else None),
            _ptr(u_accept if K > 0 else None), _ptr(u_sample), B, K, V, dt, float(temperature),
            _ptr(out["accept_len"]), _ptr(out["tokens"]), _ptr(out.get("lse_target")),
            _ptr(out.get("lse_draft")), _ptr(out.get("status")), _ptr(ws),
            ws.numel() * ws.element_size(), _stream(torch, dev, stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_sample")
    _hold(torch, dev, stream, ws if workspace is None else None, *out.values())
    return out


def spec_verify_sample_noalloc(target, draft, draft_tokens, u_accept, u_sample, temperature, *,
                               lse=True, status=True, out=None, stream=None):
    """spec_verify_sample through the entry point that allocates nothing: its
    workspace is the library's static scratch of the current device (calls
    that overlap on one device race on it).  ``out`` may hold preallocated
    outputs (the dict spec_verify_sample returns); the binding allocates any
    that are missing.  Returns that dict."""
    torch = _torch()
    lib = load_library()
    _check(target, "target", 3)
    dev = target.device
    B, K1, V = target.shape
    K = K1 - 1
    dt = _dtype_code(target)
    if K > 0:
        _check(draft, "draft", 3, target.dtype, dev)
        if tuple(draft.shape) != (B, K, V):
            raise ValueError(f"draft must be [{B},{K},{V}], got {tuple(draft.shape)}")
        _check(draft_tokens, "draft_tokens", 2, torch.int32, dev)
        _check(u_accept, "u_accept", 2, torch.float32, dev)
        if tuple(draft_tokens.shape) != (B, K) or tuple(u_accept.shape) != (B, K):
            raise ValueError("draft_tokens and u_accept must be [B, K]")
    _check(u_sample, "u_sample", 2, torch.float32, dev)
    if tuple(u_sample.shape) != (B, K + 1):
        raise ValueError("u_sample must be [B, K+1]")
    out = dict(out or {})
    shapes = {"accept_len": ((B,), torch.int32), "tokens": ((B, K + 1), torch.int32)}
    if lse:
        shapes.update(lse_target=((B, K + 1), torch.float32), lse_draft=((B, K), torch.float32))
    if status:
        shapes["status"] = ((B,), torch.int32)
    for name, (shape, dtype) in shapes.items():
        if name in out:
            _check(out[name], name, len(shape), dtype, dev)
            if tuple(out[name].shape) != shape:
                raise ValueError(f"{name} must be {list(shape)}")
        else:
            out[name] = torch.empty(shape, dtype=dtype, device=dev)
    with torch.cuda.device(dev):
        rc = lib.spec_verify_sample_noalloc(
            _ptr(target), _ptr(draft if K > 0 else None), _ptr(draft_tokens if K > 0 else None),
            _ptr(u_accept if K > 0 else None), _ptr(u_sample), B, K, V, dt, float(temperature),
            _ptr(out["accept_len"]), _ptr(out["tokens"]), _ptr(out.get("lse_target") if lse else None),
            _ptr(out.get("lse_draft") if lse else None), _ptr(out.get("status") if status else None),
            _stream(torch, dev, stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_sample_noalloc")
    _hold(torch, dev, stream, *out.values())
    return out


def spec_verify_greedy(target, draft_tokens, *, status=True, workspace=None, stream=None):
    """Greedy chain verification: target [B,K+1,V], draft_tokens [B,K] int32.
    Returns ``accept_len`` [B], ``tokens`` [B,K+1] and ``status`` [B]."""
    torch = _torch()
    lib = load_library()
    _check(target, "target", 3)
    dev = target.device
    B, K1, V = target.shape
    K = K1 - 1
    dt = _dtype_code(target)
    if K > 0:
        _check(draft_tokens, "draft_tokens", 2, torch.int32, dev)
        if tuple(draft_tokens.shape) != (B, K):
            raise ValueError("draft_tokens must be [B, K]")
    out = dict(accept_len=torch.empty(B, dtype=torch.int32, device=dev),
               tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev))
    if status:
        out["status"] = torch.empty(B, dtype=torch.int32, device=dev)
    ws = _workspace(torch, lib.sv_greedy_workspace_bytes(B, K + 1, V, dt), dev, workspace)
    with torch.cuda.device(dev):
        rc = lib.spec_verify_greedy(
            _ptr(target), _ptr(draft_tokens if K > 0 else None), B, K, V, dt,
            _ptr(out["accept_len"]), _ptr(out["tokens"]), _ptr(out.get("status")), _ptr(ws),
            ws.numel() * ws.element_size(), _stream(torch, dev, stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_greedy")
    _hold(torch, dev, stream, ws if workspace is None else None, *out.values())
    return out


def spec_verify_tree(target, node_tokens, parents, *, status=True, workspace=None, stream=None):
    """Greedy tree verification: target [B,N,V], node_tokens [B,N] and
    parents [B,N] int32.  Returns ``accept_len`` [B], ``path`` [B,N],
    ``tokens`` [B,N] and ``status`` [B]."""
    torch = _torch()
    lib = load_library()
    _check(target, "target", 3)
    dev = target.device
    B, N, V = target.shape
    dt = _dtype_code(target)
    _check(node_tokens, "node_tokens", 2, torch.int32, dev)
    _check(parents, "parents", 2, torch.int32, dev)
    if tuple(node_tokens.shape) != (B, N) or tuple(parents.shape) != (B, N):
        raise ValueError("node_tokens and parents must be [B, N]")
    out = dict(accept_len=torch.empty(B, dtype=torch.int32, device=dev),
               path=torch.empty((B, N), dtype=torch.int32, device=dev),
               tokens=torch.empty((B, N), dtype=torch.int32, device=dev))
    if status:
        out["status"] = torch.empty(B, dtype=torch.int32, device=dev)
    ws = _workspace(torch, lib.sv_greedy_workspace_bytes(B, N, V, dt), dev, workspace)
    with torch.cuda.device(dev):
        rc = lib.spec_verify_tree(
            _ptr(target), _ptr(node_tokens), _ptr(parents), B, N, V, dt, _ptr(out["accept_len"]),
            _ptr(out["path"]), _ptr(out["tokens"]), _ptr(out.get("status")), _ptr(ws),
            ws.numel() * ws.element_size(), _stream(torch, dev, stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_tree")
    _hold(torch, dev, stream, ws if workspace is None else None, *out.values())
    return out


def _lmhead_operands(torch, hidden, lm_head, lead):
    _check(hidden, "hidden", len(lead) + 1, torch.bfloat16)
    dev = hidden.device
    _check(lm_head, "lm_head", 2, torch.bfloat16, dev)
    D = hidden.shape[-1]
    V = lm_head.shape[0]
    if lm_head.shape[1] != D:
        raise ValueError(f"lm_head must be [V, {D}], got {tuple(lm_head.shape)}")
    return dev, D, V


def spec_verify_greedy_lmhead(hidden, lm_head, draft_tokens, *, status=True, workspace=None,
                              stream=None):
    """Greedy chain verification on the logits hidden @ lm_head.T, which are
    never materialised: hidden [B, K+1, D] bf16, lm_head [V, D] bf16,
    draft_tokens [B, K] int32.  Returns ``accept_len`` [B], ``tokens`` [B, K+1]
    and ``status`` [B]."""
    torch = _torch()
    lib = load_library()
    dev, D, V = _lmhead_operands(torch, hidden, lm_head, (0, 0))
    B, R = hidden.shape[:2]
    K = R - 1
    _check(draft_tokens, "draft_tokens", 2, torch.int32, dev)
    if tuple(draft_tokens.shape) != (B, K):
        raise ValueError(f"draft_tokens must be [{B}, {K}]")
    out = dict(accept_len=torch.empty(B, dtype=torch.int32, device=dev),
               tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev))
    if status:
        out["status"] = torch.empty(B, dtype=torch.int32, device=dev)
    ws = _workspace(torch, lib.sv_lmhead_workspace_bytes(B * R, V), dev, workspace)
    with torch.cuda.device(dev):
        rc = lib.spec_verify_greedy_lmhead(
            _ptr(hidden), _ptr(lm_head), _ptr(draft_tokens) if K else None, B, K, D, V,
            _ptr(out["accept_len"]), _ptr(out["tokens"]), _ptr(out.get("status")), _ptr(ws),
            ws.numel() * ws.element_size(), _stream(torch, dev, stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_greedy_lmhead")
    _hold(torch, dev, stream, ws if workspace is None else None, *out.values())
    return out


def spec_verify_tree_lmhead(hidden, lm_head, node_tokens, parents, *, status=True, workspace=None,
                            stream=None):
    """Greedy tree verification on the logits hidden @ lm_head.T (never
    materialised): hidden [B, N, D] bf16, lm_head [V, D] bf16, node_tokens and
    parents [B, N] int32.  Returns ``accept_len``, ``path``, ``tokens``, ``status``."""
    torch = _torch()
    lib = load_library()
    dev, D, V = _lmhead_operands(torch, hidden, lm_head, (0, 0))
    B, N = hidden.shape[:2]
    _check(node_tokens, "node_tokens", 2, torch.int32, dev)
    _check(parents, "parents", 2, torch.int32, dev)
    if tuple(node_tokens.shape) != (B, N) or tuple(parents.shape) != (B, N):
        raise ValueError("node_tokens and parents must be [B, N]")
    out = dict(accept_len=torch.empty(B, dtype=torch.int32, device=dev),
               path=torch.empty((B, N), dtype=torch.int32, device=dev),
               tokens=torch.empty((B, N), dtype=torch.int32, device=dev))
    if status:
        out["status"] = torch.empty(B, dtype=torch.int32, device=dev)
    ws = _workspace(torch, lib.sv_lmhead_workspace_bytes(B * N, V), dev, workspace)
    with torch.cuda.device(dev):
        rc = lib.spec_verify_tree_lmhead(
            _ptr(hidden), _ptr(lm_head), _ptr(node_tokens), _ptr(parents), B, N, D, V,
            _ptr(out["accept_len"]), _ptr(out["path"]), _ptr(out["tokens"]), _ptr(out.get("status")),
            _ptr(ws), ws.numel() * ws.element_size(), _stream(torch, dev, stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_tree_lmhead")
    _hold(torch, dev, stream, ws if workspace is None else None, *out.values())
    return out


def spec_verify_sample_lmhead(hidden, lm_head, draft, draft_tokens, u_accept, u_sample, temperature, *,
                              lse=True, status=True, workspace=None, stream=None):
    """Stochastic chain verification on the target logits hidden @ lm_head.T,
    never materialised: hidden [B, K+1, D] bf16, lm_head [V, D] bf16, draft
    [B, K, V] logits (bf16 or f32), draft_tokens [B, K] int32, u_accept [B, K]
    and u_sample [B, K+1] float32.  Returns what spec_verify_sample returns."""
    torch = _torch()
    lib = load_library()
    dev, D, V = _lmhead_operands(torch, hidden, lm_head, (0, 0))
    B, R = hidden.shape[:2]
    K = R - 1
    dt = SV_BF16
    if K > 0:
        _check(draft, "draft", 3, device=dev)
        dt = _dtype_code(draft)
        if tuple(draft.shape) != (B, K, V):
            raise ValueError(f"draft must be [{B},{K},{V}], got {tuple(draft.shape)}")
        _check(draft_tokens, "draft_tokens", 2, torch.int32, dev)
        _check(u_accept, "u_accept", 2, torch.float32, dev)
        if tuple(draft_tokens.shape) != (B, K) or tuple(u_accept.shape) != (B, K):
            raise ValueError("draft_tokens and u_accept must be [B, K]")
    _check(u_sample, "u_sample", 2, torch.float32, dev)
    if tuple(u_sample.shape) != (B, K + 1):
        raise ValueError("u_sample must be [B, K+1]")
    out = dict(accept_len=torch.empty(B, dtype=torch.int32, device=dev),
               tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev))
    if lse:
        out["lse_target"] = torch.empty((B, K + 1), dtype=torch.float32, device=dev)
        out["lse_draft"] = torch.empty((B, K), dtype=torch.float32, device=dev)
    if status:
        out["status"] = torch.empty(B, dtype=torch.int32, device=dev)
    ws = _workspace(torch, lib.sv_sample_lmhead_workspace_bytes(B, K, D, V, dt), dev, workspace)
    with torch.cuda.device(dev):
        rc = lib.spec_verify_sample_lmhead(
            _ptr(hidden), _ptr(lm_head), _ptr(draft if K > 0 else None),
            _ptr(draft_tokens if K > 0 else None), _ptr(u_accept if K > 0 else None), _ptr(u_sample),
            B, K, D, V, dt, float(temperature), _ptr(out["accept_len"]), _ptr(out["tokens"]),
            _ptr(out.get("lse_target")), _ptr(out.get("lse_draft")), _ptr(out.get("status")), _ptr(ws),
            ws.numel() * ws.element_size(), _stream(torch, dev, stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_sample_lmhead")
    _hold(torch, dev, stream, ws if workspace is None else None, *out.values())
    return out


def spec_ngram_candidates(context, lengths, queries, cap, *, status=True, workspace=None, stream=None):
    """AdaPLD lexical retrieval: context [B, L], lengths [B], queries [B, n]
    (int32 GPU tensors).  Returns ``count`` [B], ``positions`` [B, cap]
    (ascending, -1 padded) and ``status`` [B]."""
    torch = _torch()
    lib = load_library()
    _check(context, "context", 2, torch.int32)
    dev = context.device
    B, L = context.shape
    _check(lengths, "lengths", 1, torch.int32, dev)
    _check(queries, "queries", 2, torch.int32, dev)
    if lengths.shape[0] != B or queries.shape[0] != B:
        raise ValueError("lengths and queries must have B rows")
    n = queries.shape[1]
    out = dict(count=torch.empty(B, dtype=torch.int32, device=dev),
               positions=torch.empty((B, cap), dtype=torch.int32, device=dev))
    if status:
        out["status"] = torch.empty(B, dtype=torch.int32, device=dev)
    ws = _workspace(torch, lib.sv_ngram_workspace_bytes(B, L), dev, workspace)
    with torch.cuda.device(dev):
        rc = lib.spec_ngram_candidates(_ptr(context), B, L, _ptr(lengths), _ptr(queries), n, cap,
                                       _ptr(out["count"]), _ptr(out["positions"]) if cap else None,
                                       _ptr(out.get("status")), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(torch, dev, stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_ngram_candidates")
    _hold(torch, dev, stream, ws if workspace is None else None, *out.values())
    return out


def spec_commit_tree_kv(kv, tree_base, commit_base, accept_len, path, *, out=None, status=True,
                        stream=None):
    """Move the KV rows of each request's accepted tree path into consecutive
    slots.  kv: [G, B, S, ...] GPU tensor (any dtype; the trailing dimensions
    of one slot form a row of a multiple of 16 bytes); tree_base, commit_base,
    accept_len [B] and path [B, N] int32 (accept_len and path as returned by
    spec_verify_tree).  In place when ``out`` is None, else into ``out`` (same
    shape and dtype as kv).  Returns the per-request status [B] (or None)."""
    torch = _torch()
    lib = load_library()
    if kv is None or kv.dim() < 3:
        raise ValueError("kv must be [G, B, S, ...]")
    _check(kv, "kv")
    dev = kv.device
    G, B, S = kv.shape[:3]
    row_bytes = kv[0, 0, 0].numel() * kv.element_size() if kv.numel() else 0
    dst = kv if out is None else out
    if out is not None:
        _check(out, "out", kv.dim(), kv.dtype, dev)
        if tuple(out.shape) != tuple(kv.shape):
            raise ValueError("out must have the shape of kv")
    for name, t in (("tree_base", tree_base), ("commit_base", commit_base), ("accept_len", accept_len)):
        _check(t, name, 1, torch.int32, dev)
        if t.shape[0] != B:
            raise ValueError(f"{name} must be [B]")
    _check(path, "path", 2, torch.int32, dev)
    if path.shape[0] != B:
        raise ValueError("path must be [B, N]")
    N = path.shape[1]
    st = torch.empty(B, dtype=torch.int32, device=dev) if status else None
    with torch.cuda.device(dev):
        rc = lib.spec_commit_tree_kv(_ptr(kv), _ptr(dst), G, B, S, row_bytes, _ptr(tree_base),
                                     _ptr(commit_base), _ptr(accept_len), _ptr(path), N, _ptr(st),
                                     _stream(torch, dev, stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_commit_tree_kv")
    _hold(torch, dev, stream, st)
    return st


def sv_read_probe(buf, *, folds=None, stream=None):
    """Read every byte of the GPU tensor ``buf`` once (a measurement aid: the
    read rate this device reaches).  Returns ``folds`` (int32), entry i the XOR
    of the 32-bit words of the buffer's i-th 16 KB."""
    torch = _torch()
    lib = load_library()
    _check(buf, "buf")
    dev = buf.device
    nbytes = buf.numel() * buf.element_size()
    nf = lib.sv_read_probe_folds(nbytes)
    if folds is None:
        folds = torch.empty(max(nf, 1), dtype=torch.int32, device=dev)
    elif folds.numel() < nf or folds.dtype != torch.int32 or folds.device != dev:
        raise ValueError(f"folds must be int32 on {dev} with at least {nf} entries")
    with torch.cuda.device(dev):
        rc = lib.sv_read_probe(_ptr(buf), nbytes, _ptr(folds), _stream(torch, dev, stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "sv_read_probe")
    _hold(torch, dev, stream, folds)
    return folds


# ---- per-kernel timing -----------------------------------------------------------

def trace_begin(capacity: int = 4096, kernels=None) -> None:
    """Time every launch (kernels=None) or only the named kernels."""
    mask = 0
    for k in kernels or ():
        mask |= 1 << KERNELS.index(k)
    rc = load_library().sv_trace_begin(capacity, mask)
    if rc != SV_OK:
        raise SpecVerifyError(rc, "sv_trace_begin")


def trace_end(max_records: int = 1 << 16):
    """Stop tracing; return [(kernel_name, ms), ...] in launch order."""
    lib = load_library()
    recs = (KernelTime * max_records)()
    n = lib.sv_trace_end(recs, max_records)
    return [(lib.sv_kernel_name(recs[i].kernel).decode(), float(recs[i].ms))
            for i in range(min(n, max_records))]
