"""CPU oracle for verification fused with the LM-head projection (test
infrastructure: only the tests, ``__graft_entry__``'s smoke check and
``bench.py``'s CPU baseline may use it).

The logits of a verified position are the projection of the target's final
hidden state onto the vocabulary, logits = H W^T (the speculative-decoding
tutorial page, section "一轮推测解码究竟发生什么": the target scores every
draft position in one parallel pass; the DLite notes, section 2: this D x V
projection is the per-position cost).  Greedy acceptance on those logits is
the rule of the same tutorial page, section "为什么“猜错再改”不会偏离目标分布"
(keep a draft while it equals the target's argmax; emit the argmax at the
first mismatch), and the AdaPLD page's tree rule (section 3.3, Algorithm 1)
for trees.

The oracle forms the logits in fp64 from the bf16 inputs (products and sums
of bf16 values: the only rounding is fp64's), takes the first maximum of each
row, and applies the chain or tree rule written out below.  Speculative
sampling on those logits (``verify_sample``) is the sampling oracle of
``oracle/sv_oracle.c`` applied to them, rounded to fp32 on the way in: exact
for the exact recipe, whose logits are fp32 numbers, and within half an fp32
ulp of the product otherwise.

The device path accumulates in fp32 in an order it does not fix.  With
products of bf16 values exact in fp32, any order's error on a logit is at
most gamma_{D-1} * sum_k |h_k| |w_k|, gamma_n = n u / (1 - n u), u = 2^-24 (the
classical bound for a sum of D terms under any summation tree).  A row is
*certain* when its first maximum beats every other entry by more than the two
entries' bounds together: then every admissible fp32 result has the same
argmax.  Uncertain rows are flagged; a chain request (or a tree request) is
flagged when a row its result depends on is uncertain.  For the "exact"
workload recipe every partial sum is representable in fp32, so no row is
flagged (``exact=True`` skips the bound).

Pins: tests/test_lmhead_oracle.py (integer arithmetic on small cases, the
bound against fp32 sums in several orders and against a sum built to lose
about half of it, the C oracle on exactly representable logits, brute-force
tree walks, sampling on the projection against sampling on integer-exact
logits).  tests/test_lmhead_oracle_mutants.py plants a mistake in one
function at a time and checks that a pin fails.
"""

from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# Vocabulary rows widened to fp64 at a time, blocks on threads (memory and
# time only: each logit is still one full fp64 dot product).
_V_BLOCK = 8192


def _project(hidden_bits: np.ndarray, lm_head_bits: np.ndarray, absolute: bool) -> np.ndarray:
    from concurrent.futures import ThreadPoolExecutor

    H = bf16_to_f64(hidden_bits)
    if absolute:
        H = np.abs(H)
    V = lm_head_bits.shape[0]
    out = np.empty(H.shape[:-1] + (V,), dtype=np.float64)

    def block(v0):
        W = bf16_to_f64(lm_head_bits[v0:v0 + _V_BLOCK])
        out[..., v0:v0 + W.shape[0]] = H @ (np.abs(W) if absolute else W).T

    from threadpoolctl import threadpool_limits

    with threadpool_limits(1), ThreadPoolExecutor(8) as ex:
        list(ex.map(block, range(0, V, _V_BLOCK)))
    return out


def logits(hidden_bits: np.ndarray, lm_head_bits: np.ndarray) -> np.ndarray:
    """fp64 H W^T for hidden [..., D] and lm_head [V, D] (bf16 bits)."""
    return _project(hidden_bits, lm_head_bits, False)


def accumulation_bound(hidden_bits: np.ndarray, lm_head_bits: np.ndarray) -> np.ndarray:
    """Bound on |fp32 result - exact logit| for any summation order."""
    D = hidden_bits.shape[-1]
    n = D - 1
    gamma = n * U32 / (1.0 - n * U32)
    return gamma * _project(hidden_bits, lm_head_bits, True)


def row_argmax(L: np.ndarray, E: np.ndarray | None):
    """First maximum of each row and whether it is certain under the bound E."""
    a = np.argmax(L, axis=-1)
    if E is None:
        return a, np.ones(a.shape, dtype=bool)
    top = np.take_along_axis(L, a[..., None], -1)[..., 0]
    etop = np.take_along_axis(E, a[..., None], -1)[..., 0]
    hi = L + E
    np.put_along_axis(hi, a[..., None], -np.inf, -1)
    return a, (top - etop) > hi.max(axis=-1)


def greedy_chain(a: np.ndarray, drafts: np.ndarray, V: int):
    """Chain rule on per-row argmax a [B, K+1] and drafts [B, K]."""
    B, R = a.shape
    K = R - 1
    n = np.full(B, K, dtype=np.int32)
    tokens = np.full((B, K + 1), -1, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        for i in range(K):
            if drafts[b, i] != a[b, i]:
                n[b] = i
                break
        tokens[b, :n[b]] = drafts[b, :n[b]]
        tokens[b, n[b]] = a[b, n[b]]
        if K and ((drafts[b] < 0) | (drafts[b] >= V)).any():
            status[b] = 1
    return dict(accept_len=n, tokens=tokens, status=status)


def tree_walk(a: np.ndarray, node_tokens: np.ndarray, parents: np.ndarray, V: int):
    """Tree rule on per-node argmax a [B, N]: node j >= 1 is accepted when its
    parent is and its token is the argmax of the parent's row; the deepest
    accepted node (lowest index among equals) ends the path; its row's argmax
    is the bonus.  A malformed parent array gives accept_len -1, status 2."""
    B, N = a.shape
    out = dict(accept_len=np.zeros(B, np.int32), path=np.full((B, N), -1, np.int32),
               tokens=np.full((B, N), -1, np.int32), status=np.zeros(B, np.int32))
    for b in range(B):
        par = parents[b]
        if par[0] != -1 or any(not (0 <= par[j] < j) for j in range(1, N)):
            out["accept_len"][b] = -1
            out["status"][b] = 2
            continue
        ok = np.zeros(N, bool)
        depth = np.zeros(N, np.int64)
        ok[0] = True
        for j in range(1, N):
            depth[j] = depth[par[j]] + 1
            ok[j] = ok[par[j]] and node_tokens[b, j] == a[b, par[j]]
        best = 0
        for j in range(1, N):
            if ok[j] and depth[j] > depth[best]:
                best = j
        path = []
        j = best
        while j != 0:
            path.append(j)
            j = par[j]
        path.reverse()
        d = len(path)
        out["accept_len"][b] = d
        out["path"][b, :d] = path
        out["tokens"][b, :d] = node_tokens[b, path]
        out["tokens"][b, d] = a[b, best]
        if ((node_tokens[b, 1:] < 0) | (node_tokens[b, 1:] >= V)).any():
            out["status"][b] = 1
    return out


def verify_greedy(hidden_bits, lm_head_bits, drafts, exact=False):
    """Chain verification on H W^T.  Adds 'flagged' [B] (some row that decides
    the request - rows 0..accept_len - is uncertain)."""
    B, R, _ = hidden_bits.shape
    V = lm_head_bits.shape[0]
    L = logits(hidden_bits, lm_head_bits)
    E = None if exact else accumulation_bound(hidden_bits, lm_head_bits)
    a, certain = row_argmax(L, E)
    out = greedy_chain(a, drafts, V)
    out["flagged"] = np.array([not certain[b, :out["accept_len"][b] + 1].all() for b in range(B)])
    out["argmax"] = a
    return out


def verify_tree(hidden_bits, lm_head_bits, node_tokens, parents, exact=False):
    """Tree verification on H W^T.  Adds 'flagged' [B] (some node row is
    uncertain: any node's acceptance may depend on it)."""
    V = lm_head_bits.shape[0]
    L = logits(hidden_bits, lm_head_bits)
    E = None if exact else accumulation_bound(hidden_bits, lm_head_bits)
    a, certain = row_argmax(L, E)
    out = tree_walk(a, node_tokens, parents, V)
    out["flagged"] = ~certain.all(axis=1)
    out["argmax"] = a
    return out


def sample_flag_eps(hidden_bits, lm_head_bits, T):
    """Draw-margin threshold below which a sampled request may differ from a
    device result whose logits carry fp32 accumulation error (the bound above).
    With E the largest bound of any logit, every p(v) = exp(L[v]/T - lse) is
    off by a factor within exp(+-2E/T) (2E: the logit and its row's lse), so a
    ratio p/q near u <= 1 moves by at most eps = exp(2E/T) - 1, and a cell edge
    C/Z of an inverse CDF by at most 2 eps / Z.  Returns eps; a request is
    flagged when its margin is at most max(eps, 2 eps / Z)."""
    E = accumulation_bound(hidden_bits, lm_head_bits).max()
    return float(np.expm1(2.0 * E / T))


def verify_sample(hidden_bits, lm_head_bits, draft, draft_tokens, u_accept, u_sample, T, lib=None):
    """Speculative sampling (stochastic chain) on the target logits H W^T:
    hidden [B, K+1, D] and lm_head [V, D] bf16 bits, draft [B, K, V] logits
    (bf16 bits or float32).  Returns the sampling oracle's outputs (accept_len,
    tokens, lse_target, lse_draft, status, margin, Z)."""
    from . import verify_sample as sample_on_logits

    L = logits(hidden_bits, lm_head_bits).astype(np.float32)
    B, R, V = L.shape
    d = np.asarray(draft)
    if d.dtype == np.uint16:
        d = (d.astype(np.uint32) << np.uint32(16)).view(np.float32)  # exact widening
    d = np.ascontiguousarray(d, dtype=np.float32).reshape(B, R - 1, V)
    return sample_on_logits(L, d, draft_tokens, u_accept, u_sample, T, lib=lib)
