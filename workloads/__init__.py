"""Seeded synthetic inputs for batched speculative-decoding verification.

This module only *draws* inputs.  It holds none of the verifier's arithmetic
(no acceptance test, no residual, no row statistics of the verifier); both the
HIP path and the CPU oracle consume the arrays it returns, bit for bit.

What the inputs stand in for
----------------------------
The pages measure end-to-end decoding of real models (Qwen3-4B/8B, K=7) on
public benchmarks ("DLite" reading notes, section 3 and Tables 1-4).  Neither
the weights nor the datasets are available, so these generators produce logits
of the same *shape* (Qwen3 vocabulary, V=151936; draft length K=7) with simple
seeded distributions, and draft tokens/trees with a controlled agreement rate.

Named workloads (``WORKLOADS``, built by ``make_workload``)
----------------------------------------------------------
* ``sample_b1_k4_v1000_f32``: sample, B=1, K=4, V=1000, fp32, T=1.0:
  Lp ~ N(0, 2^2), Lq = Lp + N(0, 0.5^2).
* ``sample_b32_k7_qwen3``: sample, B=32, K=7, V=151936, bf16, T=1.0:
  Lp ~ N(0, 3^2) with +8 added at 20 distinct random ids per row; Lq = Lp + N(0, 1^2).
* ``sample_b256_k7_qwen3_t07``: sample, B=256, K=7, V=151936, bf16, T=0.7: Lp as in
  the previous one; per request a noise level sigma_b ~ U(0.1, 3.0); Lq = Lp + N(0, sigma_b^2).
* ``greedy_b512_k7_qwen3``: greedy, B=512 (also run at B=256), K=7, V=151936, bf16:
  Lt ~ N(0, 3^2); the draft for position i+1 equals argmax(row i) with
  probability 0.8, else a uniform vocabulary id.
* ``tree_b64_n33_qwen3``: tree, B=64, N=33, V=151936, bf16: Lt ~ N(0, 3^2); the
  AdaPLD-shaped tree of a root, an 8-node main copy path, 12 root branches each
  with one successor, and 0-3 extra leaves per request; a node's token equals
  argmax(parent row) with probability 0.7, else a uniform id.

In the sampling workloads the draft tokens are drawn from softmax(Lq/T) of the
*stored* (rounded) draft logits with the Gumbel-max trick, so the stored q is
the true proposal distribution.  The verifier's uniforms are drawn as one
(B, K+1, 2) float32 array in [0, 1): ``[..., :K, 0]`` are the acceptance draws
and ``[..., :, 1]`` the residual/bonus draws (``[b, K, 0]`` is never used).

Logits are drawn in float32 and rounded to bfloat16 with round-to-nearest-even
(torch's CPU conversion).  bf16 arrays are returned as ``uint16`` bit patterns.

Seeding: each named workload has its own ``numpy.random.SeedSequence`` seed (or
the caller's), spawned into independent streams, further split per block of 64
rows so the result does not depend on the thread count.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

VOCAB_QWEN3 = 151936
BLOCK_ROWS = 64

# Stream indices spawned from each workload's SeedSequence.
_S_TARGET, _S_SPIKES, _S_NOISE, _S_DRAFTS, _S_UNIF, _S_TREE = range(6)


@dataclass
class Workload:
    """One seeded batch of verifier inputs (host arrays)."""

    mode: str                       # "sample" | "greedy" | "tree"
    B: int
    V: int
    dtype: str                      # "f32" | "bf16"
    K: int = 0                      # chain draft length
    N: int = 0                      # tree nodes
    T: float = 1.0
    target: np.ndarray = None       # [B, K+1, V] or [B, N, V]; float32 or uint16 (bf16 bits)
    draft: np.ndarray = None        # [B, K, V] (sample mode)
    draft_tokens: np.ndarray = None  # [B, K] int32
    u_accept: np.ndarray = None     # [B, K] float32
    u_sample: np.ndarray = None     # [B, K+1] float32
    node_tokens: np.ndarray = None  # [B, N] int32
    parents: np.ndarray = None      # [B, N] int32
    hidden: np.ndarray = None       # [B, K+1 or N, D] uint16 (bf16 bits): LM-head workloads
    lm_head: np.ndarray = None      # [V, D] uint16 (bf16 bits)
    meta: dict = field(default_factory=dict)

    def rows(self) -> int:
        """Target rows verified per call: B*(K+1) for chains, B*N for trees."""
        return self.B * (self.N if self.mode.startswith("tree") else self.K + 1)


WORKLOADS = {
    "sample_b1_k4_v1000_f32": dict(mode="sample", B=1, K=4, V=1000, dtype="f32", T=1.0, seed=20261203),
    "sample_b32_k7_qwen3": dict(mode="sample", B=32, K=7, V=VOCAB_QWEN3, dtype="bf16", T=1.0, seed=20261204),
    "sample_b256_k7_qwen3_t07": dict(mode="sample", B=256, K=7, V=VOCAB_QWEN3, dtype="bf16", T=0.7,
                                     seed=20261205),
    "greedy_b512_k7_qwen3": dict(mode="greedy", B=512, K=7, V=VOCAB_QWEN3, dtype="bf16", seed=20261206),
    "tree_b64_n33_qwen3": dict(mode="tree", B=64, N=33, V=VOCAB_QWEN3, dtype="bf16", seed=20261207),
}


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); return uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_rows(seed: np.random.SeedSequence, rows: int, V: int, sigma, out: np.ndarray):
    """Fill out[rows, V] (float32) with N(0, sigma^2); sigma scalar or per-row array."""
    nblk = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS
    seeds = seed.spawn(nblk)
    sig = np.broadcast_to(np.asarray(sigma, dtype=np.float32), (rows,))

    def job(k):
        r0, r1 = k * BLOCK_ROWS, min(rows, (k + 1) * BLOCK_ROWS)
        blk = out[r0:r1]
        np.random.default_rng(seeds[k]).standard_normal(dtype=np.float32, out=blk)
        blk *= sig[r0:r1, None]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(nblk)))


def _add_spikes(seed, rows_f32: np.ndarray, count: int, height: float):
    """Add `height` at `count` distinct uniformly chosen ids of every row."""
    rng = np.random.default_rng(seed)
    R, V = rows_f32.shape
    for r in range(R):
        ids = np.unique(rng.integers(0, V, size=count))
        while ids.size < count:
            ids = np.unique(np.concatenate([ids, rng.integers(0, V, size=count - ids.size)]))
        rows_f32[r, ids] += np.float32(height)


def _gumbel_draws(seed, logits_f32: np.ndarray, T: float) -> np.ndarray:
    """One draw per row from softmax(logits/T) via argmax(logits/T + Gumbel)."""
    rows = logits_f32.shape[0]
    nblk = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS
    seeds = seed.spawn(nblk)
    out = np.empty(rows, dtype=np.int32)

    def job(k):
        r0, r1 = k * BLOCK_ROWS, min(rows, (k + 1) * BLOCK_ROWS)
        rng = np.random.default_rng(seeds[k])
        for r in range(r0, r1):
            g = -np.log(rng.standard_exponential(logits_f32.shape[1]))
            out[r] = int(np.argmax(logits_f32[r].astype(np.float64) / T + g))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(nblk)))
    return out


def _uniforms(seed, B: int, K: int):
    u = np.random.default_rng(seed).random((B, K + 1, 2), dtype=np.float32)
    return np.ascontiguousarray(u[:, :K, 0]), np.ascontiguousarray(u[:, :, 1])


def _stored(a_f32: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(a_f32) if dtype == "bf16" else np.ascontiguousarray(a_f32, np.float32)


def _as_f32(stored: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(stored) if dtype == "bf16" else stored


def make_sample(B, K, V, dtype="bf16", T=1.0, target_sigma=3.0, spikes=20, spike_height=8.0,
                noise_sigma=1.0, noise_sigma_range=None, seed=0) -> Workload:
    """Stochastic-chain inputs: target [B,K+1,V], draft [B,K,V], drafts ~ softmax(Lq/T)."""
    ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    st = ss.spawn(6)
    tgt = np.empty((B * (K + 1), V), dtype=np.float32)
    _normal_rows(st[_S_TARGET], tgt.shape[0], V, target_sigma, tgt)
    if spikes:
        _add_spikes(st[_S_SPIKES], tgt, spikes, spike_height)
    tgt = tgt.reshape(B, K + 1, V)
    nrng = st[_S_NOISE].spawn(2)
    if noise_sigma_range is not None:
        lo, hi = noise_sigma_range
        sig_b = np.random.default_rng(nrng[0]).uniform(lo, hi, size=B).astype(np.float32)
    else:
        sig_b = np.full(B, noise_sigma, dtype=np.float32)
    dr = np.empty((B * K, V), dtype=np.float32)
    _normal_rows(nrng[1], B * K, V, np.repeat(sig_b, K), dr)
    dr = dr.reshape(B, K, V)
    dr += tgt[:, :K, :]
    del_tgt = _stored(tgt, dtype)
    del tgt
    stored_dr = _stored(dr, dtype)
    del dr
    drafts = _gumbel_draws(st[_S_DRAFTS], _as_f32(stored_dr.reshape(B * K, V), dtype), T)
    ua, us = _uniforms(st[_S_UNIF], B, K)
    return Workload(mode="sample", B=B, K=K, V=V, dtype=dtype, T=float(T), target=del_tgt,
                    draft=stored_dr, draft_tokens=drafts.reshape(B, K), u_accept=ua,
                    u_sample=us, meta=dict(sigma_b=sig_b))


def _argmax_rows(rows_f32: np.ndarray) -> np.ndarray:
    """numpy.argmax per row (first occurrence of the maximum)."""
    return np.argmax(rows_f32, axis=-1).astype(np.int32)


def make_greedy(B, K, V, dtype="bf16", sigma=3.0, p_match=0.8, seed=0) -> Workload:
    """Greedy-chain inputs: target [B,K+1,V]; draft i+1 = argmax(row i) w.p. p_match."""
    ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    st = ss.spawn(6)
    tgt = np.empty((B * (K + 1), V), dtype=np.float32)
    _normal_rows(st[_S_TARGET], tgt.shape[0], V, sigma, tgt)
    stored = _stored(tgt, dtype)
    del tgt
    am = _argmax_rows(_as_f32(stored, dtype)).reshape(B, K + 1)
    rng = np.random.default_rng(st[_S_DRAFTS])
    hit = rng.random((B, K)) < p_match
    rnd = rng.integers(0, V, size=(B, K), dtype=np.int64).astype(np.int32)
    drafts = np.where(hit, am[:, :K], rnd).astype(np.int32)
    return Workload(mode="greedy", B=B, K=K, V=V, dtype=dtype, target=stored.reshape(B, K + 1, V),
                    draft_tokens=drafts, meta=dict(argmax=am))


def adapld_parents(extra: int, n_main: int = 8, n_branch: int = 12, rng=None) -> np.ndarray:
    """Parent array of an AdaPLD-shaped draft tree (topologically ordered).

    Node 0 is the root, nodes 1..n_main the main copy path, then n_branch
    branches under the root, then one successor per branch.  The last `extra`
    successor slots become extra leaves whose parent is drawn uniformly among
    the earlier nodes (root included).
    """
    N = 1 + n_main + 2 * n_branch
    par = np.empty(N, dtype=np.int32)
    par[0] = -1
    for k in range(1, n_main + 1):
        par[k] = k - 1
    b0 = 1 + n_main
    for k in range(n_branch):
        par[b0 + k] = 0
        par[b0 + n_branch + k] = b0 + k
    for e in range(extra):
        slot = N - 1 - e
        par[slot] = int(rng.integers(0, slot))
    return par


def make_tree(B, V, dtype="bf16", sigma=3.0, p_match=0.7, n_main=8, n_branch=12,
              max_extra=3, seed=0) -> Workload:
    """Greedy-tree inputs: target [B,N,V]; node token = argmax(parent row) w.p. p_match."""
    ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    st = ss.spawn(6)
    N = 1 + n_main + 2 * n_branch
    rng = np.random.default_rng(st[_S_TREE])
    parents = np.stack([adapld_parents(int(rng.integers(0, max_extra + 1)), n_main, n_branch, rng)
                        for _ in range(B)])
    tgt = np.empty((B * N, V), dtype=np.float32)
    _normal_rows(st[_S_TARGET], tgt.shape[0], V, sigma, tgt)
    stored = _stored(tgt, dtype)
    del tgt
    am = _argmax_rows(_as_f32(stored, dtype)).reshape(B, N)
    hit = rng.random((B, N)) < p_match
    rnd = rng.integers(0, V, size=(B, N), dtype=np.int64).astype(np.int32)
    par_am = np.take_along_axis(am, np.maximum(parents, 0), axis=1)
    tok = np.where(hit, par_am, rnd).astype(np.int32)
    tok[:, 0] = rnd[:, 0]
    return Workload(mode="tree", B=B, N=N, V=V, dtype=dtype, target=stored.reshape(B, N, V),
                    node_tokens=tok, parents=parents, meta=dict(argmax=am))


def make_workload(name: str, seed=None, B=None) -> Workload:
    """The named workload of ``WORKLOADS``; `B` overrides the batch (e.g. 256 for
    the greedy chain)."""
    cfg = dict(WORKLOADS[name])
    ss = np.random.SeedSequence(cfg["seed"] if seed is None else seed)
    if B is not None:
        cfg["B"] = B
    if name == "sample_b1_k4_v1000_f32":
        return make_sample(cfg["B"], cfg["K"], cfg["V"], "f32", 1.0, target_sigma=2.0, spikes=0,
                           noise_sigma=0.5, seed=ss)
    if name == "sample_b32_k7_qwen3":
        return make_sample(cfg["B"], cfg["K"], cfg["V"], "bf16", 1.0, noise_sigma=1.0, seed=ss)
    if name == "sample_b256_k7_qwen3_t07":
        return make_sample(cfg["B"], cfg["K"], cfg["V"], "bf16", 0.7,
                           noise_sigma_range=(0.1, 3.0), seed=ss)
    if name == "greedy_b512_k7_qwen3":
        return make_greedy(cfg["B"], cfg["K"], cfg["V"], "bf16", seed=ss)
    if name == "tree_b64_n33_qwen3":
        return make_tree(cfg["B"], cfg["V"], "bf16", seed=ss)
    raise ValueError(f"unknown workload {name}")


# ---- LM-head workloads: hidden states and a vocabulary projection ----------------
#
# The fused LM-head path takes the target's final hidden states H [rows, D] and
# the projection W [V, D] instead of logits.  Shapes follow Qwen3-8B (D = 4096,
# V = 151936).  Two value recipes:
#   exact:   H entries k/8 and W entries k/64 with k uniform in [-8, 8].  Every
#            product is a multiple of 2^-9 and every partial sum of D <= 8192
#            products is below 2^10 in magnitude, so an fp32 accumulation in
#            any order is exact; logits have std ~ 3.2 and exact ties occur.
#   general: H ~ N(0, 1), W ~ N(0, (3 / sqrt(D))^2), rounded to bf16; logits have
#            std ~ 3 and fp32 accumulation rounds.
# Drafts (chains) and node tokens (trees) equal the argmax of the row they are
# checked against with probability p_match, else a uniform id; p_match=None
# draws them all uniformly (no logits are formed).

LMHEAD_SHAPE = dict(B=256, K=7, D=4096, V=VOCAB_QWEN3)


_LM_BLOCK = 4096  # rows per seeded block of the LM-head operands


def _lmhead_rows(seed, rows: int, D: int, exact: bool, scale: float) -> np.ndarray:
    """bf16 bits [rows, D]: exact recipe k * scale (k uniform in [-8, 8]) or
    N(0, scale^2), drawn in seeded blocks of _LM_BLOCK rows on threads."""
    out = np.empty((rows, D), dtype=np.uint16)
    nblk = (rows + _LM_BLOCK - 1) // _LM_BLOCK
    seeds = seed.spawn(nblk)
    table = to_bf16_bits(np.arange(-8, 9, dtype=np.float32) * np.float32(scale))

    def job(k):
        r0, r1 = k * _LM_BLOCK, min(rows, (k + 1) * _LM_BLOCK)
        rng = np.random.default_rng(seeds[k])
        if exact:
            out[r0:r1] = table[rng.integers(0, 17, size=(r1 - r0, D), dtype=np.int8)]
        else:
            out[r0:r1] = to_bf16_bits(rng.standard_normal((r1 - r0, D), dtype=np.float32) * np.float32(scale))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(nblk)))
    return out


def _lmhead_values(seed, rows: int, D: int, V: int, exact: bool):
    sh, sw = seed.spawn(2)
    if exact:
        return _lmhead_rows(sh, rows, D, True, 1 / 8), _lmhead_rows(sw, V, D, True, 1 / 64)
    return _lmhead_rows(sh, rows, D, False, 1.0), _lmhead_rows(sw, V, D, False, 3.0 / np.sqrt(D))


def _lmhead_argmax(Hb: np.ndarray, Wb: np.ndarray, exact: bool) -> np.ndarray:
    """Row argmax of H W^T, for planting matching drafts (the exact recipe is
    exact in fp32; the general one uses fp64)."""
    dt = np.float32 if exact else np.float64
    h = bf16_bits_to_f32(Hb).astype(dt)
    V = Wb.shape[0]
    nblk = (V + _LM_BLOCK - 1) // _LM_BLOCK
    best = np.full((nblk, Hb.shape[0]), -np.inf)
    arg = np.zeros((nblk, Hb.shape[0]), dtype=np.int64)

    def job(k):
        v0 = k * _LM_BLOCK
        L = h @ bf16_bits_to_f32(Wb[v0:v0 + _LM_BLOCK]).astype(dt).T
        arg[k] = v0 + np.argmax(L, axis=1)
        best[k] = L.max(axis=1)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(nblk)))
    return arg[np.argmax(best, axis=0), np.arange(Hb.shape[0])]


def _lmhead_logits(Hb: np.ndarray, Wb: np.ndarray, exact: bool) -> np.ndarray:
    """H W^T as float32 [rows, V], for shaping correlated draft logits (the exact
    recipe is exact in fp32; the general one is formed in fp64 and rounded)."""
    dt = np.float32 if exact else np.float64
    h = bf16_bits_to_f32(Hb).astype(dt)
    V = Wb.shape[0]
    out = np.empty((Hb.shape[0], V), dtype=np.float32)

    def job(v0):
        out[:, v0:v0 + _LM_BLOCK] = h @ bf16_bits_to_f32(Wb[v0:v0 + _LM_BLOCK]).astype(dt).T

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(0, V, _LM_BLOCK)))
    return out


def make_sample_lmhead(B, K, D, V, exact=True, dtype="bf16", T=0.7, noise_sigma=1.0, seed=0,
                       plant=None) -> Workload:
    """Stochastic-chain inputs for the fused LM-head path: hidden [B,K+1,D] and
    lm_head [V,D] as for the greedy form; draft logits [B,K,V] are the target
    logits of the same position (H W^T) plus N(0, noise_sigma^2) for the
    `plant` requests (all by default) and independent N(0, 3^2) rows for the
    others; drafts are drawn from softmax(Lq/T) of the stored draft logits."""
    ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    st = ss.spawn(6)
    Hb, Wb = _lmhead_values(st[_S_TARGET], B * (K + 1), D, V, exact)
    H3 = Hb.reshape(B, K + 1, D)
    nrng = st[_S_NOISE].spawn(2)
    dr = np.empty((B * K, V), dtype=np.float32)
    _normal_rows(nrng[0], B * K, V, 3.0, dr)
    dr = dr.reshape(B, K, V)
    reqs = np.arange(B) if plant is None else np.asarray(plant)
    if K > 0 and len(reqs):
        L = _lmhead_logits(H3[reqs, :K].reshape(-1, D), Wb, exact)
        noise = np.empty_like(L)
        _normal_rows(nrng[1], L.shape[0], V, noise_sigma, noise)
        dr[reqs] = (L + noise).reshape(len(reqs), K, V)
        del L, noise
    stored = _stored(dr, dtype)
    del dr
    drafts = _gumbel_draws(st[_S_DRAFTS], _as_f32(stored.reshape(B * K, V), dtype), T).reshape(B, K)
    ua, us = _uniforms(st[_S_UNIF], B, K)
    return Workload(mode="sample_lmhead", B=B, K=K, V=V, dtype=dtype, T=float(T), draft=stored,
                    draft_tokens=drafts, u_accept=ua, u_sample=us, hidden=H3, lm_head=Wb,
                    meta=dict(D=D, exact=exact, noise_sigma=noise_sigma))


def make_greedy_lmhead(B, K, D, V, exact=True, p_match=0.8, seed=0, plant=None) -> Workload:
    """Greedy-chain inputs for the fused LM-head path: hidden [B,K+1,D], lm_head [V,D].
    `plant` limits the matching drafts to those requests (the others draw
    uniform drafts), so large shapes need logits of a few rows only."""
    ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    st = ss.spawn(6)
    Hb, Wb = _lmhead_values(st[_S_TARGET], B * (K + 1), D, V, exact)
    rng = np.random.default_rng(st[_S_DRAFTS])
    x = rng.integers(0, V, size=(B, K)).astype(np.int32)
    hit = rng.random((B, K)) < (p_match or 0.0)
    if p_match is not None and K > 0:
        reqs = np.arange(B) if plant is None else np.asarray(plant)
        H3 = Hb.reshape(B, K + 1, D)
        am = _lmhead_argmax(H3[reqs].reshape(-1, D), Wb, exact).reshape(len(reqs), K + 1)
        x[reqs] = np.where(hit[reqs], am[:, :K], x[reqs])
    return Workload(mode="greedy_lmhead", B=B, K=K, V=V, dtype="bf16", draft_tokens=x,
                    hidden=Hb.reshape(B, K + 1, D), lm_head=Wb,
                    meta=dict(D=D, exact=exact, p_match=p_match))


def make_tree_lmhead(B, D, V, exact=True, p_match=0.7, n_main=8, n_branch=12, max_extra=3,
                     seed=0, plant=None) -> Workload:
    """Greedy-tree inputs for the fused LM-head path: hidden [B,N,D], lm_head [V,D]
    (`plant` as for chains)."""
    ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    st = ss.spawn(6)
    N = 1 + n_main + 2 * n_branch
    rng = np.random.default_rng(st[_S_TREE])
    parents = np.stack([adapld_parents(int(rng.integers(0, max_extra + 1)), n_main, n_branch, rng)
                        for _ in range(B)])
    Hb, Wb = _lmhead_values(st[_S_TARGET], B * N, D, V, exact)
    tok = rng.integers(0, V, size=(B, N)).astype(np.int32)
    hit = rng.random((B, N)) < (p_match or 0.0)
    if p_match is not None:
        reqs = np.arange(B) if plant is None else np.asarray(plant)
        am = _lmhead_argmax(Hb.reshape(B, N, D)[reqs].reshape(-1, D), Wb, exact).reshape(len(reqs), N)
        want = np.take_along_axis(am, np.maximum(parents[reqs], 0), 1)
        tok[reqs] = np.where(hit[reqs], want, tok[reqs])
    return Workload(mode="tree_lmhead", B=B, N=N, V=V, dtype="bf16", node_tokens=tok,
                    parents=parents.astype(np.int32), hidden=Hb.reshape(B, N, D), lm_head=Wb,
                    meta=dict(D=D, exact=exact, p_match=p_match))


# ---- token streams for lexical retrieval --------------------------------------
#
# AdaPLD reuses spans of its own context (prompt plus generated text), which in
# agent and code workloads repeats heavily.  These streams imitate that: each
# request's context is built from segments that either copy an earlier span
# of the same context (probability p_copy, 8..64 tokens) or draw fresh tokens
# from a Zipf-like distribution over a working vocabulary of `working` ids
# spread over the full vocabulary.  The query is the last n tokens of the
# context (the current prefix's tail), so the self-match at the end is
# excluded by the retrieval's own rule (no continuation).

NGRAM_SHAPE = dict(B=256, L=32768, n=3, cap=64)


def make_ngram(B, L, n, lengths=None, p_copy=0.3, p_tail_copy=0.6, working=4000, V=VOCAB_QWEN3,
               seed=0) -> dict:
    """Token streams [B, L] with lengths [B] and queries [B, n] (see above).  The
    last segment of a context is a copy with probability p_tail_copy, so the
    query tail often occurs earlier, as when generation repeats its context."""
    ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    seeds = ss.spawn(B + 1)
    rng0 = np.random.default_rng(seeds[B])
    if lengths is None:
        lengths = rng0.integers(L // 4, L + 1, size=B)
    lengths = np.asarray(lengths, dtype=np.int32)
    ids = rng0.choice(V, size=working, replace=False).astype(np.int32)
    zipf = 1.0 / np.arange(1, working + 1)
    cdf = np.cumsum(zipf / zipf.sum())
    ctx = np.zeros((B, L), dtype=np.int32)

    def job(b):
        rng = np.random.default_rng(seeds[b])
        ln = int(lengths[b])
        row = ctx[b]
        t = 0
        tail_copy = rng.random() < p_tail_copy
        while t < ln:
            seg = int(rng.integers(8, 65))
            seg = min(seg, ln - t)
            last = t + seg >= ln
            if t > 64 and ((last and tail_copy) or rng.random() < p_copy):
                src = int(rng.integers(0, t - seg)) if t - seg > 0 else 0
                row[t:t + seg] = row[src:src + seg]
            else:
                # Zipf draws by inverse CDF
                row[t:t + seg] = ids[np.minimum(np.searchsorted(cdf, rng.random(seg), side="right"), working - 1)]
            t += seg

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(B)))
    q = np.stack([ctx[b, max(0, lengths[b] - n):lengths[b]] if lengths[b] >= n
                  else np.zeros(n, np.int32) for b in range(B)]).astype(np.int32)
    return dict(context=ctx, lengths=lengths, queries=q, n=n)


# Long contexts (128K tokens, a long-document reuse context): each request's
# stream is its own base stream followed by the base streams of the next
# requests in turn, so spans recur across the whole context as in a long
# conversation that quotes earlier turns.  Built from make_ngram's streams by
# concatenation only, so it costs no more to generate than the base shape.
NGRAM_LONG_SHAPE = dict(B=256, L=131072, n=3, cap=64)


def make_ngram_long(B, L, n, base_L=32768, seed=0) -> dict:
    """Token streams [B, L] (L a multiple of base_L), lengths [B] between L/2 and
    L, and queries [B, n] (the last n tokens before each length)."""
    if L % base_L:
        raise ValueError("L must be a multiple of base_L")
    ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    s_base, s_len = ss.spawn(2)
    base = make_ngram(B, base_L, n, lengths=np.full(B, base_L), seed=s_base)["context"]
    reps = L // base_L
    idx = (np.arange(B)[:, None] + np.arange(reps)[None, :]) % B
    ctx = np.ascontiguousarray(base[idx].reshape(B, L))
    lengths = np.random.default_rng(s_len).integers(L // 2, L + 1, size=B).astype(np.int32)
    q = np.stack([ctx[b, lengths[b] - n:lengths[b]] for b in range(B)]).astype(np.int32)
    return dict(context=ctx, lengths=lengths, queries=q, n=n)
