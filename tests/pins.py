"""Checks that pin the CPU oracle to facts fixed outside itself.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load(path)``)
and raises AssertionError when the oracle disagrees with:

* the speculative-sampling identities on the SD tutorial page, section
  "为什么“猜错再改”不会偏离目标分布": the accept path yields x with probability
  q(x) min(1, p(x)/q(x)) = min(p(x), q(x)); the residual norm(max(0, p - q))
  restores the rest, so the emitted token is distributed exactly as p, and
  conditioning position by position keeps the whole sequence distributed as
  the target's autoregressive joint;
* the expected number of tokens per round under i.i.d. acceptance, section
  "速度取决于两个数…": E[N] = (1 - a^(g+1)) / (1 - a);
* the round bounds (1 .. gamma+1 tokens, section "一轮推测解码究竟发生什么");
* the greedy rule (target argmax decoding; numpy.argmax gives the lowest index);
* the AdaPLD draft-tree acceptance (section 3.3), by brute force over every
  root-to-leaf path;
* library routines (scipy.special.logsumexp, numpy.searchsorted, cumsum).

Probabilities used as test expectations come from scipy.special.softmax in
float64, never from the oracle.  The enumeration checks call the oracle only at
the midpoints of the cells on which its output is constant, and weight each
cell by its exact area.
"""

from __future__ import annotations

import itertools

import numpy as np
from scipy import special, stats

import oracle

F32 = np.float32


def softmax64(logits, T=1.0):
    return special.softmax(np.asarray(logits, np.float64) / T, axis=-1)


# ---------------------------------------------------------------- cell helpers

def _cells(breaks):
    """Cells of [0,1) cut at `breaks` (points closer than 1e-9 merged):
    list of (float32 midpoint, exact width)."""
    b = np.sort(np.clip(np.concatenate([[0.0, 1.0], np.asarray(breaks, np.float64)]), 0.0, 1.0))
    kept = [0.0]
    for x in b[1:]:
        if x - kept[-1] > 1e-9:
            kept.append(float(x))
    kept[-1] = 1.0
    out = []
    for lo, hi in zip(kept[:-1], kept[1:]):
        w = hi - lo
        mid = F32(0.5 * (lo + hi))
        if not (lo < float(mid) < hi) or w < 1e-6:
            raise RuntimeError("cell too narrow for a float32 midpoint; redraw the table")
        out.append((mid, w))
    return out


def _sample_breaks(p_row, q_row=None):
    """All cut points of the inverse-CDF draw over p (and over the residual)."""
    cuts = [np.cumsum(p_row)]
    if q_row is not None:
        d = np.maximum(0.0, p_row - q_row)
        if d.sum() > 0:
            cuts.append(np.cumsum(d) / d.sum())
    return np.concatenate(cuts)


def _well_separated(p, q, gap=1e-4):
    d = np.abs(p - q)
    return np.all((d == 0) | (d > gap)) and np.all(p > gap) and np.all(q > gap)


def random_tables(rng, V, scale=1.0):
    """fp32 logit rows whose softmaxes differ clearly at every entry."""
    while True:
        lp = (rng.standard_normal(V) * scale).astype(F32)
        lq = (lp + rng.standard_normal(V) * scale).astype(F32)
        if _well_separated(softmax64(lp), softmax64(lq)):
            return lp, lq


# ------------------------------------------------------ per-position losslessness

def pin_position_lossless(lib, seed=11):
    """K = 1: P(first token = y) = p(y) exactly; accept part = min(p,q), residual
    part = max(0, p-q); bonus after acceptance ~ p of the next row."""
    rng = np.random.default_rng(seed)
    for V, T in ((3, 1.0), (5, 0.7), (8, 1.3)):
        lp0, lq0 = random_tables(rng, V)
        lp1 = (rng.standard_normal(V)).astype(F32)
        p0, q0, p1 = softmax64(lp0, T), softmax64(lq0, T), softmax64(lp1, T)
        reqs = []
        for x in range(V):
            r = p0[x] / q0[x]
            for ua, wa in _cells([min(r, 1.0)]):
                for us0, w0 in _cells(_sample_breaks(p0, q0)):
                    for us1, w1 in _cells(_sample_breaks(p1)):
                        reqs.append((x, ua, us0, us1, q0[x] * wa * w0 * w1))
        B = len(reqs)
        tgt = np.broadcast_to(np.stack([lp0, lp1])[None], (B, 2, V)).copy()
        dr = np.broadcast_to(lq0[None, None], (B, 1, V)).copy()
        x = np.array([[r[0]] for r in reqs], np.int32)
        ua = np.array([[r[1]] for r in reqs], F32)
        us = np.array([[r[2], r[3]] for r in reqs], F32)
        w = np.array([r[4] for r in reqs])
        o = oracle.verify_sample(tgt, dr, x, ua, us, T, threads=1, lib=lib)
        n, tok = o["accept_len"], o["tokens"]
        acc = np.bincount(tok[n == 1, 0], weights=w[n == 1], minlength=V)
        rej = np.bincount(tok[n == 0, 0], weights=w[n == 0], minlength=V)
        assert np.allclose(acc, np.minimum(p0, q0), atol=1e-12, rtol=0), (acc, np.minimum(p0, q0))
        assert np.allclose(rej, np.maximum(0, p0 - q0), atol=1e-12, rtol=0)
        assert np.allclose(acc + rej, p0, atol=1e-12, rtol=0)
        alpha = np.minimum(p0, q0).sum()
        bonus = np.bincount(tok[n == 1, 1], weights=w[n == 1], minlength=V)
        assert np.allclose(bonus, alpha * p1, atol=1e-12, rtol=0)
        assert np.all(tok[n == 0, 1] == -1)


# ------------------------------------------------------ sequence losslessness (K=2)

def _toy_model(rng, V, T):
    """Prefix -> logit tables for target (prefix length 0..2) and draft (0..1)."""
    while True:
        tp = {(): (rng.standard_normal(V) * 1.2).astype(F32)}
        tq = {(): (tp[()] + rng.standard_normal(V)).astype(F32)}
        for a in range(V):
            tp[(a,)] = (rng.standard_normal(V) * 1.2).astype(F32)
            tq[(a,)] = (tp[(a,)] + rng.standard_normal(V)).astype(F32)
            for b in range(V):
                tp[(a, b)] = (rng.standard_normal(V) * 1.2).astype(F32)
        if all(_well_separated(softmax64(tp[k], T), softmax64(tq[k], T)) for k in tq):
            return tp, tq


def pin_sequence_lossless(lib, seed=5, V=3, T=0.9):
    """K = 2 with prefix-dependent toy models: emitted tokens, completed by the
    target's own autoregressive steps, have exactly the target's joint law."""
    rng = np.random.default_rng(seed)
    tp, tq = _toy_model(rng, V, T)
    P = {k: softmax64(v, T) for k, v in tp.items()}
    Q = {k: softmax64(v, T) for k, v in tq.items()}
    reqs = []
    for x1 in range(V):
        for x2 in range(V):
            wq = Q[()][x1] * Q[(x1,)][x2]
            r1 = P[()][x1] / Q[()][x1]
            r2 = P[(x1,)][x2] / Q[(x1,)][x2]
            c_a1 = _cells([min(r1, 1)])
            c_a2 = _cells([min(r2, 1)])
            c_s0 = _cells(_sample_breaks(P[()], Q[()]))
            c_s1 = _cells(_sample_breaks(P[(x1,)], Q[(x1,)]))
            c_s2 = _cells(_sample_breaks(P[(x1, x2)]))
            for (a1, w1), (a2, w2), (s0, v0), (s1, v1), (s2, v2) in itertools.product(
                    c_a1, c_a2, c_s0, c_s1, c_s2):
                reqs.append((x1, x2, a1, a2, s0, s1, s2, wq * w1 * w2 * v0 * v1 * v2))
    B = len(reqs)
    tgt = np.empty((B, 3, V), F32)
    dr = np.empty((B, 2, V), F32)
    for i, r in enumerate(reqs):
        x1, x2 = r[0], r[1]
        tgt[i] = [tp[()], tp[(x1,)], tp[(x1, x2)]]
        dr[i] = [tq[()], tq[(x1,)]]
    x = np.array([[r[0], r[1]] for r in reqs], np.int32)
    ua = np.array([[r[2], r[3]] for r in reqs], F32)
    us = np.array([[r[4], r[5], r[6]] for r in reqs], F32)
    w = np.array([r[7] for r in reqs])
    o = oracle.verify_sample(tgt, dr, x, ua, us, T, threads=1, lib=lib)
    joint = np.zeros((V, V, V))
    for i in range(B):
        n = o["accept_len"][i]
        y = list(o["tokens"][i, :n + 1])
        assert 0 <= n <= 2 and all(0 <= t < V for t in y) and np.all(o["tokens"][i, n + 1:] == -1)
        # complete the round to three tokens with the target's own steps
        stack = [(y, w[i])]
        while stack:
            seq, wt = stack.pop()
            if len(seq) == 3:
                joint[tuple(seq)] += wt
                continue
            pr = P[tuple(seq)]
            for t in range(V):
                stack.append((seq + [t], wt * pr[t]))
    ref = np.zeros((V, V, V))
    for a, b, c in itertools.product(range(V), repeat=3):
        ref[a, b, c] = P[()][a] * P[(a,)][b] * P[(a, b)][c]
    assert np.allclose(joint, ref, atol=1e-12, rtol=0), np.abs(joint - ref).max()


# ------------------------------------------------------------- E[N] closed form

def _alpha_tables(alpha):
    """fp32 logits of q = (a/2, 1-a/2), p = (1-a/2, a/2): sum_v min(p,q) = a,
    with one ratio above 1 and one strictly between 0 and 1."""
    h = alpha / 2
    lp = np.log(np.array([1 - h, h])).astype(F32)
    lq = np.log(np.array([h, 1 - h])).astype(F32)
    return lp, lq


def pin_expected_accept_length(lib):
    """Exact enumeration of the accept length for K = 1..7 under prefix-free
    tables with overlap a; E[n+1] must be (1 - a^(K+1)) / (1 - a)."""
    for alpha in (0.2, 0.5, 0.8, 0.95):
        lp, lq = _alpha_tables(alpha)
        p, q = softmax64(lp), softmax64(lq)
        a_eff = np.minimum(p, q).sum()
        support = [0, 1]
        for K in range(1, 8):
            reqs = []
            for xs in itertools.product(support, repeat=K):
                wq = np.prod([q[v] for v in xs])
                cells = [_cells([min(p[v] / q[v], 1.0)]) for v in xs]
                for combo in itertools.product(*cells):
                    reqs.append((xs, [c[0] for c in combo], wq * np.prod([c[1] for c in combo])))
            B = len(reqs)
            tgt = np.broadcast_to(lp, (B, K + 1, 2)).copy()
            dr = np.broadcast_to(lq, (B, K, 2)).copy()
            x = np.array([r[0] for r in reqs], np.int32)
            ua = np.array([r[1] for r in reqs], F32)
            us = np.full((B, K + 1), F32(0.5))
            w = np.array([r[2] for r in reqs])
            o = oracle.verify_sample(tgt, dr, x, ua, us, 1.0, threads=1, lib=lib)
            EN = float(np.sum(w * (o["accept_len"] + 1)))
            closed = (1 - a_eff ** (K + 1)) / (1 - a_eff)
            assert abs(EN - closed) < 1e-12, (alpha, K, EN, closed)
            assert abs(w.sum() - 1) < 1e-12


def pin_expected_accept_length_mc(lib, trials=200_000, seed=3):
    """Monte Carlo mean of n+1 within 4 standard errors of the closed form."""
    rng = np.random.default_rng(seed)
    for alpha, K in ((0.5, 3), (0.8, 7)):
        lp, lq = _alpha_tables(alpha)
        p, q = softmax64(lp), softmax64(lq)
        a_eff = np.minimum(p, q).sum()
        x = rng.choice(2, size=(trials, K), p=q).astype(np.int32)
        tgt = np.broadcast_to(lp, (trials, K + 1, 2))
        dr = np.broadcast_to(lq, (trials, K, 2))
        ua = rng.random((trials, K), dtype=F32)
        us = rng.random((trials, K + 1), dtype=F32)
        o = oracle.verify_sample(tgt, dr, x, ua, us, 1.0, lib=lib)
        N = o["accept_len"] + 1.0
        closed = (1 - a_eff ** (K + 1)) / (1 - a_eff)
        se = N.std() / np.sqrt(trials)
        assert abs(N.mean() - closed) < 4 * se, (alpha, K, N.mean(), closed, se)


# --------------------------------------------------------------- chi-square test

def chi_square_case(trials=1_000_000, seed=7, V=8, T=1.0):
    """Inputs of ``trials`` rounds with K = 2 on prefix-dependent toy models
    (drafts drawn from the draft model), with the laws they must follow: the
    first emitted token ~ p(.|prefix), and the accept-length law obtained from
    the overlap identity, P(n >= 1) = sum min(p0, q0), then position by position."""
    rng = np.random.default_rng(seed)
    tp = {(): (rng.standard_normal(V)).astype(F32)}
    tq = {(): (tp[()] + rng.standard_normal(V) * 0.8).astype(F32)}
    for a in range(V):
        tp[(a,)] = rng.standard_normal(V).astype(F32)
        tq[(a,)] = (tp[(a,)] + rng.standard_normal(V) * 0.8).astype(F32)
    TP2 = rng.standard_normal((V, V, V)).astype(F32)  # third target row, by (x1, x2)
    P0, Q0 = softmax64(tp[()], T), softmax64(tq[()], T)
    P1 = np.stack([softmax64(tp[(a,)], T) for a in range(V)])
    Q1 = np.stack([softmax64(tq[(a,)], T) for a in range(V)])
    x1 = rng.choice(V, size=trials, p=Q0)
    cq = np.cumsum(Q1, axis=1)
    x2 = np.minimum((cq[x1] <= rng.random(trials)[:, None]).sum(1), V - 1)
    tgt = np.empty((trials, 3, V), F32)
    tgt[:, 0] = tp[()]
    tgt[:, 1] = np.stack([tp[(a,)] for a in range(V)])[x1]
    tgt[:, 2] = TP2[x1, x2]
    dr = np.empty((trials, 2, V), F32)
    dr[:, 0] = tq[()]
    dr[:, 1] = np.stack([tq[(a,)] for a in range(V)])[x1]
    x = np.stack([x1, x2], 1).astype(np.int32)
    ua = rng.random((trials, 2), dtype=F32)
    us = rng.random((trials, 3), dtype=F32)
    a0 = np.minimum(P0, Q0)
    a1 = np.minimum(P1, Q1).sum(1)
    law_n = np.array([1 - a0.sum(), (a0 * (1 - a1)).sum(), (a0 * a1).sum()])
    return dict(target=tgt, draft=dr, x=x, u_accept=ua, u_sample=us, T=T, V=V, P0=P0, law_n=law_n)


def check_chi_square(case, tokens, accept_len, pmin=1e-3):
    """The first emitted token follows P0 and the accept lengths follow their
    exact law (chi-square p-values above ``pmin``)."""
    trials, V = len(accept_len), case["V"]
    first = np.bincount(tokens[:, 0], minlength=V)
    assert stats.chisquare(first, case["P0"] * trials).pvalue > pmin
    hist = np.bincount(accept_len, minlength=3)
    assert stats.chisquare(hist, case["law_n"] * trials).pvalue > pmin


def pin_chi_square(lib, trials=1_000_000, seed=7, V=8, T=1.0):
    """10^6 rounds with K = 2 on prefix-dependent toy models: the oracle's
    first emitted token follows p(.|prefix) and its accept-length histogram
    follows the exact law obtained from the overlap identity."""
    c = chi_square_case(trials, seed, V, T)
    o = oracle.verify_sample(c["target"], c["draft"], c["x"], c["u_accept"], c["u_sample"], T, lib=lib)
    check_chi_square(c, o["tokens"], o["accept_len"])


# ---------------------------------------------------------------- special cases

def pin_special_cases(lib, seed=9):
    rng = np.random.default_rng(seed)
    B, K, V = 64, 3, 50
    # (i) identical logits: every draft accepted, bonus = inverse CDF of p_K
    lp = rng.standard_normal((B, K + 1, V)).astype(F32) * 2
    x = rng.integers(0, V, size=(B, K)).astype(np.int32)
    ua = rng.random((B, K), dtype=F32)
    us = rng.random((B, K + 1), dtype=F32)
    o = oracle.verify_sample(lp, lp[:, :K].copy(), x, ua, us, 0.8, lib=lib)
    assert np.all(o["accept_len"] == K)
    assert np.array_equal(o["tokens"][:, :K], x)
    for b in range(B):
        c = np.cumsum(softmax64(lp[b, K], 0.8))
        assert o["tokens"][b, K] == np.searchsorted(c, float(us[b, K]) * c[-1], side="right")
    # (ii) disjoint support: every draft rejected at once; token ~ p_0
    lp = np.full((B, K + 1, V), -1e4, F32)
    lq = np.full((B, K, V), -1e4, F32)
    lp[:, :, : V // 2] = rng.standard_normal((B, K + 1, V // 2))
    lq[:, :, V // 2:] = rng.standard_normal((B, K, V - V // 2))
    x = rng.integers(V // 2, V, size=(B, K)).astype(np.int32)
    o = oracle.verify_sample(lp, lq, x, ua, us, 1.0, lib=lib)
    assert np.all(o["accept_len"] == 0)
    assert np.all(o["tokens"][:, 1:] == -1)
    for b in range(B):
        c = np.cumsum(softmax64(lp[b, 0]))
        assert o["tokens"][b, 0] == np.searchsorted(c, float(us[b, 0]) * c[-1], side="right")
    # (iii) a forced rejection samples the residual max(0, p-q) by inverse CDF
    lp = rng.standard_normal((B, 2, V)).astype(F32) * 2
    lq = (lp[:, :1] + rng.standard_normal((B, 1, V)).astype(F32)).astype(F32)
    x = rng.integers(0, V, size=(B, 1)).astype(np.int32)
    r = np.array([softmax64(lp[b, 0])[x[b, 0]] / softmax64(lq[b, 0])[x[b, 0]] for b in range(B)])
    ua = np.minimum(F32(0.999999), (np.minimum(r, 1.0) + 0.5 * (1 - np.minimum(r, 1.0)))
                    ).astype(F32)[:, None]
    us = rng.random((B, 2), dtype=F32)
    o = oracle.verify_sample(lp, lq, x, ua, us, 1.0, lib=lib)
    for b in range(B):
        if r[b] >= 1:
            assert o["accept_len"][b] == 1
            continue
        assert o["accept_len"][b] == 0
        d = np.maximum(0.0, softmax64(lp[b, 0]) - softmax64(lq[b, 0]))
        c = np.cumsum(d)
        assert o["tokens"][b, 0] == np.searchsorted(c, float(us[b, 0]) * c[-1], side="right")
        assert abs(o["Z"][b] - c[-1]) < 1e-12
    # (iv) K = 0: the round is a single draw from p_0
    lp = rng.standard_normal((B, 1, V)).astype(F32)
    us = rng.random((B, 1), dtype=F32)
    o = oracle.verify_sample(lp, np.zeros((B, 0, V), F32), np.zeros((B, 0), np.int32),
                             np.zeros((B, 0), F32), us, 1.0, lib=lib)
    assert np.all(o["accept_len"] == 0)
    for b in range(B):
        c = np.cumsum(softmax64(lp[b, 0]))
        assert o["tokens"][b, 0] == np.searchsorted(c, float(us[b, 0]) * c[-1], side="right")


def pin_lse(lib, seed=2):
    rng = np.random.default_rng(seed)
    for T in (1.0, 0.7, 2.5):
        L = (rng.standard_normal((6, 3000)) * 3).astype(F32)
        m, s, lse = oracle.row_stats(L, T, lib=lib)
        ref = special.logsumexp(L.astype(np.float64) / T, axis=-1)
        assert np.allclose(lse, ref, rtol=1e-12, atol=0)
        assert np.array_equal(m, L.max(-1).astype(np.float64))
        # bf16 bit patterns decode exactly
        bits = (L.view(np.uint32) >> 16).astype(np.uint16)
        wide = (bits.astype(np.uint32) << 16).view(np.float32)
        _, _, lse16 = oracle.row_stats(bits, T, lib=lib)
        assert np.allclose(lse16, special.logsumexp(wide.astype(np.float64) / T, axis=-1),
                           rtol=1e-12, atol=0)
        # the sample path reports the same lse for target and draft rows
        B, K, V = 2, 2, 3000
        tg = L[: B * (K + 1)].reshape(B, K + 1, V)
        dr = L[: B * K].reshape(B, K, V)
        o = oracle.verify_sample(tg, dr, np.zeros((B, K), np.int32), np.zeros((B, K), F32),
                                 np.zeros((B, K + 1), F32), T, lib=lib)
        assert np.allclose(o["lse_target"], ref[: B * (K + 1)].reshape(B, K + 1), rtol=1e-12)
        assert np.allclose(o["lse_draft"], ref[: B * K].reshape(B, K), rtol=1e-12)


# ---------------------------------------------------------------- greedy chain

def pin_greedy(lib, seed=4):
    rng = np.random.default_rng(seed)
    B, K, V = 256, 4, 6
    # small integer logits give frequent tied maxima
    L = rng.integers(-2, 3, size=(B, K + 1, V)).astype(F32)
    L[0, :, :] = 0.0
    L[1, :, :] = -0.0
    L[1, :, 3] = 0.0
    am = np.argmax(L, axis=-1)
    # every accept/reject pattern: draft i matches argmax(row i) iff bit i set
    pat = np.arange(B) % (1 << K)
    match = ((pat[:, None] >> np.arange(K)) & 1).astype(bool)
    x = np.where(match, am[:, :K], (am[:, :K] + 1 + rng.integers(0, V - 1, (B, K))) % V)
    x = x.astype(np.int32)
    o = oracle.verify_greedy(L, x, lib=lib)
    for b in range(B):
        n = K if match[b].all() else int(np.argmin(match[b]))
        assert o["accept_len"][b] == n
        assert list(o["tokens"][b, :n]) == list(x[b, :n])
        assert o["tokens"][b, n] == am[b, n]
        assert np.all(o["tokens"][b, n + 1:] == -1)
    assert np.array_equal(oracle.argmax(L, lib=lib), am)
    # greedy verification of argmax-decoded drafts reproduces argmax decoding
    x = am[:, :K].astype(np.int32)
    o = oracle.verify_greedy(L, x, lib=lib)
    assert np.all(o["accept_len"] == K) and np.array_equal(o["tokens"], am)
    # an out-of-range draft never matches and is reported
    x = am[:, :K].astype(np.int32).copy()
    x[:, 1] = V + 3
    o = oracle.verify_greedy(L, x, lib=lib)
    assert np.all(o["accept_len"] == 1) and np.all(o["status"] == 1)
    assert np.array_equal(o["tokens"][:, 1], am[:, 1])


def pin_cross_mode(lib, seed=6):
    """One-hot ("hardened") target and draft rows: stochastic verify = greedy."""
    rng = np.random.default_rng(seed)
    B, K, V = 128, 5, 40
    L = rng.standard_normal((B, K + 1, V)).astype(F32)
    am = rng.integers(0, V, size=(B, K + 1))
    np.put_along_axis(L, am[..., None], F32(1e4), axis=-1)
    D = rng.standard_normal((B, K, V)).astype(F32)
    xd = np.where(rng.random((B, K)) < 0.7, am[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    np.put_along_axis(D, xd[..., None], F32(1e4), axis=-1)
    ua = rng.random((B, K), dtype=F32)
    us = rng.random((B, K + 1), dtype=F32)
    s = oracle.verify_sample(L, D, xd, ua, us, 1.0, lib=lib)
    g = oracle.verify_greedy(L, xd, lib=lib)
    assert np.array_equal(s["accept_len"], g["accept_len"])
    assert np.array_equal(s["tokens"], g["tokens"])


def pin_dead_rows(lib, seed=8):
    """Rows after the first rejection / mismatch do not influence the outputs."""
    rng = np.random.default_rng(seed)
    B, K, V = 64, 5, 30
    lp = rng.standard_normal((B, K + 1, V)).astype(F32)
    lq = (lp[:, :K] + rng.standard_normal((B, K, V))).astype(F32)
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    ua = rng.random((B, K), dtype=F32)
    us = rng.random((B, K + 1), dtype=F32)
    o = oracle.verify_sample(lp, lq, x, ua, us, 1.0, lib=lib)
    lp2, lq2 = lp.copy(), lq.copy()
    for b in range(B):
        n = o["accept_len"][b]
        lp2[b, n + 1:] = rng.standard_normal((K - n, V)) * 50
        if n + 1 < K:
            lq2[b, n + 1:] = rng.standard_normal((K - n - 1, V)) * 50
    o2 = oracle.verify_sample(lp2, lq2, x, ua, us, 1.0, lib=lib)
    assert np.array_equal(o["accept_len"], o2["accept_len"])
    assert np.array_equal(o["tokens"], o2["tokens"])
    am = np.argmax(lp, -1)
    xg = np.where(rng.random((B, K)) < 0.6, am[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    g = oracle.verify_greedy(lp, xg, lib=lib)
    lp3 = lp.copy()
    for b in range(B):
        lp3[b, g["accept_len"][b] + 1:] = rng.standard_normal((K - g["accept_len"][b], V)) * 50
    g2 = oracle.verify_greedy(lp3, xg, lib=lib)
    assert np.array_equal(g["tokens"], g2["tokens"])


# ---------------------------------------------------------------- draw margins

def _decode(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def reference_draws(target, draft, x, ua, us, T):
    """Accept lengths, drawn tokens and draw margins recomputed from the pages'
    rule with library routines only (scipy softmax in float64, numpy cumsum and
    searchsorted), never through the oracle.  The conventions are the oracle's
    stated readings: accept iff u < p/q (q = 0 accepts, an id outside [0, V)
    has ratio 0); the token is the first v whose running mass exceeds u*Z; an
    empty residual falls back to p with the same draw and counts as a boundary.
    The margin of an acceptance draw is |u - p/q| (finite ratios only); that of
    the sample draw is the distance from u to the nearer end of the chosen
    token's cell [C(v-1)/Z, C(v)/Z).  Returns a dict of arrays."""
    B, K1, V = target.shape
    K = K1 - 1
    tg, dr = _decode(target), _decode(draft)
    out = dict(accept_len=np.empty(B, np.int64), token=np.empty(B, np.int64),
               margin_accept=np.full(B, np.inf), margin_sample=np.empty(B), Z=np.empty(B))
    for b in range(B):
        n = K
        for i in range(K):
            xi = int(x[b, i])
            if 0 <= xi < V:
                p = special.softmax(tg[b, i] / T)
                q = special.softmax(dr[b, i] / T)
                r = np.inf if q[xi] == 0.0 else p[xi] / q[xi]
            else:
                r = 0.0
            u = float(ua[b, i])
            if np.isfinite(r):
                out["margin_accept"][b] = min(out["margin_accept"][b], abs(u - r))
            if not u < r:
                n = i
                break
        p = special.softmax(tg[b, n] / T)
        mass = np.maximum(0.0, p - special.softmax(dr[b, n] / T)) if n < K else p
        C = np.cumsum(mass)
        fallback = not C[-1] > 0.0
        if fallback:
            C = np.cumsum(p)
        Z = C[-1]
        u = float(us[b, n])
        v = int(np.searchsorted(C, u * Z, side="right"))
        if v >= V:  # u*Z at or past the total: the last token with mass, a boundary
            v = int(np.nonzero(np.diff(np.concatenate([[0.0], C])) > 0)[0][-1])
            m = 0.0
        else:
            lo = C[v - 1] if v > 0 else 0.0
            m = min(abs(u - lo / Z), abs(u - C[v] / Z))
        out["accept_len"][b] = n
        out["token"][b] = v
        out["margin_sample"][b] = 0.0 if fallback else m
        out["Z"][b] = Z
    return out


def check_margins(o, ref, tol=1e-9):
    """The oracle's margins equal the recomputed ones within tol (both are
    float64 with different summation orders); its decisions equal them
    wherever the recomputed margins leave room for that rounding."""
    B = len(ref["accept_len"])
    ma, ms = o["margin_accept"], o["margin_sample"]
    fin = np.isfinite(ref["margin_accept"])
    assert np.array_equal(np.isfinite(ma), fin), "which requests have an acceptance margin"
    assert np.all(np.abs(ma[fin] - ref["margin_accept"][fin]) <= tol), \
        np.abs(ma[fin] - ref["margin_accept"][fin]).max()
    assert np.all(np.abs(ms - ref["margin_sample"]) <= tol), np.abs(ms - ref["margin_sample"]).max()
    assert np.all(o["margin"] == np.minimum(ma, ms)), "margin is the smaller of the two"
    sure_a = ref["margin_accept"] > tol
    assert np.array_equal(o["accept_len"][sure_a], ref["accept_len"][sure_a])
    sure = sure_a & (ref["margin_sample"] > tol)
    n = o["accept_len"]
    assert np.array_equal(o["tokens"][np.arange(B), n][sure], ref["token"][sure])


def pin_margins(lib, seed=13):
    """Draw margins (which decide the flagged requests) recomputed independently:
    random drafts and draws, draws planted on decision boundaries, ratios above 1,
    and the empty-residual fallback."""
    rng = np.random.default_rng(seed)
    for (B, K, V, T) in ((300, 3, 6, 1.0), (200, 2, 40, 0.7), (64, 0, 9, 1.3)):
        lp = (rng.standard_normal((B, K + 1, V)) * 1.5).astype(F32)
        lq = (lp[:, :K] + rng.standard_normal((B, K, V))).astype(F32)
        P, Q = softmax64(lp, T), softmax64(lq, T)
        x = np.empty((B, K), np.int32)
        for b in range(B):
            for i in range(K):
                x[b, i] = rng.choice(V, p=Q[b, i])
        ua = rng.random((B, K), dtype=F32)
        us = rng.random((B, K + 1), dtype=F32)
        # plant draws on boundaries: an acceptance draw at its ratio, a sample
        # draw at a cell edge of the bonus row
        for b in range(0, B, 7):
            if K:
                r = P[b, 0, x[b, 0]] / Q[b, 0, x[b, 0]]
                if r < 1:
                    ua[b, 0] = F32(r)
            us[b, K] = F32(np.cumsum(P[b, K])[rng.integers(0, V - 1)])
        o = oracle.verify_sample(lp, lq, x, ua, us, T, threads=1, lib=lib)
        ref = reference_draws(lp, lq, x, ua, us, T)
        check_margins(o, ref)
        assert (o["margin"] <= 1e-6).any() and (o["margin"] > 1e-6).any()
        if K == 0:
            assert np.all(np.isinf(o["margin_accept"]))
    # empty residual: draft row = target row at a rejection forced by an
    # out-of-range id; the draw from p is a boundary case (margin 0)
    B, K, V = 8, 2, 12
    lp = rng.standard_normal((B, K + 1, V)).astype(F32)
    lq = rng.standard_normal((B, K, V)).astype(F32)
    lq[:, 1] = lp[:, 1]
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    x[:, 1] = np.where(np.arange(B) % 2, -1, V)
    ua = np.zeros((B, K), F32)
    us = rng.random((B, K + 1), dtype=F32)
    o = oracle.verify_sample(lp, lq, x, ua, us, 1.0, threads=1, lib=lib)
    ref = reference_draws(lp, lq, x, ua, us, 1.0)
    check_margins(o, ref)
    assert np.all(o["accept_len"] == 1) and np.all(o["margin_sample"] == 0.0)


def pin_margins_full_vocab(lib, requests=4):
    """The same recomputation on the first requests of the B=32 bf16 workload
    at its full vocabulary (151936)."""
    import workloads

    w = workloads.make_workload("sample_b32_k7_qwen3")
    sl = slice(0, requests)
    args = (w.target[sl], w.draft[sl], w.draft_tokens[sl], w.u_accept[sl], w.u_sample[sl], w.T)
    o = oracle.verify_sample(*args, lib=lib)
    check_margins(o, reference_draws(*args))


# ------------------------------------------------------------------------ trees

def brute_force_tree(L, tok, par):
    """Enumerate every root-to-leaf path; return (depth, node, path, tokens)
    of the deepest accepted prefix, lowest terminal node index on ties."""
    N = len(par)
    am = np.argmax(L, -1)
    children = {j: [] for j in range(N)}
    for j in range(1, N):
        children[par[j]].append(j)
    leaves = [j for j in range(N) if not children[j]]
    best = (0, 0)
    for leaf in leaves:
        path = []
        j = leaf
        while j != 0:
            path.append(j)
            j = par[j]
        path.reverse()
        # accepted prefix of this root-to-leaf path
        prev = 0
        for d, node in enumerate(path, start=1):
            if tok[node] != am[prev]:
                break
            prev = node
            if (d, -node) > (best[0], -best[1]):
                best = (d, node)
    d, node = best
    path = []
    j = node
    while j != 0:
        path.append(j)
        j = par[j]
    path.reverse()
    return d, node, path, [int(tok[j]) for j in path] + [int(am[node])]


def random_tree(rng, N):
    par = np.empty(N, np.int32)
    par[0] = -1
    for j in range(1, N):
        par[j] = rng.integers(0, j)
    return par


def pin_tree(lib, seed=10):
    rng = np.random.default_rng(seed)
    B, N, V = 400, 12, 4
    L = rng.integers(-1, 2, size=(B, N, V)).astype(F32)  # many ties
    par = np.stack([random_tree(rng, N) for _ in range(B)])
    par[:50] = np.arange(-1, N - 1)            # chains
    par[50:100] = 0                            # stars
    par[50:100, 0] = -1
    am = np.argmax(L, -1)
    pam = np.take_along_axis(am, np.maximum(par, 0), 1)
    tok = np.where(rng.random((B, N)) < 0.6, pam, rng.integers(0, V, (B, N))).astype(np.int32)
    o = oracle.verify_tree(L, tok, par, lib=lib)
    for b in range(B):
        d, node, path, toks = brute_force_tree(L[b], tok[b], par[b])
        assert o["accept_len"][b] == d, b
        assert list(o["path"][b, :d]) == path and np.all(o["path"][b, d:] == -1)
        assert list(o["tokens"][b, :d + 1]) == toks and np.all(o["tokens"][b, d + 1:] == -1)
    # a chain-shaped tree is the greedy chain
    K = N - 1
    g = oracle.verify_greedy(L[:50], tok[:50, 1:], lib=lib)
    assert np.array_equal(g["accept_len"], o["accept_len"][:50])
    assert np.array_equal(g["tokens"], o["tokens"][:50, :K + 1])
    # malformed parent arrays are reported, not walked
    bad = par[:3].copy()
    bad[0, 5] = 7
    bad[1, 0] = 0
    bad[2, 3] = -2
    ob = oracle.verify_tree(L[:3], tok[:3], bad, lib=lib)
    assert np.all(ob["accept_len"] == -1) and np.all(ob["status"] == 2)
    assert np.all(ob["tokens"] == -1) and np.all(ob["path"] == -1)


ALL_FAST = (pin_position_lossless, pin_sequence_lossless, pin_expected_accept_length,
            pin_special_cases, pin_lse, pin_greedy, pin_cross_mode, pin_dead_rows, pin_margins,
            pin_tree)
