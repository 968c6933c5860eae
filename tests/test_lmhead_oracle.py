"""The LM-head oracle (oracle/lmhead.py) against facts fixed independently of
it: integer arithmetic, fp32 sums in several orders, the C oracle on exactly
representable logits, and brute-force perturbation of the argmax (CPU only)."""

import numpy as np
import pytest

import oracle
import workloads
from oracle import lmhead


def test_logits_equal_integer_arithmetic():
    # exact recipe: H = i/8, W = j/64, so 512 * logit is the integer sum of i*j
    w = workloads.make_greedy_lmhead(3, 2, 128, 77, exact=True, p_match=None, seed=1)
    H = lmhead.bf16_to_f64(w.hidden)
    W = lmhead.bf16_to_f64(w.lm_head)
    hi = np.rint(H * 8).astype(np.int64)
    wi = np.rint(W * 64).astype(np.int64)
    assert np.array_equal(hi / 8, H) and np.array_equal(wi / 64, W)
    want = np.array([[[sum(int(hi[b, r, k]) * int(wi[v, k]) for k in range(128)) for v in range(77)]
                      for r in range(3)] for b in range(3)], dtype=np.int64)
    L = lmhead.logits(w.hidden, w.lm_head)
    assert np.array_equal(L * 512, want.astype(np.float64))


def _fp32_sums(H, W, order):
    """H [M, D] @ W.T accumulated in float32 in a given order of the D products."""
    P = (H[:, None, :] * W[None, :, :]).astype(np.float32)  # products, exact in fp32
    D = P.shape[-1]
    if order == "forward":
        idx = range(D)
    elif order == "reverse":
        idx = range(D - 1, -1, -1)
    if order in ("forward", "reverse"):
        acc = np.zeros(P.shape[:2], np.float32)
        for k in idx:
            acc = acc + P[..., k]
        return acc
    if order == "pairwise":
        x = P
        while x.shape[-1] > 1:
            if x.shape[-1] % 2:
                x = np.concatenate([x, np.zeros(x.shape[:-1] + (1,), np.float32)], -1)
            x = x[..., 0::2] + x[..., 1::2]
        return x[..., 0]
    if order == "blocks16":  # 16-term partial sums added to a running total
        acc = np.zeros(P.shape[:2], np.float32)
        for k0 in range(0, D, 16):
            part = np.zeros(P.shape[:2], np.float32)
            for k in range(k0, min(D, k0 + 16)):
                part = part + P[..., k]
            acc = acc + part
        return acc
    raise ValueError(order)


@pytest.mark.parametrize("order", ["forward", "reverse", "pairwise", "blocks16"])
def test_bound_holds_for_fp32_sums_in_any_order(order):
    w = workloads.make_greedy_lmhead(2, 3, 512, 300, exact=False, p_match=None, seed=2)
    Hb = w.hidden.reshape(-1, 512)
    H = lmhead.bf16_to_f64(Hb).astype(np.float32)
    W = lmhead.bf16_to_f64(w.lm_head).astype(np.float32)
    L = lmhead.logits(Hb, w.lm_head)
    E = lmhead.accumulation_bound(Hb, w.lm_head)
    got = _fp32_sums(H, W, order).astype(np.float64)
    err = np.abs(got - L)
    assert (err <= E).all()
    assert err.max() > 0          # the sums really do round
    assert E.max() < 1e-2 * np.abs(L).max()


def test_bound_is_nearly_attained_by_an_adversarial_sum():
    # products 1, then D-1 products just under 2^-25: each is below half an ulp of
    # the running fp32 sum (1), so a forward fp32 sum stays at exactly 1 and loses
    # (D-1) * 2^-25 (1 - 2^-8), about half the bound gamma_{D-1} * sum |h w|
    D = 4096
    h = np.full(D, 2.0 ** -13, np.float32)
    w = np.full(D, 2.0 ** -12 * (1 - 2.0 ** -8), np.float32)
    h[0] = w[0] = 1.0
    Hb = workloads.to_bf16_bits(h[None, :])
    Wb = workloads.to_bf16_bits(w[None, :])
    assert np.array_equal(workloads.bf16_bits_to_f32(Hb)[0], h)  # exactly representable
    assert np.array_equal(workloads.bf16_bits_to_f32(Wb)[0], w)
    L = lmhead.logits(Hb, Wb)[0, 0]
    E = lmhead.accumulation_bound(Hb, Wb)[0, 0]
    got = float(_fp32_sums(h[None, :], w[None, :], "forward")[0, 0])
    assert got == 1.0
    assert abs(got - L) <= E
    assert abs(got - L) >= 0.45 * E


def test_certain_rows_survive_every_admissible_perturbation():
    rng = np.random.default_rng(3)
    L = rng.normal(size=(400, 50)).round(2)  # plenty of near ties
    E = np.full_like(L, 0.004)
    a, certain = lmhead.row_argmax(L, E)
    assert 0 < certain.sum() < len(certain)
    for _ in range(200):
        P = L + rng.uniform(-1, 1, size=L.shape) * E
        assert np.array_equal(np.argmax(P[certain], -1), a[certain])
    # the adversarial perturbation (top down, all others up) moves or ties every uncertain row
    adv = L + E
    np.put_along_axis(adv, a[:, None], np.take_along_axis(L - E, a[:, None], -1), -1)
    top = np.take_along_axis(adv, a[:, None], -1)[:, 0]
    other = adv.copy()
    np.put_along_axis(other, a[:, None], -np.inf, -1)
    assert (other.max(-1)[~certain] >= top[~certain]).all()


def test_exact_recipe_matches_the_c_oracle_chain():
    w = workloads.make_greedy_lmhead(24, 5, 256, 1500, exact=True, p_match=0.8, seed=4)
    L = lmhead.logits(w.hidden, w.lm_head)
    L32 = L.astype(np.float32)
    assert np.array_equal(L32.astype(np.float64), L)  # representable exactly
    o = lmhead.verify_greedy(w.hidden, w.lm_head, w.draft_tokens, exact=True)
    c = oracle.verify_greedy(L32, w.draft_tokens)
    for k in ("accept_len", "tokens", "status"):
        assert np.array_equal(o[k], c[k]), k
    assert not o["flagged"].any()
    assert o["accept_len"].mean() > 1.0


def test_exact_recipe_has_ties_resolved_to_the_lowest_index():
    w = workloads.make_greedy_lmhead(64, 7, 64, 3000, exact=True, p_match=None, seed=5)
    L = lmhead.logits(w.hidden, w.lm_head).reshape(-1, 3000)
    a, _ = lmhead.row_argmax(L, None)
    ties = (L == L.max(-1, keepdims=True)).sum(-1) > 1
    assert ties.any()
    for r in np.flatnonzero(ties):
        assert a[r] == np.flatnonzero(L[r] == L[r].max())[0]


def test_tree_walk_matches_the_c_oracle():
    w = workloads.make_tree_lmhead(40, 128, 900, exact=True, p_match=0.8, seed=6)
    L32 = lmhead.logits(w.hidden, w.lm_head).astype(np.float32)
    o = lmhead.verify_tree(w.hidden, w.lm_head, w.node_tokens, w.parents, exact=True)
    c = oracle.verify_tree(L32, w.node_tokens, w.parents)
    for k in ("accept_len", "path", "tokens", "status"):
        assert np.array_equal(o[k], c[k]), k
    assert o["accept_len"].max() >= 3
    # malformed parent arrays and out-of-range node ids
    par = w.parents.copy()
    par[0, 5] = 7
    tok = w.node_tokens.copy()
    tok[1, 3] = 900
    o2 = lmhead.verify_tree(w.hidden, w.lm_head, tok, par, exact=True)
    c2 = oracle.verify_tree(L32, tok, par)
    for k in ("accept_len", "path", "tokens", "status"):
        assert np.array_equal(o2[k], c2[k]), k
    assert o2["status"][0] == 2 and o2["status"][1] == 1


def test_general_recipe_flags_only_near_ties():
    w = workloads.make_greedy_lmhead(32, 3, 256, 2000, exact=False, p_match=0.8, seed=7)
    o = lmhead.verify_greedy(w.hidden, w.lm_head, w.draft_tokens)
    L = lmhead.logits(w.hidden, w.lm_head)
    s = np.sort(L, -1)
    gap = s[..., -1] - s[..., -2]
    E = lmhead.accumulation_bound(w.hidden, w.lm_head)
    _, certain = lmhead.row_argmax(L, E)
    assert (gap[~certain] <= 2 * E.max()).all()
    assert certain.mean() > 0.95
    assert o["flagged"].mean() < 0.2


def _integer_logits(hidden_bits, lm_head_bits):
    """Exact-recipe logits by integer arithmetic: H = i/8, W = j/64, so the
    logit is (sum of i*j) / 512."""
    hi = np.rint(lmhead.bf16_to_f64(hidden_bits) * 8).astype(np.int64)
    wi = np.rint(lmhead.bf16_to_f64(lm_head_bits) * 64).astype(np.int64)
    return (hi @ wi.T).astype(np.float64) / 512.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sampling_on_the_projection_is_sampling_on_its_logits(dtype):
    # exact recipe: the logits the fused oracle samples from are H W^T exactly
    # (integer arithmetic here), and the rest is the pinned sampling oracle
    w = workloads.make_sample_lmhead(12, 5, 128, 700, exact=True, dtype=dtype, T=0.8, seed=8)
    L = _integer_logits(w.hidden, w.lm_head)
    L32 = L.astype(np.float32)
    assert np.array_equal(L32.astype(np.float64), L)
    d = workloads.bf16_bits_to_f32(w.draft) if dtype == "bf16" else w.draft
    o = lmhead.verify_sample(w.hidden, w.lm_head, w.draft, w.draft_tokens, w.u_accept, w.u_sample, w.T)
    c = oracle.verify_sample(L32, np.ascontiguousarray(d, np.float32), w.draft_tokens, w.u_accept,
                             w.u_sample, w.T)
    for k in ("accept_len", "tokens", "status", "lse_target", "lse_draft", "margin", "Z"):
        assert np.array_equal(o[k], c[k]), k
    # the draft logits were shaped on the target's, so drafts do get accepted
    assert o["accept_len"].mean() > 0.5


def test_sampling_flag_threshold_bounds_fp32_sums_in_any_order():
    # the relative error of every p(v) = softmax(L/T)(v) built on fp32 sums in
    # any order stays within the eps the oracle derives from the bound
    w = workloads.make_sample_lmhead(2, 3, 256, 300, exact=False, T=0.7, seed=9)
    Hb = w.hidden.reshape(-1, 256)
    H = lmhead.bf16_to_f64(Hb).astype(np.float32)
    W = lmhead.bf16_to_f64(w.lm_head).astype(np.float32)
    L = lmhead.logits(Hb, w.lm_head)
    eps = lmhead.sample_flag_eps(w.hidden, w.lm_head, w.T)
    p = np.exp(L / w.T - np.log(np.exp(L / w.T).sum(-1, keepdims=True)))
    worst = 0.0
    for order in ("forward", "reverse", "pairwise", "blocks16"):
        Lf = _fp32_sums(H, W, order).astype(np.float64)
        pf = np.exp(Lf / w.T - np.log(np.exp(Lf / w.T).sum(-1, keepdims=True)))
        worst = max(worst, np.abs(pf / p - 1).max())
    assert 0 < worst <= eps
    assert eps < 1e-2
