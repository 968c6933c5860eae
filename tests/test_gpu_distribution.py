"""The GPU sampler against the law the SD tutorial page proves, not against the
oracle (needs an MI355X).

Section "为什么“猜错再改”不会偏离目标分布" of the speculative-sampling tutorial
shows that accepting a draft x ~ q with probability min(1, p(x)/q(x)), and
otherwise drawing from norm(max(0, p - q)), emits a token distributed exactly
as p; a round that accepts every draft then draws the bonus token from the next
target row.  These tests draw many rounds with fresh uniforms on the GPU and
compare the emitted tokens with p by chi-square, so a wrong residual, a wrong
ratio or a biased inverse CDF shows even where the oracle and the GPU share a
reading of the pages.
"""

import numpy as np
import pytest
import torch
from scipy import stats

import draft_token_verification_04_amd as sv
import pins
import workloads
from gpu_helpers import dev, f32_to_dev, ints_to_dev, logits_to_dev, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lse", [True, False], ids=["full", "skip"])
def test_sampler_law_on_toy_models(lse):
    """10^6 rounds with K = 2 on prefix-dependent toy models (V = 8): the first
    emitted token follows p(.|prefix) and the accept lengths follow the law of
    the overlap identity."""
    c = pins.chi_square_case(trials=1_000_000, seed=7, V=8, T=1.0)
    note(f"toy-model law, 1e6 rounds, lse={lse}")
    g = sv.spec_verify_sample(logits_to_dev(c["target"]), logits_to_dev(c["draft"]), ints_to_dev(c["x"]),
                              f32_to_dev(c["u_accept"]), f32_to_dev(c["u_sample"]), c["T"], lse=lse)
    torch.cuda.synchronize()
    pins.check_chi_square(c, g["tokens"].cpu().numpy(), g["accept_len"].cpu().numpy())


def _mass_bins(P, width=0.02, max_bins=64):
    """Token -> bin, bins holding about `width` of P's mass each (tokens sorted by
    decreasing probability; a token heavier than `width` is a bin of its own)."""
    order = np.argsort(-P, kind="stable")
    before = np.cumsum(P[order]) - P[order]
    b = np.minimum((before / width).astype(np.int64), max_bins - 1)
    _, b = np.unique(b, return_inverse=True)  # renumber densely
    bins = np.empty(len(P), np.int64)
    bins[order] = b
    return bins, np.bincount(bins, weights=P)


def _chi2_pvalue(tokens, bins, mass):
    obs = np.bincount(bins[tokens], minlength=len(mass)).astype(np.float64)
    return stats.chisquare(obs, mass / mass.sum() * obs.sum()).pvalue


def test_sampler_law_at_full_vocabulary():
    """K = 1 at the Qwen3 vocabulary (V = 151936, bf16, T = 0.7), 204,800
    rounds in 25 calls on both read paths: the first emitted token follows p_0
    (over about 40 mass bins), the acceptance count follows
    Binomial(n, sum_v min(p_0, q_0)), and the bonus tokens of accepted rounds
    follow p_1."""
    V, T, Bc, calls = 151936, 0.7, 8192, 25
    rng = np.random.default_rng(2026)
    z = rng.standard_normal(V) * 3.0
    rows = np.stack([z, rng.standard_normal(V) * 3.0, z + rng.standard_normal(V) * 1.5]).astype(np.float32)
    bits = workloads.to_bf16_bits(rows)  # target row 0, target row 1 (bonus), draft row 0
    vals = workloads.bf16_bits_to_f32(bits).astype(np.float64)
    P0, P1, Q0 = (pins.softmax64(vals[i], T) for i in range(3))
    a = np.minimum(P0, Q0).sum()

    note(f"full-vocabulary law: V={V} K=1 B={Bc} x {calls} calls")
    d = dev()
    rows_dev = logits_to_dev(bits)  # [3, V] bf16
    tgt = torch.empty((Bc, 2, V), dtype=torch.bfloat16, device=d)
    tgt[:, 0] = rows_dev[0]
    tgt[:, 1] = rows_dev[1]
    drf = rows_dev[2].expand(Bc, 1, V).contiguous()
    first, bonus, n_acc = [], [], 0
    for c in range(calls):  # odd calls read every row (lse outputs), even calls skip rows
        x = rng.choice(V, size=(Bc, 1), p=Q0)
        ua = rng.random((Bc, 1), dtype=np.float32)
        us = rng.random((Bc, 2), dtype=np.float32)
        g = sv.spec_verify_sample(tgt, drf, ints_to_dev(x), f32_to_dev(ua), f32_to_dev(us), T,
                                  lse=c % 2 == 1)
        torch.cuda.synchronize()
        tok, n = g["tokens"].cpu().numpy(), g["accept_len"].cpu().numpy()
        assert set(np.unique(n)) <= {0, 1}
        assert np.array_equal(tok[n == 1, 0], x[n == 1, 0])  # an accepted draft is emitted as is
        assert (tok[n == 0, 1] == -1).all()
        first.append(tok[:, 0])
        bonus.append(tok[n == 1, 1])
        n_acc += int(n.sum())
    first, bonus = np.concatenate(first), np.concatenate(bonus)
    total = Bc * calls
    assert stats.binomtest(n_acc, total, a).pvalue > 1e-3
    b0, m0 = _mass_bins(P0)
    assert len(m0) >= 30
    assert _chi2_pvalue(first, b0, m0) > 1e-3
    b1, m1 = _mass_bins(P1)
    assert _chi2_pvalue(bonus, b1, m1) > 1e-3


def test_fused_lmhead_sampler_law():
    """The same law through the LM-head projection (spec_verify_sample_lmhead):
    K = 1, D = 128, V = 4096, T = 0.8, exact-recipe operands, so the target
    logits z_0, z_1 are exact and p_0, p_1 follow from a plain fp64 product.
    Every request carries the same two hidden rows and the same draft row (the
    target's row 0 plus N(0, 1) noise, so about half the drafts pass); 25 calls
    of 8192 requests with fresh uniforms give 204,800 rounds.  The acceptance
    count, the first tokens and the bonus tokens are tested as above, so the
    re-formed fp32 row and the bf16 draft row read beside it are checked
    against p, not against the oracle."""
    V, D, T, Bc, calls = 4096, 128, 0.8, 8192, 25
    w = workloads.make_sample_lmhead(1, 1, D, V, exact=True, dtype="bf16", T=T, noise_sigma=1.0, seed=11)
    h = workloads.bf16_bits_to_f32(w.hidden.reshape(2, D)).astype(np.float64)
    Wf = workloads.bf16_bits_to_f32(w.lm_head).astype(np.float64)
    z = h @ Wf.T  # exact: every product and partial sum is a multiple of 2^-9 below 2^10
    q = workloads.bf16_bits_to_f32(w.draft.reshape(1, V)).astype(np.float64)[0]
    P0, P1, Q0 = pins.softmax64(z[0], T), pins.softmax64(z[1], T), pins.softmax64(q, T)
    a = np.minimum(P0, Q0).sum()
    assert 0.2 < a < 0.9

    note(f"fused LM-head law: V={V} D={D} K=1 B={Bc} x {calls} calls")
    rng = np.random.default_rng(2027)
    hid = logits_to_dev(w.hidden.reshape(1, 2, D)).expand(Bc, 2, D).contiguous()
    lm = logits_to_dev(w.lm_head)
    drf = logits_to_dev(w.draft.reshape(1, 1, V)).expand(Bc, 1, V).contiguous()
    first, bonus, n_acc = [], [], 0
    for c in range(calls):
        x = rng.choice(V, size=(Bc, 1), p=Q0)
        ua = rng.random((Bc, 1), dtype=np.float32)
        us = rng.random((Bc, 2), dtype=np.float32)
        g = sv.spec_verify_sample_lmhead(hid, lm, drf, ints_to_dev(x), f32_to_dev(ua), f32_to_dev(us), T,
                                         lse=c % 2 == 1)
        torch.cuda.synchronize()
        tok, n = g["tokens"].cpu().numpy(), g["accept_len"].cpu().numpy()
        assert set(np.unique(n)) <= {0, 1}
        assert np.array_equal(tok[n == 1, 0], x[n == 1, 0])
        assert (tok[n == 0, 1] == -1).all()
        first.append(tok[:, 0])
        bonus.append(tok[n == 1, 1])
        n_acc += int(n.sum())
    first, bonus = np.concatenate(first), np.concatenate(bonus)
    assert stats.binomtest(n_acc, Bc * calls, a).pvalue > 1e-3
    b0, m0 = _mass_bins(P0)
    assert len(m0) >= 20
    assert _chi2_pvalue(first, b0, m0) > 1e-3
    b1, m1 = _mass_bins(P1)
    assert _chi2_pvalue(bonus, b1, m1) > 1e-3
