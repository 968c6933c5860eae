"""GPU parity of verification fused with the LM-head projection
(spec_verify_greedy_lmhead / spec_verify_tree_lmhead / spec_verify_sample_lmhead)
against oracle/lmhead.py.

Exact-recipe inputs make every fp32 accumulation exact, so every output must
match bit for bit.  General-recipe inputs round; requests whose decisive rows
are within the accumulation bound of a tie are flagged and excluded from the
exact comparison (their count is printed).  Full-size shapes (Qwen3-8B:
D = 4096, V = 151936) are checked on sampled requests the oracle can afford."""

import numpy as np
import pytest
import torch

import draft_token_verification_04_amd as sv
import workloads
from gpu_helpers import FLAG_EPS, check_sample, dev, f32_to_dev, ints_to_dev, note
from oracle import lmhead

pytestmark = pytest.mark.gpu


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def gpu_chain(w):
    g = sv.spec_verify_greedy_lmhead(bf16_dev(w.hidden), bf16_dev(w.lm_head), ints_to_dev(w.draft_tokens))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def gpu_tree(w):
    g = sv.spec_verify_tree_lmhead(bf16_dev(w.hidden), bf16_dev(w.lm_head), ints_to_dev(w.node_tokens),
                                   ints_to_dev(w.parents))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def compare(g, o, keys, reqs=None, flagged=None):
    reqs = np.arange(len(o["accept_len"])) if reqs is None else np.asarray(reqs)
    keep = np.ones(len(reqs), bool) if flagged is None else ~flagged
    for k in keys:
        assert np.array_equal(g[k][reqs][keep], o[k][keep]), k


CHAIN_EXACT = [(3, 2, 128, 77), (5, 3, 128, 1000), (7, 7, 384, 1001), (40, 7, 256, 5000), (2, 0, 128, 300),
               (33, 7, 128, 256), (1, 1, 128, 1), (9, 3, 2560, 700),
               (4, 3, 8192, 1500)]  # 128 steps of D; partial sums stay below 2^10, so still exact


@pytest.mark.parametrize("case", CHAIN_EXACT, ids=lambda c: "B{}K{}D{}V{}".format(*c))
def test_chain_exact(case):
    B, K, D, V = case
    note(f"lmhead chain exact {case}")
    w = workloads.make_greedy_lmhead(B, K, D, V, exact=True, seed=B * 100 + K)
    o = lmhead.verify_greedy(w.hidden, w.lm_head, w.draft_tokens, exact=True)
    compare(gpu_chain(w), o, ("accept_len", "tokens", "status"))


def test_chain_general_recipe():
    note("lmhead chain general")
    w = workloads.make_greedy_lmhead(64, 7, 512, 3000, exact=False, seed=11)
    o = lmhead.verify_greedy(w.hidden, w.lm_head, w.draft_tokens)
    print(f"flagged {int(o['flagged'].sum())}/64, mean accept {o['accept_len'].mean():.2f}")
    assert o["flagged"].sum() < 16
    compare(gpu_chain(w), o, ("accept_len", "tokens", "status"), flagged=o["flagged"])


@pytest.mark.parametrize("case", [(10, 128, 2000), (3, 256, 130)], ids=lambda c: "B{}D{}V{}".format(*c))
def test_tree_exact(case):
    B, D, V = case
    note(f"lmhead tree exact {case}")
    w = workloads.make_tree_lmhead(B, D, V, exact=True, p_match=0.8, seed=B + D)
    o = lmhead.verify_tree(w.hidden, w.lm_head, w.node_tokens, w.parents, exact=True)
    compare(gpu_tree(w), o, ("accept_len", "path", "tokens", "status"))


def test_tree_many_nodes():
    """1017-node trees on a 20000-id vocabulary: 157 argmax keys per node row,
    so a request's keys fill LDS several times over and the tree kernel merges
    them in chunks of rows (the full-read tree path, N > 64)."""
    note("lmhead tree many nodes")
    w = workloads.make_tree_lmhead(2, 128, 20000, exact=True, p_match=0.9, n_main=16, n_branch=500, seed=5)
    assert w.N == 1017
    o = lmhead.verify_tree(w.hidden, w.lm_head, w.node_tokens, w.parents, exact=True)
    assert o["accept_len"].max() >= 3
    compare(gpu_tree(w), o, ("accept_len", "path", "tokens", "status"))


def test_out_of_range_drafts_and_bad_parents():
    note("lmhead bad inputs")
    w = workloads.make_greedy_lmhead(6, 4, 128, 500, exact=True, seed=3)
    w.draft_tokens[1, 0] = -3
    w.draft_tokens[2, 2] = 500
    o = lmhead.verify_greedy(w.hidden, w.lm_head, w.draft_tokens, exact=True)
    assert o["status"][1] == 1 and o["status"][2] == 1
    compare(gpu_chain(w), o, ("accept_len", "tokens", "status"))
    t = workloads.make_tree_lmhead(4, 128, 500, exact=True, seed=4)
    t.parents[2, 9] = 12
    o = lmhead.verify_tree(t.hidden, t.lm_head, t.node_tokens, t.parents, exact=True)
    assert o["status"][2] == 2
    compare(gpu_tree(t), o, ("accept_len", "path", "tokens", "status"))


@pytest.mark.parametrize("exact", [True, False], ids=["exact", "general"])
def test_chain_full_size_sampled(exact):
    # Qwen3-8B shape: B=256, K=7, D=4096, V=151936; 16 sampled requests have
    # matching drafts planted and are checked against the oracle
    s = workloads.LMHEAD_SHAPE
    reqs = np.arange(0, s["B"], s["B"] // 16)
    note(f"lmhead chain full size exact={exact}")
    w = workloads.make_greedy_lmhead(s["B"], s["K"], s["D"], s["V"], exact=exact, seed=21, plant=reqs)
    g = gpu_chain(w)
    o = lmhead.verify_greedy(w.hidden[reqs], w.lm_head, w.draft_tokens[reqs], exact=exact)
    print(f"flagged {int(o['flagged'].sum())}/{len(reqs)}, mean accept {o['accept_len'].mean():.2f}")
    assert o["accept_len"].mean() > 1.0
    compare(g, o, ("accept_len", "tokens", "status"), reqs=reqs, flagged=o["flagged"] if not exact else None)
    assert ((g["accept_len"] >= 0) & (g["accept_len"] <= s["K"])).all()


def test_tree_full_size_sampled():
    note("lmhead tree full size")
    reqs = np.arange(0, 64, 8)
    w = workloads.make_tree_lmhead(64, 4096, workloads.VOCAB_QWEN3, exact=True, seed=22, plant=reqs)
    g = gpu_tree(w)
    o = lmhead.verify_tree(w.hidden[reqs], w.lm_head, w.node_tokens[reqs], w.parents[reqs], exact=True)
    assert o["accept_len"].max() >= 2
    compare(g, o, ("accept_len", "path", "tokens", "status"), reqs=reqs)


# ---- speculative sampling on the projection ------------------------------------

def gpu_sample_lm(w, **kw):
    if w.dtype == "bf16":
        d = bf16_dev(w.draft)
    else:
        d = torch.from_numpy(np.ascontiguousarray(w.draft, np.float32)).to(dev())
    g = sv.spec_verify_sample_lmhead(bf16_dev(w.hidden), bf16_dev(w.lm_head), d if w.K else None,
                                     ints_to_dev(w.draft_tokens), f32_to_dev(w.u_accept),
                                     f32_to_dev(w.u_sample), w.T, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def oracle_sample_lm(w, reqs=None):
    r = slice(None) if reqs is None else np.asarray(reqs)
    return lmhead.verify_sample(w.hidden[r], w.lm_head, w.draft[r], w.draft_tokens[r], w.u_accept[r],
                                w.u_sample[r], w.T)


SAMPLE_EXACT = [
    # B, K, D, V, draft dtype, T
    (3, 2, 128, 77, "bf16", 1.0),
    (5, 3, 128, 1000, "f32", 0.7),
    (7, 7, 384, 1001, "bf16", 1.3),     # ragged V for bf16 drafts (unaligned path)
    (40, 7, 256, 5000, "bf16", 0.7),
    (2, 0, 128, 300, "bf16", 1.0),      # K = 0: bonus draw only
    (33, 7, 128, 258, "f32", 1.0),      # V % 4 = 2: unaligned fp32 rows
    (9, 3, 2560, 700, "bf16", 0.9),
    (300, 1, 128, 520, "bf16", 1.0),    # several row tiles in both projection passes
    (2, 1024, 128, 300, "bf16", 1.0),   # the longest chain the library accepts
    (4096, 1, 128, 200, "f32", 0.8),    # a wide batch: 16 row tiles in the rows pass
    (6, 3, 8192, 1500, "bf16", 0.9),    # 128 steps of D
]


@pytest.mark.parametrize("lse", [True, False], ids=["lse", "nolse"])
@pytest.mark.parametrize("case", SAMPLE_EXACT, ids=lambda c: "B{}K{}D{}V{}{}T{}".format(*c))
def test_sample_exact(case, lse):
    B, K, D, V, dt, T = case
    note(f"lmhead sample exact {case} lse={lse}")
    w = workloads.make_sample_lmhead(B, K, D, V, exact=True, dtype=dt, T=T, seed=B * 10 + K)
    if K >= 3 and B >= 3:  # out-of-range drafts reject at their position
        w.draft_tokens[1, 0] = -3
        w.draft_tokens[2, 2] = V
    o = oracle_sample_lm(w)
    g = gpu_sample_lm(w, lse=lse)
    n_ok, n_flag, _ = check_sample(w, g, o)
    assert n_ok >= B - 2


@pytest.mark.parametrize("dt,offset", [("f32", 4), ("bf16", 2), ("bf16", 8)],
                         ids=["f32+4B", "bf16+2B", "bf16+8B"])
def test_sample_misaligned_drafts(dt, offset):
    """Draft logits that start `offset` bytes past a 16-byte boundary: their
    statistics and the draw read them with per-element loads (fp32 and bf16 at
    +2 bytes) or 8-byte ones (bf16 at +8 bytes beside the fp32 rows)."""
    B, K, D, V = 9, 3, 256, 1000
    note(f"lmhead sample misaligned drafts {dt} +{offset} bytes")
    w = workloads.make_sample_lmhead(B, K, D, V, exact=True, dtype=dt, T=0.9, seed=77 + offset)
    esz = 4 if dt == "f32" else 2
    base = torch.empty(w.draft.size + 16 // esz, dtype=torch.float32 if dt == "f32" else torch.bfloat16,
                       device=dev())
    d = base[offset // esz:offset // esz + w.draft.size].view(w.draft.shape)
    assert d.data_ptr() % 16 == offset
    if dt == "f32":
        d.copy_(torch.from_numpy(np.ascontiguousarray(w.draft, np.float32)))
    else:
        d.copy_(bf16_dev(w.draft))
    g = sv.spec_verify_sample_lmhead(bf16_dev(w.hidden), bf16_dev(w.lm_head), d, ints_to_dev(w.draft_tokens),
                                     f32_to_dev(w.u_accept), f32_to_dev(w.u_sample), w.T)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in g.items()}
    n_ok, _, _ = check_sample(w, g, oracle_sample_lm(w))
    assert n_ok >= B - 1
    assert (g["accept_len"] < K).sum() >= 2  # residual draws read the misaligned draft rows


def test_sample_general_recipe():
    # fp32 accumulation rounds: requests whose margin is within the derived
    # bound of a decision (lmhead.sample_flag_eps) are flagged and skipped;
    # lse within the bound on a logit over T
    B, K, D, V, T = 64, 7, 128, 400, 1.0
    note("lmhead sample general")
    w = workloads.make_sample_lmhead(B, K, D, V, exact=False, T=T, noise_sigma=0.5, seed=12)
    o = oracle_sample_lm(w)
    eps = lmhead.sample_flag_eps(w.hidden, w.lm_head, T)
    g = gpu_sample_lm(w)
    flagged = o["margin"] <= np.maximum(eps, 2 * eps / np.maximum(o["Z"], 1e-300)) + FLAG_EPS
    print(f"eps {eps:.2e}: flagged {int(flagged.sum())}/{B}, mean accept {o['accept_len'].mean():.2f}")
    assert flagged.sum() < B // 2
    keep = ~flagged
    assert np.array_equal(g["accept_len"][keep], o["accept_len"][keep])
    assert np.array_equal(g["tokens"][keep], o["tokens"][keep])
    E = lmhead.accumulation_bound(w.hidden, w.lm_head).max()
    assert (np.abs(g["lse_target"] - o["lse_target"]) <= E / T + 1e-5 * np.abs(o["lse_target"]) + 1e-6).all()
    assert (np.abs(g["lse_draft"] - o["lse_draft"]) <= 1e-5 * np.abs(o["lse_draft"]) + 1e-6).all()


def test_sample_full_size_sampled():
    # Qwen3-8B shape: B=256, K=7, D=4096, V=151936, bf16 draft logits, T=0.7;
    # 16 sampled requests have draft logits shaped on the target's and are
    # checked against the oracle
    s = workloads.LMHEAD_SHAPE
    reqs = np.arange(0, s["B"], s["B"] // 16)
    note("lmhead sample full size")
    w = workloads.make_sample_lmhead(s["B"], s["K"], s["D"], s["V"], exact=True, dtype="bf16", T=0.7,
                                     seed=23, plant=reqs)
    g = gpu_sample_lm(w)
    o = oracle_sample_lm(w, reqs)
    sub = {k: v[reqs] for k, v in g.items()}
    n_ok, n_flag, _ = check_sample(w, sub, o)
    print(f"unflagged {n_ok}/{len(reqs)}, mean accept {o['accept_len'].mean():.2f}")
    assert n_ok >= len(reqs) - 1
    assert o["accept_len"].mean() > 0.5
    assert ((g["accept_len"] >= 0) & (g["accept_len"] <= s["K"])).all()
    assert ((g["tokens"][np.arange(s["B"]), g["accept_len"]] >= 0)).all()


def test_sample_trace_names_each_kernel():
    note("lmhead sample trace")
    w = workloads.make_sample_lmhead(8, 3, 128, 700, exact=True, seed=3)
    sv.trace_begin(64)
    gpu_sample_lm(w)
    recs = sv.trace_end()
    assert [r[0] for r in recs] == ["lmhead_stats", "merge_parts", "rowstats", "accept", "lmhead_rows",
                                    "resid_mass", "resid_select"]
