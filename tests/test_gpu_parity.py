"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Sizes: small grids that span several segments/tiles with ragged tails
(including V not a multiple of the 16-byte vector, and misaligned pointers),
then the five workloads at full size in the launch configuration the
benchmark times.
"""

import zlib

import numpy as np
import pytest
import torch

import draft_token_verification_04_amd as sv
import golden_cases as gc
import oracle
import workloads
from gpu_helpers import (check_exact, check_lse, check_sample, dev, gpu_greedy, gpu_sample,
                         gpu_tree, ints_to_dev, logits_to_dev, f32_to_dev, note, oracle_sample)

pytestmark = pytest.mark.gpu


def test_library_is_the_hip_build():
    note("library load")
    assert torch.cuda.is_available()
    assert "gfx950" in sv.version()
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName


SAMPLE_GRID = [
    # B, K, V, dtype, T, spikes, noise
    (1, 1, 8, "f32", 1.0, 0, 0.5),
    (3, 4, 1000, "f32", 1.0, 0, 0.5),
    (5, 3, 1001, "bf16", 0.7, 0, 1.0),      # ragged, unaligned bf16 rows
    (7, 7, 4100, "bf16", 1.3, 5, 1.0),      # V % 8 = 4: unaligned for bf16
    (4, 7, 4100, "f32", 0.9, 5, 2.0),       # aligned for f32
    (33, 2, 37, "bf16", 1.0, 0, 3.0),
    (2, 7, 151936, "bf16", 0.7, 20, 0.3),   # many segments and tiles per row
    (9, 1, 70001, "f32", 1.0, 3, 0.1),      # high acceptance, ragged
    (16, 0, 5000, "bf16", 1.0, 0, 1.0),     # K = 0: bonus draw only
    (3, 3, 151936, "f32", 1.0, 20, 0.5),    # a position has more segments than a wave has lanes
    (4, 31, 2000, "bf16", 1.0, 0, 0.2),     # the largest K of the row-skipping pass
    (4, 32, 2000, "f32", 1.0, 0, 0.2),      # the smallest K beyond it: every row read
    (3, 40, 3000, "bf16", 1.0, 0, 0.3),
    (4, 5, 262144, "bf16", 0.8, 10, 0.3),   # a 256K vocabulary: 86 segment partials per position
]


# lse=True reads every row (its statistics feed the lse outputs); lse=False
# takes the path that never reads rows after a request's first rejection.
@pytest.mark.parametrize("lse", [True, False], ids=["full", "skip"])
@pytest.mark.parametrize("case", SAMPLE_GRID, ids=lambda c: "B{}K{}V{}{}T{}".format(*c[:5]))
def test_sample_grid(case, lse):
    B, K, V, dt, T, spikes, noise = case
    note(f"sample grid {case} lse={lse}")
    w = workloads.make_sample(B, K, V, dt, T, target_sigma=3.0, spikes=spikes, noise_sigma=noise,
                              seed=zlib.crc32(repr(case).encode()))
    o = oracle_sample(w)
    g = gpu_sample(w, lse=lse)
    ncmp, nflag, ndiff = check_sample(w, g, o)
    assert ncmp + nflag == B and ncmp >= 1


@pytest.mark.parametrize("lse", [True, False], ids=["full", "skip"])
@pytest.mark.parametrize("c", ["sample_b1_k4_v1000_f32", "sample_b32_k7_qwen3", "sample_b256_k7_qwen3_t07"])
def test_sample_workloads_full_size(c, lse):
    note(f"sample workload {c} lse={lse}")
    w = workloads.make_workload(c)
    o = oracle_sample(w)
    g = gpu_sample(w, lse=lse)
    ncmp, nflag, ndiff = check_sample(w, g, o)
    print(f"workload {c} lse={lse}: compared {ncmp}, flagged {nflag}, flagged-and-different {ndiff}, "
          f"mean accept {g['accept_len'].mean():.3f}")


# K <= 31 takes the row-skipping pass, larger K the full read (argmax + match).
GREEDY_GRID = [(1, 0, 8, "f32"), (5, 3, 1000, "bf16"), (6, 7, 1001, "bf16"), (33, 7, 4100, "f32"),
               (3, 7, 151936, "bf16"), (64, 70, 333, "bf16"), (2, 1, 1, "f32"),
               (40, 31, 2500, "bf16"), (40, 32, 2500, "bf16"), (7, 31, 20001, "f32"),
               (4, 7, 262144, "bf16")]


@pytest.mark.parametrize("case", GREEDY_GRID, ids=lambda c: "B{}K{}V{}{}".format(*c))
def test_greedy_grid(case):
    B, K, V, dt = case
    note(f"greedy grid {case}")
    w = workloads.make_greedy(B, K, V, dt, seed=B * 1000 + K)
    o = oracle.verify_greedy(w.target, w.draft_tokens)
    g = gpu_greedy(w)
    check_exact(g, o, ("accept_len", "tokens", "status"))


def test_greedy_ties_and_signed_zeros():
    note("greedy ties")
    rng = np.random.default_rng(5)
    B, K, V = 256, 5, 3000
    L = rng.integers(-3, 4, size=(B, K + 1, V)).astype(np.float32)
    L[:8] = -0.0
    L[8:16] = 0.0
    L[8:16, :, ::7] = -0.0
    am = np.argmax(L, -1)
    x = np.where(rng.random((B, K)) < 0.7, am[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    for dt in ("f32", "bf16"):
        LL = L if dt == "f32" else workloads.to_bf16_bits(L)
        w = workloads.Workload(mode="greedy", B=B, K=K, V=V, dtype=dt, target=LL, draft_tokens=x)
        check_exact(gpu_greedy(w), oracle.verify_greedy(LL, x), ("accept_len", "tokens", "status"))


@pytest.mark.parametrize("p_match", [1.0, 0.0, 0.5])
def test_greedy_acceptance_extremes(p_match):
    # every draft accepted (every row decides), none (only row 0 decides), mixed
    note(f"greedy p_match={p_match}")
    w = workloads.make_greedy(96, 7, 30011, "bf16", p_match=p_match, seed=11)
    o = oracle.verify_greedy(w.target, w.draft_tokens)
    g = gpu_greedy(w)
    check_exact(g, o, ("accept_len", "tokens", "status"))
    if p_match == 1.0:
        assert (o["accept_len"] == 7).all()


@pytest.mark.parametrize("B,K,V", [(96, 7, 5000), (384, 7, 151936), (40, 31, 3000)],
                         ids=["B96K7V5000", "B384K7V151936", "B40K31V3000"])
def test_greedy_plausible_mismatches_and_sample_ties(B, K, V):
    # The chain pass stops reading a request at the first draft whose logit is
    # below the largest of the first 512 logits of its row.  Here mismatching
    # drafts carry tokens that sample cannot reject: the row's second-best
    # token, or a token past the sample whose logit equals the sample's
    # maximum (a tie, left to the full decision), beside argmax and random
    # drafts and rows whose argmax lies inside the sample.  B=384 at the full
    # vocabulary takes the pass's early rejection test without rotation.
    note(f"greedy plausible mismatches B={B} K={K} V={V}")
    rng = np.random.default_rng(78 + B)
    L = workloads.to_bf16_bits(rng.standard_normal((B, K + 1, V)).astype(np.float32) * 3)
    L[:8, :, 11] = workloads.to_bf16_bits(np.full((8, K + 1), 20.0, np.float32))  # argmax in the sample
    Lf = workloads.bf16_bits_to_f32(L)
    first = Lf.argmax(-1)                                  # lowest index among equals
    masked = Lf.copy()
    np.put_along_axis(masked, first[..., None], -np.inf, axis=-1)
    second = masked.argmax(-1)
    del masked
    smax_at = Lf[..., :512].argmax(-1)
    mode = rng.choice(4, size=(B, K), p=[0.7, 0.1, 0.1, 0.1])
    x = rng.integers(0, V, size=(B, K)).astype(np.int32)
    x = np.where(mode == 0, first[:, :K], x)
    x = np.where(mode == 1, second[:, :K], x)
    tie = np.argwhere(mode == 2)
    for b, p in tie:
        t = int(rng.integers(512, V))
        L[b, p, t] = L[b, p, smax_at[b, p]]
        x[b, p] = t
    x = x.astype(np.int32)
    w = workloads.Workload(mode="greedy", B=B, K=K, V=V, dtype="bf16", target=L, draft_tokens=x)
    o = oracle.verify_greedy(L, x)
    check_exact(gpu_greedy(w), o, ("accept_len", "tokens", "status"))
    assert (o["accept_len"] >= 3).any() and (o["accept_len"] == 0).any()


@pytest.mark.parametrize("B", [512, 256])
def test_greedy_workload_full_size(B):
    note(f"greedy workload B={B} K=7 V=151936")
    w = workloads.make_workload("greedy_b512_k7_qwen3", B=B)
    o = oracle.verify_greedy(w.target, w.draft_tokens)
    g = gpu_greedy(w)
    check_exact(g, o, ("accept_len", "tokens", "status"))


def test_tree_small_random_and_degenerate():
    note("tree small")
    rng = np.random.default_rng(12)
    # N <= 64 takes the row-skipping pass, larger N the full read (argmax + tree walk)
    for (B, N, V, dt) in [(50, 12, 4, "f32"), (40, 33, 1001, "bf16"), (8, 300, 64, "bf16"),
                          (3, 1, 100, "f32"), (30, 64, 500, "bf16"), (30, 65, 500, "bf16"),
                          (15, 2, 7, "f32"), (4, 17, 262144, "bf16")]:
        L = rng.integers(-1, 2, size=(B, N, V)).astype(np.float32) if V < 10 else \
            rng.standard_normal((B, N, V)).astype(np.float32)
        LL = L if dt == "f32" else workloads.to_bf16_bits(L)
        par = np.empty((B, N), np.int32)
        par[:, 0] = -1
        for j in range(1, N):
            par[:, j] = rng.integers(0, j, size=B)
        if B >= 20:
            par[:5] = np.arange(-1, N - 1)    # chains
            par[5:10, 1:] = 0                 # stars
        am = oracle.argmax(LL)
        pam = np.take_along_axis(am, np.maximum(par, 0), 1)
        tok = np.where(rng.random((B, N)) < 0.6, pam, rng.integers(0, V, (B, N))).astype(np.int32)
        if B >= 20:
            tok[10, 3] = V + 5                # out-of-range node id
            par[11, 4] = 9 if N > 9 else -1   # malformed parent array
            par[12, 0] = 0
        w = workloads.Workload(mode="tree", B=B, N=N, V=V, dtype=dt, target=LL, node_tokens=tok,
                               parents=par)
        check_exact(gpu_tree(w), oracle.verify_tree(LL, tok, par),
                    ("accept_len", "path", "tokens", "status"))


@pytest.mark.parametrize("p_match", [1.0, 0.0])
def test_tree_acceptance_extremes(p_match):
    # every node accepted (every row needed) or none (only the root row)
    note(f"tree p_match={p_match}")
    w = workloads.make_tree(48, 20011, "bf16", p_match=p_match, seed=31)
    o = oracle.verify_tree(w.target, w.node_tokens, w.parents)
    check_exact(gpu_tree(w), o, ("accept_len", "path", "tokens", "status"))
    if p_match == 0.0:
        assert (o["accept_len"] <= 1).all()


@pytest.mark.parametrize("B,V,shape", [(40, 5000, "adapld"), (64, 151936, "adapld"), (24, 3000, "random64")])
def test_tree_plausible_mismatches_and_sample_ties(B, V, shape):
    # The tree pass rejects a child before streaming when its token's logit is
    # below the largest logit of the first 512 of its parent's row.  Here the
    # mismatching children carry tokens that sample cannot reject: the row's
    # second-best token, or a token past the sample whose logit equals the
    # sample's maximum (a tie, left to the full decision), beside argmax and
    # random tokens; the first requests also put the argmax inside the sample.
    note(f"tree plausible mismatches B={B} V={V} {shape}")
    rng = np.random.default_rng(77 + B)
    if shape == "adapld":
        par = np.stack([workloads.adapld_parents(int(rng.integers(0, 4)), rng=rng) for _ in range(B)])
    else:
        N = 64
        par = np.empty((B, N), np.int32)
        par[:, 0] = -1
        for j in range(1, N):
            par[:, j] = rng.integers(0, j, size=B)
    N = par.shape[1]
    L = workloads.to_bf16_bits(rng.standard_normal((B, N, V)).astype(np.float32) * 3)
    L[:4, :, 7] = workloads.to_bf16_bits(np.full((4, N), 20.0, np.float32))  # argmax in the sample
    Lf = workloads.bf16_bits_to_f32(L)
    first = Lf.argmax(-1)
    masked = Lf.copy()
    np.put_along_axis(masked, first[..., None], -np.inf, axis=-1)
    second = masked.argmax(-1)
    del masked
    smax_at = Lf[..., :512].argmax(-1)
    pp = np.maximum(par, 0)
    mode = rng.integers(0, 4, size=(B, N))
    tok = rng.integers(0, V, size=(B, N)).astype(np.int32)
    tok = np.where(mode == 0, np.take_along_axis(first, pp, 1), tok)
    tok = np.where(mode == 1, np.take_along_axis(second, pp, 1), tok)
    for b, c in np.argwhere(mode == 2):
        if c == 0:
            continue
        p = par[b, c]
        t = int(rng.integers(512, V))
        L[b, p, t] = L[b, p, smax_at[b, p]]  # a tie past the sample; the row's argmax stays
        tok[b, c] = t
    tok = tok.astype(np.int32)
    w = workloads.Workload(mode="tree", B=B, N=N, V=V, dtype="bf16", target=L, node_tokens=tok, parents=par)
    o = oracle.verify_tree(L, tok, par)
    check_exact(gpu_tree(w), o, ("accept_len", "path", "tokens", "status"))
    assert (o["accept_len"] >= 2).any()


def test_tree_workload_full_size():
    note("tree workload B=64 N=33 V=151936")
    w = workloads.make_workload("tree_b64_n33_qwen3")
    o = oracle.verify_tree(w.target, w.node_tokens, w.parents)
    check_exact(gpu_tree(w), o, ("accept_len", "path", "tokens", "status"))


def test_chain_shaped_tree_equals_greedy_chain():
    note("chain tree")
    w = workloads.make_greedy(64, 9, 2000, "bf16", seed=3)
    par = np.tile(np.arange(-1, 9, dtype=np.int32), (64, 1))
    tok = np.concatenate([np.zeros((64, 1), np.int32), w.draft_tokens], 1)
    t = gpu_tree(workloads.Workload(mode="tree", B=64, N=10, V=2000, dtype="bf16",
                                    target=w.target, node_tokens=tok, parents=par))
    g = gpu_greedy(w)
    assert np.array_equal(t["accept_len"], g["accept_len"])
    assert np.array_equal(t["tokens"], g["tokens"])


def test_hand_worked_examples_on_gpu():
    note("golden")
    g = gc.load()
    for c in g["sample"]:
        tgt, dr, x, ua, us = gc.sample_arrays(c)
        K = x.shape[1]
        o = sv.spec_verify_sample(logits_to_dev(tgt), logits_to_dev(dr) if K else None,
                                  ints_to_dev(x), f32_to_dev(ua), f32_to_dev(us), 1.0)
        assert int(o["accept_len"][0]) == c["accept_len"], c["name"]
        assert o["tokens"][0].tolist() == c["tokens"], c["name"]
    for c in g["greedy"]:
        tgt, x = gc.greedy_arrays(c)
        o = sv.spec_verify_greedy(logits_to_dev(tgt), ints_to_dev(x))
        assert int(o["accept_len"][0]) == c["accept_len"], c["name"]
        assert o["tokens"][0].tolist() == c["tokens"], c["name"]
    for c in g["tree"]:
        tgt, tok, par = gc.tree_arrays(c)
        o = sv.spec_verify_tree(logits_to_dev(tgt), ints_to_dev(tok), ints_to_dev(par))
        assert int(o["accept_len"][0]) == c["accept_len"], c["name"]
        assert o["path"][0].tolist() == c["path"], c["name"]
        assert o["tokens"][0].tolist() == c["tokens"], c["name"]


def test_masked_vocabulary_and_out_of_range_drafts():
    note("masked vocab / OOR drafts")
    rng = np.random.default_rng(21)
    B, K, V = 24, 4, 3000
    w = workloads.make_sample(B, K, V, "f32", 1.0, spikes=0, noise_sigma=0.7, seed=9)
    mask = rng.random((B, K + 1, V)) < 0.3
    w.target[mask] = -np.inf
    w.draft[mask[:, :K]] = -np.inf
    w.draft_tokens[3, 1] = V + 7
    w.draft_tokens[4, 0] = -2
    w.u_accept[:] = 0.0  # accept everything that can be accepted
    o = oracle_sample(w)
    for lse in (True, False):
        g = gpu_sample(w, lse=lse)
        # the two out-of-range drafts meet a zero acceptance draw: ratio 0, margin 0
        check_sample(w, g, o, planted=2)
        assert g["status"][3] == 1 and g["status"][4] == 1 and g["accept_len"][4] == 0
        # masked ids are never drawn
        for b in range(B):
            n = g["accept_len"][b]
            t = g["tokens"][b, n]
            assert not mask[b, n, t]


def test_empty_batch_and_determinism():
    note("empty batch / determinism")
    w = workloads.make_sample(0, 3, 100, "bf16", 1.0, seed=1)
    g = gpu_sample(w)
    assert g["accept_len"].shape == (0,)
    w = workloads.make_sample(12, 7, 20000, "bf16", 0.8, spikes=20, noise_sigma=1.0, seed=2)
    a, b = gpu_sample(w), gpu_sample(w)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    c, d = gpu_sample(w, lse=False), gpu_sample(w, lse=False)
    for k in c:
        assert np.array_equal(c[k], d[k]), k
        assert np.array_equal(a[k], c[k]), k  # both paths agree bit for bit
    wg = workloads.make_greedy(12, 7, 20000, "bf16", seed=2)
    a, b = gpu_greedy(wg), gpu_greedy(wg)
    assert np.array_equal(a["tokens"], b["tokens"])


def test_misaligned_pointers_take_the_general_path():
    note("misaligned pointers")
    w = workloads.make_sample(6, 3, 4096, "bf16", 1.0, spikes=3, noise_sigma=1.0, seed=4)
    o = oracle_sample(w)
    base_t = torch.empty(w.target.size + 1, dtype=torch.bfloat16, device=dev())
    base_d = torch.empty(w.draft.size + 1, dtype=torch.bfloat16, device=dev())
    t = base_t[1:].view(w.target.shape)
    d = base_d[1:].view(w.draft.shape)
    t.copy_(logits_to_dev(w.target))
    d.copy_(logits_to_dev(w.draft))
    assert t.data_ptr() % 16 != 0
    g = sv.spec_verify_sample(t, d, ints_to_dev(w.draft_tokens), f32_to_dev(w.u_accept),
                              f32_to_dev(w.u_sample), w.T)
    g = {k: v.cpu().numpy() for k, v in g.items()}
    check_sample(w, g, o)
    wg = workloads.make_greedy(6, 3, 4096, "bf16", seed=4)
    base = torch.empty(wg.target.size + 1, dtype=torch.bfloat16, device=dev())
    tt = base[1:].view(wg.target.shape)
    tt.copy_(logits_to_dev(wg.target))
    gg = sv.spec_verify_greedy(tt, ints_to_dev(wg.draft_tokens))
    check_exact({k: v.cpu().numpy() for k, v in gg.items()},
                oracle.verify_greedy(wg.target, wg.draft_tokens), ("accept_len", "tokens"))


@pytest.mark.parametrize("lse", [True, False], ids=["full", "skip"])
def test_empty_residual_draws_from_p(lse):
    """A rejected position whose draft row equals its target row: both sides
    compute p and q there alike, so max(0, p - q) is 0 everywhere and the draw
    falls back to p alone with the same uniform (the rounding rule of the
    oracle's step 5).  The rejection is forced by an out-of-range draft (ratio
    0); earlier drafts pass with u = 0.  The oracle flags such a draw (margin
    0), so here the GPU token is held to the oracle's draw from p_j as a K = 0
    bonus draw, whose own margin is checked."""
    B, K, V = 8, 3, 4096
    note(f"empty residual lse={lse}")
    w = workloads.make_sample(B, K, V, "bf16", 1.0, spikes=3, noise_sigma=1.0, seed=31)
    j = np.array([0, 1, 2, 0, 1, 2, 1, 0])
    for b in range(B):
        w.draft[b, j[b]] = w.target[b, j[b]]
        w.draft_tokens[b, j[b]] = -1 if b % 2 else V
        w.u_accept[b, :j[b]] = 0.0
    o = oracle_sample(w)
    assert np.array_equal(o["accept_len"], j) and (o["margin"] == 0.0).all()
    rows = np.ascontiguousarray(w.target[np.arange(B), j][:, None, :])
    ob = oracle.verify_sample(rows, np.zeros((B, 0, V), rows.dtype), np.zeros((B, 0), np.int32),
                              np.zeros((B, 0), np.float32), w.u_sample[np.arange(B), j][:, None], w.T)
    assert (ob["margin"] > 1e-6).all()
    assert np.array_equal(o["tokens"][np.arange(B), j], ob["tokens"][:, 0])
    g = gpu_sample(w, lse=lse)
    assert np.array_equal(g["accept_len"], j)
    assert np.array_equal(g["status"], np.ones(B, np.int32))
    assert np.array_equal(g["tokens"], o["tokens"]), (g["tokens"], o["tokens"])


def test_lse_only_rows_and_temperature_extremes():
    note("lse temperature extremes")
    for T in (0.05, 0.7, 4.0):
        w = workloads.make_sample(4, 2, 9000, "bf16", T, spikes=4, noise_sigma=0.5, seed=int(T * 100))
        o = oracle_sample(w)
        g = gpu_sample(w)
        check_lse(g["lse_target"], o["lse_target"])
        check_sample(w, g, o)


def test_workspace_reuse_with_shrinking_batches():
    note("workspace reuse")
    big = workloads.make_sample(40, 7, 8000, "bf16", 1.0, spikes=5, noise_sigma=1.0, seed=31)
    need = sv.sample_workspace_bytes(40, 7, 8000, sv.SV_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device=dev())
    for B in (40, 17, 3):
        w = workloads.make_sample(B, 7, 8000, "bf16", 1.0, spikes=5, noise_sigma=1.0, seed=B)
        g = sv.spec_verify_sample(logits_to_dev(w.target), logits_to_dev(w.draft),
                                  ints_to_dev(w.draft_tokens), f32_to_dev(w.u_accept),
                                  f32_to_dev(w.u_sample), w.T, workspace=ws)
        g = {k: v.cpu().numpy() for k, v in g.items()}
        check_sample(w, g, oracle_sample(w))
    with pytest.raises(sv.SpecVerifyError):
        sv.spec_verify_sample(logits_to_dev(big.target), logits_to_dev(big.draft),
                              ints_to_dev(big.draft_tokens), f32_to_dev(big.u_accept),
                              f32_to_dev(big.u_sample), big.T, workspace=ws[:1024])


def test_trace_records_each_kernel():
    note("trace")
    w = workloads.make_sample(8, 3, 5000, "bf16", 1.0, seed=5)
    sv.trace_begin(64)
    gpu_sample(w)
    recs = sv.trace_end()
    assert [r[0] for r in recs] == ["rowstats", "accept", "resid_mass", "resid_select"]
    assert all(ms > 0 for _, ms in recs)
    sv.trace_begin(64)
    gpu_sample(w, lse=False)
    recs = sv.trace_end()
    assert [r[0] for r in recs] == ["skip_stats", "resid_mass", "resid_select"]
    # beyond 31 drafts every row is read, lse outputs or not
    wl = workloads.make_sample(2, 40, 3000, "bf16", 1.0, seed=7)
    sv.trace_begin(64)
    gpu_sample(wl, lse=False)
    recs = sv.trace_end()
    assert [r[0] for r in recs] == ["rowstats", "accept", "resid_mass", "resid_select"]
    wg = workloads.make_greedy(8, 3, 5000, "bf16", seed=6)
    sv.trace_begin(64)
    gpu_greedy(wg)
    recs = sv.trace_end()
    assert [r[0] for r in recs] == ["skip_argmax"]
    wg = workloads.make_greedy(4, 32, 5000, "bf16", seed=7)
    sv.trace_begin(64)
    gpu_greedy(wg)
    recs = sv.trace_end()
    assert [r[0] for r in recs] == ["argmax", "match"]
    wt = workloads.make_tree(4, 5000, "bf16", seed=8)
    sv.trace_begin(64)
    gpu_tree(wt)
    recs = sv.trace_end()
    assert [r[0] for r in recs] == ["skip_tree"]


def test_maximum_draft_length_and_tree_size():
    # the largest chain (K = SV_MAX_DRAFT_LEN) and tree (N = SV_MAX_TREE_NODES) the
    # library accepts, on a short vocabulary so the oracle stays quick
    K, N = 1024, sv.SV_MAX_TREE_NODES
    note(f"max sizes K={K} N={N}")
    for noise, seed in ((0.0, 51), (0.05, 52)):   # q = p (every draft accepted), then some rejections
        w = workloads.make_sample(3, K, 64, "f32", 1.0, spikes=0, noise_sigma=noise, seed=seed)
        o = oracle_sample(w)
        for lse in (True, False):
            g = gpu_sample(w, lse=lse)
            check_sample(w, g, o)
        if noise == 0.0:
            assert (o["accept_len"] == K).all()
    for p_match, seed in ((1.0, 53), (0.998, 54)):
        wg = workloads.make_greedy(3, K, 50, "f32", p_match=p_match, seed=seed)
        og = oracle.verify_greedy(wg.target, wg.draft_tokens)
        check_exact(gpu_greedy(wg), og, ("accept_len", "tokens", "status"))
        if p_match == 1.0:
            assert (og["accept_len"] == K).all()
    rng = np.random.default_rng(55)
    B, V = 3, 40
    L = rng.standard_normal((B, N, V)).astype(np.float32)
    par = np.empty((B, N), np.int32)
    par[:, 0] = -1
    par[0, 1:] = np.arange(N - 1)                      # one chain through every node
    for j in range(1, N):
        par[1:, j] = rng.integers(max(0, j - 8), j, size=B - 1)
    am = oracle.argmax(L)
    pam = np.take_along_axis(am, np.maximum(par, 0), 1)
    tok = np.where(rng.random((B, N)) < 0.97, pam, rng.integers(0, V, (B, N))).astype(np.int32)
    tok[0] = pam[0]                                   # the chain is accepted to its end
    w = workloads.Workload(mode="tree", B=B, N=N, V=V, dtype="f32", target=L, node_tokens=tok, parents=par)
    ot = oracle.verify_tree(L, tok, par)
    check_exact(gpu_tree(w), ot, ("accept_len", "path", "tokens", "status"))
    assert ot["accept_len"][0] == N - 1
