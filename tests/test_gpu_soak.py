"""Repeated full-size calls of the row-skipping passes against the oracle
(needs an MI355X; marked slow).

The skip passes hand decisions between waves through memory words that other
waves poll, so their outputs must not depend on the timing of those
hand-offs.  Each test takes one full-size workload, generated once, and
varies what decides the rows each request needs over 200 seeds: the draft
tokens of the greedy chain (B=256 K=7 V=151936, a draft equals its row's
argmax with probability 0.8), the node tokens and extra leaves of the tree
(B=64 N=33), and the uniforms of the stochastic chain without lse outputs
(B=256 K=7 T=0.7); and, for the chain and tree passes' sampled rejections,
1000 seeded random shapes.  Every call is compared with the oracle, and each
test stops at its first mismatch.  No known failure is targeted.
"""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import (check_exact, check_sample, gpu_greedy, gpu_sample, gpu_tree, note)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

SEEDS = 200


def test_soak_greedy_chain():
    w = workloads.make_workload("greedy_b512_k7_qwen3", B=256)
    am = oracle.argmax(w.target)  # [B, K+1], lowest index on ties
    rng = np.random.default_rng(20261301)
    for s in range(SEEDS):
        if s % 20 == 0:
            note(f"soak greedy B=256 K=7 V=151936 seed {s}")
        match = rng.random((w.B, w.K)) < 0.8
        w.draft_tokens = np.where(match, am[:, :w.K], rng.integers(0, w.V, (w.B, w.K))).astype(np.int32)
        check_exact(gpu_greedy(w), oracle.verify_greedy(w.target, w.draft_tokens),
                    ("accept_len", "tokens", "status"))


def test_soak_tree():
    w = workloads.make_workload("tree_b64_n33_qwen3")
    am = oracle.argmax(w.target)  # [B, N]
    rng = np.random.default_rng(20261302)
    for s in range(SEEDS):
        if s % 20 == 0:
            note(f"soak tree B=64 N=33 V=151936 seed {s}")
        par = np.stack([workloads.adapld_parents(int(rng.integers(0, 4)), rng=rng) for _ in range(w.B)])
        pam = np.take_along_axis(am, np.maximum(par, 0), 1)
        tok = np.where(rng.random((w.B, w.N)) < 0.7, pam, rng.integers(0, w.V, (w.B, w.N))).astype(np.int32)
        tok[:, 0] = 0
        w.parents, w.node_tokens = par.astype(np.int32), tok
        check_exact(gpu_tree(w), oracle.verify_tree(w.target, w.node_tokens, w.parents),
                    ("accept_len", "path", "tokens", "status"))


@pytest.mark.parametrize("half", [0, 1])
def test_soak_stochastic_chain_without_lse(half):
    # the oracle's draws take about half a second per call here, so the 200
    # seeds run as two tests of 100
    w = workloads.make_workload("sample_b256_k7_qwen3_t07")
    rng = np.random.default_rng(20261303 + half)
    for s in range(SEEDS // 2):
        if s % 20 == 0:
            note(f"soak sample B=256 K=7 V=151936 T=0.7 (no lse) seeds {half}:{s}")
        u = rng.random((w.B, w.K + 1, 2), dtype=np.float32)
        w.u_accept, w.u_sample = np.ascontiguousarray(u[:, :w.K, 0]), np.ascontiguousarray(u[:, :, 1])
        o = oracle.verify_sample(w.target, w.draft, w.draft_tokens, w.u_accept, w.u_sample, w.T, lse=False)
        ncmp, nflag, _ = check_sample(w, gpu_sample(w, lse=False), o)
        assert ncmp >= 1


def test_soak_sampled_rejections_random_shapes():
    # The chain and tree passes settle some rejections before streaming, from a
    # 512-logit sample of each row.  1000 seeded random shapes (batch,
    # vocabulary, dtype, draft length or tree acceptance), half of them with
    # every mismatching token replaced by its row's second-best token, which
    # no sample can rule out; every call is compared with the oracle.
    rng = np.random.default_rng(20261303)
    for i in range(1000):
        mode = ("greedy", "tree")[i % 2]
        B = int(rng.choice([1, 2, 5, 16, 33, 64, 128]))
        V = int(rng.choice([7, 100, 513, 1000, 4099, 8192, 20011, 65536]))
        dt = str(rng.choice(["f32", "bf16"]))
        seed = int(rng.integers(1 << 30))
        plausible = bool(rng.integers(0, 2))
        if i % 100 == 0:
            note(f"soak sampled rejections case {i}")
        if mode == "greedy":
            K = int(rng.choice([0, 1, 3, 7, 15, 31]))
            w = workloads.make_greedy(B, K, V, dt, seed=seed, p_match=float(rng.choice([0.0, 0.5, 0.8, 1.0])))
        else:
            w = workloads.make_tree(B, V, dt, seed=seed, p_match=float(rng.choice([0.0, 0.3, 0.7, 1.0])))
        if plausible:
            L = workloads.bf16_bits_to_f32(w.target) if dt == "bf16" else w.target
            first = L.argmax(-1)
            masked = L.copy()
            np.put_along_axis(masked, first[..., None], -np.inf, -1)
            second = masked.argmax(-1)
            if mode == "greedy" and K > 0:
                x = w.draft_tokens
                w.draft_tokens = np.where(x != first[:, :K], second[:, :K], x).astype(np.int32)
            elif mode == "tree":
                pp = np.maximum(w.parents, 0)
                pa, pb = np.take_along_axis(first, pp, 1), np.take_along_axis(second, pp, 1)
                col = np.arange(w.N)[None, :]
                w.node_tokens = np.where((w.node_tokens != pa) & (col > 0), pb, w.node_tokens).astype(np.int32)
        if mode == "greedy":
            check_exact(gpu_greedy(w), oracle.verify_greedy(w.target, w.draft_tokens),
                        ("accept_len", "tokens", "status"))
        else:
            check_exact(gpu_tree(w), oracle.verify_tree(w.target, w.node_tokens, w.parents),
                        ("accept_len", "path", "tokens", "status"))
