"""The oracle against what the pages and mathematics fix (CPU only)."""

import numpy as np
import pytest

import oracle
import pins
import workloads


def test_position_lossless(olib):
    pins.pin_position_lossless(olib)


def test_sequence_lossless(olib):
    pins.pin_sequence_lossless(olib)


def test_expected_accept_length_exact(olib):
    pins.pin_expected_accept_length(olib)


def test_expected_accept_length_monte_carlo(olib):
    pins.pin_expected_accept_length_mc(olib)


def test_chi_square_million_trials(olib):
    pins.pin_chi_square(olib)


def test_special_cases(olib):
    pins.pin_special_cases(olib)


def test_lse_matches_logsumexp(olib):
    pins.pin_lse(olib)


def test_greedy_is_argmax_decoding(olib):
    pins.pin_greedy(olib)


def test_hardened_sample_equals_greedy(olib):
    pins.pin_cross_mode(olib)


def test_dead_rows_do_not_matter(olib):
    pins.pin_dead_rows(olib)


def test_draw_margins_recomputed(olib):
    pins.pin_margins(olib)


def test_draw_margins_full_vocabulary(olib):
    pins.pin_margins_full_vocab(olib)


def test_tree_brute_force(olib):
    pins.pin_tree(olib)


def test_round_bounds_on_the_small_fp32_workload(olib):
    """Every round emits n+1 tokens, 0 <= n <= K, the first n being the drafts."""
    w = workloads.make_workload("sample_b1_k4_v1000_f32")
    o = oracle.verify_sample(w.target, w.draft, w.draft_tokens, w.u_accept, w.u_sample, w.T, lib=olib)
    n = o["accept_len"]
    assert np.all((n >= 0) & (n <= w.K))
    for b in range(w.B):
        assert np.array_equal(o["tokens"][b, : n[b]], w.draft_tokens[b, : n[b]])
        assert 0 <= o["tokens"][b, n[b]] < w.V
        assert np.all(o["tokens"][b, n[b] + 1:] == -1)


def test_greedy_workload_mean_tokens_per_round(olib):
    """Workload-4 generator at a small vocabulary: drafts match with probability
    0.8 + 0.2/V per position, so mean(n+1) = (1 - a^8)/(1 - a) within 4 SE."""
    w = workloads.make_greedy(512, 7, 4096, seed=123)
    o = oracle.verify_greedy(w.target, w.draft_tokens, lib=olib)
    N = o["accept_len"] + 1.0
    a = 0.8 + 0.2 / w.V
    closed = (1 - a ** 8) / (1 - a)
    assert abs(N.mean() - closed) < 4 * N.std() / np.sqrt(w.B)


def test_tree_workload_matches_brute_force(olib):
    w = workloads.make_tree(16, 512, seed=77)
    o = oracle.verify_tree(w.target, w.node_tokens, w.parents, lib=olib)
    from workloads import bf16_bits_to_f32
    for b in range(w.B):
        d, node, path, toks = pins.brute_force_tree(bf16_bits_to_f32(w.target[b]), w.node_tokens[b],
                                                   w.parents[b])
        assert o["accept_len"][b] == d
        assert list(o["path"][b, :d]) == path
        assert list(o["tokens"][b, : d + 1]) == toks


def test_hand_worked_examples(olib):
    import golden_cases as gc

    g = gc.load()
    for c in g["sample"]:
        o = oracle.verify_sample(*gc.sample_arrays(c), 1.0, lib=olib)
        assert o["accept_len"][0] == c["accept_len"], c["name"]
        assert list(o["tokens"][0]) == c["tokens"], c["name"]
    for c in g["greedy"]:
        o = oracle.verify_greedy(*gc.greedy_arrays(c), lib=olib)
        assert o["accept_len"][0] == c["accept_len"], c["name"]
        assert list(o["tokens"][0]) == c["tokens"], c["name"]
    for c in g["tree"]:
        o = oracle.verify_tree(*gc.tree_arrays(c), lib=olib)
        assert o["accept_len"][0] == c["accept_len"], c["name"]
        assert list(o["path"][0]) == c["path"], c["name"]
        assert list(o["tokens"][0]) == c["tokens"], c["name"]
