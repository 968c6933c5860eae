"""Seeded generators: determinism, shapes, bf16 rounding, tree structure (CPU)."""

import numpy as np

import workloads


def _rne_reference(a):
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_bf16_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(200_000) * 7).astype(np.float32)
    # include exact ties between two bf16 neighbours
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    a = np.concatenate([a, ties, -ties])
    assert np.array_equal(workloads.to_bf16_bits(a), _rne_reference(a))


def test_deterministic_and_shaped():
    a = workloads.make_sample(3, 2, 257, "bf16", 0.7, seed=5)
    b = workloads.make_sample(3, 2, 257, "bf16", 0.7, seed=5)
    for k in ("target", "draft", "draft_tokens", "u_accept", "u_sample"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    assert a.target.shape == (3, 3, 257) and a.target.dtype == np.uint16
    assert a.draft.shape == (3, 2, 257)
    assert a.u_accept.shape == (3, 2) and a.u_sample.shape == (3, 3)
    assert np.all((a.u_accept >= 0) & (a.u_accept < 1))
    assert np.all((a.draft_tokens >= 0) & (a.draft_tokens < 257))


def test_spikes_added():
    w = workloads.make_sample(2, 1, 4096, "f32", 1.0, spikes=20, spike_height=8.0, seed=1)
    L = w.target.reshape(-1, 4096)
    assert np.all((L > 8.0 - 12).sum(-1) > 0)
    assert np.all((L > 6.0).sum(-1) >= 15)


def test_adapld_tree_shape():
    rng = np.random.default_rng(3)
    for extra in range(4):
        par = workloads.adapld_parents(extra, rng=rng)
        assert len(par) == 33 and par[0] == -1
        assert np.all(par[1:] >= 0) and np.all(par[1:] < np.arange(1, 33))
        assert list(par[1:9]) == list(range(0, 8))
        assert np.all(par[9:21] == 0)
        assert np.all(par[21:33 - extra] == np.arange(9, 21 - extra))


def test_greedy_drafts_follow_argmax():
    w = workloads.make_greedy(64, 7, 1000, seed=2)
    am = np.argmax(workloads.bf16_bits_to_f32(w.target), -1)
    hit = w.draft_tokens == am[:, :7]
    assert 0.7 < hit.mean() < 0.9
