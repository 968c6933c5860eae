"""The KV-commit oracle (oracle/kv_commit.py) against facts fixed independently
of it: a hand-worked example, a row-by-row copy into a separate buffer, the
rows a commit must not touch, and each status code (CPU only)."""

import numpy as np
import pytest

import oracle
import workloads
from oracle import kv_commit


def _cache(G, B, S, rb, seed):
    return np.random.default_rng(seed).integers(0, 256, size=(G, B, S, rb), dtype=np.uint8)


def test_hand_worked_example():
    # One group, one request, 8 slots of 2 bytes; row s holds (10s, 10s+1).
    # Tree at slot 2 (root 2, nodes 1..4 at slots 3..6); accepted path = nodes
    # 1 and 3 (slots 3 and 5) committed after the root: slots 3 and 4.
    src = np.array([[[[10 * s, 10 * s + 1] for s in range(8)]]], dtype=np.uint8)
    out, st = kv_commit.commit_tree_kv(src, None, [2], [3], [2], np.array([[1, 3, -1, -1]]), N=5)
    want = src.copy()
    want[0, 0, 3] = [30, 31]  # node 1 stays in place
    want[0, 0, 4] = [50, 51]  # node 3 (old slot 5) moves to slot 4
    assert st.tolist() == [0]
    assert np.array_equal(out, want)


def _random_paths(B, N, seed):
    """Accepted paths of random AdaPLD-shaped trees, from the tree oracle."""
    shape = dict(n_main=8, n_branch=12) if N == 33 else dict(n_main=2, n_branch=2, max_extra=1)
    w = workloads.make_tree(B, 50, "f32", p_match=0.8, seed=seed, **shape)
    assert w.N == N
    o = oracle.verify_tree(w.target, w.node_tokens, w.parents)
    return o["accept_len"], o["path"]


@pytest.mark.parametrize("N", [33, 7])
def test_matches_row_by_row_copy_into_a_separate_buffer(N):
    G, B, S, rb = 3, 16, 80, 16
    d, path = _random_paths(B, N, seed=N)
    assert d.max() >= 2
    rng = np.random.default_rng(1)
    tb = rng.integers(0, S - N, size=B)
    cb = rng.integers(0, S - N, size=B)
    src = _cache(G, B, S, rb, 2)
    dst = _cache(G, B, S, rb, 3)
    out, st = kv_commit.commit_tree_kv(src, dst, tb, cb, d, path, N)
    want = dst.copy()
    for b in range(B):
        for k in range(int(d[b])):
            for g in range(G):
                want[g, b, cb[b] + k] = src[g, b, tb[b] + path[b, k]]
    assert (st == 0).all()
    assert np.array_equal(out, want)


def test_in_place_equals_increasing_order_copies_when_commit_base_is_at_most_tree_base_plus_one():
    # the property the device kernel relies on: in place with commit_base <=
    # tree_base + 1, copying rows one at a time in increasing k reads every
    # source before any write lands on it
    G, B, S, rb, N = 2, 32, 64, 4, 33
    d, path = _random_paths(B, N, seed=9)
    rng = np.random.default_rng(4)
    tb = rng.integers(3, S - N, size=B)
    cb = tb + 1 - rng.integers(0, 4, size=B)
    src = _cache(G, B, S, rb, 5)
    out, st = kv_commit.commit_tree_kv(src, None, tb, cb, d, path, N)
    seq = src.copy()
    for b in range(B):
        for k in range(int(d[b])):
            seq[:, b, cb[b] + k] = seq[:, b, tb[b] + path[b, k]]
    assert (st == 0).all()
    assert np.array_equal(out, seq)


def test_rows_outside_the_committed_slots_are_untouched():
    G, B, S, rb, N = 2, 24, 70, 8, 33
    d, path = _random_paths(B, N, seed=11)
    tb = np.full(B, 20)
    cb = tb + 1
    src = _cache(G, B, S, rb, 6)
    out, _ = kv_commit.commit_tree_kv(src, None, tb, cb, d, path, N)
    mask = np.ones((G, B, S), dtype=bool)
    for b in range(B):
        mask[:, b, cb[b]:cb[b] + d[b]] = False
    assert np.array_equal(out[mask], src[mask])


def test_status_codes_and_rejected_requests_untouched():
    G, B, S, rb, N = 1, 8, 40, 4, 6
    src = _cache(G, B, S, rb, 7)
    path = np.full((B, N), -1, dtype=np.int32)
    path[:, :3] = [1, 2, 4]
    d = np.full(B, 3, dtype=np.int32)
    tb = np.full(B, 10)
    cb = np.full(B, 11)
    tb[1], cb[1] = 36, 30       # node 4 at slot 40 is out of range -> 1
    cb[2] = 38                  # commit slots 38..40 -> 1
    d[3] = 6                    # d > N-1 -> 2
    path[4, :3] = [1, 1, 2]     # not increasing -> 2
    path[5, :3] = [0, 2, 3]     # node 0 (the root) on the path -> 2
    cb[6] = 12                  # in place, tree_base + 2 -> 3
    d[7] = 0                    # nothing to commit -> 0
    out, st = kv_commit.commit_tree_kv(src, None, tb, cb, d, path, N)
    assert st.tolist() == [0, 1, 1, 2, 2, 2, 3, 0]
    for b in range(1, B):
        assert np.array_equal(out[:, b], src[:, b])
    # the same in-place-overlapping request is fine into a separate buffer
    dst = _cache(G, B, S, rb, 8)
    _, st2 = kv_commit.commit_tree_kv(src, dst, tb, cb, d, path, N)
    assert st2[6] == 0
