"""The lexical-retrieval oracle (oracle/ngram.py) against the definition
written out with loops, a hand-worked example and the properties that fix the
set (CPU only)."""

import numpy as np

import workloads
from oracle import ngram


def test_hand_worked_example():
    # context a b c a b d a b c e ; query (a b) : windows "a b" end at 1, 4, 7;
    # all have a continuation (len 10) -> {1, 4, 7}; query (b c) -> {2, 8}
    ctx = np.array([1, 2, 3, 1, 2, 4, 1, 2, 3, 5], dtype=np.int32)
    assert ngram.candidates_loop(ctx, 10, [1, 2]) == [1, 4, 7]
    assert list(ngram.candidates(ctx, 10, [1, 2])) == [1, 4, 7]
    assert list(ngram.candidates(ctx, 10, [2, 3])) == [2, 8]
    # the window ending at the last position has no continuation
    assert list(ngram.candidates(ctx, 9, [2, 3])) == [2]
    # n = 1: every occurrence of the anchor before the last position
    assert list(ngram.candidates(ctx, 10, [1])) == [0, 3, 6]


def test_vectorised_form_equals_the_loops_on_random_streams():
    w = workloads.make_ngram(12, 700, 3, seed=1)
    for n in (1, 2, 3, 5):
        for b in range(12):
            q = w["context"][b, 100:100 + n] if b % 2 else w["queries"][b, -n:]
            want = ngram.candidates_loop(w["context"][b], int(w["lengths"][b]), q)
            got = list(ngram.candidates(w["context"][b], int(w["lengths"][b]), q))
            assert got == want


def test_set_properties_and_cap():
    w = workloads.make_ngram(16, 4000, 3, seed=2)
    o = ngram.ngram_candidates(w["context"], w["lengths"], w["queries"], cap=8)
    assert o["count"].max() > 8 and (o["count"] > 0).mean() > 0.5
    for b in range(16):
        ln, q, row = int(w["lengths"][b]), w["queries"][b], w["context"][b]
        full = ngram.candidates(row, ln, q)
        assert o["count"][b] == len(full)
        k = min(8, len(full))
        assert list(o["positions"][b, :k]) == list(full[:k]) and (o["positions"][b, k:] == -1).all()
        hit = set(full.tolist())
        for p in range(2, ln - 1):  # every position in range is either in the set or fails the match
            assert (p in hit) == bool((row[p - 2:p + 1] == q).all())


def test_lengths_out_of_range_are_flagged():
    ctx = np.zeros((3, 10), dtype=np.int32)
    o = ngram.ngram_candidates(ctx, [10, 11, -1], np.zeros((3, 2), np.int32), cap=4)
    assert o["status"].tolist() == [0, 1, 1]
    assert o["count"].tolist() == [8, 0, 0]
