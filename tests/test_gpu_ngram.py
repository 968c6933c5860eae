"""GPU parity of spec_ngram_candidates (AdaPLD lexical retrieval) against
oracle/ngram.py: counts, positions and status must match exactly."""

import numpy as np
import pytest
import torch

import draft_token_verification_04_amd as sv
import workloads
from gpu_helpers import ints_to_dev, note
from oracle import ngram

pytestmark = pytest.mark.gpu


def run(ctx, lens, q, cap):
    g = sv.spec_ngram_candidates(ints_to_dev(ctx), ints_to_dev(lens), ints_to_dev(q), cap)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def check(ctx, lens, q, cap):
    o = ngram.ngram_candidates(ctx, lens, q, cap)
    g = run(ctx, lens, q, cap)
    for k in ("count", "status", "positions"):
        assert np.array_equal(g[k], o[k]), k
    return o


@pytest.mark.parametrize("n", [1, 2, 3, 5])
@pytest.mark.parametrize("cap", [0, 4, 64])
def test_random_streams(n, cap):
    note(f"ngram n={n} cap={cap}")
    w = workloads.make_ngram(24, 2900, n, seed=n * 10 + cap)
    o = check(w["context"], w["lengths"], w["queries"], cap)
    assert o["count"].sum() > 0


def test_windows_across_rows_and_chunks():
    # the same 6-gram planted so that its windows straddle 64-position rows and
    # 1024-position chunks, plus one ending exactly at the last usable position
    note("ngram boundaries")
    B, L = 6, 4200
    rng = np.random.default_rng(3)
    ctx = rng.integers(1000, 2000, size=(B, L)).astype(np.int32)
    gram = np.arange(1, 7, dtype=np.int32)
    ends = [5, 66, 127, 1026, 1100, 2050, 3075, 4100]
    for b in range(B):
        for e in ends:
            ctx[b, e - 5:e + 1] = gram
    lens = np.array([4200, 4101, 4100, 1024, 64, 6], dtype=np.int32)
    for n in (1, 3, 6):
        q = np.tile(gram[-n:], (B, 1))
        o = check(ctx, lens, q, 16)
        assert o["count"][0] == len(ends)


@pytest.mark.parametrize("n", [2, 5, 64])
def test_windows_across_lanes_rows_and_chunks_of_four_token_lanes(n):
    # a lane holds four consecutive positions of each 256-position row and a
    # wave 2048 positions: windows planted to end at every offset around lane,
    # row and chunk starts, and to reach back across them
    note(f"ngram lane/row/chunk boundaries n={n}")
    B, L = 4, 6400
    rng = np.random.default_rng(11 + n)
    ctx = rng.integers(1000, 1100, size=(B, L)).astype(np.int32)
    gram = np.arange(1, n + 1, dtype=np.int32)
    ends = [e for e in (63, 64, 67, 68, 255, 256, 258, 259, 511, 2047, 2048, 2049, 2050, 2111, 4095,
                        4096, 6143, 6144, 6397) if e >= n - 1]
    # keep the windows apart so each end is one candidate
    chosen = []
    for e in ends:
        if all(abs(e - c) >= n for c in chosen):
            chosen.append(e)
    for b in range(B):
        for e in chosen:
            ctx[b, e - n + 1:e + 1] = gram
    lens = np.array([6400, 6399, 4097, 2050], dtype=np.int32)
    o = check(ctx, lens, np.tile(gram, (B, 1)), 32)
    assert o["count"][0] == len(chosen)


def test_unaligned_context():
    # rows that are not 16-byte aligned (L % 4 != 0, and a base 4 bytes past
    # an aligned address) take the element-by-element loads
    note("ngram unaligned rows")
    B, L, n = 5, 3001, 3
    w = workloads.make_ngram(B, L, n, seed=9)
    ctx, lens, q = w["context"], w["lengths"], w["queries"]
    o = ngram.ngram_candidates(ctx, lens, q, 16)
    buf = torch.zeros(B * L + 4, dtype=torch.int32, device="cuda")
    view = buf[1:1 + B * L].view(B, L)
    view.copy_(torch.from_numpy(ctx).cuda())
    assert view.data_ptr() % 16 != 0
    g = sv.spec_ngram_candidates(view, ints_to_dev(lens), ints_to_dev(q), 16)
    torch.cuda.synchronize()
    for k in ("count", "status", "positions"):
        assert np.array_equal(g[k].cpu().numpy(), o[k]), k
    assert o["count"].sum() > 0


def test_longest_query_and_lengths_at_the_edges():
    note("ngram n=64 and edge lengths")
    B, L = 9, 1500
    rng = np.random.default_rng(4)
    ctx = rng.integers(0, 50, size=(B, L)).astype(np.int32)
    span = rng.integers(0, 50, size=70).astype(np.int32)
    ctx[:, 100:170] = span
    ctx[:, 800:870] = span
    q64 = np.tile(span[:64], (B, 1))
    lens = np.array([1500, 0, 1, 63, 64, 65, 1500, 1501, -1], dtype=np.int32)
    o = check(ctx, lens, q64, 8)
    assert o["status"].tolist() == [0, 0, 0, 0, 0, 0, 0, 1, 1]
    assert o["count"][0] == 2
    check(ctx, lens, ctx[:, 10:13].copy(), 8)


def test_full_size():
    s = workloads.NGRAM_SHAPE
    note(f"ngram full size {s}")
    w = workloads.make_ngram(s["B"], s["L"], s["n"], seed=20261207)
    o = check(w["context"], w["lengths"], w["queries"], s["cap"])
    assert (o["count"] > 0).mean() > 0.5


def test_many_candidates_far_above_cap():
    # a full-size batch where half the streams match at every position (count
    # far above cap) and the rest sparsely, so that ranks run across many
    # chunks of a request; two caps
    note("ngram many candidates")
    B, L = 256, 20000
    rng = np.random.default_rng(17)
    ctx = rng.integers(0, 3, size=(B, L)).astype(np.int32)
    ctx[: B // 2] = 7
    lens = rng.integers(L // 2, L + 1, size=B).astype(np.int32)
    lens[0] = L
    q = np.full((B, 3), 7, np.int32)
    q[B // 2:] = rng.integers(0, 3, size=(B - B // 2, 3))
    for cap in (64, 5000):
        o = check(ctx, lens, q, cap)
        assert o["count"][0] == L - 3 and (o["count"][B // 2:] > 0).all()


def test_long_contexts_full_size():
    # the bench's long shape: 256 streams of 64K..128K tokens
    shp = workloads.NGRAM_LONG_SHAPE
    note(f"ngram long contexts {shp}")
    w = workloads.make_ngram_long(shp["B"], shp["L"], shp["n"], seed=20261208)
    o = check(w["context"], w["lengths"], w["queries"], shp["cap"])
    assert o["count"].sum() > shp["B"]

