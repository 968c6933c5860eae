"""GPU parity of spec_commit_tree_kv against the KV-commit oracle: the whole
destination buffer and the status must match byte for byte."""

import numpy as np
import pytest
import torch

import draft_token_verification_04_amd as sv
import oracle
import workloads
from gpu_helpers import dev, ints_to_dev, note
from oracle import kv_commit

pytestmark = pytest.mark.gpu


def _paths(B, seed, **shape):
    w = workloads.make_tree(B, 64, "f32", p_match=0.8, seed=seed, **shape)
    o = oracle.verify_tree(w.target, w.node_tokens, w.parents)
    return w.N, o["accept_len"], o["path"]


def _run(src, dst, tb, cb, d, path):
    kv = torch.from_numpy(src).to(dev())
    out = None if dst is None else torch.from_numpy(dst).to(dev())
    st = sv.spec_commit_tree_kv(kv, ints_to_dev(tb), ints_to_dev(cb), ints_to_dev(d), ints_to_dev(path),
                                out=out)
    torch.cuda.synchronize()
    res = kv if out is None else out
    return res.cpu().numpy(), st.cpu().numpy()


def _check(src, dst, tb, cb, d, path, N):
    want, wst = kv_commit.commit_tree_kv(src, dst, tb, cb, d, path, N)
    got, gst = _run(src, dst, tb, cb, d, path)
    assert np.array_equal(gst, wst)
    assert np.array_equal(got, want)
    return wst


@pytest.mark.parametrize("rb", [16, 2048, 4112])
def test_in_place_after_the_root(rb):
    note(f"commit in place rb={rb}")
    B = 40
    N, d, path = _paths(B, seed=rb)
    G, S = 3, 90
    rng = np.random.default_rng(rb)
    src = rng.integers(0, 256, size=(G, B, S, rb), dtype=np.uint8)
    tb = rng.integers(0, S - N, size=B).astype(np.int32)
    st = _check(src, None, tb, tb + 1, d, path, N)
    assert (st == 0).all() and d.max() >= 3


def test_in_place_before_the_tree_and_into_a_separate_buffer():
    note("commit in place before the tree / out of place")
    B, G, S, rb = 48, 2, 100, 64
    N, d, path = _paths(B, seed=3)
    rng = np.random.default_rng(3)
    src = rng.integers(0, 256, size=(G, B, S, rb), dtype=np.uint8)
    tb = rng.integers(10, S - N, size=B).astype(np.int32)
    cb = (tb - rng.integers(0, 10, size=B)).astype(np.int32)
    assert (_check(src, None, tb, cb, d, path, N) == 0).all()
    dst = rng.integers(0, 256, size=src.shape, dtype=np.uint8)
    cb2 = rng.integers(0, S - N, size=B).astype(np.int32)
    assert (_check(src, dst, tb, cb2, d, path, N) == 0).all()


def test_deep_chain_paths_span_many_chunks():
    # a chain-shaped tree: the accepted path can hold hundreds of nodes, so one
    # request's copy runs over several chunks, rows split across chunk edges
    note("commit deep chains")
    B, N, G, S, rb = 6, 700, 2, 1600, 48
    rng = np.random.default_rng(8)
    d = np.array([0, 1, 699, 350, 698, 5], dtype=np.int32)
    path = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        nodes = np.sort(rng.choice(np.arange(1, N), size=d[b], replace=False))
        path[b, :d[b]] = nodes
    path[2, :699] = np.arange(1, 700)
    src = rng.integers(0, 256, size=(G, B, S, rb), dtype=np.uint8)
    tb = np.array([0, 5, 100, 800, 10, 40], dtype=np.int32)
    cb = tb + np.array([1, 1, 1, 0, -9, 1], dtype=np.int32)
    assert (_check(src, None, tb, cb, d, path, N) == 0).all()


def test_status_codes_leave_requests_untouched():
    note("commit status codes")
    G, B, S, rb, N = 2, 8, 40, 32, 6
    rng = np.random.default_rng(7)
    src = rng.integers(0, 256, size=(G, B, S, rb), dtype=np.uint8)
    path = np.full((B, N), -1, dtype=np.int32)
    path[:, :3] = [1, 2, 4]
    d = np.full(B, 3, dtype=np.int32)
    tb = np.full(B, 10, dtype=np.int32)
    cb = np.full(B, 11, dtype=np.int32)
    tb[1], cb[1] = 36, 30
    cb[2] = 38
    d[3] = 6
    path[4, :3] = [1, 1, 2]
    path[5, :3] = [0, 2, 3]
    cb[6] = 12
    d[7] = -1
    st = _check(src, None, tb, cb, d, path, N)
    assert st.tolist() == [0, 1, 1, 2, 2, 2, 3, 2]


def test_commit_after_tree_verification_at_full_size():
    # the tree workload's own accepted paths (B=64, N=33) on a cache shaped like
    # a 36-layer target with 8 KV heads of 128 bf16 values (2 KB rows)
    note("commit full size")
    w = workloads.make_workload("tree_b64_n33_qwen3")
    g = sv.spec_verify_tree(torch.from_numpy(w.target.view(np.int16)).view(torch.bfloat16).to(dev()),
                            ints_to_dev(w.node_tokens), ints_to_dev(w.parents))
    o = oracle.verify_tree(w.target, w.node_tokens, w.parents)
    d = g["accept_len"].cpu().numpy()
    path = g["path"].cpu().numpy()
    assert np.array_equal(d, o["accept_len"]) and np.array_equal(path, o["path"])
    G, B, S, rb = 72, w.B, 64, 2048
    rng = np.random.default_rng(5)
    src = rng.integers(0, 256, size=(G, B, S, rb), dtype=np.uint8)
    tb = rng.integers(0, S - w.N, size=B).astype(np.int32)
    assert (_check(src, None, tb, tb + 1, d, path, w.N) == 0).all()
