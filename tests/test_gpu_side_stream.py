"""Calls made with ``stream=`` set to a stream other than the current one
(needs an MI355X).

The binding allocates each call's workspace and outputs on the current stream
while the call's kernels run on the given stream.  Right after each call the
current stream allocates blocks of the same sizes and fills them with garbage;
if the binding let the caching allocator hand the call's blocks out again
before its kernels finished, the kernels would read garbage control words or
their outputs would be overwritten.  Every output is checked against the
oracle after both streams are drained.
"""

import numpy as np
import pytest
import torch

import draft_token_verification_04_amd as sv
import oracle
import workloads
from gpu_helpers import (check_exact, check_sample, f32_to_dev, ints_to_dev, logits_to_dev, note,
                         oracle_sample)

pytestmark = pytest.mark.gpu


def _scribble(nbytes_list, rounds=4):
    """Allocate and overwrite blocks of the given sizes on the current stream."""
    keep = []
    for _ in range(rounds):
        for n in nbytes_list:
            t = torch.empty(max(int(n), 256), dtype=torch.uint8, device="cuda")
            t.fill_(0xA5)
            keep.append(t)
    return keep


def _on_side(fn, *args, **kw):
    side = torch.cuda.Stream()
    cur = torch.cuda.current_stream()
    side.wait_stream(cur)  # the inputs were written on the current stream
    out = fn(*args, stream=side, **kw)
    sizes = [t.numel() * t.element_size() for t in out.values()] if isinstance(out, dict) else []
    junk = _scribble(sizes + [64 << 20])
    torch.cuda.synchronize()
    del junk
    return out


def test_greedy_and_tree_on_a_side_stream():
    note("side stream: greedy B=256 K=7 V=151936, tree B=64 N=33")
    w = workloads.make_workload("greedy_b512_k7_qwen3", B=256)
    t, x = logits_to_dev(w.target), ints_to_dev(w.draft_tokens)
    g = _on_side(sv.spec_verify_greedy, t, x)
    check_exact({k: v.cpu().numpy() for k, v in g.items()}, oracle.verify_greedy(w.target, w.draft_tokens),
                ("accept_len", "tokens", "status"))
    w5 = workloads.make_workload("tree_b64_n33_qwen3")
    g = _on_side(sv.spec_verify_tree, logits_to_dev(w5.target), ints_to_dev(w5.node_tokens),
                 ints_to_dev(w5.parents))
    check_exact({k: v.cpu().numpy() for k, v in g.items()},
                oracle.verify_tree(w5.target, w5.node_tokens, w5.parents),
                ("accept_len", "path", "tokens", "status"))


@pytest.mark.parametrize("lse", [True, False], ids=["full", "skip"])
def test_sample_on_a_side_stream(lse):
    note(f"side stream: sample B=32 K=7 V=151936 lse={lse}")
    w = workloads.make_workload("sample_b32_k7_qwen3")
    g = _on_side(sv.spec_verify_sample, logits_to_dev(w.target), logits_to_dev(w.draft),
                 ints_to_dev(w.draft_tokens), f32_to_dev(w.u_accept), f32_to_dev(w.u_sample), w.T, lse=lse)
    ncmp, nflag, _ = check_sample(w, {k: v.cpu().numpy() for k, v in g.items()}, oracle_sample(w))
    assert ncmp >= 1


def test_ngram_on_a_side_stream():
    note("side stream: ngram B=64")
    rng = np.random.default_rng(3)
    B, L, n = 64, 8192, 3
    ctx = rng.integers(0, 50, (B, L)).astype(np.int32)
    lengths = rng.integers(n + 1, L + 1, B).astype(np.int32)
    q = rng.integers(0, 50, (B, n)).astype(np.int32)
    g = _on_side(sv.spec_ngram_candidates, ints_to_dev(ctx), ints_to_dev(lengths), ints_to_dev(q), 16)
    from oracle import ngram

    o = ngram.ngram_candidates(ctx, lengths, q, 16)
    assert np.array_equal(g["count"].cpu().numpy(), o["count"])
    assert np.array_equal(g["positions"].cpu().numpy(), o["positions"])
