"""The entry points inside a captured HIP graph: every launch they make is a
kernel (their control words are cleared by kernels, never by memsets), so a
captured verification step replays correctly.  Each replay, with eager work and
synchronisation between replays and the inputs rewritten in place, must equal
an eager call on the same inputs."""

import numpy as np
import torch

import draft_token_verification_04_amd as sv
import workloads
from gpu_helpers import dev, f32_to_dev, ints_to_dev, logits_to_dev, note
import pytest

pytestmark = pytest.mark.gpu


def _np(d):
    return {k: v.cpu().numpy() for k, v in d.items()}


def test_verification_step_replays_inside_a_graph():
    note("graph capture and replay")
    w3 = workloads.make_sample(32, 7, 20000, "bf16", 0.8, spikes=10, noise_sigma=1.0, seed=61)
    w3b = workloads.make_sample(32, 7, 20000, "bf16", 0.8, spikes=10, noise_sigma=2.0, seed=62)
    w4 = workloads.make_greedy(32, 7, 20000, "bf16", seed=63)
    w4b = workloads.make_greedy(32, 7, 20000, "bf16", p_match=0.5, seed=64)
    w5 = workloads.make_tree(16, 20000, "bf16", seed=65)
    w5b = workloads.make_tree(16, 20000, "bf16", p_match=0.4, seed=66)
    assert w5b.N == w5.N
    # static inputs, rewritten in place between replays
    s_t, s_d = logits_to_dev(w3.target), logits_to_dev(w3.draft)
    s_x, s_ua, s_us = ints_to_dev(w3.draft_tokens), f32_to_dev(w3.u_accept), f32_to_dev(w3.u_sample)
    g_t, g_x = logits_to_dev(w4.target), ints_to_dev(w4.draft_tokens)
    t_t, t_tok, t_par = logits_to_dev(w5.target), ints_to_dev(w5.node_tokens), ints_to_dev(w5.parents)

    def load(a, b, c):
        s_t.copy_(logits_to_dev(a.target))
        s_d.copy_(logits_to_dev(a.draft))
        s_x.copy_(ints_to_dev(a.draft_tokens))
        s_ua.copy_(f32_to_dev(a.u_accept))
        s_us.copy_(f32_to_dev(a.u_sample))
        g_t.copy_(logits_to_dev(b.target))
        g_x.copy_(ints_to_dev(b.draft_tokens))
        t_t.copy_(logits_to_dev(c.target))
        t_tok.copy_(ints_to_dev(c.node_tokens))
        t_par.copy_(ints_to_dev(c.parents))

    def step():
        return dict(
            sample=sv.spec_verify_sample(s_t, s_d, s_x, s_ua, s_us, w3.T),
            sample_skip=sv.spec_verify_sample(s_t, s_d, s_x, s_ua, s_us, w3.T, lse=False),
            greedy=sv.spec_verify_greedy(g_t, g_x),
            tree=sv.spec_verify_tree(t_t, t_tok, t_par))

    def eager():
        out = step()
        torch.cuda.synchronize()
        return {k: _np(v) for k, v in out.items()}

    want = {}
    for name, sets in (("a", (w3, w4, w5)), ("b", (w3b, w4b, w5b))):
        load(*sets)
        want[name] = eager()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = step()
    for rep, name in enumerate(("a", "b", "a", "b")):
        load(*((w3, w4, w5) if name == "a" else (w3b, w4b, w5b)))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: _np(v) for k, v in captured.items()}
        for call, outs in want[name].items():
            for key, ref in outs.items():
                assert np.array_equal(got[call][key], ref), (rep, call, key)
        eager()  # eager work between replays


def test_concurrent_calls_on_two_streams():
    # separate workspaces make calls on different streams independent, including
    # the row-skipping passes whose control words live in the workspace
    note("two streams")
    ws = [workloads.make_greedy(48, 7, 30000, "bf16", seed=71 + i) for i in range(2)]
    wt = [workloads.make_tree(24, 30000, "bf16", seed=73 + i) for i in range(2)]
    ins = [(logits_to_dev(w.target), ints_to_dev(w.draft_tokens)) for w in ws]
    tins = [(logits_to_dev(w.target), ints_to_dev(w.node_tokens), ints_to_dev(w.parents)) for w in wt]
    want = []
    for (t, x), (tt, tok, par) in zip(ins, tins):
        a, b = sv.spec_verify_greedy(t, x), sv.spec_verify_tree(tt, tok, par)
        torch.cuda.synchronize()
        want.append((_np(a), _np(b)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(5):
        outs = []
        for s, (t, x), (tt, tok, par) in zip(streams, ins, tins):
            with torch.cuda.stream(s):
                outs.append((sv.spec_verify_greedy(t, x), sv.spec_verify_tree(tt, tok, par)))
        torch.cuda.synchronize()
        for (a, b), (wa, wb) in zip(outs, want):
            for k in wa:
                assert np.array_equal(_np(a)[k], wa[k]), (rep, k)
            for k in wb:
                assert np.array_equal(_np(b)[k], wb[k]), (rep, k)


def test_fused_projection_forms_replay_inside_a_graph():
    # the three LM-head entry points (the sampling form makes eight launches,
    # two of them projections) captured once and replayed on rewritten inputs
    note("graph capture of the fused LM-head forms")
    B, K, D, V = 16, 7, 256, 3000
    sa = [workloads.make_sample_lmhead(B, K, D, V, exact=True, dtype="bf16", T=0.8, seed=81 + i) for i in range(2)]
    ga = [workloads.make_greedy_lmhead(B, K, D, V, exact=True, seed=83 + i) for i in range(2)]
    ta = [workloads.make_tree_lmhead(8, D, V, exact=True, seed=85 + i) for i in range(2)]
    assert ta[0].N == ta[1].N
    bf = logits_to_dev
    W_s, W_g, W_t = bf(sa[0].lm_head), bf(ga[0].lm_head), bf(ta[0].lm_head)
    h_s, d_s = bf(sa[0].hidden), bf(sa[0].draft)
    x_s, ua, us = ints_to_dev(sa[0].draft_tokens), f32_to_dev(sa[0].u_accept), f32_to_dev(sa[0].u_sample)
    h_g, x_g = bf(ga[0].hidden), ints_to_dev(ga[0].draft_tokens)
    h_t, tok, par = bf(ta[0].hidden), ints_to_dev(ta[0].node_tokens), ints_to_dev(ta[0].parents)

    def load(i):
        # every operand of set i, the projections included
        W_s.copy_(bf(sa[i].lm_head))
        W_g.copy_(bf(ga[i].lm_head))
        W_t.copy_(bf(ta[i].lm_head))
        h_s.copy_(bf(sa[i].hidden))
        d_s.copy_(bf(sa[i].draft))
        x_s.copy_(ints_to_dev(sa[i].draft_tokens))
        ua.copy_(f32_to_dev(sa[i].u_accept))
        us.copy_(f32_to_dev(sa[i].u_sample))
        h_g.copy_(bf(ga[i].hidden))
        x_g.copy_(ints_to_dev(ga[i].draft_tokens))
        h_t.copy_(bf(ta[i].hidden))
        tok.copy_(ints_to_dev(ta[i].node_tokens))
        par.copy_(ints_to_dev(ta[i].parents))

    def step():
        return dict(sample=sv.spec_verify_sample_lmhead(h_s, W_s, d_s, x_s, ua, us, 0.8),
                    greedy=sv.spec_verify_greedy_lmhead(h_g, W_g, x_g),
                    tree=sv.spec_verify_tree_lmhead(h_t, W_t, tok, par))

    def eager():
        out = step()
        torch.cuda.synchronize()
        return {k: _np(v) for k, v in out.items()}

    want = []
    for i in range(2):
        load(i)
        want.append(eager())
    # the sets accept different numbers of drafts, so a replay that kept old results would show
    assert any((w["sample"]["accept_len"] < K).any() for w in want)
    assert not np.array_equal(want[0]["greedy"]["accept_len"], want[1]["greedy"]["accept_len"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = step()
    for rep, i in enumerate((0, 1, 0, 1)):
        load(i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: _np(v) for k, v in captured.items()}
        for call, outs in want[i].items():
            for key, ref in outs.items():
                assert np.array_equal(got[call][key], ref), (rep, call, key)
        eager()


def test_noalloc_sampler_replays_inside_a_graph():
    """The no-allocation entry point is for callers under graph capture: with
    its outputs given, the captured call allocates nothing (its scratch is the
    library's own, looked up by the eager warm-up call).  Replays with the
    inputs rewritten, and eager calls of both sampler entry points between
    them, each equal the eager call."""
    note("graph capture of the no-allocation sampler")
    wa = workloads.make_sample(48, 7, 30000, "bf16", 0.7, spikes=10, noise_sigma=1.0, seed=71)
    wb = workloads.make_sample(48, 7, 30000, "bf16", 0.7, spikes=10, noise_sigma=2.5, seed=72)
    t, d = logits_to_dev(wa.target), logits_to_dev(wa.draft)
    x, ua, us = ints_to_dev(wa.draft_tokens), f32_to_dev(wa.u_accept), f32_to_dev(wa.u_sample)

    def load(w):
        t.copy_(logits_to_dev(w.target))
        d.copy_(logits_to_dev(w.draft))
        x.copy_(ints_to_dev(w.draft_tokens))
        ua.copy_(f32_to_dev(w.u_accept))
        us.copy_(f32_to_dev(w.u_sample))

    want = {}
    for name, w in (("a", wa), ("b", wb)):
        load(w)
        want[name] = _np(sv.spec_verify_sample(t, d, x, ua, us, w.T))
    B, K = wa.B, wa.K
    outs = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev()),
            "tokens": torch.empty((B, K + 1), dtype=torch.int32, device=dev()),
            "lse_target": torch.empty((B, K + 1), dtype=torch.float32, device=dev()),
            "lse_draft": torch.empty((B, K), dtype=torch.float32, device=dev()),
            "status": torch.empty(B, dtype=torch.int32, device=dev())}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sv.spec_verify_sample_noalloc(t, d, x, ua, us, wa.T, out=outs)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sv.spec_verify_sample_noalloc(t, d, x, ua, us, wa.T, out=outs)
    for rep, name in enumerate(("a", "b", "a", "b")):
        load(wa if name == "a" else wb)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _np(outs)
        for key, ref in want[name].items():
            assert np.array_equal(got[key], ref), (rep, key)
        # eager work between replays, the no-allocation call included
        e1 = _np(sv.spec_verify_sample_noalloc(t, d, x, ua, us, wa.T, lse=False))
        e2 = _np(sv.spec_verify_sample(t, d, x, ua, us, wa.T, lse=False))
        torch.cuda.synchronize()
        for key in e2:
            assert np.array_equal(e1[key], e2[key]), (rep, key)
