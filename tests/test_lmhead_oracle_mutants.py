"""The LM-head oracle's pins have teeth: each test plants one plausible mistake
in oracle/lmhead.py (by monkeypatching a single function) and checks that a pin
in tests/test_lmhead_oracle.py then fails (CPU only)."""

import numpy as np
import pytest

import test_lmhead_oracle as pins
from oracle import lmhead


def _fails(pin, *args):
    with pytest.raises(AssertionError):
        pin(*args)


def test_vocabulary_rows_off_by_one(monkeypatch):
    real = lmhead.logits
    monkeypatch.setattr(lmhead, "logits", lambda h, w: real(h, np.roll(w, 1, axis=0)))
    _fails(pins.test_logits_equal_integer_arithmetic)


def test_positions_of_a_request_swapped(monkeypatch):
    real = lmhead.logits
    monkeypatch.setattr(lmhead, "logits", lambda h, w: real(np.ascontiguousarray(h[:, ::-1]), w))
    _fails(pins.test_logits_equal_integer_arithmetic)


def test_ties_to_the_highest_index(monkeypatch):
    real = lmhead.row_argmax

    def last_max(L, E):
        a, certain = real(L, E)
        flipped = L.shape[-1] - 1 - np.argmax(L[..., ::-1], axis=-1)
        return flipped, certain

    monkeypatch.setattr(lmhead, "row_argmax", last_max)
    _fails(pins.test_exact_recipe_has_ties_resolved_to_the_lowest_index)


def test_draft_compared_with_the_next_row(monkeypatch):
    real = lmhead.greedy_chain

    def shifted(a, drafts, V):
        return real(np.concatenate([a[:, 1:], a[:, -1:]], axis=1), drafts, V)

    monkeypatch.setattr(lmhead, "greedy_chain", shifted)
    _fails(pins.test_exact_recipe_matches_the_c_oracle_chain)


def test_tree_ignores_the_parent_acceptance(monkeypatch):
    def walk(a, node_tokens, parents, V):
        # every node whose token matches its parent's row is taken as accepted
        B, N = a.shape
        out = dict(accept_len=np.zeros(B, np.int32), path=np.full((B, N), -1, np.int32),
                   tokens=np.full((B, N), -1, np.int32), status=np.zeros(B, np.int32))
        for b in range(B):
            par = parents[b]
            if par[0] != -1 or any(not (0 <= par[j] < j) for j in range(1, N)):
                out["accept_len"][b], out["status"][b] = -1, 2
                continue
            depth = np.zeros(N, np.int64)
            ok = np.zeros(N, bool)
            ok[0] = True
            for j in range(1, N):
                depth[j] = depth[par[j]] + 1
                ok[j] = node_tokens[b, j] == a[b, par[j]]
            best = max((j for j in range(N) if ok[j]), key=lambda j: (depth[j], -j))
            path = []
            j = best
            while j != 0:
                path.append(j)
                j = par[j]
            path.reverse()
            d = len(path)
            out["accept_len"][b] = d
            out["path"][b, :d] = path
            out["tokens"][b, :d] = node_tokens[b, path]
            out["tokens"][b, d] = a[b, best]
            if ((node_tokens[b, 1:] < 0) | (node_tokens[b, 1:] >= V)).any():
                out["status"][b] = 1
        return out

    monkeypatch.setattr(lmhead, "tree_walk", walk)
    _fails(pins.test_tree_walk_matches_the_c_oracle)


def test_accumulation_bound_too_tight(monkeypatch):
    real = lmhead.accumulation_bound
    monkeypatch.setattr(lmhead, "accumulation_bound", lambda h, w: real(h, w) * 0.4)
    _fails(pins.test_bound_is_nearly_attained_by_an_adversarial_sum)


def test_temperature_applied_twice(monkeypatch):
    real = lmhead.verify_sample
    monkeypatch.setattr(lmhead, "verify_sample",
                        lambda h, w, d, x, ua, us, T, lib=None: real(h, w, d, x, ua, us, T * T, lib=lib))
    _fails(pins.test_sampling_on_the_projection_is_sampling_on_its_logits, "bf16")
