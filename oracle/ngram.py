"""CPU oracle for AdaPLD's lexical retrieval (test infrastructure: only the
tests, ``__graft_entry__``'s smoke check and ``bench.py``'s CPU baseline may use
it).

What is computed follows the AdaPLD page, section 3.2 ("lexical retrieval":
the most recent token c[i] is the query; the candidate set P holds every
position of the reuse context R where c[i] occurs and the ctxt tokens before it
match those before c[i]) and Algorithm 1 (LexicalRetrieval, then the main copy
path d_main = the tokens after the chosen position p*).

Readings taken (the section writes the window as a slice that can be read two
ways):
  * the match is an n-gram match of length n = ctxt ending at the anchor:
    R[p - k] == query[n - 1 - k] for k = 0 .. n-1, where query holds the last n
    tokens of the current prefix (query[n-1] = c[i]);
  * a candidate must have a continuation to copy, so p <= len - 2, and the
    window must fit, so p >= n - 1;
  * P is returned in ascending position order; the reranking by hidden state
    that picks p* is out of scope (it needs the target's hidden states), so the
    whole set (its size, and its first `cap` members) is the output.

Status per request: 0, or 1 if its length is outside [0, L] (then no
candidates).
"""

from __future__ import annotations

import numpy as np


def candidates_loop(context_row, length: int, query) -> list:
    """The definition written out with plain loops (small inputs)."""
    n = len(query)
    out = []
    for p in range(n - 1, length - 1):
        if all(int(context_row[p - k]) == int(query[n - 1 - k]) for k in range(n)):
            out.append(p)
    return out


def candidates(context_row, length: int, query) -> np.ndarray:
    """The same set, by comparing every window at once (sliding windows)."""
    n = len(query)
    if length - 1 <= n - 1:
        return np.zeros(0, dtype=np.int64)
    win = np.lib.stride_tricks.sliding_window_view(np.asarray(context_row[:length - 1]), n)
    hit = np.all(win == np.asarray(query)[None, :], axis=1)   # window starting at p - n + 1
    return np.flatnonzero(hit) + (n - 1)


def ngram_candidates(context, lengths, queries, cap: int):
    """context [B, L], lengths [B], queries [B, n] -> count [B], positions
    [B, cap] (ascending, -1 padded), status [B]."""
    B, L = context.shape
    count = np.zeros(B, dtype=np.int32)
    pos = np.full((B, cap), -1, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        ln = int(lengths[b])
        if ln < 0 or ln > L:
            status[b] = 1
            continue
        c = candidates(context[b], ln, queries[b])
        count[b] = len(c)
        k = min(cap, len(c))
        pos[b, :k] = c[:k]
    return dict(count=count, positions=pos, status=status)
