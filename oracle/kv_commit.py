"""CPU oracle for committing a verified draft tree's accepted path into the
target's KV cache (test infrastructure: only the tests, ``__graft_entry__``'s
smoke check and ``bench.py``'s CPU baseline may use it).

What is computed follows the AdaPLD page, Algorithm 1 (after VerifyAndAccept
returns the accepted tokens z, they are appended and the context is updated),
and section 3.3 (the draft tree is verified in one target pass): the target's
pass over the tree left one KV row per tree node; once the deepest accepted
node is known, the rows of the nodes on its path (depth 1 first) must sit in
consecutive cache slots after the context, so the next round attends to the
committed tokens in order.  The DLite notes, section 2.1, describe the same
step for the target's cache (it keeps its standard KV and causal verification).

The cache is a byte array [G][B][S][row_bytes]: G groups (e.g. one per layer
and per K/V), B requests, S slots, one row of row_bytes per token.  Node j of
request b was written at slot tree_base[b] + j; its accepted path
path_nodes[b][0..d-1] (d = accept_len[b]) goes to slots commit_base[b] + k.
All source rows are read as they were on entry (a snapshot), so the result is
that of a gather into a separate buffer followed by the writes.

Request status (the same codes as the library):
  0  committed (d = 0 commits nothing)
  1  a slot is outside [0, S)
  2  accept_len outside [0, N-1], or a path node outside [1, N) or not
     strictly increasing
  3  in place (src is dst) with commit_base in [tree_base + 2, tree_base + N),
     where a write could land on a source row of a later path node
A request with a non-zero status is left untouched.

Pins: tests/test_kv_commit_oracle.py checks a hand-worked example, the
snapshot property against a row-by-row loop on a separate buffer, the
untouched-rows invariant and each status code.
"""

from __future__ import annotations

import numpy as np


def request_status(tree_base: int, commit_base: int, d: int, path: np.ndarray, N: int, S: int,
                   in_place: bool) -> int:
    """Status code of one request (see the module docstring)."""
    if d < 0 or d > N - 1:
        return 2
    p = np.asarray(path[:d], dtype=np.int64)
    if d > 0 and (p.min() < 1 or p.max() >= N or np.any(np.diff(p) <= 0)):
        return 2
    if d == 0:
        return 0
    if tree_base < 0 or tree_base + p[-1] >= S or commit_base < 0 or commit_base + d > S:
        return 1
    if in_place and tree_base + 2 <= commit_base < tree_base + N:
        return 3
    return 0


def commit_tree_kv(src: np.ndarray, dst: np.ndarray | None, tree_base, commit_base, accept_len,
                   path_nodes, N: int):
    """Commit every request's accepted path.

    src: uint8 [G, B, S, row_bytes]; dst: the same shape, or None for in place
    (the result then replaces src's contents in a copy).  Returns (out, status)
    where out is the destination buffer after the call and status is int32 [B].
    """
    G, B, S, _ = src.shape
    in_place = dst is None
    snapshot = src.copy()
    out = src.copy() if in_place else dst.copy()
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        d = int(accept_len[b])
        st = request_status(int(tree_base[b]), int(commit_base[b]), d, path_nodes[b], N, S, in_place)
        status[b] = st
        if st != 0 or d == 0:
            continue
        slots = int(tree_base[b]) + np.asarray(path_nodes[b][:d], dtype=np.int64)
        rows = snapshot[:, b, slots, :]                       # [G, d, row_bytes]
        out[:, b, int(commit_base[b]):int(commit_base[b]) + d, :] = rows
    return out, status
