"""Oracle: greedy acceptance of a verified draft tree.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring).

What is computed, and which passage it follows
-----------------------------------------------
"The Microsecond Verdict: Validating a DDTree Kernel Fix Under Time Pressure", sections "The
Crash That Demanded a Fix" and "What Was Learned": after verification, the tree-accept step
performs greedy acceptance -- the longest prefix on which the drafter and the target agree --
by walking the accepted path from the root through the tree's child and sibling links and
recording it in a path buffer; the walk is capped at ``q_len`` nodes, since a valid accepted
path never holds more nodes than the tree.  "Race Conditions, Buffer Aliasing, and the
Architecture of a Native DDTree Inference Engine", section "The Cache Compaction Problem", says
what the path is for: its rows are the ones kept in the cache.

Readings (the pages describe the walk, not its exact rule):

* Node ``i``'s draft token ``draft[i]`` is the token the drafter proposed at that position; the
  root (node 0) holds the last committed token and is always accepted.
* ``target[i]`` is the target model's greedy token after the context ending at node ``i`` (the
  argmax of the verify forward's logits at row ``P + i``).
* From the current node ``c`` the walk moves to a child ``j`` (``parents[j] == c``) whose draft
  token equals ``target[c]``.  Children are examined in increasing node index -- the order in
  which the builder appends them, which is the first-child / next-sibling order -- and the first
  match is taken.  A drafter proposes distinct tokens among siblings, so at most one child
  matches on real trees; the order only decides degenerate inputs.
* The walk stops when no child matches.  Its results are the path (node indices, strictly
  increasing from 0), its length, and ``target`` at the last accepted node: the target's token
  for the position right after the accepted tokens.
* ``parents`` must be a valid tree (``parents[0] == -1``, ``0 <= parents[i] < i``); anything else
  is rejected here, as in the verify oracle.
"""
from __future__ import annotations

import numpy as np


def validate_parents(parents: np.ndarray) -> None:
    parents = np.asarray(parents, dtype=np.int64)
    if len(parents) < 1 or parents[0] != -1:
        raise ValueError("parents[0] must be -1")
    for i in range(1, len(parents)):
        if not 0 <= parents[i] < i:
            raise ValueError(f"parents[{i}]={parents[i]} is not an earlier node")


def children(parents: np.ndarray, node: int) -> list[int]:
    """The children of ``node`` in increasing index (the builder's append order)."""
    return [j for j in range(len(parents)) if int(parents[j]) == node]


def tree_accept(parents: np.ndarray, draft: np.ndarray, target: np.ndarray):
    """Greedy acceptance of one stream's tree.  Returns ``(path, next_token)``.

    ``path`` lists the accepted node indices starting with the root; ``next_token`` is
    ``target`` at the last of them.  The walk is capped at ``len(parents)`` nodes.
    """
    validate_parents(parents)
    q = len(parents)
    path = [0]
    cur = 0
    while len(path) < q:
        nxt = None
        for j in children(parents, cur):
            if int(draft[j]) == int(target[cur]):
                nxt = j
                break
        if nxt is None:
            break
        path.append(nxt)
        cur = nxt
    return np.array(path, dtype=np.int32), int(target[cur])


def tree_accept_streams(parents: np.ndarray, draft: np.ndarray, target: np.ndarray, keep_stride: int | None = None):
    """Greedy acceptance for every stream: ``(keep [S, keep_stride] padded with -1, n_keep [S],
    next_token [S])``."""
    parents = np.asarray(parents)
    s_count, q = parents.shape
    stride = q if keep_stride is None else keep_stride
    keep = np.full((s_count, stride), -1, dtype=np.int32)
    n_keep = np.zeros(s_count, dtype=np.int32)
    nxt = np.zeros(s_count, dtype=np.int32)
    for s in range(s_count):
        path, t = tree_accept(parents[s], draft[s], target[s])
        keep[s, : len(path)] = path
        n_keep[s] = len(path)
        nxt[s] = t
    return keep, n_keep, nxt
