"""Oracle: best-first construction of the draft tree from the drafter's per-position top-k.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring).

What is computed, and which passage it follows
-----------------------------------------------
"Building the Foundation: Architecting a Native CUDA DDTree Inference Engine", sections "Tie-
Breaking and Numerical Precision", "The Single-Threaded Heap Design" and "Assumptions Underlying
the Design": the tree builder expands a best-first heap of candidate nodes keyed by cumulative
log-weight; it emits the parents, node tokens, depths and log-weights (plus a visibility matrix
and the child/sibling "retrieve" links); the budget is at most 64 and the depth at most 15; ties
in the log-weight are broken by insertion order; a candidate's next sibling gets the log-weight
``logw - lp[depth-1, rank] + lp[depth-1, rank+1]`` evaluated in float32 in exactly that order;
and the heap can run empty before the budget is reached only when top-k is 1 and the chain is
shorter than the budget.

Readings (the pages give the heap's keys and one expression, not the whole procedure):

* Inputs per request: for every draft position ``d < D`` the drafter's top ``K`` tokens
  ``tok[d, :]`` with their log-probabilities ``lp[d, :]`` sorted in decreasing order, and the
  root token (the last committed token).
* Node 0 is the root (depth 0, log-weight 0).  A node at depth ``d >= 1`` with rank ``r`` carries
  token ``tok[d-1, r]``.
* The heap starts with the root's first child: depth 1, rank 0, log-weight ``lp[0, 0]``.
  Popping a candidate (highest log-weight; equal log-weights in insertion order) appends it as
  the next node and pushes, in this order, its next sibling (same parent, rank + 1, when
  rank + 1 < K; log-weight by the pages' expression) and its first child (depth + 1, rank 0, when
  depth < D; log-weight ``logw + lp[depth, 0]``).  All log-weights are float32 sums.
* ``budget`` counts the nodes after the root; the tree has ``min(budget, available) + 1``
  nodes and at most 64 in all (budget <= 63), the verify attention's limit.
* Retrieve links: ``first_child[i]`` is the first node appended with parent ``i`` and
  ``next_sibling[i]`` the next node appended with the same parent (-1 when none).  Siblings are
  appended in rank order, since rank r + 1 only enters the heap when rank r leaves it.
* Visibility: node ``i`` sees node ``j`` iff ``j`` is ``i`` or an ancestor of ``i`` (a 64-bit mask
  per node, bit ``j``).
"""
from __future__ import annotations

import heapq

import numpy as np


def tree_build(lp: np.ndarray, tok: np.ndarray, budget: int, root_token: int = -1) -> dict:
    """Best-first tree for one request.  ``lp``, ``tok``: ``[D, K]``.  Returns a dict of arrays
    of length ``n_nodes``: parents, tokens, depths, ranks, logw (float32), first_child,
    next_sibling, anc (uint64 masks)."""
    lp = np.asarray(lp, dtype=np.float32)
    tok = np.asarray(tok)
    d_max, k = lp.shape
    if not 1 <= budget <= 63:
        raise ValueError("budget must be in [1, 63]")
    heap = []
    ins = 0
    heapq.heappush(heap, (-lp[0, 0], ins, 1, 0, 0, lp[0, 0]))  # (-logw, insertion id, depth, rank, parent, logw)
    ins += 1
    parents, tokens, depths, ranks, logw = [-1], [root_token], [0], [0], [np.float32(0.0)]
    while len(parents) < budget + 1 and heap:
        _, _, d, r, p, w = heapq.heappop(heap)
        idx = len(parents)
        parents.append(p)
        tokens.append(int(tok[d - 1, r]))
        depths.append(d)
        ranks.append(r)
        logw.append(w)
        if r + 1 < k:
            ws = np.float32(np.float32(w - lp[d - 1, r]) + lp[d - 1, r + 1])
            heapq.heappush(heap, (-ws, ins, d, r + 1, p, ws))
            ins += 1
        if d < d_max:
            wc = np.float32(w + lp[d, 0])
            heapq.heappush(heap, (-wc, ins, d + 1, 0, idx, wc))
            ins += 1
    n = len(parents)
    first_child = np.full(n, -1, np.int32)
    next_sibling = np.full(n, -1, np.int32)
    last = {}
    for i in range(1, n):
        p = parents[i]
        if p in last:
            next_sibling[last[p]] = i
        else:
            first_child[p] = i
        last[p] = i
    anc = np.zeros(n, np.uint64)
    for i in range(n):
        m = np.uint64(1) << np.uint64(i)
        if i > 0:
            m |= anc[parents[i]]
        anc[i] = m
    return {"parents": np.array(parents, np.int32), "tokens": np.array(tokens, np.int32),
            "depths": np.array(depths, np.int32), "ranks": np.array(ranks, np.int32),
            "logw": np.array(logw, np.float32), "first_child": first_child, "next_sibling": next_sibling,
            "anc": anc, "n_nodes": n}
