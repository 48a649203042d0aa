"""Pins for the best-first tree-builder oracle (CPU only).

* Top-B: log-weights only decrease along child and sibling edges (log-probabilities are <= 0
  and sorted in decreasing order), so the best-first tree with budget B is the B highest-weight
  nodes of the whole K-ary product tree of depth D.  That set is found here by enumerating every
  node with fp64 path sums, with no heap.
* The log-weights are the fp64 path sums up to fp32 rounding, nodes come out in non-increasing
  order, the structure (parents, depths, tokens, rank order of siblings, retrieve links) is
  consistent, and the visibility masks equal the verify oracle's ancestor-or-self relation.
* The pages' edge cases: the heap running empty with top-1, and ties taken in insertion order.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth
from oracle import build as ob


def enumerate_top(lp, budget):
    d_max, k = lp.shape
    nodes = []
    for d in range(1, d_max + 1):
        for ranks in itertools.product(range(k), repeat=d):
            w = float(sum(float(lp[i, r]) for i, r in enumerate(ranks)))
            nodes.append((w, ranks))
    nodes.sort(key=lambda x: -x[0])
    return nodes, {r for _, r in nodes[:budget]}


def rank_paths(t):
    paths = {0: ()}
    for i in range(1, t["n_nodes"]):
        paths[i] = paths[int(t["parents"][i])] + (int(t["ranks"][i]),)
    return paths


@pytest.mark.parametrize("d_max,k", [(1, 5), (2, 3), (3, 3), (4, 2), (5, 3), (3, 6)])
def test_top_b_set(d_max, k):
    checked = 0
    for stream in range(30):
        lp, tok = synth.drafter_topk(3, stream, d_max, k, temperature=1.5)
        total = sum(k ** d for d in range(1, d_max + 1))
        for budget in sorted({1, 2, 5, min(total, 20), min(total, 63)}):
            nodes, best = enumerate_top(lp, budget)
            if budget < len(nodes) and nodes[budget - 1][0] - nodes[budget][0] < 1e-4:
                continue  # a near tie at the cut: fp32 rounding may legitimately swap it
            t = ob.tree_build(lp, tok, budget)
            assert t["n_nodes"] == min(budget, total) + 1
            assert set(list(rank_paths(t).values())[1:]) == best
            checked += 1
    assert checked > 50


def test_weights_order_structure_and_links():
    for stream in range(40):
        d_max, k, budget = 6, 4, 40
        lp, tok = synth.drafter_topk(5, stream, d_max, k)
        t = ob.tree_build(lp, tok, budget, root_token=777)
        n = t["n_nodes"]
        paths = rank_paths(t)
        for i in range(1, n):
            exact = sum(float(lp[j, r]) for j, r in enumerate(paths[i]))
            assert abs(float(t["logw"][i]) - exact) < 1e-5 * max(1.0, abs(exact))
            p = int(t["parents"][i])
            assert 0 <= p < i and t["depths"][i] == t["depths"][p] + 1
            assert t["tokens"][i] == tok[t["depths"][i] - 1, t["ranks"][i]]
        assert t["tokens"][0] == 777 and t["parents"][0] == -1
        assert np.all(np.diff(t["logw"][1:].astype(np.float64)) <= 1e-6)  # best first
        for i in range(n):  # siblings appended in rank order 0, 1, 2, ...
            kids = [j for j in range(n) if t["parents"][j] == i]
            assert [int(t["ranks"][j]) for j in kids] == list(range(len(kids)))
            assert t["first_child"][i] == (kids[0] if kids else -1)
            for a, b in zip(kids, kids[1:] + [-1]):
                assert t["next_sibling"][a] == b
        anc = oracle.ancestor_or_self(t["parents"])
        for i in range(n):
            bits = [(int(t["anc"][i]) >> j) & 1 for j in range(n)]
            assert bits == anc[i].astype(int).tolist()


def test_heap_empties_early_with_top1():
    lp, tok = synth.drafter_topk(7, 0, 5, 1)
    t = ob.tree_build(lp, tok, 20)
    assert t["n_nodes"] == 6 and t["parents"].tolist() == [-1, 0, 1, 2, 3, 4]


def test_ties_go_in_insertion_order():
    # After the first pop (depth 1, rank 0, w = -1) the heap gets the sibling (w = -2, inserted
    # first) and the child (w = -1 + -1 = -2): equal weights, so the sibling comes out first.
    lp = np.array([[-1.0, -2.0], [-1.0, -3.0]], np.float32)
    tok = np.array([[10, 11], [20, 21]], np.int32)
    t = ob.tree_build(lp, tok, 3)
    assert t["depths"].tolist() == [0, 1, 1, 2] and t["ranks"].tolist() == [0, 0, 1, 0]
    assert t["parents"].tolist() == [-1, 0, 0, 1]


def _rne_f32(x):
    """Round an exact rational to the nearest float32, ties to even (normal range only), from
    the definition: the float32 grid near |x| has spacing 2^(e - 23) with 2^e <= |x| < 2^(e+1)."""
    from fractions import Fraction
    if x == 0:
        return Fraction(0)
    e = abs(x.numerator).bit_length() - abs(x.denominator).bit_length()
    while Fraction(2) ** e > abs(x):
        e -= 1
    while Fraction(2) ** (e + 1) <= abs(x):
        e += 1
    ulp = Fraction(2) ** (e - 23)
    q = x / ulp
    n = q.numerator // q.denominator
    rest = q - n
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n * ulp


def test_sibling_weight_evaluated_in_the_pages_order():
    """The pages fix one expression for bit parity: a sibling's weight is
    ``logw - lp[d-1, r] + lp[d-1, r+1]`` in float32, left to right ("Building the Foundation",
    sections "Tie-Breaking and Numerical Precision" and "Assumptions Underlying the Design",
    Assumption 4).  With lp = [[-0.61, -1.61], [-0.13, -2.38]] the depth-2, rank-1 sibling of
    node 1 has, by exact arithmetic with one float32 rounding per operation:
      w = rn(-0.61 + -0.13) = -0.74 (0xbf3d70a4)
      rn(rn(w - -0.13) + -2.38) = 0xc03f5c2a   (the pages' order)
      rn(w + rn(-2.38 - -0.13)) = 0xc03f5c29   (reassociated: one ulp apart)
    The oracle must produce the first."""
    from fractions import Fraction

    lp = np.array([[-0.61, -1.61], [-0.13, -2.38]], np.float32)
    tok = np.array([[10, 11], [20, 21]], np.int32)
    x = {name: Fraction(float(v)) for name, v in (("a0", lp[0, 0]), ("b0", lp[1, 0]), ("b1", lp[1, 1]))}
    w = _rne_f32(x["a0"] + x["b0"])
    pages = _rne_f32(_rne_f32(w - x["b0"]) + x["b1"])
    reassoc = _rne_f32(w + _rne_f32(x["b1"] - x["b0"]))
    bits = lambda v: int(np.array([float(v)], np.float32).view(np.uint32)[0])  # exact: v is on the grid
    assert bits(w) == 0xBF3D70A4
    assert bits(pages) == 0xC03F5C2A and bits(reassoc) == 0xC03F5C29
    t = ob.tree_build(lp, tok, 6)  # the whole 2 + 4 node product tree
    idx = [i for i in range(t["n_nodes"]) if t["depths"][i] == 2 and t["ranks"][i] == 1 and t["parents"][i] == 1]
    assert len(idx) == 1
    assert int(t["logw"][idx[0]:idx[0] + 1].view(np.uint32)[0]) == 0xC03F5C2A


def test_signed_zero_weights_tie():
    """-0.0 and +0.0 are equal weights, so they pop in insertion order.  With
    lp = [[-0, +0, -0], [-0, +0, -0]] (IEEE sums, round to nearest):
      pop 1: (depth 1, rank 0) w = -0; offers its sibling (-0 - -0) + +0 = +0 (insertion 1)
             and its child -0 + -0 = -0 (insertion 2);
      pop 2: insertion 1 (w = +0); offers (+0 - +0) + -0 = +0 and +0 + -0 = +0 (insertions 3, 4);
      pop 3: insertion 2, the depth-2 child of node 1, weight -0 -- ahead of the later +0
             candidates although an order that puts +0 above -0 would take insertion 3."""
    lp = np.array([[-0.0, 0.0, -0.0], [-0.0, 0.0, -0.0]], np.float32)
    tok = np.arange(6, dtype=np.int32).reshape(2, 3)
    t = ob.tree_build(lp, tok, 3)
    assert t["parents"].tolist() == [-1, 0, 0, 1]
    assert t["depths"].tolist() == [0, 1, 1, 2] and t["ranks"].tolist() == [0, 0, 1, 0]
    assert np.signbit(t["logw"]).tolist() == [False, True, False, True]


def test_rejects_budget_out_of_range():
    lp, tok = synth.drafter_topk(1, 0, 3, 2)
    for b in (0, 64):
        with pytest.raises(ValueError):
            ob.tree_build(lp, tok, b)


def test_pins_catch_planted_mistakes(monkeypatch):
    import heapq

    ORIG = ob.tree_build

    def variant(wrong_row=False, child_first=False, reassoc=False):
        def build(lp, tok, budget, root_token=-1):
            lp = np.asarray(lp, np.float32)
            d_max, k = lp.shape
            heap, ins = [(-lp[0, 0], 0, 1, 0, 0, lp[0, 0])], 1
            parents, depths, ranks, logw = [-1], [0], [0], [np.float32(0)]
            while len(parents) < budget + 1 and heap:
                _, _, d, r, p, w = heapq.heappop(heap)
                idx = len(parents)
                parents.append(p), depths.append(d), ranks.append(r), logw.append(w)
                pushes = []
                if r + 1 < k:
                    row = d if (wrong_row and d < d_max) else d - 1
                    if reassoc:  # w + (lp[r+1] - lp[r]): the same real number, another rounding
                        ws = np.float32(w + np.float32(lp[row, r + 1] - lp[d - 1, r]))
                    else:
                        ws = np.float32(np.float32(w - lp[d - 1, r]) + lp[row, r + 1])
                    pushes.append((-ws, d, r + 1, p, ws))
                if d < d_max:
                    wc = np.float32(w + lp[d, 0])
                    pushes.append((-wc, d + 1, 0, idx, wc))
                if child_first:
                    pushes.reverse()
                for key, dd, rr, pp, ww in pushes:
                    heapq.heappush(heap, (key, ins, dd, rr, pp, ww))
                    ins += 1
            out = ORIG(lp, tok, budget, root_token)
            out.update(parents=np.array(parents, np.int32), depths=np.array(depths, np.int32),
                       ranks=np.array(ranks, np.int32), logw=np.array(logw, np.float32), n_nodes=len(parents))
            return out
        return build

    for mutant, pin in ((variant(wrong_row=True), test_weights_order_structure_and_links),
                        (variant(child_first=True), test_ties_go_in_insertion_order),
                        (variant(reassoc=True), test_sibling_weight_evaluated_in_the_pages_order)):
        monkeypatch.setattr(ob, "tree_build", mutant)
        with pytest.raises(AssertionError):
            pin()
        monkeypatch.setattr(ob, "tree_build", ORIG)
