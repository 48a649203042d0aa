"""Pins for the greedy-acceptance oracle (CPU only).

Each pin checks ``oracle.tree_accept`` against something other than itself:

* a chain tree, where acceptance has a closed form (the leading run of agreements);
* the deepest-consistent-node formulation: a node is consistent when every edge on its root path
  has ``draft[child] == target[parent]``; with sibling tokens distinct the consistent nodes form
  one chain from the root, and the accepted path is that chain (computed upward from each node,
  not by the downward search);
* planted inputs from ``synth.accept_case``, built so that the accepted path is known;
* agreement with autoregressive greedy decoding, token for token: for a deterministic synthetic
  target model ``f`` the accepted draft tokens plus the next token equal the first tokens that
  ``f`` generates one at a time.  This is the invariant the pages' engine validated ("Building
  the Foundation: Architecting a Native CUDA DDTree Inference Engine", section "Conclusion":
  tree-greedy output equals autoregressive greedy output);
* the degenerate cases of the reading (no match, duplicate sibling tokens, a full-length chain).
"""
import itertools

import numpy as np
import pytest

import synth
from oracle import accept as acc


def root_path(parents, v):
    out = []
    while v >= 0:
        out.append(int(v))
        v = int(parents[v])
    return out[::-1]


def deepest_consistent(parents, draft, target):
    """Accepted path by the upward formulation (independent of the greedy loop)."""
    best = [0]
    for v in range(len(parents)):
        p = root_path(parents, v)
        if all(int(draft[p[k + 1]]) == int(target[p[k]]) for k in range(len(p) - 1)):
            if len(p) > len(best):
                best = p
    return best


def test_chain_closed_form():
    rng = np.random.default_rng(0)
    for q in (1, 2, 5, 17, 64):
        for _ in range(20):
            parents = np.arange(-1, q - 1, dtype=np.int32)
            draft = rng.integers(0, 3, size=q).astype(np.int32)
            target = rng.integers(0, 3, size=q).astype(np.int32)
            k = 0
            while k + 1 < q and draft[k + 1] == target[k]:
                k += 1
            path, nxt = acc.tree_accept(parents, draft, target)
            assert path.tolist() == list(range(k + 1))
            assert nxt == target[k]


@pytest.mark.parametrize("tree", ["uniform", "chain70"])
def test_deepest_consistent_node(tree):
    rng = np.random.default_rng(1)
    for case in range(200):
        q = int(rng.integers(1, 34))
        parents = synth.sample_parents(synth.rng_for(11, case, synth.TAG_PARENTS), q, tree)
        draft = synth.draft_tokens(synth.rng_for(11, case, synth.TAG_DRAFT_TOK), parents, vocab=4 + q)
        target = rng.integers(0, 4 + q, size=q).astype(np.int32)
        # make agreement frequent: copy a random child's draft token into some targets
        for c in range(q):
            kids = [j for j in range(q) if parents[j] == c]
            if kids and rng.random() < 0.7:
                target[c] = draft[kids[int(rng.integers(0, len(kids)))]]
        path, nxt = acc.tree_accept(parents, draft, target)
        assert path.tolist() == deepest_consistent(parents, draft, target)
        assert nxt == target[path[-1]]


def test_all_small_trees_exhaustive_tokens():
    """Every valid tree with q <= 4 and every draft/target assignment over a 2-token vocabulary
    (sibling tokens distinct), against the upward formulation."""
    for q in range(1, 5):
        for par in itertools.product(*[range(i) for i in range(1, q)]):
            parents = np.array((-1,) + par, dtype=np.int32)
            for dr in itertools.product(range(2), repeat=q):
                draft = np.array(dr, dtype=np.int32)
                sib_ok = all(draft[a] != draft[b] for a in range(1, q) for b in range(a + 1, q)
                             if parents[a] == parents[b])
                if not sib_ok:
                    continue
                for tg in itertools.product(range(2), repeat=q):
                    target = np.array(tg, dtype=np.int32)
                    path, nxt = acc.tree_accept(parents, draft, target)
                    assert path.tolist() == deepest_consistent(parents, draft, target)
                    assert nxt == target[path[-1]]


@pytest.mark.parametrize("q", [1, 9, 33, 64])
def test_planted_paths(q):
    for stream in range(50):
        parents, draft, target, planted = synth.accept_case(7, stream, q)
        path, nxt = acc.tree_accept(parents, draft, target)
        assert path.tolist() == planted.tolist()
        assert nxt == target[planted[-1]]


def test_workload_tokens_accept_the_drawn_leaf_path():
    b = synth.make_batch(synth.WORKLOADS["s8-p1024-q33"])
    keep, n_keep, nxt = acc.tree_accept_streams(b.parents, b.draft_tok, b.target_tok)
    assert (n_keep == b.n_keep).all()
    for s in range(len(n_keep)):
        assert (keep[s, : n_keep[s]] == b.keep[s, : b.n_keep[s]]).all()
        assert nxt[s] == b.target_tok[s, b.keep[s, b.n_keep[s] - 1]]


def f_target(ctx, vocab):
    """A deterministic synthetic target model: the next token as a function of the context."""
    h = 1469598103934665603
    for t in ctx:
        h = ((h ^ (int(t) + 1)) * 1099511628211) & ((1 << 64) - 1)
    return int(h % vocab)


def test_matches_autoregressive_greedy():
    rng = np.random.default_rng(3)
    vocab = 5
    for case in range(300):
        q = int(rng.integers(1, 40))
        parents = synth.sample_parents(synth.rng_for(21, case, synth.TAG_PARENTS), q, "uniform")
        prompt = [int(x) for x in rng.integers(0, vocab, size=4)]
        # drafter: distinct candidates per parent, the target's choice included with probability 0.6
        draft = np.zeros(q, np.int32)
        draft[0] = prompt[-1]
        ctx = {0: prompt}
        for j in range(1, q):
            p = int(parents[j])
            used = {int(draft[k]) for k in range(1, j) if parents[k] == p}
            want = f_target(ctx[p], vocab)
            if want not in used and rng.random() < 0.6:
                draft[j] = want
            else:
                free = [t for t in range(vocab) if t not in used]
                draft[j] = free[int(rng.integers(0, len(free)))] if free else want
            ctx[j] = ctx[p] + [int(draft[j])]
        if len({(int(parents[j]), int(draft[j])) for j in range(1, q)}) != q - 1:
            continue  # a parent ran out of distinct tokens; skip the degenerate draw
        target = np.array([f_target(ctx[i], vocab) for i in range(q)], np.int32)
        path, nxt = acc.tree_accept(parents, draft, target)
        accepted = [int(draft[i]) for i in path[1:]] + [nxt]
        seq = list(prompt)
        ar = []
        for _ in range(len(accepted)):
            t = f_target(seq, vocab)
            ar.append(t)
            seq.append(t)
        assert accepted == ar


def test_no_match_keeps_root_only():
    parents = np.array([-1, 0, 0, 1], np.int32)
    draft = np.array([9, 1, 2, 3], np.int32)
    target = np.array([5, 7, 7, 7], np.int32)
    path, nxt = acc.tree_accept(parents, draft, target)
    assert path.tolist() == [0] and nxt == 5


def test_duplicate_sibling_tokens_take_the_lowest_index():
    parents = np.array([-1, 0, 0, 2, 1], np.int32)
    draft = np.array([0, 4, 4, 6, 8], np.int32)
    target = np.array([4, 8, 6, 1, 2], np.int32)
    path, nxt = acc.tree_accept(parents, draft, target)
    assert path.tolist() == [0, 1, 4] and nxt == 2


def test_full_length_chain_hits_the_bound_exactly():
    q = 64
    parents = np.arange(-1, q - 1, dtype=np.int32)
    draft = np.arange(q, dtype=np.int32)
    target = np.arange(1, q + 1, dtype=np.int32)
    path, nxt = acc.tree_accept(parents, draft, target)
    assert len(path) == q and nxt == q


@pytest.mark.parametrize("parents", [[0, 0], [-1, 1], [-1, 0, 2], [-1, -1], [-1, 0, 5]])
def test_rejects_malformed_trees(parents):
    p = np.array(parents, np.int32)
    with pytest.raises(ValueError):
        acc.tree_accept(p, np.zeros(len(p), np.int32), np.zeros(len(p), np.int32))


def test_pins_catch_planted_mistakes(monkeypatch):
    """Mistakes planted in a copy of the walk (on the CPU) must fail a pin above."""
    def last_match(parents, draft, target):
        q = len(parents)
        path, cur = [0], 0
        while len(path) < q:
            kids = [j for j in acc.children(parents, cur) if int(draft[j]) == int(target[cur])]
            if not kids:
                break
            cur = kids[-1]
            path.append(cur)
        return np.array(path, np.int32), int(target[cur])

    def own_target(parents, draft, target):  # compares draft[j] with target[j] instead of target[parent]
        q = len(parents)
        path, cur = [0], 0
        while len(path) < q:
            kids = [j for j in acc.children(parents, cur) if int(draft[j]) == int(target[j])]
            if not kids:
                break
            cur = kids[0]
            path.append(cur)
        return np.array(path, np.int32), int(target[cur])

    def parent_next(parents, draft, target):  # next token read at the parent of the last node
        path, _ = ORIG(parents, draft, target)
        return path, int(target[path[-2]]) if len(path) > 1 else int(target[0]) + 1

    ORIG = acc.tree_accept
    for mutant, pin in ((last_match, test_duplicate_sibling_tokens_take_the_lowest_index),
                        (own_target, test_chain_closed_form),
                        (parent_next, test_matches_autoregressive_greedy)):
        monkeypatch.setattr(acc, "tree_accept", mutant)
        with pytest.raises(AssertionError):
            pin()
        monkeypatch.setattr(acc, "tree_accept", ORIG)
