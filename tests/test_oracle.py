"""Pins for the fp64 oracle, checked against things other than the oracle itself.

* brute force: a scalar per-(query, head, key) evaluation over every valid tree with at most six
  nodes, visibility found by walking ``parents`` by hand;
* a chain-shaped tree is ordinary causal attention (``torch`` scaled-dot-product attention, fp64);
* every node's output is causal attention over its own root-to-node path;
* closed form for zero queries: the output is the mean of the visible latent rows and
  ``lse = ln(#visible)``;
* the lse merge of a prefix-only and a tree-only attention gives the full result;
* special cases: one query is plain single-query decode; a star tree; an empty prefix;
* equivariances: heads, streams, topological relabelling of the tree;
* the absorb identity: standard MLA with random up-projections equals the absorbed form;
* bf16 widening agrees with torch's bf16 -> fp64 conversion.

The cache-geometry passages are on "Race Conditions, Buffer Aliasing, and the Architecture of a
Native DDTree Inference Engine", section "The Cache Compaction Problem".
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import verify as ov
import synth

SCALE = 1.0 / math.sqrt(192.0)
TOL = 1e-10


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _inputs(rng, q, p, h, dl=512, dr=64):
    return (_rand(rng, q, h, dl), _rand(rng, q, h, dr), _rand(rng, p + q, dl), _rand(rng, p + q, dr))


def all_trees(q):
    """Every parents[] array with parents[0] = -1 and parents[i] in [0, i)."""
    for choice in itertools.product(*[range(i) for i in range(1, q)]):
        yield np.array((-1,) + choice, dtype=np.int64)


def brute_force(ql, qp, c, k, p, parents, scale=SCALE):
    """Scalar evaluation: explicit ancestor walk, one dot product per (query, head, key)."""
    q, h = ql.shape[0], ql.shape[1]
    out = np.zeros((q, h, c.shape[1]))
    lse = np.zeros((q, h))
    for i in range(q):
        seen = set(range(p))
        node = i
        while node != -1:
            seen.add(p + node)
            node = int(parents[node])
        keys = sorted(seen)
        for hh in range(h):
            s = [scale * (math.fsum(ql[i, hh] * c[t]) + math.fsum(qp[i, hh] * k[t])) for t in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            lse[i, hh] = m + math.log(z)
            for wt, t in zip(w, keys):
                out[i, hh] += (wt / z) * c[t]
    return out, lse


def sdpa(q, k, v, mask, scale=SCALE):
    """torch reference attention (fp64, CPU).  q [H, Nq, D], k/v [Nk, D], mask [Nq, Nk] bool."""
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(k)[None].expand(q.shape[0], -1, -1)
    vt = torch.from_numpy(v)[None].expand(q.shape[0], -1, -1)
    mt = torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale)
    logits = (qt @ kt.transpose(-1, -2)) * scale
    lse = torch.logsumexp(logits.masked_fill(~mt, float("-inf")), dim=-1)
    return out.numpy(), lse.numpy()


# ---------------------------------------------------------------- brute force over all trees

@pytest.mark.parametrize("q", [1, 2, 3, 4, 5, 6])
def test_brute_force_all_small_trees(q):
    rng = np.random.default_rng(100 + q)
    prefixes = [0, 1, 5] if q <= 5 else [3]
    n_trees = 0
    for p in prefixes:
        ql, qp, c, k = _inputs(rng, q, p, 2)
        for parents in all_trees(q):
            o, l = oracle.verify_attn_f64(ql, qp, c, k, p, parents)
            bo, bl = brute_force(ql, qp, c, k, p, parents)
            assert np.abs(o - bo).max() < TOL
            assert np.abs(l - bl).max() < TOL
            n_trees += 1
    assert n_trees == len(prefixes) * math.factorial(q - 1)


# ---------------------------------------------------------------- invariants vs torch

def _chain(q):
    return np.arange(-1, q - 1, dtype=np.int64)


@pytest.mark.parametrize("q,p", [(9, 17), (33, 40), (5, 0)])
def test_chain_is_causal_attention(q, p):
    rng = np.random.default_rng(q * 1000 + p)
    h = 3
    ql, qp, c, k = _inputs(rng, q, p, h)
    o, l = oracle.verify_attn_f64(ql, qp, c, k, p, _chain(q))
    qcat = np.concatenate([ql, qp], axis=2).transpose(1, 0, 2)  # [H, Q, 576]
    kcat = np.concatenate([c, k], axis=1)
    mask = np.arange(p + q)[None, :] <= (p + np.arange(q))[:, None]
    ro, rl = sdpa(qcat, kcat, c, mask)
    assert np.abs(o - ro.transpose(1, 0, 2)).max() < TOL
    assert np.abs(l - rl.T).max() < TOL


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_each_node_is_causal_attention_over_its_path(seed):
    rng = np.random.default_rng(seed)
    q, p, h = 17, 11, 2
    parents = synth.sample_parents(synth.rng_for(seed, 0, 4), q)
    ql, qp, c, k = _inputs(rng, q, p, h)
    o, l = oracle.verify_attn_f64(ql, qp, c, k, p, parents)
    for i in range(q):
        path = []
        node = i
        while node != -1:
            path.append(node)
            node = int(parents[node])
        rows = list(range(p)) + [p + j for j in reversed(path)]
        kk, vv = np.concatenate([c, k], axis=1)[rows], c[rows]
        qi = np.concatenate([ql[i], qp[i]], axis=1)[:, None, :]  # [H, 1, 576]
        ro, rl = sdpa(qi, kk, vv, np.ones((1, len(rows)), dtype=bool))
        assert np.abs(o[i] - ro[:, 0]).max() < TOL
        assert np.abs(l[i] - rl[:, 0]).max() < TOL


def _depth(parents):
    d = []
    for i in range(len(parents)):
        n, node = 0, i
        while parents[node] != -1:
            node = int(parents[node])
            n += 1
        d.append(n)
    return np.array(d)


@pytest.mark.parametrize("p", [0, 1, 64])
def test_zero_queries_closed_form(p):
    """q = 0: every visible key scores 0, so out = mean of visible c_kv, lse = ln(count)."""
    rng = np.random.default_rng(7 + p)
    q, h = 33, 2
    parents = synth.sample_parents(synth.rng_for(9, p, 4), q)
    _, _, c, k = _inputs(rng, q, p, h)
    o, l = oracle.verify_attn_f64(np.zeros((q, h, 512)), np.zeros((q, h, 64)), c, k, p, parents)
    dep = _depth(parents)
    for i in range(q):
        count = p + dep[i] + 1
        assert np.allclose(l[i], math.log(count), atol=TOL, rtol=0)
        rows = list(range(p))
        node = i
        while node != -1:
            rows.append(p + node)
            node = int(parents[node])
        assert len(rows) == count
        assert np.abs(o[i] - c[rows].mean(axis=0)[None]).max() < TOL


def test_lse_merge_of_prefix_and_tree_parts():
    rng = np.random.default_rng(11)
    q, p, h = 21, 30, 3
    parents = synth.sample_parents(synth.rng_for(11, 0, 4), q)
    ql, qp, c, k = _inputs(rng, q, p, h)
    o, l = oracle.verify_attn_f64(ql, qp, c, k, p, parents)
    # prefix part: unmasked attention over rows [0, P)
    qcat = np.concatenate([ql, qp], axis=2).transpose(1, 0, 2)
    kcat = np.concatenate([c, k], axis=1)
    po, pl = sdpa(qcat, kcat[:p], c[:p], np.ones((q, p), dtype=bool))
    po, pl = po.transpose(1, 0, 2), pl.T
    # tree part: the same tree with an empty prefix
    to, tl = oracle.verify_attn_f64(ql, qp, c[p:], k[p:], 0, parents)
    ml = np.logaddexp(pl, tl)
    mo = np.exp(pl - ml)[..., None] * po + np.exp(tl - ml)[..., None] * to
    assert np.abs(l - ml).max() < TOL
    assert np.abs(o - mo).max() < TOL


def test_single_query_is_plain_decode():
    rng = np.random.default_rng(12)
    p, h = 50, 4
    ql, qp, c, k = _inputs(rng, 1, p, h)
    o, l = oracle.verify_attn_f64(ql, qp, c, k, p, np.array([-1]))
    qcat = np.concatenate([ql, qp], axis=2).transpose(1, 0, 2)
    ro, rl = sdpa(qcat, np.concatenate([c, k], axis=1), c, np.ones((1, p + 1), dtype=bool))
    assert np.abs(o - ro.transpose(1, 0, 2)).max() < TOL
    assert np.abs(l - rl.T).max() < TOL


def test_star_tree_with_empty_prefix():
    rng = np.random.default_rng(13)
    q, h = 9, 2
    parents = np.array([-1] + [0] * (q - 1))
    ql, qp, c, k = _inputs(rng, q, 0, h)
    o, l = oracle.verify_attn_f64(ql, qp, c, k, 0, parents)
    mask = np.zeros((q, q), dtype=bool)
    mask[:, 0] = True
    mask[np.arange(q), np.arange(q)] = True
    qcat = np.concatenate([ql, qp], axis=2).transpose(1, 0, 2)
    ro, rl = sdpa(qcat, np.concatenate([c, k], axis=1), c, mask)
    assert np.abs(o - ro.transpose(1, 0, 2)).max() < TOL
    assert np.abs(l - rl.T).max() < TOL


# ---------------------------------------------------------------- equivariances

def test_head_permutation():
    rng = np.random.default_rng(14)
    q, p, h = 9, 7, 5
    parents = synth.sample_parents(synth.rng_for(14, 0, 4), q)
    ql, qp, c, k = _inputs(rng, q, p, h)
    perm = rng.permutation(h)
    o, l = oracle.verify_attn_f64(ql, qp, c, k, p, parents)
    po, pl = oracle.verify_attn_f64(ql[:, perm], qp[:, perm], c, k, p, parents)
    assert np.array_equal(po, o[:, perm]) or np.abs(po - o[:, perm]).max() < TOL
    assert np.abs(pl - l[:, perm]).max() < TOL


def test_streams_are_independent():
    b = synth.random_inputs(15, streams=3, prefix=10, q_len=5, heads=2)
    o, l = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 10, b.parents)
    ckv2 = b.ckv.copy()
    ckv2[1] ^= 0x0101  # perturb stream 1 only
    o2, l2 = oracle.verify_attn(b.q_lat, b.q_pe, ckv2, b.kpe, 10, b.parents)
    assert np.array_equal(o[0], o2[0]) and np.array_equal(o[2], o2[2])
    assert np.array_equal(l[0], l2[0]) and np.array_equal(l[2], l2[2])
    assert not np.array_equal(o[1], o2[1])


def test_topological_relabelling():
    """Renumbering the nodes in another parent-before-child order, with the tree rows and
    queries moved alike, permutes the outputs: the mask depends only on ancestry."""
    rng = np.random.default_rng(16)
    q, p, h = 12, 6, 2
    parents = synth.sample_parents(synth.rng_for(16, 0, 4), q)
    # random topological order: repeatedly pick a random node whose parent is already placed
    placed, order = set(), []
    while len(order) < q:
        ready = [i for i in range(q) if i not in placed and (parents[i] == -1 or parents[i] in placed)]
        pick = ready[rng.integers(0, len(ready))]
        order.append(pick)
        placed.add(pick)
    new_of_old = {old: new for new, old in enumerate(order)}
    new_parents = np.array([-1 if parents[old] == -1 else new_of_old[parents[old]] for old in order])
    ql, qp, c, k = _inputs(rng, q, p, h)
    o, l = oracle.verify_attn_f64(ql, qp, c, k, p, parents)
    rows = list(range(p)) + [p + old for old in order]
    no, nl = oracle.verify_attn_f64(ql[order], qp[order], c[rows], k[rows], p, new_parents)
    assert np.abs(no - o[order]).max() < TOL
    assert np.abs(nl - l[order]).max() < TOL


# ---------------------------------------------------------------- absorb identity

def test_absorb_identity_with_random_up_projections():
    """Standard MLA: k_nope = W_UK c, v = W_UV c, scores over [q_nope | q_pe] . [k_nope | k_pe]
    with scale 1/sqrt(128 + 64).  Absorbed: q_lat = W_UK^T q_nope, out = W_UV out_lat."""
    rng = np.random.default_rng(17)
    q, p, h, d = 9, 13, 3, 128
    parents = synth.sample_parents(synth.rng_for(17, 0, 4), q)
    w_uk = rng.standard_normal((h, d, 512)) / math.sqrt(512)
    w_uv = rng.standard_normal((h, d, 512)) / math.sqrt(512)
    q_nope = rng.standard_normal((q, h, d))
    q_pe = rng.standard_normal((q, h, 64))
    c = rng.standard_normal((p + q, 512))
    k_pe = rng.standard_normal((p + q, 64))
    mask = np.zeros((q, p + q), dtype=bool)
    mask[:, :p] = True
    for i in range(q):
        node = i
        while node != -1:
            mask[i, p + node] = True
            node = int(parents[node])
    std_out = np.zeros((q, h, d))
    for hh in range(h):
        k_full = np.concatenate([c @ w_uk[hh].T, k_pe], axis=1)  # [L, 192]
        v = c @ w_uv[hh].T                                       # [L, 128]
        qh = np.concatenate([q_nope[:, hh], q_pe[:, hh]], axis=1)[None]
        ro, _ = sdpa(qh, k_full, v, mask, scale=1.0 / math.sqrt(d + 64))
        std_out[:, hh] = ro[0]
    q_lat = np.einsum("hdc,qhd->qhc", w_uk, q_nope)
    out_lat, _ = oracle.verify_attn_f64(q_lat, q_pe, c, k_pe, p, parents)
    absorbed = np.einsum("hdc,qhc->qhd", w_uv, out_lat)
    assert abs(oracle.DEFAULT_SCALE - 1.0 / math.sqrt(d + 64)) < 1e-15
    assert np.abs(absorbed - std_out).max() < 1e-9


# ---------------------------------------------------------------- bf16 widening, validation

def test_bf16_widening_matches_torch():
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite values only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), ref)


def test_rejects_malformed_parents():
    with pytest.raises(ValueError):
        oracle.ancestor_or_self(np.array([0, 0]))
    with pytest.raises(ValueError):
        oracle.ancestor_or_self(np.array([-1, 1]))
    with pytest.raises(ValueError):
        oracle.ancestor_or_self(np.array([-1, 0, 3, 1]))


# ---------------------------------------------------------------- planted mistakes are caught

def _pins_pass():
    try:
        test_chain_is_causal_attention(9, 17)
        test_zero_queries_closed_form(1)
        test_each_node_is_causal_attention_over_its_path(0)
        test_absorb_identity_with_random_up_projections()
    except AssertionError:
        return False
    return True


MUTANTS = {
    "drop_rope_term": ("scores_absorbed",
                       lambda ql, qp, c, k, scale: scale * np.matmul(ql, c.T)),
    "wrong_scale": ("scores_absorbed",
                    lambda ql, qp, c, k, scale: (np.matmul(ql, c.T) + np.matmul(qp, k.T)) / 24.0),
    "rope_sign": ("scores_absorbed",
                  lambda ql, qp, c, k, scale: scale * (np.matmul(ql, c.T) - np.matmul(qp, k.T))),
    "no_self": ("visibility", None),
    "prefix_off_by_one": ("visibility", None),
    "parent_not_ancestor": ("visibility", None),
}


def _mutant_visibility(kind):
    real = ov.visibility

    def vis(parents, prefix_len):
        v = real(parents, prefix_len).copy()
        q = len(parents)
        if kind == "no_self":
            for i in range(1, q):
                v[i, prefix_len + i] = False
        elif kind == "prefix_off_by_one" and prefix_len > 0:
            v[:, prefix_len - 1] = False
        elif kind == "parent_not_ancestor":
            for i in range(q):
                v[i, prefix_len:] = False
                v[i, prefix_len + i] = True
                if parents[i] >= 0:
                    v[i, prefix_len + parents[i]] = True
                v[i, prefix_len] = True
        return v
    return vis


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail_a_pin(name, monkeypatch):
    assert _pins_pass()
    attr, fn = MUTANTS[name]
    if fn is None:
        fn = _mutant_visibility(name)
    monkeypatch.setattr(ov, attr, fn)
    assert not _pins_pass(), f"planted mistake {name} went unnoticed"
