"""GPU parity: ddtree_tree_build through the C ABI, bit-exact against the best-first oracle
(parents, tokens, depths, float32 log-weights, retrieve links, ancestor masks, node count), and
the whole step chained on the device: build -> verify -> accept + compact."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, dev_bf16, dev_i32, host_bits

pytestmark = pytest.mark.gpu


def drafter(seed, streams, d, k, quantize=None):
    lps, toks = [], []
    for s in range(streams):
        lp, tok = synth.drafter_topk(seed, s, d, k)
        if quantize:
            lp = -np.sort(-np.round(lp / quantize) * quantize, axis=1).astype(np.float32)  # many exact ties
        lps.append(lp)
        toks.append(tok)
    return np.stack(lps), np.stack(toks)


def check_build(lib, lp, tok, budget, roots=None, what=""):
    s_count = lp.shape[0]
    print(f"[build] {what} S={s_count} D={lp.shape[1]} K={lp.shape[2]} budget={budget}", flush=True)
    par, tks, n, ex = lib.tree_build(torch.from_numpy(lp).to("cuda:0"), dev_i32(tok), budget,
                                     root_tokens=None if roots is None else dev_i32(roots), extras=True)
    torch.cuda.synchronize()
    par, tks, n = par.cpu().numpy(), tks.cpu().numpy(), n.cpu().numpy()
    ex = {k: v.cpu().numpy() for k, v in ex.items()}
    for s in range(s_count):
        ref = oracle.tree_build(lp[s], tok[s], budget, -1 if roots is None else int(roots[s]))
        m = ref["n_nodes"]
        assert n[s] == m, (what, s)
        assert np.array_equal(par[s, :m], ref["parents"]), (what, s)
        assert np.array_equal(tks[s, :m], ref["tokens"]), (what, s)
        assert np.array_equal(ex["depths"][s, :m], ref["depths"]), (what, s)
        assert np.array_equal(ex["logw"][s, :m].view(np.uint32), ref["logw"].view(np.uint32)), (what, s)
        assert np.array_equal(ex["first_child"][s, :m], ref["first_child"]), (what, s)
        assert np.array_equal(ex["next_sibling"][s, :m], ref["next_sibling"]), (what, s)
        assert np.array_equal(ex["anc"][s, :m].view(np.uint64), ref["anc"]), (what, s)
        assert (par[s, m:] == -2).all() and (tks[s, m:] == -2).all(), (what, s)  # untouched past n_nodes
    return n


@pytest.mark.parametrize("d,k,budget", [(8, 4, 32), (15, 8, 63), (4, 3, 20), (1, 5, 5), (64, 64, 63),
                                        (2, 64, 63), (63, 2, 63),
                                        # budget 33: the smallest on the two-slot pool (32 and
                                        # below take the one-slot kernel); budget 1: one pop
                                        (6, 16, 33), (3, 2, 1)])
def test_build_matches_oracle(lib, d, k, budget):
    lp, tok = drafter(20 + d, 64, d, k)
    roots = np.arange(64, dtype=np.int32) + 1000
    n = check_build(lib, lp, tok, budget, roots, f"d={d} k={k}")
    assert (n == budget + 1).all()


def test_heap_runs_empty(lib):
    lp, tok = drafter(3, 8, 5, 1)
    n = check_build(lib, lp, tok, 20, what="top-1 chain")
    assert (n == 6).all()
    lp, tok = drafter(4, 8, 3, 2)  # 2 + 4 + 8 = 14 nodes in the whole product tree
    n = check_build(lib, lp, tok, 63, what="small product tree")
    assert (n == 15).all()


def test_ties_follow_insertion_order(lib):
    lp, tok = drafter(5, 64, 10, 6, quantize=0.25)
    check_build(lib, lp, tok, 63, what="quantized log-probs (ties)")
    lp = np.zeros((4, 6, 5), np.float32) - 1.0  # every candidate of a level ties
    tok = np.arange(4 * 6 * 5, dtype=np.int32).reshape(4, 6, 5)
    check_build(lib, lp, tok, 40, what="all-equal log-probs")


def test_signed_zero_log_probs_tie(lib):
    """Log-probabilities of exactly 0 with either sign (a saturated drafter): -0.0 and +0.0
    compare equal, so candidates weighing either are taken in insertion order, and the float32
    weights keep the signs that IEEE sums give them."""
    rng = np.random.default_rng(77)
    lp = np.where(rng.random((16, 6, 5)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    lp[:, :, 3:] = np.float32(-1.0)
    tok = np.arange(16 * 6 * 5, dtype=np.int32).reshape(16, 6, 5)
    assert (np.signbit(lp[:, :, :3]).any() and (~np.signbit(lp[:, :, :3])).any())
    check_build(lib, lp, tok, 40, what="signed zeros")


def test_build_verify_accept_compact_chain(lib):
    """The step on the device: build the trees, verify them, accept against planted target
    tokens and compact, each stage fed by the previous stage's device outputs."""
    s_count, d, k, budget, prefix = 8, 8, 4, 32, 300
    q = budget + 1
    lp, tok = drafter(77, s_count, d, k)
    roots = np.arange(s_count, dtype=np.int32) + 5
    par, tks, n = lib.tree_build(torch.from_numpy(lp).to("cuda:0"), dev_i32(tok), budget, root_tokens=dev_i32(roots))
    b = synth.random_inputs(78, s_count, prefix, q)
    out, lse = lib.verify_attn(dev_bf16(b.q_lat), dev_bf16(b.q_pe), dev_bf16(b.ckv), dev_bf16(b.kpe), prefix, par)
    torch.cuda.synchronize()
    parents = par.cpu().numpy()
    draft = tks.cpu().numpy()
    assert (n.cpu().numpy() == q).all()
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, prefix, parents)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "verify on built trees")
    target = np.zeros_like(draft)
    for s in range(s_count):
        path = synth.accepted_path(synth.rng_for(78, s, synth.TAG_LEAF), parents[s])
        target[s] = synth.target_tokens(synth.rng_for(78, s, synth.TAG_TARGET_TOK), parents[s], draft[s], path)
    c, kp = dev_bf16(b.ckv), dev_bf16(b.kpe)
    keep, n_keep, nxt = lib.accept_compact(c, kp, prefix, par, tks, dev_i32(target))
    torch.cuda.synchronize()
    rk, rn, rx = oracle.tree_accept_streams(parents, draft, target)
    assert np.array_equal(n_keep.cpu().numpy(), rn) and np.array_equal(nxt.cpu().numpy(), rx)
    rc, rkp = oracle.compact_kv(b.ckv, b.kpe, prefix, rk, rn)
    assert np.array_equal(host_bits(c), rc) and np.array_equal(host_bits(kp), rkp)
