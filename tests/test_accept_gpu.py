"""GPU parity: ddtree_tree_accept and ddtree_accept_compact through the C ABI, bit-exact against
the greedy-acceptance oracle (keep, n_keep, next_token) and, for the fused call, against the
oracle's acceptance followed by its out-of-place compaction on the whole cache buffers."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, dev_bf16, dev_i32, guarded_bf16, guarded_i32, host_bits

pytestmark = pytest.mark.gpu


def run_accept(lib, parents, draft, target, stride=None, status=None):
    s, q = parents.shape
    stride = q if stride is None else stride
    keep = torch.full((s, stride), -7, dtype=torch.int32, device="cuda:0")
    keep, n_keep, nxt = lib.tree_accept(dev_i32(parents), dev_i32(draft), dev_i32(target), keep=keep, status=status)
    torch.cuda.synchronize()
    return keep.cpu().numpy(), n_keep.cpu().numpy(), nxt.cpu().numpy()


def check_accept(lib, parents, draft, target, what="", stride=None):
    print(f"[accept] {what} S={parents.shape[0]} Q={parents.shape[1]}", flush=True)
    keep, n_keep, nxt = run_accept(lib, parents, draft, target, stride)
    rk, rn, rx = oracle.tree_accept_streams(parents, draft, target)
    assert np.array_equal(n_keep, rn), what
    assert np.array_equal(nxt, rx), what
    for s in range(parents.shape[0]):
        assert np.array_equal(keep[s, : rn[s]], rk[s, : rn[s]]), (what, s)
        assert (keep[s, rn[s]:] == -7).all(), (what, s)  # entries past n_keep untouched
    return rn


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workloads(lib, name):
    b = synth.make_batch(synth.WORKLOADS[name], with_path=True)
    rn = check_accept(lib, b.parents, b.draft_tok, b.target_tok, name)
    assert np.array_equal(rn, b.n_keep)  # the planted leaf paths


@pytest.mark.parametrize("q", [1, 2, 9, 33, 63, 64])
def test_planted_depths(lib, q):
    cases = [synth.accept_case(31, s, q) for s in range(96)]
    parents = np.stack([c[0] for c in cases])
    draft = np.stack([c[1] for c in cases])
    target = np.stack([c[2] for c in cases])
    rn = check_accept(lib, parents, draft, target, f"planted q={q}")
    assert np.array_equal(rn, [len(c[3]) for c in cases])


def test_degenerate_cases(lib):
    q = 64
    chain = np.arange(-1, q - 1, dtype=np.int32)
    rows = [
        (chain, np.arange(q), np.arange(1, q + 1)),                      # full chain: n = 64
        (chain, np.arange(q), np.zeros(q)),                               # nothing past the root
        (np.r_[-1, np.zeros(q - 1)], np.arange(q), np.full(q, 40)),        # star: child 40
        (np.r_[-1, 0, 0, 2, 1, np.arange(5, q) - 1], np.r_[0, 4, 4, 6, 8, np.arange(5, q)],
         np.r_[4, 8, 6, 1, 2, np.arange(5, q)]),                           # duplicate sibling tokens
    ]
    parents = np.stack([r[0] for r in rows]).astype(np.int32)
    draft = np.stack([r[1] for r in rows]).astype(np.int32)
    target = np.stack([r[2] for r in rows]).astype(np.int32)
    rn = check_accept(lib, parents, draft, target, "degenerate", stride=70)
    assert rn.tolist()[:3] == [64, 1, 2]


def test_malformed_trees_flagged(lib):
    """Malformed trees are flagged with n_keep = 0 and next_token = -1; nothing is written outside
    keep, n_keep, next_token and the status word (guard bands of canary bytes around each)."""
    parents, draft, target, _ = synth.accept_case(5, 0, 17)
    bad = np.stack([parents] * 4).astype(np.int32)
    d = np.stack([draft] * 4)
    t = np.stack([target] * 4)
    bad[1, 5] = 5      # self loop
    bad[2, 0] = 0      # root with a parent
    bad[3, 9] = 12     # forward link (would allow a cycle)
    keep = Guarded((4, 17), torch.int32, fill=-7)
    n_keep = Guarded((4,), torch.int32, fill=-7)
    nxt = Guarded((4,), torch.int32, fill=-7)
    status = Guarded((1,), torch.int32, fill=0)
    lib.tree_accept(dev_i32(bad), dev_i32(d), dev_i32(t), keep=keep.t, n_keep=n_keep.t, next_token=nxt.t,
                    status=status.t)
    torch.cuda.synchronize()
    assert status.t.item() & 1
    k, n, x = keep.t.cpu().numpy(), n_keep.t.cpu().numpy(), nxt.t.cpu().numpy()
    assert n.tolist()[1:] == [0, 0, 0] and x.tolist()[1:] == [-1, -1, -1]
    path, xr = oracle.tree_accept(parents, draft, target)
    assert n[0] == len(path) and x[0] == xr and np.array_equal(k[0, : len(path)], path)
    assert (k[0, len(path):] == -7).all() and (k[1:] == -7).all()
    for g in (keep, n_keep, nxt, status):
        assert g.intact(), "write outside a buffer"


def fused(lib, b, prefix):
    c, k = dev_bf16(b.ckv), dev_bf16(b.kpe)
    keep, n_keep, nxt = lib.accept_compact(c, k, prefix, dev_i32(b.parents), dev_i32(b.draft_tok),
                                           dev_i32(b.target_tok))
    torch.cuda.synchronize()
    return host_bits(c), host_bits(k), keep.cpu().numpy(), n_keep.cpu().numpy(), nxt.cpu().numpy()


@pytest.mark.parametrize("name", [synth.HEADLINE, "s8-p1024-q33", "s1-p4096-q33-chain"])
def test_accept_compact_fused(lib, name):
    w = synth.WORKLOADS[name]
    b = synth.make_batch(w)
    print(f"[accept_compact] {name}", flush=True)
    gc, gk, keep, n_keep, nxt = fused(lib, b, w.prefix)
    rk, rn, rx = oracle.tree_accept_streams(b.parents, b.draft_tok, b.target_tok)
    assert np.array_equal(n_keep, rn) and np.array_equal(nxt, rx)
    rc, rkp = oracle.compact_kv(b.ckv, b.kpe, w.prefix, rk, rn)
    assert np.array_equal(gc, rc)
    assert np.array_equal(gk, rkp)


def test_accept_compact_planted_and_malformed(lib):
    """The fused call on planted trees with one malformed stream, which stays untouched; nothing
    is written outside the cache buffers, keep, n_keep, next_token and the status word (guard
    bands of canary bytes around each)."""
    q, prefix = 33, 50
    cases = [synth.accept_case(41, s, q) for s in range(12)]
    parents = np.stack([c[0] for c in cases]).astype(np.int32)
    parents[4, 7] = 9  # malformed: stream 4 must stay untouched
    b = synth.random_inputs(77, 12, prefix, q)
    b.parents = parents
    b.draft_tok = np.stack([c[1] for c in cases])
    b.target_tok = np.stack([c[2] for c in cases])
    print("[accept_compact] planted + malformed", flush=True)
    c, k = guarded_bf16(b.ckv), guarded_bf16(b.kpe)
    keep = Guarded((12, q), torch.int32, fill=-7)
    n_keep = Guarded((12,), torch.int32, fill=-7)
    nxt = Guarded((12,), torch.int32, fill=-7)
    status = Guarded((1,), torch.int32, fill=0)
    lib.accept_compact(c.t, k.t, prefix, dev_i32(b.parents), dev_i32(b.draft_tok), dev_i32(b.target_tok),
                       keep=keep.t, n_keep=n_keep.t, next_token=nxt.t, status=status.t)
    torch.cuda.synchronize()
    gc, gk = host_bits(c.t), host_bits(k.t)
    n_k, nx = n_keep.t.cpu().numpy(), nxt.t.cpu().numpy()
    assert n_k[4] == 0 and nx[4] == -1 and status.t.item() & 1
    good = [s for s in range(12) if s != 4]
    rk = np.full((12, q), -1, np.int32)
    rn = np.zeros(12, np.int32)
    for s in good:
        path, x = oracle.tree_accept(parents[s], b.draft_tok[s], b.target_tok[s])
        rk[s, : len(path)] = path
        rn[s] = len(path)
        assert nx[s] == x and n_k[s] == len(path)
    rc, rkp = oracle.compact_kv(b.ckv, b.kpe, prefix, rk, rn)
    assert np.array_equal(gc, rc)
    assert np.array_equal(gk, rkp)
    for g in (c, k, keep, n_keep, nxt, status):
        assert g.intact(), "write outside a buffer"
