"""GPU parity: ddtree_compact_kv_layers and ddtree_accept_compact_layers through the C ABI.  Every
layer's cache must equal, bit for bit, the compaction oracle applied to that layer alone; the
acceptance outputs must equal the greedy-acceptance oracle; per-stream prefixes advance by the
accepted count exactly once, whatever the number of layers."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, guarded_bf16, dev_bf16, dev_i32, host_bits

pytestmark = pytest.mark.gpu


def trees(seed, s_count, q):
    cases = [synth.accept_case(seed, s, q) for s in range(s_count)]
    parents = np.stack([c[0] for c in cases]).astype(np.int32)
    draft = np.stack([c[1] for c in cases]).astype(np.int32)
    target = np.stack([c[2] for c in cases]).astype(np.int32)
    return parents, draft, target


def upload(layers):
    return [(dev_bf16(c), dev_bf16(k)) for c, k in layers]


def check_layers(dev_layers, host_layers, prefixes, keep, n_keep, what):
    for l, ((c, k), (hc, hk)) in enumerate(zip(dev_layers, host_layers)):
        rc, rk = oracle.compact_kv_ragged(hc, hk, prefixes, keep, n_keep)
        assert np.array_equal(host_bits(c), rc), (what, l)
        assert np.array_equal(host_bits(k), rk), (what, l)


@pytest.mark.parametrize("n_layers,s_count,prefix,q", [(5, 8, 300, 33), (61, 4, 64, 17), (128, 2, 40, 9),
                                                        (3, 64, 100, 64)])
def test_accept_compact_layers_uniform(lib, n_layers, s_count, prefix, q):
    print(f"[layers] accept+compact L={n_layers} S={s_count} P={prefix} Q={q}", flush=True)
    parents, draft, target = trees(50 + q, s_count, q)
    host = synth.layer_caches(60 + n_layers, n_layers, s_count, prefix + q + 3)
    dev = upload(host)
    keep, n_keep, nxt = lib.accept_compact_layers(dev, prefix, dev_i32(parents), dev_i32(draft), dev_i32(target))
    torch.cuda.synchronize()
    rk, rn, rx = oracle.tree_accept_streams(parents, draft, target)
    assert np.array_equal(n_keep.cpu().numpy(), rn) and np.array_equal(nxt.cpu().numpy(), rx)
    kk = keep.cpu().numpy()
    for s in range(s_count):
        assert np.array_equal(kk[s, : rn[s]], rk[s, : rn[s]])
    check_layers(dev, host, [prefix] * s_count, rk, rn, "uniform")


def test_accept_compact_layers_ragged_advances_once(lib):
    q, n_layers = 33, 7
    prefixes = np.array([0, 17, 300, 64, 10, 299], np.int32)
    rows = 300 + q
    parents, draft, target = trees(71, len(prefixes), q)
    parents[5, 3] = 7  # malformed tree: nothing moves, prefix kept
    pl_host = prefixes.copy()
    pl_host[4] = rows - q + 1  # tree block past the end: flagged, nothing moves
    host = synth.layer_caches(72, n_layers, len(prefixes), rows)
    dev = upload(host)
    pl = dev_i32(pl_host)
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    print("[layers] ragged accept+compact", flush=True)
    keep, n_keep, nxt = lib.accept_compact_layers(dev, pl, dev_i32(parents), dev_i32(draft), dev_i32(target),
                                                  status=status)
    torch.cuda.synchronize()
    assert status.item() == 4 | 1
    rn = np.zeros(len(prefixes), np.int32)
    rk = np.full((len(prefixes), q), -1, np.int32)
    for s in range(len(prefixes)):
        if s == 5:
            continue
        path, x = oracle.tree_accept(parents[s], draft[s], target[s])
        rk[s, : len(path)] = path
        rn[s] = len(path)
        assert nxt.cpu().numpy()[s] == x
    assert np.array_equal(n_keep.cpu().numpy(), rn)
    moved = rn.copy()
    moved[4] = 0
    check_layers(dev, host, pl_host, rk, moved, "ragged")
    assert np.array_equal(pl.cpu().numpy(), pl_host + moved)


def test_compact_kv_layers(lib):
    q, n_layers = 33, 6
    prefixes = np.array([0, 17, 300, 64], np.int32)
    rows = 300 + q
    parents, _, _ = trees(81, len(prefixes), q)
    keep = np.full((len(prefixes), q), -1, np.int32)
    n_keep = np.zeros(len(prefixes), np.int32)
    for s in range(len(prefixes)):
        path = synth.accepted_path(synth.rng_for(81, s, synth.TAG_LEAF), parents[s])
        keep[s, : len(path)] = path
        n_keep[s] = len(path)
    host = synth.layer_caches(82, n_layers, len(prefixes), rows)
    print("[layers] compact, uniform and ragged", flush=True)
    dev = upload(host)
    lib.compact_kv_layers(dev, 200, dev_i32(keep), dev_i32(n_keep))
    torch.cuda.synchronize()
    check_layers(dev, host, [200] * len(prefixes), keep, n_keep, "uniform")
    dev = upload(host)
    pl = dev_i32(prefixes)
    lib.compact_kv_layers(dev, pl, dev_i32(keep), dev_i32(n_keep))
    torch.cuda.synchronize()
    check_layers(dev, host, prefixes, keep, n_keep, "ragged")
    assert np.array_equal(pl.cpu().numpy(), prefixes)  # read only


def test_compact_kv_layers_bad_keep(lib):
    """Invalid keep rows are flagged and skipped in every layer; nothing is written outside the
    layers' caches or the status word (guard bands of canary bytes around each)."""
    q, n_layers, prefix = 9, 4, 50
    parents, _, _ = trees(91, 3, q)
    keep = np.array([[0, 2, 5, -1, -1, -1, -1, -1, -1],
                     [0, 3, 3, -1, -1, -1, -1, -1, -1],   # not strictly increasing
                     [0, 1, 2, 3, 4, 5, 6, 7, 8]], np.int32)
    n_keep = np.array([3, 3, 10], np.int32)              # stream 2: more than keep_stride
    host = synth.layer_caches(92, n_layers, 3, prefix + q)
    guarded = [(guarded_bf16(c), guarded_bf16(k)) for c, k in host]
    dev = [(c.t, k.t) for c, k in guarded]
    status = Guarded((1,), torch.int32, fill=0)
    lib.compact_kv_layers(dev, prefix, dev_i32(keep), dev_i32(n_keep), status=status.t)
    torch.cuda.synchronize()
    assert status.t.item() == 2
    check_layers(dev, host, [prefix] * 3, keep, np.array([3, 0, 0], np.int32), "bad keep")
    assert status.intact() and all(c.intact() and k.intact() for c, k in guarded), "write outside a buffer"


def test_one_layer_equals_single_cache_call(lib):
    w = synth.WORKLOADS["s8-p1024-q33"]
    b = synth.make_batch(w)
    c1, k1 = dev_bf16(b.ckv), dev_bf16(b.kpe)
    c2, k2 = dev_bf16(b.ckv), dev_bf16(b.kpe)
    args = (dev_i32(b.parents), dev_i32(b.draft_tok), dev_i32(b.target_tok))
    o1 = lib.accept_compact(c1, k1, w.prefix, *args)
    o2 = lib.accept_compact_layers([(c2, k2)], w.prefix, *args)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(k1, k2)
    for a, b2 in zip(o1, o2):
        assert torch.equal(a, b2)


def test_grouped_layers_and_long_paths(lib):
    """Enough (stream, layer) pairs that each workgroup takes several layers, with paths from one
    row to 64 rows: a full 64-node chain moves 63 rows per layer, one layer per register round;
    short paths fit many layers in one round."""
    n_layers, s_count, q, prefix = 128, 32, 64, 10
    parents, draft, target = trees(101, s_count, q)
    parents[0] = np.arange(-1, q - 1)                   # full chain, accepted to the end
    draft[0] = np.arange(q)
    target[0] = np.arange(1, q + 1)
    parents[1], draft[1], target[1] = parents[0], draft[0], np.zeros(q, np.int32)  # root only
    host = synth.layer_caches(102, n_layers, s_count, prefix + q + 1)
    dev = upload(host)
    print(f"[layers] grouped L={n_layers} S={s_count} Q={q}", flush=True)
    keep, n_keep, _ = lib.accept_compact_layers(dev, prefix, dev_i32(parents), dev_i32(draft), dev_i32(target))
    torch.cuda.synchronize()
    rk, rn, _ = oracle.tree_accept_streams(parents, draft, target)
    assert rn[0] == q and rn[1] == 1
    assert np.array_equal(n_keep.cpu().numpy(), rn)
    check_layers(dev, host, [prefix] * s_count, rk, rn, "grouped accept")
    dev = upload(host)
    lib.compact_kv_layers(dev, prefix, dev_i32(rk), dev_i32(rn))
    torch.cuda.synchronize()
    check_layers(dev, host, [prefix] * s_count, rk, rn, "grouped compact")
