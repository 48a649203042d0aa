"""GPU parity: ddtree_append_tree_kv through the C ABI against the fp64 append oracle.

Rows outside each tree block must stay bit-identical.  Inside it, the kernel sums and rotates in
fp32 and rounds once to bf16, while the oracle rounds the exact result; so each stored value must
lie within one bf16 spacing of the exact value, plus, for the rotary part, the fp32 error bound of
its two-product sum (which matters only where the two products nearly cancel), and the bit
patterns must agree with the oracle's for all but a small fraction of values."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, dev_bf16, dev_i32, guarded_bf16, host_bits

pytestmark = pytest.mark.gpu

F32_EPS = 2.0 ** -24
MAX_MISMATCH = 0.005  # fp32 relative error ~1e-6 vs bf16 spacing ~4e-3: flips are rare


def spacing(v):
    """bf16 spacing at |v| (normal range)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def check_block(got_c, got_k, kv, w, eps, cos, sin, p, parents, what):
    q = kv.shape[0]
    depth = oracle.tree_depths(parents)
    ref_c, ref_k = oracle.tree_rows(kv, w, eps, cos, sin, p, parents)
    ex_c = np.stack([oracle.rms_norm(kv[i, :512], w, eps) for i in range(q)])
    ex_k = np.stack([oracle.rope_neox(kv[i, 512:], cos[p + depth[i]], sin[p + depth[i]]) for i in range(q)])
    mag_k = np.stack([np.abs(kv[i, 512:].astype(np.float64)) * np.concatenate(
        [np.abs(cos[p + depth[i]]), np.abs(cos[p + depth[i]])]) + np.abs(np.roll(kv[i, 512:], 32).astype(np.float64))
        * np.concatenate([np.abs(sin[p + depth[i]]), np.abs(sin[p + depth[i]])]) for i in range(q)])
    gc = oracle.bf16_bits_to_f64(got_c)
    gk = oracle.bf16_bits_to_f64(got_k)
    assert (np.abs(gc - ex_c) <= spacing(ex_c) + 8 * F32_EPS * np.abs(ex_c)).all(), what
    assert (np.abs(gk - ex_k) <= spacing(ex_k) + 8 * F32_EPS * mag_k).all(), what
    mism = (np.count_nonzero(got_c != ref_c) + np.count_nonzero(got_k != ref_k)) / (got_c.size + got_k.size)
    assert mism <= MAX_MISMATCH, (what, mism)
    return mism


def run(lib, s_count, q, prefixes, rows, seed, tree="uniform", rope_rows=None, ragged=True, parents=None):
    kv, w = synth.append_inputs(seed, s_count, q)
    if parents is None:
        parents = np.stack([synth.sample_parents(synth.rng_for(seed, s, synth.TAG_PARENTS), q, tree)
                            for s in range(s_count)])
    rope_rows = rope_rows or (max(prefixes) + q)
    cos, sin = synth.rope_tables(rope_rows)
    cache = synth.layer_caches(seed, 1, s_count, rows)[0]
    # guard bands of canary bytes around the cache and the status word: nothing may be written
    # outside them, whatever the streams' prefixes or trees
    gc_, gk_ = guarded_bf16(cache[0]), guarded_bf16(cache[1])
    status = Guarded((1,), torch.int32, fill=0)
    prefix_arg = dev_i32(np.array(prefixes)) if ragged else int(prefixes[0])
    lib.append_tree_kv(gc_.t, gk_.t, prefix_arg, dev_i32(parents), torch.from_numpy(kv).cuda(),
                       torch.from_numpy(w).cuda(), 1e-6, torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda(),
                       status=status.t)
    torch.cuda.synchronize()
    assert gc_.intact() and gk_.intact() and status.intact(), "write outside a buffer"
    return host_bits(gc_.t), host_bits(gk_.t), cache, kv, w, cos, sin, parents, status.t.item()


@pytest.mark.parametrize("q", [1, 9, 33, 64])
def test_append_matches_oracle(lib, q):
    prefixes = [0, 5, 1000, 4096 - q, 77, 3, 640, 31]
    rows = 4096 + 3
    print(f"[append] q={q} prefixes={prefixes}", flush=True)
    gc, gk, (c0, k0), kv, w, cos, sin, parents, st = run(lib, 8, q, prefixes, rows, 200 + q)
    assert st == 0
    for s, p in enumerate(prefixes):
        outside = np.ones(rows, bool)
        outside[p:p + q] = False
        assert np.array_equal(gc[s, outside], c0[s, outside]) and np.array_equal(gk[s, outside], k0[s, outside])
        check_block(gc[s, p:p + q], gk[s, p:p + q], kv[s], w, 1e-6, cos, sin, p, parents[s], f"q={q} s={s}")


def test_uniform_prefix_and_deep_chains(lib):
    q, p = 64, 200
    parents = np.stack([np.arange(-1, q - 1), np.r_[-1, np.zeros(q - 1)], np.arange(-1, q - 1)]).astype(np.int32)
    print("[append] chains and a star, one prefix", flush=True)
    gc, gk, _, kv, w, cos, sin, parents, st = run(lib, 3, q, [p] * 3, p + q, 301, ragged=False, parents=parents,
                                                  rope_rows=p + q)
    assert st == 0
    for s in range(3):
        check_block(gc[s, p:], gk[s, p:], kv[s], w, 1e-6, cos, sin, p, parents[s], f"chain/star s={s}")


def test_bad_streams_untouched_and_flagged(lib):
    q = 9
    parents = np.stack([synth.sample_parents(synth.rng_for(5, s, synth.TAG_PARENTS), q) for s in range(4)])
    parents[1, 4] = 6                        # not an earlier node
    prefixes = [10, 10, 50, 60]              # streams 2 and 3: block past the cache end (55 rows)
    rows = 55
    print("[append] malformed / out-of-range streams", flush=True)
    gc, gk, (c0, k0), kv, w, cos, sin, _, st = run(lib, 4, q, prefixes, rows, 6, rope_rows=64, parents=parents)
    assert st == 1 | 4
    for s in (1, 2, 3):
        assert np.array_equal(gc[s], c0[s]) and np.array_equal(gk[s], k0[s])
    check_block(gc[0, 10:19], gk[0, 10:19], kv[0], w, 1e-6, cos, sin, 10, parents[0], "good stream")
    chain = np.tile(np.arange(-1, q - 1, dtype=np.int32), (2, 1))
    gc, gk, (c0, k0), *_, st = run(lib, 2, q, [40, 56], 80, 7, rope_rows=64, parents=chain)
    assert st == 8                           # stream 1: positions 56 .. 64, the table has 64 rows
    assert np.array_equal(gc[1], c0[1]) and np.array_equal(gk[1], k0[1])
    assert not np.array_equal(gc[0], c0[0])
