"""Pins for the per-stream-prefix oracles (CPU only): each stream must equal the uniform oracle run
alone on a cache cut to exactly that stream's rows, and equal prefixes must reproduce the uniform
batch result."""
import numpy as np

import oracle
import synth


def test_ragged_verify_is_per_stream_uniform():
    q, s_count = 9, 4
    prefixes = [0, 3, 17, 40]
    rows = max(prefixes) + q
    b = synth.random_inputs(5, s_count, max(prefixes), q, heads=2)
    out, lse = oracle.verify_attn_ragged(b.q_lat, b.q_pe, b.ckv, b.kpe, prefixes, b.parents)
    for s, p in enumerate(prefixes):
        ref_o, ref_l = oracle.verify_attn(b.q_lat[s:s + 1], b.q_pe[s:s + 1], b.ckv[s:s + 1, : p + q],
                                          b.kpe[s:s + 1, : p + q], p, b.parents[s:s + 1])
        assert np.array_equal(out[s], ref_o[0]) and np.array_equal(lse[s], ref_l[0])
    assert rows == b.ckv.shape[1]


def test_ragged_equal_prefixes_match_uniform():
    b = synth.random_inputs(6, 3, 12, 5, heads=2)
    o1, l1 = oracle.verify_attn_ragged(b.q_lat, b.q_pe, b.ckv, b.kpe, [12, 12, 12], b.parents)
    o2, l2 = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 12, b.parents)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_ragged_compaction_is_per_stream():
    rng = np.random.default_rng(0)
    ckv = rng.integers(0, 65535, size=(3, 30, 512), dtype=np.uint16)
    kpe = rng.integers(0, 65535, size=(3, 30, 64), dtype=np.uint16)
    prefixes = [0, 7, 20]
    keep = np.array([[0, 2, 5, -1], [0, 1, 3, 4], [0, 3, -1, -1]], np.int32)
    n_keep = np.array([3, 4, 2], np.int32)
    c, k = oracle.compact_kv_ragged(ckv, kpe, prefixes, keep, n_keep)
    for s, p in enumerate(prefixes):
        exp_c = ckv[s].copy()
        exp_k = kpe[s].copy()
        for i in range(n_keep[s]):
            exp_c[p + i] = ckv[s, p + keep[s, i]]
            exp_k[p + i] = kpe[s, p + keep[s, i]]
        assert np.array_equal(c[s], exp_c) and np.array_equal(k[s], exp_k)
