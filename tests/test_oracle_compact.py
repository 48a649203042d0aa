"""Pins for the compaction oracle.

"Race Conditions, Buffer Aliasing, and the Architecture of a Native DDTree Inference Engine",
section "The Cache Compaction Problem": the kept rows move from ``P + keep[i]`` to ``P + i``;
because the kept path is strictly increasing, ``keep[i] >= i``, so a *sequential* in-place
gather in increasing ``i`` only ever reads rows it has not yet written (and agrees with the
out-of-place gather), while a parallel or differently ordered in-place gather can read a row
after its writer has already overwritten it.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "compaction_race.json")


def forward_in_place(ckv, kpe, p, keep, n_keep):
    """Sequential in-place gather, i increasing (reads ahead, writes behind)."""
    c, k = ckv.copy(), kpe.copy()
    for s in range(c.shape[0]):
        for i in range(int(n_keep[s])):
            c[s, p + i] = c[s, p + keep[s, i]]
            k[s, p + i] = k[s, p + keep[s, i]]
    return c, k


def reverse_in_place(rows, p, keep, n):
    r = list(rows)
    for i in reversed(range(n)):
        r[p + i] = r[p + keep[i]]
    return r


def test_golden_race_example():
    g = json.load(open(GOLDEN))
    p, q, keep, n = g["prefix_len"], g["q_len"], g["keep"], g["n_keep"]
    rows = np.array(g["rows_before"], dtype=np.uint16)
    ckv = np.repeat(rows[None, :, None], 512, axis=2)
    kpe = np.repeat(rows[None, :, None], 64, axis=2)
    kp = np.full((1, q), -1, np.int32)
    kp[0, :n] = keep
    c, k = oracle.compact_kv(ckv, kpe, p, kp, np.array([n]))
    assert c[0, :, 0].tolist() == g["rows_after_gather"]
    assert (c[0] == c[0, :, :1]).all() and (k[0] == k[0, :, :1]).all()
    assert k[0, :, 0].tolist() == g["rows_after_gather"]
    # the racy order of the same in-place gather gives the wrong answer the page warns about
    assert reverse_in_place(g["rows_before"], p, keep, n) == g["rows_after_reverse_order_in_place"]
    assert g["rows_after_reverse_order_in_place"] != g["rows_after_gather"]


@pytest.mark.parametrize("seed", range(5))
def test_matches_sequential_forward_gather_on_seeded_paths(seed):
    b = synth.random_inputs(seed, streams=4, prefix=8, q_len=33, heads=1)
    c, k = oracle.compact_kv(b.ckv, b.kpe, 8, b.keep, b.n_keep)
    fc, fk = forward_in_place(b.ckv, b.kpe, 8, b.keep, b.n_keep)
    assert np.array_equal(c, fc) and np.array_equal(k, fk)
    for s in range(4):  # untouched rows stay bit-identical
        n = b.n_keep[s]
        assert np.array_equal(c[s, :8], b.ckv[s, :8])
        assert np.array_equal(c[s, 8 + n:], b.ckv[s, 8 + n:])


def test_kept_path_is_strictly_increasing_root_path():
    """keep[i] >= i holds for every path the generator emits (child index > parent index)."""
    for seed in range(20):
        b = synth.random_inputs(seed, streams=2, prefix=0, q_len=33, heads=1)
        for s in range(2):
            n = b.n_keep[s]
            kp = b.keep[s, :n]
            assert kp[0] == 0 and (np.diff(kp) > 0).all() and (kp >= np.arange(n)).all()
            for a, bb in zip(kp[:-1], kp[1:]):
                assert b.parents[s, bb] == a


def test_zero_keep_is_noop_and_input_untouched():
    b = synth.random_inputs(3, streams=2, prefix=4, q_len=9, heads=1)
    before = b.ckv.copy()
    c, k = oracle.compact_kv(b.ckv, b.kpe, 4, b.keep, np.zeros(2, np.int32))
    assert np.array_equal(c, b.ckv) and np.array_equal(k, b.kpe)
    assert np.array_equal(before, b.ckv)


@pytest.mark.parametrize("keep,n", [([0, 2, 2], 3), ([0, 3, 1], 3), ([0, 9], 2), ([-1], 1), ([0], 5)])
def test_rejects_bad_keep(keep, n):
    q = 9
    ckv = np.zeros((1, 4 + q, 512), np.uint16)
    kpe = np.zeros((1, 4 + q, 64), np.uint16)
    kp = np.full((1, q), -1, np.int32)
    kp[0, :len(keep)] = keep
    with pytest.raises(ValueError):
        oracle.compact_kv(ckv, kpe, 4, kp, np.array([n]))
