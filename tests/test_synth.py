"""The seeded generator: determinism, tree validity, bf16 rounding (checked against torch)."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0],
                                 dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(x), ref)


def test_deterministic():
    a = synth.random_inputs(5, streams=2, prefix=16, q_len=9, heads=4)
    b = synth.random_inputs(5, streams=2, prefix=16, q_len=9, heads=4)
    for f in ("q_lat", "q_pe", "ckv", "kpe", "parents", "keep", "n_keep"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = synth.random_inputs(6, streams=2, prefix=16, q_len=9, heads=4)
    assert not np.array_equal(a.ckv, c.ckv)


def test_stream_prefix_regenerates_alone():
    w = synth.WORKLOADS["s8-p1024-q33"]
    full = synth.make_batch(w, streams=3)
    one = synth.make_batch(w, streams=1)
    assert np.array_equal(full.ckv[0], one.ckv[0])
    assert np.array_equal(full.parents[0], one.parents[0])


def _depth(parents):
    d = np.zeros(len(parents), int)
    for i in range(1, len(parents)):
        d[i] = d[parents[i]] + 1
    return d


def test_trees_valid_and_depth_capped():
    for tree in ("uniform", "chain70"):
        for seed in range(200):
            p = synth.sample_parents(synth.rng_for(seed, 0, synth.TAG_PARENTS), 64, tree)
            assert p[0] == -1
            assert all(0 <= p[i] < i for i in range(1, 64))
            assert _depth(p).max() <= synth.MAX_DEPTH


def test_chain_heavy_trees_are_deeper():
    du = np.mean([_depth(synth.sample_parents(synth.rng_for(s, 0, 4), 33, "uniform")).mean()
                  for s in range(200)])
    dc = np.mean([_depth(synth.sample_parents(synth.rng_for(s, 0, 4), 33, "chain70")).mean()
                  for s in range(200)])
    assert dc > 2 * du


def test_workload_shapes():
    w = synth.WORKLOADS["s1-p256-q9"]
    b = synth.make_batch(w)
    assert b.q_lat.shape == (1, 9, 64, 512) and b.q_pe.shape == (1, 9, 64, 64)
    assert b.ckv.shape == (1, 265, 512) and b.kpe.shape == (1, 265, 64)
    assert b.q_lat.dtype == np.uint16 and b.parents.dtype == np.int32
