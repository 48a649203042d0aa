"""GPU parity over seeded random shapes: ddtree_verify_attn_ex and _ragged against the fp64 oracle.

Each case draws its stream count, prefix length(s), q_len (1..64) and split request (automatic or
forced, so that both merge chunk widths and both workgroup groups are exercised) from a fixed
seed, then compares every output element with the oracle at the parity bars.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _uniform_case(i):
    rng = np.random.default_rng([20261203, i])
    return (int(rng.integers(1, 6)), int(rng.integers(0, 700)), int(rng.integers(1, 65)),
            int(rng.choice([0, 0, 1, 2, 3, 4, 5, 9])))


def _ragged_case(i):
    rng = np.random.default_rng([20261204, i])
    s = int(rng.integers(2, 9))
    return s, int(rng.integers(1, 65)), [int(x) for x in rng.integers(0, 500, size=s)], int(rng.choice([0, 1, 3, 5]))


@pytest.mark.parametrize("i", range(24))
def test_random_uniform_shapes(lib, i):
    s, p, q, splits = _uniform_case(i)
    _say(f"[sweep {i}] S={s} P={p} Q={q} splits={splits}")
    b = synth.random_inputs(5000 + i, s, p, q)
    out, lse = lib.verify_attn_ex(dev_bf16(b.q_lat), dev_bf16(b.q_pe), dev_bf16(b.ckv), dev_bf16(b.kpe), p,
                                  dev_i32(b.parents), num_splits=splits)
    torch.cuda.synchronize()
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, p, b.parents)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, f"sweep {i}")


@pytest.mark.parametrize("i", range(8))
def test_random_ragged_shapes(lib, i):
    s, q, prefixes, splits = _ragged_case(i)
    _say(f"[ragged sweep {i}] S={s} Q={q} prefixes={prefixes} splits={splits}")
    parts = [synth.random_inputs(7000 + 17 * i + k, 1, max(prefixes), q) for k in range(s)]
    q_lat, q_pe = np.concatenate([x.q_lat for x in parts]), np.concatenate([x.q_pe for x in parts])
    ckv, kpe = np.concatenate([x.ckv for x in parts]), np.concatenate([x.kpe for x in parts])
    par = np.concatenate([x.parents for x in parts])
    out, lse = lib.verify_attn_ragged(dev_bf16(q_lat), dev_bf16(q_pe), dev_bf16(ckv), dev_bf16(kpe),
                                      dev_i32(np.array(prefixes)), max(prefixes), dev_i32(par), num_splits=splits)
    torch.cuda.synchronize()
    ro, rl = oracle.verify_attn_ragged(q_lat, q_pe, ckv, kpe, prefixes, par)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, f"ragged sweep {i}")
