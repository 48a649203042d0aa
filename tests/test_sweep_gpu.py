"""GPU parity over seeded random shapes: ddtree_verify_attn_ex and _ragged against the fp64 oracle.

Each case draws its stream count, prefix length(s), q_len (1..64) and split request (automatic or
forced, so that both merge chunk widths and both workgroup groups are exercised) from a fixed
seed, then compares every output element with the oracle at the parity bars.  A third family adds
cache strides past the tree block and explicit softmax scales.
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


def _padded_case(i):
    rng = np.random.default_rng([20261205, i])
    return (int(rng.integers(1, 13)), int(rng.integers(0, 3001)), int(rng.integers(1, 65)),
            int(rng.choice([0, 0, 1, 2, 3, 4, 6, 8, 13, 17, 33, 64])), int(rng.choice([1, 31, 200])),
            float(rng.choice([0.0, 0.03, 0.11])))


@pytest.mark.parametrize("i", range(16))
def test_random_padded_scaled_shapes(lib, i):
    """Longer prefixes, a cache stride past the tree block (the rows between are bf16 NaN, which
    no call may read) and explicit softmax scales; the no-alloc entry point, where the plan fits
    its scratch, bitwise equal to the workspace one."""
    s, p, q, splits, pad, scale = _padded_case(i)
    _say(f"[padded sweep {i}] S={s} P={p} Q={q} splits={splits} pad={pad} scale={scale}")
    b = synth.random_inputs(9000 + i, s, p, q)
    rows = p + q
    ckv = np.full((s, rows + pad, 512), 0x7FC0, np.uint16)
    kpe = np.full((s, rows + pad, 64), 0x7FC0, np.uint16)
    ckv[:, :rows], kpe[:, :rows] = b.ckv, b.kpe
    args = (dev_bf16(b.q_lat), dev_bf16(b.q_pe), dev_bf16(ckv), dev_bf16(kpe), p, dev_i32(b.parents))
    out, lse = lib.verify_attn_ex(*args, num_splits=splits, scale=scale)
    if lib.workspace_size(p, q, s, splits) <= lib.NOALLOC_SCRATCH_BYTES:
        o2, l2 = lib.verify_attn_noalloc(*args, num_splits=splits, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o2.view(torch.int32), out.view(torch.int32))
        assert torch.equal(l2.view(torch.int32), lse.view(torch.int32))
    torch.cuda.synchronize()
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, p, b.parents,
                                **({"scale": scale} if scale else {}))
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, f"padded sweep {i}")
