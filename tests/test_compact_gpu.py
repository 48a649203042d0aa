"""GPU parity: ddtree_compact_kv through the C ABI, bit-exact on the whole cache buffers
against the out-of-place oracle gather (rows outside the kept range must be untouched)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, dev_bf16, dev_i32, guarded_bf16, guarded_i32, host_bits

pytestmark = pytest.mark.gpu


def run_compact(lib, ckv_bits, kpe_bits, prefix, keep, n_keep, status=None):
    c, k = dev_bf16(ckv_bits), dev_bf16(kpe_bits)
    lib.compact_kv(c, k, prefix, dev_i32(keep), dev_i32(n_keep), status=status)
    torch.cuda.synchronize()
    return host_bits(c), host_bits(k)


def check(lib, ckv, kpe, prefix, keep, n_keep, what=""):
    print(f"[compact] {what} S={ckv.shape[0]} rows={ckv.shape[1]} P={prefix}", flush=True)
    gc, gk = run_compact(lib, ckv, kpe, prefix, keep, n_keep)
    rc, rk = oracle.compact_kv(ckv, kpe, prefix, keep, n_keep)
    assert np.array_equal(gc, rc), what
    assert np.array_equal(gk, rk), what


def test_headline_workload_accepted_paths(lib):
    w = synth.WORKLOADS[synth.HEADLINE]
    b = synth.make_batch(w)
    assert (b.n_keep >= 1).all() and (b.n_keep <= 16).all()
    check(lib, b.ckv, b.kpe, w.prefix, b.keep, b.n_keep, w.name)


@pytest.mark.parametrize("name", ["s1-p256-q9", "s8-p1024-q33", "s64-p1024-q9", "s1-p4096-q33-chain"])
def test_workload_paths(lib, name):
    w = synth.WORKLOADS[name]
    b = synth.make_batch(w)
    check(lib, b.ckv, b.kpe, w.prefix, b.keep, b.n_keep, name)


def _cache(seed, s, rows):
    rng = synth.rng_for(seed, 0, 9)
    return synth.bf16_normal(rng, (s, rows, 512)), synth.bf16_normal(rng, (s, rows, 64))


@pytest.mark.parametrize("n", [0, 1, 2, 16, 33, 64])
def test_racy_shift_patterns(lib, n):
    """keep = [0, 2, 3, 4, ...]: every reader j >= 1 reads the row its neighbour j+1 writes."""
    q = 65 if n == 64 else 64
    prefix = 37
    ckv, kpe = _cache(10 + n, 3, prefix + q)
    keep = np.full((3, q), -1, np.int32)
    n_keep = np.zeros(3, np.int32)
    for s in range(3):
        seq = [0] + list(range(2, n + 1)) if n > 0 else []
        if s == 1:
            seq = list(range(q - n, q))  # the tail of the block (maximum distance)
        if s == 2:
            seq = list(range(n))  # identity: nothing moves
        keep[s, :len(seq)] = seq
        n_keep[s] = len(seq)
    for rep in range(20):  # different schedules, same answer every time
        check(lib, ckv, kpe, prefix, keep, n_keep, f"racy n={n} rep={rep}")


def test_random_increasing_subsets(lib):
    rng = np.random.default_rng(3)
    for trial in range(10):
        s, q, prefix = 8, int(rng.integers(1, 65)), int(rng.integers(0, 300))
        ckv, kpe = _cache(100 + trial, s, prefix + q + int(rng.integers(0, 5)))
        keep = np.full((s, q), -1, np.int32)
        n_keep = np.zeros(s, np.int32)
        for st in range(s):
            n = int(rng.integers(0, q + 1))
            sel = np.sort(rng.choice(q, size=n, replace=False)).astype(np.int32)
            keep[st, :n] = sel
            n_keep[st] = n
        check(lib, ckv, kpe, prefix, keep, n_keep, f"random trial {trial}")


def test_invalid_keep_is_flagged_and_stream_untouched(lib):
    """Invalid keep rows are flagged and their streams left untouched; nothing is written outside
    the cache buffers or the status word, and keep / n_keep are only read (guard bands of canary
    bytes on both sides of every buffer)."""
    ckv, kpe = _cache(7, 4, 50 + 9)
    keep = np.tile(np.arange(9, dtype=np.int32), (4, 1))
    keep[0, :3] = [0, 3, 4]   # stream 0: valid
    n_keep = np.array([3, 3, 3, 10], np.int32)
    keep[1, :3] = [0, 4, 4]   # not strictly increasing
    keep[2, :3] = [0, 2, 99]  # beyond the cache
    # stream 3: n_keep larger than the keep row
    c, k = guarded_bf16(ckv), guarded_bf16(kpe)
    gkeep, gn = guarded_i32(keep), guarded_i32(n_keep)
    status = Guarded((1,), torch.int32, fill=0)
    lib.compact_kv(c.t, k.t, 50, gkeep.t, gn.t, status=status.t)
    torch.cuda.synchronize()
    gc, gk = host_bits(c.t), host_bits(k.t)
    assert int(status.t.item()) & lib.STATUS_BAD_KEEP
    rc, rk = oracle.compact_kv(ckv[:1], kpe[:1], 50, keep[:1], n_keep[:1])
    assert np.array_equal(gc[0], rc[0]) and np.array_equal(gk[0], rk[0])
    for s in (1, 2, 3):
        assert np.array_equal(gc[s], ckv[s]) and np.array_equal(gk[s], kpe[s])
    assert np.array_equal(gkeep.t.cpu().numpy(), keep) and np.array_equal(gn.t.cpu().numpy(), n_keep)
    for g in (c, k, gkeep, gn, status):
        assert g.intact(), "write outside a buffer"
