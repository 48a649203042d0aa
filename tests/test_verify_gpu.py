"""GPU parity: ddtree_verify_attn / _ex through the C ABI against the fp64 oracle.

Bars: max |err| <= 2e-2 and mean |err| <= 2e-3 on out_lat and on lse.  Sizes span several key
tiles, ragged tails, the empty prefix, one-node trees, the 64-node maximum, forced key splits,
and the five seeded workloads (the 64-stream one in its benchmark launch configuration).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, assert_close, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(lib, b, prefix, splits=None, scale=0.0):
    ql, qp, c, k = dev_bf16(b.q_lat), dev_bf16(b.q_pe), dev_bf16(b.ckv), dev_bf16(b.kpe)
    par = dev_i32(b.parents)
    if splits is None:
        out, lse = lib.verify_attn(ql, qp, c, k, prefix, par)
    else:
        out, lse = lib.verify_attn_ex(ql, qp, c, k, prefix, par, num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(lib, b, prefix, splits=None, streams=None, what=""):
    _say(f"[verify] {what} S={b.parents.shape[0]} P={prefix} Q={b.parents.shape[1]} splits={splits}")
    out, lse = run(lib, b, prefix, splits)
    idx = range(b.parents.shape[0]) if streams is None else streams
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, prefix, b.parents, streams=idx)
    return assert_close(out[list(idx)], lse[list(idx)], ro, rl, what)


SMALL = [
    (1, 0, 1), (1, 1, 1), (1, 0, 2), (2, 5, 9), (1, 63, 1), (1, 64, 64), (3, 100, 63),
    (1, 127, 2), (2, 130, 17), (1, 31, 33), (2, 200, 64), (4, 64, 1),
]


@pytest.mark.parametrize("s,p,q", SMALL)
def test_small_shapes_no_split(lib, s, p, q):
    b = synth.random_inputs(1000 + 7 * p + q, s, p, q)
    check(lib, b, p, what=f"small {s},{p},{q}")


@pytest.mark.parametrize("s,p,q,splits", [(1, 300, 9, 2), (2, 300, 33, 5), (1, 1000, 64, 16), (1, 64, 64, 2),
                                          (3, 129, 5, 3), (1, 4000, 33, 0),
                                          # odd-node workgroups dispatched partly ahead of the
                                          # pairs: 25 of them (5 splits of 2 tiles; 8 first),
                                          # and 24 (8 first)
                                          (5, 300, 9, 7), (24, 40, 3, 1),
                                          # the 64-split maximum (257 tiles: 52 splits of 5
                                          # tiles, seven merge chunks), a request above it, and
                                          # a request above the tile count (4 splits of 1 tile)
                                          (1, 8192, 17, 64), (1, 8192, 17, 1000), (2, 100, 9, 64)])
def test_forced_and_auto_splits(lib, s, p, q, splits):
    b = synth.random_inputs(2000 + p + q, s, p, q)
    check(lib, b, p, splits=splits, what=f"split {s},{p},{q}/{splits}")


@pytest.mark.parametrize("name", ["s1-p256-q9", "s8-p1024-q33", "s64-p1024-q9", "s1-p4096-q33-chain"])
def test_workloads_full(lib, name):
    w = synth.WORKLOADS[name]
    b = synth.make_batch(w)
    check(lib, b, w.prefix, splits=0, what=name)


def test_headline_workload_all_streams(lib):
    """The 64-stream, prefix-4096, q_len-33 launch exactly as the benchmark runs it (automatic
    split choice, per-XCD block renumbering, part of the odd node's workgroups dispatched ahead
    of the pairs, split merge): every one of the 64 streams is checked element by element."""
    w = synth.WORKLOADS[synth.HEADLINE]
    b = synth.make_batch(w)
    check(lib, b, w.prefix, splits=0, what=w.name)


def test_plain_entry_matches_ex(lib):
    b = synth.random_inputs(31, 3, 700, 33)
    o1, l1 = run(lib, b, 700)
    o2, l2 = run(lib, b, 700, splits=1)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_deterministic(lib):
    b = synth.random_inputs(32, 2, 500, 17)
    o1, l1 = run(lib, b, 500, splits=3)
    o2, l2 = run(lib, b, 500, splits=3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_chain_star_and_empty_prefix(lib):
    rng = np.random.default_rng(5)
    for parents, p in ((np.arange(-1, 32, dtype=np.int32), 77), (np.array([-1] + [0] * 20, np.int32), 0),
                       (np.arange(-1, 63, dtype=np.int32), 0)):
        q = len(parents)
        b = synth.random_inputs(int(rng.integers(1 << 30)), 1, p, q)
        b.parents[0] = parents
        check(lib, b, p, what=f"structured q={q} p={p}")


def test_large_score_in_late_key_takes_second_pass(lib):
    """A key far into the prefix scores ~200 log2 units above the first 32 keys: the reference
    max of the first pass is unsafe and the kernel must repeat with the exact max."""
    b = synth.random_inputs(41, 1, 900, 9)
    qp = oracle.bf16_bits_to_f64(b.q_pe)[0]
    row = 24.0 * qp[0, 0]  # rotary key aligned with head 0 of node 0: score ~ 100+ (natural log)
    b.kpe[0, 700] = synth.f32_to_bf16_bits(row.astype(np.float32))
    out, lse = run(lib, b, 900, splits=1)
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 900, b.parents)
    assert rl[0, 0, 0] > 100.0  # the planted key dominates head 0
    assert_close(out, lse, ro, rl, "late huge score")


def test_all_scores_far_below_zero(lib):
    """All scores around -300 (natural log units): probabilities only stay representable if the
    reference max tracks the true max."""
    b = synth.random_inputs(42, 2, 300, 17)
    qpe = oracle.bf16_bits_to_f64(b.q_pe)
    kpe = oracle.bf16_bits_to_f64(b.kpe)
    b.q_pe[:] = synth.f32_to_bf16_bits((0 * qpe + 8.0).astype(np.float32))
    b.kpe[:] = synth.f32_to_bf16_bits((0 * kpe - 8.0).astype(np.float32))
    out, lse = run(lib, b, 300, splits=2)
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 300, b.parents)
    assert rl.max() < -200
    assert_close(out, lse, ro, rl, "very negative scores")


def test_custom_scale(lib):
    b = synth.random_inputs(43, 1, 129, 9)
    ql, qp, c, k = dev_bf16(b.q_lat), dev_bf16(b.q_pe), dev_bf16(b.ckv), dev_bf16(b.kpe)
    out, lse = lib.verify_attn_ex(ql, qp, c, k, 129, dev_i32(b.parents), scale=0.05)
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 129, b.parents, scale=0.05)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "scale 0.05")


def test_kv_row_stride_larger_than_needed(lib):
    """kv_rows > prefix + q_len: rows past the tree block are never read (filled with NaN)."""
    b = synth.random_inputs(44, 2, 150, 9)
    rows = 150 + 9 + 13
    ckv = np.full((2, rows, 512), 0x7FC0, np.uint16)  # bf16 NaN
    kpe = np.full((2, rows, 64), 0x7FC0, np.uint16)
    ckv[:, :159] = b.ckv
    kpe[:, :159] = b.kpe
    out, lse = lib.verify_attn_ex(dev_bf16(b.q_lat), dev_bf16(b.q_pe), dev_bf16(ckv), dev_bf16(kpe), 150,
                                  dev_i32(b.parents), num_splits=2)
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 150, b.parents)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "kv_rows stride")


def test_malformed_parents_flag_status_and_stay_in_bounds(lib):
    """A bad parents[] entry sets the status bit; the walk stops there; the other streams are
    unaffected; nothing is written outside out_lat, lse, the workspace and the status word
    (guard bands of canary bytes on both sides of each), with and without key splits."""
    b = synth.random_inputs(45, 3, 100, 9)
    bad = b.parents.copy()
    bad[1, 5] = 7  # not an earlier node
    bad[1, 0] = 3  # root must be -1
    for splits in (1, 3):
        out = Guarded((3, 9, 64, 512), torch.float32)
        lse = Guarded((3, 9, 64), torch.float32)
        status = Guarded((1,), torch.int32, fill=0)
        need = lib.workspace_size(100, 9, 3, splits)
        ws = Guarded((max(need, 1),), torch.uint8) if need else None
        lib.verify_attn_ex(dev_bf16(b.q_lat), dev_bf16(b.q_pe), dev_bf16(b.ckv), dev_bf16(b.kpe), 100,
                           dev_i32(bad), out=out.t, lse=lse.t, status=status.t, num_splits=splits,
                           workspace=None if ws is None else ws.t)
        torch.cuda.synchronize()
        assert int(status.t.item()) & lib.STATUS_BAD_PARENTS
        ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 100, b.parents, streams=[0, 2])
        o, l = out.t.cpu().numpy(), lse.t.cpu().numpy()
        assert_close(o[[0, 2]], l[[0, 2]], ro, rl, "good streams beside a bad one")
        assert np.isfinite(o).all()
        for g in (out, lse, status) + ((ws,) if ws is not None else ()):
            assert g.intact(), f"write outside a buffer (splits={splits})"
        assert splits == 1 or need > 0


def test_low_side_second_pass_from_a_fully_masked_first_tile(lib):
    """The reference max of a split is taken from its first tile; when that tile is fully masked
    for a node, the reference is 0 and every visible score of the node can sit far below it.
    P = 48, q_len 64, two splits of two 32-key tiles: split 1 holds tree nodes 16..63, and its
    first tile (nodes 16..47) is fully masked for node 50, a child of the root.  All scores are
    near -295 (natural log), the node's own row near -259, so exponentials against a reference of
    0 underflow: only the exact-max second pass gives the right split partial, and since node
    50's own row dominates its softmax, that partial decides the output."""
    b = synth.random_inputs(46, 1, 48, 64)
    par = b.parents[0]
    par[50] = 0
    for j in range(51, 64):  # nobody descends from 50, so only node 50 sees its row
        if par[j] == 50:
            par[j] = 0
    qpe = np.full(b.q_pe.shape, 8.0, np.float32)
    kpe = np.full(b.kpe.shape, -8.0, np.float32)
    kpe[0, 48 + 50] = -7.0
    b.q_pe[:] = synth.f32_to_bf16_bits(qpe)
    b.kpe[:] = synth.f32_to_bf16_bits(kpe)
    assert lib.num_splits(48, 64, 1, 2) == 2
    out, lse = run(lib, b, 48, splits=2)
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 48, b.parents)
    assert -270 < rl[0, 50].max() < -250 and rl[0, 50].min() > -270  # node 50's own row dominates
    assert rl.max() < -200
    assert_close(out, lse, ro, rl, "low-side second pass")


@pytest.mark.parametrize("splits", [0, 3])
def test_many_streams(lib, splits):
    """A wide launch: 603 streams (not a multiple of the 8 per-XCD runs, so the runs differ in
    length by one), prefix 40, q_len 5 (two node pairs and the odd node).  Every output is
    finite; 40 streams spread over the batch, the first and the last included, are compared
    with the oracle element by element."""
    s_count, p, q = 603, 40, 5
    b = synth.random_inputs(47, s_count, p, q)
    idx = sorted(set(np.linspace(0, s_count - 1, 40).astype(int).tolist()))
    _say(f"[verify] many streams S={s_count} P={p} Q={q} splits={splits}")
    out, lse = run(lib, b, p, splits)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, p, b.parents, streams=idx)
    assert_close(out[idx], lse[idx], ro, rl, f"many streams, splits={splits}")


def test_zero_queries_give_the_mean_of_the_visible_rows(lib):
    """With q_lat = q_pe = 0 every visible score is 0: out is the plain mean of the visible c_kv
    rows and lse = ln(prefix + depth + 1), in closed form, checked against the oracle and against
    the closed form itself, unsplit and split."""
    b = synth.random_inputs(48, 3, 333, 17)
    b.q_lat[:] = 0
    b.q_pe[:] = 0
    depth = np.stack([oracle.tree_depths(par) for par in b.parents])
    for splits in (1, 5):
        out, lse = run(lib, b, 333, splits)
        ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 333, b.parents)
        assert_close(out, lse, ro, rl, f"zero queries, splits={splits}")
        closed = np.log(333.0 + depth + 1.0)[:, :, None].repeat(64, axis=2)
        assert np.abs(lse - closed).max() < 1e-5


def test_second_pass_in_one_node_workgroups(lib):
    """Both triggers of the exact-max second pass inside the workgroups of the odd node (whose
    two head blocks split their score chain over two waves each):
    high side -- q_len 3, a key late in the prefix scores ~100 (natural log) above the rest for
    one head of node 2 (the odd node);
    low side -- q_len 63, prefix 48, two splits of two tiles: node 62, a child of the root, finds
    split 1's first tile fully masked (reference max 0) while its visible scores sit near -259."""
    # high side
    b = synth.random_inputs(49, 2, 900, 3)
    qp = oracle.bf16_bits_to_f64(b.q_pe)[1]
    b.kpe[1, 700] = synth.f32_to_bf16_bits((24.0 * qp[2, 5]).astype(np.float32))
    for splits in (1, 4):
        out, lse = run(lib, b, 900, splits)
        ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 900, b.parents)
        assert rl[1, 2, 5] > 100.0
        assert_close(out, lse, ro, rl, f"one-node high side, splits={splits}")
    # low side
    b = synth.random_inputs(50, 1, 48, 63)
    par = b.parents[0]
    par[62] = 0
    b.q_pe[:] = synth.f32_to_bf16_bits(np.full(b.q_pe.shape, 8.0, np.float32))
    kpe = np.full(b.kpe.shape, -8.0, np.float32)
    kpe[0, 48 + 62] = -7.0
    b.kpe[:] = synth.f32_to_bf16_bits(kpe)
    assert lib.num_splits(48, 63, 1, 2) == 2
    out, lse = run(lib, b, 48, splits=2)
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 48, b.parents)
    assert -270 < rl[0, 62].min() and rl[0, 62].max() < -250 and rl.max() < -200
    assert_close(out, lse, ro, rl, "one-node low side")
