"""GPU parity for per-stream (ragged) prefix lengths through the C ABI:
ddtree_verify_attn_ragged against the per-stream oracle (tolerance bars), ddtree_compact_kv_ragged
and ddtree_accept_compact_ragged bit-exact, the device-side prefix advance, and a two-step
verify -> accept/compact -> verify loop with the prefixes kept on the device."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, assert_close, dev_bf16, dev_i32, host_bits

pytestmark = pytest.mark.gpu


def ragged_batch(seed, prefixes, q, heads=synth.HEADS):
    """Inputs for streams with the given prefixes; the cache holds max(prefixes) + q rows."""
    b = synth.random_inputs(seed, len(prefixes), max(prefixes), q, heads=heads)
    return b


def run_ragged(lib, b, prefixes, max_prefix, splits=0, status=None):
    out, lse = lib.verify_attn_ragged(dev_bf16(b.q_lat), dev_bf16(b.q_pe), dev_bf16(b.ckv), dev_bf16(b.kpe),
                                      dev_i32(np.array(prefixes)), max_prefix, dev_i32(b.parents),
                                      num_splits=splits, status=status)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("q", [9, 33])
@pytest.mark.parametrize("splits", [0, 1, 4, 8])
def test_ragged_verify(lib, q, splits):
    prefixes = [0, 1, 31, 32, 33, 100, 640, 1024]
    print(f"[ragged] q={q} splits={splits} prefixes={prefixes}", flush=True)
    b = ragged_batch(100 + q, prefixes, q)
    out, lse = run_ragged(lib, b, prefixes, max(prefixes), splits)
    ro, rl = oracle.verify_attn_ragged(b.q_lat, b.q_pe, b.ckv, b.kpe, prefixes, b.parents)
    assert_close(out, lse, ro, rl, f"ragged q={q} splits={splits}")


@pytest.mark.parametrize("s_count", [13, 27, 64, 65])
def test_ragged_stream_counts(lib, s_count):
    """Ragged launches of up to 64 streams place the streams on the XCDs by prefix length (a
    ranking with ties, dealt in snake order with a partial last round when the count is not a
    multiple of 8); above 64 they keep the plain order.  Every stream must be computed exactly
    once: the outputs start as NaN and every stream is checked against the oracle."""
    q = 9
    rng = np.random.default_rng(300 + s_count)
    prefixes = rng.integers(0, 260, size=s_count)
    prefixes[::5] = 128  # ties
    prefixes = [int(x) for x in prefixes]
    print(f"[ragged] {s_count} streams, prefixes in [0, 260)", flush=True)
    b = ragged_batch(400 + s_count, prefixes, q)
    out = torch.full((s_count, q, synth.HEADS, 512), float("nan"), dtype=torch.float32, device="cuda:0")
    lse = torch.full((s_count, q, synth.HEADS), float("nan"), dtype=torch.float32, device="cuda:0")
    lib.verify_attn_ragged(dev_bf16(b.q_lat), dev_bf16(b.q_pe), dev_bf16(b.ckv), dev_bf16(b.kpe),
                           dev_i32(np.array(prefixes)), max(prefixes), dev_i32(b.parents), out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.verify_attn_ragged(b.q_lat, b.q_pe, b.ckv, b.kpe, prefixes, b.parents)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, f"ragged {s_count} streams")


def test_equal_prefixes_match_uniform_call_bitwise(lib):
    p, q = 700, 33
    b = synth.random_inputs(8, 4, p, q)
    args = [dev_bf16(b.q_lat), dev_bf16(b.q_pe), dev_bf16(b.ckv), dev_bf16(b.kpe)]
    for splits in (0, 5):
        o1, l1 = lib.verify_attn_ex(*args, p, dev_i32(b.parents), num_splits=splits)
        o2, l2 = lib.verify_attn_ragged(*args, dev_i32(np.full(4, p)), p, dev_i32(b.parents), num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_long_prefixes(lib):
    prefixes = [32768, 20000]
    q = 33
    print(f"[ragged] long prefixes {prefixes}", flush=True)
    b = ragged_batch(9, prefixes, q)
    out, lse = run_ragged(lib, b, prefixes, max(prefixes))
    ro, rl = oracle.verify_attn_ragged(b.q_lat, b.q_pe, b.ckv, b.kpe, prefixes, b.parents)
    assert_close(out, lse, ro, rl, "long prefixes")


def test_bad_prefixes_are_poisoned_and_flagged(lib):
    """Out-of-range prefix entries poison their streams and set the status bit; the neighbours
    are right; nothing is written outside out_lat, lse, the workspace and the status word (guard
    bands of canary bytes around each), with the automatic plan and with forced splits."""
    prefixes = [5, -1, 2000, 7]
    q, max_p = 9, 1024
    b = ragged_batch(10, [5, 0, max_p, 7], q)
    for splits in (0, 4):
        out = Guarded((4, q, 64, 512), torch.float32)
        lse = Guarded((4, q, 64), torch.float32)
        status = Guarded((1,), torch.int32, fill=0)
        need = lib.workspace_size(max_p, q, 4, splits)
        ws = Guarded((need,), torch.uint8) if need else None
        lib.verify_attn_ragged(dev_bf16(b.q_lat), dev_bf16(b.q_pe), dev_bf16(b.ckv), dev_bf16(b.kpe),
                               dev_i32(np.array(prefixes)), max_p, dev_i32(b.parents), out=out.t, lse=lse.t,
                               num_splits=splits, workspace=None if ws is None else ws.t, status=status.t)
        torch.cuda.synchronize()
        o, l = out.t.cpu().numpy(), lse.t.cpu().numpy()
        assert status.t.item() & 4
        assert np.isnan(o[1]).all() and np.isnan(l[1]).all()
        assert np.isnan(o[2]).all() and np.isnan(l[2]).all()
        ro, rl = oracle.verify_attn_ragged(b.q_lat[[0, 3]], b.q_pe[[0, 3]], b.ckv[[0, 3]], b.kpe[[0, 3]], [5, 7],
                                           b.parents[[0, 3]])
        assert_close(o[[0, 3]], l[[0, 3]], ro, rl, "good streams beside bad ones")
        for g in (out, lse, status) + ((ws,) if ws is not None else ()):
            assert g.intact(), f"write outside a buffer (splits={splits})"
        assert splits == 0 or need > 0


def test_compact_ragged(lib):
    q = 33
    prefixes = [0, 17, 300, 64]
    b = ragged_batch(11, prefixes, q)
    keep = np.full((4, q), -1, np.int32)
    n_keep = np.zeros(4, np.int32)
    for s in range(4):
        path = synth.accepted_path(synth.rng_for(11, s, synth.TAG_LEAF), b.parents[s])
        keep[s, : len(path)] = path
        n_keep[s] = len(path)
    c, k = dev_bf16(b.ckv), dev_bf16(b.kpe)
    lib.compact_kv_ragged(c, k, dev_i32(np.array(prefixes)), dev_i32(keep), dev_i32(n_keep))
    torch.cuda.synchronize()
    rc, rk = oracle.compact_kv_ragged(b.ckv, b.kpe, prefixes, keep, n_keep)
    assert np.array_equal(host_bits(c), rc) and np.array_equal(host_bits(k), rk)


def accept_tokens(seed, parents):
    draft = np.zeros_like(parents)
    target = np.zeros_like(parents)
    for s in range(parents.shape[0]):
        path = synth.accepted_path(synth.rng_for(seed, s, synth.TAG_LEAF), parents[s])
        draft[s] = synth.draft_tokens(synth.rng_for(seed, s, synth.TAG_DRAFT_TOK), parents[s])
        target[s] = synth.target_tokens(synth.rng_for(seed, s, synth.TAG_TARGET_TOK), parents[s], draft[s], path)
    return draft, target


def test_accept_compact_ragged_advances_prefixes(lib):
    q = 33
    prefixes = np.array([0, 17, 300, 64, 10], np.int32)
    rows = 300 + q
    b = synth.random_inputs(12, 5, 300, q)
    draft, target = accept_tokens(12, b.parents)
    pl = dev_i32(prefixes.copy())
    pl_host = prefixes.copy()
    pl_host[4] = rows  # tree block past the end: flagged, nothing moves
    pl = dev_i32(pl_host)
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    c, k = dev_bf16(b.ckv), dev_bf16(b.kpe)
    keep, n_keep, nxt = lib.accept_compact_ragged(c, k, pl, dev_i32(b.parents), dev_i32(draft), dev_i32(target),
                                                  status=status)
    torch.cuda.synchronize()
    rk, rn, rx = oracle.tree_accept_streams(b.parents, draft, target)
    assert np.array_equal(n_keep.cpu().numpy(), rn) and np.array_equal(nxt.cpu().numpy(), rx)
    assert status.item() & 4
    rn_moved = rn.copy()
    rn_moved[4] = 0
    rc, rkp = oracle.compact_kv_ragged(b.ckv, b.kpe, pl_host, rk, rn_moved)
    assert np.array_equal(host_bits(c), rc) and np.array_equal(host_bits(k), rkp)
    expect = pl_host + rn_moved
    assert np.array_equal(pl.cpu().numpy(), expect)


def test_device_side_loop(lib):
    """verify -> accept/compact (prefixes advanced on the device) -> verify again at the new
    prefixes, with only new tree rows written by the host in between."""
    q, s_count, p0 = 9, 6, 200
    rows = p0 + 2 * q + 16
    b1 = synth.random_inputs(13, s_count, rows - q, q)  # cache of `rows` rows
    prefixes = np.array([200, 150, 0, 77, 199, 31], np.int32)
    draft, target = accept_tokens(13, b1.parents)
    ckv_h, kpe_h = b1.ckv.copy(), b1.kpe.copy()
    c, k = dev_bf16(ckv_h), dev_bf16(kpe_h)
    pl = dev_i32(prefixes)
    par = dev_i32(b1.parents)
    out1, lse1 = lib.verify_attn_ragged(dev_bf16(b1.q_lat), dev_bf16(b1.q_pe), c, k, pl, rows - q, par)
    lib.accept_compact_ragged(c, k, pl, par, dev_i32(draft), dev_i32(target))
    torch.cuda.synchronize()
    ro1, rl1 = oracle.verify_attn_ragged(b1.q_lat, b1.q_pe, ckv_h, kpe_h, prefixes, b1.parents)
    assert_close(out1.cpu().numpy(), lse1.cpu().numpy(), ro1, rl1, "loop step 1")
    rk, rn, _ = oracle.tree_accept_streams(b1.parents, draft, target)
    ckv_h, kpe_h = oracle.compact_kv_ragged(ckv_h, kpe_h, prefixes, rk, rn)
    prefixes2 = prefixes + rn
    assert np.array_equal(pl.cpu().numpy(), prefixes2)
    # the next tree: new rows at [prefix2, prefix2 + q) from a fresh draw, new queries and parents
    b2 = synth.random_inputs(14, s_count, rows - q, q)
    for s in range(s_count):
        ckv_h[s, prefixes2[s]: prefixes2[s] + q] = b2.ckv[s, :q]
        kpe_h[s, prefixes2[s]: prefixes2[s] + q] = b2.kpe[s, :q]
    c.copy_(dev_bf16(ckv_h))
    k.copy_(dev_bf16(kpe_h))
    out2, lse2 = lib.verify_attn_ragged(dev_bf16(b2.q_lat), dev_bf16(b2.q_pe), c, k, pl, rows - q,
                                        dev_i32(b2.parents))
    torch.cuda.synchronize()
    ro2, rl2 = oracle.verify_attn_ragged(b2.q_lat, b2.q_pe, ckv_h, kpe_h, prefixes2, b2.parents)
    assert_close(out2.cpu().numpy(), lse2.cpu().numpy(), ro2, rl2, "loop step 2")
