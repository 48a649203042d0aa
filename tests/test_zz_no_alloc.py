"""ddtree_verify_attn_noalloc through the C ABI: the entry point for callers that cannot allocate
keeps its split partials in the library's own scratch array.  Its outputs must equal those of
ddtree_verify_attn_ex (same plan, same kernels: bitwise) and meet the oracle's bars, on two calls
in a row (the second smaller, so it runs over the first call's leftovers in the scratch), with a
plan that falls back to fit the scratch, and under HIP graph capture; a forced split count too
large for the scratch is refused before anything is launched."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, dev_bf16, dev_i32

pytestmark = pytest.mark.gpu


def inputs(seed, s, p, q):
    b = synth.random_inputs(seed, s, p, q)
    return b, (dev_bf16(b.q_lat), dev_bf16(b.q_pe), dev_bf16(b.ckv), dev_bf16(b.kpe), dev_i32(b.parents))


def both(lib, t, prefix, splits):
    ql, qp, c, k, par = t
    s, q = par.shape
    o1 = torch.full((s, q, 64, 512), float("nan"), device="cuda:0")
    l1 = torch.full((s, q, 64), float("nan"), device="cuda:0")
    o2, l2 = torch.full_like(o1, float("nan")), torch.full_like(l1, float("nan"))
    lib.verify_attn_ex(ql, qp, c, k, prefix, par, out=o1, lse=l1, num_splits=splits)
    lib.verify_attn_noalloc(ql, qp, c, k, prefix, par, out=o2, lse=l2, num_splits=splits)
    torch.cuda.synchronize()
    return o1.cpu().numpy(), l1.cpu().numpy(), o2.cpu().numpy(), l2.cpu().numpy()


def test_noalloc_matches_ex_on_two_calls_in_a_row(lib):
    # first call: 2 streams, prefix 4096, q_len 33, automatic plan (7 splits: partials in the scratch)
    print("[noalloc] S=2 P=4096 Q=33 auto", flush=True)
    assert lib.num_splits(4096, 33, 2, 0) > 1 and 0 < lib.workspace_size(4096, 33, 2, 0) <= lib.NOALLOC_SCRATCH_BYTES
    b, t = inputs(61, 2, 4096, 33)
    o1, l1, o2, l2 = both(lib, t, 4096, 0)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)) and np.array_equal(l1.view(np.uint32),
                                                                                     l2.view(np.uint32))
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 4096, b.parents)
    assert_close(o2, l2, ro, rl, "noalloc, first call")
    # second call, smaller: 1 stream, prefix 300, q_len 9, 3 forced splits
    print("[noalloc] S=1 P=300 Q=9 splits=3", flush=True)
    b, t = inputs(62, 1, 300, 9)
    o1, l1, o2, l2 = both(lib, t, 300, 3)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)) and np.array_equal(l1.view(np.uint32),
                                                                                     l2.view(np.uint32))
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 300, b.parents)
    assert_close(o2, l2, ro, rl, "noalloc, second call")


def test_noalloc_on_a_side_stream(lib):
    """The scratch address is looked up for the GPU of the stream the call runs on; a call on a
    torch side stream equals ddtree_verify_attn_ex on the same stream, bitwise."""
    print("[noalloc] S=1 P=500 Q=17 splits=4 on a side stream", flush=True)
    b, (ql, qp, c, k, par) = inputs(64, 1, 500, 17)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o1, l1 = lib.verify_attn_ex(ql, qp, c, k, 500, par, num_splits=4, stream=side)
        o2, l2 = lib.verify_attn_noalloc(ql, qp, c, k, 500, par, num_splits=4, stream=side)
    side.synchronize()
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)) and torch.equal(l1.view(torch.int32),
                                                                                    l2.view(torch.int32))
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 500, b.parents)
    assert_close(o2.cpu().numpy(), l2.cpu().numpy(), ro, rl, "noalloc, side stream")


def test_noalloc_plan_falls_back_to_fit_the_scratch(lib):
    # the automatic plan of ddtree_verify_attn_ex needs more than the scratch holds here
    print("[noalloc] S=2 P=4096 Q=64 auto (fallback plan)", flush=True)
    assert lib.workspace_size(4096, 64, 2, 0) > lib.NOALLOC_SCRATCH_BYTES
    b, (ql, qp, c, k, par) = inputs(63, 2, 4096, 64)
    out, lse = lib.verify_attn_noalloc(ql, qp, c, k, 4096, par)
    torch.cuda.synchronize()
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 4096, b.parents)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "noalloc fallback plan")


def test_noalloc_refuses_a_forced_plan_larger_than_the_scratch(lib):
    s, p, q = 64, 4096, 33
    assert lib.workspace_size(p, q, s, 64) > lib.NOALLOC_SCRATCH_BYTES
    ql = torch.empty((s, q, 64, 512), dtype=torch.bfloat16, device="cuda:0")
    qp = torch.empty((s, q, 64, 64), dtype=torch.bfloat16, device="cuda:0")
    c = torch.empty((s, p + q, 512), dtype=torch.bfloat16, device="cuda:0")
    k = torch.empty((s, p + q, 64), dtype=torch.bfloat16, device="cuda:0")
    par = torch.zeros((s, q), dtype=torch.int32, device="cuda:0")
    with pytest.raises(lib.DDTreeError) as e:
        lib.verify_attn_noalloc(ql, qp, c, k, p, par, num_splits=64)
    assert e.value.code == lib.ERR_WORKSPACE


def test_noalloc_under_graph_capture(lib):
    """Captured once, replayed three times with eager work on the same scratch in between (an
    eager no-alloc call on other inputs, outputs refilled with NaN): every replay reproduces the
    eager result bit for bit."""
    print("[noalloc] graph capture S=2 P=700 Q=9", flush=True)
    b, (ql, qp, c, k, par) = inputs(65, 2, 700, 9)
    assert lib.num_splits(700, 9, 2, 0) > 1  # the partials go through the scratch
    out = torch.empty((2, 9, 64, 512), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((2, 9, 64), dtype=torch.float32, device="cuda:0")
    lib.verify_attn_noalloc(ql, qp, c, k, 700, par, out=out, lse=lse)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    ro, rl = oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, 700, b.parents)
    assert_close(ref_o.cpu().numpy(), ref_l.cpu().numpy(), ro, rl, "noalloc eager")
    # other inputs for the eager calls between replays (they overwrite the scratch)
    _, t2 = inputs(66, 3, 300, 17)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm-up call on a side stream before capture
        lib.verify_attn_noalloc(ql, qp, c, k, 700, par, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.verify_attn_noalloc(ql, qp, c, k, 700, par, out=out, lse=lse)
    for replay in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        lib.verify_attn_noalloc(*t2[:4], 300, t2[4], num_splits=3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref_o.view(torch.int32)), replay
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), replay
