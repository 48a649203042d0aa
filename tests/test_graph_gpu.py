"""The device step captured in one HIP graph and replayed: the calls allocate nothing and never
synchronise, so a caller can capture them.  Each replay restores the cache from a pristine copy
(a device copy, no memset), writes the tree rows, runs the verify attention (split, with a
workspace) and the fused acceptance + compaction; every replay must reproduce the eager run bit
for bit, with eager work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_bf16, dev_i32

pytestmark = pytest.mark.gpu


def test_step_replays_match_eager(lib):
    s_count, prefix, q = 8, 700, 33
    b = synth.random_inputs(61, s_count, prefix, q)
    kv, nw = synth.append_inputs(62, s_count, q)
    cos, sin = synth.rope_tables(prefix + q)
    draft = np.zeros_like(b.parents)
    target = np.zeros_like(b.parents)
    for s in range(s_count):
        path = synth.accepted_path(synth.rng_for(61, s, synth.TAG_LEAF), b.parents[s])
        draft[s] = synth.draft_tokens(synth.rng_for(61, s, synth.TAG_DRAFT_TOK), b.parents[s])
        target[s] = synth.target_tokens(synth.rng_for(61, s, synth.TAG_TARGET_TOK), b.parents[s], draft[s], path)
    dev = "cuda:0"
    ql, qp = dev_bf16(b.q_lat), dev_bf16(b.q_pe)
    ckv0, kpe0 = dev_bf16(b.ckv), dev_bf16(b.kpe)
    ckv, kpe = ckv0.clone(), kpe0.clone()
    par, dr, tg = dev_i32(b.parents), dev_i32(draft), dev_i32(target)
    kv_d, nw_d = torch.from_numpy(kv).to(dev), torch.from_numpy(nw).to(dev)
    cos_d, sin_d = torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev)
    out = torch.empty((s_count, q, 64, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((s_count, q, 64), dtype=torch.float32, device=dev)
    nbytes = lib.workspace_size(prefix, q, s_count, 4)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    keep = torch.empty((s_count, q), dtype=torch.int32, device=dev)
    n_keep = torch.empty((s_count,), dtype=torch.int32, device=dev)
    nxt = torch.empty((s_count,), dtype=torch.int32, device=dev)

    def step():
        ckv.copy_(ckv0)
        kpe.copy_(kpe0)
        lib.append_tree_kv(ckv, kpe, prefix, par, kv_d, nw_d, 1e-6, cos_d, sin_d)
        lib.verify_attn_ex(ql, qp, ckv, kpe, prefix, par, out=out, lse=lse, num_splits=4, workspace=ws)
        lib.accept_compact(ckv, kpe, prefix, par, dr, tg, keep=keep, n_keep=n_keep, next_token=nxt)

    print("[graph] eager step", flush=True)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, ckv, kpe, keep, n_keep, nxt)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        print(f"[graph] replay {r}", flush=True)
        for t in (out, lse, keep, n_keep, nxt):
            t.fill_(0)  # eager work between replays; the replay must rewrite everything
        ckv.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((out, lse, ckv, kpe, keep, n_keep, nxt), ref):
            assert torch.equal(got, want), f"replay {r}"
