"""Benchmark: tree-verify MLA-absorb attention, greedy acceptance and KV compaction on one MI355X.

One step = one pass of the whole hot path over one batch: ``ddtree_verify_attn_ex`` (64 heads,
latent 512 + rope 64, tree mask from parents[]) followed by ``ddtree_accept_compact`` (greedy
acceptance of each stream's tree against synthetic target tokens, then the in-place compaction
of the accepted root-to-leaf path, one launch).  Inputs are seeded synthetic bf16 ~ N(0,1) and
token ids (no dataset is involved) and are resident in HBM before the timed region starts.

Prints one JSON line.  ``value`` is TFLOP/s of the verify attention counted over visible
(query, key) pairs only, divided by the whole step time (verify + accept + compaction).  The
``detail`` object also carries per-call times of ``ddtree_tree_accept`` over the stream and
budget grid the pages report, of the fused call, of ``ddtree_compact_kv`` alone, and of
``ddtree_tree_build`` (depth 15, top-8) for 1/8/64 requests and budgets 8/32/63, and the verify
throughput against the peak scaled to the shader clock that amdsmi reads during a few seconds of
back-to-back calls (``detail.sustained``).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify-attn us/call & TFLOP/s (64 heads, q_len 33, prefix 4096); % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "tree_verify_mla_absorb_amd", "csrc", "verify_attn.hip")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "verify_attn_s64_p4096_q33_pmc.txt")


def kernel_sha() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def visible_pairs(parents: np.ndarray, prefix: int) -> int:
    """Sum over streams and nodes of the number of visible keys: prefix + depth + 1."""
    total = 0
    for row in parents:
        depth = np.zeros(len(row), np.int64)
        for i in range(1, len(row)):
            depth[i] = depth[row[i]] + 1
        total += int((prefix + depth + 1).sum())
    return total


def algorithmic_bytes(w, streams: int) -> int:
    """KV read once per stream + Q + out + lse + parents."""
    s, q, l, h = streams, w.q_len, w.kv_rows, w.heads
    return (s * l * (512 + 64) * 2 + s * q * h * (512 + 64) * 2 + s * q * h * 512 * 4 + s * q * h * 4
            + s * q * 4)


def read_traffic():
    """HBM bytes per verify launch from the committed rocprofv3 counter summary, when that
    summary was taken on the current kernel source (else None)."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_bytes or m_sha.group(1) != kernel_sha():
        return None
    return float(m_bytes.group(1))


def cpu_baseline(w, b, budget_s: float = 12.0):
    """The fp64 oracle, as it stands, on the streams of the same workload (the batch ``b`` the GPU
    run uses), one stream at a time in order and around again until about ``budget_s`` seconds
    of CPU work; scaled to TFLOP/s of algorithmic work."""
    import oracle

    cores = oracle_threads()
    t_total, done, flops = 0.0, 0, 0.0
    while t_total < budget_s:
        s = done % w.streams
        t0 = time.perf_counter()
        oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, w.prefix, b.parents, streams=[s])
        t_total += time.perf_counter() - t0
        flops += 2.0 * w.heads * (576 + 512) * visible_pairs(b.parents[s:s + 1], w.prefix)
        done += 1
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 oracle, {done} stream evaluations over streams 0..{min(done, w.streams) - 1} "
                      f"of {w.streams} of workload {w.name} ({t_total:.1f} s)"}


def oracle_threads() -> int:
    """Threads the oracle's BLAS runs on (the host cores it uses)."""
    try:
        from threadpoolctl import threadpool_info
        return max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def oracle_seconds_per_call(w, b, min_s: float = 1.0) -> dict:
    """The fp64 oracle, as it stands, on every stream of workload ``w`` (batch ``b``) in order,
    repeated until at least ``min_s`` seconds: seconds for one whole call (all streams)."""
    import oracle
    t_total, done = 0.0, 0
    while t_total < min_s or done < w.streams:
        s = done % w.streams
        t0 = time.perf_counter()
        oracle.verify_attn(b.q_lat, b.q_pe, b.ckv, b.kpe, w.prefix, b.parents, streams=[s])
        t_total += time.perf_counter() - t0
        done += 1
    return {"oracle_s_per_call": round(t_total / done * w.streams, 5), "oracle_cores": oracle_threads(),
            "oracle_stream_evaluations": done}


def host_info() -> dict:
    """Versions and machine identity for the line: git HEAD (when the tree is a checkout), a hash
    of the library sources, the ROCm and HIP versions, the GPU and the host CPU."""
    import subprocess
    info = {}
    try:
        info["git_head"] = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], stdout=subprocess.PIPE,
                                          stderr=subprocess.DEVNULL, text=True, timeout=10).stdout.strip() or None
    except Exception:
        info["git_head"] = None
    h = hashlib.sha256()
    for sub in ("include", os.path.join("tree_verify_mla_absorb_amd", "csrc")):
        d = os.path.join(ROOT, sub)
        for f in sorted(os.listdir(d)):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    info["library_source_sha256"] = h.hexdigest()[:16]
    build_info = os.path.join(ROOT, "tree_verify_mla_absorb_amd", "libddtree.build.json")
    if os.path.exists(build_info):  # written by the build next to the library
        b = json.load(open(build_info))
        info["library_built_from_git_head"] = b.get("git_head")
        info["library_built_dirty"] = b.get("git_dirty")
    try:
        info["rocm_version"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        info["rocm_version"] = None
    try:
        import torch
        info["torch_hip_version"] = torch.version.hip
        info["gpu"] = torch.cuda.get_device_name(0)
    except Exception:
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["host_cpu"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    info["host_cpus_visible"] = os.cpu_count()
    return info


def time_calls(fn, n: int = 100, replays: int = 5) -> float:
    """Microseconds per call of ``fn`` on the GPU: ``n`` calls captured in one HIP graph (so the
    host's per-call overhead drops out), replayed ``replays`` times, median replay."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / n * 1e3)
    return float(np.median(times))


PEAK_CLOCK_MHZ = 2400.0  # the shader clock the dense bf16 peak is quoted at


def clock_summary(samples, us_per_call: float, flops: float, skip_s: float = 1.1) -> dict:
    """Verify throughput against the dense bf16 peak scaled to the shader clock the part held.

    ``samples`` are (seconds since the load started, GFX clock MHz, socket power W) read on the host
    while the load ran.  amdsmi's readings are averages over a period of up to a second, so the
    first ``skip_s`` seconds (which still show the idle part) are left out.  The peak scales with
    the clock: 2500 TFLOP/s at 2400 MHz."""
    kept = [s for s in samples if s[0] >= skip_s and s[1] > 0] or [s for s in samples if s[1] > 0]
    if not kept:
        return {"error": "no clock samples"}
    clk = float(np.median([s[1] for s in kept]))
    pw = [s[2] for s in kept if s[2] > 0]
    achieved = flops / (us_per_call * 1e-6) / 1e12
    peak_at = PEAK_BF16_TFLOPS * clk / PEAK_CLOCK_MHZ
    return {"verify_us_per_call": round(us_per_call, 2), "gfx_clock_mhz_median": round(clk, 1),
            "gfx_clock_mhz_range": [round(min(s[1] for s in kept), 1), round(max(s[1] for s in kept), 1)],
            "socket_power_w_median": round(float(np.median(pw)), 1) if pw else None,
            "samples": len(kept), "tflops": round(achieved, 2), "peak_at_clock_tflops": round(peak_at, 1),
            "frac_at_clock": round(achieved / peak_at, 4)}


def sustained_clock(fn, flops: float, seconds: float = 3.0, per_graph: int = 20) -> dict:
    """Back-to-back calls of ``fn`` for about ``seconds`` (replays of one HIP graph of ``per_graph``
    calls), with the GFX clock and socket power read through amdsmi while they run."""
    import torch
    try:
        torch.cuda.clock_rate(0)
        torch.cuda.power_draw(0)
    except Exception as e:  # amdsmi missing or not permitted: no figure rather than a guess
        return {"error": f"{type(e).__name__}: {str(e)[:100]}"}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    reps = max(1, int(seconds / (a.elapsed_time(b) * 1e-3)))
    a.record()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    b.record()
    samples = []
    while not b.query():
        samples.append((time.perf_counter() - t0, float(torch.cuda.clock_rate(0)), float(torch.cuda.power_draw(0))))
        time.sleep(0.05)
    torch.cuda.synchronize()
    return clock_summary(samples, a.elapsed_time(b) * 1e3 / (reps * per_graph), flops)


def accept_table(lib, dev):
    """``ddtree_tree_accept`` us/call for 1, 8, 64 streams and budgets 8, 32 (q_len 9, 33)."""
    import torch
    import synth
    table = {}
    for streams in (1, 8, 64):
        for q in (9, 33):
            cases = [synth.accept_case(90 + q, s, q) for s in range(streams)]
            par = torch.from_numpy(np.stack([c[0] for c in cases]).astype(np.int32)).to(dev)
            dr = torch.from_numpy(np.stack([c[1] for c in cases]).astype(np.int32)).to(dev)
            tg = torch.from_numpy(np.stack([c[2] for c in cases]).astype(np.int32)).to(dev)
            keep = torch.empty((streams, q), dtype=torch.int32, device=dev)
            n_keep = torch.empty((streams,), dtype=torch.int32, device=dev)
            nxt = torch.empty((streams,), dtype=torch.int32, device=dev)
            us = time_calls(lambda: lib.tree_accept(par, dr, tg, keep=keep, n_keep=n_keep, next_token=nxt))
            table[f"streams{streams}_budget{q - 1}"] = round(us, 2)
    return table


def build_table(lib, dev, depth: int = 15, topk: int = 8):
    """``ddtree_tree_build`` us/call for 1, 8, 64 requests and budgets 8, 32, 63 (depth 15, top-8)."""
    import torch
    import synth
    table = {}
    for streams in (1, 8, 64):
        pairs = [synth.drafter_topk(60, s, depth, topk) for s in range(streams)]
        lp = torch.from_numpy(np.stack([p[0] for p in pairs])).to(dev)
        tok = torch.from_numpy(np.stack([p[1] for p in pairs])).to(dev)
        for budget in (8, 32, 63):
            par = torch.empty((streams, budget + 1), dtype=torch.int32, device=dev)
            ntok = torch.empty_like(par)
            n = torch.empty((streams,), dtype=torch.int32, device=dev)
            args = [lib._ptr(lp), lib._ptr(tok), None, depth, topk, budget, streams, lib._ptr(par), lib._ptr(ntok),
                    lib._ptr(n), None, None, None, None, None]

            def call():
                rc = lib.LIB.ddtree_tree_build(*args, lib._stream(None))
                assert rc == 0, rc

            us = time_calls(call)
            table[f"streams{streams}_budget{budget}"] = round(us, 2)
    return table


def layers_table(lib, dev, w, parents, draft_tok, target_tok, keep_bits, n_keep_bits, n_layers: int = 61):
    """Acceptance plus compaction of ``n_layers`` caches of the workload's geometry (61: the
    DeepSeek-V3 / Kimi-K2 layer count): one ``ddtree_accept_compact_layers`` call against one
    ``ddtree_accept_compact`` call per layer.  The caches are device allocations whose contents do
    not matter (the gather copies bits)."""
    import torch
    rows = w.kv_rows
    caches = [(torch.empty((w.streams, rows, 512), dtype=torch.bfloat16, device=dev),
               torch.empty((w.streams, rows, 64), dtype=torch.bfloat16, device=dev)) for _ in range(n_layers)]
    keep = torch.empty((w.streams, w.q_len), dtype=torch.int32, device=dev)
    n_keep = torch.empty((w.streams,), dtype=torch.int32, device=dev)
    nxt = torch.empty((w.streams,), dtype=torch.int32, device=dev)
    fused = time_calls(lambda: lib.accept_compact_layers(caches, w.prefix, parents, draft_tok, target_tok, keep=keep,
                                                         n_keep=n_keep, next_token=nxt))

    def per_layer():
        for c, k in caches:
            lib.accept_compact(c, k, w.prefix, parents, draft_tok, target_tok, keep=keep, n_keep=n_keep,
                               next_token=nxt)

    looped = time_calls(per_layer, n=20)
    moved_rows = sum(int((keep_bits[s, :n_keep_bits[s]] != np.arange(n_keep_bits[s])).sum())
                     for s in range(w.streams))
    moved_bytes = 2 * moved_rows * (512 + 64) * 2 * n_layers  # read + write of each moved row
    del caches
    torch.cuda.empty_cache()
    return {"layers": n_layers, "us_per_call": round(fused, 2), "per_layer_calls_us": round(looped, 2),
            "moved_bytes": moved_bytes, "gbs": round(moved_bytes / (fused * 1e-6) / 1e9, 1)}


MALL_BYTES = 256 << 20  # the part's last-level cache (Infinity Cache)


def workloads_table(lib, dev, skip: str, with_oracle: bool = True):
    """``ddtree_verify_attn_ex`` (automatic split plan) us/call, TFLOP/s and % of the bf16 peak on
    every named workload but ``skip``: 100 calls in one HIP graph, median of 5 replays.  These
    workloads fit in the last-level cache, so that figure is warm; ``cold_us_per_call`` rotates
    through copies of the inputs and outputs totalling at least twice that cache, one copy per
    call, so that every call finds its data evicted.  With ``with_oracle``, each entry also gives
    the fp64 oracle's seconds for the same whole call on the host's cores."""
    import torch
    import synth
    table = {}
    for name, w in synth.WORKLOADS.items():
        if name == skip:
            continue
        b = synth.make_batch(w, with_path=False)

        def up(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

        ql, qp, ckv, kpe = up(b.q_lat), up(b.q_pe), up(b.ckv), up(b.kpe)
        par = torch.from_numpy(b.parents).to(dev)
        out = torch.empty((w.streams, w.q_len, w.heads, 512), dtype=torch.float32, device=dev)
        lse = torch.empty((w.streams, w.q_len, w.heads), dtype=torch.float32, device=dev)
        nbytes = lib.workspace_size(w.prefix, w.q_len, w.streams, 0)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev) if nbytes else None
        us = time_calls(lambda: lib.verify_attn_ex(ql, qp, ckv, kpe, w.prefix, par, out=out, lse=lse, workspace=ws))
        flops = 2.0 * w.heads * (576 + 512) * visible_pairs(b.parents, w.prefix)
        tf = flops / (us * 1e-6) / 1e12
        # cold: one copy per call, copies totalling at least twice the last-level cache
        per_copy = sum(t.numel() * t.element_size() for t in (ql, qp, ckv, kpe, par, out, lse))
        n_copies = max(2, -(-2 * MALL_BYTES // per_copy))
        copies = [tuple(t.clone() for t in (ql, qp, ckv, kpe, par, out, lse)) for _ in range(n_copies)]
        turn = [0]

        def cold_call():
            c = copies[turn[0] % n_copies]
            turn[0] += 1
            lib.verify_attn_ex(c[0], c[1], c[2], c[3], w.prefix, c[4], out=c[5], lse=c[6], workspace=ws)

        cold_us = time_calls(cold_call, n=max(n_copies, 20))
        table[name] = {"us_per_call": round(us, 2), "tflops": round(tf, 2),
                       "pct_mfma_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                       "splits": lib.num_splits(w.prefix, w.q_len, w.streams, 0),
                       "cold_us_per_call": round(cold_us, 2), "cold_copies": n_copies}
        del ql, qp, ckv, kpe, out, lse, ws, copies
        if with_oracle:
            o = oracle_seconds_per_call(w, b)
            table[name].update(o)
            table[name]["oracle_over_gpu"] = round(o["oracle_s_per_call"] / (us * 1e-6), 1)
    torch.cuda.empty_cache()
    return table


def ragged_table(lib, dev, w, q_lat, q_pe, ckv, kpe, parents_bits):
    """``ddtree_verify_attn_ragged`` on the workload's inputs with per-stream prefixes drawn
    uniformly from [prefix / 4, prefix] (a batch after some steps of compaction): us/call and
    TFLOP/s over each stream's own visible keys, next to the uniform-prefix call."""
    import torch
    import synth
    rng = synth.rng_for(w.seed, 0, 99)
    prefixes = rng.integers(w.prefix // 4, w.prefix + 1, size=w.streams).astype(np.int32)
    pl = torch.from_numpy(prefixes).to(dev)
    par = torch.from_numpy(parents_bits).to(dev)
    out = torch.empty((w.streams, w.q_len, w.heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((w.streams, w.q_len, w.heads), dtype=torch.float32, device=dev)
    nbytes = lib.workspace_size(w.prefix, w.q_len, w.streams, 0)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev) if nbytes else None
    us = time_calls(lambda: lib.verify_attn_ragged(q_lat, q_pe, ckv, kpe, pl, w.prefix, par, out=out, lse=lse,
                                                   workspace=ws), n=20, replays=3)
    flops = sum(2.0 * w.heads * (576 + 512) * visible_pairs(parents_bits[s:s + 1], int(prefixes[s]))
                for s in range(w.streams))
    return {"prefixes": f"uniform in [{w.prefix // 4}, {w.prefix}], mean {prefixes.mean():.0f}",
            "us_per_call": round(us, 2), "tflops": round(flops / (us * 1e-6) / 1e12, 2)}


def append_table(lib, dev, w, parents):
    """``ddtree_append_tree_kv`` us/call on the workload's trees: the projection's fp32 rows in,
    the bf16 cache rows out, at the workload's prefix (tables cover the positions)."""
    import torch
    import synth
    kv, nw = synth.append_inputs(7, w.streams, w.q_len)
    cos, sin = synth.rope_tables(w.prefix + w.q_len)
    kv_d, nw_d = torch.from_numpy(kv).to(dev), torch.from_numpy(nw).to(dev)
    cos_d, sin_d = torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev)
    ckv = torch.empty((w.streams, w.kv_rows, 512), dtype=torch.bfloat16, device=dev)
    kpe = torch.empty((w.streams, w.kv_rows, 64), dtype=torch.bfloat16, device=dev)
    us = time_calls(lambda: lib.append_tree_kv(ckv, kpe, w.prefix, parents, kv_d, nw_d, 1e-6, cos_d, sin_d))
    nbytes = w.streams * w.q_len * (576 * 4 + 576 * 2)  # fp32 rows in, bf16 rows out
    return {"us_per_call": round(us, 2), "bytes": nbytes, "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def _db_rows(path: str, sql: str):
    import sqlite3
    con = sqlite3.connect(path)
    try:
        return list(con.execute(sql))
    finally:
        con.close()


def summarize_trace(db: str, command: str, skip: int = 0, bench_log: str = None) -> str:
    """Per-kernel dispatch statistics of a ``rocprofv3 --kernel-trace`` database, as text.
    ``avg_timed_us`` leaves out each kernel's first ``skip`` dispatches (the warm-up steps).
    With ``bench_log`` (the profiled command's stdout), the JSON line that command printed is
    kept beside the trace, with the verify kernel's roofline fraction recomputed from the
    trace's own average next to the line's (which comes from HIP events in the same run)."""
    rows = _db_rows(db, "select name, start, duration from kernels order by start")
    per = {}
    for name, _, dur in rows:
        per.setdefault(name, []).append(dur / 1e3)
    lines = [f"command: {command}", "units: microseconds per dispatch (trace durations in ns / 1000)",
             f"kernel_source_sha256: {kernel_sha()}", f"warm-up dispatches left out of avg_timed_us: {skip}", "",
             f"{'kernel':66s} {'calls':>5s} {'avg_us':>9s} {'avg_timed_us':>12s} {'min_us':>9s} {'max_us':>9s}"]
    for name, d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        short = name if len(name) <= 66 else name[:63] + "..."
        timed = d[skip:] if len(d) > skip else d
        lines.append(f"{short:66s} {len(d):5d} {sum(d) / len(d):9.2f} {sum(timed) / len(timed):12.2f} "
                     f"{min(d):9.2f} {max(d):9.2f}")
    if bench_log:
        line = None
        for text in open(bench_log):
            if text.startswith("{") and '"metric"' in text:
                line = json.loads(text)
        if line is not None:
            def timed_avg(d):
                t = d[skip:] if len(d) > skip else d
                return sum(t) / len(t)
            verify = [d for name, d in per.items() if "verify_attn_kernel" in name]
            merge = [d for name, d in per.items() if "verify_combine_kernel" in name]
            lines += ["", f"bench line printed by the profiled command: {json.dumps(line)}"]
            if verify and "detail" in line and "flop_visible_pairs" in line["detail"]:
                flop = line["detail"]["flop_visible_pairs"]
                avg = timed_avg(verify[0])
                # one verify call = the attention kernel plus, when a group is split, one merge
                call = avg + (timed_avg(merge[0]) if merge and len(merge[0]) == len(verify[0]) else 0.0)
                frac = flop / (avg * 1e-6) / 1e12 / PEAK_BF16_TFLOPS
                frac_call = flop / (call * 1e-6) / 1e12 / PEAK_BF16_TFLOPS
                lines += [f"verify_attn_kernel avg_timed_us (trace): {avg:.2f}",
                          f"verify call (attention kernel + merge kernel) avg_timed_us (trace): {call:.2f}",
                          f"verify_us_per_call (line, HIP events around each call): "
                          f"{line['detail'].get('verify_us_per_call')}",
                          f"roofline frac from the trace: kernel alone {frac:.4f}, whole call {frac_call:.4f}; "
                          f"from the line (whole call): {line.get('roofline', {}).get('frac')}"]
    return "\n".join(lines) + "\n"


def _pmc_mean(db: str, kernel_substr: str, counter: str) -> float:
    rows = _db_rows(db, "select name, counter_name, counter_value from pmc_events")
    vals = [v for name, cn, v in rows if kernel_substr in name and cn == counter]
    if not vals:
        raise SystemExit(f"no {counter} samples for {kernel_substr} in {db}")
    return sum(vals) / len(vals)


def summarize_pmc(fetch_db: str, write_db: str, copy_fetch_db: str, copy_write_db: str, copy_bytes: int,
                  commands: str) -> str:
    """HBM bytes per verify launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled
    by what the same counter reads for a plain device copy of ``copy_bytes``."""
    copy_kernel = "copyBuffer"
    cf = _pmc_mean(copy_fetch_db, copy_kernel, "FETCH_SIZE") * 1024.0
    cw = _pmc_mean(copy_write_db, copy_kernel, "WRITE_SIZE") * 1024.0
    f_scale, w_scale = copy_bytes / cf, copy_bytes / cw
    kf = _pmc_mean(fetch_db, "verify_attn_kernel", "FETCH_SIZE") * 1024.0
    kw = _pmc_mean(write_db, "verify_attn_kernel", "WRITE_SIZE") * 1024.0
    total = kf * f_scale + kw * w_scale
    lines = [f"commands: {commands}",
             f"kernel_source_sha256: {kernel_sha()}",
             f"copy_bytes: {copy_bytes}",
             f"copy_fetch_size_bytes: {cf:.0f}  -> fetch scale {f_scale:.4f}",
             f"copy_write_size_bytes: {cw:.0f}  -> write scale {w_scale:.4f}",
             f"verify_fetch_size_bytes_raw: {kf:.0f}  scaled: {kf * f_scale:.0f}",
             f"verify_write_size_bytes_raw: {kw:.0f}  scaled: {kw * w_scale:.0f}",
             f"hbm_bytes_per_launch: {total:.0f}"]
    return "\n".join(lines) + "\n"


def summarize_counters(db: str, command: str) -> str:
    """Mean per verify launch of every counter in a ``rocprofv3 --pmc`` database, plus the MFMA
    utilisation (busy cycles of the matrix units over active cycles, per SIMD) and the MFMA
    FLOPs these counters imply."""
    rows = _db_rows(db, "select name, dispatch_id, counter_name, counter_value from pmc_events")
    tot = {}  # (counter, dispatch) -> sum over the counter's hardware instances
    for name, disp, cn, v in rows:
        if "verify_attn_kernel" in name:
            tot[(cn, disp)] = tot.get((cn, disp), 0.0) + v
    if not tot:
        raise SystemExit(f"no verify_attn_kernel samples in {db}")
    per = {}
    for (cn, _), v in tot.items():
        per.setdefault(cn, []).append(v)
    mean = {k: sum(v) / len(v) for k, v in per.items()}
    lines = [f"command: {command}", f"kernel_source_sha256: {kernel_sha()}",
             "counter means per verify_attn_kernel dispatch (hardware instances summed):"]
    lines += [f"  {k}: {mean[k]:.6g}  (dispatches: {len(per[k])})" for k in sorted(mean)]
    if "MfmaUtil" in mean:
        lines.append(f"mfma_busy_pct: {mean['MfmaUtil']:.2f}")
    if "MfmaFlopsBF16" in mean:
        lines.append(f"mfma_bf16_flop_per_launch: {mean['MfmaFlopsBF16']:.6g}")
    if "SQ_LDS_BANK_CONFLICT" in mean and "SQ_LDS_IDX_ACTIVE" in mean and mean["SQ_LDS_IDX_ACTIVE"]:
        lines.append(f"lds_bank_conflict_cycles_per_active_cycle: "
                     f"{mean['SQ_LDS_BANK_CONFLICT'] / mean['SQ_LDS_IDX_ACTIVE']:.4f}")
    return "\n".join(lines) + "\n"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail-tables", action="store_true",
                    help="skip the per-call tables of the other entry points and workloads (for profiler "
                         "runs that must see only the step's own launches)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES, 3 times (for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("DB", "COMMAND", "SKIP"),
                    help="print a per-kernel summary of a rocprofv3 kernel-trace database and exit")
    ap.add_argument("--bench-log", default=None,
                    help="with --summarize-trace: the profiled command's stdout, whose JSON line is kept "
                         "beside the trace")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("DB", "COMMAND"),
                    help="print the verify launch's mean counters (MFMA utilisation, LDS) and exit")
    ap.add_argument("--summarize-pmc", nargs=6,
                    metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB", "COPY_BYTES", "COMMANDS"),
                    help="print HBM bytes per verify launch from FETCH_SIZE / WRITE_SIZE runs and exit")
    args = ap.parse_args()
    if args.summarize_trace:
        db, cmd, skip = args.summarize_trace
        print(summarize_trace(db, cmd, int(skip), args.bench_log), end="")
        return 0
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters), end="")
        return 0
    if args.summarize_pmc:
        f, w, cf, cw, nbytes, cmds = args.summarize_pmc
        print(summarize_pmc(f, w, cf, cw, int(nbytes), cmds), end="")
        return 0
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on exactly one GPU; --gpus must be 1 "
                                   "(streams would shard across GPUs with no communication between them)"}))
        return 2

    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "launches": 3}), flush=True)
        return 0

    import synth
    from tree_verify_mla_absorb_amd import _lib

    name = args.workload or synth.HEADLINE
    w = synth.WORKLOADS[name]
    b = synth.make_batch(w)
    dev = "cuda:0"

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q_lat, q_pe, ckv, kpe = up(b.q_lat), up(b.q_pe), up(b.ckv), up(b.kpe)
    parents = torch.from_numpy(b.parents).to(dev)
    draft_tok = torch.from_numpy(b.draft_tok).to(dev)
    target_tok = torch.from_numpy(b.target_tok).to(dev)
    keep = torch.from_numpy(b.keep).to(dev)
    n_keep = torch.from_numpy(b.n_keep).to(dev)
    next_tok = torch.empty((w.streams,), dtype=torch.int32, device=dev)
    out = torch.empty((w.streams, w.q_len, w.heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((w.streams, w.q_len, w.heads), dtype=torch.float32, device=dev)
    splits = _lib.num_splits(w.prefix, w.q_len, w.streams, args.num_splits)
    ws_bytes = _lib.workspace_size(w.prefix, w.q_len, w.streams, args.num_splits)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(ev_a=None, ev_b=None):
        if ev_a is not None:
            ev_a.record(stream)
        _lib.verify_attn_ex(q_lat, q_pe, ckv, kpe, w.prefix, parents, out=out, lse=lse,
                            num_splits=args.num_splits, workspace=ws, stream=stream)
        if ev_b is not None:
            ev_b.record(stream)
        _lib.accept_compact(ckv, kpe, w.prefix, parents, draft_tok, target_tok, keep=keep, n_keep=n_keep,
                            next_token=next_tok, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(*evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    verify_ms = float(np.mean([a.elapsed_time(bb) for a, bb in evs]))

    # per-call times of the other entry points and workloads (outside the timed steps)
    tables = {}
    if not args.no_detail_tables:
        fused_us = time_calls(lambda: _lib.accept_compact(ckv, kpe, w.prefix, parents, draft_tok, target_tok,
                                                          keep=keep, n_keep=n_keep, next_token=next_tok))
        compact_us = time_calls(lambda: _lib.compact_kv(ckv, kpe, w.prefix, keep, n_keep))
        # read + write of every kept row that moves (a row kept in place, such as the root, is skipped)
        compact_moved = 2 * (512 + 64) * 2 * sum(int((b.keep[s, :b.n_keep[s]] != np.arange(b.n_keep[s])).sum())
                                                 for s in range(w.streams))
        tables = {
            "sustained": sustained_clock(
                lambda: _lib.verify_attn_ex(q_lat, q_pe, ckv, kpe, w.prefix, parents, out=out, lse=lse,
                                            num_splits=args.num_splits, workspace=ws),
                2.0 * w.heads * (576 + 512) * visible_pairs(b.parents, w.prefix)),
            "accept_compact_us_per_call": round(fused_us, 2),
            "compact_kv_us_per_call": round(compact_us, 2),
            "compact_kv_moved_bytes": compact_moved,
            "compact_kv_gbs": round(compact_moved / (compact_us * 1e-6) / 1e9, 1),
            "tree_accept_us_per_call": accept_table(_lib, dev),
            "tree_build_us_per_call": build_table(_lib, dev),
            "accept_compact_layers": layers_table(_lib, dev, w, parents, draft_tok, target_tok, b.keep, b.n_keep),
            "append_tree_kv": append_table(_lib, dev, w, parents),
            "verify_other_workloads": workloads_table(_lib, dev, w.name, with_oracle=not args.no_cpu_baseline),
            "verify_ragged": ragged_table(_lib, dev, w, q_lat, q_pe, ckv, kpe, b.parents),
        }

    flops = 2.0 * w.heads * (576 + 512) * visible_pairs(b.parents, w.prefix)
    tflops_step = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (verify_ms * 1e-3) / 1e12
    traffic = read_traffic()
    res = {
        "metric": METRIC,
        "value": round(tflops_step, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "streams": w.streams, "heads": w.heads, "prefix": w.prefix,
                   "q_len": w.q_len, "tree": w.tree, "seed": w.seed, "num_splits": splits,
                   "step": "verify_attn + accept_compact"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "detail": {"verify_us_per_call": round(verify_ms * 1e3, 2),
                   "accept_compact_us_per_call_incl_gap": round((ms_step - verify_ms) * 1e3, 2),
                   **tables,
                   "verify_tflops": round(achieved, 2),
                   "pct_mfma_peak": round(100 * achieved / PEAK_BF16_TFLOPS, 2),
                   "algorithmic_bytes": algorithmic_bytes(w, w.streams),
                   "hbm_gbs_algorithmic": round(algorithmic_bytes(w, w.streams) / (verify_ms * 1e-3) / 1e9, 1),
                   "flop_visible_pairs": flops, "wall_s_timed": round(wall, 3),
                   "kernel_source_sha256": kernel_sha()},
    }
    res["detail"]["host"] = host_info()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, b)
        # the same oracle timing, as seconds for the whole call (all streams)
        rate = res["cpu_baseline"]["value"] * 1e12  # FLOP/s
        res["detail"]["oracle_s_per_call"] = round(flops / rate, 3)
        res["detail"]["oracle_over_gpu"] = round(flops / rate / (verify_ms * 1e-3), 1)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
