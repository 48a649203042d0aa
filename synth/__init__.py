"""Seeded synthetic inputs for tree-verify MLA-absorb attention and KV compaction.

This module holds none of the method's arithmetic.  It only draws inputs: bf16 activations
(standard normal, rounded to bf16 by round-to-nearest-even on the fp32 bits), draft trees as
``parents[]`` arrays, an accepted root-to-leaf path per stream, and token ids for the tree
nodes: the drafter's token of every node (distinct among siblings) and the target model's
greedy token at every node, planted so that the accepted path is the drawn one.  Both the
oracle and the HIP path consume exactly these arrays, bit for bit.

Shapes follow the pages' engine ("Race Conditions, Buffer Aliasing, and the Architecture of a
Native DDTree Inference Engine", section "The Cache Compaction Problem"): one latent cache per
stream, the committed prefix in rows ``[0, P)`` and tree node ``i`` in row ``P + i``; a child
always has a larger node index than its parent.  The tree sizes respect the limits of the
tree builder on "Building the Foundation: Architecting a Native CUDA DDTree Inference Engine",
section "The Single-Threaded Heap Design" (budget at most 64, depth at most 15).

Every random draw uses ``numpy.random.Generator(PCG64(SeedSequence([seed, stream, tag])))`` so that
any stream can be regenerated on its own (per-layer caches add the layer:
``SeedSequence([seed, stream, tag, layer])``).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEADS = 64
D_LATENT = 512
D_ROPE = 64
MAX_DEPTH = 15

TAG_Q_LAT, TAG_Q_PE, TAG_CKV, TAG_KPE, TAG_PARENTS, TAG_LEAF = 0, 1, 2, 3, 4, 5
TAG_DRAFT_TOK, TAG_TARGET_TOK, TAG_ACCEPT_DEPTH, TAG_DRAFTER = 6, 7, 8, 9
TAG_LAYER_CKV, TAG_LAYER_KPE = 10, 11
TAG_KV_PROJ, TAG_NORM_W = 12, 13
VOCAB = 163840  # synthetic vocabulary size for token ids


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: ``streams`` independent requests sharing one launch."""

    name: str
    streams: int
    prefix: int
    q_len: int
    tree: str = "uniform"  # "uniform" or "chain70"
    seed: int = 0
    heads: int = HEADS

    @property
    def kv_rows(self) -> int:
        return self.prefix + self.q_len


# The five seeded workloads: small single stream; eight mid-length streams; many small query
# blocks; one long chain-heavy stream; sixty-four long streams followed by compaction.
WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in (
        Workload("s1-p256-q9", 1, 256, 9, "uniform", seed=1),
        Workload("s8-p1024-q33", 8, 1024, 33, "uniform", seed=2),
        Workload("s64-p1024-q9", 64, 1024, 9, "uniform", seed=3),
        Workload("s1-p4096-q33-chain", 1, 4096, 33, "chain70", seed=4),
        Workload("s64-p4096-q33", 64, 4096, 33, "uniform", seed=5),
    )
}
HEADLINE = "s64-p4096-q33"


def rng_for(seed: int, stream: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, tag])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even), returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


def sample_parents(rng: np.random.Generator, q_len: int, tree: str = "uniform",
                   max_depth: int = MAX_DEPTH) -> np.ndarray:
    """Draw a draft tree as ``parents[]``: node 0 is the root, every parent index is smaller.

    ``uniform``: parent of node i drawn uniformly from [0, i-1]; if that parent already sits at
    the depth cap, redraw uniformly among the earlier nodes below the cap.
    ``chain70``: with probability 0.7 the parent is node i-1 (when it is below the cap), else the
    uniform rule.
    """
    parents = np.full(q_len, -1, dtype=np.int32)
    depth = np.zeros(q_len, dtype=np.int32)
    for i in range(1, q_len):
        if tree == "chain70" and rng.random() < 0.7 and depth[i - 1] < max_depth:
            p = i - 1
        else:
            p = int(rng.integers(0, i))
            if depth[p] >= max_depth:
                ok = np.nonzero(depth[:i] < max_depth)[0]
                p = int(ok[rng.integers(0, len(ok))])
        parents[i] = p
        depth[i] = depth[p] + 1
    return parents


def accepted_path(rng: np.random.Generator, parents: np.ndarray) -> np.ndarray:
    """A root-to-leaf path (node indices, strictly increasing), leaf drawn uniformly."""
    q = len(parents)
    has_child = np.zeros(q, dtype=bool)
    has_child[parents[1:]] = True
    leaves = np.nonzero(~has_child)[0]
    node = int(leaves[rng.integers(0, len(leaves))])
    path = []
    while node >= 0:
        path.append(node)
        node = int(parents[node])
    return np.array(path[::-1], dtype=np.int32)


def draft_tokens(rng: np.random.Generator, parents: np.ndarray, vocab: int = VOCAB) -> np.ndarray:
    """The drafter's token of every node: uniform ids, redrawn until distinct among siblings
    (a drafter proposes distinct candidates at one position).  The root's entry is the last
    committed token."""
    q = len(parents)
    tok = rng.integers(0, vocab, size=q, dtype=np.int64).astype(np.int32)
    for j in range(1, q):
        sib = [int(tok[k]) for k in range(1, j) if parents[k] == parents[j]]
        while int(tok[j]) in sib:
            tok[j] = rng.integers(0, vocab)
    return tok


def target_tokens(rng: np.random.Generator, parents: np.ndarray, draft: np.ndarray, path: np.ndarray,
                  vocab: int = VOCAB) -> np.ndarray:
    """The target model's greedy token at every node, planted so that greedy acceptance follows
    ``path`` (a root-based chain of nodes) and stops at its last node: along the path the target
    agrees with the next node's draft token, at the last node it differs from every child's
    draft token, and elsewhere it is uniform."""
    q = len(parents)
    tgt = rng.integers(0, vocab, size=q, dtype=np.int64).astype(np.int32)
    for k in range(len(path) - 1):
        tgt[path[k]] = draft[path[k + 1]]
    last = int(path[-1])
    kids = {int(draft[j]) for j in range(q) if parents[j] == last}
    while int(tgt[last]) in kids:
        tgt[last] = rng.integers(0, vocab)
    return tgt


@dataclass
class Batch:
    """Inputs for one launch, bf16 payloads stored as uint16 bit patterns."""

    workload: Workload
    q_lat: np.ndarray   # uint16 [S, Q, H, 512]
    q_pe: np.ndarray    # uint16 [S, Q, H, 64]
    ckv: np.ndarray     # uint16 [S, L, 512]
    kpe: np.ndarray     # uint16 [S, L, 64]
    parents: np.ndarray  # int32 [S, Q]
    keep: np.ndarray    # int32 [S, Q]  (accepted path, padded with -1)
    n_keep: np.ndarray  # int32 [S]
    draft_tok: np.ndarray | None = None   # int32 [S, Q]
    target_tok: np.ndarray | None = None  # int32 [S, Q]  (greedy acceptance yields keep)
    extra: dict = field(default_factory=dict)


def make_batch(w: Workload, streams: int | None = None, with_path: bool = True) -> Batch:
    """Generate the inputs of workload ``w`` (optionally only its first ``streams`` streams)."""
    s_count = w.streams if streams is None else streams
    q, l, h = w.q_len, w.kv_rows, w.heads
    q_lat = np.empty((s_count, q, h, D_LATENT), np.uint16)
    q_pe = np.empty((s_count, q, h, D_ROPE), np.uint16)
    ckv = np.empty((s_count, l, D_LATENT), np.uint16)
    kpe = np.empty((s_count, l, D_ROPE), np.uint16)
    parents = np.empty((s_count, q), np.int32)
    keep = np.full((s_count, q), -1, np.int32)
    n_keep = np.zeros(s_count, np.int32)
    draft = np.zeros((s_count, q), np.int32) if with_path else None
    target = np.zeros((s_count, q), np.int32) if with_path else None
    for s in range(s_count):
        q_lat[s] = bf16_normal(rng_for(w.seed, s, TAG_Q_LAT), (q, h, D_LATENT))
        q_pe[s] = bf16_normal(rng_for(w.seed, s, TAG_Q_PE), (q, h, D_ROPE))
        ckv[s] = bf16_normal(rng_for(w.seed, s, TAG_CKV), (l, D_LATENT))
        kpe[s] = bf16_normal(rng_for(w.seed, s, TAG_KPE), (l, D_ROPE))
        parents[s] = sample_parents(rng_for(w.seed, s, TAG_PARENTS), q, w.tree)
        if with_path:
            path = accepted_path(rng_for(w.seed, s, TAG_LEAF), parents[s])
            keep[s, : len(path)] = path
            n_keep[s] = len(path)
            draft[s] = draft_tokens(rng_for(w.seed, s, TAG_DRAFT_TOK), parents[s])
            target[s] = target_tokens(rng_for(w.seed, s, TAG_TARGET_TOK), parents[s], draft[s], path)
    return Batch(w, q_lat, q_pe, ckv, kpe, parents, keep, n_keep, draft, target)


def drafter_topk(seed: int, stream: int, depth: int, topk: int, vocab: int = 1000, temperature: float = 2.0):
    """A drafter's per-position top-k for one request: ``(lp [depth, topk] float32, tok [depth,
    topk] int32)``.  Each position's logits are N(0, temperature^2) over ``vocab`` ids; ``lp`` are
    the log-softmax values of the ``topk`` most likely ids, in decreasing order, and ``tok`` those
    ids (distinct within a position)."""
    rng = rng_for(seed, stream, TAG_DRAFTER)
    lp = np.empty((depth, topk), np.float32)
    tok = np.empty((depth, topk), np.int32)
    for d in range(depth):
        logits = rng.standard_normal(vocab) * temperature
        logp = logits - (np.log(np.exp(logits - logits.max()).sum()) + logits.max())
        order = np.argsort(-logp, kind="stable")[:topk]
        lp[d] = logp[order].astype(np.float32)
        tok[d] = order.astype(np.int32)
    return lp, tok


def accept_case(seed: int, stream: int, q_len: int, tree: str = "uniform", vocab: int = VOCAB):
    """A tree with tokens whose greedy acceptance stops at a uniformly drawn depth of a uniformly
    drawn root-to-leaf path.  Returns (parents, draft, target, planted path)."""
    parents = sample_parents(rng_for(seed, stream, TAG_PARENTS), q_len, tree)
    full = accepted_path(rng_for(seed, stream, TAG_LEAF), parents)
    depth = int(rng_for(seed, stream, TAG_ACCEPT_DEPTH).integers(0, len(full)))
    path = full[: depth + 1]
    draft = draft_tokens(rng_for(seed, stream, TAG_DRAFT_TOK), parents, vocab)
    target = target_tokens(rng_for(seed, stream, TAG_TARGET_TOK), parents, draft, path, vocab)
    return parents, draft, target, path


def random_inputs(seed: int, streams: int, prefix: int, q_len: int, heads: int = HEADS,
                  tree: str = "uniform") -> Batch:
    """Ad-hoc sizes for tests (same recipe as the named workloads)."""
    return make_batch(Workload(f"adhoc-{seed}", streams, prefix, q_len, tree, seed, heads))


def layer_caches(seed: int, n_layers: int, streams: int, rows: int):
    """One latent cache per model layer, all of the same geometry: a list of ``(ckv [streams,
    rows, 512], kpe [streams, rows, 64])`` bf16 bit arrays, each layer drawn independently."""
    out = []
    for layer in range(n_layers):
        ckv = np.empty((streams, rows, D_LATENT), np.uint16)
        kpe = np.empty((streams, rows, D_ROPE), np.uint16)
        for s in range(streams):
            ckv[s] = bf16_normal(np.random.Generator(np.random.PCG64(np.random.SeedSequence(
                [seed, s, TAG_LAYER_CKV, layer]))), (rows, D_LATENT))
            kpe[s] = bf16_normal(np.random.Generator(np.random.PCG64(np.random.SeedSequence(
                [seed, s, TAG_LAYER_KPE, layer]))), (rows, D_ROPE))
        out.append((ckv, kpe))
    return out


def rope_tables(rows: int, base: float = 10000.0):
    """The caller's rotary tables, float32 ``[rows, 32]`` each: angle ``pos * base**(-j / 32)``
    for the 32 rotated pairs of a 64-value rotary row (the usual frequency ladder)."""
    inv = base ** (-np.arange(32, dtype=np.float64) / 32.0)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def append_inputs(seed: int, streams: int, q_len: int):
    """Inputs of the tree-row append: the key/value projection's float32 output ``[streams,
    q_len, 576]`` (standard normal, scaled by 2 so that the norm has work to do) and the
    RMSNorm weight ``[512]`` (uniform in [0.5, 1.5])."""
    kv = np.empty((streams, q_len, D_LATENT + D_ROPE), np.float32)
    for s in range(streams):
        kv[s] = 2.0 * rng_for(seed, s, TAG_KV_PROJ).standard_normal((q_len, D_LATENT + D_ROPE), dtype=np.float32)
    w = rng_for(seed, 0, TAG_NORM_W).uniform(0.5, 1.5, D_LATENT).astype(np.float32)
    return kv, w
