"""fp64 oracle: tree-verify MLA-absorb attention with visibility masking.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring).

What is computed, and which passage it follows
-----------------------------------------------
"Race Conditions, Buffer Aliasing, and the Architecture of a Native DDTree Inference Engine",
section "The Mission: A Native DDTree Engine", names the kernel: tree-verify attention in the
MLA-absorb form, with visibility masking, inside a DeepSeekV3/Kimi-style MLA transformer.  The
same page, section "The Cache Compaction Problem", fixes the cache geometry: the tree block is
appended after the committed prefix (node ``i`` at row ``P + i``), a child's index is always
larger than its parent's, and the accepted tokens form a root-to-node path.
"Building the Foundation: Architecting a Native CUDA DDTree Inference Engine", section "The
Single-Threaded Heap Design", has the tree builder emit ``parents`` and a visibility matrix.

Readings (the pages name the operation but do not write its formula):

* Visibility: node ``i`` sees every prefix row and the tree rows of its ancestors and itself.
  That is the plain reading of a draft tree whose verification keeps one root-to-node path:
  each node is scored as the continuation of its own path.
* Absorbed MLA: per head, the query is already mapped into the shared latent space
  (``q_lat``, 512-d) plus the rotary part (``q_pe``, 64-d).  Keys are the shared rows
  ``[c_kv | k_pe]`` (576-d); values are the latent rows ``c_kv`` alone (512-d).  The output is the
  latent attention output; the per-head up-projection is outside this operation.
* Scale ``1/sqrt(192)``: the softmax scale of a DeepSeek-V3-style head (128 no-rope + 64 rope
  dims), which the absorbed form keeps unchanged.
* ``lse`` is the natural log of the sum of ``exp(scaled score)`` over the visible keys.
* RoPE is not applied here: ``q_pe`` and ``k_pe`` arrive already rotated.
"""
from __future__ import annotations

import math

import numpy as np

DEFAULT_SCALE = 1.0 / math.sqrt(192.0)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ancestor_or_self(parents: np.ndarray) -> np.ndarray:
    """Boolean ``A[i, j]``: tree node ``j`` is node ``i`` itself or one of its ancestors.

    ``parents[0] == -1`` marks the root and every other parent index lies in ``[0, i)`` (a child
    is created after its parent).  Anything else is rejected.
    """
    parents = np.asarray(parents, dtype=np.int64)
    q = len(parents)
    if q < 1 or parents[0] != -1:
        raise ValueError("parents[0] must be -1")
    for i in range(1, q):
        if not 0 <= parents[i] < i:
            raise ValueError(f"parents[{i}]={parents[i]} is not an earlier node")
    anc = np.zeros((q, q), dtype=bool)
    for i in range(q):
        j = i
        while j >= 0:
            anc[i, j] = True
            j = parents[j]
    return anc


def visibility(parents: np.ndarray, prefix_len: int) -> np.ndarray:
    """Boolean ``V[i, t]`` over the ``prefix_len + q_len`` cache rows of one stream."""
    anc = ancestor_or_self(parents)
    q = anc.shape[0]
    vis = np.zeros((q, prefix_len + q), dtype=bool)
    vis[:, :prefix_len] = True
    vis[:, prefix_len:] = anc
    return vis


def scores_absorbed(q_lat: np.ndarray, q_pe: np.ndarray, ckv: np.ndarray, kpe: np.ndarray,
                    scale: float) -> np.ndarray:
    """Scaled scores ``[Q, H, L]``: ``scale * (q_lat . c_kv[t] + q_pe . k_pe[t])`` (float64)."""
    return scale * (np.matmul(q_lat, ckv.T) + np.matmul(q_pe, kpe.T))


def masked_softmax_attention(scores: np.ndarray, vis: np.ndarray, values: np.ndarray):
    """Softmax over the visible keys only; returns ``(out [Q,H,Dv], lse [Q,H])``.

    ``scores`` is ``[Q, H, L]``, ``vis`` is ``[Q, L]`` (shared by the heads), ``values``
    ``[L, Dv]``.  Every row must see at least one key.
    """
    if not vis.any(axis=1).all():
        raise ValueError("a query sees no key")
    s = np.where(vis[:, None, :], scores, -np.inf)
    m = s.max(axis=2, keepdims=True)
    w = np.exp(s - m)  # exp(-inf) = 0 for hidden keys
    z = w.sum(axis=2, keepdims=True)
    lse = (m + np.log(z))[..., 0]
    out = np.matmul(w / z, values)
    return out, lse


def verify_attn_f64(q_lat: np.ndarray, q_pe: np.ndarray, ckv: np.ndarray, kpe: np.ndarray,
                    prefix_len: int, parents, scale: float = DEFAULT_SCALE):
    """One stream in float64: ``q_lat [Q,H,512]``, ``q_pe [Q,H,64]``, ``ckv [P+Q,512]``,
    ``kpe [P+Q,64]`` -> ``(out [Q,H,512], lse [Q,H])``."""
    q = len(parents)
    rows = prefix_len + q
    if q_lat.shape[0] != q or q_pe.shape[0] != q or ckv.shape[0] != rows or kpe.shape[0] != rows:
        raise ValueError("shape mismatch")
    vis = visibility(parents, prefix_len)
    s = scores_absorbed(q_lat, q_pe, ckv, kpe, scale)
    return masked_softmax_attention(s, vis, ckv)


def verify_attn_stream(q_lat_bits, q_pe_bits, ckv_bits, kpe_bits, prefix_len: int, parents,
                       scale: float = DEFAULT_SCALE):
    """One stream from bf16 bit patterns: ``q_lat [Q,H,512]``, ``q_pe [Q,H,64]``,
    ``ckv [>=P+Q, 512]``, ``kpe [>=P+Q, 64]``; rows past ``P + Q`` are ignored."""
    rows = prefix_len + len(parents)
    return verify_attn_f64(bf16_bits_to_f64(q_lat_bits), bf16_bits_to_f64(q_pe_bits),
                           bf16_bits_to_f64(ckv_bits[:rows]), bf16_bits_to_f64(kpe_bits[:rows]),
                           prefix_len, parents, scale)


def verify_attn(q_lat_bits, q_pe_bits, ckv_bits, kpe_bits, prefix_len: int, parents,
                scale: float = DEFAULT_SCALE, streams=None):
    """All streams (or the listed ones): ``out [S,Q,H,512]``, ``lse [S,Q,H]`` in float64.

    Streams are independent; each is processed on its own to bound memory.
    """
    parents = np.asarray(parents)
    idx = range(parents.shape[0]) if streams is None else list(streams)
    outs, lses = [], []
    for s in idx:
        o, l = verify_attn_stream(q_lat_bits[s], q_pe_bits[s], ckv_bits[s], kpe_bits[s],
                                  prefix_len, parents[s], scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def verify_attn_ragged(q_lat_bits, q_pe_bits, ckv_bits, kpe_bits, prefix_lens, parents,
                       scale: float = DEFAULT_SCALE):
    """Streams with their own prefix lengths: stream ``s`` is ``verify_attn_stream`` with
    ``prefix_lens[s]`` (its tree block at rows ``[prefix_lens[s], prefix_lens[s] + Q)``).

    After compaction each stream's committed prefix grows by its own accepted count ("Race
    Conditions, Buffer Aliasing, and the Architecture of a Native DDTree Inference Engine",
    section "The Cache Compaction Problem": the accepted rows join the prefix), so streams of one
    batch hold different prefix lengths.
    """
    parents = np.asarray(parents)
    outs, lses = [], []
    for s in range(parents.shape[0]):
        o, l = verify_attn_stream(q_lat_bits[s], q_pe_bits[s], ckv_bits[s], kpe_bits[s],
                                  int(prefix_lens[s]), parents[s], scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)
