"""Oracle: the draft tree's key/value rows written into the latent cache at their offset.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring).

What is computed, and which passages it follows
------------------------------------------------
"Race Conditions, Buffer Aliasing, and the Architecture of a Native DDTree Inference Engine":

* section "Scratch Buffer Architecture: Managing Transformer Activations": the key/value
  projection's GEMM yields un-normalised activations; RMSNorm normalises them and writes the
  result straight into the cache at the right offset;
* section "Assumptions, Input Knowledge, and Output Knowledge": the model is DeepSeek-V3 / Kimi
  style (MLA, RMSNorm, NeoX rotary embeddings);
* section "The Cache Compaction Problem": tree node ``i`` occupies cache row ``P + i`` after a
  ``P``-row prefix.

Readings (the pages name the steps, not their formulas):

* The input row of a node is the projection's float32 output, 576 values: 512 latent values, then
  64 rotary values (the split the absorbed attention reads back as ``c_kv`` and ``k_pe``).
* Latent part, RMSNorm: ``y = x / sqrt(mean(x**2) + eps) * w`` with the norm's weight ``w``
  (512 values).
* Rotary part, NeoX rotation: the two 32-value halves rotate as pairs ``(j, j + 32)`` by the
  caller's tables at the node's position: ``out[j] = x[j] cos - x[j+32] sin``,
  ``out[j+32] = x[j+32] cos + x[j] sin`` (``cos``, ``sin`` rows of 32 values per position).
* Position of node ``i``: ``P + depth(i)``.  The root (depth 0) is the token right after the
  ``P`` committed rows (positions ``0 .. P-1``); siblings are alternatives for one position.
* Stored values: bf16, the exact result rounded to nearest, ties to even.
"""
from __future__ import annotations

import math

import numpy as np

D_LATENT = 512
D_ROPE = 64
HALF = D_ROPE // 2


def bf16_round_bits(v) -> np.ndarray:
    """float64 values -> bf16 bit patterns (uint16), rounded once, to nearest, ties to even.

    The value is scaled to the bf16 significand grid of its binade (8 significant bits; below
    2**-126 the fixed subnormal spacing 2**-133) and rounded there, so there is no intermediate
    rounding to float32.  Values beyond the largest bf16 round to infinity; NaN stays NaN."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    for idx, x in np.ndenumerate(v):
        if math.isnan(x):
            out[idx] = 0x7FC0
            continue
        sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
        a = abs(x)
        if a == 0.0:
            out[idx] = sign
            continue
        if math.isinf(a):
            out[idx] = sign | 0x7F80
            continue
        _, e = math.frexp(a)                   # a = m * 2**e, m in [0.5, 1)
        ulp_exp = max(e - 1, -126) - 7         # bf16 spacing in a's binade
        q = a / math.ldexp(1.0, ulp_exp)       # exact: a power-of-two scaling
        r = math.floor(q)
        frac = q - r
        if frac > 0.5 or (frac == 0.5 and r % 2 == 1):
            r += 1
        rounded = math.ldexp(float(r), ulp_exp)
        if rounded >= math.ldexp(1.0, 128):    # past the largest bf16 (overflow)
            out[idx] = sign | 0x7F80
            continue
        bits = int(np.array(rounded, dtype=np.float32).view(np.uint32)) >> 16  # exact in fp32
        out[idx] = sign | bits
    return out


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of one latent row in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / math.sqrt(float(np.mean(x * x)) + eps) * np.asarray(weight, dtype=np.float64)


def rope_neox(x: np.ndarray, cos_row: np.ndarray, sin_row: np.ndarray) -> np.ndarray:
    """NeoX rotation of one 64-value rotary row by one position's 32 (cos, sin) pairs."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(cos_row, dtype=np.float64)
    s = np.asarray(sin_row, dtype=np.float64)
    lo, hi = x[:HALF], x[HALF:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s])


def tree_depths(parents: np.ndarray) -> np.ndarray:
    """Depth of every node (root 0); ``parents[0] == -1`` and every other parent is an earlier
    node, else ValueError."""
    parents = np.asarray(parents, dtype=np.int64)
    if len(parents) < 1 or parents[0] != -1:
        raise ValueError("parents[0] must be -1")
    depth = np.zeros(len(parents), np.int64)
    for i in range(1, len(parents)):
        if not 0 <= parents[i] < i:
            raise ValueError(f"parents[{i}]={parents[i]} is not an earlier node")
        depth[i] = depth[parents[i]] + 1
    return depth


def tree_rows(kv: np.ndarray, weight: np.ndarray, eps: float, rope_cos: np.ndarray, rope_sin: np.ndarray,
              prefix_len: int, parents: np.ndarray):
    """The cache rows of one stream's tree: ``(ckv bits [Q, 512], kpe bits [Q, 64])``.

    ``kv``: float32 ``[Q, 576]``; ``rope_cos`` / ``rope_sin``: ``[rows, 32]``."""
    kv = np.asarray(kv, dtype=np.float32)
    depth = tree_depths(parents)
    q = kv.shape[0]
    ckv = np.empty((q, D_LATENT), np.uint16)
    kpe = np.empty((q, D_ROPE), np.uint16)
    for i in range(q):
        pos = prefix_len + int(depth[i])
        if not 0 <= pos < len(rope_cos):
            raise ValueError(f"position {pos} outside the rotary tables")
        ckv[i] = bf16_round_bits(rms_norm(kv[i, :D_LATENT], weight, eps))
        kpe[i] = bf16_round_bits(rope_neox(kv[i, D_LATENT:], rope_cos[pos], rope_sin[pos]))
    return ckv, kpe


def append_tree_kv(ckv_bits: np.ndarray, kpe_bits: np.ndarray, kv: np.ndarray, weight: np.ndarray, eps: float,
                   rope_cos: np.ndarray, rope_sin: np.ndarray, prefix_lens, parents: np.ndarray):
    """New ``(ckv, kpe)`` cache arrays ``[S, rows, .]`` with every stream's tree rows written at
    ``[prefix_lens[s], prefix_lens[s] + Q)``; all other rows unchanged.  Inputs are not modified."""
    new_c = np.array(ckv_bits, copy=True)
    new_k = np.array(kpe_bits, copy=True)
    q = kv.shape[1]
    for s in range(new_c.shape[0]):
        p = int(prefix_lens[s])
        if p < 0 or p + q > new_c.shape[1]:
            raise ValueError("tree block outside the cache")
        new_c[s, p:p + q], new_k[s, p:p + q] = tree_rows(kv[s], weight, eps, rope_cos, rope_sin, p, parents[s])
    return new_c, new_k
