"""Oracle: post-accept KV cache compaction (out-of-place gather).

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring).

"Race Conditions, Buffer Aliasing, and the Architecture of a Native DDTree Inference Engine",
section "The Cache Compaction Problem": after verification the accepted tokens form a path
through the tree; their rows are gathered from the appended block into a contiguous run right
after the prefix.  ``keep`` maps each new position ``i`` to an old block position, and because a
child always comes after its parent the kept positions are strictly increasing, so
``keep[i] >= i``.  The page shows that doing this gather in place with many threads races (a
reader of row ``P + keep[j]`` can meet the writer of that same row) and fixes it by gathering
into scratch first.  Fancy indexing on a snapshot is that out-of-place gather by construction.

Readings: ``keep`` indexes the tree block (row ``P + keep[i]``); rows outside
``[P, P + n_keep)`` are left bit-identical; ``n_keep == 0`` is a no-op.
"""
from __future__ import annotations

import numpy as np


def validate_keep(keep_row: np.ndarray, n: int, prefix_len: int, kv_rows: int) -> None:
    keep_row = np.asarray(keep_row, dtype=np.int64)
    if n < 0 or n > len(keep_row):
        raise ValueError("n_keep out of range")
    k = keep_row[:n]
    if n and (k[0] < 0 or prefix_len + k[-1] >= kv_rows):
        raise ValueError("keep index out of range")
    if n > 1 and not (np.diff(k) > 0).all():
        raise ValueError("keep must be strictly increasing")


def compact_kv(ckv_bits: np.ndarray, kpe_bits: np.ndarray, prefix_len: int, keep: np.ndarray,
               n_keep: np.ndarray):
    """Return new ``(ckv, kpe)`` arrays ``[S, rows, 512]`` / ``[S, rows, 64]`` after the gather.

    For every stream ``s`` and ``i < n_keep[s]``: row ``P + i`` takes the old row
    ``P + keep[s, i]``.  Inputs are never modified.
    """
    old_c = np.asarray(ckv_bits)
    old_k = np.asarray(kpe_bits)
    new_c = old_c.copy()
    new_k = old_k.copy()
    for s in range(old_c.shape[0]):
        n = int(n_keep[s])
        validate_keep(keep[s], n, prefix_len, old_c.shape[1])
        src = prefix_len + np.asarray(keep[s][:n], dtype=np.int64)
        new_c[s, prefix_len:prefix_len + n] = old_c[s, src]
        new_k[s, prefix_len:prefix_len + n] = old_k[s, src]
    return new_c, new_k


def compact_kv_ragged(ckv_bits: np.ndarray, kpe_bits: np.ndarray, prefix_lens, keep: np.ndarray,
                      n_keep: np.ndarray):
    """``compact_kv`` with a prefix length per stream: for every stream ``s`` and
    ``i < n_keep[s]``, row ``prefix_lens[s] + i`` takes the old row ``prefix_lens[s] + keep[s, i]``."""
    new_c = np.array(ckv_bits, copy=True)
    new_k = np.array(kpe_bits, copy=True)
    for s in range(new_c.shape[0]):
        c, k = compact_kv(ckv_bits[s:s + 1], kpe_bits[s:s + 1], int(prefix_lens[s]), keep[s:s + 1],
                          n_keep[s:s + 1])
        new_c[s], new_k[s] = c[0], k[0]
    return new_c, new_k
