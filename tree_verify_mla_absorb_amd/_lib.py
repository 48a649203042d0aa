"""Thin ctypes binding over ``libddtree.so`` (declared in ``include/ddtree.h``).

Argument marshalling only: torch supplies device memory and the current HIP stream; every step
of the computation runs in the library's gfx950 kernels.  There is no fallback: if the library
is missing or fails to load, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libddtree.so")

OK = 0
ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ALIAS, ERR_WORKSPACE, ERR_HIP = -1, -2, -3, -4, -5, -6
STATUS_BAD_PARENTS, STATUS_BAD_KEEP, STATUS_BAD_PREFIX, STATUS_BAD_POSITION = 1, 2, 4, 8
HEADS, D_LATENT, D_ROPE, MAX_Q_LEN, MAX_LAYERS = 64, 512, 64, 64, 128
NOALLOC_SCRATCH_BYTES = 64 << 20  # DDTREE_NOALLOC_SCRATCH_BYTES


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python tree_verify_mla_absorb_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.ddtree_verify_attn.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, vp, vp, vp]
    lib.ddtree_verify_attn.restype = i32
    lib.ddtree_verify_attn_ex.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, vp, vp, i32, f32, i32, vp, sz,
                                          vp, vp]
    lib.ddtree_verify_attn_ex.restype = i32
    lib.ddtree_verify_attn_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, vp, vp, i32, f32, i32, vp, vp]
    lib.ddtree_verify_attn_noalloc.restype = i32
    lib.ddtree_verify_attn_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.ddtree_verify_attn_workspace_size.restype = sz
    lib.ddtree_verify_attn_num_splits.argtypes = [i32, i32, i32, i32]
    lib.ddtree_verify_attn_num_splits.restype = i32
    lib.ddtree_compact_kv.argtypes = [vp, i32, vp, vp, i32, vp, vp]
    lib.ddtree_compact_kv.restype = i32
    lib.ddtree_tree_accept.argtypes = [vp, vp, vp, i32, i32, vp, i32, vp, vp, vp, vp]
    lib.ddtree_tree_accept.restype = i32
    lib.ddtree_accept_compact.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, vp, vp, vp, vp]
    lib.ddtree_accept_compact.restype = i32
    lib.ddtree_verify_attn_ragged.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, vp, i32, f32, i32, vp, sz,
                                              vp, vp]
    lib.ddtree_verify_attn_ragged.restype = i32
    lib.ddtree_compact_kv_ragged.argtypes = [vp, vp, vp, vp, i32, vp, vp]
    lib.ddtree_compact_kv_ragged.restype = i32
    lib.ddtree_accept_compact_ragged.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp, vp]
    lib.ddtree_accept_compact_ragged.restype = i32
    lib.ddtree_tree_build.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ddtree_tree_build.restype = i32
    lib.ddtree_compact_kv_layers.argtypes = [vp, i32, i32, vp, vp, vp, i32, vp, vp]
    lib.ddtree_compact_kv_layers.restype = i32
    lib.ddtree_accept_compact_layers.argtypes = [vp, i32, i32, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp, vp]
    lib.ddtree_accept_compact_layers.restype = i32
    lib.ddtree_append_tree_kv.argtypes = [vp, i32, vp, vp, i32, vp, vp, f32, vp, vp, i32, vp, vp]
    lib.ddtree_append_tree_kv.restype = i32
    lib.ddtree_status_string.argtypes = [i32]
    lib.ddtree_status_string.restype = ctypes.c_char_p
    lib.ddtree_version.argtypes = []
    lib.ddtree_version.restype = i32
    return lib


LIB = _load()

EXPORTED = (
    "ddtree_verify_attn",
    "ddtree_verify_attn_ex",
    "ddtree_verify_attn_noalloc",
    "ddtree_verify_attn_workspace_size",
    "ddtree_verify_attn_num_splits",
    "ddtree_compact_kv",
    "ddtree_tree_accept",
    "ddtree_accept_compact",
    "ddtree_verify_attn_ragged",
    "ddtree_compact_kv_ragged",
    "ddtree_accept_compact_ragged",
    "ddtree_tree_build",
    "ddtree_compact_kv_layers",
    "ddtree_accept_compact_layers",
    "ddtree_append_tree_kv",
    "ddtree_status_string",
    "ddtree_version",
)


class KVCache(ctypes.Structure):
    """``ddtree_kv_cache``: device pointers plus the per-stream row count."""

    _fields_ = [("ckv", ctypes.c_void_p), ("kpe", ctypes.c_void_p), ("kv_rows", ctypes.c_int),
                ("n_streams", ctypes.c_int)]


class DDTreeError(RuntimeError):
    def __init__(self, code: int):
        self.code = code
        super().__init__(f"ddtree error {code}: {status_string(code)}")


def status_string(code: int) -> str:
    return LIB.ddtree_status_string(int(code)).decode()


def version() -> int:
    return int(LIB.ddtree_version())


def _check(code: int) -> None:
    if code != OK:
        raise DDTreeError(code)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtypes, device=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


_BF16 = (torch.bfloat16, torch.int16)


def workspace_size(prefix_len: int, q_len: int, n_streams: int, num_splits: int = 0) -> int:
    return int(LIB.ddtree_verify_attn_workspace_size(prefix_len, q_len, n_streams, num_splits))


def num_splits(prefix_len: int, q_len: int, n_streams: int, num_splits: int = 0) -> int:
    n = int(LIB.ddtree_verify_attn_num_splits(prefix_len, q_len, n_streams, num_splits))
    _check(min(n, 0))
    return n


def _outputs(q_lat, out, lse):
    s, q, h = q_lat.shape[0], q_lat.shape[1], q_lat.shape[2]
    if out is None:
        out = torch.empty((s, q, h, D_LATENT), dtype=torch.float32, device=q_lat.device)
    if lse is None:
        lse = torch.empty((s, q, h), dtype=torch.float32, device=q_lat.device)
    _need(out, "out", (torch.float32,))
    _need(lse, "lse", (torch.float32,))
    return out, lse


def _shapes(q_lat, q_pe, ckv, kpe, parents):
    for t, n in ((q_lat, "q_lat"), (q_pe, "q_pe"), (ckv, "ckv"), (kpe, "kpe")):
        _need(t, n, _BF16)
    _need(parents, "parents", (torch.int32,))
    s, q = parents.shape
    if q_lat.shape != (s, q, HEADS, D_LATENT) or q_pe.shape != (s, q, HEADS, D_ROPE):
        raise ValueError("q_lat / q_pe shape mismatch")
    if ckv.shape[0] != s or ckv.shape[2] != D_LATENT or kpe.shape[:2] != ckv.shape[:2] or kpe.shape[2] != D_ROPE:
        raise ValueError("ckv / kpe shape mismatch")
    return s, q, ckv.shape[1]


def verify_attn(q_lat, q_pe, ckv, kpe, prefix_len: int, parents, *, out=None, lse=None, stream=None):
    """``ddtree_verify_attn``: one launch, no split, cache rows exactly ``prefix_len + q_len``."""
    s, q, rows = _shapes(q_lat, q_pe, ckv, kpe, parents)
    if rows != prefix_len + q:
        raise ValueError("ckv must hold exactly prefix_len + q_len rows per stream (use verify_attn_ex)")
    out, lse = _outputs(q_lat, out, lse)
    _check(LIB.ddtree_verify_attn(_ptr(q_lat), _ptr(q_pe), _ptr(ckv), _ptr(kpe), int(prefix_len), _ptr(parents),
                                  int(q), int(s), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def verify_attn_ex(q_lat, q_pe, ckv, kpe, prefix_len: int, parents, *, out=None, lse=None, scale: float = 0.0,
                   num_splits: int = 0, workspace=None, status=None, stream=None):
    """``ddtree_verify_attn_ex``.  ``workspace`` (uint8 device tensor) is allocated here when the
    chosen split count needs one and none is given."""
    s, q, rows = _shapes(q_lat, q_pe, ckv, kpe, parents)
    out, lse = _outputs(q_lat, out, lse)
    need = workspace_size(prefix_len, q, s, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_lat.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if status is not None:
        _need(status, "status", (torch.int32,))
    _check(LIB.ddtree_verify_attn_ex(_ptr(q_lat), _ptr(q_pe), _ptr(ckv), _ptr(kpe), int(prefix_len), _ptr(parents),
                                     int(q), int(s), _ptr(out), _ptr(lse), int(rows), float(scale),
                                     int(num_splits), _ptr(workspace), nbytes, _ptr(status), _stream(stream)))
    return out, lse


def verify_attn_noalloc(q_lat, q_pe, ckv, kpe, prefix_len: int, parents, *, out=None, lse=None, scale: float = 0.0,
                        num_splits: int = 0, status=None, stream=None):
    """``ddtree_verify_attn_noalloc``: ``verify_attn_ex`` with the split partials in the library's
    own scratch array (no workspace)."""
    s, q, rows = _shapes(q_lat, q_pe, ckv, kpe, parents)
    out, lse = _outputs(q_lat, out, lse)
    if status is not None:
        _need(status, "status", (torch.int32,))
    _check(LIB.ddtree_verify_attn_noalloc(_ptr(q_lat), _ptr(q_pe), _ptr(ckv), _ptr(kpe), int(prefix_len),
                                          _ptr(parents), int(q), int(s), _ptr(out), _ptr(lse), int(rows),
                                          float(scale), int(num_splits), _ptr(status), _stream(stream)))
    return out, lse


def verify_attn_ragged(q_lat, q_pe, ckv, kpe, prefix_lens, max_prefix_len: int, parents, *, out=None, lse=None,
                       scale: float = 0.0, num_splits: int = 0, workspace=None, status=None, stream=None):
    """``ddtree_verify_attn_ragged``: ``prefix_lens`` is a device int32 ``[S]`` tensor bounded by
    ``max_prefix_len``.  ``workspace`` is allocated here when needed and not given."""
    s, q, rows = _shapes(q_lat, q_pe, ckv, kpe, parents)
    _need(prefix_lens, "prefix_lens", (torch.int32,))
    if prefix_lens.shape != (s,):
        raise ValueError("prefix_lens must be [S]")
    out, lse = _outputs(q_lat, out, lse)
    need = workspace_size(max_prefix_len, q, s, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_lat.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if status is not None:
        _need(status, "status", (torch.int32,))
    _check(LIB.ddtree_verify_attn_ragged(_ptr(q_lat), _ptr(q_pe), _ptr(ckv), _ptr(kpe), _ptr(prefix_lens),
                                         int(max_prefix_len), _ptr(parents), int(q), int(s), _ptr(out), _ptr(lse),
                                         int(rows), float(scale), int(num_splits), _ptr(workspace), nbytes,
                                         _ptr(status), _stream(stream)))
    return out, lse


def compact_kv_ragged(ckv, kpe, prefix_lens, keep, n_keep, *, status=None, stream=None) -> None:
    """``ddtree_compact_kv_ragged`` in place; ``prefix_lens`` device int32 ``[S]``."""
    _need(ckv, "ckv", _BF16)
    _need(kpe, "kpe", _BF16)
    for t, name in ((prefix_lens, "prefix_lens"), (keep, "keep"), (n_keep, "n_keep")):
        _need(t, name, (torch.int32,))
    if status is not None:
        _need(status, "status", (torch.int32,))
    s, rows = ckv.shape[0], ckv.shape[1]
    if kpe.shape[:2] != (s, rows) or keep.dim() != 2 or keep.shape[0] != s or n_keep.shape != (s,) \
            or prefix_lens.shape != (s,):
        raise ValueError("shape mismatch")
    cache = KVCache(ckv.data_ptr(), kpe.data_ptr(), int(rows), int(s))
    _check(LIB.ddtree_compact_kv_ragged(ctypes.byref(cache), _ptr(prefix_lens), _ptr(keep), _ptr(n_keep),
                                        int(keep.shape[1]), _ptr(status), _stream(stream)))


def compact_kv(ckv, kpe, prefix_len: int, keep, n_keep, *, status=None, stream=None) -> None:
    """``ddtree_compact_kv`` in place on ``ckv [S, rows, 512]`` / ``kpe [S, rows, 64]``."""
    _need(ckv, "ckv", _BF16)
    _need(kpe, "kpe", _BF16)
    _need(keep, "keep", (torch.int32,))
    _need(n_keep, "n_keep", (torch.int32,))
    if status is not None:
        _need(status, "status", (torch.int32,))
    s, rows = ckv.shape[0], ckv.shape[1]
    if kpe.shape[:2] != (s, rows) or keep.dim() != 2 or keep.shape[0] != s or n_keep.shape != (s,):
        raise ValueError("shape mismatch")
    cache = KVCache(ckv.data_ptr(), kpe.data_ptr(), int(rows), int(s))
    _check(LIB.ddtree_compact_kv(ctypes.byref(cache), int(prefix_len), _ptr(keep), _ptr(n_keep), int(keep.shape[1]),
                                 _ptr(status), _stream(stream)))


def _accept_inputs(parents, draft_tokens, target_tokens, keep, n_keep, next_token, status):
    for t, name in ((parents, "parents"), (draft_tokens, "draft_tokens"), (target_tokens, "target_tokens")):
        _need(t, name, (torch.int32,))
    if parents.dim() != 2 or draft_tokens.shape != parents.shape or target_tokens.shape != parents.shape:
        raise ValueError("parents / draft_tokens / target_tokens must share one [S, Q] shape")
    s, q = parents.shape
    dev = parents.device
    if keep is None:
        keep = torch.full((s, q), -1, dtype=torch.int32, device=dev)
    if n_keep is None:
        n_keep = torch.empty((s,), dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty((s,), dtype=torch.int32, device=dev)
    _need(keep, "keep", (torch.int32,))
    _need(n_keep, "n_keep", (torch.int32,))
    _need(next_token, "next_token", (torch.int32,))
    if status is not None:
        _need(status, "status", (torch.int32,))
    if keep.dim() != 2 or keep.shape[0] != s or n_keep.shape != (s,) or next_token.shape != (s,):
        raise ValueError("output shape mismatch")
    return s, q, keep, n_keep, next_token


def tree_accept(parents, draft_tokens, target_tokens, *, keep=None, n_keep=None, next_token=None, status=None,
                stream=None):
    """``ddtree_tree_accept``: greedy acceptance; returns ``(keep [S, K], n_keep [S], next_token [S])``."""
    s, q, keep, n_keep, next_token = _accept_inputs(parents, draft_tokens, target_tokens, keep, n_keep, next_token,
                                                    status)
    _check(LIB.ddtree_tree_accept(_ptr(parents), _ptr(draft_tokens), _ptr(target_tokens), int(q), int(s), _ptr(keep),
                                  int(keep.shape[1]), _ptr(n_keep), _ptr(next_token), _ptr(status),
                                  _stream(stream)))
    return keep, n_keep, next_token


def accept_compact(ckv, kpe, prefix_len: int, parents, draft_tokens, target_tokens, *, keep=None, n_keep=None,
                   next_token=None, status=None, stream=None):
    """``ddtree_accept_compact``: acceptance, then the in-place compaction of ``ckv`` / ``kpe``, in one
    launch; returns ``(keep, n_keep, next_token)``."""
    _need(ckv, "ckv", _BF16)
    _need(kpe, "kpe", _BF16)
    s, q, keep, n_keep, next_token = _accept_inputs(parents, draft_tokens, target_tokens, keep, n_keep, next_token,
                                                    status)
    rows = ckv.shape[1]
    if ckv.shape[0] != s or kpe.shape[:2] != (s, rows):
        raise ValueError("shape mismatch")
    cache = KVCache(ckv.data_ptr(), kpe.data_ptr(), int(rows), int(s))
    _check(LIB.ddtree_accept_compact(ctypes.byref(cache), int(prefix_len), _ptr(parents), _ptr(draft_tokens),
                                     _ptr(target_tokens), int(q), _ptr(keep), int(keep.shape[1]), _ptr(n_keep),
                                     _ptr(next_token), _ptr(status), _stream(stream)))
    return keep, n_keep, next_token


def accept_compact_ragged(ckv, kpe, prefix_lens, parents, draft_tokens, target_tokens, *, keep=None, n_keep=None,
                          next_token=None, status=None, stream=None):
    """``ddtree_accept_compact_ragged``: like ``accept_compact`` with a device int32 ``[S]``
    ``prefix_lens``, which the call advances by each stream's accepted count."""
    _need(ckv, "ckv", _BF16)
    _need(kpe, "kpe", _BF16)
    _need(prefix_lens, "prefix_lens", (torch.int32,))
    s, q, keep, n_keep, next_token = _accept_inputs(parents, draft_tokens, target_tokens, keep, n_keep, next_token,
                                                    status)
    rows = ckv.shape[1]
    if ckv.shape[0] != s or kpe.shape[:2] != (s, rows) or prefix_lens.shape != (s,):
        raise ValueError("shape mismatch")
    cache = KVCache(ckv.data_ptr(), kpe.data_ptr(), int(rows), int(s))
    _check(LIB.ddtree_accept_compact_ragged(ctypes.byref(cache), _ptr(prefix_lens), _ptr(parents),
                                            _ptr(draft_tokens), _ptr(target_tokens), int(q), _ptr(keep),
                                            int(keep.shape[1]), _ptr(n_keep), _ptr(next_token), _ptr(status),
                                            _stream(stream)))
    return keep, n_keep, next_token


def _layer_table(caches):
    """``caches``: a sequence of ``(ckv [S, rows, 512], kpe [S, rows, 64])`` pairs, one per layer."""
    caches = list(caches)
    if not caches:
        raise ValueError("at least one layer")
    table = (KVCache * len(caches))()
    for i, (ckv, kpe) in enumerate(caches):
        _need(ckv, f"caches[{i}].ckv", _BF16)
        _need(kpe, f"caches[{i}].kpe", _BF16)
        if kpe.shape[:2] != ckv.shape[:2]:
            raise ValueError("shape mismatch")
        table[i] = KVCache(ckv.data_ptr(), kpe.data_ptr(), int(ckv.shape[1]), int(ckv.shape[0]))
    return table, int(caches[0][0].shape[0])


def _prefix_arg(prefix, s):
    """An int (every stream) or a device int32 ``[S]`` tensor (per stream)."""
    if isinstance(prefix, torch.Tensor):
        _need(prefix, "prefix_lens", (torch.int32,))
        if prefix.shape != (s,):
            raise ValueError("prefix_lens must be [S]")
        return 0, _ptr(prefix)
    return int(prefix), None


def compact_kv_layers(caches, prefix, keep, n_keep, *, status=None, stream=None) -> None:
    """``ddtree_compact_kv_layers``: the compaction of ``compact_kv`` (``prefix`` an int) or
    ``compact_kv_ragged`` (``prefix`` a device int32 ``[S]``, read only) applied to every layer's
    ``(ckv, kpe)`` in ``caches``, in one launch."""
    table, s = _layer_table(caches)
    _need(keep, "keep", (torch.int32,))
    _need(n_keep, "n_keep", (torch.int32,))
    if status is not None:
        _need(status, "status", (torch.int32,))
    if keep.dim() != 2 or keep.shape[0] != s or n_keep.shape != (s,):
        raise ValueError("shape mismatch")
    p, pl = _prefix_arg(prefix, s)
    _check(LIB.ddtree_compact_kv_layers(table, len(table), p, pl, _ptr(keep), _ptr(n_keep), int(keep.shape[1]),
                                        _ptr(status), _stream(stream)))


def accept_compact_layers(caches, prefix, parents, draft_tokens, target_tokens, *, keep=None, n_keep=None,
                          next_token=None, status=None, stream=None):
    """``ddtree_accept_compact_layers``: acceptance once, then the compaction of every layer's
    ``(ckv, kpe)``.  ``prefix`` is an int (every stream) or a device int32 ``[S]`` tensor, which the
    call advances by each stream's accepted count.  Returns ``(keep, n_keep, next_token)``."""
    table, s = _layer_table(caches)
    s2, q, keep, n_keep, next_token = _accept_inputs(parents, draft_tokens, target_tokens, keep, n_keep,
                                                     next_token, status)
    if s2 != s:
        raise ValueError("shape mismatch")
    p, pl = _prefix_arg(prefix, s)
    _check(LIB.ddtree_accept_compact_layers(table, len(table), p, pl, _ptr(parents), _ptr(draft_tokens),
                                            _ptr(target_tokens), int(q), _ptr(keep), int(keep.shape[1]),
                                            _ptr(n_keep), _ptr(next_token), _ptr(status), _stream(stream)))
    return keep, n_keep, next_token


def append_tree_kv(ckv, kpe, prefix, parents, kv, norm_weight, eps: float, rope_cos, rope_sin, *, status=None,
                   stream=None) -> None:
    """``ddtree_append_tree_kv``: write every stream's tree rows into ``ckv [S, rows, 512]`` /
    ``kpe [S, rows, 64]`` at ``prefix`` (an int, or a device int32 ``[S]``): RMSNorm of
    ``kv [S, Q, 576]``'s latent part with ``norm_weight [512]``, NeoX rotation of its rotary part
    by ``rope_cos`` / ``rope_sin [rows, 32]`` at position prefix + depth (all fp32)."""
    _need(ckv, "ckv", _BF16)
    _need(kpe, "kpe", _BF16)
    _need(parents, "parents", (torch.int32,))
    for t, name in ((kv, "kv"), (norm_weight, "norm_weight"), (rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
        _need(t, name, (torch.float32,))
    if status is not None:
        _need(status, "status", (torch.int32,))
    s, rows = ckv.shape[0], ckv.shape[1]
    if parents.dim() != 2 or parents.shape[0] != s:
        raise ValueError("parents must be [S, Q]")
    q = parents.shape[1]
    if kpe.shape[:2] != (s, rows) or kv.shape != (s, q, D_LATENT + D_ROPE) or norm_weight.shape != (D_LATENT,) \
            or rope_cos.dim() != 2 or rope_cos.shape[1] != 32 or rope_sin.shape != rope_cos.shape:
        raise ValueError("shape mismatch")
    p, pl = _prefix_arg(prefix, s)
    cache = KVCache(ckv.data_ptr(), kpe.data_ptr(), int(rows), int(s))
    _check(LIB.ddtree_append_tree_kv(ctypes.byref(cache), p, pl, _ptr(parents), int(q), _ptr(kv), _ptr(norm_weight),
                                     float(eps), _ptr(rope_cos), _ptr(rope_sin), int(rope_cos.shape[0]),
                                     _ptr(status), _stream(stream)))


def tree_build(logprobs, topk_tokens, budget: int, *, root_tokens=None, extras: bool = False, stream=None):
    """``ddtree_tree_build``: ``logprobs`` fp32 ``[S, D, K]`` (rows decreasing), ``topk_tokens`` int32
    ``[S, D, K]``.  Returns ``(parents, node_tokens, n_nodes)`` (``[S, budget + 1]`` rows); with
    ``extras`` also a dict of depths, logw, first_child, next_sibling and anc (int64 view of the
    uint64 masks)."""
    _need(logprobs, "logprobs", (torch.float32,))
    _need(topk_tokens, "topk_tokens", (torch.int32,))
    if logprobs.dim() != 3 or topk_tokens.shape != logprobs.shape:
        raise ValueError("logprobs / topk_tokens must share one [S, D, K] shape")
    if root_tokens is not None:
        _need(root_tokens, "root_tokens", (torch.int32,))
    s, d, k = logprobs.shape
    q = int(budget) + 1
    dev = logprobs.device
    parents = torch.full((s, q), -2, dtype=torch.int32, device=dev)
    tokens = torch.full((s, q), -2, dtype=torch.int32, device=dev)
    n_nodes = torch.empty((s,), dtype=torch.int32, device=dev)
    ex = {}
    if extras:
        ex = {"depths": torch.full((s, q), -2, dtype=torch.int32, device=dev),
              "logw": torch.full((s, q), float("nan"), dtype=torch.float32, device=dev),
              "first_child": torch.full((s, q), -2, dtype=torch.int32, device=dev),
              "next_sibling": torch.full((s, q), -2, dtype=torch.int32, device=dev),
              "anc": torch.zeros((s, q), dtype=torch.int64, device=dev)}
    _check(LIB.ddtree_tree_build(_ptr(logprobs), _ptr(topk_tokens), _ptr(root_tokens), int(d), int(k), int(budget),
                                 int(s), _ptr(parents), _ptr(tokens), _ptr(n_nodes), _ptr(ex.get("depths")),
                                 _ptr(ex.get("logw")), _ptr(ex.get("first_child")), _ptr(ex.get("next_sibling")),
                                 _ptr(ex.get("anc")), _stream(stream)))
    if extras:
        return parents, tokens, n_nodes, ex
    return parents, tokens, n_nodes
