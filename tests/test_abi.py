"""The C-ABI library on the CPU: it loads, exports every function ``include/ddtree.h`` declares,
and rejects invalid arguments with the documented codes before anything is launched.

Every call here is built to fail host-side validation (the fake pointers are never
dereferenced), so no kernel is ever launched from these tests.
"""
import ctypes
import os
import re

import pytest

from tree_verify_mla_absorb_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ddtree.h")

A = 0x10000  # fake, 16-byte aligned device addresses, far apart
B = 0x20000000
C = 0x40000000
D = 0x60000000
E = 0x80000000
F = 0xA0000000
G = 0xC0000000


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(ddtree_[a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert names == sorted(_lib.EXPORTED), names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert _lib.version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert _lib.status_string(code) not in ("", "unknown status")
    assert _lib.status_string(-99) == "unknown status"


def verify(q_lat=A, q_pe=B, ckv=C, kpe=D, prefix=100, parents=E, q=9, s=2, out=F, lse=G, rows=None, splits=1,
           ws=None, ws_bytes=0, status=None, scale=0.0):
    rows = prefix + q if rows is None else rows
    return _lib.LIB.ddtree_verify_attn_ex(q_lat, q_pe, ckv, kpe, prefix, parents, q, s, out, lse, rows, scale,
                                          splits, ws, ws_bytes, status, None)


@pytest.mark.parametrize("field", ["q_lat", "q_pe", "ckv", "kpe", "parents", "out", "lse"])
def test_null_pointers(field):
    kw = {field: None}
    assert verify(**kw) == _lib.ERR_NULL
    assert verify(**kw, q=0) == _lib.ERR_NULL  # NULL is reported first


@pytest.mark.parametrize("kw", [dict(q=0), dict(q=65), dict(s=0), dict(prefix=-1), dict(rows=50),
                                dict(splits=-1)])
def test_bad_shapes(kw):
    assert verify(**kw) == _lib.ERR_SHAPE


def test_plain_entry_rejects_shapes():
    f = _lib.LIB.ddtree_verify_attn
    assert f(A, B, C, D, 10, E, 65, 1, F, G, None) == _lib.ERR_SHAPE
    assert f(A, B, C, D, 10, E, 9, 0, F, G, None) == _lib.ERR_SHAPE
    assert f(None, B, C, D, 10, E, 9, 1, F, G, None) == _lib.ERR_NULL


@pytest.mark.parametrize("field", ["q_lat", "q_pe", "ckv", "kpe", "out"])
def test_misaligned(field):
    base = {"q_lat": A, "q_pe": B, "ckv": C, "kpe": D, "out": F}[field]
    assert verify(**{field: base + 8}) == _lib.ERR_ALIGN


def test_aliasing_outputs():
    assert verify(out=A) == _lib.ERR_ALIAS          # out over q_lat
    assert verify(lse=C + 64) == _lib.ERR_ALIAS     # lse inside ckv
    assert verify(lse=F + 1024) == _lib.ERR_ALIAS   # lse inside out


def test_workspace_required_for_splits():
    need = _lib.workspace_size(1000, 9, 2, 4)
    assert _lib.num_splits(1000, 9, 2, 4) == 4

    def a256(x):
        return (x + 255) // 256 * 256
    # node pairs: 2 streams x 4 pairs x 128 rows; last node: 2 streams x 64 rows; 4 splits each
    rows0, rows1 = 2 * 4 * 128, 2 * 64
    assert need == (a256(4 * rows0 * 512 * 4) + a256(4 * rows1 * 512 * 4) + a256(4 * rows0 * 4)
                    + a256(4 * rows1 * 4))
    assert verify(prefix=1000, splits=4) == _lib.ERR_WORKSPACE
    assert verify(prefix=1000, splits=4, ws=0x100000000, ws_bytes=need - 4) == _lib.ERR_WORKSPACE
    assert verify(prefix=1000, splits=4, ws=0x100000008, ws_bytes=need) == _lib.ERR_WORKSPACE  # misaligned
    assert verify(prefix=1000, splits=4, ws=F, ws_bytes=need) == _lib.ERR_ALIAS  # workspace over out


def test_split_queries():
    assert _lib.workspace_size(100, 9, 1, 1) == 0
    assert _lib.LIB.ddtree_verify_attn_workspace_size(100, 0, 1, 1) == 0
    assert _lib.LIB.ddtree_verify_attn_num_splits(100, 65, 1, 1) == _lib.ERR_SHAPE
    # splits never exceed the number of 32-key tiles and every split is non-empty
    assert _lib.num_splits(0, 9, 1, 32) == 1          # 9 keys: one tile
    assert _lib.num_splits(100, 9, 1, 32) == 4        # 109 keys: four tiles
    assert _lib.num_splits(4096, 33, 1, 13) == 13     # 130 tiles: 10 per split
    assert _lib.num_splits(4096, 33, 1, 40) == 33     # 130 tiles: 4 per split -> 33 splits
    assert _lib.num_splits(8192, 17, 1, 64) == 52     # 257 tiles: 5 per split -> 52 splits
    assert _lib.num_splits(8192, 17, 1, 1000) == 52   # requests above 64 are taken as 64
    assert _lib.num_splits(100, 9, 2, 64) == 4        # never more splits than tiles


def compact(ckv=A, kpe=C, rows=300, s=2, prefix=100, keep=E, n_keep=F, stride=33, status=None, cache=True):
    c = _lib.KVCache(ckv, kpe, rows, s)
    return _lib.LIB.ddtree_compact_kv(ctypes.byref(c) if cache else None, prefix, keep, n_keep, stride, status,
                                      None)


def test_compact_argument_errors():
    assert compact(cache=False) == _lib.ERR_NULL
    assert compact(ckv=None) == _lib.ERR_NULL
    assert compact(keep=None) == _lib.ERR_NULL
    assert compact(n_keep=None) == _lib.ERR_NULL
    assert compact(s=0) == _lib.ERR_SHAPE
    assert compact(prefix=-1) == _lib.ERR_SHAPE
    assert compact(prefix=301) == _lib.ERR_SHAPE
    assert compact(stride=0) == _lib.ERR_SHAPE
    assert compact(ckv=A + 8) == _lib.ERR_ALIGN
    assert compact(keep=E + 2) == _lib.ERR_ALIGN
    assert compact(kpe=A + 1024) == _lib.ERR_ALIAS


def accept(parents=A, draft=B, target=C, q=9, s=2, keep=D, stride=9, n_keep=E, nxt=F, status=None):
    return _lib.LIB.ddtree_tree_accept(parents, draft, target, q, s, keep, stride, n_keep, nxt, status, None)


def test_accept_argument_errors():
    for field in ("parents", "draft", "target", "keep", "n_keep"):
        assert accept(**{field: None}) == _lib.ERR_NULL
    assert accept(q=0) == _lib.ERR_SHAPE
    assert accept(q=65, stride=65) == _lib.ERR_SHAPE
    assert accept(s=0) == _lib.ERR_SHAPE
    assert accept(stride=8) == _lib.ERR_SHAPE          # keep rows must hold a full-length path
    assert accept(keep=D + 2) == _lib.ERR_ALIGN
    assert accept(nxt=F + 1) == _lib.ERR_ALIGN
    assert accept(keep=A) == _lib.ERR_ALIAS             # keep over parents
    assert accept(n_keep=D + 8) == _lib.ERR_ALIAS       # n_keep inside keep
    assert accept(nxt=E + 4) == _lib.ERR_ALIAS          # next_token over n_keep
    assert accept(nxt=None, n_keep=C + 16) == _lib.ERR_ALIAS  # n_keep inside target


def accept_compact(rows=300, s=2, prefix=100, q=9, keep=D, nxt=F, parents=A, cache=True):
    c = _lib.KVCache(G, G + 0x10000000, rows, s)
    return _lib.LIB.ddtree_accept_compact(ctypes.byref(c) if cache else None, prefix, parents, B, C, q, keep, q, E,
                                          nxt, None, None)


def test_accept_compact_argument_errors():
    assert accept_compact(cache=False) == _lib.ERR_NULL
    assert accept_compact(parents=None) == _lib.ERR_NULL
    assert accept_compact(prefix=292) == _lib.ERR_SHAPE   # tree block past the cache rows
    assert accept_compact(s=0) == _lib.ERR_SHAPE
    assert accept_compact(keep=G + 64) == _lib.ERR_ALIAS  # keep inside the latent cache


def test_ragged_argument_errors():
    L = _lib.LIB
    # verify: prefix_lens is required; max_prefix_len bounds kv_rows like prefix_len does
    assert L.ddtree_verify_attn_ragged(A, B, C, D, None, 100, E, 9, 2, F, G, 109, 0.0, 1, None, 0, None,
                                       None) == _lib.ERR_NULL
    assert L.ddtree_verify_attn_ragged(A, B, C, D, 0xE0000000, 100, E, 9, 2, F, G, 108, 0.0, 1, None, 0, None,
                                       None) == _lib.ERR_SHAPE
    assert L.ddtree_verify_attn_ragged(A, B, C, D, 0xE0000002, 100, E, 9, 2, F, G, 109, 0.0, 1, None, 0, None,
                                       None) == _lib.ERR_ALIGN
    assert L.ddtree_verify_attn_ragged(A, B, C, D, F, 100, E, 9, 2, F, G, 109, 0.0, 1, None, 0, None,
                                       None) == _lib.ERR_ALIAS  # prefix_lens over out
    c = _lib.KVCache(G, G + 0x10000000, 300, 2)
    assert L.ddtree_compact_kv_ragged(ctypes.byref(c), None, E, F, 9, None, None) == _lib.ERR_NULL
    assert L.ddtree_compact_kv_ragged(ctypes.byref(c), G + 64, E, F, 9, None, None) == _lib.ERR_ALIAS
    assert L.ddtree_accept_compact_ragged(ctypes.byref(c), None, A, B, C, 9, D, 9, E, F, None, None) == _lib.ERR_NULL
    assert L.ddtree_accept_compact_ragged(ctypes.byref(c), D + 8, A, B, C, 9, D, 9, E, F, None,
                                          None) == _lib.ERR_ALIAS  # prefix_lens inside keep


def build(lp=A, tok=B, d=8, k=4, budget=32, s=2, parents=C, tokens=D, n_nodes=E, anc=None):
    return _lib.LIB.ddtree_tree_build(lp, tok, None, d, k, budget, s, parents, tokens, n_nodes, None, None, None, None,
                                      anc, None)


def test_build_argument_errors():
    for field in ("lp", "tok", "parents", "tokens", "n_nodes"):
        assert build(**{field: None}) == _lib.ERR_NULL
    for kw in (dict(d=0), dict(d=65), dict(k=0), dict(k=65), dict(budget=0), dict(budget=64), dict(s=0)):
        assert build(**kw) == _lib.ERR_SHAPE
    assert build(lp=A + 2) == _lib.ERR_ALIGN
    assert build(anc=F + 4) == _lib.ERR_ALIGN
    assert build(parents=A) == _lib.ERR_ALIAS            # output over an input
    assert build(tokens=C + 4 * 33) == _lib.ERR_ALIAS    # node_tokens inside parents ([2][33] int32)


def layer_table(n, rows=300, s=2, bad=None):
    """n fake caches, far apart above 4 GiB; ``bad`` = (layer, field, value) overrides one entry."""
    t = (_lib.KVCache * max(n, 1))()
    for i in range(n):
        t[i] = _lib.KVCache(0x100000000 + i * 0x200000, 0x100000000 + i * 0x200000 + 0x100000, rows, s)
    if bad is not None:
        setattr(t[bad[0]], bad[1], bad[2])
    return t


def compact_layers(n=4, prefix=100, prefix_lens=None, keep=E, n_keep=F, stride=33, table=None):
    t = layer_table(n) if table is None else table
    return _lib.LIB.ddtree_compact_kv_layers(t, n, prefix, prefix_lens, keep, n_keep, stride, None, None)


def accept_layers(n=4, prefix=100, prefix_lens=None, q=9, keep=D, parents=A, table=None):
    t = layer_table(n) if table is None else table
    return _lib.LIB.ddtree_accept_compact_layers(t, n, prefix, prefix_lens, parents, B, C, q, keep, q, E, F, None,
                                                 None)


@pytest.mark.parametrize("call", [compact_layers, accept_layers])
def test_layers_argument_errors(call):
    assert call(table=None, n=0) == _lib.ERR_SHAPE
    assert call(n=_lib.MAX_LAYERS + 1) == _lib.ERR_SHAPE
    assert call(table=layer_table(4, bad=(2, "ckv", None))) == _lib.ERR_NULL
    assert call(table=layer_table(4, bad=(3, "kv_rows", 301))) == _lib.ERR_SHAPE     # geometry differs
    assert call(table=layer_table(4, bad=(1, "n_streams", 3))) == _lib.ERR_SHAPE
    assert call(table=layer_table(4, bad=(2, "kpe", 0x100000000 + 2 * 0x200000 + 8))) == _lib.ERR_ALIGN
    # layer 3's latent cache starts inside layer 2's
    assert call(table=layer_table(4, bad=(3, "ckv", 0x100000000 + 2 * 0x200000 + 0x1000))) == _lib.ERR_ALIAS
    # the last of 128 layers is checked too
    t = layer_table(_lib.MAX_LAYERS, bad=(_lib.MAX_LAYERS - 1, "kpe", 0x100000000 + 5 * 0x200000))
    assert call(n=_lib.MAX_LAYERS, table=t) == _lib.ERR_ALIAS
    assert call(keep=0x100000000 + 3 * 0x200000 + 0x100040) == _lib.ERR_ALIAS       # keep inside layer 3's kpe
    assert call(prefix=-1) == _lib.ERR_SHAPE
    assert call(prefix_lens=G + 2) == _lib.ERR_ALIGN


def test_layers_prefix_bounds():
    assert compact_layers(prefix=301) == _lib.ERR_SHAPE          # prefix past the cache rows
    assert accept_layers(prefix=292) == _lib.ERR_SHAPE           # tree block past the cache rows
    assert accept_layers(prefix=-5, prefix_lens=G, q=0) == _lib.ERR_SHAPE
    assert accept_layers(prefix_lens=D + 8) == _lib.ERR_ALIAS    # prefix_lens inside keep
    assert compact_layers(keep=None) == _lib.ERR_NULL
    assert accept_layers(parents=None) == _lib.ERR_NULL


def append(prefix=100, prefix_lens=None, parents=A, q=9, kv=B, w=C, eps=1e-6, cos=D, sin=E, rope_rows=4096,
           status=None, cache=True, rows=300, s=2):
    c = _lib.KVCache(G, G + 0x10000000, rows, s)
    return _lib.LIB.ddtree_append_tree_kv(ctypes.byref(c) if cache else None, prefix, prefix_lens, parents, q, kv, w,
                                          eps, cos, sin, rope_rows, status, None)


def test_append_argument_errors():
    assert append(cache=False) == _lib.ERR_NULL
    for field in ("parents", "kv", "w", "cos", "sin"):
        assert append(**{field: None}) == _lib.ERR_NULL
    for kw in (dict(q=0), dict(q=65), dict(s=0), dict(rope_rows=0), dict(eps=-1.0), dict(eps=float("inf")),
               dict(eps=float("nan")), dict(prefix=292), dict(prefix=-1), dict(rows=8, prefix_lens=F)):
        assert append(**kw) == _lib.ERR_SHAPE, kw
    assert append(kv=B + 4) == _lib.ERR_ALIGN
    assert append(w=C + 8) == _lib.ERR_ALIGN
    assert append(cos=D + 2) == _lib.ERR_ALIGN
    assert append(prefix_lens=F + 2) == _lib.ERR_ALIGN
    assert append(kv=G + 0x10000000 + 64) == _lib.ERR_ALIAS   # kv inside the rotary cache
    assert append(cos=G + 1024) == _lib.ERR_ALIAS              # table inside the latent cache
    assert append(status=B + 16) == _lib.ERR_ALIAS             # status word inside kv


def test_automatic_split_plan_on_the_five_workloads():
    """The plan the library picks for each seeded workload on a 256-CU part (the count it assumes
    when no device answers).  These are the plans measured best, or within 2% of the best, in a
    sweep of forced split counts on the GPU; the reported count is the larger group's."""
    assert _lib.num_splits(256, 9, 1, 0) == 5        # one stream, 9 tiles: 5 splits of 2, one merge
    assert _lib.num_splits(1024, 33, 8, 0) == 1      # 136 workgroups fit at once: no split
    assert _lib.num_splits(1024, 9, 64, 0) == 3      # the odd node split 3 ways (11 tiles each), pairs whole
    assert _lib.num_splits(4096, 33, 1, 0) == 10     # one long stream: 10 splits of 13 tiles
    assert _lib.num_splits(4096, 33, 64, 0) == 4     # 1024 pair workgroups = 4 rounds; odd node x4
    assert _lib.workspace_size(1024, 33, 8, 0) == 0  # unsplit: no workspace

    def ws(rows0, splits0, rows1, splits1):  # partial out + lse per split group, 256-B aligned
        al = lambda x: (x + 255) // 256 * 256
        return (al(splits0 * rows0 * 2048) + al(splits1 * rows1 * 2048) + al(splits0 * rows0 * 4)
                + al(splits1 * rows1 * 4))
    # the long stream's 16 node pairs (2048 query-head rows) and its odd node, 10 splits each
    assert _lib.workspace_size(4096, 33, 1, 0) == ws(2048, 10, 64, 10)
    assert _lib.workspace_size(256, 9, 1, 0) == ws(512, 5, 64, 5)
    assert _lib.workspace_size(4096, 33, 64, 0) == ws(0, 1, 64 * 64, 4)
    assert _lib.workspace_size(1024, 9, 64, 0) == ws(0, 1, 64 * 64, 3)


def noalloc(q_lat=A, q_pe=B, ckv=C, kpe=D, prefix=100, parents=E, q=9, s=2, out=F, lse=G, splits=0, status=None):
    return _lib.LIB.ddtree_verify_attn_noalloc(q_lat, q_pe, ckv, kpe, prefix, parents, q, s, out, lse, prefix + q,
                                               0.0, splits, status, None)


def test_noalloc_validation_before_any_launch():
    m = re.search(r"#define DDTREE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES
    assert noalloc(q_lat=None) == _lib.ERR_NULL
    assert noalloc(q=65) == _lib.ERR_SHAPE
    assert noalloc(ckv=C + 2) == _lib.ERR_ALIGN
    assert noalloc(out=A) == _lib.ERR_ALIAS
    # a forced split count whose partials exceed the scratch is refused on the host
    assert _lib.workspace_size(4096, 33, 64, 64) > _lib.NOALLOC_SCRATCH_BYTES
    assert noalloc(prefix=4096, q=33, s=64, splits=64) == _lib.ERR_WORKSPACE
