"""Host-only checks of the C ABI (no GPU needed): the library loads, exports every
function include/dfkv.h declares, and refuses bad arguments with the documented
status before any launch.  Every call here fails validation, so nothing reaches
the GPU; the fake device addresses are never dereferenced."""
import ctypes as C
import os
import re

import pytest

from store_dfkv_project_amd import dfkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dfkv.h")

A = 0x7F0000000000          # fake, 256-byte aligned device addresses, far apart
MB = 1 << 20


def addr(i: int) -> int:
    return A + i * 64 * 1024 * MB


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dfkv_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 11, names
    lib = C.CDLL(dfkv.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"
    assert set(names) == set(dfkv.EXPORTED), "binding and header disagree"


def test_status_strings_and_version():
    for s in range(-6, 1):
        assert dfkv.dfkv_status_string(s).startswith("DFKV_")
    assert "gfx950" in dfkv.dfkv_version()


def geom(**over):
    base = dict(kind=0, n_tgt=3, tgt_hidden=4096, hidden=4096, n_layers=5, n_kv_heads=8, head_dim=128, latent_dim=0,
                rope_dim=128, eps=1e-6, page_size=64, width=4, block_size=16)
    base.update(over)
    return dfkv.make_geom(**base)


def mla_geom(**over):
    base = dict(kind=1, n_tgt=3, tgt_hidden=7168, hidden=7168, n_layers=3, n_kv_heads=1, head_dim=0, latent_dim=512,
                rope_dim=64, eps=1e-6, page_size=64, width=4, block_size=7)
    base.update(over)
    return dfkv.make_geom(**base)


def status_of(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except dfkv.DfkvError as e:
        return e.status
    return dfkv.DFKV_OK


@pytest.mark.parametrize("over,want", [
    (dict(kind=2), dfkv.DFKV_ERR_SHAPE),
    (dict(head_dim=96, rope_dim=96), dfkv.DFKV_ERR_SHAPE),
    (dict(rope_dim=64), dfkv.DFKV_ERR_SHAPE),
    (dict(n_layers=33), dfkv.DFKV_ERR_SHAPE),
    (dict(n_layers=0), dfkv.DFKV_ERR_SHAPE),
    (dict(hidden=4000), dfkv.DFKV_ERR_SHAPE),
    (dict(tgt_hidden=100), dfkv.DFKV_ERR_SHAPE),
    (dict(width=0), dfkv.DFKV_ERR_SHAPE),
    (dict(page_size=0), dfkv.DFKV_ERR_SHAPE),
    (dict(eps=-1.0), dfkv.DFKV_ERR_SHAPE),
])
def test_workspace_size_rejects_bad_geometry(over, want):
    assert status_of(dfkv.dfkv_workspace_size, geom(**over), 1) == want


def test_workspace_size_mla_and_null():
    assert dfkv.dfkv_workspace_size(mla_geom(), 1) > 0
    assert status_of(dfkv.dfkv_workspace_size, mla_geom(latent_dim=500), 1) == dfkv.DFKV_ERR_SHAPE
    assert status_of(dfkv.dfkv_workspace_size, mla_geom(n_kv_heads=2), 1) == dfkv.DFKV_ERR_SHAPE
    out = C.c_size_t(0)
    assert dfkv.lib().dfkv_workspace_size(None, 1, C.byref(out)) == dfkv.DFKV_ERR_NULL
    assert dfkv.lib().dfkv_workspace_size(C.byref(geom()), 1, None) == dfkv.DFKV_ERR_NULL
    assert status_of(dfkv.dfkv_workspace_size, geom(), -1) == dfkv.DFKV_ERR_SHAPE
    # the small-batch plan is smaller than the large-batch one
    assert dfkv.dfkv_workspace_size(geom(), 1) < dfkv.dfkv_workspace_size(geom(), 64)


def project_args(**over):
    g = over.pop("g", geom())
    ws = dfkv.dfkv_workspace_size(g, 1)
    a = dict(geom=g, weights=dfkv.make_weights(addr(1), addr(2), addr(3), addr(4)), hidden=addr(5),
             hidden_row_stride=12288, n_reqs=1, ctx_len_in=addr(6), cos_sin=addr(7), cache_len=4096,
             kv_out=addr(8), flags=dfkv.DFKV_FUSE_NORM_ROPE, ws=addr(9), ws_bytes=ws - 1, stream=0)
    a.update(over)
    return a


@pytest.mark.parametrize("over,want", [
    (dict(hidden=None), dfkv.DFKV_ERR_NULL),
    (dict(kv_out=None), dfkv.DFKV_ERR_NULL),
    (dict(ws=None), dfkv.DFKV_ERR_NULL),
    (dict(weights=dfkv.make_weights(addr(1), None, addr(3), addr(4))), dfkv.DFKV_ERR_NULL),
    (dict(cos_sin=None), dfkv.DFKV_ERR_NULL),
    (dict(hidden=addr(5) + 8), dfkv.DFKV_ERR_LAYOUT),
    (dict(hidden_row_stride=12280), dfkv.DFKV_ERR_LAYOUT),
    (dict(hidden_row_stride=12289), dfkv.DFKV_ERR_LAYOUT),
    (dict(kv_out=addr(8) + 2), dfkv.DFKV_ERR_LAYOUT),
    (dict(flags=2), dfkv.DFKV_ERR_SHAPE),
    (dict(cache_len=0), dfkv.DFKV_ERR_SHAPE),
    (dict(), dfkv.DFKV_ERR_WORKSPACE),
    (dict(n_reqs=-1), dfkv.DFKV_ERR_SHAPE),
])
def test_project_validation(over, want):
    assert status_of(dfkv.dfkv_project, **project_args(**over)) == want


def test_pack_fc_weight_validation():
    f = dfkv.dfkv_pack_fc_weight
    assert status_of(f, geom(), None, addr(2)) == dfkv.DFKV_ERR_NULL
    assert status_of(f, geom(), addr(1), None) == dfkv.DFKV_ERR_NULL
    assert dfkv.lib().dfkv_pack_fc_weight(None, addr(1), addr(2), None) == dfkv.DFKV_ERR_NULL
    assert status_of(f, geom(hidden=4000), addr(1), addr(2)) == dfkv.DFKV_ERR_SHAPE
    assert status_of(f, geom(), addr(1) + 8, addr(2)) == dfkv.DFKV_ERR_LAYOUT
    assert status_of(f, geom(), addr(1), addr(2) + 2) == dfkv.DFKV_ERR_LAYOUT
    # the packed copy over the row-major one
    assert status_of(f, geom(), addr(1), addr(1) + 1024) == dfkv.DFKV_ERR_ALIAS


def test_project_packed_weight_checks():
    ok_ws = dfkv.dfkv_workspace_size(geom(), 1)
    w = lambda pk: dfkv.make_weights(addr(1), addr(2), addr(3), addr(4), w_fc_packed=pk)
    assert status_of(dfkv.dfkv_project, **project_args(weights=w(addr(10) + 8), ws_bytes=ok_ws)) == dfkv.DFKV_ERR_LAYOUT
    # the packed weight over kv_out, or inside the workspace
    assert status_of(dfkv.dfkv_project, **project_args(weights=w(addr(8)), ws_bytes=ok_ws)) == dfkv.DFKV_ERR_ALIAS
    assert status_of(dfkv.dfkv_project, **project_args(weights=w(addr(9) + 256), ws_bytes=ok_ws)) == \
        dfkv.DFKV_ERR_ALIAS
    # the fc stage alone takes the same weights struct
    fc = dict(geom=geom(), weights=w(addr(10)), hidden=addr(5), hidden_row_stride=12288, n_reqs=1, ws=addr(9),
              ws_bytes=ok_ws, stream=0)
    assert status_of(dfkv.dfkv_project_fc, **dict(fc, weights=None)) == dfkv.DFKV_ERR_NULL
    assert status_of(dfkv.dfkv_project_fc, **dict(fc, weights=w(addr(10) + 2))) == dfkv.DFKV_ERR_LAYOUT
    assert status_of(dfkv.dfkv_project_fc, **dict(fc, weights=w(addr(9)))) == dfkv.DFKV_ERR_ALIAS
    assert status_of(dfkv.dfkv_project_fc, **dict(fc, ws_bytes=ok_ws - 256)) == dfkv.DFKV_ERR_WORKSPACE


def test_pack_stream_weight_validation():
    f = dfkv.dfkv_pack_stream_weight
    assert status_of(f, 4096, 12288, None, addr(2)) == dfkv.DFKV_ERR_NULL
    assert status_of(f, 4096, 12288, addr(1), None) == dfkv.DFKV_ERR_NULL
    for rows, cols in ((4088, 12288), (4096, 12224), (0, 128), (16, 0), (-16, 128)):
        assert status_of(f, rows, cols, addr(1), addr(2)) == dfkv.DFKV_ERR_SHAPE, (rows, cols)
    assert status_of(f, 4096, 12288, addr(1) + 8, addr(2)) == dfkv.DFKV_ERR_LAYOUT
    assert status_of(f, 4096, 12288, addr(1), addr(2) + 2) == dfkv.DFKV_ERR_LAYOUT
    # the tiled copy over the row-major one (either way round)
    assert status_of(f, 4096, 12288, addr(1), addr(1) + 4096) == dfkv.DFKV_ERR_ALIAS
    assert status_of(f, 4096, 12288, addr(1) + 4096, addr(1)) == dfkv.DFKV_ERR_ALIAS


def test_project_stream_weight_checks():
    ok_ws = dfkv.dfkv_workspace_size(geom(), 1)
    w = lambda fs=None, ks=None: dfkv.make_weights(addr(1), addr(2), addr(3), addr(4), w_fc_stream=fs, w_kv_stream=ks)
    P = dfkv.dfkv_project
    assert status_of(P, **project_args(weights=w(fs=addr(10) + 8), ws_bytes=ok_ws)) == dfkv.DFKV_ERR_LAYOUT
    assert status_of(P, **project_args(weights=w(ks=addr(11) + 4), ws_bytes=ok_ws)) == dfkv.DFKV_ERR_LAYOUT
    # a tiled weight over kv_out, or inside the workspace
    assert status_of(P, **project_args(weights=w(fs=addr(8)), ws_bytes=ok_ws)) == dfkv.DFKV_ERR_ALIAS
    assert status_of(P, **project_args(weights=w(ks=addr(9) + 256), ws_bytes=ok_ws)) == dfkv.DFKV_ERR_ALIAS
    assert status_of(P, **project_args(weights=w(ks=addr(8) - 1024), ws_bytes=ok_ws)) == dfkv.DFKV_ERR_ALIAS
    # the fc stage checks the tiled fc weight only, the K/V stage the tiled K/V weight only
    fc = dict(geom=geom(), hidden=addr(5), hidden_row_stride=12288, n_reqs=1, ws=addr(9), ws_bytes=ok_ws, stream=0)
    assert status_of(dfkv.dfkv_project_fc, **dict(fc, weights=w(fs=addr(10) + 2))) == dfkv.DFKV_ERR_LAYOUT
    assert status_of(dfkv.dfkv_project_fc, **dict(fc, weights=w(fs=addr(9)))) == dfkv.DFKV_ERR_ALIAS
    kv = dict(geom=geom(), n_reqs=1, ctx_len_in=addr(6), cos_sin=addr(7), cache_len=4096, kv_out=addr(8),
              flags=dfkv.DFKV_FUSE_NORM_ROPE, ws=addr(9), ws_bytes=ok_ws, stream=0)
    assert status_of(dfkv.dfkv_project_kv, **dict(kv, weights=w(ks=addr(11) + 2))) == dfkv.DFKV_ERR_LAYOUT
    assert status_of(dfkv.dfkv_project_kv, **dict(kv, weights=w(ks=addr(8)))) == dfkv.DFKV_ERR_ALIAS


def test_project_alias_checks():
    ok_ws = dfkv.dfkv_workspace_size(geom(), 1)
    # kv_out inside the hidden rows
    assert status_of(dfkv.dfkv_project, **project_args(kv_out=addr(5) + 4096, ws_bytes=ok_ws)) == dfkv.DFKV_ERR_ALIAS
    # kv_out inside the workspace
    assert status_of(dfkv.dfkv_project, **project_args(kv_out=addr(9) + 256, ws_bytes=ok_ws)) == dfkv.DFKV_ERR_ALIAS
    # kv_out over a weight
    assert status_of(dfkv.dfkv_project, **project_args(kv_out=addr(3), ws_bytes=ok_ws)) == dfkv.DFKV_ERR_ALIAS
    # the workspace over the hidden rows
    assert status_of(dfkv.dfkv_project, **project_args(ws=addr(5), ws_bytes=ok_ws)) == dfkv.DFKV_ERR_ALIAS


def test_project_zero_requests_is_a_no_op():
    assert status_of(dfkv.dfkv_project, **project_args(n_reqs=0)) == dfkv.DFKV_OK


def requests(**over):
    a = dict(n_reqs=2, ctx_len_in=addr(20), n_acc=addr(21), alloc_limit=addr(22), is_dummy=addr(23), row_valid=None,
             block_table=addr(24), bt_row_stride=8, bt_cols=8, accepted_tokens=addr(25), acc_stride_req=4,
             acc_stride_tok=1, mask_token_id=7)
    a.update(over)
    return dfkv.make_requests(**a)


def pool(g=None, **over):
    g = g or geom()
    L = g.n_layers
    a = dict(k=[addr(30 + l) for l in range(L)], v=[addr(40 + l) for l in range(L)], stride_page=64 * 8 * 128,
             stride_slot=8 * 128, stride_head=128, num_pages=100)
    a.update(over)
    return dfkv.make_pool(**a)


def outputs(**over):
    a = dict(slot=addr(50), write_mask=addr(51), c_pos=addr(52), bonus=addr(53), emb_ids=addr(54), q_pos=addr(55),
             ctx_len_out=addr(56), seq_len=addr(57))
    a.update(over)
    return dfkv.make_outputs(**a)


@pytest.mark.parametrize("pool_over,want", [
    (dict(stride_page=100), dfkv.DFKV_ERR_LAYOUT),
    (dict(stride_slot=0), dfkv.DFKV_ERR_LAYOUT),
    (dict(stride_head=64), dfkv.DFKV_ERR_LAYOUT),
    (dict(stride_slot=8 * 128 + 4), dfkv.DFKV_ERR_LAYOUT),
    (dict(stride_page=10 * 128), dfkv.DFKV_ERR_LAYOUT),
    (dict(k=[addr(30) + 8] + [addr(31 + l) for l in range(4)]), dfkv.DFKV_ERR_LAYOUT),
    (dict(v=[addr(40 + l) for l in range(4)]), dfkv.DFKV_ERR_NULL),
])
def test_paged_store_pool_validation(pool_over, want):
    st = status_of(dfkv.dfkv_paged_store, geom(), addr(60), requests(), pool(**pool_over), addr(50), addr(51),
                   stream=0)
    assert st == want


def test_paged_store_other_validation():
    # NULL slot output, table stride shorter than its columns, slot over a pool, kv over a pool
    assert status_of(dfkv.dfkv_paged_store, geom(), addr(60), requests(), pool(), None, addr(51), stream=0) == \
        dfkv.DFKV_ERR_NULL
    assert status_of(dfkv.dfkv_paged_store, geom(), addr(60), requests(bt_row_stride=4), pool(), addr(50), addr(51),
                     stream=0) == dfkv.DFKV_ERR_LAYOUT
    assert status_of(dfkv.dfkv_paged_store, geom(), addr(60), requests(), pool(), addr(31) + 64, addr(51),
                     stream=0) == dfkv.DFKV_ERR_ALIAS
    assert status_of(dfkv.dfkv_paged_store, geom(), addr(40) + 128, requests(), pool(), addr(50), addr(51),
                     stream=0) == dfkv.DFKV_ERR_ALIAS
    # the HND layout ([page][head][slot][dim]) is accepted by validation up to the launch; MLA pool
    g = mla_geom()
    p = dfkv.make_pool([addr(30 + l) for l in range(3)], None, 64 * 576, 570, 0, 10)
    assert status_of(dfkv.dfkv_paged_store, g, addr(60), requests(), p, addr(50), addr(51), stream=0) == \
        dfkv.DFKV_ERR_LAYOUT
    # zero requests: nothing to do
    assert status_of(dfkv.dfkv_paged_store, geom(), None, requests(n_reqs=0), None, None, None, stream=0) == \
        dfkv.DFKV_OK


def test_advance_validation():
    assert status_of(dfkv.dfkv_advance, geom(), requests(), outputs(ctx_len_out=addr(20)), stream=0) == \
        dfkv.DFKV_ERR_ALIAS                     # in-place ctx_len advance is refused
    assert status_of(dfkv.dfkv_advance, geom(), requests(), outputs(q_pos=addr(52) + 4), stream=0) == \
        dfkv.DFKV_ERR_ALIAS                     # two outputs overlap
    assert status_of(dfkv.dfkv_advance, geom(), requests(accepted_tokens=None), outputs(), stream=0) == \
        dfkv.DFKV_ERR_NULL
    assert status_of(dfkv.dfkv_advance, geom(), requests(acc_stride_tok=-1), outputs(), stream=0) == \
        dfkv.DFKV_ERR_LAYOUT
    assert status_of(dfkv.dfkv_advance, geom(), requests(n_acc=None), outputs(), stream=0) == dfkv.DFKV_ERR_NULL
    assert status_of(dfkv.dfkv_advance, geom(), requests(n_reqs=-3), outputs(), stream=0) == dfkv.DFKV_ERR_SHAPE
    # the block placement needs the pool's page count: dfkv_advance refuses to place a block
    assert status_of(dfkv.dfkv_advance, geom(), requests(), outputs(block_slot=addr(58)), stream=0) == \
        dfkv.DFKV_ERR_SHAPE


def test_block_placement_validation():
    g = geom()
    # block_slot over q_pos, over the block table, misaligned; no block table to place from
    assert status_of(dfkv.dfkv_store_advance, g, addr(60), requests(), pool(), outputs(block_slot=addr(55) + 8),
                     stream=0) == dfkv.DFKV_ERR_ALIAS
    assert status_of(dfkv.dfkv_store_advance, g, addr(60), requests(), pool(), outputs(block_slot=addr(24)),
                     stream=0) == dfkv.DFKV_ERR_ALIAS
    assert status_of(dfkv.dfkv_store_advance, g, addr(60), requests(), pool(), outputs(block_slot=addr(58) + 4),
                     stream=0) == dfkv.DFKV_ERR_LAYOUT


def test_step_validation():
    g = geom()
    ws = dfkv.dfkv_workspace_size(g, 2)
    w = dfkv.make_weights(addr(1), addr(2), addr(3), addr(4))
    base = dict(geom=g, weights=w, hidden=addr(5), hidden_row_stride=12288, requests=requests(), cos_sin=addr(7),
                cache_len=4096, kv_out=addr(8), pool=pool(), outputs=outputs(), ws=addr(9), ws_bytes=ws, stream=0)
    # a bookkeeping output inside the workspace
    a = dict(base, outputs=outputs(seq_len=addr(9) + 512))
    assert status_of(dfkv.dfkv_step, **a) == dfkv.DFKV_ERR_ALIAS
    # kv_out over a pool
    a = dict(base, kv_out=addr(30))
    assert status_of(dfkv.dfkv_step, **a) == dfkv.DFKV_ERR_ALIAS
    a = dict(base, ws_bytes=ws - 256)
    assert status_of(dfkv.dfkv_step, **a) == dfkv.DFKV_ERR_WORKSPACE
    a = dict(base, pool=pool(stride_slot=3))
    assert status_of(dfkv.dfkv_step, **a) == dfkv.DFKV_ERR_LAYOUT


def test_fork_join_validation():
    """The overlapped projection validates as dfkv_project before touching any stream or event."""
    g = geom()
    ws = dfkv.dfkv_workspace_size(g, 2)
    w = dfkv.make_weights(addr(1), addr(2), addr(3), addr(4))
    base = dict(geom=g, weights=w, hidden=addr(5), hidden_row_stride=12288, n_reqs=2, ctx_len_in=addr(6),
                cos_sin=addr(7), cache_len=4096, kv_out=addr(8), flags=1, ws=addr(9), ws_bytes=ws, main=0, aux=0,
                fork=addr(11), join=addr(12))
    assert status_of(dfkv.dfkv_project_fork, **dict(base, fork=0)) == dfkv.DFKV_ERR_NULL
    assert status_of(dfkv.dfkv_project_fork, **dict(base, join=0)) == dfkv.DFKV_ERR_NULL
    assert status_of(dfkv.dfkv_project_fork, **dict(base, ws_bytes=ws - 256)) == dfkv.DFKV_ERR_WORKSPACE
    assert status_of(dfkv.dfkv_project_fork, **dict(base, kv_out=addr(5))) == dfkv.DFKV_ERR_ALIAS
    # DFKV_FORK_RECORDED is dfkv_project_fork's alone; other bits stay rejected
    recorded = dfkv.DFKV_FUSE_NORM_ROPE | dfkv.DFKV_FORK_RECORDED
    assert status_of(dfkv.dfkv_project_fork, **dict(base, flags=recorded, fork=0)) == dfkv.DFKV_ERR_NULL
    assert status_of(dfkv.dfkv_project_fork, **dict(base, flags=recorded, ws_bytes=ws - 256)) == \
        dfkv.DFKV_ERR_WORKSPACE
    assert status_of(dfkv.dfkv_project_fork, **dict(base, flags=4)) == dfkv.DFKV_ERR_SHAPE
    assert status_of(dfkv.dfkv_join, 0, 0) == dfkv.DFKV_ERR_NULL


def test_block_table_decode_validation():
    f = dfkv.dfkv_block_table_decode
    base = dict(offsets=addr(1), off_stride_req=8, off_stride_blk=1, n_reqs=4, max_blocks=8, n_tokens=addr(2),
                page_size=64, divisor=2, page_count_out=addr(3), table_out=addr(4), table_row_stride=8, stream=0)
    assert status_of(f, **dict(base, divisor=0)) == dfkv.DFKV_ERR_SHAPE
    assert status_of(f, **dict(base, page_size=0)) == dfkv.DFKV_ERR_SHAPE
    assert status_of(f, **dict(base, max_blocks=-1)) == dfkv.DFKV_ERR_SHAPE
    assert status_of(f, **dict(base, n_tokens=None)) == dfkv.DFKV_ERR_NULL
    assert status_of(f, **dict(base, table_row_stride=7)) == dfkv.DFKV_ERR_LAYOUT
    assert status_of(f, **dict(base, off_stride_blk=-1)) == dfkv.DFKV_ERR_LAYOUT
    assert status_of(f, **dict(base, table_out=addr(1) + 64)) == dfkv.DFKV_ERR_ALIAS   # table over the offsets
    assert status_of(f, **dict(base, page_count_out=addr(4) + 16)) == dfkv.DFKV_ERR_ALIAS
    assert status_of(f, **dict(base, n_reqs=0, offsets=None, n_tokens=None)) == dfkv.DFKV_OK


def test_strict_accept_validation():
    f = dfkv.dfkv_strict_accept
    base = dict(target=addr(1), t_stride_req=4, t_stride_tok=1, draft=addr(2), d_stride_req=3, d_stride_tok=1,
                n_reqs=8, width=4, n_acc_out=addr(3), accepted_out=addr(4), stream=0)
    assert status_of(f, **dict(base, width=0)) == dfkv.DFKV_ERR_SHAPE
    assert status_of(f, **dict(base, n_reqs=-1)) == dfkv.DFKV_ERR_SHAPE
    assert status_of(f, **dict(base, draft=None)) == dfkv.DFKV_ERR_NULL
    assert status_of(f, **dict(base, t_stride_tok=-1)) == dfkv.DFKV_ERR_LAYOUT
    assert status_of(f, **dict(base, accepted_out=addr(1) + 32)) == dfkv.DFKV_ERR_ALIAS
    assert status_of(f, **dict(base, n_acc_out=addr(2) + 8)) == dfkv.DFKV_ERR_ALIAS
    assert status_of(f, **dict(base, n_reqs=0, target=None)) == dfkv.DFKV_OK


def test_paged_store_rows_validation():
    f = dfkv.dfkv_paged_store_rows
    base = dict(geom=geom(), kv=addr(60), n_rows=10, row_req=addr(61), row_pos=addr(62), n_reqs=2,
                alloc_limit=addr(63), block_table=addr(64), bt_row_stride=8, bt_cols=8, pool=pool(),
                slot_out=addr(50), write_mask_out=addr(51), stream=0)
    assert status_of(f, **dict(base, n_rows=-1)) == dfkv.DFKV_ERR_SHAPE
    assert status_of(f, **dict(base, row_pos=None)) == dfkv.DFKV_ERR_NULL
    assert status_of(f, **dict(base, bt_row_stride=4)) == dfkv.DFKV_ERR_LAYOUT
    assert status_of(f, **dict(base, slot_out=addr(61) + 8)) == dfkv.DFKV_ERR_ALIAS     # over row_req
    assert status_of(f, **dict(base, kv=addr(30))) == dfkv.DFKV_ERR_ALIAS               # kv over a pool
    assert status_of(f, **dict(base, pool=pool(stride_slot=3))) == dfkv.DFKV_ERR_LAYOUT
    assert status_of(f, **dict(base, n_rows=0, kv=None)) == dfkv.DFKV_OK


def test_rope_cache_validation():
    r = dfkv.make_rope(1e6, 64)
    assert status_of(dfkv.dfkv_rope_cache_build, dfkv.make_rope(1e6, 63), addr(7), 10, stream=0) == \
        dfkv.DFKV_ERR_SHAPE
    assert status_of(dfkv.dfkv_rope_cache_build, r, addr(7), 0, stream=0) == dfkv.DFKV_ERR_SHAPE
    assert status_of(dfkv.dfkv_rope_cache_build, r, None, 10, stream=0) == dfkv.DFKV_ERR_NULL
    assert status_of(dfkv.dfkv_rope_cache_build, r, addr(7) + 2, 10, stream=0) == dfkv.DFKV_ERR_LAYOUT
    assert status_of(dfkv.dfkv_rope_cache_build, dfkv.make_rope(1e6, 64, yarn=True, factor=0.0, orig_ctx=4096),
                     addr(7), 10, stream=0) == dfkv.DFKV_ERR_SHAPE
    assert status_of(dfkv.dfkv_rope_cache_build, dfkv.make_rope(1.0, 64), addr(7), 10, stream=0) == \
        dfkv.DFKV_ERR_SHAPE


def test_norm_rope_validation():
    g = geom()
    assert status_of(dfkv.dfkv_norm_rope, g, addr(4), 1, addr(6), addr(7), 4096, None, stream=0) == dfkv.DFKV_ERR_NULL
    assert status_of(dfkv.dfkv_norm_rope, g, addr(4), 1, addr(6), addr(7), 4096, addr(8) + 2, stream=0) == \
        dfkv.DFKV_ERR_LAYOUT
    assert status_of(dfkv.dfkv_norm_rope, g, addr(4), 1, addr(6), addr(7), 4096, addr(7) + 1024, stream=0) == \
        dfkv.DFKV_ERR_ALIAS
    assert status_of(dfkv.dfkv_norm_rope, g, addr(4), 1, addr(6), addr(7), 0, addr(8), stream=0) == \
        dfkv.DFKV_ERR_SHAPE


def test_step_noalloc_validation():
    """The static-scratch step refuses, before touching a GPU, a plan larger than its scratch (the dense
    drafter at 64 requests of 16 rows needs about 84 MB) and NULL geometry or requests."""
    g = geom(width=16)
    assert dfkv.dfkv_workspace_size(g, 64) > dfkv.DFKV_NOALLOC_SCRATCH_BYTES
    assert dfkv.dfkv_workspace_size(geom(), 16) <= dfkv.DFKV_NOALLOC_SCRATCH_BYTES
    assert dfkv.dfkv_workspace_size(mla_geom(), 16) <= dfkv.DFKV_NOALLOC_SCRATCH_BYTES
    w = dfkv.make_weights(addr(1), addr(2), addr(3), addr(4))
    base = dict(geom=g, weights=w, hidden=addr(5), hidden_row_stride=12288, requests=requests(n_reqs=64),
                cos_sin=addr(7), cache_len=4096, kv_out=addr(8), pool=pool(), outputs=outputs(), stream=0)
    assert status_of(dfkv.dfkv_step_noalloc, **base) == dfkv.DFKV_ERR_WORKSPACE
    assert status_of(dfkv.dfkv_step_noalloc, **dict(base, geom=None)) == dfkv.DFKV_ERR_NULL
    assert status_of(dfkv.dfkv_step_noalloc, **dict(base, requests=None)) == dfkv.DFKV_ERR_NULL
    assert status_of(dfkv.dfkv_step_noalloc, **dict(base, geom=geom(kind=2))) == dfkv.DFKV_ERR_SHAPE
