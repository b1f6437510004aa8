"""Projection kernels on the GPU against the oracle: cos/sin cache, k_norm/RoPE,
and the fc -> hidden_norm -> stacked GEMM -> k_norm/RoPE projection on both the
small-batch (split-K weight streaming) and the large-batch (tiled) paths, with
ragged row counts.  K/V within |d| <= 2e-2 + 1e-2*|ref|."""
import numpy as np
import pytest

from dfkv_workloads import GQA, MLA, Geometry, RopeSpec, Workload, bf16_bits, make_weights, MASK_TOKEN_ID
from gpu_helpers import assert_close_bf16, small_geom

pytestmark = pytest.mark.gpu

ROPES = [
    ("plain-64", RopeSpec(theta=1e6, rot=64), 200),
    ("plain-128", RopeSpec(theta=1e6, rot=128), 40000),
    ("yarn40-64", RopeSpec(theta=1e6, rot=64, yarn=True, factor=40.0, orig_ctx=4096.0), 393216 + 32),
    ("yarn4-128", RopeSpec(theta=1e6, rot=128, yarn=True, factor=4.0, orig_ctx=32768.0), 65536 + 40),
    ("yarn40-64-trunc", RopeSpec(theta=1e6, rot=64, yarn=True, factor=40.0, orig_ctx=4096.0, truncate=True), 5000),
    ("plain-16-1e4", RopeSpec(theta=1e4, rot=16), 3000),
]


@pytest.mark.parametrize("name,rope,cache_len", ROPES, ids=[r[0] for r in ROPES])
def test_rope_cache_matches_oracle(orc, name, rope, cache_len):
    """Both caches take fp64 angles; they may differ only by fp32 rounding of nearly equal doubles."""
    import torch
    from store_dfkv_project_amd import dfkv
    from store_dfkv_project_amd.step import rope_struct
    cs = torch.empty((cache_len, rope.rot), dtype=torch.float32, device="cuda")
    dfkv.dfkv_rope_cache_build(rope_struct(rope), cs)
    got = cs.cpu().numpy()
    want = orc.rope_cache(rope, cache_len)
    diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    bad = diff > np.maximum(ulp, 1e-9)
    assert not bad.any(), f"{int(bad.sum())} entries differ; max diff {diff.max()}"


def _proj_workload(geom: Geometry, B: int, seed: int, rope: RopeSpec, cache_len: int, ctx_hi: int) -> Workload:
    rng = np.random.default_rng(seed)
    W = geom.width
    N = B * W
    hidden = np.full((N, geom.k_in + 8), 0x7FC0, np.uint16)      # NaN padding past k_in: never read
    hidden[:, :geom.k_in] = bf16_bits(rng.standard_normal((N, geom.k_in)).astype(np.float32))
    w = make_weights(geom, rng)
    ctx = rng.integers(0, ctx_hi, size=B).astype(np.int32)
    ctx[0] = 0                                                   # position 0: rotation is the identity
    if B > 2:
        ctx[1] = cache_len + 5                                   # past the cache: clamped to its last row
    return Workload(config_id=-1, name="proj", geom=geom, rope=rope, n_reqs=B, hidden=hidden,
                    hidden_row_stride=geom.k_in + 8, w_fc=w["w_fc"], w_hnorm=w["w_hnorm"], w_kv=w["w_kv"],
                    w_knorm=w["w_knorm"], ctx_len=ctx, n_acc=np.full(B, W, np.int32),
                    alloc_limit=np.full(B, 1 << 30, np.int32), is_dummy=np.zeros(B, np.uint8), row_valid=None,
                    block_table=np.zeros((B, 1), np.int32), accepted_tokens=np.zeros((B, W), np.int32),
                    acc_stride_req=W, acc_stride_tok=1, mask_token_id=MASK_TOKEN_ID, num_pages=1,
                    cache_len=cache_len)


GQA_G = Geometry(kind=GQA, n_tgt=2, tgt_hidden=256, hidden=384, n_layers=2, n_kv_heads=2, head_dim=128, latent_dim=0,
                 rope_dim=128, eps=1e-6, page_size=16, width=4, block_size=4)
GQA_G64 = Geometry(kind=GQA, n_tgt=3, tgt_hidden=256, hidden=256, n_layers=2, n_kv_heads=2, head_dim=64, latent_dim=0,
                   rope_dim=64, eps=1e-6, page_size=16, width=4, block_size=4)
GQA_G256 = Geometry(kind=GQA, n_tgt=1, tgt_hidden=640, hidden=512, n_layers=1, n_kv_heads=3, head_dim=256,
                    latent_dim=0, rope_dim=256, eps=1e-6, page_size=16, width=3, block_size=4)
# stacked K/V widths divisible by 160 (5 layers x 2 x nkv x 64): the large-batch K/V GEMM with
# 160-feature tiles and the packed normalised hidden state
GQA_W1 = Geometry(kind=GQA, n_tgt=2, tgt_hidden=256, hidden=256, n_layers=5, n_kv_heads=1, head_dim=64, latent_dim=0,
                  rope_dim=64, eps=1e-6, page_size=16, width=4, block_size=4)
GQA_W2 = Geometry(kind=GQA, n_tgt=1, tgt_hidden=384, hidden=384, n_layers=5, n_kv_heads=2, head_dim=64, latent_dim=0,
                  rope_dim=64, eps=1e-6, page_size=16, width=4, block_size=4)
# k_in = 2048: the large-batch fc GEMM splits over k (2 splits) ahead of the packed hidden_norm
GQA_W3 = Geometry(kind=GQA, n_tgt=2, tgt_hidden=1024, hidden=256, n_layers=5, n_kv_heads=1, head_dim=64, latent_dim=0,
                  rope_dim=64, eps=1e-6, page_size=16, width=4, block_size=4)
MLA_G = Geometry(kind=MLA, n_tgt=2, tgt_hidden=256, hidden=512, n_layers=2, n_kv_heads=1, head_dim=0, latent_dim=512,
                 rope_dim=64, eps=1e-6, page_size=16, width=4, block_size=7)

PROJ_CASES = [
    # name, geom, B, rope
    ("gqa128-B1", GQA_G, 1, RopeSpec(theta=1e6, rot=128)),
    ("gqa128-B5", GQA_G, 5, RopeSpec(theta=1e6, rot=128, yarn=True, factor=4.0, orig_ctx=1024.0)),
    ("gqa128-B9-ng3", GQA_G, 9, RopeSpec(theta=1e6, rot=128)),
    ("gqa128-B16-ng4", GQA_G, 16, RopeSpec(theta=1e6, rot=128)),
    ("gqa128-B17-tiled", GQA_G, 17, RopeSpec(theta=1e6, rot=128)),
    ("gqa128-B40-tiled", GQA_G, 40, RopeSpec(theta=1e6, rot=128, yarn=True, factor=4.0, orig_ctx=1024.0)),
    ("gqa64-B2", GQA_G64, 2, RopeSpec(theta=1e6, rot=64)),
    ("gqa64-B37-tiled", GQA_G64, 37, RopeSpec(theta=1e6, rot=64)),
    ("gqa256-B3", GQA_G256, 3, RopeSpec(theta=1e4, rot=256)),
    ("gqa256-B30-tiled", GQA_G256, 30, RopeSpec(theta=1e4, rot=256)),
    ("gqaW640-B40", GQA_W1, 40, RopeSpec(theta=1e6, rot=64)),
    ("gqaW640-B70", GQA_W1, 70, RopeSpec(theta=1e6, rot=64)),
    ("gqaW640-B70-splitfc", GQA_W3, 70, RopeSpec(theta=1e6, rot=64)),
    ("gqaW1280-B130", GQA_W2, 130, RopeSpec(theta=1e6, rot=64, yarn=True, factor=4.0, orig_ctx=1024.0)),
    ("mla-B1", MLA_G, 1, RopeSpec(theta=1e6, rot=64, yarn=True, factor=40.0, orig_ctx=4096.0)),
    ("mla-B3", MLA_G, 3, RopeSpec(theta=1e6, rot=64, yarn=True, factor=40.0, orig_ctx=4096.0)),
    ("mla-B33-tiled", MLA_G, 33, RopeSpec(theta=1e6, rot=64, yarn=True, factor=40.0, orig_ctx=4096.0)),
]


def _run_case(orc, name, geom, B, rope, seed=7):
    import torch
    from store_dfkv_project_amd import dfkv
    from store_dfkv_project_amd.step import DeviceStep
    wl = _proj_workload(geom, B, seed, rope, cache_len=3000, ctx_hi=2900)
    ds = DeviceStep(wl)
    cs = orc.rope_cache(rope, wl.cache_len)
    ref = orc.project(geom, wl.hidden, wl.w_fc, wl.w_hnorm, wl.w_kv, wl.w_knorm, wl.ctx_len, cs)
    return wl, ds, ref


@pytest.mark.parametrize("name,geom,B,rope", PROJ_CASES, ids=[c[0] for c in PROJ_CASES])
def test_project_matches_oracle(orc, name, geom, B, rope):
    import torch
    from store_dfkv_project_amd import dfkv
    wl, ds, ref = _run_case(orc, name, geom, B, rope)
    # unfused: kv_out = y (stacked GEMM output before k_norm / RoPE)
    ds.kv_out.fill_(0x7FC0)
    ds.project(flags=0)
    torch.cuda.synchronize()
    assert_close_bf16(ds.bits(ds.kv_out), ref["y"], f"{name} y")
    # standalone k_norm + RoPE on the GPU's y
    y_gpu_in = ds.kv_out.clone()
    y_gpu = ds.kv_out.clone()
    ds.norm_rope(y_gpu)
    torch.cuda.synchronize()
    want_nr = orc.norm_rope(geom, ds.bits(ds.kv_out), wl.w_knorm, wl.ctx_len, orc.rope_cache(rope, wl.cache_len))
    assert_close_bf16(ds.bits(y_gpu), want_nr, f"{name} norm_rope")
    # fused
    ds.kv_out.fill_(0x7FC0)
    ds.project(flags=dfkv.DFKV_FUSE_NORM_ROPE)
    torch.cuda.synchronize()
    stats = assert_close_bf16(ds.bits(ds.kv_out), ref["kv"], f"{name} kv")
    if geom.kind == GQA:
        # V has no norm and no rotation: the fused V halves are the unfused projection's, bit for bit
        got, y_bits = ds.bits(ds.kv_out).reshape(ds.N, -1), ds.bits(y_gpu_in).reshape(ds.N, -1)
        kv = geom.n_kv_heads * geom.head_dim
        for l in range(geom.n_layers):
            v0 = l * geom.per_layer + kv
            assert np.array_equal(got[:, v0:v0 + kv], y_bits[:, v0:v0 + kv]), f"{name} layer {l} V"
    # deterministic: a second call gives the same bits
    first = ds.kv_out.clone()
    ds.project(flags=dfkv.DFKV_FUSE_NORM_ROPE)
    torch.cuda.synchronize()
    assert torch.equal(first, ds.kv_out), "projection is not deterministic"
    # the two stages compose to the whole projection
    ds.kv_out.fill_(0x7FC0)
    ds.project_fc()
    ds.project_kv(flags=dfkv.DFKV_FUSE_NORM_ROPE)
    torch.cuda.synchronize()
    assert torch.equal(first, ds.kv_out), "dfkv_project_fc + dfkv_project_kv differ from dfkv_project"


def test_workspace_shared_across_batch_sizes(orc):
    """One workspace (sized for the largest call) serves alternating batch sizes: tickets self-reset."""
    import torch
    from store_dfkv_project_amd import dfkv
    from store_dfkv_project_amd.step import DeviceStep, geom_struct
    rope = RopeSpec(theta=1e6, rot=128)
    cases = []
    for B in (1, 16, 3, 40, 1):
        wl = _proj_workload(GQA_G, B, 100 + B, rope, cache_len=3000, ctx_hi=2900)
        cases.append(wl)
    need = max(dfkv.dfkv_workspace_size(geom_struct(GQA_G), wl.n_reqs) for wl in cases)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    dfkv.dfkv_workspace_init(ws, need)
    cs_o = orc.rope_cache(rope, 3000)
    for wl in cases:
        ds = DeviceStep(wl)
        ds.ws, ds.ws_bytes = ws, need
        ds.project()
        torch.cuda.synchronize()
        ref = orc.project(GQA_G, wl.hidden, wl.w_fc, wl.w_hnorm, wl.w_kv, wl.w_knorm, wl.ctx_len, cs_o)
        assert_close_bf16(ds.bits(ds.kv_out), ref["kv"], f"B={wl.n_reqs}")


@pytest.mark.parametrize("kind", [GQA, MLA])
def test_norm_rope_far_positions(orc, kind):
    """k_norm + RoPE with YaRN at positions up to 393k, on random y."""
    import torch
    from store_dfkv_project_amd.step import DeviceStep
    geom = GQA_G if kind == GQA else MLA_G
    rope = (RopeSpec(theta=1e6, rot=128, yarn=True, factor=4.0, orig_ctx=32768.0) if kind == GQA else
            RopeSpec(theta=1e6, rot=64, yarn=True, factor=40.0, orig_ctx=4096.0))
    wl = _proj_workload(geom, 6, 3, rope, cache_len=393216 + 64, ctx_hi=393216)
    wl.ctx_len[:] = [0, 393216, 131072, 2048, 65530, 393216 + 63]
    ds = DeviceStep(wl)
    rng = np.random.default_rng(5)
    y = bf16_bits((rng.standard_normal((ds.N, geom.out_dim)) * 2).astype(np.float32))
    ds.kv_out.copy_(torch.from_numpy(y.view(np.int16)).cuda())
    ds.ctx_len.copy_(torch.from_numpy(wl.ctx_len).cuda())
    ds.norm_rope(ds.kv_out)
    torch.cuda.synchronize()
    want = orc.norm_rope(geom, y, wl.w_knorm, wl.ctx_len, orc.rope_cache(rope, wl.cache_len))
    got = ds.bits(ds.kv_out)
    assert_close_bf16(got, want, "norm_rope far positions")
    if kind == GQA:
        # V heads are untouched: every V element keeps its input bits
        kv = geom.n_kv_heads * geom.head_dim
        for l in range(geom.n_layers):
            v0 = l * geom.per_layer + kv
            assert np.array_equal(got.reshape(ds.N, -1)[:, v0:v0 + kv], y.reshape(ds.N, -1)[:, v0:v0 + kv]), l


@pytest.mark.parametrize("geom,B", [(GQA_W1, 40), (GQA_G, 30)], ids=["gqaW640-B40", "gqa128-B30"])
def test_finalize_unaligned_operands(orc, geom, B):
    """k_norm weights and the cos/sin cache only as aligned as the interface requires (2 and 4 bytes):
    the finalize reads them element by element instead of in 16-byte pieces, with the same result
    against the oracle."""
    import torch
    from store_dfkv_project_amd import dfkv
    rope = RopeSpec(theta=1e6, rot=geom.rope_dim)
    wl, ds, ref = _run_case(orc, "unaligned", geom, B, rope)
    ds.kv_out.fill_(0x7FC0)
    ds.project(flags=dfkv.DFKV_FUSE_NORM_ROPE)
    torch.cuda.synchronize()
    assert_close_bf16(ds.bits(ds.kv_out), ref["kv"], "aligned")
    w_fc, w_hn, w_kv, w_kn = ds.weights[0]
    kn_buf = torch.zeros(w_kn.numel() + 8, dtype=w_kn.dtype, device=w_kn.device)
    kn_mis = kn_buf[1:1 + w_kn.numel()].view(w_kn.shape)
    kn_mis.copy_(w_kn)
    cs = ds.cos_sin
    cs_buf = torch.zeros(cs.numel() + 4, dtype=cs.dtype, device=cs.device)
    cs_mis = cs_buf[1:1 + cs.numel()].view(cs.shape)
    cs_mis.copy_(cs)
    assert kn_mis.data_ptr() % 16 == 2 and cs_mis.data_ptr() % 16 == 4
    ds.weight_structs[0] = dfkv.make_weights(w_fc, w_hn, w_kv, kn_mis, w_fc_packed=ds.w_fc_packed[0])
    ds.cos_sin = cs_mis
    ds.kv_out.fill_(0x7FC0)
    ds.project(flags=dfkv.DFKV_FUSE_NORM_ROPE)
    torch.cuda.synchronize()
    assert_close_bf16(ds.bits(ds.kv_out), ref["kv"], "unaligned")


@pytest.mark.parametrize("H,K", [(256, 512), (384, 768), (4096, 12288)])
def test_pack_fc_weight_layout(H, K):
    """dfkv_pack_fc_weight puts element (o, k) where the header's formula says: checked against the same
    permutation written as a reshape of the [H][K] matrix."""
    import torch
    from store_dfkv_project_amd import dfkv
    from store_dfkv_project_amd.step import geom_struct
    g = Geometry(kind=GQA, n_tgt=1, tgt_hidden=K, hidden=H, n_layers=1, n_kv_heads=1, head_dim=64, latent_dim=0,
                 rope_dim=64, eps=1e-6, page_size=16, width=4, block_size=4)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(H + K)
    w = torch.randint(-32768, 32768, (H, K), dtype=torch.int16, device="cuda", generator=gen)
    pk = torch.empty_like(w)
    dfkv.dfkv_pack_fc_weight(geom_struct(g), w, pk)
    torch.cuda.synchronize()
    # o = 64 b + 32 j + fr, k = 64 it + 32 h + 8 s + e  ->  [b][it][s][j][h][fr][e]
    want = w.view(H // 64, 2, 32, K // 64, 2, 4, 8).permute(0, 3, 5, 1, 4, 2, 6).reshape(H, K)
    assert torch.equal(pk, want)


@pytest.mark.parametrize("rows,cols", [(16, 128), (48, 384), (32, 1280), (1728, 7168), (4096, 12288)])
def test_pack_stream_weight_layout(rows, cols):
    """dfkv_pack_stream_weight puts element (o, k) where the header's formula says: the formula evaluated
    for every element on the host, and, for whole 1024-column ranges, the same permutation written as a
    reshape of the [rows][cols] matrix."""
    import torch
    from store_dfkv_project_amd import dfkv
    gen = torch.Generator(device="cuda")
    gen.manual_seed(rows + cols)
    w = torch.randint(-32768, 32768, (rows, cols), dtype=torch.int16, device="cuda", generator=gen)
    st = torch.empty_like(w)
    dfkv.dfkv_pack_stream_weight(rows, cols, w, st)
    torch.cuda.synchronize()
    o = torch.arange(rows, device="cuda", dtype=torch.int64)[:, None]
    k = torch.arange(cols, device="cuda", dtype=torch.int64)[None, :]
    kb, j = k // 128, k // 1024
    width = torch.clamp(cols // 128 - 8 * j, max=8)
    block = j * 8 * (rows // 16) + (o // 16) * width + kb % 8
    idx = block * 2048 + ((k % 128) // 32 * 64 + (k % 32) // 8 * 16 + o % 16) * 8 + k % 8
    flat = st.reshape(-1)
    assert torch.equal(flat[idx.reshape(-1)], w.reshape(-1))
    if cols % 1024 == 0:
        # o = 16 ob + c16, k = 1024 j + 128 w + 32 u + 8 q + e  ->  [j][ob][w][u][q][c16][e]
        want = w.view(rows // 16, 16, cols // 1024, 8, 4, 4, 8).permute(2, 0, 3, 4, 5, 1, 6).reshape(rows, cols)
        assert torch.equal(st, want)


# row counts through every weight-streaming kernel: the staged K/V groups (<= 16 rows) and the
# streaming GEMM with 1-4 row groups (17-64 rows)
STREAM_CASES = [("gqa128-B1", GQA_G, 1), ("gqa128-B4", GQA_G, 4), ("gqa128-B5", GQA_G, 5), ("gqa128-B9", GQA_G, 9),
                ("gqa128-B16", GQA_G, 16), ("gqa64-B2", GQA_G64, 2), ("gqa256-B3", GQA_G256, 3),
                ("gqa256-B21", GQA_G256, 21), ("gqaW640-B10", GQA_W1, 10), ("mla-B1", MLA_G, 1),
                ("mla-B3", MLA_G, 3), ("mla-B12", MLA_G, 12)]


@pytest.mark.parametrize("name,geom,B", STREAM_CASES, ids=[c[0] for c in STREAM_CASES])
def test_stream_weights_same_bits(orc, name, geom, B):
    """At <= 64 rows the streaming GEMMs read the tiled fc and K/V weights when given them: the projection
    (whole and staged) is bit for bit the one from the row-major weights, with either tiled copy alone
    too, and matches the oracle."""
    import torch
    from store_dfkv_project_amd import dfkv
    rope = RopeSpec(theta=1e6, rot=geom.rope_dim)
    wl, ds, ref = _run_case(orc, name, geom, B, rope)
    assert ds.N <= 64 and ds.w_stream[0][0] is not None and ds.w_stream[0][1] is not None
    tiled_struct = ds.weight_structs[0]

    def run(struct, staged=False):
        ds.weight_structs[0] = struct
        ds.kv_out.fill_(0x7FC0)
        if staged:
            ds.project_fc()
            ds.project_kv(flags=dfkv.DFKV_FUSE_NORM_ROPE)
        else:
            ds.project(flags=dfkv.DFKV_FUSE_NORM_ROPE)
        torch.cuda.synchronize()
        return ds.kv_out.clone()

    tiled = run(tiled_struct)
    assert_close_bf16(ds.bits(tiled), ref["kv"], f"{name} tiled")
    assert torch.equal(run(tiled_struct, staged=True), tiled), "staged projection with tiled weights differs"
    w_fc, w_hn, w_kv, w_kn = ds.weights[0]
    fs, ks = ds.w_stream[0]
    for label, struct in (("row-major", dfkv.make_weights(w_fc, w_hn, w_kv, w_kn)),
                          ("tiled fc only", dfkv.make_weights(w_fc, w_hn, w_kv, w_kn, w_fc_stream=fs)),
                          ("tiled K/V only", dfkv.make_weights(w_fc, w_hn, w_kv, w_kn, w_kv_stream=ks))):
        assert torch.equal(run(struct), tiled), f"{label} weights give different bits"
    ds.weight_structs[0] = tiled_struct


PACK_CASES = [("gqa128-B30", GQA_G, 30), ("gqaW640-B70", GQA_W1, 70), ("mla-B33", MLA_G, 33), ("gqa64-B37", GQA_G64, 37)]


@pytest.mark.parametrize("name,geom,B", PACK_CASES, ids=[c[0] for c in PACK_CASES])
def test_packed_fc_weight_same_bits(orc, name, geom, B):
    """Above 64 rows the fc GEMM reads the packed weight when given one: the projection (whole and
    staged) is bit for bit the one from the row-major weight, and matches the oracle."""
    import torch
    from store_dfkv_project_amd import dfkv
    rope = RopeSpec(theta=1e6, rot=geom.rope_dim)
    wl, ds, ref = _run_case(orc, name, geom, B, rope)
    assert ds.w_fc_packed[0] is not None
    ds.kv_out.fill_(0x7FC0)
    ds.project(flags=dfkv.DFKV_FUSE_NORM_ROPE)
    torch.cuda.synchronize()
    packed = ds.kv_out.clone()
    assert_close_bf16(ds.bits(packed), ref["kv"], f"{name} packed")
    ds.kv_out.fill_(0x7FC0)
    ds.project_fc()
    ds.project_kv(flags=dfkv.DFKV_FUSE_NORM_ROPE)
    torch.cuda.synchronize()
    assert torch.equal(packed, ds.kv_out), "staged projection with the packed weight differs"
    ds.weight_structs[0] = dfkv.make_weights(*ds.weights[0])
    ds.kv_out.fill_(0x7FC0)
    ds.project(flags=dfkv.DFKV_FUSE_NORM_ROPE)
    torch.cuda.synchronize()
    assert torch.equal(packed, ds.kv_out), "packed and row-major fc weights give different bits"


@pytest.mark.parametrize("geom,B", [(GQA_G, 1), (GQA_G, 4), (MLA_G, 3)], ids=["gqa128-B1", "gqa128-B4", "mla-B3"])
def test_unfused_project_without_ctx(orc, geom, B):
    """An unfused projection (flags 0) needs no context lengths, cos/sin cache or k_norm weights, and
    the header lets a caller pass NULL for them: the call is accepted, the small-batch K/V kernels
    (<= 16 rows) read none of them, and y matches the oracle -- through dfkv_project and through the
    two stages."""
    import torch
    from store_dfkv_project_amd import dfkv
    rope = RopeSpec(theta=1e6, rot=geom.rope_dim)
    wl, ds, ref = _run_case(orc, "no-ctx", geom, B, rope)
    assert ds.N <= 16
    w_fc, w_hn, w_kv, _ = ds.weights[0]
    fs, ks = ds.w_stream[0]
    no_kn = dfkv.make_weights(w_fc, w_hn, w_kv, None, w_fc_stream=fs, w_kv_stream=ks)
    ds.kv_out.fill_(0x7FC0)
    dfkv.dfkv_project(ds.gs, no_kn, ds.hidden, wl.hidden_row_stride, wl.n_reqs, None, None, 0, ds.kv_out, 0,
                      ds.ws, ds.ws_bytes)
    torch.cuda.synchronize()
    assert_close_bf16(ds.bits(ds.kv_out), ref["y"], "dfkv_project without ctx_len_in")
    first = ds.kv_out.clone()
    ds.kv_out.fill_(0x7FC0)
    dfkv.dfkv_project_fc(ds.gs, no_kn, ds.hidden, wl.hidden_row_stride, wl.n_reqs, ds.ws, ds.ws_bytes)
    dfkv.dfkv_project_kv(ds.gs, no_kn, wl.n_reqs, None, None, 0, ds.kv_out, 0, ds.ws, ds.ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(first, ds.kv_out), "staged unfused projection differs"
