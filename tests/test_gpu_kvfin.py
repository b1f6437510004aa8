"""The small-batch K/V kernels (up to 16 token rows: hidden_norm + the stacked K/V
GEMM as split-K groups, then k_norm/RoPE, the paged store and the advance in a
one-hop finalize kernel fed by bookkeeping the GEMM kernel gathered).

dfkv_step must give the same bits as the staged path (dfkv_project_fc,
dfkv_project_kv, then the separate store/advance kernel), match the oracle, work
with one workspace across batch sizes, and replay from a captured graph bit for
bit."""
import dataclasses

import numpy as np
import pytest

from dfkv_workloads import GQA, MLA, bf16_bits, make_weights, make_workload
from gpu_helpers import (assert_close_bf16, compare_bookkeeping, edge_workload, expected_pool_torch,
                         oracle_bookkeeping, small_geom)

pytestmark = pytest.mark.gpu

# Geometries the kernel takes: hidden a multiple of 1024 (K/V splits of 8 k-blocks per wave set), at
# most 16 token rows.
CASES = [
    # (seed, kind, B, W, pg, layout, L, nkv, hd, n_tgt, tgt_hidden, hidden)
    (11, GQA, 1, 4, 4, "nhd", 2, 2, 64, 1, 1024, 1024),
    (12, GQA, 4, 4, 4, "hnd", 3, 2, 64, 3, 512, 1024),
    (13, GQA, 3, 5, 16, "nhd", 2, 1, 128, 2, 1024, 2048),
    (14, GQA, 16, 1, 1, "nhd", 1, 3, 256, 1, 1536, 1024),
    (15, GQA, 2, 8, 8, "hnd", 2, 4, 128, 2, 1024, 3072),
    (16, MLA, 1, 4, 4, "nhd", 3, 1, 0, 2, 1024, 1024),
    (17, MLA, 4, 4, 16, "nhd", 2, 1, 0, 1, 2048, 2048),
    (18, MLA, 5, 3, 2, "nhd", 1, 1, 0, 3, 512, 1024),
    # latent of 1024 (two 16-byte chunks per lane) and a rope part of 128 (a latent of 448)
    (19, MLA, 2, 4, 8, "nhd", 2, 1, 0, 1, 1024, 1024, 1024, 64),
    (20, MLA, 3, 4, 8, "nhd", 2, 1, 0, 2, 512, 1024, 448, 128),
    # rows that fill part of a wave of the finishing kernel: hd 64 (8 rows a wave) with 5 rows, hd 256
    # (2 rows a wave) with 3, one MLA row with a latent of 1024 (two latent chunks a lane)
    (22, GQA, 5, 1, 4, "hnd", 2, 2, 64, 2, 1024, 2048),
    (23, GQA, 1, 3, 2, "nhd", 3, 1, 256, 1, 1536, 1024),
    (24, MLA, 1, 1, 4, "nhd", 2, 1, 0, 1, 1024, 1024, 1024, 64),
]


def _workload(case, bs=5):
    seed, kind, B, W, pg, layout, L, nkv, hd, n_tgt, tgt_hidden, hidden = case[:12]
    R, P = case[12:14] if len(case) > 12 else (512 if kind == MLA else 64, 64)
    geom = small_geom(kind, L=L, nkv=nkv, hd=hd if kind == GQA else 64, R=R, P=P, pg=pg,
                      W=W, bs=bs, n_tgt=n_tgt, tgt_hidden=tgt_hidden, hidden=hidden)
    wl = edge_workload(seed, geom, B, transposed_tokens=bool(seed % 2), with_row_valid=seed % 3 != 0)
    rng = np.random.default_rng(seed + 500)
    w = make_weights(geom, rng)
    N = B * W
    stride = geom.k_in + 8
    hid = np.full((N, stride), 0x7FC0, np.uint16)                 # NaN padding past k_in: never read
    hid[:, :geom.k_in] = bf16_bits(rng.standard_normal((N, geom.k_in)).astype(np.float32))
    return dataclasses.replace(wl, hidden=hid, hidden_row_stride=stride, w_fc=w["w_fc"], w_hnorm=w["w_hnorm"],
                               w_kv=w["w_kv"], w_knorm=w["w_knorm"]), layout


def _state(ds):
    return {k: v.clone() for k, v in (("kv", ds.kv_out), ("pool", ds.pool_t), ("slot", ds.slot),
                                      ("mask", ds.write_mask), ("ctx", ds.ctx_len_out), ("q", ds.q_pos),
                                      ("emb", ds.emb_ids), ("seq", ds.seq_len), ("bonus", ds.bonus),
                                      ("cpos", ds.c_pos), ("block", ds.block_slot))}


@pytest.mark.parametrize("case", CASES, ids=[f"seed{c[0]}-{'gqa' if c[1] == GQA else 'mla'}-M{c[2] * c[3]}"
                                             for c in CASES])
def test_step_equals_stages_and_oracle(orc, case):
    import torch
    from store_dfkv_project_amd import dfkv
    from store_dfkv_project_amd.step import DeviceStep
    wl, layout = _workload(case)
    assert wl.n_rows <= 16
    print(f"[kvfin] {case}", flush=True)
    a = DeviceStep(wl, pool_layout=layout, pool_seed=case[0])
    b = DeviceStep(wl, pool_layout=layout, pool_seed=case[0])
    before = a.pool_t.clone()
    assert torch.equal(before, b.pool_t)
    a.step()
    b.project_fc()
    b.project_kv(flags=dfkv.DFKV_FUSE_NORM_ROPE)
    b.store_advance()
    torch.cuda.synchronize()
    sa, sb = _state(a), _state(b)
    for k in sa:
        assert torch.equal(sa[k], sb[k]), f"{k}: dfkv_step differs from the staged path"
    # against the oracle
    want = oracle_bookkeeping(orc, wl)
    compare_bookkeeping(a.outputs_host(), want, f"kvfin {case}")
    exp = expected_pool_torch(a, before, a.kv_out, want["slot"], want["write_mask"])
    assert torch.equal(a.pool_t, exp), "pool differs from the expected pool"
    cs = orc.rope_cache(wl.rope, wl.cache_len)
    ref = orc.project(wl.geom, wl.hidden, wl.w_fc, wl.w_hnorm, wl.w_kv, wl.w_knorm, wl.ctx_len, cs)
    assert_close_bf16(a.bits(a.kv_out), ref["kv"], f"kvfin kv {case}")
    # again on the same workspace: same bits
    a.pool_t.copy_(before)
    a.kv_out.fill_(0x7FC0)
    a.step()
    torch.cuda.synchronize()
    for k, v in _state(a).items():
        assert torch.equal(v, sa[k]), f"second call: {k} differs"


def test_mixed_batches_one_workspace(orc):
    """Calls of different batch sizes (this kernel's and the larger-batch path) share one workspace."""
    import torch
    from store_dfkv_project_amd import dfkv
    from store_dfkv_project_amd.step import DeviceStep, geom_struct
    cs = None
    steps = []
    for i, B in enumerate((1, 4, 9, 2, 1, 6, 3)):           # M = 4, 16, 36 (larger-batch path), 8, 4, 24 (same), 12
        wl, _ = _workload((40 + i, GQA, B, 4, 16, "nhd", 2, 2, 128, 2, 512, 1024))
        steps.append(wl)
    need = max(dfkv.dfkv_workspace_size(geom_struct(wl.geom), wl.n_reqs) for wl in steps)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    dfkv.dfkv_workspace_init(ws, need)
    for wl in steps:
        ds = DeviceStep(wl, pool_seed=wl.n_reqs)
        ds.ws, ds.ws_bytes = ws, need
        before = ds.pool_t.clone()
        ds.step()
        torch.cuda.synchronize()
        want = oracle_bookkeeping(orc, wl)
        compare_bookkeeping(ds.outputs_host(), want, f"B={wl.n_reqs}")
        exp = expected_pool_torch(ds, before, ds.kv_out, want["slot"], want["write_mask"])
        assert torch.equal(ds.pool_t, exp), f"B={wl.n_reqs}: pool differs"
        cs = orc.rope_cache(wl.rope, wl.cache_len)
        ref = orc.project(wl.geom, wl.hidden, wl.w_fc, wl.w_hnorm, wl.w_kv, wl.w_knorm, wl.ctx_len, cs)
        assert_close_bf16(ds.bits(ds.kv_out), ref["kv"], f"B={wl.n_reqs} kv")


@pytest.mark.parametrize("cfg", [1, 3])
def test_bs1_graph_replay(orc, cfg):
    """The bs=1 workloads' step captured once and replayed, with eager work between replays: every
    replay reproduces the eager step bit for bit."""
    import torch
    from store_dfkv_project_amd.step import DeviceStep
    wl = make_workload(cfg, ctx_choice=2048)
    assert wl.n_rows <= 16
    ds = DeviceStep(wl)
    before = ds.pool_t.clone()
    ds.step()
    torch.cuda.synchronize()
    eager = _state(ds)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    ds.pool_t.copy_(before)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        ds.step()
    torch.cuda.synchronize()
    for rep in range(4):
        ds.pool_t.copy_(before)
        for t in (ds.kv_out, ds.slot, ds.write_mask, ds.ctx_len_out, ds.q_pos, ds.emb_ids, ds.seq_len, ds.bonus,
                  ds.c_pos):
            t.fill_(-7 if t.dtype != torch.uint8 else 7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in _state(ds).items():
            assert torch.equal(v, eager[k]), f"replay {rep}: {k} differs from the eager step"


# Block placement at the edges of the GEMM kernel's placing lanes: 16 requests x 24 block positions fill
# every lane the kernel has for it; 8 x 64 exceed them, and the step takes the streaming path, whose
# finalize places the block.
@pytest.mark.parametrize("case,bs", [((21, GQA, 16, 1, 4, "nhd", 2, 2, 64, 1, 1024, 1024), 24),
                                     ((22, GQA, 8, 2, 8, "nhd", 2, 2, 64, 1, 1024, 1024), 64),
                                     ((23, MLA, 4, 4, 4, "nhd", 2, 1, 0, 1, 1024, 1024), 100)],
                         ids=["lanes-full", "streaming-path", "mla-streaming-path"])
def test_block_placement_edges(orc, case, bs):
    import torch
    from store_dfkv_project_amd.step import DeviceStep
    wl, layout = _workload(case, bs=bs)
    print(f"[kvfin block placement] {case} bs={bs}", flush=True)
    ds = DeviceStep(wl, pool_layout=layout, pool_seed=case[0])
    before = ds.pool_t.clone()
    ds.step()
    torch.cuda.synchronize()
    want = oracle_bookkeeping(orc, wl)
    compare_bookkeeping(ds.outputs_host(), want, f"block placement {case}")
    assert (want["block_slot"] >= 0).any() and (want["block_slot"] < 0).any()
    assert torch.equal(ds.pool_t, expected_pool_torch(ds, before, ds.kv_out, want["slot"], want["write_mask"]))
