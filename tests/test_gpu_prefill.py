"""Prefill-shaped (ragged) context and the dense per-slot buffer: the same store at other shapes and
layouts (TensorRT-LLM PR #20550 "fuse the decode-step drafter bookkeeping into Triton kernels": the
single-latent context scatter among its fused kernels; PR #13995 "DFlash performance optimizations":
the per-slot buffer [max_batch, L, max_ctx + block, nkv, hd] of the older dense variant).

Ragged rows: dfkv_project with width 1 (each row its own RoPE position) then dfkv_paged_store_rows; the
destinations are bit-exact against the oracle's, the pool against the rows scattered by torch indexing,
the projection within the tolerance.  Dense buffer: dfkv_store_advance on a pool whose page is a batch
slot of max_ctx + block positions."""
import dataclasses

import numpy as np
import pytest

from dfkv_workloads import GQA, MLA, MASK_TOKEN_ID, Geometry, RopeSpec, Workload, bf16_bits, make_weights
from gpu_helpers import assert_close_bf16, compare_bookkeeping, expected_pool_torch, oracle_bookkeeping

pytestmark = pytest.mark.gpu

GQA_P = Geometry(kind=GQA, n_tgt=2, tgt_hidden=256, hidden=384, n_layers=2, n_kv_heads=2, head_dim=128, latent_dim=0,
                 rope_dim=128, eps=1e-6, page_size=16, width=1, block_size=4)
MLA_P = Geometry(kind=MLA, n_tgt=2, tgt_hidden=256, hidden=512, n_layers=2, n_kv_heads=1, head_dim=0, latent_dim=512,
                 rope_dim=64, eps=1e-6, page_size=16, width=1, block_size=7)


def _ragged(seed, geom, lens):
    rng = np.random.default_rng(seed)
    B = len(lens)
    start = rng.integers(0, 400, size=B).astype(np.int32)
    row_req = np.repeat(np.arange(B, dtype=np.int32), lens)
    row_pos = np.concatenate([start[r] + np.arange(n, dtype=np.int32) for r, n in enumerate(lens)]).astype(np.int32)
    N = int(row_req.size)
    pg = geom.page_size
    cols = int((start.max() + max(lens)) // pg + 2)
    P = B * cols + 8
    bt = (rng.permutation(P)[:B * cols]).reshape(B, cols).astype(np.int32)
    lim = (start + np.array(lens)).astype(np.int32)
    if B > 1:
        bt[rng.random((B, cols)) < 0.1] = -1
        bt[0, 0] = P + 3                                  # a page past the pool
        lim = (lim - rng.integers(0, 6, size=B)).astype(np.int32)     # some rows past the limit
    rng2 = np.random.default_rng(seed + 1)
    hidden = bf16_bits(rng2.standard_normal((N, geom.k_in)).astype(np.float32))
    w = make_weights(geom, rng2)
    cache_len = int(row_pos.max()) + 8
    # the projection view: one "request" per row, width 1, RoPE position = the row's position
    wl = Workload(config_id=-1, name="prefill", geom=geom, rope=RopeSpec(theta=1e6, rot=geom.rope_dim), n_reqs=N,
                  hidden=hidden, hidden_row_stride=geom.k_in, w_fc=w["w_fc"], w_hnorm=w["w_hnorm"], w_kv=w["w_kv"],
                  w_knorm=w["w_knorm"], ctx_len=row_pos, n_acc=np.ones(N, np.int32),
                  alloc_limit=np.full(N, 1 << 30, np.int32), is_dummy=np.zeros(N, np.uint8), row_valid=None,
                  block_table=np.zeros((N, 1), np.int32), accepted_tokens=np.zeros((N, 1), np.int32),
                  acc_stride_req=1, acc_stride_tok=1, mask_token_id=MASK_TOKEN_ID, num_pages=P, cache_len=cache_len)
    return wl, row_req, row_pos, B, lim, bt, P


@pytest.mark.parametrize("geom,lens", [(GQA_P, [1, 37, 120, 5, 200]), (MLA_P, [64, 3, 90]), (GQA_P, [1])],
                         ids=["gqa-ragged", "mla-ragged", "gqa-one-row"])
def test_ragged_prefill_store(orc, geom, lens):
    import torch
    from store_dfkv_project_amd import dfkv
    from store_dfkv_project_amd.step import DeviceStep
    wl, row_req, row_pos, B, lim, bt, P = _ragged(31, geom, lens)
    print(f"[prefill] kind {geom.kind} rows {wl.n_reqs}", flush=True)
    ds = DeviceStep(wl, pool_seed=5)
    ds.project()
    torch.cuda.synchronize()
    cs = orc.rope_cache(wl.rope, wl.cache_len)
    ref = orc.project(geom, wl.hidden, wl.w_fc, wl.w_hnorm, wl.w_kv, wl.w_knorm, wl.ctx_len, cs)
    assert_close_bf16(ds.bits(ds.kv_out), ref["kv"], "prefill kv")
    before = ds.pool_t.clone()
    N = wl.n_reqs
    slot = torch.full((N,), -5, dtype=torch.int64, device="cuda")
    wm = torch.full((N,), 7, dtype=torch.uint8, device="cuda")
    d = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in
         (("rq", row_req), ("rp", row_pos), ("lim", lim), ("bt", bt))}
    dfkv.dfkv_paged_store_rows(ds.gs, ds.kv_out, N, d["rq"], d["rp"], B, d["lim"], d["bt"], bt.shape[1], bt.shape[1],
                               ds.pool, slot, wm)
    torch.cuda.synchronize()
    want_slot, want_wm = orc.row_slots(geom, row_req, row_pos, B, lim, bt, P)
    assert np.array_equal(slot.cpu().numpy(), want_slot)
    assert np.array_equal(wm.cpu().numpy(), want_wm)
    assert want_wm.sum() > 0 and (N == 1 or (want_wm == 0).any())
    assert torch.equal(ds.pool_t, expected_pool_torch(ds, before, ds.kv_out, want_slot, want_wm))


def test_dense_per_slot_buffer(orc):
    """The per-slot buffer [max_batch][L][T][nkv][hd] (K and V buffers) through dfkv_store_advance: a page is a
    batch slot of T = max_ctx + block positions, the table has one column (the request's slot)."""
    import torch
    from dfkv_workloads import make_workload
    from store_dfkv_project_amd import dfkv
    from store_dfkv_project_amd.step import DeviceStep
    print("[prefill] dense per-slot buffer", flush=True)
    base = make_workload(0)
    g0 = base.geom
    T = 128 + g0.block_size                                # max_ctx + block
    g = dataclasses.replace(g0, page_size=T)
    B, W, L, nkv, hd = base.n_reqs, g.width, g.n_layers, g.n_kv_heads, g.head_dim
    max_batch = 6
    rng = np.random.default_rng(12)
    slots = rng.permutation(max_batch)[:B].astype(np.int32)
    wl = dataclasses.replace(base, geom=g, block_table=slots.reshape(B, 1), num_pages=max_batch,
                             alloc_limit=np.minimum(base.alloc_limit, T).astype(np.int32))
    ds = DeviceStep(wl, pool_seed=6)                      # for the projection, requests and outputs
    ds.project()
    torch.cuda.synchronize()
    bufk = torch.randint(-32768, 32768, (max_batch, L, T, nkv, hd), dtype=torch.int16, device="cuda")
    bufv = torch.randint(-32768, 32768, (max_batch, L, T, nkv, hd), dtype=torch.int16, device="cuda")
    k0, v0 = bufk.clone(), bufv.clone()
    pool = dfkv.make_pool([bufk[:, l] for l in range(L)], [bufv[:, l] for l in range(L)], L * T * nkv * hd, nkv * hd,
                          hd, max_batch)
    dfkv.dfkv_store_advance(ds.gs, ds.kv_out, ds.req, pool, ds.outs)
    torch.cuda.synchronize()
    want = oracle_bookkeeping(orc, wl)
    compare_bookkeeping(ds.outputs_host(), want, "dense buffer")
    rows = np.nonzero(want["write_mask"])[0]
    assert rows.size > 0
    kv = ds.kv_out.view(B * W, L, 2, nkv, hd)
    for n in rows:
        s = int(want["slot"][n])
        b, pos = s // T, s % T
        k0[b, :, pos] = kv[n, :, 0]
        v0[b, :, pos] = kv[n, :, 1]
    assert torch.equal(bufk, k0) and torch.equal(bufv, v0)
