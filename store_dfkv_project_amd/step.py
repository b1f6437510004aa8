"""Device buffers for one decode step, wired to the libdfkv entry points.

Plumbing only: torch allocates device memory and supplies the stream; every
step of the path runs in libdfkv's HIP kernels through ``dfkv``.  A step is
described by any object with the fields of ``dfkv_workloads.Workload`` (host
numpy arrays; bf16 tensors as uint16 bit patterns).
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import dfkv

GQA, MLA = dfkv.DFKV_GQA, dfkv.DFKV_MLA


def _dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def geom_struct(geom) -> dfkv.dfkv_geom:
    return dfkv.make_geom(kind=geom.kind, n_tgt=geom.n_tgt, tgt_hidden=geom.tgt_hidden, hidden=geom.hidden,
                          n_layers=geom.n_layers, n_kv_heads=geom.n_kv_heads, head_dim=geom.head_dim,
                          latent_dim=geom.latent_dim, rope_dim=geom.rope_dim, eps=geom.eps,
                          page_size=geom.page_size, width=geom.width, block_size=geom.block_size)


def rope_struct(rope) -> dfkv.dfkv_rope:
    return dfkv.make_rope(rope.theta, rope.rot, rope.yarn, rope.factor, rope.orig_ctx, rope.beta_fast,
                          rope.beta_slow, rope.truncate)


class DeviceStep:
    """All device buffers of one step.

    pool_layout: "nhd" ([page][slot][head][dim]) or "hnd" ([page][head][slot][dim]); MLA pools are
    [page][slot][R+P].  weight_copies > 1 keeps that many copies of the weights at distinct addresses
    (so that a timing loop can rotate through them and read them from HBM, not from the cache).
    pack_fc: also give each copy a packed fc weight (dfkv_pack_fc_weight), which the large-batch fc
    GEMM then reads.  pack_stream: also give each copy tiled fc and K/V weights
    (dfkv_pack_stream_weight), which the weight-streaming GEMMs of <= 64 rows then read; None packs
    them when the workload has <= 64 rows.
    """

    def __init__(self, wl, device: str = "cuda", pool_layout: str = "nhd", weight_copies: int = 1,
                 pool_seed: int = 1234, with_weights: bool = True, pack_fc: bool = True,
                 pack_stream: Optional[bool] = None):
        self.wl = wl
        g = wl.geom
        self.geom = g
        self.gs = geom_struct(g)
        self.device = device
        B, W = wl.n_reqs, g.width
        N = B * W
        self.N = N
        self.O = g.out_dim
        # projection inputs
        self.hidden = _dev(wl.hidden, device)
        self.weights = []
        self.w_fc_packed = []
        self.w_stream = []
        self.weight_structs = []
        if pack_stream is None:
            pack_stream = N <= 64
        if with_weights and wl.w_fc is not None:
            base = [_dev(wl.w_fc, device), _dev(wl.w_hnorm, device), _dev(wl.w_kv, device), _dev(wl.w_knorm, device)]
            for c in range(weight_copies):
                ws = base if c == 0 else [t.clone() for t in base]
                self.weights.append(ws)
                pk = None
                if pack_fc:
                    pk = torch.empty_like(ws[0])
                    dfkv.dfkv_pack_fc_weight(self.gs, ws[0], pk)
                self.w_fc_packed.append(pk)
                st = (None, None)
                if pack_stream:
                    st = (torch.empty_like(ws[0]), torch.empty_like(ws[2]))
                    dfkv.dfkv_pack_stream_weight(g.hidden, g.k_in, ws[0], st[0])
                    dfkv.dfkv_pack_stream_weight(g.out_dim, g.hidden, ws[2], st[1])
                self.w_stream.append(st)
                self.weight_structs.append(dfkv.make_weights(*ws, w_fc_packed=pk, w_fc_stream=st[0],
                                                             w_kv_stream=st[1]))
        # request state
        self.ctx_len = _dev(wl.ctx_len.astype(np.int32), device)
        self.n_acc = _dev(wl.n_acc.astype(np.int32), device)
        self.alloc_limit = _dev(wl.alloc_limit.astype(np.int32), device)
        self.is_dummy = _dev(wl.is_dummy.astype(np.uint8), device)
        self.row_valid = None if wl.row_valid is None else _dev(wl.row_valid.astype(np.uint8), device)
        self.block_table = _dev(wl.block_table.astype(np.int32), device)
        self.accepted = _dev(wl.accepted_tokens.astype(np.int32), device)
        bt_cols = wl.block_table.shape[1]
        self.req = dfkv.make_requests(B, self.ctx_len, self.n_acc, self.alloc_limit, self.is_dummy, self.row_valid,
                                      self.block_table, bt_cols, bt_cols, self.accepted, wl.acc_stride_req,
                                      wl.acc_stride_tok, wl.mask_token_id)
        # one cos/sin cache, built on the GPU
        self.cache_len = wl.cache_len
        self.cos_sin = torch.empty((wl.cache_len, g.rope_dim), dtype=torch.float32, device=device)
        dfkv.dfkv_rope_cache_build(rope_struct(wl.rope), self.cos_sin, wl.cache_len)
        # pools (one allocation, per-layer views), random-byte pre-image
        P, pg = wl.num_pages, g.page_size
        gen = torch.Generator(device=device)
        gen.manual_seed(pool_seed)
        if g.kind == GQA:
            nkv, hd = g.n_kv_heads, g.head_dim
            if pool_layout == "nhd":
                shape = (g.n_layers, 2, P, pg, nkv, hd)
                sp, ss, sh = pg * nkv * hd, nkv * hd, hd
            elif pool_layout == "hnd":
                shape = (g.n_layers, 2, P, nkv, pg, hd)
                sp, ss, sh = nkv * pg * hd, hd, pg * hd
            else:
                raise ValueError(pool_layout)
            self.pool_t = torch.randint(-32768, 32768, shape, dtype=torch.int16, device=device, generator=gen)
            ks = [self.pool_t[l, 0] for l in range(g.n_layers)]
            vs = [self.pool_t[l, 1] for l in range(g.n_layers)]
        else:
            row = g.latent_dim + g.rope_dim
            shape = (g.n_layers, P, pg, row)
            sp, ss, sh = pg * row, row, 0
            self.pool_t = torch.randint(-32768, 32768, shape, dtype=torch.int16, device=device, generator=gen)
            ks = [self.pool_t[l] for l in range(g.n_layers)]
            vs = None
        self.pool_layout = pool_layout
        self.pool_strides = (sp, ss, sh)
        self.pool = dfkv.make_pool(ks, vs, sp, ss, sh, P)
        # outputs
        self.kv_out = torch.zeros((N, self.O), dtype=torch.int16, device=device)
        self.slot = torch.zeros(N, dtype=torch.int64, device=device)
        self.write_mask = torch.zeros(N, dtype=torch.uint8, device=device)
        self.c_pos = torch.zeros(N, dtype=torch.int32, device=device)
        self.bonus = torch.zeros(B, dtype=torch.int32, device=device)
        self.emb_ids = torch.zeros(B * g.block_size, dtype=torch.int32, device=device)
        self.q_pos = torch.zeros(B * g.block_size, dtype=torch.int32, device=device)
        self.ctx_len_out = torch.zeros(B, dtype=torch.int32, device=device)
        self.seq_len = torch.zeros(B, dtype=torch.int32, device=device)
        # block placement (written by store_advance / step; -7 marks an entry nothing wrote)
        self.block_slot = torch.full((B * g.block_size,), -7, dtype=torch.int64, device=device)
        self.outs = dfkv.make_outputs(self.slot, self.write_mask, self.c_pos, self.bonus, self.emb_ids, self.q_pos,
                                      self.ctx_len_out, self.seq_len, self.block_slot)
        # dfkv_advance takes no pool, so it places no block
        self.outs_adv = dfkv.make_outputs(self.slot, self.write_mask, self.c_pos, self.bonus, self.emb_ids,
                                          self.q_pos, self.ctx_len_out, self.seq_len)
        # workspace
        self.ws_bytes = dfkv.dfkv_workspace_size(self.gs, B)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        dfkv.dfkv_workspace_init(self.ws, self.ws.numel())

    # -- entry points ------------------------------------------------------------
    def project(self, flags: int = dfkv.DFKV_FUSE_NORM_ROPE, copy: int = 0, stream=None, kv_out=None):
        dfkv.dfkv_project(self.gs, self.weight_structs[copy], self.hidden, self.wl.hidden_row_stride, self.wl.n_reqs,
                          self.ctx_len, self.cos_sin, self.cache_len, self.kv_out if kv_out is None else kv_out,
                          flags, self.ws, self.ws_bytes, stream)

    def project_fork(self, main, aux, fork, join, flags: int = dfkv.DFKV_FUSE_NORM_ROPE, copy: int = 0):
        """The projection on `aux` after the work queued on `main` so far (with DFKV_FORK_RECORDED in
        `flags`: after the `fork` the caller recorded); `join` recorded after it (fork / join: raw
        hipEvent_t handles)."""
        dfkv.dfkv_project_fork(self.gs, self.weight_structs[copy], self.hidden, self.wl.hidden_row_stride,
                               self.wl.n_reqs, self.ctx_len, self.cos_sin, self.cache_len, self.kv_out, flags,
                               self.ws, self.ws_bytes, main, aux, fork, join)

    def project_fc(self, copy: int = 0, stream=None):
        dfkv.dfkv_project_fc(self.gs, self.weight_structs[copy], self.hidden, self.wl.hidden_row_stride,
                             self.wl.n_reqs, self.ws, self.ws_bytes, stream)

    def project_kv(self, flags: int = dfkv.DFKV_FUSE_NORM_ROPE, copy: int = 0, stream=None):
        dfkv.dfkv_project_kv(self.gs, self.weight_structs[copy], self.wl.n_reqs, self.ctx_len, self.cos_sin,
                             self.cache_len, self.kv_out, flags, self.ws, self.ws_bytes, stream)

    def norm_rope(self, kv, stream=None):
        dfkv.dfkv_norm_rope(self.gs, self.weights[0][3], self.wl.n_reqs, self.ctx_len, self.cos_sin, self.cache_len,
                            kv, stream)

    def paged_store(self, kv=None, stream=None):
        dfkv.dfkv_paged_store(self.gs, self.kv_out if kv is None else kv, self.req, self.pool, self.slot,
                              self.write_mask, stream)

    def advance(self, stream=None):
        dfkv.dfkv_advance(self.gs, self.req, self.outs_adv, stream)

    def store_advance(self, kv=None, stream=None):
        dfkv.dfkv_store_advance(self.gs, self.kv_out if kv is None else kv, self.req, self.pool, self.outs, stream)

    def step(self, copy: int = 0, stream=None):
        dfkv.dfkv_step(self.gs, self.weight_structs[copy], self.hidden, self.wl.hidden_row_stride, self.req,
                       self.cos_sin, self.cache_len, self.kv_out, self.pool, self.outs, self.ws, self.ws_bytes, stream)

    # -- host views --------------------------------------------------------------
    def bits(self, t: torch.Tensor) -> np.ndarray:
        return t.cpu().numpy().view(np.uint16)

    def outputs_host(self) -> dict:
        g = self.geom
        B = self.wl.n_reqs
        return dict(slot=self.slot.cpu().numpy(), write_mask=self.write_mask.cpu().numpy(),
                    c_pos=self.c_pos.cpu().numpy().reshape(B, g.width), bonus=self.bonus.cpu().numpy(),
                    emb_ids=self.emb_ids.cpu().numpy().reshape(B, g.block_size),
                    q_pos=self.q_pos.cpu().numpy().reshape(B, g.block_size),
                    ctx_len=self.ctx_len_out.cpu().numpy(), seq_len=self.seq_len.cpu().numpy(),
                    block_slot=self.block_slot.cpu().numpy().reshape(B, g.block_size))

    def pool_slot_view(self, layer: int, half: int = 0) -> torch.Tensor:
        """Pool of one layer as [num_pages*page_size, slot_elems] rows (NHD / MLA layouts)."""
        g = self.geom
        if g.kind == GQA:
            t = self.pool_t[layer, half]
            if self.pool_layout == "hnd":
                t = t.transpose(1, 2)
            return t.reshape(-1, g.n_kv_heads * g.head_dim)
        return self.pool_t[layer].reshape(-1, g.latent_dim + g.rope_dim)
