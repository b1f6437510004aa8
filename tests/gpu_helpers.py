"""Helpers for the GPU parity tests: tolerance checks, edge-case step builders,
and pool expectations built independently of the HIP library."""
from __future__ import annotations

import dataclasses

import numpy as np

from dfkv_workloads import (GQA, MLA, Geometry, RopeSpec, Workload, bits_to_f32, make_block_table, make_workload,
                            MASK_TOKEN_ID, VOCAB)

# Tolerance for projected K/V (bf16 inputs, fp32 accumulation): elementwise
# |got - ref| <= ATOL + RTOL*|ref|.  A plain 2e-2 absolute bound alone would
# reject legitimate one-spacing bf16 differences once |x| >= 4 (spacing 2^-5).
ATOL = 2e-2
RTOL = 1e-2


def assert_close_bf16(got_bits, ref_bits, what: str = "", atol: float = ATOL, rtol: float = RTOL) -> dict:
    g = bits_to_f32(np.asarray(got_bits, np.uint16)).astype(np.float64)
    r = bits_to_f32(np.asarray(ref_bits, np.uint16)).astype(np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    err = np.abs(g - r)
    bound = atol + rtol * np.abs(r)
    bad = err > bound
    rel = err / np.maximum(np.abs(r), 1e-6)
    # the bound read literally, each part alone: elements off by more than 2e-2, and the largest
    # relative error where the relative part is the tighter one (|ref| >= 2)
    big = np.abs(r) >= 2.0
    stats = dict(max_abs=float(err.max(initial=0.0)), max_rel_of_large=float(rel[np.abs(r) > 0.1].max(initial=0.0)),
                 max_rel_ref_ge_2=float(rel[big].max(initial=0.0)), n_abs_over_2e_2=int((err > atol).sum()),
                 n=int(err.size))
    if bad.any():
        i = np.argmax(err - bound)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance; "
                             f"worst at flat {int(i)}: got {g.flat[i]!r} ref {r.flat[i]!r}; {stats}")
    return stats


def small_geom(kind: int, L: int = 2, nkv: int = 2, hd: int = 64, R: int = 64, P: int = 64, pg: int = 4, W: int = 4,
               bs: int = 3, n_tgt: int = 1, tgt_hidden: int = 128, hidden: int = 128) -> Geometry:
    if kind == GQA:
        return Geometry(kind=GQA, n_tgt=n_tgt, tgt_hidden=tgt_hidden, hidden=hidden, n_layers=L, n_kv_heads=nkv,
                        head_dim=hd, latent_dim=0, rope_dim=hd, eps=1e-6, page_size=pg, width=W, block_size=bs)
    return Geometry(kind=MLA, n_tgt=n_tgt, tgt_hidden=tgt_hidden, hidden=hidden, n_layers=L, n_kv_heads=1,
                    head_dim=0, latent_dim=R, rope_dim=P, eps=1e-6, page_size=pg, width=W, block_size=bs)


def edge_workload(seed: int, geom: Geometry, B: int, num_pages: int = 64, transposed_tokens: bool = False,
                  with_row_valid: bool = True) -> Workload:
    """Bookkeeping edge cases: dummies, n_acc in [0, W], requests at / over their allocation, contexts
    that outrun their pages, negative / out-of-range / all-negative / all-zero table rows, optional
    per-row rejection.  Page ids are unique across the whole batch (page 0 is reserved for at most one
    all-zero row), so no two rows share a destination."""
    rng = np.random.default_rng(seed)
    W, pg = geom.width, geom.page_size
    cols = int(rng.integers(2, 7))
    ctx = rng.integers(0, cols * pg + 3, size=B).astype(np.int32)
    n_acc = rng.integers(0, W + 1, size=B).astype(np.int32)
    lim = np.where(rng.random(B) < 0.5, rng.integers(0, cols * pg + 1, size=B),
                   cols * pg).astype(np.int32)
    dummy = (rng.random(B) < 0.15).astype(np.uint8)
    need = B * cols
    P = max(num_pages, need + 2)
    ids = (rng.permutation(P - 1)[:need] + 1).reshape(B, cols).astype(np.int32)  # page 0 reserved
    bt = ids.copy()
    bad = rng.random((B, cols)) < 0.2
    bt[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1 - rng.integers(0, 5, size=int(bad.sum())),
                       P + rng.integers(0, 5, size=int(bad.sum())))
    special = rng.permutation(B)
    if B >= 1:
        bt[special[0], :] = -1                   # all-negative row
    if B >= 2 and pg >= W:
        bt[special[1], :] = 0                    # all-zero row (page 0 used only here)
    if B >= 3:
        ctx[special[2]] = lim[special[2]] + 2    # context that outran its allocation
    if B >= 4:
        n_acc[special[3]] = W
        ctx[special[3]] = max(0, int(lim[special[3]]) - 1)   # at the allocation ceiling
    row_valid = (rng.random(B * W) < 0.8).astype(np.uint8) if with_row_valid else None
    tok = rng.integers(0, VOCAB, size=(B, W)).astype(np.int32)
    if transposed_tokens:
        acc_buf, sr, st = np.ascontiguousarray(tok.T), 1, B
    else:
        acc_buf, sr, st = tok, W, 1
    N = B * W
    hidden = np.zeros((N, geom.k_in), np.uint16)
    return Workload(config_id=-1, name=f"edge-{seed}", geom=geom, rope=RopeSpec(theta=1e4, rot=geom.rope_dim),
                    n_reqs=B, hidden=hidden, hidden_row_stride=geom.k_in, w_fc=None, w_hnorm=None, w_kv=None,
                    w_knorm=None, ctx_len=ctx, n_acc=n_acc, alloc_limit=lim, is_dummy=dummy, row_valid=row_valid,
                    block_table=bt, accepted_tokens=acc_buf, acc_stride_req=sr, acc_stride_tok=st,
                    mask_token_id=MASK_TOKEN_ID, num_pages=P, cache_len=int(max(ctx.max(), lim.max()) + W + 8))


def oracle_bookkeeping(orc, wl: Workload) -> dict:
    return orc.bookkeeping(wl.geom, wl.n_reqs, wl.ctx_len, wl.n_acc, wl.alloc_limit, wl.is_dummy, wl.row_valid,
                           wl.block_table, wl.accepted_tokens, wl.acc_stride_req, wl.acc_stride_tok,
                           wl.mask_token_id, wl.num_pages)


def compare_bookkeeping(got: dict, want: dict, what: str = "") -> None:
    for k in ("slot", "write_mask", "c_pos", "bonus", "emb_ids", "q_pos", "ctx_len", "seq_len", "block_slot"):
        g, w = np.asarray(got[k]).reshape(-1), np.asarray(want[k]).reshape(-1)
        if not np.array_equal(g, w):
            i = int(np.nonzero(g != w)[0][0])
            raise AssertionError(f"{what}: {k} differs at {i}: got {g[i]} want {w[i]}")


def expected_pool_torch(ds, before, kv_dev, slot: np.ndarray, write_mask: np.ndarray):
    """The pool after the step, built with torch indexing from the pre-image: every written row's
    layer slices land at their slot; nothing else changes."""
    import torch
    exp = before.clone()
    g = ds.geom
    rows = np.nonzero(write_mask)[0]
    if rows.size == 0:
        return exp
    rows_t = torch.from_numpy(rows).to(kv_dev.device)
    slots_t = torch.from_numpy(slot[rows]).to(kv_dev.device)
    kvr = kv_dev[rows_t].view(len(rows), g.n_layers, -1)
    if g.kind == GQA:
        nkv, hd, pg, P = g.n_kv_heads, g.head_dim, g.page_size, ds.wl.num_pages
        page, off = slots_t // pg, slots_t % pg
        for l in range(g.n_layers):
            for half in range(2):
                src = kvr[:, l, half * nkv * hd:(half + 1) * nkv * hd].reshape(len(rows), nkv, hd)
                if ds.pool_layout == "nhd":
                    exp[l, half][page, off] = src
                else:
                    exp[l, half][page, :, off] = src
    else:
        row = g.latent_dim + g.rope_dim
        for l in range(g.n_layers):
            exp[l].view(-1, row)[slots_t] = kvr[:, l, :]
    return exp
