"""Seeded synthetic inputs for the decode-step context-KV update.

This module only draws data: tensor shapes, value distributions and the
request mix of the five workloads (tiny, dense bs=1, dense bs=64, MLA bs=1,
stress bs=256).  It holds none of the method's arithmetic, so both the HIP
library's tests/benchmark and the CPU oracle can consume what it produces.

Everything is returned as host numpy arrays; bf16 tensors are ``uint16``
bit patterns.  The drafter shapes follow the pages' workloads:

* dense (GQA) drafter of a Qwen3-8B-class target: three captured target
  layers of hidden 4096, drafter hidden 4096, five drafter layers with 8 KV
  heads of dim 128 (TensorRT-LLM PR #13995 "DFlash performance
  optimizations", commit "migrate draft path to per-layer cached K/V pool");
* MLA DSpark drafter: single 512-wide latent plus 64 rope dims per layer,
  one pool geometry shared by all layers (TensorRT-LLM PR #20550,
  TLLM_DFLASH_FUSED_PROLOGUE).

Verify width W = K+1 rows per request (PR #13995, commit "drop K-1 filler
tokens from target gen input").
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

GQA = 0
MLA = 1

VOCAB = 151936
MASK_TOKEN_ID = 151935


@dataclass(frozen=True)
class Geometry:
    kind: int            # GQA or MLA
    n_tgt: int           # captured target layers
    tgt_hidden: int      # hidden size of each captured layer
    hidden: int          # drafter hidden H (fc output)
    n_layers: int        # drafter layers L
    n_kv_heads: int      # GQA: KV heads; MLA: 1
    head_dim: int        # GQA: head dim; MLA: 0
    latent_dim: int      # MLA: latent width R; GQA: 0
    rope_dim: int        # rotated dims per head (GQA: head_dim; MLA: rope part P)
    eps: float           # one eps for hidden_norm and the k/latent norm
    page_size: int
    width: int           # W = K+1 rows per request
    block_size: int      # drafter block (query length of the next draft block)

    @property
    def k_in(self) -> int:
        return self.n_tgt * self.tgt_hidden

    @property
    def per_layer(self) -> int:
        if self.kind == GQA:
            return 2 * self.n_kv_heads * self.head_dim
        return self.latent_dim + self.rope_dim

    @property
    def out_dim(self) -> int:
        return self.n_layers * self.per_layer

    @property
    def knorm_dim(self) -> int:
        return self.head_dim if self.kind == GQA else self.latent_dim

    @property
    def slot_elems(self) -> int:
        """bf16 elements one token occupies in one layer's K (or latent) pool."""
        if self.kind == GQA:
            return self.n_kv_heads * self.head_dim
        return self.latent_dim + self.rope_dim


@dataclass(frozen=True)
class RopeSpec:
    theta: float
    rot: int
    yarn: bool = False
    factor: float = 1.0
    orig_ctx: float = 0.0
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    truncate: bool = False


@dataclass
class Workload:
    """One step's inputs.  Row ``n = r*W + i`` is token i of request r."""
    config_id: int
    name: str
    geom: Geometry
    rope: RopeSpec
    n_reqs: int
    # projection inputs
    hidden: np.ndarray            # uint16 [N, hidden_row_stride] (only first k_in used)
    hidden_row_stride: int
    w_fc: np.ndarray              # uint16 [H, k_in]
    w_hnorm: np.ndarray           # uint16 [H]
    w_kv: np.ndarray              # uint16 [O, H]
    w_knorm: np.ndarray           # uint16 [L, knorm_dim]
    # request state
    ctx_len: np.ndarray           # int32 [B]
    n_acc: np.ndarray             # int32 [B]
    alloc_limit: np.ndarray       # int32 [B]
    is_dummy: np.ndarray          # uint8 [B]
    row_valid: Optional[np.ndarray]  # uint8 [N] or None
    block_table: np.ndarray       # int32 [B, bt_cols] (row stride = bt_cols)
    accepted_tokens: np.ndarray   # int32 buffer; element (r, t) at r*acc_stride_req + t*acc_stride_tok
    acc_stride_req: int
    acc_stride_tok: int
    mask_token_id: int
    num_pages: int
    cache_len: int
    meta: dict = field(default_factory=dict)

    @property
    def n_rows(self) -> int:
        return self.n_reqs * self.geom.width


# ---------------------------------------------------------------------------
# data helpers (no method arithmetic)
# ---------------------------------------------------------------------------

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 samples to bf16 (nearest, ties to even); return bit patterns.

    Used only to turn random draws into bf16 input tensors."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return bf16_bits(x)


def make_weights(geom: Geometry, rng: np.random.Generator) -> dict:
    """Weights N(0, std=1/sqrt(fan_in)); norm weights 1 + N(0, 0.02)."""
    H, Kin, O = geom.hidden, geom.k_in, geom.out_dim
    return dict(
        w_fc=_normal_bf16(rng, (H, Kin), std=1.0 / math.sqrt(Kin)),
        w_hnorm=_normal_bf16(rng, (H,), std=0.02, mean=1.0),
        w_kv=_normal_bf16(rng, (O, H), std=1.0 / math.sqrt(H)),
        w_knorm=_normal_bf16(rng, (geom.n_layers, geom.knorm_dim), std=0.02, mean=1.0),
    )


def page_aligned_limit(ctx: np.ndarray, need: int, pg: int) -> np.ndarray:
    """Allocation limit = pages_allocated * page_size, with enough pages for ctx+need tokens."""
    return (((ctx.astype(np.int64) + need + pg - 1) // pg) * pg).astype(np.int32)


def make_block_table(rng: np.random.Generator, ctx: np.ndarray, limit: np.ndarray, pg: int,
                     num_pages: int, bt_cols: Optional[int] = None) -> np.ndarray:
    """Random non-contiguous block tables.

    Pages that cover positions [ctx, limit) are distinct across requests and
    drawn without replacement; entries below the ctx page are never touched by
    the step and are drawn with replacement; entries past the allocation are -1.
    """
    B = len(ctx)
    lim_pages = (limit.astype(np.int64) + pg - 1) // pg
    if bt_cols is None:
        bt_cols = int(max(1, lim_pages.max()))
    bt = np.full((B, bt_cols), -1, dtype=np.int32)
    first_win = np.minimum(ctx.astype(np.int64) // pg, lim_pages)
    n_win = int(np.maximum(lim_pages - first_win, 0).sum())
    if n_win > num_pages:
        raise ValueError(f"pool of {num_pages} pages too small for {n_win} writable pages")
    win_ids = rng.permutation(num_pages)[:n_win].astype(np.int32)
    k = 0
    for r in range(B):
        a, b = int(first_win[r]), int(min(lim_pages[r], bt_cols))
        if a > 0:
            bt[r, :min(a, bt_cols)] = rng.integers(0, num_pages, size=min(a, bt_cols), dtype=np.int32)
        if b > a:
            bt[r, a:b] = win_ids[k:k + (b - a)]
            k += b - a
    return bt


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def _geom_dense(W: int, bs_blk: int) -> Geometry:
    return Geometry(kind=GQA, n_tgt=3, tgt_hidden=4096, hidden=4096, n_layers=5, n_kv_heads=8,
                    head_dim=128, latent_dim=0, rope_dim=128, eps=1e-6, page_size=64,
                    width=W, block_size=bs_blk)


GEOMS = {
    0: Geometry(kind=GQA, n_tgt=3, tgt_hidden=256, hidden=256, n_layers=2, n_kv_heads=2, head_dim=64,
                latent_dim=0, rope_dim=64, eps=1e-6, page_size=16, width=4, block_size=4),
    1: _geom_dense(4, 16),
    2: _geom_dense(16, 16),
    3: Geometry(kind=MLA, n_tgt=3, tgt_hidden=7168, hidden=7168, n_layers=3, n_kv_heads=1, head_dim=0,
                latent_dim=512, rope_dim=64, eps=1e-6, page_size=64, width=4, block_size=7),
    4: _geom_dense(16, 16),
}

ROPES = {
    0: RopeSpec(theta=1e6, rot=64),
    1: RopeSpec(theta=1e6, rot=128),
    2: RopeSpec(theta=1e6, rot=128),
    3: RopeSpec(theta=1e6, rot=64, yarn=True, factor=40.0, orig_ctx=4096.0, truncate=False),
    4: RopeSpec(theta=1e6, rot=128, yarn=True, factor=4.0, orig_ctx=32768.0, truncate=False),
}

NAMES = {
    0: "tiny-gqa-b2",
    1: "dense-gqa-bs1",
    2: "dense-gqa-bs64",
    3: "mla-dspark-bs1",
    4: "stress-gqa-yarn-bs256",
}

DEFAULT_POOL_PAGES = {0: 32, 1: 512, 2: 4096, 3: 2048, 4: 2048}
CTX_CHOICES = {1: (2048, 32768), 3: (2048, 131072, 393216)}


def make_workload(config_id: int, ctx_choice: Optional[int] = None, seed: Optional[int] = None,
                  num_pages: Optional[int] = None, weights: bool = True,
                  n_reqs: Optional[int] = None) -> Workload:
    """Build one step's inputs for a workload.

    ``ctx_choice`` picks the fixed context length of the bs=1 workloads
    (dense: 2048 / 32768; MLA: 2048 / 131072 / 393216).  ``n_reqs`` overrides
    the batch (used for scaled-down parity cases of the same recipe).
    """
    geom, rope = GEOMS[config_id], ROPES[config_id]
    rng = np.random.default_rng(1000 + config_id if seed is None else seed)
    W, pg, bs_blk = geom.width, geom.page_size, geom.block_size
    P = DEFAULT_POOL_PAGES[config_id] if num_pages is None else num_pages
    B = {0: 2, 1: 1, 2: 64, 3: 1, 4: 256}[config_id] if n_reqs is None else n_reqs

    w = make_weights(geom, rng) if weights else dict(w_fc=None, w_hnorm=None, w_kv=None, w_knorm=None)
    row_stride = geom.k_in + (64 if config_id == 4 else 0)
    N = B * W
    hidden = np.zeros((N, row_stride), dtype=np.uint16)
    hidden[:, :geom.k_in] = _normal_bf16(rng, (N, geom.k_in))
    if row_stride > geom.k_in:
        hidden[:, geom.k_in:] = 0x7FC0  # NaN in the padding: must never be read

    is_dummy = np.zeros(B, dtype=np.uint8)
    row_valid = None
    meta = {}
    if config_id == 0:
        n_acc = rng.integers(1, W + 1, size=B).astype(np.int32)
        ctx = rng.integers(8, 101, size=B).astype(np.int32)
        limit = np.full(B, 128, dtype=np.int32)
        bt = make_block_table(rng, ctx, limit, pg, P, bt_cols=8)
    elif config_id in (1, 3):
        c = CTX_CHOICES[config_id][0] if ctx_choice is None else ctx_choice
        n_acc = rng.integers(1, W + 1, size=B).astype(np.int32)
        ctx = np.full(B, c, dtype=np.int32)
        limit = page_aligned_limit(ctx, W + bs_blk, pg)
        bt = make_block_table(rng, ctx, limit, pg, P)
        meta["ctx_len"] = c
    elif config_id == 2:
        n_acc = rng.integers(1, W + 1, size=B).astype(np.int32)
        ctx = rng.integers(512, 32769, size=B).astype(np.int32)
        limit = page_aligned_limit(ctx, W + bs_blk, pg)
        row_valid = (rng.random(N) >= 0.10).astype(np.uint8)
        bt = make_block_table(rng, ctx, limit, pg, P)
    elif config_id == 4:
        n_acc = rng.integers(1, W + 1, size=B).astype(np.int32)
        ctx = rng.integers(1024, 65537, size=B).astype(np.int32)
        limit = page_aligned_limit(ctx, W + bs_blk, pg)
        near = rng.random(B) < 0.20
        # requests within 8 tokens of a page-aligned allocation limit
        lim_near = (((ctx.astype(np.int64) + pg - 1) // pg) * pg).astype(np.int32)
        d = rng.integers(0, 9, size=B).astype(np.int32)
        ctx = np.where(near, lim_near - d, ctx).astype(np.int32)
        limit = np.where(near, lim_near, limit).astype(np.int32)
        is_dummy = (rng.random(B) < 0.10).astype(np.uint8)
        bt = make_block_table(rng, ctx, limit, pg, P)
        meta["near_limit"] = near.astype(np.uint8)
    else:
        raise KeyError(config_id)

    # accepted tokens: [B, W] row-major, except the stress workload which stores
    # them transposed ([W, B]) so the per-request view is strided.
    tok = rng.integers(0, VOCAB, size=(B, W)).astype(np.int32)
    if config_id == 4:
        acc_buf = np.ascontiguousarray(tok.T)
        acc_sr, acc_st = 1, B
    else:
        acc_buf = tok
        acc_sr, acc_st = W, 1

    max_pos = int(max(int(limit.max()), int(ctx.max()) + W) + bs_blk)
    cache_len = max_pos + 1

    return Workload(config_id=config_id, name=NAMES[config_id], geom=geom, rope=rope, n_reqs=B,
                    hidden=hidden, hidden_row_stride=row_stride, w_fc=w["w_fc"], w_hnorm=w["w_hnorm"],
                    w_kv=w["w_kv"], w_knorm=w["w_knorm"], ctx_len=ctx, n_acc=n_acc, alloc_limit=limit,
                    is_dummy=is_dummy, row_valid=row_valid, block_table=bt, accepted_tokens=acc_buf,
                    acc_stride_req=acc_sr, acc_stride_tok=acc_st, mask_token_id=MASK_TOKEN_ID,
                    num_pages=P, cache_len=cache_len, meta=meta)


def with_geometry(wl: Workload, **changes) -> Workload:
    return dataclasses.replace(wl, **changes)


def pool_bytes_per_page(geom: Geometry) -> int:
    """Bytes of one page across all layers (K and V pools for GQA, latent pool for MLA)."""
    per_layer = geom.page_size * geom.slot_elems * 2
    return geom.n_layers * per_layer * (2 if geom.kind == GQA else 1)


def random_pool_bytes(nbytes: int, seed: int) -> np.ndarray:
    """Random (nonzero) byte pre-image for a pool."""
    return np.frombuffer(np.random.default_rng(seed).bytes(nbytes), dtype=np.uint8).copy()
