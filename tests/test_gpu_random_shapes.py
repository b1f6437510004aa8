"""dfkv_step on seeded random geometries and batch sizes against the oracle: bookkeeping bit-exact,
the pool byte-exact, K/V within the tolerance, and the fused V halves equal to the unfused
projection's.  The shapes are drawn inside what the interface accepts (GQA head dim 64/128/256 with
full rotation; MLA latent a multiple of 64 up to 1024 with an even rope part up to 128, their sum a
multiple of 64; hidden sizes multiples of 128) and the row counts span the three paths: up to 16
rows (split-K groups + finishing kernel), 17 to 64 (streaming GEMMs + finalize) and above 64 (MFMA
GEMMs, 128- or 256-token tiles).  A second, wider draw reaches 32 layers, hidden sizes from 128 to
8192 and k_in above 20000.  Each case prints its draw first."""
import dataclasses

import numpy as np
import pytest

from dfkv_workloads import GQA, MLA, bf16_bits, make_weights
from gpu_helpers import (assert_close_bf16, compare_bookkeeping, edge_workload, expected_pool_torch,
                         oracle_bookkeeping, small_geom)

pytestmark = pytest.mark.gpu

SEEDS = list(range(40))


def _draw(seed):
    rng = np.random.default_rng(9000 + seed)
    kind = GQA if rng.random() < 0.6 else MLA
    n_tgt = int(rng.integers(1, 4))
    tgt_hidden = 128 * int(rng.integers(1, 9))
    hidden = 128 * int(rng.choice([2, 3, 4, 8, 12, 16]))
    L = int(rng.integers(1, 6))
    W = int(rng.integers(1, 17))
    # row counts over the three paths, with at least 5 requests where the rows allow (the edge workload
    # gives its first four requests special tables and contexts)
    target_rows = int(rng.choice([int(rng.integers(5, 17)), int(rng.integers(17, 65)), int(rng.integers(65, 300))]))
    W = min(W, max(1, target_rows // 5))
    B = max(1, target_rows // W)
    pg = int(rng.choice([1, 2, 4, 16, 64]))
    bs = int(rng.integers(1, 9))
    if kind == GQA:
        hd = int(rng.choice([64, 128, 256]))
        nkv = int(rng.integers(1, 5))
        geom = small_geom(GQA, L=L, nkv=nkv, hd=hd, pg=pg, W=W, bs=bs, n_tgt=n_tgt, tgt_hidden=tgt_hidden,
                          hidden=hidden)
    else:
        P = 2 * int(rng.integers(1, 65))
        R = 64 * int(rng.integers(1, 17))
        while (R + P) % 64:
            P += 2
            if P > 128:
                P = 2
        geom = small_geom(MLA, L=L, R=R, P=P, pg=pg, W=W, bs=bs, n_tgt=n_tgt, tgt_hidden=tgt_hidden,
                          hidden=hidden)
    return geom, B, rng


def _draw_wide(seed):
    """Wider geometries: up to 32 layers, hidden sizes from 128 to 8192, k_in up to 25600 and up to
    about 700 rows, with the oracle's work and the pool's size bounded (None outside the bounds)."""
    rng = np.random.default_rng(77000 + seed)
    kind = GQA if rng.random() < 0.6 else MLA
    n_tgt = int(rng.integers(1, 6))
    tgt_hidden = 128 * int(rng.integers(1, 41))
    hidden = 128 * int(rng.choice([1, 2, 5, 8, 16, 24, 32, 40, 56, 64]))
    L = int(rng.choice([1, 2, 3, 7, 12, 16, 32]))
    W = int(rng.integers(1, 17))
    target_rows = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 65)), int(rng.integers(65, 700))]))
    W = min(W, max(1, target_rows // 5)) if target_rows >= 5 else 1
    B = max(1, target_rows // W)
    pg = int(rng.choice([1, 2, 4, 16, 64, 128]))
    bs = int(rng.integers(1, 17))
    if kind == GQA:
        hd = int(rng.choice([64, 128, 256]))
        nkv = int(rng.choice([1, 2, 4, 8]))
        geom = small_geom(GQA, L=L, nkv=nkv, hd=hd, pg=pg, W=W, bs=bs, n_tgt=n_tgt, tgt_hidden=tgt_hidden,
                          hidden=hidden)
        per_slot = L * 2 * nkv * hd * 2
    else:
        R = 64 * int(rng.integers(1, 17))
        P = int(rng.choice([64, 128]))
        geom = small_geom(MLA, L=L, R=R, P=P, pg=pg, W=W, bs=bs, n_tgt=n_tgt, tgt_hidden=tgt_hidden, hidden=hidden)
        per_slot = L * (R + P) * 2
    if B * W * (geom.k_in * geom.hidden + geom.hidden * geom.out_dim) > 4e10:
        return None
    if max(64, 6 * B + 2) * pg * per_slot > 2e9:     # the edge workload's pages, every layer
        return None
    return geom, B, rng


# wide draws that cover: 32 layers, hidden 128 and 8192, k_in above 20000, a large-batch GQA finalize
# with more chunks per row than one pass of its workgroup, and each of the three paths
WIDE_SEEDS = [2, 3, 8, 22, 28, 32, 33, 36, 45, 49, 51, 58, 63, 74, 79, 81, 101, 106, 119]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_step(orc, seed):
    _run(orc, seed, _draw(seed))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("seed", WIDE_SEEDS)
def test_wide_shape_step(orc, seed):
    drawn = _draw_wide(seed)
    assert drawn is not None
    _run(orc, seed, drawn)


def _run(orc, seed, drawn):
    import torch
    from store_dfkv_project_amd.step import DeviceStep
    geom, B, rng = drawn
    print(f"[random] seed {seed}: kind={'GQA' if geom.kind == GQA else 'MLA'} k_in={geom.k_in} H={geom.hidden} "
          f"L={geom.n_layers} O={geom.out_dim} W={geom.width} B={B} rows={B * geom.width} pg={geom.page_size} "
          f"block={geom.block_size}", flush=True)
    wl = edge_workload(1000 + seed, geom, B, transposed_tokens=bool(seed % 2), with_row_valid=seed % 3 != 0)
    w = make_weights(geom, rng)
    N = B * geom.width
    stride = geom.k_in + 8 * int(rng.integers(0, 3))
    hid = np.full((N, stride), 0x7FC0, np.uint16)               # NaN padding past k_in: never read
    hid[:, :geom.k_in] = bf16_bits(rng.standard_normal((N, geom.k_in)).astype(np.float32))
    wl = dataclasses.replace(wl, hidden=hid, hidden_row_stride=stride, w_fc=w["w_fc"], w_hnorm=w["w_hnorm"],
                             w_kv=w["w_kv"], w_knorm=w["w_knorm"])
    layout = "hnd" if seed % 4 == 1 else "nhd"
    ds = DeviceStep(wl, pool_layout=layout, pool_seed=seed)
    before = ds.pool_t.clone()
    ds.step()
    torch.cuda.synchronize()
    want = oracle_bookkeeping(orc, wl)
    compare_bookkeeping(ds.outputs_host(), want, f"seed {seed}")
    exp = expected_pool_torch(ds, before, ds.kv_out, want["slot"], want["write_mask"])
    assert torch.equal(ds.pool_t, exp), f"seed {seed}: pool differs"
    cs = orc.rope_cache(wl.rope, wl.cache_len)
    ref = orc.project(geom, wl.hidden, wl.w_fc, wl.w_hnorm, wl.w_kv, wl.w_knorm, wl.ctx_len, cs)
    got = ds.bits(ds.kv_out)
    assert_close_bf16(got, ref["kv"], f"seed {seed} kv")
    if geom.kind == GQA:
        # V halves: the unfused projection's bits
        ds.project(flags=0)
        torch.cuda.synchronize()
        y = ds.bits(ds.kv_out).reshape(N, -1)
        kv = geom.n_kv_heads * geom.head_dim
        for l in range(geom.n_layers):
            v0 = l * geom.per_layer + kv
            assert np.array_equal(got.reshape(N, -1)[:, v0:v0 + kv], y[:, v0:v0 + kv]), f"seed {seed} layer {l} V"
