"""CPU oracle of the decode-step context-KV update (numpy front end).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check and
by the benchmark's CPU-baseline leg, never by the product path.  It wraps
``libdfkv_oracle.so`` (plain C, fp64, built from ``dfkv_oracle.c`` in this
folder with gcc) and shares nothing with the HIP library.

bf16 tensors are numpy ``uint16`` bit patterns.  Each function names the
passage of the pages it follows in the C source's comments.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dfkv_oracle.c")
LIB = os.path.join(HERE, "libdfkv_oracle.so")


def build(out: str = LIB, mutant: int = 0, openmp: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2: no fast-math, no reassociation).  sanitize: with
    AddressSanitizer and UndefinedBehaviorSanitizer (the loading process must preload libasan)."""
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-fvisibility=hidden",
           f"-DDFKV_ORACLE_MUTANT={int(mutant)}", SRC, "-o", out + ".tmp", "-lm"]
    if openmp:
        cmd.insert(1, "-fopenmp")
    if sanitize:
        cmd[1:1] = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_P = C.c_void_p
_I = C.c_int
_I64 = C.c_int64
_D = C.c_double


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"] or a.ndim == 0
    return a.ctypes.data_as(C.c_void_p)


class Oracle:
    """Handle on one build of the oracle library (the real one, or a planted mutant)."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            if path == LIB:
                build()
            else:
                raise FileNotFoundError(path)
        self.path = path
        L = C.CDLL(path)
        L.dfkv_oracle_threads.argtypes = []
        L.dfkv_oracle_threads.restype = C.c_int
        L.dfkv_oracle_bf16_to_f64.argtypes = [C.c_uint16]
        L.dfkv_oracle_bf16_to_f64.restype = C.c_double
        L.dfkv_oracle_f64_to_bf16.argtypes = [C.c_double]
        L.dfkv_oracle_f64_to_bf16.restype = C.c_uint16
        L.dfkv_oracle_linear.argtypes = [_I, _I, _I, _P, _I64, _P, _P, _I64]
        L.dfkv_oracle_rmsnorm.argtypes = [_I, _I, _P, _I64, _P, _D, _P, _I64]
        L.dfkv_oracle_inv_freq.argtypes = [_D, _I, _I, _D, _D, _D, _D, _I, _P, _P]
        L.dfkv_oracle_rope_cache.argtypes = [_D, _I, _I, _D, _D, _D, _D, _I, _P, _I]
        L.dfkv_oracle_rope_neox.argtypes = [_I, _P, _P, _P]
        L.dfkv_oracle_norm_rope.argtypes = [_I, _I, _I, _I, _I, _I, _D, _I, _P, _I, _P, _P, _P, _I, _P, _I64]
        L.dfkv_oracle_project.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _D, _I, _P, _I64, _P, _I,
                                          _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P]
        L.dfkv_oracle_bookkeeping.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I64, _I, _I,
                                              _P, _I64, _I64, C.c_int32, _P, _P, _P, _P, _P, _P, _P, _P]
        L.dfkv_oracle_store.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I64, _I64, _I64]
        L.dfkv_oracle_block_placement.argtypes = [_I, _I, _I, _P, _P, _P, _P, _I64, _I, _I, _P]
        L.dfkv_oracle_block_table_decode.argtypes = [_I, _I, _P, _I64, _I64, _P, _I, _I, _P, _P, _I64]
        L.dfkv_oracle_strict_accept.argtypes = [_I, _I, _P, _I64, _I64, _P, _I64, _I64, _P, _P]
        L.dfkv_oracle_row_slots.argtypes = [_I, _P, _P, _I, _P, _P, _I64, _I, _I, _I, _P, _P]
        for fn in ("dfkv_oracle_linear", "dfkv_oracle_rmsnorm", "dfkv_oracle_inv_freq", "dfkv_oracle_rope_cache",
                   "dfkv_oracle_rope_neox", "dfkv_oracle_norm_rope", "dfkv_oracle_project",
                   "dfkv_oracle_bookkeeping", "dfkv_oracle_store", "dfkv_oracle_block_placement",
                   "dfkv_oracle_block_table_decode", "dfkv_oracle_strict_accept", "dfkv_oracle_row_slots"):
            getattr(L, fn).restype = None
        self.lib = L

    def threads(self) -> int:
        return int(self.lib.dfkv_oracle_threads())

    # -- scalars -----------------------------------------------------------
    def bf16_to_f64(self, h: int) -> float:
        return self.lib.dfkv_oracle_bf16_to_f64(int(h))

    def f64_to_bf16(self, x: float) -> int:
        return int(self.lib.dfkv_oracle_f64_to_bf16(float(x)))

    def round_bf16(self, a: np.ndarray) -> np.ndarray:
        a = np.asarray(a, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint16)
        flat_in, flat_out = a.reshape(-1), out.reshape(-1)
        f = self.lib.dfkv_oracle_f64_to_bf16
        for i in range(flat_in.size):
            flat_out[i] = f(float(flat_in[i]))
        return out

    # -- stages --------------------------------------------------------------
    def linear(self, x: np.ndarray, w: np.ndarray, ldx: Optional[int] = None) -> np.ndarray:
        """y = bf16(x @ w.T); x [n, >=k] uint16 (row stride ldx), w [o, k] uint16."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        n = x.shape[0]
        o, k = w.shape
        ldx = x.shape[1] if ldx is None else ldx
        y = np.empty((n, o), dtype=np.uint16)
        self.lib.dfkv_oracle_linear(n, k, o, _ptr(x), ldx, _ptr(w), _ptr(y), o)
        return y

    def rmsnorm(self, x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        n, d = x.shape
        y = np.empty_like(x)
        self.lib.dfkv_oracle_rmsnorm(n, d, _ptr(x), d, _ptr(w), float(eps), _ptr(y), d)
        return y

    def inv_freq(self, rope) -> tuple:
        inv = np.empty(rope.rot // 2, dtype=np.float64)
        m = np.zeros(1, dtype=np.float64)
        self.lib.dfkv_oracle_inv_freq(rope.theta, rope.rot, int(rope.yarn), rope.factor, rope.orig_ctx,
                                      rope.beta_fast, rope.beta_slow, int(rope.truncate), _ptr(inv), _ptr(m))
        return inv, float(m[0])

    def rope_cache(self, rope, cache_len: int) -> np.ndarray:
        cs = np.empty((cache_len, rope.rot), dtype=np.float32)
        self.lib.dfkv_oracle_rope_cache(rope.theta, rope.rot, int(rope.yarn), rope.factor, rope.orig_ctx,
                                        rope.beta_fast, rope.beta_slow, int(rope.truncate), _ptr(cs), cache_len)
        return cs

    def rope_neox(self, u: np.ndarray, cs_row: np.ndarray) -> np.ndarray:
        u = np.ascontiguousarray(u, dtype=np.uint16)
        cs_row = np.ascontiguousarray(cs_row, dtype=np.float32)
        out = np.empty_like(u)
        self.lib.dfkv_oracle_rope_neox(u.size, _ptr(u), _ptr(cs_row), _ptr(out))
        return out

    def norm_rope(self, geom, y: np.ndarray, w_knorm: np.ndarray, ctx_len: np.ndarray, cs: np.ndarray,
                  row_ids: Optional[Sequence[int]] = None) -> np.ndarray:
        out = np.array(y, dtype=np.uint16, copy=True, order="C")
        n = out.shape[0]
        rid = None if row_ids is None else np.ascontiguousarray(row_ids, dtype=np.int32)
        ctx = np.ascontiguousarray(ctx_len, dtype=np.int32)
        wk = np.ascontiguousarray(w_knorm, dtype=np.uint16)
        cs = np.ascontiguousarray(cs, dtype=np.float32)
        self.lib.dfkv_oracle_norm_rope(geom.kind, geom.n_layers, geom.n_kv_heads, geom.head_dim, geom.latent_dim,
                                       geom.rope_dim, float(geom.eps), geom.width, _ptr(rid), n, _ptr(ctx), _ptr(wk),
                                       _ptr(cs), cs.shape[0], _ptr(out), out.shape[1])
        return out

    def project(self, geom, hidden: np.ndarray, w_fc, w_hnorm, w_kv, w_knorm, ctx_len, cs,
                row_ids: Optional[Sequence[int]] = None) -> dict:
        """Projection of the selected rows (all rows when row_ids is None).

        ``hidden`` holds every row of the step ([N, row_stride]); only the
        selected rows are computed.  Returns f, g, y (pre norm/RoPE) and kv."""
        hidden = np.ascontiguousarray(hidden, dtype=np.uint16)
        if row_ids is None:
            row_ids = np.arange(hidden.shape[0], dtype=np.int32)
        rid = np.ascontiguousarray(row_ids, dtype=np.int32)
        x = np.ascontiguousarray(hidden[rid])
        n = len(rid)
        H, O = geom.hidden, geom.out_dim
        f = np.empty((n, H), np.uint16)
        g = np.empty((n, H), np.uint16)
        y = np.empty((n, O), np.uint16)
        kv = np.empty((n, O), np.uint16)
        ctx = np.ascontiguousarray(ctx_len, dtype=np.int32)
        cs = np.ascontiguousarray(cs, dtype=np.float32)
        args = [np.ascontiguousarray(a, dtype=np.uint16) for a in (w_fc, w_hnorm, w_kv, w_knorm)]
        self.lib.dfkv_oracle_project(geom.kind, geom.k_in, H, geom.n_layers, geom.n_kv_heads, geom.head_dim,
                                     geom.latent_dim, geom.rope_dim, float(geom.eps), geom.width,
                                     _ptr(x), x.shape[1], _ptr(rid), n, *[_ptr(a) for a in args], _ptr(ctx),
                                     _ptr(cs), cs.shape[0], _ptr(f), _ptr(g), _ptr(y), _ptr(kv))
        return dict(f=f, g=g, y=y, kv=kv, row_ids=rid)

    def bookkeeping(self, geom, n_reqs, ctx_len, n_acc, alloc_limit, is_dummy, row_valid, block_table,
                    accepted_tokens, acc_stride_req, acc_stride_tok, mask_token_id, num_pages,
                    bt_stride: Optional[int] = None) -> dict:
        B, W, bs = n_reqs, geom.width, geom.block_size
        N = B * W
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        bt_cols = bt.shape[1] if bt.ndim == 2 else int(bt.size // max(B, 1))
        bt_stride = bt_cols if bt_stride is None else bt_stride
        out = dict(slot=np.empty(N, np.int64), write_mask=np.empty(N, np.uint8), c_pos=np.empty(N, np.int32),
                   bonus=np.empty(B, np.int32), emb_ids=np.empty(B * bs, np.int32), q_pos=np.empty(B * bs, np.int32),
                   ctx_len=np.empty(B, np.int32), seq_len=np.empty(B, np.int32))
        rv = None if row_valid is None else np.ascontiguousarray(row_valid, dtype=np.uint8)
        ins = [np.ascontiguousarray(a, dtype=t) for a, t in ((ctx_len, np.int32), (n_acc, np.int32),
                                                             (alloc_limit, np.int32), (is_dummy, np.uint8))]
        acc = np.ascontiguousarray(accepted_tokens, dtype=np.int32)
        self.lib.dfkv_oracle_bookkeeping(B, W, bs, geom.page_size, *[_ptr(a) for a in ins], _ptr(rv), _ptr(bt),
                                         bt_stride, bt_cols, num_pages, _ptr(acc), acc_stride_req, acc_stride_tok,
                                         int(mask_token_id), _ptr(out["slot"]), _ptr(out["write_mask"]),
                                         _ptr(out["c_pos"]), _ptr(out["bonus"]), _ptr(out["emb_ids"]),
                                         _ptr(out["q_pos"]), _ptr(out["ctx_len"]), _ptr(out["seq_len"]))
        out["emb_ids"] = out["emb_ids"].reshape(B, bs)
        out["q_pos"] = out["q_pos"].reshape(B, bs)
        out["c_pos"] = out["c_pos"].reshape(B, W)
        out["block_slot"] = self.block_placement(geom, n_reqs, out["ctx_len"], alloc_limit, is_dummy, bt, bt_stride,
                                                 bt_cols, num_pages)
        return out

    def block_placement(self, geom, n_reqs, ctx_new, alloc_limit, is_dummy, block_table, bt_stride, bt_cols,
                        num_pages) -> np.ndarray:
        """Slots of the next draft block's own positions ctx' + j, j < block_size ([B, block_size] int64, -1 where
        the position is not in an allocated page): the block placement of the downstream commit quoted on the
        PR #20550 page."""
        B, bs = n_reqs, geom.block_size
        out = np.empty(B * bs, np.int64)
        ins = [np.ascontiguousarray(a, dtype=t) for a, t in ((ctx_new, np.int32), (alloc_limit, np.int32),
                                                             (is_dummy, np.uint8))]
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        self.lib.dfkv_oracle_block_placement(B, bs, geom.page_size, *[_ptr(a) for a in ins], _ptr(bt), bt_stride,
                                             bt_cols, num_pages, _ptr(out))
        return out.reshape(B, bs)

    def block_table_decode(self, offsets_buf: np.ndarray, s_req: int, s_blk: int, n_reqs: int, max_blocks: int,
                           n_tokens, page_size: int, divisor: int):
        """Draft-KV block-table decode (PR #20550 page: page counts and the decoded table; clamped and divided
        offsets).  `offsets_buf` is the storage of a strided view: element (r, b) at r*s_req + b*s_blk.
        Returns (page_count [B] int32, table [B, max_blocks] int32)."""
        buf = np.ascontiguousarray(offsets_buf, dtype=np.int32)
        cnt = np.empty(n_reqs, np.int32)
        tbl = np.empty((n_reqs, max_blocks), np.int32)
        nt = np.ascontiguousarray(n_tokens, dtype=np.int32)
        self.lib.dfkv_oracle_block_table_decode(n_reqs, max_blocks, _ptr(buf), s_req, s_blk, _ptr(nt), page_size,
                                                divisor, _ptr(cnt), _ptr(tbl), max_blocks)
        return cnt, tbl

    def strict_accept(self, target_buf, t_sr: int, t_st: int, draft_buf, d_sr: int, d_st: int, n_reqs: int,
                      width: int):
        """Strict acceptance of a uniform-width draft (the downstream commit quoted on the PR #20550 page).
        Returns (n_acc [B] int32, accepted [B, width] int32 = the target's tokens)."""
        t = np.ascontiguousarray(target_buf, dtype=np.int32)
        d = np.ascontiguousarray(draft_buf, dtype=np.int32)
        n_acc = np.empty(n_reqs, np.int32)
        acc = np.empty((n_reqs, width), np.int32)
        self.lib.dfkv_oracle_strict_accept(n_reqs, width, _ptr(t), t_sr, t_st, _ptr(d), d_sr, d_st, _ptr(n_acc),
                                           _ptr(acc))
        return n_acc, acc

    def row_slots(self, geom, row_req, row_pos, n_reqs: int, alloc_limit, block_table, num_pages: int,
                  bt_stride: Optional[int] = None):
        """Destinations of prefill-shaped (ragged) rows: row n of request row_req[n] at position row_pos[n]
        (the single-latent context scatter of the PR #20550 page at any row count).  Returns (slot, write_mask)."""
        rq = np.ascontiguousarray(row_req, dtype=np.int32)
        rp = np.ascontiguousarray(row_pos, dtype=np.int32)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        bt_cols = bt.shape[1] if bt.ndim == 2 else int(bt.size // max(n_reqs, 1))
        bt_stride = bt_cols if bt_stride is None else bt_stride
        n = rq.size
        slot, wm = np.empty(n, np.int64), np.empty(n, np.uint8)
        self.lib.dfkv_oracle_row_slots(n, _ptr(rq), _ptr(rp), n_reqs, _ptr(np.ascontiguousarray(alloc_limit, np.int32)),
                                       _ptr(bt), bt_stride, bt_cols, geom.page_size, num_pages, _ptr(slot), _ptr(wm))
        return slot, wm

    def store(self, geom, kv: np.ndarray, slot: np.ndarray, write_mask: np.ndarray, pools_k: Sequence[np.ndarray],
              pools_v: Optional[Sequence[np.ndarray]], s_page: int, s_slot: int, s_head: int) -> None:
        """Write into host pools in place (each pool a contiguous uint16 array)."""
        kv = np.ascontiguousarray(kv, dtype=np.uint16)
        L = geom.n_layers
        for p in list(pools_k) + list(pools_v or []):
            assert p.dtype == np.uint16 and p.flags["C_CONTIGUOUS"]
        pk = (C.c_void_p * L)(*[p.ctypes.data for p in pools_k])
        pv = (C.c_void_p * L)(*[p.ctypes.data for p in pools_v]) if pools_v is not None else None
        self.lib.dfkv_oracle_store(geom.kind, L, geom.n_kv_heads, geom.head_dim, geom.latent_dim, geom.rope_dim,
                                   geom.page_size, kv.shape[0], _ptr(kv), _ptr(np.ascontiguousarray(slot, np.int64)),
                                   _ptr(np.ascontiguousarray(write_mask, np.uint8)), pk, pv, s_page, s_slot, s_head)


_default: Optional[Oracle] = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
