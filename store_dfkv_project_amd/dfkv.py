"""ctypes binding of libdfkv (include/dfkv.h).

Argument marshalling only: every function here has the name of the C entry
point it calls, turns tensors into pointers and the current HIP stream into a
``hipStream_t``, and raises :class:`DfkvError` when the call returns a status
other than ``DFKV_OK``.  All computation happens in the HIP kernels of
``libdfkv.so``; there is no fallback path -- importing this module fails if
the library has not been built.

Pointer arguments accept a torch tensor (``data_ptr()``), a numpy array, a
plain integer address, or ``None`` (NULL).
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdfkv.so")

DFKV_OK = 0
DFKV_ERR_NULL = -1
DFKV_ERR_SHAPE = -2
DFKV_ERR_LAYOUT = -3
DFKV_ERR_ALIAS = -4
DFKV_ERR_WORKSPACE = -5
DFKV_ERR_HIP = -6
DFKV_NOALLOC_SCRATCH_BYTES = 8 << 20   # include/dfkv.h: the static scratch of dfkv_step_noalloc

DFKV_GQA = 0
DFKV_MLA = 1
DFKV_MAX_LAYERS = 32
DFKV_FUSE_NORM_ROPE = 1
DFKV_FORK_RECORDED = 2

EXPORTED = ("dfkv_status_string", "dfkv_version", "dfkv_hip_error_string", "dfkv_workspace_size", "dfkv_workspace_init",
            "dfkv_rope_cache_build", "dfkv_project", "dfkv_project_fc", "dfkv_project_kv", "dfkv_norm_rope", "dfkv_paged_store", "dfkv_advance",
            "dfkv_store_advance", "dfkv_step", "dfkv_project_fork", "dfkv_join", "dfkv_block_table_decode",
            "dfkv_strict_accept", "dfkv_paged_store_rows", "dfkv_pack_fc_weight", "dfkv_pack_stream_weight",
            "dfkv_step_noalloc")


class dfkv_geom(C.Structure):
    _fields_ = [("kind", C.c_int32), ("n_tgt", C.c_int32), ("tgt_hidden", C.c_int32), ("hidden", C.c_int32),
                ("n_layers", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("latent_dim", C.c_int32), ("rope_dim", C.c_int32), ("eps", C.c_float), ("page_size", C.c_int32),
                ("width", C.c_int32), ("block_size", C.c_int32)]


class dfkv_weights(C.Structure):
    _fields_ = [("w_fc", C.c_void_p), ("w_hnorm", C.c_void_p), ("w_kv", C.c_void_p), ("w_knorm", C.c_void_p),
                ("w_fc_packed", C.c_void_p), ("w_fc_stream", C.c_void_p), ("w_kv_stream", C.c_void_p)]


class dfkv_requests(C.Structure):
    _fields_ = [("n_reqs", C.c_int32), ("ctx_len_in", C.c_void_p), ("n_acc", C.c_void_p),
                ("alloc_limit", C.c_void_p), ("is_dummy", C.c_void_p), ("row_valid", C.c_void_p),
                ("block_table", C.c_void_p), ("bt_row_stride", C.c_int64), ("bt_cols", C.c_int32),
                ("accepted_tokens", C.c_void_p), ("acc_stride_req", C.c_int64), ("acc_stride_tok", C.c_int64),
                ("mask_token_id", C.c_int32)]


class dfkv_pool(C.Structure):
    _fields_ = [("k", C.c_void_p * DFKV_MAX_LAYERS), ("v", C.c_void_p * DFKV_MAX_LAYERS),
                ("stride_page", C.c_int64), ("stride_slot", C.c_int64), ("stride_head", C.c_int64),
                ("num_pages", C.c_int32)]


class dfkv_outputs(C.Structure):
    _fields_ = [("slot", C.c_void_p), ("write_mask", C.c_void_p), ("c_pos", C.c_void_p), ("bonus", C.c_void_p),
                ("emb_ids", C.c_void_p), ("q_pos", C.c_void_p), ("ctx_len_out", C.c_void_p),
                ("seq_len", C.c_void_p), ("block_slot", C.c_void_p)]


class dfkv_rope(C.Structure):
    _fields_ = [("theta", C.c_double), ("rot", C.c_int32), ("yarn", C.c_int32), ("factor", C.c_double),
                ("orig_ctx", C.c_double), ("beta_fast", C.c_double), ("beta_slow", C.c_double),
                ("truncate", C.c_int32)]


class DfkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = dfkv_status_string(status) if _lib is not None else str(status)
        if status == DFKV_ERR_HIP and _lib is not None:
            msg += f" ({dfkv_hip_error_string()})"
        super().__init__(f"{where}: {msg}")


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run store_dfkv_project_amd.build.build() (hipcc, gfx950)")
    # One HIP runtime per process: torch ships its own libamdhip64.so.7, and the
    # tensors handed to libdfkv live in torch's runtime.  Importing torch first
    # makes the dynamic loader bind libdfkv's libamdhip64.so.7 to that same copy
    # (same SONAME) instead of loading a second runtime from /opt/rocm.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = C.CDLL(LIB_PATH)
    P, I32, I64, SZ, U32 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_uint32
    gp, wp, rp, pp, op = (C.POINTER(dfkv_geom), C.POINTER(dfkv_weights), C.POINTER(dfkv_requests),
                          C.POINTER(dfkv_pool), C.POINTER(dfkv_outputs))
    sig = {
        "dfkv_status_string": ([C.c_int], C.c_char_p),
        "dfkv_version": ([], C.c_char_p),
        "dfkv_hip_error_string": ([], C.c_char_p),
        "dfkv_workspace_size": ([gp, I32, C.POINTER(C.c_size_t)], C.c_int),
        "dfkv_workspace_init": ([P, SZ, P], C.c_int),
        "dfkv_rope_cache_build": ([C.POINTER(dfkv_rope), P, I32, P], C.c_int),
        "dfkv_project": ([gp, wp, P, I64, I32, P, P, I32, P, U32, P, SZ, P], C.c_int),
        "dfkv_project_fc": ([gp, wp, P, I64, I32, P, SZ, P], C.c_int),
        "dfkv_pack_fc_weight": ([gp, P, P, P], C.c_int),
        "dfkv_pack_stream_weight": ([I64, I64, P, P, P], C.c_int),
        "dfkv_project_kv": ([gp, wp, I32, P, P, I32, P, U32, P, SZ, P], C.c_int),
        "dfkv_norm_rope": ([gp, P, I32, P, P, I32, P, P], C.c_int),
        "dfkv_paged_store": ([gp, P, rp, pp, P, P, P], C.c_int),
        "dfkv_advance": ([gp, rp, op, P], C.c_int),
        "dfkv_store_advance": ([gp, P, rp, pp, op, P], C.c_int),
        "dfkv_step": ([gp, wp, P, I64, rp, P, I32, P, pp, op, P, SZ, P], C.c_int),
        "dfkv_step_noalloc": ([gp, wp, P, I64, rp, P, I32, P, pp, op, P], C.c_int),
        "dfkv_project_fork": ([gp, wp, P, I64, I32, P, P, I32, P, U32, P, SZ, P, P, P, P], C.c_int),
        "dfkv_join": ([P, P], C.c_int),
        "dfkv_block_table_decode": ([P, I64, I64, I32, I32, P, I32, I32, P, P, I64, P], C.c_int),
        "dfkv_strict_accept": ([P, I64, I64, P, I64, I64, I32, I32, P, P, P], C.c_int),
        "dfkv_paged_store_rows": ([gp, P, I32, P, P, I32, P, P, I64, I32, pp, P, P, P], C.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


_lib: Optional[C.CDLL] = None
_lib = _load()


def lib() -> C.CDLL:
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError(f"cannot take a device pointer of {type(x)!r}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ref(x):
    return None if x is None else C.byref(x)


def _check(status: int, where: str) -> None:
    if status != DFKV_OK:
        raise DfkvError(status, where)


def make_geom(**kw) -> dfkv_geom:
    g = dfkv_geom()
    for k, v in kw.items():
        setattr(g, k, v)
    return g


def make_weights(w_fc, w_hnorm, w_kv, w_knorm, w_fc_packed=None, w_fc_stream=None, w_kv_stream=None) -> dfkv_weights:
    return dfkv_weights(_ptr(w_fc), _ptr(w_hnorm), _ptr(w_kv), _ptr(w_knorm), _ptr(w_fc_packed), _ptr(w_fc_stream),
                        _ptr(w_kv_stream))


def make_requests(n_reqs, ctx_len_in, n_acc, alloc_limit, is_dummy, row_valid, block_table, bt_row_stride, bt_cols,
                  accepted_tokens, acc_stride_req, acc_stride_tok, mask_token_id) -> dfkv_requests:
    return dfkv_requests(int(n_reqs), _ptr(ctx_len_in), _ptr(n_acc), _ptr(alloc_limit), _ptr(is_dummy),
                         _ptr(row_valid), _ptr(block_table), int(bt_row_stride), int(bt_cols), _ptr(accepted_tokens),
                         int(acc_stride_req), int(acc_stride_tok), int(mask_token_id))


def make_pool(k: Sequence, v: Optional[Sequence], stride_page: int, stride_slot: int, stride_head: int,
              num_pages: int) -> dfkv_pool:
    p = dfkv_pool()
    for i, t in enumerate(k):
        p.k[i] = _ptr(t)
    for i, t in enumerate(v or []):
        p.v[i] = _ptr(t)
    p.stride_page, p.stride_slot, p.stride_head, p.num_pages = stride_page, stride_slot, stride_head, num_pages
    return p


def make_outputs(slot=None, write_mask=None, c_pos=None, bonus=None, emb_ids=None, q_pos=None, ctx_len_out=None,
                 seq_len=None, block_slot=None) -> dfkv_outputs:
    return dfkv_outputs(_ptr(slot), _ptr(write_mask), _ptr(c_pos), _ptr(bonus), _ptr(emb_ids), _ptr(q_pos),
                        _ptr(ctx_len_out), _ptr(seq_len), _ptr(block_slot))


def make_rope(theta, rot, yarn=False, factor=1.0, orig_ctx=0.0, beta_fast=32.0, beta_slow=1.0,
              truncate=False) -> dfkv_rope:
    return dfkv_rope(float(theta), int(rot), int(bool(yarn)), float(factor), float(orig_ctx), float(beta_fast),
                     float(beta_slow), int(bool(truncate)))


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def dfkv_status_string(status: int) -> str:
    return _lib.dfkv_status_string(int(status)).decode()


def dfkv_version() -> str:
    return _lib.dfkv_version().decode()


def dfkv_hip_error_string() -> str:
    return _lib.dfkv_hip_error_string().decode()


def dfkv_workspace_size(geom: dfkv_geom, n_reqs: int) -> int:
    out = C.c_size_t(0)
    _check(_lib.dfkv_workspace_size(_ref(geom), int(n_reqs), C.byref(out)), "dfkv_workspace_size")
    return int(out.value)


def dfkv_workspace_init(ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(_lib.dfkv_workspace_init(_ptr(ws), int(nbytes), _stream(stream)), "dfkv_workspace_init")


def dfkv_rope_cache_build(rope: dfkv_rope, cos_sin, cache_len: Optional[int] = None, stream=None) -> None:
    n = cache_len if cache_len is not None else int(cos_sin.shape[0])
    _check(_lib.dfkv_rope_cache_build(_ref(rope), _ptr(cos_sin), int(n), _stream(stream)), "dfkv_rope_cache_build")


def dfkv_project(geom, weights, hidden, hidden_row_stride, n_reqs, ctx_len_in, cos_sin, cache_len, kv_out, flags,
                 ws, ws_bytes, stream=None) -> None:
    _check(_lib.dfkv_project(_ref(geom), _ref(weights), _ptr(hidden), int(hidden_row_stride), int(n_reqs),
                             _ptr(ctx_len_in), _ptr(cos_sin), int(cache_len), _ptr(kv_out), int(flags), _ptr(ws),
                             int(ws_bytes), _stream(stream)), "dfkv_project")


def dfkv_project_fork(geom, weights, hidden, hidden_row_stride, n_reqs, ctx_len_in, cos_sin, cache_len, kv_out,
                      flags, ws, ws_bytes, main, aux, fork, join) -> None:
    """`fork`/`join`: hipEvent_t handles (torch.cuda.Event.cuda_event after the event exists)."""
    _check(_lib.dfkv_project_fork(_ref(geom), _ref(weights), _ptr(hidden), int(hidden_row_stride), int(n_reqs),
                                  _ptr(ctx_len_in), _ptr(cos_sin), int(cache_len), _ptr(kv_out), int(flags),
                                  _ptr(ws), int(ws_bytes), _stream(main), _stream(aux), C.c_void_p(fork),
                                  C.c_void_p(join)), "dfkv_project_fork")


def dfkv_block_table_decode(offsets, off_stride_req, off_stride_blk, n_reqs, max_blocks, n_tokens, page_size,
                            divisor, page_count_out, table_out, table_row_stride, stream=None) -> None:
    _check(_lib.dfkv_block_table_decode(_ptr(offsets), int(off_stride_req), int(off_stride_blk), int(n_reqs),
                                        int(max_blocks), _ptr(n_tokens), int(page_size), int(divisor),
                                        _ptr(page_count_out), _ptr(table_out), int(table_row_stride),
                                        _stream(stream)), "dfkv_block_table_decode")


def dfkv_strict_accept(target, t_stride_req, t_stride_tok, draft, d_stride_req, d_stride_tok, n_reqs, width,
                       n_acc_out, accepted_out, stream=None) -> None:
    _check(_lib.dfkv_strict_accept(_ptr(target), int(t_stride_req), int(t_stride_tok), _ptr(draft),
                                   int(d_stride_req), int(d_stride_tok), int(n_reqs), int(width), _ptr(n_acc_out),
                                   _ptr(accepted_out), _stream(stream)), "dfkv_strict_accept")


def dfkv_paged_store_rows(geom, kv, n_rows, row_req, row_pos, n_reqs, alloc_limit, block_table, bt_row_stride,
                          bt_cols, pool, slot_out, write_mask_out, stream=None) -> None:
    _check(_lib.dfkv_paged_store_rows(_ref(geom), _ptr(kv), int(n_rows), _ptr(row_req), _ptr(row_pos), int(n_reqs),
                                      _ptr(alloc_limit), _ptr(block_table), int(bt_row_stride), int(bt_cols),
                                      _ref(pool), _ptr(slot_out), _ptr(write_mask_out), _stream(stream)),
           "dfkv_paged_store_rows")


def dfkv_join(main, join) -> None:
    _check(_lib.dfkv_join(_stream(main), C.c_void_p(join)), "dfkv_join")


def dfkv_project_fc(geom, weights, hidden, hidden_row_stride, n_reqs, ws, ws_bytes, stream=None) -> None:
    _check(_lib.dfkv_project_fc(_ref(geom), _ref(weights), _ptr(hidden), int(hidden_row_stride), int(n_reqs),
                                _ptr(ws), int(ws_bytes), _stream(stream)), "dfkv_project_fc")


def dfkv_pack_fc_weight(geom, w_fc, w_fc_packed, stream=None) -> None:
    _check(_lib.dfkv_pack_fc_weight(_ref(geom), _ptr(w_fc), _ptr(w_fc_packed), _stream(stream)),
           "dfkv_pack_fc_weight")


def dfkv_pack_stream_weight(rows, cols, w, w_stream, stream=None) -> None:
    _check(_lib.dfkv_pack_stream_weight(int(rows), int(cols), _ptr(w), _ptr(w_stream), _stream(stream)),
           "dfkv_pack_stream_weight")


def dfkv_project_kv(geom, weights, n_reqs, ctx_len_in, cos_sin, cache_len, kv_out, flags, ws, ws_bytes,
                    stream=None) -> None:
    _check(_lib.dfkv_project_kv(_ref(geom), _ref(weights), int(n_reqs), _ptr(ctx_len_in), _ptr(cos_sin),
                                int(cache_len), _ptr(kv_out), int(flags), _ptr(ws), int(ws_bytes), _stream(stream)),
           "dfkv_project_kv")


def dfkv_norm_rope(geom, w_knorm, n_reqs, ctx_len_in, cos_sin, cache_len, kv, stream=None) -> None:
    _check(_lib.dfkv_norm_rope(_ref(geom), _ptr(w_knorm), int(n_reqs), _ptr(ctx_len_in), _ptr(cos_sin),
                               int(cache_len), _ptr(kv), _stream(stream)), "dfkv_norm_rope")


def dfkv_paged_store(geom, kv, requests, pool, slot_out, write_mask_out, stream=None) -> None:
    _check(_lib.dfkv_paged_store(_ref(geom), _ptr(kv), _ref(requests), _ref(pool), _ptr(slot_out),
                                 _ptr(write_mask_out), _stream(stream)), "dfkv_paged_store")


def dfkv_advance(geom, requests, outputs, stream=None) -> None:
    _check(_lib.dfkv_advance(_ref(geom), _ref(requests), _ref(outputs), _stream(stream)), "dfkv_advance")


def dfkv_store_advance(geom, kv, requests, pool, outputs, stream=None) -> None:
    _check(_lib.dfkv_store_advance(_ref(geom), _ptr(kv), _ref(requests), _ref(pool), _ref(outputs),
                                   _stream(stream)), "dfkv_store_advance")


def dfkv_step(geom, weights, hidden, hidden_row_stride, requests, cos_sin, cache_len, kv_out, pool, outputs, ws,
              ws_bytes, stream=None) -> None:
    _check(_lib.dfkv_step(_ref(geom), _ref(weights), _ptr(hidden), int(hidden_row_stride), _ref(requests),
                          _ptr(cos_sin), int(cache_len), _ptr(kv_out), _ref(pool), _ref(outputs), _ptr(ws),
                          int(ws_bytes), _stream(stream)), "dfkv_step")


def dfkv_step_noalloc(geom, weights, hidden, hidden_row_stride, requests, cos_sin, cache_len, kv_out, pool, outputs,
                      stream=None) -> None:
    _check(_lib.dfkv_step_noalloc(_ref(geom), _ref(weights), _ptr(hidden), int(hidden_row_stride), _ref(requests),
                                  _ptr(cos_sin), int(cache_len), _ptr(kv_out), _ref(pool), _ref(outputs),
                                  _stream(stream)), "dfkv_step_noalloc")
