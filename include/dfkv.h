/*
 * dfkv.h -- C ABI of libdfkv: the decode-step context-KV update of a
 * DFlash / DSpark block drafter on one MI355X (gfx950) GPU.
 *
 * One step takes the target model's captured hidden states for the K+1
 * verified tokens of every generation request and
 *   1. projects them into every drafter layer's context K/V (or MLA latent):
 *      fc over the concatenated target layers, hidden_norm (RMSNorm), one
 *      GEMM stacked across all drafter layers, per-layer k_norm with stacked
 *      weights and one shared eps, and RoPE read from one cos/sin cache;
 *   2. does the per-request bookkeeping: bonus token, query and context
 *      positions, embedding ids, the rejected-row mask, the clamp to the
 *      request's allocation, the block-table page lookup, the ctx_len advance
 *      with the dummy-slot reset, and seq_lens;
 *   3. writes the accepted rows into every layer's paged pool.
 *
 * Sources (page titles and sections):
 *  [P20550]  TensorRT-LLM PR #20550 "DFlash / MLA DSpark: fuse the decode-step
 *            drafter bookkeeping into Triton kernels": sections
 *            TLLM_DFLASH_FUSED_PROLOGUE, TLLM_DFLASH_OVERLAP_CONTEXT_PROJECTION,
 *            Test Coverage; and the downstream commit quoted on that page
 *            ("per-request bookkeeping ... one kernel stores the context
 *            latents of every drafter layer").
 *  [P13995]  TensorRT-LLM PR #13995 "DFlash performance optimizations":
 *            commits "migrate draft path to per-layer cached K/V pool",
 *            "fuse cross-layer k_norm", "match RoPE between context and query
 *            for YaRN", "fuse query-input build", "drop K-1 filler tokens".
 *  [I20548]  TensorRT-LLM issue #20548 "DFlash / MLA DSpark decode spends
 *            ~0.2 ms per step in small bookkeeping kernels": Description.
 *
 * Conventions for every call
 *  - All tensors are device pointers (hipMalloc'd memory) unless a field
 *    says "host".  bf16 tensors are raw IEEE bfloat16 bit patterns.  The
 *    caller owns every buffer; the library never allocates device memory
 *    and keeps no pointer after a call returns.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream).  No call synchronises the host, allocates, or reads
 *    the environment, so every call may be captured into a hipGraph; a
 *    captured graph keeps the pointers and sizes of capture time.
 *  - Host-side validation runs before any launch.  On any status other than
 *    DFKV_OK nothing was launched and no device memory was touched, except
 *    DFKV_ERR_HIP, which reports a launch failure.
 *  - Bad device *values* (a negative or out-of-range page, n_acc > W, a
 *    position past the block table or the allocation) are not errors: the
 *    write predicate of dfkv_paged_store turns them into "no write", and no
 *    access goes out of bounds.
 *  - Row n of a step is token i = n % W of request r = n / W, with
 *    W = geom.width = K+1 (uniform verify width, [P13995] "drop K-1 filler
 *    tokens"; strict acceptance of a uniform-width draft, [P20550]
 *    downstream commit).
 */
#ifndef DFKV_H
#define DFKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *dfkv_stream_t; /* a hipStream_t */

typedef enum dfkv_status {
    DFKV_OK = 0,
    DFKV_ERR_NULL = -1,      /* a required pointer is NULL */
    DFKV_ERR_SHAPE = -2,     /* unsupported or inconsistent sizes */
    DFKV_ERR_LAYOUT = -3,    /* misaligned pointer, too-small stride, bad pool strides */
    DFKV_ERR_ALIAS = -4,     /* an output overlaps an input it must not overlap */
    DFKV_ERR_WORKSPACE = -5, /* workspace too small */
    DFKV_ERR_HIP = -6        /* a kernel launch failed */
} dfkv_status;

enum { DFKV_GQA = 0, DFKV_MLA = 1 };
enum { DFKV_MAX_LAYERS = 32 };

/* dfkv_project flags (DFKV_FORK_RECORDED: dfkv_project_fork only) */
enum { DFKV_FUSE_NORM_ROPE = 1u, DFKV_FORK_RECORDED = 2u };

/* Geometry of the drafter and of the step.
 *  GQA: each layer's stacked projection row is [2][n_kv_heads][head_dim]
 *       (index 0 = K, 1 = V); rope_dim must equal head_dim (full rotation);
 *       head_dim in {64, 128, 256}.
 *  MLA: each layer's row is [latent_dim + rope_dim]; n_kv_heads = 1,
 *       head_dim = 0; latent_dim and latent_dim + rope_dim multiples of 64,
 *       rope_dim even and <= 128 ([P20550] single-latent pool geometry
 *       shared by all layers).
 *  n_tgt * tgt_hidden and hidden: multiples of 128.
 *  eps: one eps for hidden_norm and the k/latent norm ([P13995] "fuse
 *  cross-layer k_norm": all layers share one variance epsilon). */
typedef struct dfkv_geom {
    int32_t kind;
    int32_t n_tgt;
    int32_t tgt_hidden;
    int32_t hidden;
    int32_t n_layers;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t latent_dim;
    int32_t rope_dim;
    float eps;
    int32_t page_size;
    int32_t width;      /* W = K+1 verify rows per request */
    int32_t block_size; /* drafter block: query length of the next draft block */
} dfkv_geom;

/* Drafter weights, nn.Linear layout [out][in] row-major, bf16, 16-byte aligned.
 *  w_fc    [hidden][n_tgt * tgt_hidden]
 *  w_hnorm [hidden]
 *  w_kv    [n_layers * per_layer][hidden]  (per_layer = 2*nkv*hd or R+P)
 *  w_knorm [n_layers][head_dim] (GQA k_norm) or [n_layers][latent_dim] (MLA)
 *  w_fc_packed  NULL, or the copy of w_fc that dfkv_pack_fc_weight wrote (same
 *          size, 16-byte aligned): above 64 rows the fc GEMM then reads it
 *          instead of w_fc, with the same result bit for bit (only the order of
 *          its bytes in memory differs).  w_fc itself is still required: at
 *          64 rows or fewer the fc streams w_fc (or w_fc_stream).
 *  w_fc_stream, w_kv_stream  NULL, or the copies of w_fc and w_kv that
 *          dfkv_pack_stream_weight wrote (same sizes, 16-byte aligned): at 64
 *          rows or fewer the weight-streaming GEMMs then read them instead of
 *          w_fc and w_kv, with the same result bit for bit.  Either may be given
 *          without the other. */
typedef struct dfkv_weights {
    const void *w_fc;
    const void *w_hnorm;
    const void *w_kv;
    const void *w_knorm;
    const void *w_fc_packed;
    const void *w_fc_stream;
    const void *w_kv_stream;
} dfkv_weights;

/* Request state of one step (all device arrays).
 *  ctx_len_in   [B] int32  context length before the step
 *  n_acc        [B] int32  accepted rows this step (a prefix of the W rows)
 *  alloc_limit  [B] int32  tokens the request may hold (pages allocated * page_size,
 *                          with any max_ctx ceiling folded in by the caller)
 *  is_dummy     [B] uint8  padded dummy slot: no writes, ctx_len reset to 0
 *  row_valid    [B*W] uint8 or NULL: extra per-row rejection mask
 *  block_table  element (r, j) at r*bt_row_stride + j, j < bt_cols (int32 page ids)
 *  accepted_tokens element (r, t) at r*acc_stride_req + t*acc_stride_tok (int32;
 *                  any strided view, e.g. a transposed [W][B] tensor)
 *  mask_token_id   id of the drafter's mask token */
typedef struct dfkv_requests {
    int32_t n_reqs;
    const int32_t *ctx_len_in;
    const int32_t *n_acc;
    const int32_t *alloc_limit;
    const uint8_t *is_dummy;
    const uint8_t *row_valid;
    const int32_t *block_table;
    int64_t bt_row_stride;
    int32_t bt_cols;
    const int32_t *accepted_tokens;
    int64_t acc_stride_req;
    int64_t acc_stride_tok;
    int32_t mask_token_id;
} dfkv_requests;

/* Per-layer paged pools (bf16).  k[l], v[l]: device base pointers, 16-byte
 * aligned (MLA: k[l] is the latent pool, v unused).  Element (page, off, head, e)
 * of a GQA pool is at page*stride_page + off*stride_slot + head*stride_head + e;
 * a token's MLA latent row (R+P elements) is at page*stride_page + off*stride_slot.
 * Strides in elements, multiples of 8; e is contiguous.  Both the
 * [page][slot][head][dim] and the [page][head][slot][dim] layouts are expressible. */
typedef struct dfkv_pool {
    void *k[DFKV_MAX_LAYERS];
    void *v[DFKV_MAX_LAYERS];
    int64_t stride_page;
    int64_t stride_slot;
    int64_t stride_head;
    int32_t num_pages;
} dfkv_pool;

/* Bookkeeping outputs (device arrays; none may overlap an input).
 *  slot        [B*W] int64  page*page_size + offset of each written row, -1 if none
 *  write_mask  [B*W] uint8  1 iff the row was written into the pools
 *  c_pos       [B*W] int32  context / RoPE position ctx_len_in + i
 *  bonus       [B]   int32  last accepted token, accepted[r][clamp(n_acc,1,W)-1]
 *  emb_ids     [B*block_size] int32  [bonus, mask_token_id x (block_size-1)]
 *  q_pos       [B*block_size] int32  ctx_len_out + j
 *  ctx_len_out [B]   int32  dummy ? 0 : min(ctx_len_in + n_acc, alloc_limit)
 *                           (also the advertised context length)
 *  seq_len     [B]   int32  ctx_len_out + block_size
 *  block_slot  [B*block_size] int64 or NULL: placement of the next draft block's
 *                           own positions q_pos in the pages ([P20550] downstream
 *                           commit: the bookkeeping kernel places the block, which
 *                           the drafter's block decode takes instead of gathering
 *                           the page table again): page*page_size + offset of
 *                           position q = q_pos[r][j], -1 when the request is a
 *                           dummy, q >= alloc_limit, q/page_size >= bt_cols or the
 *                           page is outside [0, num_pages).  Written by
 *                           dfkv_store_advance and dfkv_step (which know the pool's
 *                           page count); dfkv_advance requires it NULL. */
typedef struct dfkv_outputs {
    int64_t *slot;
    uint8_t *write_mask;
    int32_t *c_pos;
    int32_t *bonus;
    int32_t *emb_ids;
    int32_t *q_pos;
    int32_t *ctx_len_out;
    int32_t *seq_len;
    int64_t *block_slot;
} dfkv_outputs;

/* RoPE parameters.  yarn = 0: plain RoPE (RoFormer), inverse frequencies
 * theta^(-2i/rot).  yarn = 1: YaRN "NTK-by-parts" in the HF formulation
 * (correction range from beta_fast / beta_slow over orig_ctx, floor/ceil
 * only if truncate, linear ramp blending inv and inv/factor, attention factor
 * 0.1*ln(factor)+1 applied to cos and sin).  [P13995] "match RoPE between
 * context and query for YaRN": context K and query K must read one cache. */
typedef struct dfkv_rope {
    double theta;
    int32_t rot;
    int32_t yarn;
    double factor;
    double orig_ctx;
    double beta_fast;
    double beta_slow;
    int32_t truncate;
} dfkv_rope;

/* Human-readable name of a status. */
const char *dfkv_status_string(dfkv_status s);

/* Library version string (static storage). */
const char *dfkv_version(void);

/* After a call returned DFKV_ERR_HIP: the HIP runtime's description of the
 * failed launch (per host thread; static storage). */
const char *dfkv_hip_error_string(void);

/* Bytes of workspace dfkv_project / dfkv_step need for n_reqs requests
 * (f and its row statistics, split-K partials, the K/V stage's bookkeeping
 * hand-off).  Writes *bytes.
 * Errors: NULL if g or bytes is NULL; SHAPE for an unsupported geometry. */
dfkv_status dfkv_workspace_size(const dfkv_geom *g, int32_t n_reqs, size_t *bytes);

/* Zero-fill a workspace with a kernel (not a memset, so it may sit in a captured
 * graph).  Optional: the workspace carries no state from one call to the next
 * (it holds the call's intermediates: f and its statistics, the K/V GEMM's
 * partial sums), so one workspace sized for the largest batch serves every batch
 * size.  Two calls that share one workspace must not run concurrently.
 * Errors: NULL; LAYOUT (not 16-byte aligned); HIP. */
dfkv_status dfkv_workspace_init(void *ws, size_t ws_bytes, dfkv_stream_t stream);

/* Build the one cos/sin cache that context K (this library) and query K (the
 * drafter) both read.  cos_sin: device float [cache_len][rot]; row p holds
 * m*cos(p*inv_i) for i < rot/2, then m*sin(p*inv_i).  Angles and values are
 * computed in fp64 on the GPU and stored as fp32 (an fp32 angle at position
 * 4e5 would be off by several hundredths of a radian).  [P13995] "match RoPE
 * between context and query for YaRN".
 * Errors: NULL; SHAPE (rot odd or <= 0, cache_len <= 0, factor <= 0 under
 * YaRN, theta <= 1); LAYOUT (cos_sin not 4-byte aligned); HIP. */
dfkv_status dfkv_rope_cache_build(const dfkv_rope *rope, float *cos_sin, int32_t cache_len,
                                  dfkv_stream_t stream);

/* Write w_fc (bf16 [hidden][n_tgt * tgt_hidden], 16-byte aligned) in the order
 * the large-batch fc GEMM reads it: element (o, k) goes to bf16 index
 *   ((((o/64) * (K/64) + k/64) * 4 + s) * 2 + (o/32)%2) * 512 + (o%32 + 32*h) * 8 + e,
 * K = n_tgt*tgt_hidden, k%64 = 32*h + 8*s + e (h < 2, s < 4, e < 8): the fragments
 * the 64 lanes of one wave load for one MFMA step sit in 1 KB in a row.  Done once
 * per weight (weights are static); put the result in dfkv_weights.w_fc_packed.
 * A memory layout of this library for the MI355X matrix cores, not an operation
 * of the method: the GEMM's arithmetic is unchanged.
 * For callers that keep one copy of w_fc: the large-batch path only needs the
 * packed copy, the small-batch path (<= 64 rows) only the row-major one.
 *  w_fc_packed: device memory of hidden*K*2 bytes, 16-byte aligned; must not
 *               overlap w_fc.
 * Errors: NULL; SHAPE (geometry); LAYOUT (alignment); ALIAS; HIP. */
dfkv_status dfkv_pack_fc_weight(const dfkv_geom *g, const void *w_fc, void *w_fc_packed, dfkv_stream_t stream);

/* Write a weight w (bf16 [rows][cols] row-major, 16-byte aligned: w_fc with
 * rows = hidden, cols = n_tgt*tgt_hidden, or w_kv with rows = n_layers*per_layer,
 * cols = hidden) in the order the weight-streaming GEMMs of <= 64 rows read it.
 * With kb = k/128, j = kb/8, width = min(8, cols/128 - 8*j), element (o, k)
 * goes to bf16 index
 *   (j*8*(rows/16) + (o/16)*width + kb%8) * 2048
 *     + ((k%128)/32 * 64 + (k%32)/8 * 16 + o%16) * 8 + k%8.
 * A block of 16 rows x 128 columns is 4 KB in a row and each 1 KB of it is what
 * the 64 lanes of a wave load in one instruction; the (up to) 8 blocks of one
 * row group and 1024-column range sit next to each other (the 8 waves of a
 * workgroup, which owns 16 rows, read them at the same time), and those runs of
 * all row groups follow each other, so the workgroups together sweep the
 * weight front to back.  Done once per weight (weights are
 * static); put the result in dfkv_weights.w_fc_stream or w_kv_stream.  A memory
 * layout of this library, not an operation of the method: the GEMMs'
 * arithmetic is unchanged.
 *  rows: a positive multiple of 16; cols: a positive multiple of 128.
 *  w_stream: device memory of rows*cols*2 bytes, 16-byte aligned; must not
 *            overlap w.
 * Errors: NULL; SHAPE (rows or cols); LAYOUT (alignment); ALIAS; HIP. */
dfkv_status dfkv_pack_stream_weight(int64_t rows, int64_t cols, const void *w, void *w_stream,
                                    dfkv_stream_t stream);

/* Context projection of all N = n_reqs*W rows ([P20550]
 * TLLM_DFLASH_OVERLAP_CONTEXT_PROJECTION: fc + hidden_norm + latent GEMM +
 * RMSNorm/RoPE; [P13995] one GEMM stacked across drafter layers).
 *   f  = bf16(hidden . w_fc^T)                         [N][hidden]
 *   g  = bf16(w_hnorm * f / sqrt(mean(f^2) + eps))      (hidden_norm)
 *   y  = bf16(g . w_kv^T)                               [N][O]
 * With DFKV_FUSE_NORM_ROPE, kv_out = y with k_norm and RoPE applied as in
 * dfkv_norm_rope; without it, kv_out = y.
 * Reads only hidden, the weights, cos_sin and the pre-step ctx_len_in (never
 * n_acc), so it may run on a side stream overlapped with sample/accept.
 *  hidden: bf16, row n at n*hidden_row_stride, first n_tgt*tgt_hidden
 *          elements used; rows 16-byte aligned.
 *  kv_out: bf16 [N][O] contiguous, 16-byte aligned; must not overlap hidden,
 *          the weights, cos_sin or ws.
 *  ctx_len_in, cos_sin/cache_len, w->w_knorm: needed only with
 *          DFKV_FUSE_NORM_ROPE; without it they may be NULL / 0 and are not
 *          read.
 *  ws: >= dfkv_workspace_size bytes of device memory.
 * Errors: NULL, SHAPE, LAYOUT, ALIAS, WORKSPACE, HIP. */
dfkv_status dfkv_project(const dfkv_geom *g, const dfkv_weights *w, const void *hidden,
                         int64_t hidden_row_stride, int32_t n_reqs, const int32_t *ctx_len_in,
                         const float *cos_sin, int32_t cache_len, void *kv_out, uint32_t flags,
                         void *ws, size_t ws_bytes, dfkv_stream_t stream);

/* The two stages of dfkv_project, for callers that want to place them apart
 * (dfkv_project == dfkv_project_fc then dfkv_project_kv on the same stream and
 * workspace).
 * dfkv_project_fc: f = bf16(hidden . w_fc^T) and what hidden_norm needs of it
 *   (its row statistics and w_hnorm-weighted copy, or the normalised rows) into
 *   ws.  Reads hidden, w_fc (or w_fc_packed / w_fc_stream) and w_hnorm only.
 * dfkv_project_kv: from what dfkv_project_fc left in ws (same geometry and
 *   n_reqs): hidden_norm, the stacked GEMM and, with DFKV_FUSE_NORM_ROPE,
 *   k_norm + RoPE into kv_out.
 * Arguments, layouts and errors as dfkv_project. */
dfkv_status dfkv_project_fc(const dfkv_geom *g, const dfkv_weights *w, const void *hidden,
                            int64_t hidden_row_stride, int32_t n_reqs, void *ws, size_t ws_bytes,
                            dfkv_stream_t stream);
dfkv_status dfkv_project_kv(const dfkv_geom *g, const dfkv_weights *w, int32_t n_reqs, const int32_t *ctx_len_in,
                            const float *cos_sin, int32_t cache_len, void *kv_out, uint32_t flags, void *ws,
                            size_t ws_bytes, dfkv_stream_t stream);

/* k_norm (or latent norm) and RoPE in place on a stacked projection y.
 * GQA, every K head (l, h) of every row: u = bf16(w_knorm[l] * y / sqrt(mean(y^2)+eps)),
 * then NeoX half-split rotation at pos = ctx_len_in[r] + i from cache row
 * min(max(pos,0), cache_len-1):  k[j] = bf16(u[j]c_j - u[j+h]s_j),
 * k[j+h] = bf16(u[j+h]c_j + u[j]s_j), h = rot/2.  V heads are untouched.
 * MLA, every layer: the latent_dim part is RMSNorm'ed with w_knorm[l], the
 * rope_dim part is rotated (no norm).  ([P13995] "fuse cross-layer k_norm":
 * one RMSNorm over [N, L, nkv, hd] times the stacked weights; "match RoPE
 * between context and query for YaRN".)
 *  kv: bf16 [N][O] contiguous, 16-byte aligned.
 * Errors: NULL, SHAPE, LAYOUT, ALIAS (kv overlapping cos_sin or w_knorm), HIP. */
dfkv_status dfkv_norm_rope(const dfkv_geom *g, const void *w_knorm, int32_t n_reqs,
                           const int32_t *ctx_len_in, const float *cos_sin, int32_t cache_len,
                           void *kv, dfkv_stream_t stream);

/* Paged store of the gen tokens' context K/V ([P20550] TLLM_DFLASH_FUSED_PROLOGUE:
 * rejected-row mask, clamp to the request's allocation, page lookup, write to
 * every layer; downstream commit: pool entries outside the step's destinations
 * stay unchanged, every destination is written).  For row n (request r, token i),
 * pos = ctx_len_in[r] + i, the row is written iff
 *   !is_dummy[r] && i < n_acc[r] && (row_valid == NULL || row_valid[n])
 *   && 0 <= pos < alloc_limit[r] && pos/page_size < bt_cols
 *   && 0 <= page < num_pages, page = block_table[r][pos/page_size];
 * then every layer l receives the row's layer-l K and V (GQA) or latent (MLA)
 * at (page, pos % page_size).  slot_out/write_mask_out as in dfkv_outputs.
 *  kv: bf16 [N][O] (the output of dfkv_project with DFKV_FUSE_NORM_ROPE).
 * Errors: NULL, SHAPE, LAYOUT (pool alignment/strides), ALIAS (outputs over
 * inputs or pools), HIP. */
dfkv_status dfkv_paged_store(const dfkv_geom *g, const void *kv, const dfkv_requests *req,
                             const dfkv_pool *pool, int64_t *slot_out, uint8_t *write_mask_out,
                             dfkv_stream_t stream);

/* Row-wise paged store of prefill-shaped (ragged) context ([P20550]: the
 * single-latent context scatter, here at any per-request row count): row n of
 * kv ([n_rows][O] bf16, as dfkv_project writes it) belongs to request
 * row_req[n] at position row_pos[n].  It is written into every layer's pool
 * (same layout rules as dfkv_paged_store) when 0 <= r < n_reqs,
 * 0 <= pos < alloc_limit[r], pos/page_size < bt_cols and 0 <= page < num_pages
 * with page = block_table[r*bt_row_stride + pos/page_size]; slot_out[n] =
 * page*page_size + pos%page_size or -1, write_mask_out[n] = 1 iff written.
 * Every other pool byte is unchanged.  The rows' projection is dfkv_project
 * with geom.width = 1 and ctx_len_in = row_pos (each row its own RoPE
 * position).  A dense per-slot buffer [max_batch][L][T][nkv][hd] is this pool
 * with page_size = T, one page per request (its batch slot) and stride_page =
 * L*T*nkv*hd, k[l] = buffer + l*T*nkv*hd.
 * Errors: NULL, SHAPE, LAYOUT (pool, table stride), ALIAS (outputs over inputs
 * or pools, kv over a pool), HIP. */
dfkv_status dfkv_paged_store_rows(const dfkv_geom *g, const void *kv, int32_t n_rows, const int32_t *row_req,
                                  const int32_t *row_pos, int32_t n_reqs, const int32_t *alloc_limit,
                                  const int32_t *block_table, int64_t bt_row_stride, int32_t bt_cols,
                                  const dfkv_pool *pool, int64_t *slot_out, uint8_t *write_mask_out,
                                  dfkv_stream_t stream);

/* Per-request advance ([P20550] TLLM_DFLASH_FUSED_PROLOGUE: bonus token, query
 * and context positions, embedding ids, ctx_len advance with the clamp and the
 * dummy-slot reset, advertised context length; downstream commit: seq_lens;
 * [P13995] "fuse query-input build": positions by broadcast-add, embedding ids
 * [bonus, mask...]).  Writes out->c_pos, bonus, emb_ids, q_pos, ctx_len_out,
 * seq_len (slot and write_mask are ignored and may be NULL; block_slot must be
 * NULL: placing the block needs the pool's page count, see dfkv_store_advance).
 * ctx_len_out must not overlap ctx_len_in (no in-place advance).
 * Errors: NULL, SHAPE (also a non-NULL block_slot), ALIAS, HIP. */
dfkv_status dfkv_advance(const dfkv_geom *g, const dfkv_requests *req, const dfkv_outputs *out,
                         dfkv_stream_t stream);

/* dfkv_paged_store and dfkv_advance in one coalesced launch; writes every
 * field of *out (block_slot when it is not NULL: the block placement).
 * Errors as the two calls. */
dfkv_status dfkv_store_advance(const dfkv_geom *g, const void *kv, const dfkv_requests *req,
                               const dfkv_pool *pool, const dfkv_outputs *out, dfkv_stream_t stream);

/* Strict acceptance of a uniform-width draft ([P20550] downstream commit:
 * strict acceptance of a uniform-width draft is one launch; ragged
 * verification keeps its path).  Request r verified W = width = K+1 tokens:
 * target element (r, i), i < W, at r*t_stride_req + i*t_stride_tok is the
 * target's token at verify position i; draft element (r, i), i < K, at
 * r*d_stride_req + i*d_stride_tok is the i-th drafted token (any strided
 * views; int32).  The draft is accepted up to its first mismatch and the
 * target's token after it is the bonus:
 *   n_acc[r]          = 1 + max{ m <= K : draft(r, i) == target(r, i), i < m }
 *   accepted[r*W + i] = target(r, i)   (the first n_acc[r] are the accepted ones)
 * n_acc and accepted feed dfkv_requests (acc_stride_req = W, acc_stride_tok = 1).
 * Errors: NULL; SHAPE (n_reqs < 0, width < 1); LAYOUT (negative strides);
 * ALIAS (outputs overlapping each other or the inputs); HIP. */
dfkv_status dfkv_strict_accept(const int32_t *target, int64_t t_stride_req, int64_t t_stride_tok,
                               const int32_t *draft, int64_t d_stride_req, int64_t d_stride_tok,
                               int32_t n_reqs, int32_t width, int32_t *n_acc_out, int32_t *accepted_out,
                               dfkv_stream_t stream);

/* Draft-KV block-table decode ([P20550]: the refresh of the draft block table,
 * "page counts and decoded table"; downstream commit: the decode of blocks per
 * request with clamped and divided offsets is one launch).  Request r holds
 * n_tokens[r] tokens of draft context; offsets element (r, b) is at
 * r*off_stride_req + b*off_stride_blk (any strided view, e.g. a transposed
 * tensor; int32, counting in units of 1/divisor page, negative = no page).
 *   page_count[r] = clamp(ceil(n_tokens[r] / page_size), 0, max_blocks)
 *   table[r][b]   = b < page_count[r] && offsets(r, b) >= 0
 *                   ? offsets(r, b) / divisor : -1       (b < max_blocks)
 * table row r starts at table_out + r*table_row_stride (int32); the result is
 * a block table for dfkv_requests (bt_row_stride = table_row_stride,
 * bt_cols = max_blocks).  One launch; no value is read out of bounds.
 * Errors: NULL; SHAPE (n_reqs, max_blocks < 0; page_size, divisor <= 0);
 * LAYOUT (negative offset strides, table_row_stride < max_blocks); ALIAS
 * (outputs overlapping each other or the inputs); HIP. */
dfkv_status dfkv_block_table_decode(const int32_t *offsets, int64_t off_stride_req, int64_t off_stride_blk,
                                    int32_t n_reqs, int32_t max_blocks, const int32_t *n_tokens,
                                    int32_t page_size, int32_t divisor, int32_t *page_count_out,
                                    int32_t *table_out, int64_t table_row_stride, dfkv_stream_t stream);

/* Overlapped context projection ([P20550] TLLM_DFLASH_OVERLAP_CONTEXT_PROJECTION:
 * the gen tokens' context projection forks onto an aux stream ahead of
 * sample/accept).  dfkv_project_fork validates exactly as dfkv_project, then
 * records `fork` on `main` (so that everything already queued on main -- the
 * target forward that produced `hidden` -- comes first), makes `aux` wait for
 * it, queues the projection on `aux` and records `join` on `aux`.  The
 * projection reads only the hidden states, the weights, the cos/sin cache and
 * the pre-step ctx_len_in (never n_acc), so sample/accept may run on `main`
 * meanwhile.  dfkv_join makes `main` wait for `join`: call it before anything
 * on `main` reads kv_out or the workspace (dfkv_store_advance).  Streams and
 * events (hipStream_t, hipEvent_t) are the caller's; both calls may be
 * captured into one hipGraph together with the work on `main`.
 * With DFKV_FORK_RECORDED in `flags` the caller has already recorded `fork` on
 * `main` at the fork point, and the call only makes `aux` wait for it (`main`
 * is not used).  The caller may then queue sample/accept on `main` before this
 * call, so that in a captured graph the main-stream work comes first in
 * capture order: HIP's graph launch keeps such a graph's first branch, here
 * the sample/accept work, on one hardware queue, and the later work on `main`
 * (the store) follows it there instead of the projection, which saves a
 * cross-queue hand-off per step.
 * Errors: as dfkv_project (nothing queued, no event recorded); NULL for a NULL
 * event; HIP when recording or waiting fails. */
dfkv_status dfkv_project_fork(const dfkv_geom *g, const dfkv_weights *w, const void *hidden,
                              int64_t hidden_row_stride, int32_t n_reqs, const int32_t *ctx_len_in,
                              const float *cos_sin, int32_t cache_len, void *kv_out, uint32_t flags,
                              void *ws, size_t ws_bytes, dfkv_stream_t main, dfkv_stream_t aux,
                              void *fork, void *join);
dfkv_status dfkv_join(dfkv_stream_t main, void *join);

/* One whole step: dfkv_project(DFKV_FUSE_NORM_ROPE) into kv_out, then
 * dfkv_store_advance.  ctx_len_in is taken from req.  Errors as the parts. */
dfkv_status dfkv_step(const dfkv_geom *g, const dfkv_weights *w, const void *hidden,
                      int64_t hidden_row_stride, const dfkv_requests *req, const float *cos_sin,
                      int32_t cache_len, void *kv_out, const dfkv_pool *pool, const dfkv_outputs *out,
                      void *ws, size_t ws_bytes, dfkv_stream_t stream);

/* dfkv_step for callers that cannot allocate (code under graph capture, tight
 * serving loops, harnesses that forbid allocation): the same arguments, kernels
 * and results, without ws/ws_bytes -- the workspace is a static device array of
 * DFKV_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends (its address is looked up once per device, on the
 * first call there).  Allocates nothing.  The array carries nothing that a
 * call reads from one call to the next.  Every call on one GPU shares that
 * GPU's array: two calls that overlap on one GPU (on different streams, or
 * concurrently from several host threads) race and must not be issued.
 * Errors as dfkv_step; WORKSPACE when the call's workspace
 * (dfkv_workspace_size) exceeds DFKV_NOALLOC_SCRATCH_BYTES -- every plan of up
 * to 64 rows of the workloads' drafters fits; HIP when the array's address
 * cannot be obtained. */
enum { DFKV_NOALLOC_SCRATCH_BYTES = 8 << 20 };
dfkv_status dfkv_step_noalloc(const dfkv_geom *g, const dfkv_weights *w, const void *hidden,
                              int64_t hidden_row_stride, const dfkv_requests *req, const float *cos_sin,
                              int32_t cache_len, void *kv_out, const dfkv_pool *pool, const dfkv_outputs *out,
                              dfkv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DFKV_H */
