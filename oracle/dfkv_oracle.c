/*
 * dfkv_oracle.c -- plain, slow CPU oracle for the decode-step context-KV
 * update of a DFlash / DSpark block drafter.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the HIP library; the two are written independently
 * from the pages and meet only in the tests.
 *
 * Arithmetic: every dot product and every norm accumulates in fp64.  Results
 * are rounded to bf16 (nearest, ties to even) exactly at the stage
 * boundaries that the drafter's torch path materialises: after fc, after
 * hidden_norm, after the stacked K/V GEMM, after k_norm and after RoPE.
 *
 * Sources (page titles and sections; see the tests for the pins):
 *  - fc + hidden_norm + latent GEMM + RMSNorm/RoPE as the gen tokens'
 *    context projection: TensorRT-LLM PR #20550 "fuse the decode-step drafter
 *    bookkeeping into Triton kernels", section TLLM_DFLASH_OVERLAP_CONTEXT_
 *    PROJECTION.
 *  - One GEMM stacked across drafter layers on the K+1 accepted tokens, then a
 *    per-layer scatter: TensorRT-LLM PR #13995 "DFlash performance
 *    optimizations", commit "migrate draft path to per-layer cached K/V pool".
 *  - k_norm as one RMSNorm over [N, L, nkv, hd] times stacked per-layer
 *    weights with one shared eps: PR #13995, commit "fuse cross-layer k_norm".
 *  - Context K and query K rotate from one cos/sin cache (HF YaRN formulation,
 *    truncate=false honoured): PR #13995, commit "match RoPE between context
 *    and query for YaRN".
 *  - Rejected-row mask, clamp to the allocation, page lookup, write to every
 *    layer, ctx_len advance with clamp and dummy reset, advertised context
 *    length: PR #20550, section TLLM_DFLASH_FUSED_PROLOGUE, and the
 *    downstream commit quoted on that page (per-request bookkeeping: bonus
 *    token, query/RoPE positions, destination pages/offsets/write mask,
 *    seq_lens; pool entries outside the destinations unchanged).
 *
 * Parity pins: every function below is pinned by a CPU test (closed forms,
 * brute force, library special cases, planted mutants).  The rounding order
 * inside the projection beyond the bf16 tolerance is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef DFKV_ORACLE_MUTANT
#define DFKV_ORACLE_MUTANT 0 /* >0 only in the test suite's planted-mistake builds */
#endif

#define EXPORT __attribute__((visibility("default")))

#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the oracle's parallel loops use (1 without OpenMP). */
EXPORT int dfkv_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp64                                                             */
/* ------------------------------------------------------------------------ */

EXPORT double dfkv_oracle_bf16_to_f64(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round an fp64 value to the nearest bf16 (ties to even), by definition:
 * bf16 has 8 significant bits and the fp32 exponent range, so the spacing of
 * representable values around |x| in [2^e, 2^(e+1)) is 2^(e-7), and below
 * 2^-126 (subnormal) it is 2^-133.  rint() rounds half to even in the default
 * floating-point environment. */
EXPORT uint16_t dfkv_oracle_f64_to_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    double ax = fabs(x);
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isinf(x))
        return sign | 0x7F80;
    if (ax == 0.0)
        return sign;
    int e;
    frexp(ax, &e);              /* ax = m * 2^e, m in [0.5, 1): leading bit is 2^(e-1) */
    int lead = e - 1;
    if (lead < -126)
        lead = -126;            /* subnormal range keeps the 2^-133 spacing */
    double q = ldexp(1.0, lead - 7);
    double r = rint(ax / q) * q;
    if (r >= ldexp(1.0, 128))   /* rounds past the largest finite bf16 */
        return sign | 0x7F80;
    float rf = (float)r;        /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

#define B2D(h) dfkv_oracle_bf16_to_f64(h)
#define D2B(x) dfkv_oracle_f64_to_bf16(x)

/* ------------------------------------------------------------------------ */
/* Linear layer without bias: y[n][j] = bf16( sum_k x[n][k] * w[j][k] )      */
/* w is an nn.Linear weight, [out, in] row-major.                           */
/* ------------------------------------------------------------------------ */

EXPORT void dfkv_oracle_linear(int n_rows, int k_in, int n_out,
                               const uint16_t *x, int64_t ldx,
                               const uint16_t *w,
                               uint16_t *y, int64_t ldy)
{
#pragma omp parallel for schedule(static)
    for (int j = 0; j < n_out; ++j) {
        for (int n = 0; n < n_rows; ++n) {
            double acc = 0.0;
            for (int k = 0; k < k_in; ++k) {
#if DFKV_ORACLE_MUTANT == 5 /* planted: transposed weight index */
                acc += B2D(x[(int64_t)n * ldx + k]) * B2D(w[(int64_t)k * n_out + j]);
#else
                acc += B2D(x[(int64_t)n * ldx + k]) * B2D(w[(int64_t)j * k_in + k]);
#endif
            }
            y[(int64_t)n * ldy + j] = D2B(acc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* RMSNorm with weight: y = bf16( w * x / sqrt(mean(x^2) + eps) )            */
/* ------------------------------------------------------------------------ */

EXPORT void dfkv_oracle_rmsnorm(int n_rows, int dim, const uint16_t *x, int64_t ldx,
                                const uint16_t *w, double eps, uint16_t *y, int64_t ldy)
{
    for (int n = 0; n < n_rows; ++n) {
        const uint16_t *xr = x + (int64_t)n * ldx;
        double ss = 0.0;
        for (int d = 0; d < dim; ++d) {
            double v = B2D(xr[d]);
            ss += v * v;
        }
#if DFKV_ORACLE_MUTANT == 6 /* planted: sum instead of mean */
        double inv = 1.0 / sqrt(ss + eps);
#else
        double inv = 1.0 / sqrt(ss / dim + eps);
#endif
        for (int d = 0; d < dim; ++d)
            y[(int64_t)n * ldy + d] = D2B(B2D(w[d]) * (B2D(xr[d]) * inv));
    }
}

/* ------------------------------------------------------------------------ */
/* cos/sin cache, built in fp64 and stored as fp32:                          */
/*   cs[p][i] = m*cos(p*inv_i), cs[p][rot/2 + i] = m*sin(p*inv_i), i<rot/2   */
/* Plain RoPE (Su et al., RoFormer): inv_i = theta^(-2i/rot), m = 1.         */
/* YaRN "NTK-by-parts" with attention temperature (Peng et al., 2023), in    */
/* the HF formulation: correction dims from beta_fast/beta_slow, floor/ceil  */
/* only when truncate != 0, a linear ramp between them blending the original */
/* inverse frequency (below lo) with the one divided by factor (above hi),   */
/* and m = 0.1*ln(factor) + 1.                                               */
/* ------------------------------------------------------------------------ */

static double yarn_correction_dim(double n_rot, int rot, double theta, double orig_ctx)
{
    /* the dim index whose wavelength completes n_rot turns over orig_ctx positions */
    return (rot * log(orig_ctx / (n_rot * 2.0 * M_PI))) / (2.0 * log(theta));
}

EXPORT void dfkv_oracle_inv_freq(double theta, int rot, int yarn, double factor, double orig_ctx,
                                 double beta_fast, double beta_slow, int truncate,
                                 double *inv_out, double *mscale_out)
{
    int half = rot / 2;
    for (int i = 0; i < half; ++i)
        inv_out[i] = pow(theta, -(2.0 * i) / rot);
    double m = 1.0;
    if (yarn) {
        double lo = yarn_correction_dim(beta_fast, rot, theta, orig_ctx);
        double hi = yarn_correction_dim(beta_slow, rot, theta, orig_ctx);
        if (truncate) {
            lo = floor(lo);
            hi = ceil(hi);
        }
        if (lo < 0.0)
            lo = 0.0;
        if (hi > rot - 1)
            hi = rot - 1;
        if (lo == hi)
            hi += 0.001;
        for (int i = 0; i < half; ++i) {
            double ramp = (i - lo) / (hi - lo);
            if (ramp < 0.0) ramp = 0.0;
            if (ramp > 1.0) ramp = 1.0;
#if DFKV_ORACLE_MUTANT == 7 /* planted: ramp direction reversed */
            ramp = 1.0 - ramp;
#endif
            inv_out[i] = (inv_out[i] / factor) * ramp + inv_out[i] * (1.0 - ramp);
        }
        if (factor > 1.0)
            m = 0.1 * log(factor) + 1.0;
    }
    *mscale_out = m;
}

EXPORT void dfkv_oracle_rope_cache(double theta, int rot, int yarn, double factor, double orig_ctx,
                                   double beta_fast, double beta_slow, int truncate,
                                   float *cs, int cache_len)
{
    int half = rot / 2;
    double *inv = (double *)malloc(sizeof(double) * (half > 0 ? half : 1));
    double m;
    dfkv_oracle_inv_freq(theta, rot, yarn, factor, orig_ctx, beta_fast, beta_slow, truncate, inv, &m);
#pragma omp parallel for schedule(static)
    for (int p = 0; p < cache_len; ++p) {
        for (int i = 0; i < half; ++i) {
            double a = (double)p * inv[i];
#if DFKV_ORACLE_MUTANT == 12 /* planted: the angle formed in fp32 */
            a = (double)((float)p * (float)inv[i]);
#endif
            cs[(int64_t)p * rot + i] = (float)(cos(a) * m);
            cs[(int64_t)p * rot + half + i] = (float)(sin(a) * m);
        }
    }
    free(inv);
}

/* NeoX (half-split) rotation of one vector u[0..rot) at cache row cs_row:
 *   out[j]       = bf16( u[j]*c_j - u[j+h]*s_j )
 *   out[j+h]     = bf16( u[j+h]*c_j + u[j]*s_j ),   h = rot/2.               */
EXPORT void dfkv_oracle_rope_neox(int rot, const uint16_t *u, const float *cs_row, uint16_t *out)
{
    int h = rot / 2;
    for (int j = 0; j < h; ++j) {
        double c = cs_row[j], s = cs_row[h + j];
        double a = B2D(u[j]), b = B2D(u[j + h]);
#if DFKV_ORACLE_MUTANT == 3 /* planted: the two halves' sin terms swapped */
        out[j] = D2B(a * c + b * s);
        out[j + h] = D2B(b * c - a * s);
#else
        out[j] = D2B(a * c - b * s);
        out[j + h] = D2B(b * c + a * s);
#endif
    }
}

/* ------------------------------------------------------------------------ */
/* k_norm (or latent norm) + RoPE on the stacked projection y, in place.     */
/* Row n is token i = n % W of request r = n / W; its RoPE position is the   */
/* pre-step ctx_len[r] + i, read from cache row min(max(pos,0), cache_len-1).*/
/* GQA view of a row: [L][2][nkv][hd] (index 0 = K, 1 = V); V is untouched. */
/* MLA view of a row: [L][R + P]: RMSNorm on the R latent dims, RoPE (no    */
/* norm) on the P rope dims.                                                 */
/* row_ids (nullable) gives the global row index of each of the n_rows rows. */
/* ------------------------------------------------------------------------ */

EXPORT void dfkv_oracle_norm_rope(int kind, int n_layers, int nkv, int hd, int latent, int rope_dim,
                                  double eps, int W, const int32_t *row_ids, int n_rows,
                                  const int32_t *ctx_len_in, const uint16_t *w_knorm,
                                  const float *cs, int cache_len, uint16_t *y, int64_t ldy)
{
    int per_layer = kind == 0 ? 2 * nkv * hd : latent + rope_dim;
    uint16_t *tmp = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(per_layer + 1));
    for (int t = 0; t < n_rows; ++t) {
        int n = row_ids ? row_ids[t] : t;
        int r = n / W, i = n % W;
        int64_t pos = (int64_t)ctx_len_in[r] + i;
        int64_t p = pos < 0 ? 0 : (pos > cache_len - 1 ? cache_len - 1 : pos);
        const float *cs_row = cs + p * rope_dim;
        uint16_t *row = y + (int64_t)t * ldy;
        for (int l = 0; l < n_layers; ++l) {
            uint16_t *lay = row + (int64_t)l * per_layer;
            if (kind == 0) {
                for (int h = 0; h < nkv; ++h) {
                    uint16_t *kh = lay + h * hd; /* K block comes first in the layer */
                    dfkv_oracle_rmsnorm(1, hd, kh, hd, w_knorm + (int64_t)l * hd, eps, tmp, hd);
                    dfkv_oracle_rope_neox(rope_dim, tmp, cs_row, kh);
                    for (int d = rope_dim; d < hd; ++d)
                        kh[d] = tmp[d];
                }
            } else {
                dfkv_oracle_rmsnorm(1, latent, lay, latent, w_knorm + (int64_t)l * latent, eps, tmp, latent);
                memcpy(lay, tmp, sizeof(uint16_t) * latent);
                dfkv_oracle_rope_neox(rope_dim, lay + latent, cs_row, tmp);
                memcpy(lay + latent, tmp, sizeof(uint16_t) * rope_dim);
            }
        }
    }
    free(tmp);
}

/* ------------------------------------------------------------------------ */
/* The whole projection for a set of rows: fc -> hidden_norm -> stacked      */
/* K/V GEMM -> k_norm + RoPE.  Intermediates f, g (both [n_rows][H]) and y   */
/* ([n_rows][O], before k_norm/RoPE) are returned for stage checks; kv gets  */
/* the final [n_rows][O].                                                    */
/* ------------------------------------------------------------------------ */

EXPORT void dfkv_oracle_project(int kind, int k_in, int H, int n_layers, int nkv, int hd, int latent,
                                int rope_dim, double eps, int W,
                                const uint16_t *x, int64_t ldx, const int32_t *row_ids, int n_rows,
                                const uint16_t *w_fc, const uint16_t *w_hnorm, const uint16_t *w_kv,
                                const uint16_t *w_knorm, const int32_t *ctx_len_in,
                                const float *cs, int cache_len,
                                uint16_t *f, uint16_t *g, uint16_t *y, uint16_t *kv)
{
    int O = n_layers * (kind == 0 ? 2 * nkv * hd : latent + rope_dim);
    dfkv_oracle_linear(n_rows, k_in, H, x, ldx, w_fc, f, H);
    dfkv_oracle_rmsnorm(n_rows, H, f, H, w_hnorm, eps, g, H);
    dfkv_oracle_linear(n_rows, H, O, g, H, w_kv, y, O);
    memcpy(kv, y, sizeof(uint16_t) * (size_t)n_rows * O);
    dfkv_oracle_norm_rope(kind, n_layers, nkv, hd, latent, rope_dim, eps, W, row_ids, n_rows,
                          ctx_len_in, w_knorm, cs, cache_len, kv, O);
}

/* ------------------------------------------------------------------------ */
/* Bookkeeping for request r, token i (row = r*W + i), with c = ctx_len[r],  */
/* n = n_acc[r], lim = alloc_limit[r], d = is_dummy[r]:                      */
/*   pos = c + i                                 (context / RoPE position)   */
/*   w   = !d && i < n && row_valid[row] && 0 <= pos < lim                   */
/*         && pos/pg < bt_cols && 0 <= page < num_pages                      */
/*         with page = block_table[r][pos/pg]                                */
/*   slot = w ? page*pg + pos%pg : -1                                        */
/*   ctx' = d ? 0 : min(c + n, lim)               (advance, clamp, reset)    */
/*   bonus = accepted[r][clamp(n, 1, W) - 1]                                 */
/*   emb_ids[r] = [bonus, mask_id x (bs_blk-1)], q_pos[r][j] = ctx' + j,     */
/*   seq_len[r] = ctx' + bs_blk.                                             */
/* ------------------------------------------------------------------------ */

static int row_writes(int i, int32_t c, int32_t n, int32_t lim, uint8_t d, const uint8_t *row_valid,
                      int row, const int32_t *bt_row, int bt_cols, int pg, int num_pages, int64_t *slot)
{
    int64_t pos = (int64_t)c + i;
    *slot = -1;
    if (d)
        return 0;
    if (!(i < n))
        return 0;
    if (row_valid && !row_valid[row])
        return 0;
#if DFKV_ORACLE_MUTANT == 1 /* planted: off-by-one clamp */
    if (pos < 0 || pos > lim)
        return 0;
#else
    if (pos < 0 || pos >= lim)
        return 0;
#endif
    int64_t pidx = pos / pg;
    if (pidx >= bt_cols)
        return 0;
    int32_t page = bt_row[pidx];
    if (page < 0 || page >= num_pages)
        return 0;
    *slot = (int64_t)page * pg + pos % pg;
    return 1;
}

EXPORT void dfkv_oracle_bookkeeping(int B, int W, int bs_blk, int pg,
                                    const int32_t *ctx_len, const int32_t *n_acc, const int32_t *alloc_limit,
                                    const uint8_t *is_dummy, const uint8_t *row_valid,
                                    const int32_t *bt, int64_t bt_stride, int bt_cols, int num_pages,
                                    const int32_t *acc_tok, int64_t acc_sr, int64_t acc_st, int32_t mask_id,
                                    int64_t *slot_out, uint8_t *write_mask_out, int32_t *c_pos_out,
                                    int32_t *bonus_out, int32_t *emb_ids_out, int32_t *q_pos_out,
                                    int32_t *ctx_len_out, int32_t *seq_len_out)
{
    for (int r = 0; r < B; ++r) {
        int32_t c = ctx_len[r], n = n_acc[r], lim = alloc_limit[r];
        uint8_t d = is_dummy[r];
#if DFKV_ORACLE_MUTANT == 2 /* planted: dummy slots neither skipped nor reset */
        d = 0;
#endif
        for (int i = 0; i < W; ++i) {
            int row = r * W + i;
            int64_t slot;
            int w = row_writes(i, c, n, lim, d, row_valid, row, bt + (int64_t)r * bt_stride, bt_cols, pg,
                               num_pages, &slot);
            slot_out[row] = slot;
            write_mask_out[row] = (uint8_t)w;
            c_pos_out[row] = (int32_t)((int64_t)c + i);
        }
        int64_t adv = (int64_t)c + n;
        int32_t ctx_new = d ? 0 : (int32_t)(adv < lim ? adv : lim);
        int nb = n < 1 ? 1 : (n > W ? W : n);
        int32_t bonus = acc_tok[(int64_t)r * acc_sr + (int64_t)(nb - 1) * acc_st];
        bonus_out[r] = bonus;
        ctx_len_out[r] = ctx_new;
        seq_len_out[r] = ctx_new + bs_blk;
        for (int j = 0; j < bs_blk; ++j) {
            emb_ids_out[(int64_t)r * bs_blk + j] = j == 0 ? bonus : mask_id;
            q_pos_out[(int64_t)r * bs_blk + j] = ctx_new + j;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Block placement (the downstream commit quoted on the PR #20550 page: the  */
/* bookkeeping kernel also places the next draft block's own positions in    */
/* the pages, which the drafter's block decode takes instead of gathering    */
/* the page table again).  For request r and j < bs_blk, with ctx' from the  */
/* advance above:                                                            */
/*   pos = ctx' + j                               (the block's query position) */
/*   v   = !d && 0 <= pos < lim && pos/pg < bt_cols && 0 <= page < num_pages */
/*         with page = block_table[r][pos/pg]                                */
/*   block_slot[r][j] = v ? page*pg + pos%pg : -1                            */
/* ------------------------------------------------------------------------ */

EXPORT void dfkv_oracle_block_placement(int B, int bs_blk, int pg, const int32_t *ctx_new,
                                        const int32_t *alloc_limit, const uint8_t *is_dummy,
                                        const int32_t *bt, int64_t bt_stride, int bt_cols, int num_pages,
                                        int64_t *block_slot_out)
{
    for (int r = 0; r < B; ++r) {
        const int32_t *bt_row = bt + (int64_t)r * bt_stride;
        for (int j = 0; j < bs_blk; ++j) {
            int64_t pos = (int64_t)ctx_new[r] + j;
            int64_t slot = -1;
#if DFKV_ORACLE_MUTANT == 8 /* planted: the block may reach one position past the allocation */
            if (!is_dummy[r] && pos >= 0 && pos <= alloc_limit[r] && pos / pg < bt_cols) {
#else
            if (!is_dummy[r] && pos >= 0 && pos < alloc_limit[r] && pos / pg < bt_cols) {
#endif
                int32_t page = bt_row[pos / pg];
                if (page >= 0 && page < num_pages)
                    slot = (int64_t)page * pg + pos % pg;
            }
            block_slot_out[(int64_t)r * bs_blk + j] = slot;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Draft-KV block-table decode (PR #20550 page: the refresh of the draft      */
/* block table, "page counts and decoded table"; downstream commit: the       */
/* decode of blocks per request with clamped and divided offsets, checked on  */
/* a strided view of the offsets tensor, an all-negative row, an all-zero row */
/* and about half negative or zero entries).  Reading: request r holds        */
/* n_tokens[r] tokens of draft context; offsets[r][b] counts in units of      */
/* 1/divisor page (negative: no page).                                        */
/*   page_count[r] = clamp(ceil(n_tokens[r] / page_size), 0, max_blocks)      */
/*   table[r][b]   = b < page_count[r] && offsets[r][b] >= 0                  */
/*                   ? offsets[r][b] / divisor : -1                           */
/* ------------------------------------------------------------------------ */

EXPORT void dfkv_oracle_block_table_decode(int B, int max_blocks, const int32_t *offsets, int64_t s_req,
                                           int64_t s_blk, const int32_t *n_tokens, int page_size, int divisor,
                                           int32_t *page_count_out, int32_t *table_out, int64_t t_stride)
{
    for (int r = 0; r < B; ++r) {
        int64_t n = n_tokens[r];
        int64_t pages = n <= 0 ? 0 : (n + page_size - 1) / page_size;
#if DFKV_ORACLE_MUTANT == 9 /* planted: pages rounded down */
        pages = n <= 0 ? 0 : n / page_size;
#endif
        if (pages > max_blocks)
            pages = max_blocks;
        page_count_out[r] = (int32_t)pages;
        for (int b = 0; b < max_blocks; ++b) {
            int32_t off = offsets[(int64_t)r * s_req + (int64_t)b * s_blk];
            table_out[(int64_t)r * t_stride + b] = (b < pages && off >= 0) ? off / divisor : -1;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Strict acceptance of a uniform-width draft (the downstream commit quoted  */
/* on the PR #20550 page: strict acceptance of a uniform-width draft is one  */
/* launch; ragged verification keeps its path).  Request r verified W = K+1  */
/* tokens: the target's token at each of the W positions, target[r][i], and  */
/* the K drafted tokens draft[r][i].  The draft is accepted up to its first  */
/* mismatch, and the target's token after the last accepted draft token is   */
/* the bonus:                                                                */
/*   n_acc[r]       = 1 + max{ m <= K : draft[r][i] == target[r][i], i < m } */
/*   accepted[r][i] = target[r][i], i < W   (the first n_acc[r] are valid)   */
/* ------------------------------------------------------------------------ */

EXPORT void dfkv_oracle_strict_accept(int B, int W, const int32_t *target, int64_t t_sr, int64_t t_st,
                                      const int32_t *draft, int64_t d_sr, int64_t d_st, int32_t *n_acc_out,
                                      int32_t *accepted_out)
{
    for (int r = 0; r < B; ++r) {
        int m = 0;
        while (m < W - 1 && draft[(int64_t)r * d_sr + (int64_t)m * d_st] ==
                                target[(int64_t)r * t_sr + (int64_t)m * t_st])
            ++m;
#if DFKV_ORACLE_MUTANT == 10 /* planted: the bonus token not counted */
        n_acc_out[r] = m;
#else
        n_acc_out[r] = 1 + m;
#endif
        for (int i = 0; i < W; ++i)
            accepted_out[(int64_t)r * W + i] = target[(int64_t)r * t_sr + (int64_t)i * t_st];
    }
}

/* ------------------------------------------------------------------------ */
/* Destinations of prefill-shaped (ragged) context rows: the single-latent   */
/* context scatter the PR #20550 page lists among its fused kernels, at any  */
/* per-request row count.  Row n belongs to request r = row_req[n] at        */
/* position pos = row_pos[n]:                                                */
/*   w = 0 <= r < B && 0 <= pos < lim[r] && pos/pg < bt_cols                 */
/*       && 0 <= page < num_pages, page = block_table[r][pos/pg]             */
/*   slot = w ? page*pg + pos%pg : -1                                        */
/* (the rows are then stored by dfkv_oracle_store).                          */
/* ------------------------------------------------------------------------ */

EXPORT void dfkv_oracle_row_slots(int n_rows, const int32_t *row_req, const int32_t *row_pos, int B,
                                  const int32_t *alloc_limit, const int32_t *bt, int64_t bt_stride, int bt_cols,
                                  int pg, int num_pages, int64_t *slot_out, uint8_t *write_mask_out)
{
    for (int n = 0; n < n_rows; ++n) {
        int32_t r = row_req[n];
        int64_t pos = row_pos[n], slot = -1;
        if (r >= 0 && r < B && pos >= 0 && pos < alloc_limit[r] && pos / pg < bt_cols) {
            int32_t page = bt[(int64_t)r * bt_stride + pos / pg];
#if DFKV_ORACLE_MUTANT == 11 /* planted: the page bound off by one */
            if (page >= 0 && page <= num_pages)
#else
            if (page >= 0 && page < num_pages)
#endif
                slot = (int64_t)page * pg + pos % pg;
        }
        slot_out[n] = slot;
        write_mask_out[n] = (uint8_t)(slot >= 0);
    }
}

/* ------------------------------------------------------------------------ */
/* Paged store: every written row goes into every layer's pool.              */
/* GQA: layer l's K pool gets kv[row][l][0][h][:] at                         */
/*      page*s_page + off*s_slot + h*s_head, its V pool kv[row][l][1][h][:]. */
/* MLA: layer l's latent pool gets the whole R+P row slice at                */
/*      page*s_page + off*s_slot.                                            */
/* pools_k / pools_v: host arrays of n_layers pool base pointers (bf16).     */
/* Every other pool element is left as it was.                               */
/* ------------------------------------------------------------------------ */

EXPORT void dfkv_oracle_store(int kind, int n_layers, int nkv, int hd, int latent, int rope_dim, int pg,
                              int n_rows, const uint16_t *kv, const int64_t *slot, const uint8_t *write_mask,
                              uint16_t *const *pools_k, uint16_t *const *pools_v,
                              int64_t s_page, int64_t s_slot, int64_t s_head)
{
    int per_layer = kind == 0 ? 2 * nkv * hd : latent + rope_dim;
    int64_t O = (int64_t)n_layers * per_layer;
    for (int row = 0; row < n_rows; ++row) {
        if (!write_mask[row])
            continue;
        int64_t page = slot[row] / pg, off = slot[row] % pg;
        const uint16_t *src = kv + (int64_t)row * O;
        for (int l = 0; l < n_layers; ++l) {
#if DFKV_ORACLE_MUTANT == 4 /* planted: wrong layer stride into the row */
            const uint16_t *lay = src + (int64_t)l * (per_layer / 2);
#else
            const uint16_t *lay = src + (int64_t)l * per_layer;
#endif
            if (kind == 0) {
                for (int h = 0; h < nkv; ++h) {
                    uint16_t *dk = pools_k[l] + page * s_page + off * s_slot + h * s_head;
                    uint16_t *dv = pools_v[l] + page * s_page + off * s_slot + h * s_head;
                    for (int e = 0; e < hd; ++e) {
                        dk[e] = lay[h * hd + e];
                        dv[e] = lay[nkv * hd + h * hd + e];
                    }
                }
            } else {
                uint16_t *dl = pools_k[l] + page * s_page + off * s_slot;
                for (int e = 0; e < latent + rope_dim; ++e)
                    dl[e] = lay[e];
            }
        }
    }
}
