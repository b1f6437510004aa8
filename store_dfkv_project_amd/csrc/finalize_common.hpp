// finalize_common.hpp -- device code shared by the finalize kernel (k_finalize)
// and the small-batch K/V kernel (k_kvfin): the write predicate and slot of a
// row, the per-request advance, and the k_norm / RoPE arithmetic of one head or
// latent (kept in one place so that both kernels round identically).
//
// Sources (page titles and sections):
//  * TensorRT-LLM PR #20550 "fuse the decode-step drafter bookkeeping into
//    Triton kernels", section TLLM_DFLASH_FUSED_PROLOGUE: rejected-row mask,
//    clamp to the request's allocation, page lookup, write to every layer; the
//    ctx_len advance with the clamp, the dummy-slot reset and the advertised
//    context length; bonus token, query/context positions, embedding ids.  The
//    downstream commit quoted on that page adds seq_lens.
//  * TensorRT-LLM PR #13995 "DFlash performance optimizations": commit "fuse
//    cross-layer k_norm" (one RMSNorm over every K head times stacked per-layer
//    weights, one eps) and commit "match RoPE between context and query for
//    YaRN" (context K rotated from the one cos/sin cache, NeoX half split).
#pragma once

#include "dfkv_internal.hpp"

namespace dfkv {

// Write predicate of token i of a request from the request's fields (pre-step ctx_len c, accepted
// count n, allocation limit lim, dummy flag d) and the row's valid flag rv: true when the row is
// written, with its position pos and block-table column pidx.
__device__ __forceinline__ bool row_write_pred(const FinalizeParams &p, int32_t c, int32_t n, int32_t lim, uint8_t d,
                                               uint8_t rv, int i, int64_t &pos, int64_t &pidx) {
    pos = (int64_t)c + i;
    pidx = 0;
    if (d || !(i < n) || !rv || pos < 0 || pos >= (int64_t)lim) return false;
    pidx = pos / p.pg;
    return pidx < p.bt_cols;
}

// Write predicate and slot of token i of request r (row = r*W + i).  The request's
// fields are loaded together; only the block-table entry depends on them.
__device__ __forceinline__ bool row_destination(const FinalizeParams &p, int r, int i, int row, int64_t &slot) {
    const uint8_t d = p.dummy[r];
    const int32_t n = p.n_acc[r];
    const int32_t c = p.ctx_len[r];
    const int32_t lim = p.limit[r];
    const uint8_t rv = p.row_valid ? p.row_valid[row] : (uint8_t)1;
    slot = -1;
    int64_t pos, pidx;
    if (!row_write_pred(p, c, n, lim, d, rv, i, pos, pidx)) return false;
    const int32_t page = p.bt[(int64_t)r * p.bt_stride + pidx];
    if (page < 0 || page >= p.num_pages) return false;
    slot = (int64_t)page * p.pg + (pos - pidx * p.pg);
    return true;
}

// Element offset of a slot inside every layer's pool (page, then slot within the page).
__device__ __forceinline__ int64_t slot_offset(const FinalizeParams &p, int64_t slot) {
    const int64_t page = slot / p.pg;
    return page * p.sp + (slot - page * p.pg) * p.ss;
}

// Placement of position ctx_new + j of the next draft block of request r (the downstream commit
// quoted on the PR #20550 page: the bookkeeping places the block's own positions in the pages):
// page * pg + offset, or -1 for a dummy request, a position outside [0, lim), past the block
// table, or in a page outside [0, num_pages).
__device__ __forceinline__ bool block_position_ok(const FinalizeParams &p, int32_t ctx_new, int32_t lim, bool d,
                                                  int j, int64_t &pos, int64_t &pidx) {
    pos = (int64_t)ctx_new + j;
    pidx = 0;
    if (d || pos < 0 || pos >= (int64_t)lim) return false;
    pidx = pos / p.pg;
    return pidx < p.bt_cols;
}
__device__ __forceinline__ int64_t block_page_slot(const FinalizeParams &p, int32_t page, int64_t pos, int64_t pidx) {
    return (page >= 0 && page < p.num_pages) ? (int64_t)page * p.pg + (pos - pidx * p.pg) : -1;
}
__device__ __forceinline__ int64_t block_position_slot(const FinalizeParams &p, int r, int32_t ctx_new, int32_t lim,
                                                       bool d, int j) {
    int64_t pos, pidx;
    if (!block_position_ok(p, ctx_new, lim, d, j, pos, pidx)) return -1;
    return block_page_slot(p, p.bt[(int64_t)r * p.bt_stride + pidx], pos, pidx);
}

// The per-request outputs of request r, written by the calling workgroup.
__device__ __forceinline__ void request_advance(const FinalizeParams &p, int r) {
    const int32_t c = p.ctx_len[r], n = p.n_acc[r], lim = p.limit[r];
    const bool d = p.dummy[r] != 0;
    const int64_t adv = (int64_t)c + n;
    const int32_t ctx_new = d ? 0 : (int32_t)(adv < (int64_t)lim ? adv : (int64_t)lim);
    const int nb = n < 1 ? 1 : (n > p.W ? p.W : n);
    const int32_t bonus = p.acc[(int64_t)r * p.acc_sr + (int64_t)(nb - 1) * p.acc_st];
    for (int j = threadIdx.x; j < p.bs_blk; j += blockDim.x) {
        p.emb[(int64_t)r * p.bs_blk + j] = j == 0 ? bonus : p.mask_id;
        p.q_pos[(int64_t)r * p.bs_blk + j] = ctx_new + j;
    }
    for (int j = threadIdx.x; j < p.W; j += blockDim.x) p.c_pos[(int64_t)r * p.W + j] = (int32_t)((int64_t)c + j);
    if (p.block_slot)
        for (int j = threadIdx.x; j < p.bs_blk; j += blockDim.x)
            p.block_slot[(int64_t)r * p.bs_blk + j] = block_position_slot(p, r, ctx_new, lim, d, j);
    if (threadIdx.x == 0) {
        p.bonus[r] = bonus;
        p.ctx_out[r] = ctx_new;
        p.seq_len[r] = ctx_new + p.bs_blk;
    }
}

// One element of a row of the stacked projection from fp32 split partials [S][M][O], summed in
// split order and rounded to bf16 (the K/V GEMM's output), as fp32.
__device__ __forceinline__ float part_y(const float *part, int S, int M, int O, int row, int64_t col) {
    float y = 0.f;
    for (int s = 0; s < S; ++s) y += part[((int64_t)s * M + row) * O + col];
    return bf2f(f2bf(y));
}

// k_norm then RoPE of one GQA K head held by one wave: lane holds a[q2] = y[j], b[q2] = y[j + hd/2]
// for j = lane + 64*q2 < hd/2 (zeros elsewhere).  ka/kb receive the rotated, rounded pair.
//   u = bf16(w * y / sqrt(mean(y^2) + eps));  k[j] = bf16(u[j] c - u[j+h] s), k[j+h] = bf16(u[j+h] c + u[j] s)
__device__ __forceinline__ void knorm_rope_head(const float a[2], const float b[2], int hd, float eps,
                                                const uint16_t *wk, const float *cs, int lane, uint16_t ka[2],
                                                uint16_t kb[2]) {
    const int half = hd >> 1;
    float ss = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) ss += a[q2] * a[q2] + b[q2] * b[q2];
    ss = wave_sum(ss);
    const float rinv = 1.0f / sqrtf(ss / (float)hd + eps);
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
        const int j = lane + q2 * 64;
        ka[q2] = kb[q2] = 0;
        if (j < half) {
            const float ua = bf2f(f2bf(bf2f(wk[j]) * (a[q2] * rinv)));
            const float ub = bf2f(f2bf(bf2f(wk[j + half]) * (b[q2] * rinv)));
            const float c = cs[j], sn = cs[half + j];
            ka[q2] = f2bf(ua * c - ub * sn);
            kb[q2] = f2bf(ub * c + ua * sn);
        }
    }
}

// 1/rms of an MLA latent held by one wave (v[q2] = y[lane + 64*q2], zeros past the latent).
__device__ __forceinline__ float latent_rinv(const float v[16], int R, float eps) {
    float ss = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < 16; ++q2) ss += v[q2] * v[q2];
    ss = wave_sum(ss);
    return 1.0f / sqrtf(ss / (float)R + eps);
}

// One normalised latent element: bf16(w * (y * rinv)).
__device__ __forceinline__ uint16_t latent_elem(uint16_t w, float y, float rinv) { return f2bf(bf2f(w) * (y * rinv)); }

// RoPE of one rotated pair (no norm), as the MLA rope part takes it.
__device__ __forceinline__ void rope_pair(float ra, float rb, float c, float sn, uint16_t &ka, uint16_t &kb) {
    ka = f2bf(ra * c - rb * sn);
    kb = f2bf(rb * c + ra * sn);
}

}  // namespace dfkv
