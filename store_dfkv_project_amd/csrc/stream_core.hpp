// stream_core.hpp -- one workgroup's share of the weight-streaming GEMM used at
// small batch (M = B*W <= 64 token rows), on bf16 MFMA 16x16x32 (k_stream).
//
// At M <= 64 the fc and stacked K/V GEMMs are bound by reading the weights once
// from HBM (TensorRT-LLM PR #13995 "DFlash performance optimizations", commit
// "migrate draft path to per-layer cached K/V pool": one GEMM stacked across
// the drafter layers on the K+1 accepted tokens; PR #20550, section
// TLLM_DFLASH_OVERLAP_CONTEXT_PROJECTION: fc + hidden_norm + latent GEMM).
//
// Design for gfx950:
//  * a workgroup owns 16 output features (one MFMA row group) and a K range
//    (the whole K for fc; a split of it for the K/V GEMM when there are too few
//    tiles to fill the chip);
//  * the weight rows are the MFMA A operand: for MFMA u of a 128-wide k-block,
//    lane (q = lane/16, c = lane%16) reads the 16 bytes at (4u + q)*16 of row c,
//    so each load instruction reads 64 contiguous bytes of each of 16 rows; the
//    activation (B) fragment uses the same k permutation, which leaves every
//    dot product unchanged;
//  * with a tiled weight (dfkv_pack_stream_weight) the same pieces come from a
//    copy in which each 16-row x 128-column block is 4 KB in a row, ordered as
//    the lanes load it (each load instruction reads 1 KB in a row), the 8
//    blocks the 8 waves read at once sit side by side (32 KB), and those runs
//    follow each other tile by tile, so the workgroups together sweep the
//    weight front to back (measured on MI355X: the bs=1 fc stream 20.8 -> 17.8
//    us for 100.8 MB, the MLA fc 61.9 -> 50.9 us for 308 MB);
//  * the waves of a workgroup take interleaved k-blocks; each wave keeps a ring
//    of D k-blocks of weights (and activations) in flight;
//  * fc reads its activations (hidden rows) through L2 in the register ring; its
//    epilogue rounds f = bf16(y) and writes each 16-column tile's per-row sum of
//    squares of f (the hidden_norm statistic);
//  * the K/V GEMM at <= 16 rows first stages g = bf16(w_hn * f / rms) for its k
//    range in LDS (rms from those sums, reduced in a fixed order), so hidden_norm
//    is rounded exactly where the drafter rounds it; above 16 rows it reads g
//    written by a separate hidden_norm kernel;
//  * the K/V GEMM writes fp32 split partial sums [S][M][O], reduced in split
//    order by whoever finalizes the rows.
#pragma once

#include "dfkv_internal.hpp"

namespace dfkv {

// LDS the caller provides: red [WAVES][16][16*NG+1] floats and, with STAGE, g [M][kc+8] bf16.
template <int NG, int WAVES>
constexpr int stream_red_floats() { return WAVES * 16 * (16 * NG + 1); }

template <int NG, int WAVES, int D, bool STAGE>
__device__ __forceinline__ void stream_tile(const StreamParams &p, int t, int s, float *red, uint16_t *sh_g,
                                            float *sh_rinv) {
    constexpr int NP = 16 * NG + 1;
    constexpr int NT = WAVES * 64;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q = lane >> 4, c16 = lane & 15;
    const int M = p.M;
    // this lane's 16-byte piece u of 128-wide k-block kb: row t*16 + c16, columns kb*128 + (4u + q)*8 of
    // a row-major weight; piece u*64 + q*16 + c16 of block stream_block(kb, t) of a tiled one
    const uint16_t *wl = p.w_tiled ? p.w + (q * 16 + c16) * 8 : p.w + (int64_t)(t * 16 + c16) * p.K + q * 8;
    auto wpiece = [&](int64_t kb) -> const uint16_t * {
        return p.w_tiled ? wl + stream_block(kb, t, p.O, p.K) * 2048 : wl + kb * 128;
    };
    const int w_u = p.w_tiled ? 512 : 32;
    const int kb0 = s * p.nbs;  // first k-block (128 wide) of the split
    const int kc = p.nbs * 128, ldg = kc + 8;
    const int nbw = wave < p.nbs ? (p.nbs - wave + WAVES - 1) / WAVES : 0;

    u32x4 a[D][4];
    u32x4 b[STAGE ? 1 : D][NG][4];
    auto load = [&](int slot, int j) {
        const int64_t kb = kb0 + wave + j * WAVES, k = kb * 128;
        const uint16_t *wp = wpiece(kb);
#pragma unroll
        for (int u = 0; u < 4; ++u) a[slot][u] = load_streamed(wp + u * w_u);
        if (!STAGE) {
#pragma unroll
            for (int ng = 0; ng < NG; ++ng) {
                const int n = ng * 16 + c16;
                if (n < M) {
                    const uint16_t *xr = p.x + (int64_t)n * p.ldx + k;
#pragma unroll
                    for (int u = 0; u < 4; ++u) b[slot][ng][u] = *(const u32x4 *)(xr + (u * 4 + q) * 8);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) b[slot][ng][u] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (d < nbw) load(d, d);

    if (STAGE) {
        // one hop: this thread's f and w_hn chunks (at most kStageChunks), and the row statistics
        const int c8n = kc >> 3;
        u32x4 fv[kStageChunks], wv[kStageChunks];
#pragma unroll
        for (int i = 0; i < kStageChunks; ++i) {
            const int idx = tid + i * NT;
            if (idx < M * c8n) {
                const int n = idx / c8n, c8 = idx - (idx / c8n) * c8n;
                const int64_t kk = (int64_t)kb0 * 128 + (c8 << 3);
                fv[i] = *(const u32x4 *)(p.x + (int64_t)n * p.ldx + kk);
                wv[i] = *(const u32x4 *)(p.w_hn + kk);
            }
        }
        for (int n = wave; n < M; n += WAVES) {  // rinv[n] = 1/sqrt(mean(f[n]^2) + eps), fixed order
            float ss = 0.f;
            for (int tt = lane; tt < p.T_in; tt += 64) ss += p.ss_in[(int64_t)tt * M + n];
            ss = wave_sum(ss);
            if (lane == 0) sh_rinv[n] = 1.0f / sqrtf(ss / (float)p.K + p.eps);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kStageChunks; ++i) {
            const int idx = tid + i * NT;
            if (idx < M * c8n) {
                const int n = idx / c8n, c8 = idx - (idx / c8n) * c8n;
                const float rinv = sh_rinv[n];
                u32x4 gv;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    gv[e] = pack2(bf_lo(wv[i][e]) * (bf_lo(fv[i][e]) * rinv), bf_hi(wv[i][e]) * (bf_hi(fv[i][e]) * rinv));
                *(u32x4 *)(sh_g + n * ldg + (c8 << 3)) = gv;
            }
        }
        __syncthreads();
    }

    f32x4 acc[NG];
#pragma unroll
    for (int ng = 0; ng < NG; ++ng) acc[ng] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int j0 = 0; j0 < nbw; j0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int j = j0 + d;
            if (j >= nbw) break;
            const int kl = (wave + j * WAVES) * 128;  // k offset inside the split
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bf16x8 av = __builtin_bit_cast(bf16x8, a[d][u]);
#pragma unroll
                for (int ng = 0; ng < NG; ++ng) {
                    u32x4 v;
                    if (STAGE) {
                        const int n = ng * 16 + c16;
                        v = n < M ? *(const u32x4 *)(sh_g + n * ldg + kl + (u * 4 + q) * 8) : u32x4{0u, 0u, 0u, 0u};
                    } else {
                        v = b[d][ng][u];
                    }
                    acc[ng] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, v), acc[ng],
                                                                     0, 0, 0);
                }
            }
            if (j + D < nbw) load(d, j + D);
        }
    }

    // C fragment of 16x16x32: lane holds output rows 4*q + v (features) of column c16 (token).
#pragma unroll
    for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[(wave * 16 + q * 4 + v) * NP + ng * 16 + c16] = acc[ng][v];
    __syncthreads();

    if (p.out) {
        // fc: f = bf16(y) (two features per thread, one 32-bit store) and the tile's per-row sum of
        // squares of f (the hidden_norm statistic)
        for (int idx = tid; idx < 8 * M; idx += NT) {
            const int o2 = idx & 7, n = idx >> 3;
            uint16_t fb[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int o = 2 * o2 + h;
                float y = 0.f;
#pragma unroll
                for (int w = 0; w < WAVES; ++w) y += red[(w * 16 + o) * NP + n];
                fb[h] = f2bf(y);
            }
            red[(2 * o2) * NP + n] = bf2f(fb[0]);
            red[(2 * o2 + 1) * NP + n] = bf2f(fb[1]);
            *(uint32_t *)(p.out + (int64_t)n * p.O + t * 16 + 2 * o2) = (uint32_t)fb[0] | ((uint32_t)fb[1] << 16);
        }
        __syncthreads();
        for (int n = tid; n < M; n += NT) {
            float ss = 0.f;
#pragma unroll
            for (int o = 0; o < 16; ++o) ss += red[o * NP + n] * red[o * NP + n];
            p.ss_out[(int64_t)t * M + n] = ss;
        }
    } else {
        for (int idx = tid; idx < 16 * M; idx += NT) {
            const int o = idx & 15, n = idx >> 4;
            float y = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) y += red[(w * 16 + o) * NP + n];
            p.part[((int64_t)s * M + n) * p.O + t * 16 + o] = y;
        }
    }
}

}  // namespace dfkv
