// k_skinny.hip -- weight-streaming split-K GEMM for the context projection at
// small batch (M = B*W <= 64 token rows), on bf16 MFMA 16x16x32.
//
// At M <= 64 the fc and stacked K/V GEMMs are bound by reading the weights
// once from HBM (TensorRT-LLM PR #13995 "DFlash performance optimizations",
// commit "migrate draft path to per-layer cached K/V pool": one GEMM stacked
// across all drafter layers on the K+1 accepted tokens; PR #20550, section
// TLLM_DFLASH_OVERLAP_CONTEXT_PROJECTION: fc + hidden_norm + latent GEMM +
// RMSNorm/RoPE).  Design for gfx950:
//  * work item = (tile of 64 output features, split of K); the grid holds
//    several items per CU so every CU keeps enough weight bytes in flight;
//  * the weight tile is the MFMA A operand: lane (q = lane/16, c = lane%16)
//    reads 64 contiguous bytes of weight row c, so 4 lanes cover 256 B of a row;
//    the activation fragment uses the same k permutation, so the dot product is
//    unchanged while every load is a 16-byte vector load;
//  * the item's activations (the B operand, M padded to 16 per group) are
//    staged once in LDS -- for the K/V GEMM with hidden_norm already applied --
//    and every k-block's fragments are read from there, so only the weight
//    stream lives in registers (double buffered across k-blocks);
//  * the 4 waves of a workgroup split the tile's K range and meet in LDS;
//  * split-K partials go to the workspace; the last workgroup to arrive on a
//    tile (agent-scope fence + ticket) sums them in a fixed order, so results
//    are deterministic, then runs the epilogue:
//      FC: round to bf16 f and the tile's per-row sum of squares (hidden_norm
//          statistic, summed in a fixed order by the next GEMM);
//      KV: the output tile is rounded to bf16 and,
//          with the fused epilogue, the last tile of each K head (GQA) or layer
//          (MLA) applies k_norm and RoPE to the whole group;
//  * tiles of one output feature range are mapped to one XCD (blockIdx % 8),
//    so the split-K partials of a tile stay in one L2.
#include "dfkv_internal.hpp"

namespace dfkv {

// Largest k extent (elements) of one work item's staged activations, per NG.
template <int NG> struct SkCfg {
    static constexpr int KC = NG == 1 ? 1024 : (NG == 2 ? 512 : 256);
    static constexpr int LDB = KC + 8;  // padded LDS row of the staged operand (bf16)
    static constexpr int RED_BYTES = 4 * 64 * (16 * NG + 1) * 4;
    static constexpr int STG_BYTES = 16 * NG * LDB * 2;
    static constexpr int SMEM = RED_BYTES > STG_BYTES ? RED_BYTES : STG_BYTES;
};

__device__ __forceinline__ void sk_load_a(const SkinnyParams &p, int t, int64_t kk, int c16, u32x4 (&a)[4][4]) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
        const u32x4 *src = (const u32x4 *)(p.w + (int64_t)(t * 64 + gi * 16 + c16) * p.K + kk);
#pragma unroll
        for (int u = 0; u < 4; ++u) a[gi][u] = src[u];
    }
}

// One k-block of 128: B fragments from the staged operand in LDS (same k
// permutation as the weights: lane group q owns 32 contiguous k), then
// 4 row groups x NG token groups x 4 MFMAs.
template <int NG>
__device__ __forceinline__ void sk_compute(const u32x4 (&a)[4][4], const uint16_t *sb, int kl, int q, int c16, int M,
                                           f32x4 (&acc)[4][NG]) {
    bf16x8 bf[NG][4];
#pragma unroll
    for (int ng = 0; ng < NG; ++ng) {
        const int n = ng * 16 + c16;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (n < M) v = *(const u32x4 *)(sb + n * SkCfg<NG>::LDB + kl + q * 32 + u * 8);
            bf[ng][u] = __builtin_bit_cast(bf16x8, v);
        }
    }
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bf16x8 av = __builtin_bit_cast(bf16x8, a[gi][u]);
#pragma unroll
            for (int ng = 0; ng < NG; ++ng)
                acc[gi][ng] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bf[ng][u], acc[gi][ng], 0, 0, 0);
        }
}

// Signal arrival on a ticket; returns true in every thread of the last arriver.
__device__ __forceinline__ bool arrive_last(int32_t *ticket, int count, int *sh_flag) {
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        const int last = (old == count - 1);
        if (last) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *sh_flag = last;
    }
    __syncthreads();
    const bool last = *sh_flag != 0;
    if (last) __threadfence();
    return last;
}

template <int NG, int MODE>
__global__ __launch_bounds__(256, 2) void k_skinny(const SkinnyParams p) {
    using Cfg = SkCfg<NG>;
    constexpr int NP = 16 * NG + 1;  // padded row of the cross-wave reduction buffer
    __shared__ __attribute__((aligned(16))) char smem[Cfg::SMEM];
    __shared__ int sh_flag;
    uint16_t *sb = (uint16_t *)smem;                      // staged B operand [16*NG][LDB]
    float(*red)[64][NP] = (float(*)[64][NP])smem;         // after the main loop: [4 waves][64][NP]

    const int T = p.O >> 6;
    const int bid = blockIdx.x;
    int t, s;
    if ((T & 7) == 0) {  // all splits of a tile on one XCD
        const int x = bid & 7, j = bid >> 3;
        t = (j / p.S) * 8 + x;
        s = j - (j / p.S) * p.S;
    } else {
        t = bid / p.S;
        s = bid - t * p.S;
    }
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q = lane >> 4, c16 = lane & 15;
    const int M = p.M;
    const int nb = p.nb_split;
    const int Kc = nb * 128;
    const int64_t k0 = (int64_t)s * Kc;

    // first weight block in flight before the activations are staged
    u32x4 a0[4][4], a1[4][4];
    int bb = wave;
    if (bb < nb) sk_load_a(p, t, k0 + (int64_t)bb * 128 + q * 32, c16, a0);

    // stage this item's activations: FC copies hidden rows; KV applies hidden_norm,
    // g = bf16(w_hn * (f * rinv)), with rinv from the per-tile sums of squares
    // written by the fc epilogue (summed in a fixed order)
    __shared__ float sh_rinv[16 * NG];
    if (MODE == SK_KV) {
        if (tid < M) {
            const int Tin = p.K >> 6;
            float ss = 0.f;
            for (int tt = 0; tt < Tin; ++tt) ss += p.ss_in[(int64_t)tt * M + tid];
            sh_rinv[tid] = 1.0f / sqrtf(ss / (float)p.K + p.nr.eps);
        }
        __syncthreads();
    }
    const int c8n = Kc >> 3;
    for (int idx = tid; idx < M * c8n; idx += 256) {
        const int n = idx / c8n, c8 = idx - (idx / c8n) * c8n;
        const int64_t kk = k0 + (c8 << 3);
        u32x4 v = *(const u32x4 *)(p.x + (int64_t)n * p.ldx + kk);
        if (MODE == SK_KV) {
            const float rinv = sh_rinv[n];
            const u32x4 wv = *(const u32x4 *)(p.w_hn + kk);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = pack2(bf_lo(wv[e]) * (bf_lo(v[e]) * rinv), bf_hi(wv[e]) * (bf_hi(v[e]) * rinv));
        }
        *(u32x4 *)(sb + n * Cfg::LDB + (c8 << 3)) = v;
    }
    __syncthreads();

    f32x4 acc[4][NG];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) acc[gi][ng] = f32x4{0.f, 0.f, 0.f, 0.f};

    if constexpr (NG <= 2) {
        // weights double buffered: the next k-block's loads are in flight during this block's MFMAs
        while (bb < nb) {
            int nx = bb + 4;
            if (nx < nb) sk_load_a(p, t, k0 + (int64_t)nx * 128 + q * 32, c16, a1);
            sk_compute<NG>(a0, sb, bb * 128, q, c16, M, acc);
            bb = nx;
            if (bb >= nb) break;
            nx = bb + 4;
            if (nx < nb) sk_load_a(p, t, k0 + (int64_t)nx * 128 + q * 32, c16, a0);
            sk_compute<NG>(a1, sb, bb * 128, q, c16, M, acc);
            bb = nx;
        }
    } else {
        // wider token groups need the registers for accumulators: single buffer
        while (bb < nb) {
            sk_compute<NG>(a0, sb, bb * 128, q, c16, M, acc);
            bb += 4;
            if (bb < nb) sk_load_a(p, t, k0 + (int64_t)bb * 128 + q * 32, c16, a0);
        }
    }
    __syncthreads();  // the staged operand is dead; its LDS becomes the reduction buffer

    // C fragment of 16x16x32: lane holds rows 4*q + v (output features) of column c16 (token).
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
#pragma unroll
        for (int ng = 0; ng < NG; ++ng)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wave][gi * 16 + q * 4 + v][ng * 16 + c16] = acc[gi][ng][v];
    __syncthreads();

    // y[o][n] (fp32) for this tile into red[0]
    if (p.S == 1) {
        for (int idx = tid; idx < 64 * M; idx += 256) {
            const int o = idx / M, n = idx - (idx / M) * M;
            red[0][o][n] = red[0][o][n] + red[1][o][n] + red[2][o][n] + red[3][o][n];
        }
    } else {
        for (int idx = tid; idx < 64 * M; idx += 256) {
            const int o = idx / M, n = idx - (idx / M) * M;
            p.part[((int64_t)s * p.O + t * 64 + o) * M + n] = red[0][o][n] + red[1][o][n] + red[2][o][n] + red[3][o][n];
        }
        if (!arrive_last(p.ticket + t, p.S, &sh_flag)) return;
        for (int idx = tid; idx < 64 * M; idx += 256) {
            const int o = idx / M, n = idx - (idx / M) * M;
            float y = 0.f;
            for (int ss = 0; ss < p.S; ++ss) y += p.part[((int64_t)ss * p.O + t * 64 + o) * M + n];
            red[0][o][n] = y;
        }
    }
    __syncthreads();

    const int col0 = t * 64;
    if (MODE == SK_FC) {
        for (int n = wave; n < M; n += 4) {
            const uint16_t yb = f2bf(red[0][lane][n]);
            p.f_out[(int64_t)n * p.O + col0 + lane] = yb;
            const float fv = bf2f(yb);
            const float ss = wave_sum(fv * fv);
            if (lane == 0) p.ss_out[(int64_t)t * M + n] = ss;
        }
        return;
    }

    for (int n = wave; n < M; n += 4) p.kv_out[(int64_t)n * p.O + col0 + lane] = f2bf(red[0][lane][n]);
    if (!p.fuse) return;

    const NormRopeGeom &g = p.nr;
    const int l = col0 / g.per_layer;
    const int off = col0 - l * g.per_layer;
    int gid, tpg;
    if (g.kind == DFKV_GQA) {
        if (off >= g.nkv * g.hd) return;  // V tile: no norm, no rotation
        const int h = off / g.hd;
        gid = l * g.nkv + h;
        tpg = g.hd >> 6;
    } else {
        gid = l;
        tpg = g.per_layer >> 6;
    }
    if (tpg > 1) {
        if (!arrive_last(p.gticket + gid, tpg, &sh_flag)) return;
    } else {
        __threadfence();  // make this workgroup's staged rows visible to its other waves
        __syncthreads();
    }
    if (g.kind == DFKV_GQA) {
        const int h = gid - l * g.nkv;
        for (int n = wave; n < M; n += 4)
            norm_rope_gqa_head(g, p.kv_out + (int64_t)n * p.O + (int64_t)l * g.per_layer + h * g.hd, l, n, lane);
    } else {
        for (int n = wave; n < M; n += 4)
            norm_rope_mla_layer(g, p.kv_out + (int64_t)n * p.O + (int64_t)l * g.per_layer, l, n, lane);
    }
}

template <int NG>
static hipError_t launch_ng(const SkinnyParams &p, int mode, hipStream_t s) {
    const int grid = (p.O >> 6) * p.S;
    if (mode == SK_FC) return launch1(k_skinny<NG, SK_FC>, dim3(grid), dim3(256), s, p);
    return launch1(k_skinny<NG, SK_KV>, dim3(grid), dim3(256), s, p);
}

hipError_t launch_skinny(const SkinnyParams &p, int mode, hipStream_t s) {
    if (p.M <= 0) return hipSuccess;
    const int ng = (p.M + 15) / 16;
    switch (ng) {
        case 1: return launch_ng<1>(p, mode, s);
        case 2: return launch_ng<2>(p, mode, s);
        case 3: return launch_ng<3>(p, mode, s);
        case 4: return launch_ng<4>(p, mode, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dfkv
