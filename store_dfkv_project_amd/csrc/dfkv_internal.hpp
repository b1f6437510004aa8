// dfkv_internal.hpp -- device helpers and the launch interface shared by the
// libdfkv translation units (gfx950 only; not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dfkv.h"

namespace dfkv {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// ---------------------------------------------------------------------------
// Projection epilogue helpers shared by the standalone norm/RoPE kernel and
// the GEMM epilogues.  One wave handles one (row, head) or one (row, layer).
// ---------------------------------------------------------------------------

struct NormRopeGeom {
    int32_t kind, n_layers, nkv, hd, latent, rope_dim, per_layer, width, cache_len;
    int32_t out_dim;  // O
    float eps;
    const uint16_t *w_knorm;
    const int32_t *ctx_len_in;
    const float *cos_sin;
};

__device__ __forceinline__ const float *rope_row(const NormRopeGeom &g, int row) {
    int r = row / g.width, i = row - r * g.width;
    int64_t pos = (int64_t)g.ctx_len_in[r] + i;
    int64_t p = pos < 0 ? 0 : (pos > g.cache_len - 1 ? g.cache_len - 1 : pos);
    return g.cos_sin + p * g.rope_dim;
}

// GQA K head of hd (<= 256) elements at `x` (bf16, in place), layer l.
// Lane handles the NeoX pairs (j, j + hd/2) for j = lane, lane + 64.
__device__ __forceinline__ void norm_rope_gqa_head(const NormRopeGeom &g, uint16_t *x, int l, int row, int lane) {
    const int half = g.hd >> 1;
    float a[2], b[2];
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        int j = lane + q * kWave;
        a[q] = b[q] = 0.f;
        if (j < half) {
            a[q] = bf2f(x[j]);
            b[q] = bf2f(x[j + half]);
            ss += a[q] * a[q] + b[q] * b[q];
        }
    }
    ss = wave_sum(ss);
    const float rinv = 1.0f / sqrtf(ss / (float)g.hd + g.eps);
    const float *cs = rope_row(g, row);
    const uint16_t *wk = g.w_knorm + (int64_t)l * g.hd;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        int j = lane + q * kWave;
        if (j < half) {
            float ua = bf2f(f2bf(bf2f(wk[j]) * (a[q] * rinv)));
            float ub = bf2f(f2bf(bf2f(wk[j + half]) * (b[q] * rinv)));
            float c = cs[j], s = cs[half + j];
            x[j] = f2bf(ua * c - ub * s);
            x[j + half] = f2bf(ub * c + ua * s);
        }
    }
}

// MLA layer slice at `x`: latent (RMSNorm with w_knorm[l]) then rope part (rotation only).
__device__ __forceinline__ void norm_rope_mla_layer(const NormRopeGeom &g, uint16_t *x, int l, int row, int lane) {
    const int R = g.latent;
    float v[16];  // R <= 1024
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        int e = lane + q * kWave;
        v[q] = 0.f;
        if (e < R) {
            v[q] = bf2f(x[e]);
            ss += v[q] * v[q];
        }
    }
    ss = wave_sum(ss);
    const float rinv = 1.0f / sqrtf(ss / (float)R + g.eps);
    const uint16_t *wk = g.w_knorm + (int64_t)l * R;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        int e = lane + q * kWave;
        if (e < R) x[e] = f2bf(bf2f(wk[e]) * (v[q] * rinv));
    }
    const int half = g.rope_dim >> 1;  // <= 64
    if (lane < half) {
        const float *cs = rope_row(g, row);
        uint16_t *rp = x + R;
        float a = bf2f(rp[lane]), b = bf2f(rp[lane + half]);
        float c = cs[lane], s = cs[half + lane];
        rp[lane] = f2bf(a * c - b * s);
        rp[lane + half] = f2bf(b * c + a * s);
    }
}

// ---------------------------------------------------------------------------
// Launch interface (host side, C++ linkage inside the library)
// ---------------------------------------------------------------------------

// Launch a kernel whose only parameter is a struct passed by value, returning the
// status of this launch alone (hipLaunchKernel; the process-wide "last error" that
// other code may have left behind is neither read nor cleared).
template <typename P>
inline hipError_t launch1(void (*kernel)(P), dim3 grid, dim3 block, hipStream_t s, const P &p) {
    P copy = p;
    void *args[] = {(void *)&copy};
    return hipLaunchKernel((const void *)kernel, grid, block, args, 0, s);
}

// Record a failed HIP call for dfkv_hip_error_string (per host thread).
void note_hip_error(hipError_t e);

struct StoreParams {
    const uint16_t *kv;
    int64_t kv_ld;
    int32_t B, W, bs_blk, pg, L, kind, nkv, hd, per_layer;
    const int32_t *ctx_len, *n_acc, *limit;
    const uint8_t *dummy, *row_valid;
    const int32_t *bt;
    int64_t bt_stride;
    int32_t bt_cols, num_pages;
    const int32_t *acc;
    int64_t acc_sr, acc_st;
    int32_t mask_id;
    uint16_t *pk[DFKV_MAX_LAYERS];
    uint16_t *pv[DFKV_MAX_LAYERS];
    int64_t sp, ss, sh;
    int64_t *slot;
    uint8_t *wmask;
    int32_t *c_pos, *bonus, *emb, *q_pos, *ctx_out, *seq_len;
};
hipError_t launch_store_advance(const StoreParams &p, bool store, bool advance, hipStream_t s);

hipError_t launch_norm_rope(const NormRopeGeom &g, uint16_t *kv, int n_rows, hipStream_t s);
hipError_t launch_hidden_norm(const uint16_t *f, const uint16_t *w, uint16_t *g, int n_rows, int H, float eps,
                              hipStream_t s);
hipError_t launch_rope_cache(const dfkv_rope &r, float *cs, int cache_len, hipStream_t s);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);

// Skinny split-K projection GEMM (M <= 64 token rows).
enum { SK_FC = 0, SK_KV = 1 };
struct SkinnyParams {
    const uint16_t *w;   // [O][K]
    const uint16_t *x;   // FC: hidden rows (ldx); KV: f rows [M][K]
    int64_t ldx;
    int32_t M, K, O, S, nb_split;  // k-blocks of 128 per split
    float *part;                   // [S][O][M]
    int32_t *ticket;               // [O/64]
    // FC epilogue
    uint16_t *f_out;   // [M][O]
    float *ss_out;     // [O/64][M]
    // KV prologue (hidden_norm) and epilogue
    const uint16_t *w_hn;
    const float *ss_in;  // [K/64][M]
    uint16_t *kv_out;    // [M][O]
    int32_t *gticket;    // norm-group tickets
    int32_t fuse;
    NormRopeGeom nr;
};
hipError_t launch_skinny(const SkinnyParams &p, int mode, hipStream_t s);

// Tiled MFMA GEMM for larger M: out[n][o] = bf16(sum_k x[n][k] w[o][k]).
struct TiledParams {
    const uint16_t *x;
    int64_t ldx;
    const uint16_t *w;
    uint16_t *out;
    int64_t ldo;
    int32_t M, K, O;
};
hipError_t launch_tiled(const TiledParams &p, hipStream_t s);

}  // namespace dfkv
