// k_misc.hip -- hidden_norm (large-batch path), the cos/sin cache builder and a
// zero-fill kernel.
#include <math.h>

#include "dfkv_internal.hpp"

namespace dfkv {

// ---------------------------------------------------------------------------
// hidden_norm: g[n][:] = bf16(w * f[n][:] / sqrt(mean(f[n]^2) + eps)); one
// workgroup per row (used by the large-batch path; the small-batch path folds
// it into the stacked GEMM's operand load).  When the fc GEMM was split over
// k, f is first formed here: f = bf16(sum over the S fp32 partials, in split
// order), written out and then normalised.  k_hidden_norm_packed (below) writes g
// in the fragment order of k_gemm_w's token operand instead.
// ---------------------------------------------------------------------------
struct HiddenNormArgs {
    const uint16_t *w;
    uint16_t *f, *g;
    const float *part;   // [S][n_rows][H] fp32 partial sums of f, or null (f is given)
    int S, n_rows, H;
    float eps;
    int packed;          // rows per workgroup of k_hidden_norm_packed (0: row-major k_hidden_norm)
};

__global__ __launch_bounds__(256) void k_hidden_norm(const HiddenNormArgs a) {
    const uint16_t *w = a.w;
    uint16_t *g = a.g;
    const int H = a.H;
    const float eps = a.eps;
    const int row = blockIdx.x;
    uint16_t *x = a.f + (int64_t)row * H;
    __shared__ float red[4];
    float ss = 0.f;
    for (int c = threadIdx.x; c < (H >> 3); c += blockDim.x) {
        u32x4 v;
        if (a.part) {
            // each thread writes and later re-reads the same chunks of f: no cross-thread hand-off
            float s8[8];
            const float *src = a.part + (int64_t)row * H + (c << 3);
#pragma unroll
            for (int e = 0; e < 8; ++e) s8[e] = 0.f;
            for (int sp = 0; sp < a.S; ++sp) {
                const float4 lo = *(const float4 *)(src + (int64_t)sp * a.n_rows * H);
                const float4 hi = *(const float4 *)(src + (int64_t)sp * a.n_rows * H + 4);
                s8[0] += lo.x; s8[1] += lo.y; s8[2] += lo.z; s8[3] += lo.w;
                s8[4] += hi.x; s8[5] += hi.y; s8[6] += hi.z; s8[7] += hi.w;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = pack2(s8[2 * q], s8[2 * q + 1]);
            *(u32x4 *)(x + (c << 3)) = v;
        } else {
            v = *(const u32x4 *)(x + (c << 3));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float a = bf_lo(v[q]), b = bf_hi(v[q]);
            ss += a * a + b * b;
        }
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = red[0] + red[1] + red[2] + red[3];
    const float rinv = 1.0f / sqrtf(tot / (float)H + eps);
    for (int c = threadIdx.x; c < (H >> 3); c += blockDim.x) {
        const u32x4 v = *(const u32x4 *)(x + (c << 3));
        const u32x4 wv = *(const u32x4 *)(w + (c << 3));
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = pack2(bf_lo(wv[q]) * (bf_lo(v[q]) * rinv), bf_hi(wv[q]) * (bf_hi(v[q]) * rinv));
        *(u32x4 *)(g + (int64_t)row * H + (c << 3)) = o;
    }
}

// hidden_norm into the packed token order, R rows (1, 2 or 4) per workgroup: the R rows'
// f (summed from the partials and rounded, or as given) is staged in LDS while each row's sum of
// squares is taken, then every 16-byte piece of g goes out in packed order, where the R rows'
// pieces of one (stage, slice, lane half) are R*16 bytes in a row.  Rows past n_rows (up to the
// next multiple of 64) come out zero.  f is not written back.
constexpr int kHnpThreads = 512;
constexpr int kHnpLds = 128 * 1024;   // the larger of the two LDS sizes (R * H * 2 bytes fit in it)

template <int LDS>
__global__ __launch_bounds__(kHnpThreads) void k_hidden_norm_packed(const HiddenNormArgs ain) {
    // the kernel arguments in one round of scalar loads: a field read where the code first needs it
    // is a round trip of its own through the scalar cache, which starts cold in every kernel
    HiddenNormArgs a = ain;
    asm volatile("" : "+s"(a.packed), "+s"(a.H), "+s"(a.S), "+s"(a.n_rows) : "s"(a.w), "s"(a.f), "s"(a.g), "s"(a.part),
                 "s"(a.eps));
    __shared__ __attribute__((aligned(16))) uint8_t hn_lds[LDS];
    uint16_t *rows = (uint16_t *)hn_lds;                // [R][H] bf16
    __shared__ float ssp[8], rinv_s[4];
    const int R = a.packed;                             // rows per workgroup: 1, 2 or 4
    const int lgR = R >> 1;                             // log2(R), so that no division by R is needed
    const int H = a.H, cpr = H >> 3;                    // 16-byte chunks per row
    const int n0 = blockIdx.x * R;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // phase 1: wpr = 8 / R waves per row, each summing every wpr-th run of 64 chunks
    const int wpr = 8 >> lgR;
    {
        const int r = wave >> (3 - lgR), part = wave & (wpr - 1);
        const int n = n0 + r;
        float ss = 0.f;
        for (int c = part * 64 + lane; c < cpr; c += 64 * wpr) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (n < a.n_rows) {
                if (a.part) {
                    float s8[8];
                    const float *src = a.part + (int64_t)n * H + (c << 3);
#pragma unroll
                    for (int e = 0; e < 8; ++e) s8[e] = 0.f;
                    for (int sp = 0; sp < a.S; ++sp) {
                        const float4 lo = *(const float4 *)(src + (int64_t)sp * a.n_rows * H);
                        const float4 hi = *(const float4 *)(src + (int64_t)sp * a.n_rows * H + 4);
                        s8[0] += lo.x; s8[1] += lo.y; s8[2] += lo.z; s8[3] += lo.w;
                        s8[4] += hi.x; s8[5] += hi.y; s8[6] += hi.z; s8[7] += hi.w;
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = pack2(s8[2 * q], s8[2 * q + 1]);
                } else {
                    v = *(const u32x4 *)(a.f + (int64_t)n * H + (c << 3));
                }
            }
            *(u32x4 *)(rows + (int64_t)r * H + (c << 3)) = v;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float x = bf_lo(v[q]), y = bf_hi(v[q]);
                ss += x * x + y * y;
            }
        }
        ss = wave_sum(ss);
        if (lane == 0) ssp[wave] = ss;
    }
    __syncthreads();
    if (tid < R) {
        float ss = 0.f;
        for (int q = 0; q < wpr; ++q) ss += ssp[tid * wpr + q];
        rinv_s[tid] = 1.0f / sqrtf(ss / (float)H + a.eps);
    }
    __syncthreads();
    // phase 2: piece p = (q, r), q = (it*4 + s)*2 + fh in memory order, r the row in the group
    const int iters = H >> 6;
    const int64_t b = n0 >> 6, j = (n0 >> 5) & 1, fr0 = n0 & 31;
    for (int p = tid; p < R * cpr; p += kHnpThreads) {
        const int r = p & (R - 1), q = p >> lgR;
        const int fh = q & 1, sl = (q >> 1) & 3, it = q >> 3;
        const int k = 64 * it + 32 * fh + 8 * sl;
        const u32x4 v = *(const u32x4 *)(rows + (int64_t)r * H + k);
        const u32x4 wv = *(const u32x4 *)(a.w + k);
        const float ri = rinv_s[r];
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = pack2(bf_lo(wv[e]) * (bf_lo(v[e]) * ri), bf_hi(wv[e]) * (bf_hi(v[e]) * ri));
        const int64_t dst = ((((b * iters + it) * 4 + sl) * 2 + j) * 64 + fr0 + r + 32 * fh) * 8;
        *(u32x4 *)(a.g + dst) = o;
    }
}

// Rows per workgroup of the packed variant: 4 or 2 when their rows fit 32 KB of LDS (several
// workgroups per CU, so that some read while others write: measured at 4096 x 4096, R = 4 takes
// 15.5 us, R = 1 32 us) and the padded rows still give at least 256 workgroups, else 1.
int hidden_norm_rows(int n_rows, int H) {
    const int Mp = (n_rows + 63) / 64 * 64;
    for (int R = 4; R > 1; R >>= 1)
        if ((int64_t)R * H * 2 <= kHnpLds / 4 && Mp / R >= 256) return R;
    return 1;
}

hipError_t launch_hidden_norm(uint16_t *f, const float *part, int S, const uint16_t *w, uint16_t *g, int n_rows,
                              int H, float eps, bool packed, hipStream_t s) {
    if (n_rows == 0) return hipSuccess;
    if (H % (packed ? 64 : 8) != 0 || (part && S < 1)) return hipErrorInvalidValue;
    if (!packed)
        return launch1(k_hidden_norm, dim3(n_rows), dim3(256), s, HiddenNormArgs{w, f, g, part, S, n_rows, H, eps, 0});
    const int R = hidden_norm_rows(n_rows, H);
    const int64_t lds = (int64_t)R * H * 2;
    if (lds > kHnpLds) return hipErrorInvalidValue;
    const int Mp = (n_rows + 63) / 64 * 64;
    const HiddenNormArgs args{w, f, g, part, S, n_rows, H, eps, R};
    // the smallest LDS size that holds the rows (LDS per workgroup bounds workgroups per CU)
    if (lds <= kHnpLds / 4) return launch1(k_hidden_norm_packed<kHnpLds / 4>, dim3(Mp / R), dim3(kHnpThreads), s, args);
    if (lds <= kHnpLds / 2) return launch1(k_hidden_norm_packed<kHnpLds / 2>, dim3(Mp / R), dim3(kHnpThreads), s, args);
    return launch1(k_hidden_norm_packed<kHnpLds>, dim3(Mp / R), dim3(kHnpThreads), s, args);
}

// ---------------------------------------------------------------------------
// A row-major bf16 matrix [rows][K] rewritten in the fragment order of
// gemm_pack_index (the large-batch GEMM's per-wave operand): one thread per
// 16-byte chunk, which moves whole (8 consecutive k stay together).
// ---------------------------------------------------------------------------
struct PackArgs {
    const uint16_t *src;
    uint16_t *dst;
    int64_t rows, K;
};

__global__ __launch_bounds__(256) void k_pack_rows(const PackArgs a) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t cpr = a.K >> 3;
    if (t >= a.rows * cpr) return;
    const int64_t n = t / cpr, c = t - n * cpr;
    *(u32x4 *)(a.dst + gemm_pack_index(n, c << 3, a.K >> 6)) = *(const u32x4 *)(a.src + n * a.K + (c << 3));
}

hipError_t launch_pack_rows(const uint16_t *src, uint16_t *dst, int64_t rows, int64_t K, hipStream_t s) {
    if (rows % 64 != 0 || K % 64 != 0 || rows <= 0) return hipErrorInvalidValue;
    const int64_t chunks = rows * (K >> 3);
    return launch1(k_pack_rows, dim3((unsigned)((chunks + 255) / 256)), dim3(256), s, PackArgs{src, dst, rows, K});
}

// A row-major bf16 matrix [rows][K] rewritten in the weight-streaming order of stream_pack_index:
// one thread per 16-byte chunk (8 consecutive k stay together), writes contiguous along threads.
__global__ __launch_bounds__(256) void k_pack_stream(const PackArgs a) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= a.rows * (a.K >> 3)) return;
    // t enumerates destination chunks: block blk = j*8*T + ob*width + w (stream_block), piece (u, q, c16)
    const int64_t T = a.rows >> 4, blk = t >> 8, piece = t & 255;
    const int64_t j = blk / (8 * T), rem = blk - j * 8 * T, left = (a.K >> 7) - 8 * j, width = left < 8 ? left : 8;
    const int64_t ob = rem / width, kb = 8 * j + (rem - ob * width);
    const int u = (int)(piece >> 6), q = (int)((piece >> 4) & 3), c16 = (int)(piece & 15);
    const int64_t o = ob * 16 + c16, k = kb * 128 + (4 * u + q) * 8;
    *(u32x4 *)(a.dst + (t << 3)) = *(const u32x4 *)(a.src + o * a.K + k);
}

hipError_t launch_pack_stream(const uint16_t *src, uint16_t *dst, int64_t rows, int64_t K, hipStream_t s) {
    if (rows % 16 != 0 || K % 128 != 0 || rows <= 0) return hipErrorInvalidValue;
    const int64_t chunks = rows * (K >> 3);
    return launch1(k_pack_stream, dim3((unsigned)((chunks + 255) / 256)), dim3(256), s, PackArgs{src, dst, rows, K});
}

// ---------------------------------------------------------------------------
// cos/sin cache in fp64 (stored fp32).  Plain RoPE: inv_i = theta^(-2i/rot).
// YaRN (Peng et al. 2023, "NTK-by-parts" + attention temperature, in the HF
// formulation that honours truncate=false): the correction dim for n turns is
// rot*ln(orig_ctx/(2*pi*n)) / (2 ln theta); lo from beta_fast, hi from
// beta_slow, clamped to [0, rot-1] (floor/ceil first only if truncate); a
// linear ramp over i in [lo, hi] moves inv_i from the original value to
// inv_i/factor; cos and sin are scaled by 0.1*ln(factor) + 1.
// One thread per (position, pair index).
// ---------------------------------------------------------------------------
struct RopeCacheArgs {
    dfkv_rope r;
    float *cs;
    int cache_len;
};

__global__ __launch_bounds__(256) void k_rope_cache(const RopeCacheArgs args) {
    const dfkv_rope &r = args.r;
    float *cs = args.cs;
    const int cache_len = args.cache_len;
    const int half = r.rot >> 1;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)cache_len * half) return;
    const int p = (int)(t / half);
    const int i = (int)(t - (int64_t)p * half);
    double inv = pow(r.theta, -(2.0 * i) / (double)r.rot);
    double m = 1.0;
    if (r.yarn) {
        const double two_pi = 6.283185307179586476925286766559;
        const double denom = 2.0 * log(r.theta);
        double lo = (double)r.rot * log(r.orig_ctx / (r.beta_fast * two_pi)) / denom;
        double hi = (double)r.rot * log(r.orig_ctx / (r.beta_slow * two_pi)) / denom;
        if (r.truncate) {
            lo = floor(lo);
            hi = ceil(hi);
        }
        lo = lo < 0.0 ? 0.0 : lo;
        hi = hi > (double)(r.rot - 1) ? (double)(r.rot - 1) : hi;
        if (lo == hi) hi += 0.001;
        double ramp = ((double)i - lo) / (hi - lo);
        ramp = ramp < 0.0 ? 0.0 : (ramp > 1.0 ? 1.0 : ramp);
        inv = (inv / r.factor) * ramp + inv * (1.0 - ramp);
        if (r.factor > 1.0) m = 0.1 * log(r.factor) + 1.0;
    }
    const double a = (double)p * inv;
    cs[(int64_t)p * r.rot + i] = (float)(cos(a) * m);
    cs[(int64_t)p * r.rot + half + i] = (float)(sin(a) * m);
}

hipError_t launch_rope_cache(const dfkv_rope &r, float *cs, int cache_len, hipStream_t s) {
    const int64_t n = (int64_t)cache_len * (r.rot / 2);
    if (n == 0) return hipSuccess;
    return launch1(k_rope_cache, dim3((unsigned)((n + 255) / 256)), dim3(256), s, RopeCacheArgs{r, cs, cache_len});
}

// ---------------------------------------------------------------------------
// Zero-fill with vector stores (used to prepare a workspace; a kernel rather
// than a memset node so that it can sit inside a captured graph).
// ---------------------------------------------------------------------------
struct FillArgs {
    uint32_t *p;
    size_t n_words;
};

__global__ __launch_bounds__(256) void k_fill_zero(const FillArgs a) {
    uint32_t *p = a.p;
    const size_t n_words = a.n_words;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s) {
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    return launch1(k_fill_zero, dim3((unsigned)blocks), dim3(256), s, FillArgs{(uint32_t *)p, words});
}

}  // namespace dfkv

namespace dfkv {

// ---------------------------------------------------------------------------
// Draft-KV block-table decode (TensorRT-LLM PR #20550 "fuse the decode-step
// drafter bookkeeping into Triton kernels": the refresh of the draft block
// table, page counts and decoded table; the downstream commit quoted on that
// page: blocks per request, clamped and divided offsets, one launch).
//   count[r]    = clamp(ceil(n_tokens[r] / page_size), 0, max_blocks)
//   table[r][b] = b < count[r] && off(r, b) >= 0 ? off(r, b) / divisor : -1
// One thread per table entry; the entries of a row are consecutive threads, so
// the table stores coalesce (the strided offset view need not).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bt_decode(const BtDecodeArgs a) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)a.B * a.max_blocks) return;
    const int r = (int)(e / a.max_blocks), b = (int)(e - (int64_t)r * a.max_blocks);
    const int64_t n = a.n_tokens[r];
    int64_t pages = n <= 0 ? 0 : (n + a.page_size - 1) / a.page_size;
    pages = pages < a.max_blocks ? pages : a.max_blocks;
    if (b == 0) a.count[r] = (int32_t)pages;
    int32_t t = -1;
    if (b < pages) {
        const int32_t off = a.off[(int64_t)r * a.s_req + (int64_t)b * a.s_blk];
        if (off >= 0) t = off / a.divisor;
    }
    a.table[(int64_t)r * a.t_stride + b] = t;
}

// rows with no blocks still get their page count
__global__ __launch_bounds__(256) void k_bt_count(const BtDecodeArgs a) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r < a.B) a.count[r] = 0;
}

hipError_t launch_bt_decode(const BtDecodeArgs &a, hipStream_t s) {
    if (a.B <= 0) return hipSuccess;
    if (a.max_blocks == 0) return launch1(k_bt_count, dim3((unsigned)((a.B + 255) / 256)), dim3(256), s, a);
    const int64_t n = (int64_t)a.B * a.max_blocks;
    return launch1(k_bt_decode, dim3((unsigned)((n + 255) / 256)), dim3(256), s, a);
}

}  // namespace dfkv

namespace dfkv {

// ---------------------------------------------------------------------------
// Strict acceptance of a uniform-width draft (the downstream commit quoted on
// the TensorRT-LLM PR #20550 page): n_acc = 1 + the draft's prefix that equals
// the target's tokens; the accepted tokens are the target's.  One wave per
// request: lane i compares position i (i < K), the first mismatch is the
// lowest lane with a mismatch (a ballot), and lanes copy the target's tokens.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_strict_accept(const AcceptArgs a) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= a.B) return;
    const int K = a.W - 1;
    int first = K;                        // first mismatching position, K when the draft matches fully
    for (int i0 = 0; i0 < K; i0 += 64) {
        const int i = i0 + lane;
        const bool miss = i < K && a.draft[(int64_t)r * a.d_sr + (int64_t)i * a.d_st] !=
                                       a.target[(int64_t)r * a.t_sr + (int64_t)i * a.t_st];
        const unsigned long long m = __ballot(miss);
        if (m) {
            first = i0 + __ffsll((long long)m) - 1;
            break;
        }
    }
    if (lane == 0) a.n_acc[r] = 1 + first;
    for (int i = lane; i < a.W; i += 64) a.acc[(int64_t)r * a.W + i] = a.target[(int64_t)r * a.t_sr + (int64_t)i * a.t_st];
}

hipError_t launch_strict_accept(const AcceptArgs &a, hipStream_t s) {
    if (a.B <= 0) return hipSuccess;
    return launch1(k_strict_accept, dim3((unsigned)((a.B + 3) / 4)), dim3(256), s, a);
}

}  // namespace dfkv
