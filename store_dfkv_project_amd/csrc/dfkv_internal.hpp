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

// a / b for integers 0 <= a < 2^21 and b >= 1, given rb = 1 / b in fp32: the fp32 product of a + 0.5
// and rb is within 2^-22 relative of (a + 0.5) / b, whose fraction part is at least 0.5 / b away from
// an integer, so truncation gives floor(a / b) exactly -- a few instructions where a 32-bit integer
// division by a value known only at run time takes about thirty, on the path to a kernel's first loads.
__device__ __forceinline__ int div_small(int a, float rb) { return (int)(((float)a + 0.5f) * rb); }

// 16 bytes of a weight that a step streams exactly once (the weight-streaming GEMMs at small batch),
// loaded non-temporally: the stream then does not evict what the step reads again from the caches
// (the next kernels' code and arguments, the fc output, the split partials).  Measured on MI355X:
// dense drafter at 4 rows 40.6 -> 38.5 us per step, MLA drafter at 4 rows 66.0 -> 60.5 us.
__device__ __forceinline__ u32x4 load_streamed(const uint16_t *p) {
    return __builtin_nontemporal_load((const u32x4 *)p);
}

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
// Two fp32 -> two bf16 (lo in the low half), round to nearest, ties to even: one
// v_cvt_pk_bf16_f32 on gfx950 (f2bf's rounding for every non-NaN input, denormals included).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// v plus the value DPP control CTRL moves to this lane (rows outside ROWM add nothing).
template <int CTRL, int ROWM = 0xF>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWM, 0xF, false));
}

// Sum over the 64 lanes of a wave, in every lane, by DPP moves (no LDS round trips): quad_perm
// [1,0,3,2] and [2,3,0,1] sum each quad, row_ror:4 and :8 each row of 16, row_bcast:15 into rows
// 1 and 3 and row_bcast:31 into rows 2 and 3 leave the total in lane 63, which is read back.
__device__ __forceinline__ float wave_sum(float v) {
    v = dpp_add<0xB1>(v);
    v = dpp_add<0x4E>(v);
    v = dpp_add<0x124>(v);
    v = dpp_add<0x128>(v);
    v = dpp_add<0x142, 0xA>(v);
    v = dpp_add<0x143, 0xC>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ---------------------------------------------------------------------------
// Geometry of the k_norm / RoPE epilogue.
// ---------------------------------------------------------------------------

struct NormRopeGeom {
    int32_t kind, n_layers, nkv, hd, latent, rope_dim, per_layer, width, cache_len;
    int32_t out_dim;  // O
    float eps;
    const uint16_t *w_knorm;
    const int32_t *ctx_len_in;
    const float *cos_sin;
};

// cos/sin cache row of token row `row`: position ctx_len_in[r] + i, clamped to the cache.
__device__ __forceinline__ const float *rope_row(const NormRopeGeom &g, int row) {
    const int r = row / g.width, i = row - r * g.width;
    const int64_t pos = (int64_t)g.ctx_len_in[r] + i;
    const int64_t p = pos < 0 ? 0 : (pos > g.cache_len - 1 ? g.cache_len - 1 : pos);
    return g.cos_sin + p * g.rope_dim;
}

// ---------------------------------------------------------------------------
// Launch interface (host side, C++ linkage inside the library)
// ---------------------------------------------------------------------------

// Launch a kernel whose only parameter is a struct passed by value, returning the
// status of this launch alone (hipLaunchKernel; the process-wide "last error" that
// other code may have left behind is neither read nor cleared).
template <typename P>
inline hipError_t launch1(void (*kernel)(P), dim3 grid, dim3 block, hipStream_t s, const P &p, size_t shmem = 0) {
    P copy = p;
    void *args[] = {(void *)&copy};
    return hipLaunchKernel((const void *)kernel, grid, block, args, shmem, s);
}

// Record a failed HIP call for dfkv_hip_error_string (per host thread).
void note_hip_error(hipError_t e);

// Finalize: k_norm/RoPE + paged store + advance (one workgroup per row x layer).
struct FinalizeParams {
    // source rows of the stacked projection: fp32 split-K partials [S][M][O], or bf16 rows [N][O]
    const float *part;
    int32_t S, M, O;
    const uint16_t *src;
    uint16_t *kv_out;  // final bf16 rows [N][O], or NULL
    int32_t norm, store, advance;
    NormRopeGeom nr;
    // request state
    int32_t B, W, bs_blk, pg, L, kind, nkv, hd, per_layer;
    const int32_t *ctx_len, *n_acc, *limit;
    const uint8_t *dummy, *row_valid;
    const int32_t *bt;
    int64_t bt_stride;
    int32_t bt_cols, num_pages;
    const int32_t *acc;
    int64_t acc_sr, acc_st;
    int32_t mask_id;
    // pools
    uint16_t *pk[DFKV_MAX_LAYERS];
    uint16_t *pv[DFKV_MAX_LAYERS];
    int64_t sp, ss, sh;
    // outputs
    int64_t *slot;
    uint8_t *wmask;
    int32_t *c_pos, *bonus, *emb, *q_pos, *ctx_out, *seq_len;
    int64_t *block_slot;   // [B][bs_blk] or null: placement of the next draft block
    const int32_t *row_req, *row_pos;   // row-wise store: each row's request and position
};
hipError_t launch_finalize(const FinalizeParams &p, hipStream_t s);
hipError_t launch_advance(const FinalizeParams &p, hipStream_t s);
hipError_t launch_store_rows(const FinalizeParams &p, hipStream_t s);   // p.M rows, every layer

// Strict acceptance of a uniform-width draft (k_misc.hip)
struct AcceptArgs {
    const int32_t *target;
    int64_t t_sr, t_st;
    const int32_t *draft;
    int64_t d_sr, d_st;
    int32_t B, W;
    int32_t *n_acc, *acc;
};
hipError_t launch_strict_accept(const AcceptArgs &a, hipStream_t s);

// Draft-KV block-table decode (k_misc.hip)
struct BtDecodeArgs {
    const int32_t *off;
    int64_t s_req, s_blk;
    const int32_t *n_tokens;
    int32_t B, max_blocks, page_size, divisor;
    int32_t *count, *table;
    int64_t t_stride;
};
hipError_t launch_bt_decode(const BtDecodeArgs &a, hipStream_t s);

// part != null: f = bf16(sum of the S fp32 partials [S][n_rows][H]) is formed and written first;
// packed: g in k_gemm_w's token order (gemm_pack_index), ceil(n_rows / 64) * 64 rows, padding zero
hipError_t launch_hidden_norm(uint16_t *f, const float *part, int S, const uint16_t *w, uint16_t *g, int n_rows,
                              int H, float eps, bool packed, hipStream_t s);
hipError_t launch_rope_cache(const dfkv_rope &r, float *cs, int cache_len, hipStream_t s);
// dst = src [rows][K] (rows and K multiples of 64) in the fragment order of gemm_pack_index
hipError_t launch_pack_rows(const uint16_t *src, uint16_t *dst, int64_t rows, int64_t K, hipStream_t s);
// Weight-streaming order of a [rows][cols] bf16 matrix (dfkv_pack_stream_weight): blocks of 16 rows
// x 128 columns; the (up to 8) blocks of one row group and 1024-column range side by side, those
// runs row group after row group, then the next 1024 columns; inside a block, the 16-byte pieces in
// the order the 64 lanes of a wave load them (load u of lane (q, c16) is row c16, columns
// (4u + q) * 8 .. + 8).  stream_block is the block of column block kb, row group ob (in 4 KB units).
__host__ __device__ inline int64_t stream_block(int64_t kb, int64_t ob, int64_t rows, int64_t cols) {
    const int64_t j = kb >> 3, left = (cols >> 7) - 8 * j, width = left < 8 ? left : 8;
    return j * 8 * (rows >> 4) + ob * width + (kb & 7);
}
__host__ __device__ inline int64_t stream_pack_index(int64_t o, int64_t k, int64_t rows, int64_t cols) {
    return stream_block(k >> 7, o >> 4, rows, cols) * 2048 +
           ((((k & 127) >> 5) * 64 + ((k & 31) >> 3) * 16 + (o & 15)) << 3) + (k & 7);
}
hipError_t launch_pack_stream(const uint16_t *src, uint16_t *dst, int64_t rows, int64_t cols, hipStream_t s);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);

// Weight-streaming projection GEMM (M <= 64 token rows).
constexpr int kMaxSplitK = 8192;    // largest k extent of one K/V split
constexpr int kStageChunks = 4;     // 16-byte chunks of f each of 512 threads stages
// Whether a K/V split of nbs k-blocks over M rows stages g = hidden_norm(f) in LDS (<= 32 KB).
inline bool stage_fits(int64_t M, int nbs) { return M <= 16 && M * nbs * 16 <= 512 * kStageChunks; }
struct StreamParams {
    const uint16_t *w;  // [O][K] weights: row-major, or (w_tiled) in the streaming order below
    int32_t w_tiled;    // w as dfkv_pack_stream_weight writes it
    const uint16_t *x;  // activation rows (row stride ldx): hidden for fc; f (staged) or g for the K/V GEMM
    int64_t ldx;
    int32_t M, K, O, S, nbs;  // nbs: 128-wide k-blocks per split
    uint16_t *out;            // fc: f [M][O] (S == 1), or NULL
    float *ss_out;            // fc: per 16-column tile sums of squares of f [O/16][M]
    const uint16_t *w_hn;     // K/V staging: hidden_norm weight [K]
    const float *ss_in;       // K/V staging: [T_in][M] sums of squares of f
    int32_t T_in;
    float eps;
    float *part;              // K/V: fp32 [S][M][O] partial sums (out == NULL)
};
hipError_t launch_stream(const StreamParams &p, hipStream_t s);

// K/V stage of the small-batch step (M <= 16 rows): hidden_norm + the stacked K/V GEMM as split-K
// groups (k_kvgroups), then the finalize (k_kvfinal) -- k_kvfin.hip.
constexpr int kKvMaxRows = 16;
constexpr int kKvBlockLane0 = 128;  // k_kvgroups group 0: first lane placing the next draft block
constexpr int kKvMaxBlockPositions = 512 - kKvBlockLane0;  // requests x block_size it can place
constexpr int kKvSlots = 512;    // resident workgroups of k_kvgroups: 2 per CU x 256 CUs
// Row/request bookkeeping left in the workspace by k_kvgroups for k_kvfinal (byte offsets):
// slot int64 [16], ctx / ctx_new / bonus int32 [16] each, then the rows' cos/sin values fp32 [16][rot].
constexpr int kKvBookCtx = 128, kKvBookCtxNew = 192, kKvBookBonus = 256, kKvBookCs = 384;
struct KvParams {
    StreamParams kv;          // the K/V GEMM: kv.S splits of kv.nbs k-blocks, g staged in LDS
    FinalizeParams fin;       // k_norm/RoPE, store, advance
    void *book;               // bookkeeping area of the workspace
    int32_t n_groups;         // kv.S splits x (O/16/ntg) tile groups
    int32_t groups;           // tile groups per split, n_groups / kv.S (set by launch_kv)
    int32_t ntg;              // tiles per group
    int32_t unit_cols;        // output columns per unit (head_dim for GQA, latent + rope for MLA)
    int32_t n_units;          // O / unit_cols
    int32_t fin_rows;         // rows per k_kvfinal workgroup (set by launch_kv)
};
hipError_t launch_kv(const KvParams &p, hipStream_t s);
size_t kv_book_bytes(int rot);

// 256 x 256-tile MFMA GEMM with an LDS ring fed by direct-to-LDS loads (k_gemm.hip):
// out = bf16(x . w^T), or with S > 1 splits of k, fp32 partial sums part[S][M][O].
struct GemmParams {
    const uint16_t *x;
    int64_t ldx;
    const uint16_t *w;
    uint16_t *out;
    int64_t ldo;
    float *part;
    int32_t M, K, O, S;
    int32_t w_packed;   // k_gemm: w is packed in fragment order over the features (gemm_pack_index)
};
hipError_t launch_gemm(const GemmParams &p, hipStream_t s);
int gemm_tiles(int M, int O);   // output tiles of launch_gemm (times S workgroups)
// K/V GEMM with 160-feature tiles (k_gemm_w): S = 1, bf16 out; gemm_w_rows(O) is 160 when O divides by it
hipError_t launch_gemm_w(const GemmParams &p, hipStream_t s);
int gemm_w_rows(int O);
// Token operand of k_gemm_w, packed in MFMA fragment order: element k of token n (K = 64 * iters)
// sits at gemm_pack_index(n, k, iters) (in bf16 elements).  Token n belongs to block b = n / 64,
// fragment j = (n / 32) % 2, lane row fr = n % 32; k to stage it = k / 64, where k % 64 = 32 fh +
// 8 s + e (lane half fh, MFMA slice s, element e); the 64 lanes (fr + 32 fh) of one (b, it, s, j)
// hold 1 KB in a row.  The buffer spans ceil(M / 64) * 64 tokens.
__host__ __device__ inline int64_t gemm_pack_index(int64_t n, int64_t k, int64_t iters) {
    const int64_t b = n >> 6, j = (n >> 5) & 1, fr = n & 31;
    const int64_t it = k >> 6, r = k & 63, fh = r >> 5, s = (r >> 3) & 3, e = r & 7;
    return ((((b * iters + it) * 4 + s) * 2 + j) * 64 + fr + 32 * fh) * 8 + e;
}

}  // namespace dfkv
