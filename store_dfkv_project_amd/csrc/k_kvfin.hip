// k_kvfin.hip -- the K/V stage of the small-batch step (M = B*W <= 16 token
// rows) in two launches: hidden_norm + the stacked K/V GEMM as split-K groups
// (k_kvgroups), then k_norm / RoPE, kv_out, the paged store into every layer's
// pool and the per-request advance (k_kvfinal).
//
// Sources (page titles and sections): TensorRT-LLM PR #20550 "fuse the
// decode-step drafter bookkeeping into Triton kernels", sections
// TLLM_DFLASH_OVERLAP_CONTEXT_PROJECTION (fc + hidden_norm + latent GEMM +
// RMSNorm/RoPE) and TLLM_DFLASH_FUSED_PROLOGUE (mask, clamp, page lookup, write
// to every layer, advance); TensorRT-LLM PR #13995 "DFlash performance
// optimizations" (one GEMM stacked across layers; fused cross-layer k_norm; one
// cos/sin cache for context and query).
//
// Input: f = bf16(hidden . w_fc^T) and its per-16-column sums of squares, left in
// the workspace by the fc kernel (k_stream) that runs before these.
//
// k_kvgroups: S splits of the K/V GEMM's k range times groups of ntg 16-feature
// tiles (interleaved: group g of G takes tiles g, g + G, ...); one workgroup per
// (split, group), all of them resident at
// once (the group count is chosen to fit the chip's workgroup slots), each with
// the same amount of weights to stream.  A group stages g = hidden_norm(f) for
// its split in LDS once, streams its tiles' weights through a ring of
// registers, and writes each tile's fp32 partial sums.  Group 0 also gathers,
// while it streams, everything the finalize needs of the rows and requests
// (destination slot, cos/sin values, advance outputs) into the workspace, so
// that no dependent load sits on the step's tail.
//
// k_kvfinal: one workgroup per unit -- a GQA K or V head, or an MLA layer's
// latent + rope -- and block of rows: one round of loads straight into registers
// (each lane's chunks of the split partials, their k_norm weights and cos/sin
// values, the row's slot), then the per-head arithmetic (the rounding points of
// knorm_rope_head in finalize_common.hpp) into kv_out and the pools; one more
// workgroup writes the bookkeeping outputs.  Measured on MI355X, this is faster
// than finalizing inside the GEMM kernel by the last arriving group: there every
// dependent hop (store drain, arrival atomic, partial loads) waited behind the
// weight stream.
#include "finalize_common.hpp"

namespace dfkv {

constexpr int kKvWaves = 8;
constexpr int kKvThreads = kKvWaves * 64;
// Waves per SIMD of k_kvgroups (4: <= 128 VGPRs, two workgroups per CU; overridable when building).
#ifndef DFKV_KV_WPE
#define DFKV_KV_WPE 4
#endif
constexpr int kKvWPE = DFKV_KV_WPE;
constexpr int kKvStatMax = 8;   // row statistics per lane held in registers (hidden <= 8192)

// Row and request bookkeeping group 0 leaves in the workspace for the finalize kernel.
__device__ __forceinline__ int64_t *book_slot(void *b) { return (int64_t *)b; }
__device__ __forceinline__ int32_t *book_ctx(void *b) { return (int32_t *)((char *)b + kKvBookCtx); }
__device__ __forceinline__ int32_t *book_ctx_new(void *b) { return (int32_t *)((char *)b + kKvBookCtxNew); }
__device__ __forceinline__ int32_t *book_bonus(void *b) { return (int32_t *)((char *)b + kKvBookBonus); }
__device__ __forceinline__ float *book_cs(void *b) { return (float *)((char *)b + kKvBookCs); }

// ---------------------------------------------------------------------------
// k_kvfinal: one workgroup per unit
// ---------------------------------------------------------------------------

// The bookkeeping outputs from what k_kvgroups' group 0 left in the workspace (slot, write mask,
// context positions; bonus, embedding ids, query positions, advanced ctx_len, seq_len): one hop of
// loads, then the stores.  A workgroup of its own, so that this hop runs beside the units' work
// instead of after it.
__device__ __forceinline__ void kvfinal_bookkeeping(const FinalizeParams &p, void *book) {
    const int tid = threadIdx.x, Mall = p.M;
    // every load first (one round), then the stores: rows (slot, context position; tid < M <= 16),
    // block positions (embedding id, query position; tid < B*block_size <= 384), requests (tid < B)
    const int32_t *ctx = book_ctx(book), *ctx_new = book_ctx_new(book), *bonus = book_bonus(book);
    const bool row = tid < Mall, blk = p.advance && tid < p.B * p.bs_blk, req = p.advance && tid < p.B;
    const int rr = row ? tid / p.W : 0, ri = row ? tid - rr * p.W : 0;
    const int br = blk ? tid / p.bs_blk : 0, bj = blk ? tid - br * p.bs_blk : 0;
    const int64_t slot = row && p.store ? book_slot(book)[tid] : -1;
    const int32_t c = row && p.advance ? ctx[rr] : 0;
    const int32_t b_bonus = blk ? bonus[br] : 0, b_cn = blk ? ctx_new[br] : 0;
    const int32_t r_bonus = req ? bonus[tid] : 0, r_cn = req ? ctx_new[tid] : 0;
    if (row && p.store) {
        p.slot[tid] = slot;
        p.wmask[tid] = slot >= 0 ? 1 : 0;
    }
    if (row && p.advance) p.c_pos[tid] = (int32_t)((int64_t)c + ri);
    if (blk) {
        p.emb[tid] = bj == 0 ? b_bonus : p.mask_id;
        p.q_pos[tid] = b_cn + bj;
    }
    if (req) {
        p.bonus[tid] = r_bonus;
        p.ctx_out[tid] = r_cn;
        p.seq_len[tid] = r_cn + p.bs_blk;
    }
}

// Unit u (a GQA K or V head: columns [u*hd, (u+1)*hd); an MLA layer: latent + rope) for the rows
// [n0, n0 + fin_rows): GQA rows 512/hd to a wave, MLA rows two waves each (below).
__global__ __launch_bounds__(kKvThreads) void k_kvfinal(const KvParams kp) {
    const FinalizeParams &p = kp.fin;
    // Kernel arguments are read through the scalar cache, which starts cold in every kernel, and the
    // compiler reads a field where the code first needs it: each such place is a round trip of its
    // own before the first data load (eight here).  Naming the fields the unit path needs in empty asm
    // statements makes them live in scalar registers at this point, so that their loads go out
    // together with one wait (measured on MI355X: 0.35 us per step, dense drafter at 4 rows).
    asm volatile("" ::"s"(p.M), "s"(kp.fin_rows), "s"(p.L), "s"(p.O), "s"(p.S), "s"(kp.unit_cols),
                 "s"(p.kind), "s"(p.nkv), "s"(p.per_layer), "s"(p.norm), "s"(p.nr.rope_dim), "s"(p.nr.latent),
                 "s"(p.store), "s"(p.pg));
    asm volatile("" ::"s"(kp.book), "s"(p.nr.w_knorm), "s"(p.part), "s"(p.kv_out), "s"(p.sp), "s"(p.ss), "s"(p.sh),
                 "s"(p.nr.eps));
    // grid (row block, unit of the layer, layer), plus the slice z = L whose first workgroup writes the
    // bookkeeping outputs (the others of that slice have nothing to do)
    if ((int)blockIdx.z == p.L) {
        if (blockIdx.x == 0 && blockIdx.y == 0) kvfinal_bookkeeping(p, kp.book);
        return;
    }
    const bool gqa = p.kind == DFKV_GQA;
    const int u = gqa ? (int)blockIdx.z * 2 * p.nkv + (int)blockIdx.y : (int)blockIdx.z, rb = (int)blockIdx.x;
    const int n0 = rb * kp.fin_rows;
    const int M = p.M - n0 < kp.fin_rows ? p.M - n0 : kp.fin_rows;  // rows of this workgroup
    const int Mall = p.M, O = p.O, S = p.S;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int cols = kp.unit_cols;
    const int l = (int)blockIdx.z;
    const int rem = gqa ? (int)blockIdx.y : 0;
    const bool is_v = gqa && rem >= p.nkv;
    const int h = is_v ? rem - p.nkv : rem;
    const int64_t col0 = gqa ? (int64_t)u * cols : (int64_t)l * p.per_layer;
    const bool norm = p.norm && !is_v;
    const int rot = p.nr.rope_dim;
    const int nwk = gqa ? cols : p.nr.latent;
    void *book = kp.book;

    if (gqa) {
        // GQA: every lane takes one 16-byte chunk of a head of one row (hd/8 lanes per row, 512/hd rows
        // per wave).  One round of loads straight into registers -- the chunk's split partials, its
        // k_norm weights, its cos/sin values and the row's slot -- then, in registers, the arithmetic
        // of knorm_rope_head (u = bf16(w y / rms), k = bf16(u c -/+ u' s) with the NeoX partner u' of
        // the other half of the head; the head's sum of squares over its lanes by the first DPP
        // steps of wave_sum, which give the same bits as wave_sum over the head alone), then the
        // stores.  No LDS and no barrier: measured on MI355X, 1.1 us off the dense drafter's K/V stage
        // at 4 rows (the MLA rows below, a whole wave each with two or three chunks per lane, were
        // 1 us slower this way).
        const int hd = cols, hq = hd >> 4;
        const int lgl = __builtin_ctz((unsigned)hd) - 3;                 // log2(lanes per row)
        const int lpr = 1 << lgl, li = lane & (lpr - 1);
        if ((wave << (6 - lgl)) >= M) return;                             // a wave with no row
        const int n = (wave << (6 - lgl)) + (lane >> lgl);                // row inside the block
        const bool rowok = n < M;
        const int64_t row = n0 + (rowok ? n : 0);
        // loads: the row's slot, the chunk's k_norm weights and cos/sin values, its split partials
        const int64_t slot = rowok && p.store ? book_slot(book)[row] : -1;
        const u32x4 wv = norm ? *(const u32x4 *)(p.nr.w_knorm + (int64_t)l * nwk + 8 * li) : u32x4{0u, 0u, 0u, 0u};
        const bool first = li < hq;
        const int j0 = (first ? li : li - hq) * 8;
        const f32x4 *cp = (const f32x4 *)(book_cs(book) + row * rot + j0);
        f32x4 cv[2], sv[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            cv[k] = norm && rowok ? cp[k] : f32x4{0.f, 0.f, 0.f, 0.f};
            sv[k] = norm && rowok ? cp[(rot >> 3) + k] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // the chunk's 8 split partial sums, added in split order (SB splits per round of loads)
        constexpr int SB = 8;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const float *src = p.part + row * O + col0 + 8 * li;
        for (int s0 = 0; s0 < S; s0 += SB) {
            f32x4 lo[SB], hi[SB];
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                const bool ld = rowok && s0 + k < S;
                const f32x4 *q = (const f32x4 *)(src + (int64_t)(s0 + k) * Mall * O);
                lo[k] = ld ? q[0] : f32x4{0.f, 0.f, 0.f, 0.f};
                hi[k] = ld ? q[1] : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                if (s0 + k >= S) break;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[e] += lo[k][e];
                    acc[4 + e] += hi[k][e];
                }
            }
        }
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = pack2(acc[2 * e], acc[2 * e + 1]);
        if (norm) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += bf_lo(v[e]) * bf_lo(v[e]) + bf_hi(v[e]) * bf_hi(v[e]);
            // the head's sum over its lpr lanes: quads, then 8, 16 and 32 lanes
            ss = dpp_add<0xB1>(ss);
            ss = dpp_add<0x4E>(ss);
            if (lpr == 8) ss += __shfl_xor(ss, 4, kWave);
            if (lpr >= 16) {
                ss = dpp_add<0x124>(ss);
                ss = dpp_add<0x128>(ss);
            }
            if (lpr == 32) ss += __shfl_xor(ss, 16, kWave);
            const float rinv = __builtin_amdgcn_rsqf(ss * (1.0f / (float)hd) + p.nr.eps);
            u32x4 w, pw;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = pack2(bf_lo(wv[e]) * (bf_lo(v[e]) * rinv), bf_hi(wv[e]) * (bf_hi(v[e]) * rinv));
            // RoPE (NeoX): the partner chunk is hq lanes away, inside the row's lanes
#pragma unroll
            for (int e = 0; e < 4; ++e) pw[e] = (uint32_t)__shfl_xor((int)w[e], hq, kWave);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float ul = bf_lo(w[e]), uh = bf_hi(w[e]), pl = bf_lo(pw[e]), ph = bf_hi(pw[e]);
                const float cl = cv[e >> 1][2 * (e & 1)], ch = cv[e >> 1][2 * (e & 1) + 1];
                const float sl = sv[e >> 1][2 * (e & 1)], sh = sv[e >> 1][2 * (e & 1) + 1];
                v[e] = first ? pack2(ul * cl - pl * sl, uh * ch - ph * sh) : pack2(ul * cl + pl * sl, uh * ch + ph * sh);
            }
        }
        if (rowok) {
            if (p.kv_out) *(u32x4 *)(p.kv_out + row * O + col0 + 8 * li) = v;
            if (slot >= 0)
                *(u32x4 *)((is_v ? p.pv[l] : p.pk[l]) + slot_offset(p, slot) + (int64_t)h * p.sh + 8 * li) = v;
        }
        return;
    }

    // MLA: two waves per row -- one for the latent (lane c holds latent chunks c and c + 64), one for the
    // rope part (lanes < P/8) -- each with one round of loads straight into registers, then the latent
    // norm by a wave sum, or the rope part's rotation, and the stores (no LDS, no barrier).
    {
        const int R = p.nr.latent, qr = R >> 3, qp = rot >> 3;
        if ((wave >> 1) >= M) return;                                   // a wave with no row
        const bool latent = (wave & 1) == 0;
        const int64_t row = n0 + (wave >> 1);
        const int64_t slot = p.store ? book_slot(book)[row] : -1;
        uint16_t *d = slot >= 0 ? p.pk[l] + slot_offset(p, slot) : nullptr;
        uint16_t *out = p.kv_out ? p.kv_out + row * O + col0 : nullptr;
        // chunks of this lane: latent c = lane, lane + 64 (R <= 1024); rope part c = qr + lane
        int64_t cc[2];
        bool ok[2];
        if (latent) {
            cc[0] = lane; cc[1] = lane + 64;
            ok[0] = lane < qr; ok[1] = lane + 64 < qr;
        } else {
            cc[0] = qr + lane; cc[1] = 0;
            ok[0] = lane < qp; ok[1] = false;
        }
        u32x4 wv[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
        f32x4 cv[2], sv[2];
        if (latent) {
#pragma unroll
            for (int k = 0; k < 2; ++k)
                if (norm && ok[k]) wv[k] = *(const u32x4 *)(p.nr.w_knorm + (int64_t)l * nwk + 8 * cc[k]);
        }
        const int hq = rot >> 4;
        const bool first = lane < hq;
        {
            const int j0 = (first ? lane : lane - hq) * 8;
            const f32x4 *cp = (const f32x4 *)(book_cs(book) + row * rot + (j0 < (rot >> 1) ? j0 : 0));
            const bool ld = !latent && norm && lane < qp;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                cv[k] = ld ? cp[k] : f32x4{0.f, 0.f, 0.f, 0.f};
                sv[k] = ld ? cp[(rot >> 3) + k] : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        // the chunks' split partials, added in split order (SB splits per round of loads)
        constexpr int SB = 8;
        float acc[2][8];
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
        const float *src = p.part + row * O + col0;
        for (int s0 = 0; s0 < S; s0 += SB) {
            f32x4 lo[2][SB], hi[2][SB];
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int j = 0; j < SB; ++j) {
                    const bool ld = ok[k] && s0 + j < S;
                    const f32x4 *q = (const f32x4 *)(src + (int64_t)(s0 + j) * Mall * O + 8 * cc[k]);
                    lo[k][j] = ld ? q[0] : f32x4{0.f, 0.f, 0.f, 0.f};
                    hi[k][j] = ld ? q[1] : f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int j = 0; j < SB; ++j) {
                    if (s0 + j >= S) break;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[k][e] += lo[k][j][e];
                        acc[k][4 + e] += hi[k][j][e];
                    }
                }
        }
        u32x4 v[2];
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[k][e] = pack2(acc[k][2 * e], acc[k][2 * e + 1]);
        if (latent) {
            // rinv over both chunks of every lane (zeros where there is none)
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) ss += bf_lo(v[k][e]) * bf_lo(v[k][e]) + bf_hi(v[k][e]) * bf_hi(v[k][e]);
            if (norm) {
                ss = wave_sum(ss);
                const float rinv = __builtin_amdgcn_rsqf(ss * (1.0f / (float)R) + p.nr.eps);
#pragma unroll
                for (int k = 0; k < 2; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[k][e] = pack2(bf_lo(wv[k][e]) * (bf_lo(v[k][e]) * rinv), bf_hi(wv[k][e]) * (bf_hi(v[k][e]) * rinv));
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                if (!ok[k]) continue;
                if (out) *(u32x4 *)(out + 8 * cc[k]) = v[k];
                if (d) *(u32x4 *)(d + 8 * cc[k]) = v[k];
            }
        } else {
            // the rope part, rotated without a norm (NeoX: the partner chunk is hq lanes away)
            if (norm) {
                u32x4 pw;
#pragma unroll
                for (int e = 0; e < 4; ++e) pw[e] = (uint32_t)__shfl_xor((int)v[0][e], hq, kWave);
                if (lane < 2 * hq) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float ul = bf_lo(v[0][e]), uh = bf_hi(v[0][e]), pl = bf_lo(pw[e]), ph = bf_hi(pw[e]);
                        const float cl = cv[e >> 1][2 * (e & 1)], ch = cv[e >> 1][2 * (e & 1) + 1];
                        const float sl = sv[e >> 1][2 * (e & 1)], sh = sv[e >> 1][2 * (e & 1) + 1];
                        v[0][e] = first ? pack2(ul * cl - pl * sl, uh * ch - ph * sh)
                                        : pack2(ul * cl + pl * sl, uh * ch + ph * sh);
                    }
                }
            }
            if (ok[0]) {
                if (out) *(u32x4 *)(out + 8 * cc[0]) = v[0];
                if (d) *(u32x4 *)(d + 8 * cc[0]) = v[0];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// k_kvgroups: one workgroup per (split, tile group)
// ---------------------------------------------------------------------------

// Group (s, g): split s of the K/V GEMM (k-blocks [s*nbs, (s+1)*nbs), nbs a multiple of the wave
// count, so every wave takes nbs/8 blocks of every tile) over tiles g, g + G, ..., g + (ntg-1)*G
// (G groups per split), so that the groups of a split stream neighbouring tiles at the same time
// (with a tiled weight, G adjacent 4 KB blocks of each k-block).  Same per-tile
// arithmetic as the staged K/V GEMM of stream_core.hpp: waves interleave the split's blocks, their
// sums are added in wave order.
// The staging hop's loads are issued before the weight ring, so that g is ready while the ring is in
// flight (measured on MI355X against the ring first: MLA drafter at 4 rows, K/V stage 0.65 us
// shorter; dense drafter at 4 rows, step 0.2 us shorter).
// D: weight k-blocks in flight per wave.  With two groups per CU one is enough -- 16 waves keep
// 64 KB per CU in flight, and a deeper ring only queues in front of the other group's staging hop
// (measured: dense drafter at 4 rows, 38.1 us per step with 3, 37.5 with 2, 37.4 with 1); with one
// group per CU two (MLA drafter at 4 rows, K/V stage 11.5 us with 2 or 3, 11.8 with 1).
template <int D>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(kKvWPE, 8))) void k_kvgroups(
    const KvParams kp) {
    constexpr int WAVES = kKvWaves, NT = kKvThreads, NP = 17;
    __shared__ float red[2 * kKvWaves * 16 * 17];
    __shared__ float sh_rinv[16];
    extern __shared__ __attribute__((aligned(16))) uint16_t sh_g[];  // g [M][kc + 8]
    const StreamParams &p = kp.kv;
    const FinalizeParams &fin = kp.fin;
    // the kernel arguments of the main path in one round of scalar loads (see k_kvfinal)
    asm volatile("" ::"s"(kp.ntg), "s"(kp.groups), "s"(p.M), "s"(p.nbs), "s"(p.K), "s"(p.O), "s"(p.w_tiled), "s"(p.ldx), "s"(p.T_in),
                 "s"(p.eps), "s"(fin.norm), "s"(fin.store), "s"(fin.advance), "s"(p.w), "s"(p.x), "s"(p.w_hn),
                 "s"(p.ss_in), "s"(p.part));
    // grid (group of the split, split): group t0 of split s takes tiles t0 + i*groups
    const int groups = kp.groups, s = (int)blockIdx.y, t0 = (int)blockIdx.x;
    // group 0 gathers the rows' and requests' fields, but only for a call that uses them: an
    // unfused projection (no norm, store or advance) may pass no ctx_len_in at all
    const bool book = blockIdx.x == 0 && blockIdx.y == 0 && (fin.norm || fin.store || fin.advance);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q = lane >> 4, c16 = lane & 15;
    const int M = p.M, ntg = kp.ntg;
    const int kb0 = s * p.nbs, kc = p.nbs * 128, ldg = kc + 8;
    const int nbw = p.nbs / WAVES;      // blocks per wave per tile (the same for every wave)
    const int total = ntg * nbw;        // this wave's blocks over the group
    const float rnbw = 1.0f / (float)nbw;

    u32x4 a[D][4];
    // this lane's 16-byte piece u of k-block kb of tile t = t0 + i*groups: row t*16 + c16, columns
    // kb*128 + (4u + q)*8 of a row-major weight; piece u*64 + q*16 + c16 of block stream_block(kb, t)
    // of a tiled one
    const uint16_t *wl = p.w_tiled ? p.w + (q * 16 + c16) * 8 : p.w + (int64_t)(t0 * 16 + c16) * p.K + q * 8;
    const int w_u = p.w_tiled ? 512 : 32;
    auto load = [&](int slot, int f) {
        const int i = div_small(f, rnbw), j = f - i * nbw;
        const int64_t kb = kb0 + wave + j * WAVES;
        const uint16_t *wp = p.w_tiled ? wl + stream_block(kb, t0 + (int64_t)i * groups, p.O, p.K) * 2048
                                       : wl + (int64_t)i * groups * 16 * p.K + kb * 128;
#pragma unroll
        for (int u = 0; u < 4; ++u) a[slot][u] = load_streamed(wp + u * w_u);
    };
    // Staging hop: the row statistics and f, w_hn for g, then the ring's first D blocks (a wave
    // with fewer blocks reloads its last one: never consumed); in group 0, with them, the rows' and
    // requests' fields (wave 0 lanes: row tid; wave 1 lanes: request tid - 64).  With at most 8
    // rows and T_in <= 64 * kKvStatMax, wave w takes row w's statistics in one round (a loop that
    // waited load by load put four to seven dependent round trips behind the ring).  The statistics
    // and the ring are loaded unconditionally, with clamped addresses, and so is every use of the
    // statistics: a conditional load or use lets the compiler sink the load into a branch or wait on
    // it early.  The staging chunks past the M rows are skipped instead (each costs the CU's memory
    // pipeline as much as a ring block: measured 0.15 - 0.3 us more per step when they were loaded).
    const bool stat_regs = M <= WAVES && p.T_in <= 64 * kKvStatMax;
    float sst[kKvStatMax];
    {
        const int n_ld = wave < M ? wave : M - 1;
#pragma unroll
        for (int i = 0; i < kKvStatMax; ++i) {
            const int tt = lane + 64 * i;
            sst[i] = p.ss_in[(int64_t)(tt < p.T_in ? tt : p.T_in - 1) * M + n_ld];
        }
    }
    const int c8n = kc >> 3;
    const float rc8n = 1.0f / (float)c8n;
    u32x4 fv[kStageChunks], wv[kStageChunks];
#pragma unroll
    for (int i = 0; i < kStageChunks; ++i) {
        const int idx = tid + i * NT;
        if (idx < M * c8n) {
            const int n = div_small(idx, rc8n), c8 = idx - n * c8n;
            const int64_t kk = (int64_t)kb0 * 128 + (c8 << 3);
            fv[i] = *(const u32x4 *)(p.x + (int64_t)n * p.ldx + kk);
            wv[i] = *(const u32x4 *)(p.w_hn + kk);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) load(d, d < total ? d : total - 1);
    // (block lanes, from 128: one per position of the next draft block of each request)
    const bool row_lane = book && tid < M, req_lane = book && tid >= 64 && tid - 64 < fin.B;
    const bool blk_lane = book && fin.advance && fin.block_slot && tid >= kKvBlockLane0 &&
                          tid - kKvBlockLane0 < fin.B * fin.bs_blk;
    const int rr = row_lane ? tid / fin.W
                            : (req_lane ? tid - 64 : (blk_lane ? (tid - kKvBlockLane0) / fin.bs_blk : 0));
    const int ri = row_lane ? tid - rr * fin.W : 0;
    const int bj = blk_lane ? tid - kKvBlockLane0 - rr * fin.bs_blk : 0;
    int32_t c = 0, n_acc = 0, lim = 0;
    uint8_t dmy = 0, rv = 1;
    if (row_lane || req_lane || blk_lane) {
        c = fin.nr.ctx_len_in[rr];
        if (fin.store || fin.advance) {
            n_acc = fin.n_acc[rr];
            lim = fin.limit[rr];
            dmy = fin.dummy[rr];
        }
        if (row_lane && fin.store && fin.row_valid) rv = fin.row_valid[tid];
    }
    // rinv[n] = 1/sqrt(mean(f[n]^2) + eps), fixed order: lane l adds tt = l, l + 64, ... of row n
    // (from the registers above, else a loop).
    float ssr = 0.f;
#pragma unroll
    for (int i = 0; i < kKvStatMax; ++i) ssr += lane + 64 * i < p.T_in ? sst[i] : 0.f;
    ssr = wave_sum(ssr);
    if (stat_regs) {
        if (lane == 0 && wave < M) sh_rinv[wave] = 1.0f / sqrtf(ssr / (float)p.K + p.eps);
    } else {
        for (int n = wave; n < M; n += WAVES) {
            float ss = 0.f;
            for (int tt = lane; tt < p.T_in; tt += 64) ss += p.ss_in[(int64_t)tt * M + n];
            ss = wave_sum(ss);
            if (lane == 0) sh_rinv[n] = 1.0f / sqrtf(ss / (float)p.K + p.eps);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kStageChunks; ++i) {
        const int idx = tid + i * NT;
        if (idx < M * c8n) {
            const int n = div_small(idx, rc8n), c8 = idx - n * c8n;
            const float rinv = sh_rinv[n];
            u32x4 gv;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                gv[e] = pack2(bf_lo(wv[i][e]) * (bf_lo(fv[i][e]) * rinv), bf_hi(wv[i][e]) * (bf_hi(fv[i][e]) * rinv));
            *(u32x4 *)(sh_g + n * ldg + (c8 << 3)) = gv;
        }
    }
    // Group 0's second hop, issued now and stored only after the GEMM: the row's block-table entry
    // (when it passes the write predicate), the request's bonus token, the rows' cos/sin values.
    int64_t pos = 0, pidx = 0;
    bool wr = false;
    int32_t page = -1, bonus = 0;
    if (row_lane && fin.store) {
        wr = row_write_pred(fin, c, n_acc, lim, dmy, rv, ri, pos, pidx);
        if (wr) page = fin.bt[(int64_t)rr * fin.bt_stride + pidx];
    }
    if (req_lane && fin.advance) {
        const int nb = n_acc < 1 ? 1 : (n_acc > fin.W ? fin.W : n_acc);
        bonus = fin.acc[(int64_t)rr * fin.acc_sr + (int64_t)(nb - 1) * fin.acc_st];
    }
    int64_t bpos = 0, bpidx = 0;
    int32_t bpage = -1;
    bool bok = false;
    if (blk_lane) {
        const int64_t adv = (int64_t)c + n_acc;
        const int32_t cn = dmy ? 0 : (int32_t)(adv < (int64_t)lim ? adv : (int64_t)lim);
        bok = block_position_ok(fin, cn, lim, dmy != 0, bj, bpos, bpidx);
        if (bok) bpage = fin.bt[(int64_t)rr * fin.bt_stride + bpidx];
    }
    __syncthreads();
    constexpr int CSN = kKvMaxRows * 256 / kKvThreads;  // cos/sin values per thread, at most
    float csv[CSN];
    const int rot = fin.nr.rope_dim;
    if (book && fin.norm) {
        // the rows' positions, for the cos/sin rows (ctx from row lanes, through LDS)
        int *sh_pos = (int *)sh_rinv;   // sh_rinv is free again: g is staged
        if (row_lane) {
            const int64_t cp = (int64_t)c + ri;
            sh_pos[tid] = (int)(cp < 0 ? 0 : (cp > fin.nr.cache_len - 1 ? fin.nr.cache_len - 1 : cp));
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < CSN; ++k) {
            const int e = tid + k * NT;
            csv[k] = e < M * rot ? fin.nr.cos_sin[(int64_t)sh_pos[e / rot] * rot + (e - (e / rot) * rot)] : 0.f;
        }
    }

    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int f0 = 0; f0 < total; f0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int f = f0 + d;
            if (f >= total) break;
            const int i = div_small(f, rnbw), j = f - i * nbw;
            const int kl = (wave + j * WAVES) * 128;  // k offset inside the split
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const u32x4 v = c16 < M ? *(const u32x4 *)(sh_g + c16 * ldg + kl + (u * 4 + q) * 8)
                                        : u32x4{0u, 0u, 0u, 0u};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[d][u]),
                                                              __builtin_bit_cast(bf16x8, v), acc, 0, 0, 0);
            }
            if (f + D < total) load(d, f + D);
            if (j == nbw - 1) {
                // tile i done: wave sums into red[i & 1], then the workgroup adds them in wave order
                float *rb = red + (i & 1) * (WAVES * 16 * NP);
#pragma unroll
                for (int v = 0; v < 4; ++v) rb[(wave * 16 + q * 4 + v) * NP + c16] = acc[v];
                acc = f32x4{0.f, 0.f, 0.f, 0.f};
                __syncthreads();
                const int t = t0 + i * groups;
                for (int idx = tid; idx < 16 * M; idx += NT) {
                    const int o = idx & 15, n = idx >> 4;
                    float y = 0.f;
#pragma unroll
                    for (int w = 0; w < WAVES; ++w) y += rb[(w * 16 + o) * NP + n];
                    p.part[((int64_t)s * M + n) * p.O + t * 16 + o] = y;
                }
            }
        }
    }

    if (!book) return;
    // group 0: what the finalize needs of the rows and requests
    void *bk = kp.book;
    if (row_lane)
        book_slot(bk)[tid] =
            (wr && page >= 0 && page < fin.num_pages) ? (int64_t)page * fin.pg + (pos - pidx * fin.pg) : -1;
    if (blk_lane) fin.block_slot[tid - kKvBlockLane0] = bok ? block_page_slot(fin, bpage, bpos, bpidx) : -1;
    if (req_lane) {
        const int64_t adv = (int64_t)c + n_acc;
        book_ctx(bk)[rr] = c;
        book_ctx_new(bk)[rr] = dmy ? 0 : (int32_t)(adv < (int64_t)lim ? adv : (int64_t)lim);
        book_bonus(bk)[rr] = bonus;
    }
    if (fin.norm) {
#pragma unroll
        for (int k = 0; k < CSN; ++k) {
            const int e = tid + k * NT;
            if (e < M * rot) book_cs(bk)[e] = csv[k];
        }
    }
}

size_t kv_book_bytes(int rot) { return (size_t)kKvBookCs + (size_t)kKvMaxRows * (size_t)rot * 4; }

hipError_t launch_kv(const KvParams &params, hipStream_t s) {
    if (params.fin.M <= 0) return hipSuccess;
    KvParams p = params;
    const int tpu = p.unit_cols / 16;
    // the shapes the kernels index by: g's staging chunks, the row bookkeeping, the cos/sin registers
    if (p.kv.nbs % kKvWaves != 0 || p.kv.nbs <= 0 || p.ntg <= 0 || p.ntg > tpu || p.n_groups % p.kv.S != 0 ||
        !stage_fits(p.kv.M, p.kv.nbs) || p.kv.M != p.fin.M || p.fin.M > kKvMaxRows || p.fin.B > kKvMaxRows ||
        p.fin.nr.rope_dim > 256)
        return hipErrorInvalidValue;
    const size_t M = (size_t)p.kv.M;
    const size_t g_bytes = M * (size_t)(p.kv.nbs * 128 + 8) * 2;
    const bool two_per_cu = p.n_groups > kKvSlots / 2;
    p.groups = p.n_groups / p.kv.S;
    hipError_t e = launch1(two_per_cu ? k_kvgroups<1> : k_kvgroups<2>, dim3((unsigned)p.groups, (unsigned)p.kv.S),
                           dim3(kKvThreads), s, p, g_bytes);
    if (e != hipSuccess) return e;
    // finalize: rows per workgroup -- each wave holds 512 / hd rows of a GQA head; an MLA row takes two
    // waves (latent, rope part)
    const int rows = p.fin.kind == DFKV_GQA ? kKvWaves * (512 / p.unit_cols) : kKvWaves / 2;
    p.fin_rows = rows;
    const unsigned nrb = (unsigned)((M + rows - 1) / rows);
    // grid (row block, unit of the layer, layer) and one more layer slice for the bookkeeping outputs
    const unsigned upl = (unsigned)(p.n_units / p.fin.L);
    if (upl * (unsigned)p.fin.L != (unsigned)p.n_units) return hipErrorInvalidValue;
    return launch1(k_kvfinal, dim3(nrb, upl, (unsigned)p.fin.L + 1), dim3(kKvThreads), s, p);
}

}  // namespace dfkv
