// k_gemm.hip -- bf16 MFMA GEMM for the projection at larger batch (M = B*W > 64
// rows), where the fc and stacked K/V GEMMs are bound by the matrix cores
// rather than by streaming the weights (TensorRT-LLM PR #13995 "DFlash
// performance optimizations", commit "fuse cross-layer k_norm": at bs=64 the
// GEMMs dominate the step).
//
//   out[n][o] = bf16( sum_k x[n][k] * w[o][k] )    (both operands K-contiguous)
//   or, split over k, fp32 partial sums part[s][n][o] that the consumer adds.
//
// Design for gfx950:
//  * a workgroup of 4 waves (one per SIMD, one workgroup per CU) computes a
//    256 (tokens) x 256 (features) tile; wave w takes all 256 tokens and
//    features 64 w .. +64: an 8 x 2 grid of v_mfma_f32_32x32x16_bf16
//    accumulators, 256 accumulation registers per lane.  When 256-token tiles
//    would leave most CUs idle, tiles are 128 tokens tall (a 4 x 2 grid): a GEMM
//    split over k to fill the chip then needs half the splits, and writes half
//    the fp32 partials (at 1024 x 12288 x 4096: 2 splits and 32 MB instead of 4
//    and 64 MB, the fc stage 108.5 -> 104.1 us; 4 splits of 128-token tiles, two
//    workgroups per CU, took 109.8 us, and 128-token tiles at 4096 rows, two
//    workgroups per CU, were slower than 256-token tiles, 345 against 328 us);
//  * what bounds a GEMM on this chip, short of the matrix cores, is LDS
//    bandwidth (measured: staging both operands of 64 x 128 wave tiles through
//    LDS took 63% of such a kernel's time in loads and fragment reads).  Here
//    only the token tile, which all 4 waves read, goes through LDS -- global ->
//    LDS directly (global_load_lds_dwordx4) into a ring of four 64-k slots of
//    32 KB, filled three stages ahead; each wave's weight fragments are its own
//    and go straight into registers, a slice's registers reloaded with the next
//    stage's slice as soon as its MFMAs are issued.  Per 64-k stage and CU:
//    128 KB of LDS fragment reads + 32 KB of LDS writes against 256 MFMAs;
//  * the token fragments of the next slice are read between the MFMAs of the
//    current one (order pinned with scheduling barriers), and the one barrier
//    per stage sits before its last slice, so the next stage's first fragments
//    are read while that slice multiplies;
//  * LDS rows hold 64 k (eight 16-byte chunks); chunk c of row r sits at
//    position c ^ ((r / 2) % 8), so the fragment reads of consecutive rows fall
//    on distinct banks;
//  * tiles are mapped so that the 32 workgroups of one XCD (workgroups are
//    dealt to the 8 XCDs round robin) cover a compact block of tiles, which
//    their shared L2 then serves;
//  * the epilogue goes through LDS so that every store is a 16-byte run;
//  * rows past M (tokens) or O (features) load row M-1 / O-1 instead (valid
//    memory, results discarded), so no load is ever out of bounds.
// Measured at M = 4096, K = 12288, O = 4096: about 1.1-1.2 PFLOP/s, as fast as
// the vendor BLAS on the same box (whose clock drops to about 1.9 GHz under a
// full MFMA load, where the 2.5 PFLOP/s peak assumes 2.4 GHz).
#include "dfkv_internal.hpp"

namespace dfkv {

constexpr int GBN = 256, GBK = 64;
constexpr int GTHREADS = 256;                    // 4 waves, one per SIMD
constexpr int GCPR = GBK / 8;                    // 16-byte chunks per LDS row
constexpr int GFN = GBN / 4 / 32;
constexpr int GNS = GBK / 16;                    // MFMA k slices per stage
constexpr int GEP = GBN + 8;                     // fp32 row stride of the epilogue tile in LDS
constexpr int GSLOTS = 4;                      // token-tile ring in LDS
constexpr int gemm_smem(int bm) { return GSLOTS * bm * GBK * 2 > 64 * GEP * 4 ? GSLOTS * bm * GBK * 2 : 64 * GEP * 4; }

typedef __attribute__((address_space(3))) void lds_void;

// LDS position of 16-byte chunk c of row r: c ^ swz(r).  Rows are 128 bytes; the reads of one
// fragment touch consecutive rows at the same chunk, which this spreads over the 64 banks.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Wave w computes all 256 tokens x features w*64 .. +64.  k is permuted inside each 64-wide stage so
// that a lane's weight fragment is 64 contiguous bytes: MFMA slice s, lane half h takes physical
// k = 32 h + 8 s + (0..7), for both operands, which leaves every dot product unchanged.
template <bool PACKED_W, int GBM>
__global__ __launch_bounds__(GTHREADS, 1) void k_gemm(const GemmParams pin) {
    constexpr int GA_STAGE = GBM * GBK * 2;          // token tile of one stage in LDS: 32 KB (16 KB)
    constexpr int GFM = GBM / 32;
    constexpr int GCPT = GBM * GCPR / GTHREADS;      // token-tile chunks per thread per stage (8 or 4)
    static_assert(GCPT == 8 || GCPT == 4, "the waits below are counted for 256- and 128-token tiles");
    __shared__ __attribute__((aligned(16))) uint8_t smem[gemm_smem(GBM)];

    // the kernel arguments in one round of scalar loads: a field read where the code first needs it
    // is a round trip of its own through the scalar cache, which starts cold in every kernel (the
    // sizes pass through the statement, so that no arithmetic on them starts before it)
    GemmParams p = pin;
    asm volatile("" : "+s"(p.M), "+s"(p.K), "+s"(p.O), "+s"(p.S) : "s"(p.x), "s"(p.ldx), "s"(p.w), "s"(p.out),
                 "s"(p.ldo), "s"(p.part));
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nx = (p.O + GBN - 1) / GBN, ny = (p.M + GBM - 1) / GBM;
    const int tiles = nx * ny;
    // the divisions by values known only at run time by div_small (every operand is below 2^21)
    const int split = div_small((int)blockIdx.x, 1.0f / (float)tiles);
    int t = (int)blockIdx.x - split * tiles;
    // XCD-aware order: when the tile count divides by 8, the tiles of XCD x (workgroups b with
    // b % 8 == x) become the consecutive logical tiles x*tiles/8 .. +tiles/8
    if (tiles % 8 == 0) t = (t % 8) * (tiles / 8) + t / 8;
    // logical tile -> (tm, tn) in bands of up to 4 token tiles, feature-major inside a band
    const int band = ny < 4 ? ny : 4;
    const int per_band = band * nx;
    const int b0 = div_small(t, 1.0f / (float)per_band), in_b = t - b0 * per_band;
    const int rows_b = (b0 + 1) * band <= ny ? band : ny - b0 * band;
    const int tn = div_small(in_b, 1.0f / (float)rows_b), tm = b0 * band + in_b - tn * rows_b;
    const int m0 = tm * GBM, o0 = tn * GBN;
    const int iters = p.K / GBK;
    const float rS = 1.0f / (float)p.S;
    const int it0 = div_small(split * iters, rS), it1 = div_small((split + 1) * iters, rS);
    const int fr = lane & 31, fh = lane >> 5;

    // token tile: this thread's chunks, chunk L = (i*4 + wave)*64 + lane -> row L/8, LDS position
    // L%8, global chunk (L%8) ^ swz(row)
    const uint16_t *asrc[GCPT];
#pragma unroll
    for (int i = 0; i < GCPT; ++i) {
        const int L = (i * 4 + wave) * 64 + lane, row = L >> 3, c = (L & 7) ^ swz(row);
        const int n = m0 + row < p.M ? m0 + row : p.M - 1;
        asrc[i] = p.x + (int64_t)n * p.ldx + c * 8;
    }
    auto issue_a = [&](int it) {
        uint8_t *base = smem + (it & (GSLOTS - 1)) * GA_STAGE;
        const int k0 = it * GBK;
#pragma unroll
        for (int i = 0; i < GCPT; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(asrc[i] + k0), (lds_void *)(base + (i * 4 + wave) * 1024),
                                             16, 0, 0);
    };
    // weight fragments: feature o0 + wave*64 + 32 j + fr, 16 bytes at physical k = k0 + 32 fh + 8 s.
    // Row-major weights: two rows per fragment load and lane pair.  Packed weights (gemm_pack_index
    // over the features): the 64 lanes' fragments of one (block, stage, slice, j) are 1 KB in a row.
    const uint16_t *bsrc[GFN];
    const uint8_t *bpk;
    if (PACKED_W) {
        const int nblk = (p.O + 63) >> 6;
        const int b = (o0 >> 6) + wave < nblk ? (o0 >> 6) + wave : nblk - 1;
        bpk = (const uint8_t *)p.w + ((int64_t)b * iters * 512 + lane) * 16;
    } else {
#pragma unroll
        for (int j = 0; j < GFN; ++j) {
            const int o = o0 + wave * 64 + 32 * j + fr;
            bsrc[j] = p.w + (int64_t)(o < p.O ? o : p.O - 1) * p.K + 32 * fh;
        }
    }
    // The weight loads are inline assembly, waited for by hand with the counts below: the compiler's
    // own wait insertion cannot follow them around the loop next to the loads into LDS and would wait
    // for every outstanding load before each slice.  A wait names the registers it guards, so no use
    // of them can move above it.
    u32x4 bw[GNS][GFN];
    auto load_b = [&](int it, int s) {
#pragma unroll
        for (int j = 0; j < GFN; ++j) {
            const void *src = PACKED_W ? (const void *)(bpk + (int64_t)((it * GNS + s) * GFN + j) * 1024)
                                       : (const void *)(bsrc[j] + it * GBK + 8 * s);
            asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(bw[s][j]) : "v"(src));
        }
    };
    static_assert(GFN == 2, "the waits name GFN registers per slice");
    // token fragments of slice s from LDS: row 32 i + fr, physical chunk 4 fh + s
    bf16x8 af[2][GFM];
    auto read_a = [&](const uint8_t *sa, int s, int set) {
#pragma unroll
        for (int i = 0; i < GFM; ++i) {
            const int r = 32 * i + fr;
            af[set][i] = *(const bf16x8 *)(sa + r * (GCPR * 16) + (((4 * fh + s) ^ swz(r)) << 4));
        }
    };
    auto slot = [&](int it) { return smem + (it & (GSLOTS - 1)) * GA_STAGE; };

    f32x16 acc[GFM][GFN];
#pragma unroll
    for (int i = 0; i < GFM; ++i)
#pragma unroll
        for (int j = 0; j < GFN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // Loads past the last stage are issued all the same (the wait counts assume them), for stage
    // it1-1 instead: the same bytes into the same slot, the same weights into unused registers.
    auto last = [&](int it) { return it < it1 ? it : it1 - 1; };

    // Per stage it each thread issues, in order: the weights of stage it+1, slices 0-2 (GFN loads
    // each, into the registers slice s of `it` has just used), the token tile of stage it+3 (GCPT),
    // the weights of stage it+1, slice 3.  Waiting for the weights of slice s of stage it (issued
    // one stage earlier) leaves 6 + GCPT later loads outstanding (14 for 256-token tiles, 10 for
    // 128).  Between slices 2 and 3 sits the stage boundary: the token tile of it+1 (issued two
    // stages earlier) has landed once at most 14 + GCPT later loads are outstanding (16 + GCPT in
    // steady state; the first stage has 14 + GCPT, and waiting for that many always only also
    // waits for the weights of slice 3, issued a stage ago); the barrier makes every
    // wave's part visible and proves every wave done reading the slot of stage it-1 (its last
    // fragments were read during slice 2 of it-1 and used by slice 3), which then takes stage
    // it+3; slice 0 of it+1 is read while slice 3 of `it` multiplies.
    auto stage = [&](int it) {
        const uint8_t *sa = slot(it);
        const int nb = last(it + 1);
#pragma unroll
        for (int s = 0; s < GNS; ++s) {
            if (s + 1 == GNS) {
                if constexpr (GCPT == 8) asm volatile("s_waitcnt vmcnt(22)" ::: "memory");
                else asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
                __builtin_amdgcn_s_barrier();
                issue_a(last(it + 3));
            }
            // the fragments of the next slice (slice 0 of it+1 after slice 3) are read between the
            // MFMAs of this one, into the other fragment set
            const uint8_t *rs = s + 1 < GNS ? sa : slot(it + 1);
            const int rsl = (s + 1) & (GNS - 1), rset = (s + 1) & 1;
            if constexpr (GCPT == 8) asm volatile("s_waitcnt vmcnt(14)" : "+v"(bw[s][0]), "+v"(bw[s][1]));
            else asm volatile("s_waitcnt vmcnt(10)" : "+v"(bw[s][0]), "+v"(bw[s][1]));
            __builtin_amdgcn_sched_barrier(0);
            // one fragment read after each of the first GFM MFMAs: the last read has the other half of
            // the slice's MFMAs to land in
#pragma unroll
            for (int m = 0; m < GFM * GFN; ++m) {
                const int i = m / GFN, j = m % GFN;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][i], __builtin_bit_cast(bf16x8, bw[s][j]),
                                                                    acc[i][j], 0, 0, 0);
                if (m < GFM) {
                    const int r = 32 * m + fr;
                    af[rset][m] = *(const bf16x8 *)(rs + r * (GCPR * 16) + (((4 * fh + rsl) ^ swz(r)) << 4));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            load_b(nb, s);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (it0 < it1) {
        // prologue: token tiles it0, it0+1; weights of it0, slices 0-2; token tile it0+2; weights of
        // it0, slice 3 -- the steady-state order.  Tile it0 has landed once 8 + 2 GCPT later loads
        // are outstanding.
        issue_a(it0);
        issue_a(last(it0 + 1));
#pragma unroll
        for (int s = 0; s < GNS - 1; ++s) load_b(it0, s);
        issue_a(last(it0 + 2));
        load_b(it0, GNS - 1);
        if constexpr (GCPT == 8) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        read_a(slot(it0), 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        for (int it = it0; it < it1; ++it) stage(it);
    }

    // Every load has landed before the epilogue: none into LDS may be in flight when the workgroup
    // ends, and the registers of the last (unused) weight loads must not be reused while they are.
#pragma unroll
    for (int s = 0; s < GNS; ++s) asm volatile("s_waitcnt vmcnt(0)" : "+v"(bw[s][0]), "+v"(bw[s][1]));

    // Epilogue through LDS, 64 tokens at a time: the waves write their accumulators as fp32 rows
    // (stride GEP floats: the two lane halves, 4 rows apart, then fall on different banks), then
    // all threads store whole 16-byte runs of a row.
    // D fragment of 32x32: lane holds column lane%32 (feature) and rows 8*(v/4) + 4*(lane/32) + v%4.
    __builtin_amdgcn_s_barrier();    // every wave is past its last fragment read
    float *ep = (float *)smem;
    const bool vec_out = p.part == nullptr && (p.ldo & 7) == 0 && (((uintptr_t)p.out) & 15) == 0;
    const bool vec_part = p.part != nullptr && (p.O & 3) == 0 && (((uintptr_t)p.part) & 15) == 0;
#pragma unroll
    for (int r = 0; r < GFM / 2; ++r) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int j = 0; j < GFN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = 32 * ii + ((v >> 2) << 3) + (fh << 2) + (v & 3);
                    ep[row * GEP + wave * 64 + 32 * j + fr] = acc[2 * r + ii][j][v];
                }
        __syncthreads();
        const int nr0 = m0 + 64 * r;
        if (p.part) {
            // fp32: 64 threads per row, 4 columns each
#pragma unroll
            for (int pass = 0; pass < 16; ++pass) {
                const int row = pass * 4 + (tid >> 6), c = (tid & 63) * 4;
                const int n = nr0 + row, o = o0 + c;
                if (n >= p.M) continue;
                const float *src = ep + row * GEP + c;
                float *dst = p.part + ((int64_t)split * p.M + n) * p.O + o;
                if (vec_part && o + 4 <= p.O) {
                    *(float4 *)dst = *(const float4 *)src;
                } else {
                    for (int e = 0; e < 4 && o + e < p.O; ++e) dst[e] = src[e];
                }
            }
        } else {
            // bf16: 32 threads per row, 8 columns each
#pragma unroll
            for (int pass = 0; pass < 8; ++pass) {
                const int row = pass * 8 + (tid >> 5), c = (tid & 31) * 8;
                const int n = nr0 + row, o = o0 + c;
                if (n >= p.M) continue;
                const float *src = ep + row * GEP + c;
                uint16_t *dst = p.out + (int64_t)n * p.ldo + o;
                if (vec_out && o + 8 <= p.O) {
                    const float4 lo = *(const float4 *)src, hi = *(const float4 *)(src + 4);
                    u32x4 pk;
                    pk[0] = (uint32_t)f2bf(lo.x) | ((uint32_t)f2bf(lo.y) << 16);
                    pk[1] = (uint32_t)f2bf(lo.z) | ((uint32_t)f2bf(lo.w) << 16);
                    pk[2] = (uint32_t)f2bf(hi.x) | ((uint32_t)f2bf(hi.y) << 16);
                    pk[3] = (uint32_t)f2bf(hi.z) | ((uint32_t)f2bf(hi.w) << 16);
                    *(u32x4 *)dst = pk;
                } else {
                    for (int e = 0; e < 8 && o + e < p.O; ++e) dst[e] = f2bf(src[e]);
                }
            }
        }
        __syncthreads();
    }
}

// Token tile height: 128 when 256-token tiles would leave most CUs idle (fewer than 192 tiles),
// which halves the k splits such a GEMM needs to fill the chip, and with them its fp32 partials.
static int gemm_bm(int M, int O) { return ((O + GBN - 1) / GBN) * ((M + 255) / 256) < 192 ? 128 : 256; }

int gemm_tiles(int M, int O) {
    const int bm = gemm_bm(M, O);
    return ((O + GBN - 1) / GBN) * ((M + bm - 1) / bm);
}

hipError_t launch_gemm(const GemmParams &p, hipStream_t s) {
    if (p.M <= 0) return hipSuccess;
    if (p.K % GBK != 0 || p.S < 1 || p.S > p.K / GBK || (p.S > 1 && !p.part) || (p.S == 1 && !p.part && !p.out))
        return hipErrorInvalidValue;
    const unsigned tiles = (unsigned)gemm_tiles(p.M, p.O);
    const bool small = gemm_bm(p.M, p.O) == 128;
    if (p.w_packed) {
        if (p.O % 64 != 0) return hipErrorInvalidValue;
        return launch1(small ? k_gemm<true, 128> : k_gemm<true, 256>, dim3(tiles * (unsigned)p.S), dim3(GTHREADS), s, p);
    }
    return launch1(small ? k_gemm<false, 128> : k_gemm<false, 256>, dim3(tiles * (unsigned)p.S), dim3(GTHREADS), s, p);
}

}  // namespace dfkv
