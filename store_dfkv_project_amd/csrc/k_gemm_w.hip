// k_gemm_w.hip -- bf16 MFMA GEMM for the stacked K/V projection at larger batch, with the
// weights as the shared operand: tiles of 32*FM features x 256 tokens.
//
//   out[n][o] = bf16( sum_k g[n][k] * w[o][k] )    (w K-contiguous, g packed by k_hidden_norm, S = 1)
//
// The stacked K/V output width of a dense drafter (layers x 2 x kv heads x head dim, e.g.
// 5 x 2 x 8 x 128 = 10240) divides by 160 but its tiles of 256 x 256 do not fill 256 CUs evenly
// (1024 rows: 160 tiles, 96 CUs idle; 4096 rows: 640 tiles, 2.5 rounds).  With 160-feature tiles
// the same GEMM has 256 tiles at 1024 rows and 1024 (four full rounds) at 4096.
//
// The same design as k_gemm with the operand roles exchanged: a workgroup of 4 waves (one per
// SIMD, one workgroup per CU); the weight tile (32*FM rows), read by all 4 waves, goes global ->
// LDS directly (global_load_lds_dwordx4) into a ring of four 64-k slots filled three stages
// ahead, rows XOR-swizzled; wave w owns tokens 64 w .. +64 of the tile, whose fragments are its own
// and load straight into registers one stage ahead (inline assembly with hand-counted
// s_waitcnt vmcnt); accumulators FM x 2 of v_mfma_f32_32x32x16_bf16 (16*FM*2 registers per
// lane).  Weight fragments of the next slice are read from LDS between the MFMAs of the current
// one; one barrier per stage, before its last slice.  The epilogue goes through LDS, 32 tokens
// per wave at a time, so every store is a 16-byte run.  The tokens come packed in fragment order
// (gemm_pack_index, written so by k_hidden_norm), so each of a wave's token loads reads 1 KB in a
// row instead of two 16-byte pieces of 32 rows; blocks of 64 tokens past the packed ones load the
// last block instead (valid memory, results discarded).  The feature count must divide by 32*FM.
#include "dfkv_internal.hpp"

namespace dfkv {

namespace {

constexpr int WTHREADS = 256;   // 4 waves, one per SIMD
constexpr int WBK = 64;         // k per stage
constexpr int WNS = WBK / 16;   // MFMA k slices per stage
constexpr int WSLOTS = 4;       // weight-tile ring in LDS
constexpr int WBM = 256;        // tokens per tile: 64 per wave

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int wswz(int r) { return (r >> 1) & 7; }

template <int FM>
struct WCfg {
    static constexpr int XR = 32 * FM;                // feature rows per tile
    static constexpr int STAGE = XR * WBK * 2;        // bytes of one weight slot
    static constexpr int CPT = XR * (WBK / 8) / WTHREADS;   // weight chunks per thread per stage
    static constexpr int EPS = XR + 4;                // fp32 row stride of the epilogue tile
    static constexpr int EPB = 32 * EPS * 4;          // epilogue bytes per wave (32 tokens)
    static constexpr int SMEM = WSLOTS * STAGE > 4 * EPB ? WSLOTS * STAGE : 4 * EPB;
    // loads per stage and thread: 8 token loads (4 slices x 2 fragments) + CPT weight chunks
    static constexpr int WAIT_Y = 6 + CPT;            // waiting for one slice's token fragments
    static constexpr int WAIT_X = 14 + CPT;           // waiting for the weight tile of the next stage
    static constexpr int WAIT_P = 8 + 2 * CPT;        // prologue: the first weight tile
    static_assert(XR * (WBK / 8) % WTHREADS == 0, "weight chunks must spread evenly over the threads");
};

}  // namespace

// k is permuted inside each 64-wide stage exactly as in k_gemm: MFMA slice s, lane half h takes
// physical k = 32 h + 8 s + (0..7) of both operands, so a lane's token fragment over a stage is 64
// contiguous bytes and every dot product is unchanged.
template <int FM, bool PACKED>
__global__ __launch_bounds__(WTHREADS, 1) void k_gemm_w(const GemmParams pin) {
    using C = WCfg<FM>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::SMEM];
    // the kernel arguments in one round of scalar loads (see k_gemm)
    GemmParams p = pin;
    asm volatile("" : "+s"(p.M), "+s"(p.K), "+s"(p.O) : "s"(p.x), "s"(p.ldx), "s"(p.w), "s"(p.out), "s"(p.ldo));

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nx = p.O / C::XR, ny = (p.M + WBM - 1) / WBM;
    const int tiles = nx * ny;
    int t = blockIdx.x;
    // XCD-aware order (workgroups are dealt to the 8 XCDs round robin): when the tile count divides
    // by 8, the tiles of XCD x become the consecutive logical tiles x*tiles/8 .. +tiles/8
    if (tiles % 8 == 0) t = (t % 8) * (tiles / 8) + t / 8;
    // logical tile -> (tm, tn) in bands of up to 4 token tiles, feature-major inside a band
    const int band = ny < 4 ? ny : 4;
    const int per_band = band * nx;
    const int b0 = div_small(t, 1.0f / (float)per_band), in_b = t - b0 * per_band;   // (operands < 2^21)
    const int rows_b = (b0 + 1) * band <= ny ? band : ny - b0 * band;
    const int tn = div_small(in_b, 1.0f / (float)rows_b), tm = b0 * band + in_b - tn * rows_b;
    const int n0 = tm * WBM, o0 = tn * C::XR;
    const int it0 = 0, it1 = p.K / WBK;
    const int fr = lane & 31, fh = lane >> 5;

    // weight tile: this thread's chunks, chunk L = (i*4 + wave)*64 + lane -> row L/8, LDS position
    // L%8, global chunk (L%8) ^ swz(row)
    const uint16_t *xsrc[C::CPT];
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
        const int L = (i * 4 + wave) * 64 + lane, row = L >> 3, c = (L & 7) ^ wswz(row);
        xsrc[i] = p.w + (int64_t)(o0 + row) * p.K + c * 8;
    }
    auto slot = [&](int it) { return smem + (it & (WSLOTS - 1)) * C::STAGE; };
    auto issue_x = [&](int it) {
        uint8_t *base = slot(it);
        const int k0 = it * WBK;
#pragma unroll
        for (int i = 0; i < C::CPT; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(xsrc[i] + k0), (lds_void *)(base + (i * 4 + wave) * 1024),
                                             16, 0, 0);
    };
    // token fragments: token n0 + wave*64 + 32 j + fr, 16 bytes at physical k = k0 + 32 fh + 8 s.
    // Row-major tokens: two rows per fragment load and lane pair.  Packed tokens (gemm_pack_index):
    // the 64 lanes' fragments of one (block, stage, slice, j) are 1 KB in a row.
    const uint16_t *ysrc[2];
    const uint8_t *ypk;
    if (PACKED) {
        const int nblk = (p.M + 63) >> 6;
        const int b = (n0 >> 6) + wave < nblk ? (n0 >> 6) + wave : nblk - 1;
        ypk = (const uint8_t *)p.x + ((int64_t)b * it1 * 512 + lane) * 16;
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wave * 64 + 32 * j + fr;
            ysrc[j] = p.x + (int64_t)(n < p.M ? n : p.M - 1) * p.ldx + 32 * fh;
        }
    }
    // The token loads are inline assembly, waited for by hand (see k_gemm): a wait names the
    // registers it guards, so no use of them can move above it.
    u32x4 ya[WNS][2];
    auto load_y = [&](int it, int s) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const void *src = PACKED ? (const void *)(ypk + (int64_t)((it * WNS + s) * 2 + j) * 1024)
                                     : (const void *)(ysrc[j] + it * WBK + 8 * s);
            asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(ya[s][j]) : "v"(src));
        }
    };
    // weight fragments of slice s from LDS: row 32 i + fr, physical chunk 4 fh + s
    bf16x8 wf[2][FM];
    auto read_w = [&](const uint8_t *sa, int s, int set) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int r = 32 * i + fr;
            wf[set][i] = *(const bf16x8 *)(sa + r * 128 + (((4 * fh + s) ^ wswz(r)) << 4));
        }
    };

    f32x16 acc[FM][2];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // Loads past the last stage are issued all the same (the wait counts assume them), for stage
    // it1-1 instead: the same bytes into the same slot, the same tokens into unused registers.
    auto last = [&](int it) { return it < it1 ? it : it1 - 1; };

    // Per stage it each thread issues, in order: the tokens of stage it+1, slices 0-2 (2 loads each,
    // into the registers slice s of `it` has just used), the weight tile of stage it+3 (CPT), the
    // tokens of stage it+1, slice 3.  Waiting for the tokens of slice s of stage it leaves 6 + CPT
    // later loads outstanding.  Before slice 3 sits the stage boundary: the weight tile of it+1 has
    // landed once at most 14 + CPT later loads are outstanding (16 + CPT in steady state), and the
    // barrier makes every wave's part visible and proves every wave done reading the slot of stage
    // it-1, which then takes stage it+3; slice 0 of it+1 is read while slice 3 of `it` multiplies.
    auto stage = [&](int it) {
        const uint8_t *sa = slot(it);
        const int nb = last(it + 1);
#pragma unroll
        for (int s = 0; s < WNS; ++s) {
            if (s + 1 == WNS) {
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::WAIT_X) : "memory");
                __builtin_amdgcn_s_barrier();
                issue_x(last(it + 3));
            }
            const uint8_t *rs = s + 1 < WNS ? sa : slot(it + 1);
            const int rsl = (s + 1) & (WNS - 1), rset = (s + 1) & 1;
            asm volatile("s_waitcnt vmcnt(%2)" : "+v"(ya[s][0]), "+v"(ya[s][1]) : "n"(C::WAIT_Y));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < FM * 2; ++m) {
                const int i = m / 2, j = m % 2;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ya[s][j]), wf[s & 1][i],
                                                                    acc[i][j], 0, 0, 0);
                if (m < FM) {
                    const int r = 32 * m + fr;
                    wf[rset][m] = *(const bf16x8 *)(rs + r * 128 + (((4 * fh + rsl) ^ wswz(r)) << 4));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            load_y(nb, s);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (it0 < it1) {
        // prologue in the steady-state order: weight tiles it0, it0+1; tokens of it0, slices 0-2;
        // weight tile it0+2; tokens of it0, slice 3.
        issue_x(it0);
        issue_x(last(it0 + 1));
#pragma unroll
        for (int s = 0; s < WNS - 1; ++s) load_y(it0, s);
        issue_x(last(it0 + 2));
        load_y(it0, WNS - 1);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::WAIT_P) : "memory");
        __builtin_amdgcn_s_barrier();
        read_w(slot(it0), 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        for (int it = it0; it < it1; ++it) stage(it);
    }

    // Every load has landed before the epilogue (none into LDS may be in flight when the LDS is
    // reused or the workgroup ends).
#pragma unroll
    for (int s = 0; s < WNS; ++s) asm volatile("s_waitcnt vmcnt(0)" : "+v"(ya[s][0]), "+v"(ya[s][1]));

    // Epilogue: two rounds of 32 tokens per wave.  Each wave writes its accumulators of fragment j as
    // fp32 rows of its own LDS area (token rows, feature columns), then the whole workgroup stores the
    // 128 rows as 16-byte runs of bf16.
    // D fragment of 32x32: lane holds column lane%32 (feature) and rows 8*(v/4) + 4*(lane/32) + v%4.
    __builtin_amdgcn_s_barrier();   // every wave is past its last fragment read
    constexpr int RCH = C::XR / 8;  // 16-byte bf16 runs per token row
    const bool vec_out = (p.ldo & 7) == 0 && (((uintptr_t)p.out) & 15) == 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float *ep = (float *)(smem + wave * C::EPB);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = ((v >> 2) << 3) + (fh << 2) + (v & 3);
                ep[row * C::EPS + 32 * i + fr] = acc[i][j][v];
            }
        __syncthreads();
        for (int q = tid; q < 128 * RCH; q += WTHREADS) {
            const int row = q / RCH, c = (q - row * RCH) * 8;   // row = 32 * (wave of the row) + token
            const int wv = row >> 5, tr = row & 31;
            const int n = n0 + wv * 64 + 32 * j + tr;
            if (n >= p.M) continue;
            const float *src = (const float *)(smem + wv * C::EPB) + tr * C::EPS + c;
            uint16_t *dst = p.out + (int64_t)n * p.ldo + o0 + c;
            if (vec_out) {
                const float4 lo = *(const float4 *)src, hi = *(const float4 *)(src + 4);
                u32x4 pk;
                pk[0] = pack2(lo.x, lo.y);
                pk[1] = pack2(lo.z, lo.w);
                pk[2] = pack2(hi.x, hi.y);
                pk[3] = pack2(hi.z, hi.w);
                *(u32x4 *)dst = pk;
            } else {
                for (int e = 0; e < 8; ++e) dst[e] = f2bf(src[e]);
            }
        }
        __syncthreads();
    }
}

// Feature-tile heights this kernel is built for (32 * FM); 0 when none divides O.
int gemm_w_rows(int O) { return O > 0 && O % 160 == 0 ? 160 : 0; }

hipError_t launch_gemm_w(const GemmParams &p, hipStream_t s) {
    if (p.M <= 0) return hipSuccess;
    if (p.K % WBK != 0 || p.K < WBK || p.S != 1 || p.part || !p.out || gemm_w_rows(p.O) != 160)
        return hipErrorInvalidValue;
    const unsigned tiles = (unsigned)(p.O / 160) * (unsigned)((p.M + WBM - 1) / WBM);
    return launch1(k_gemm_w<5, true>, dim3(tiles), dim3(WTHREADS), s, p);
}

}  // namespace dfkv
