// k_tiled.hip -- LDS-tiled bf16 MFMA GEMM for the projection at larger batch
// (M = B*W > 64 rows), where the fc and stacked K/V GEMMs are bound by the
// matrix cores rather than by streaming the weights (TensorRT-LLM PR #13995
// "DFlash performance optimizations", commit "fuse cross-layer k_norm": at
// bs=64 the GEMMs dominate the step).
//
//   out[n][o] = bf16( sum_k x[n][k] * w[o][k] )    (both operands K-contiguous)
//
// Tile 128 (tokens) x 128 (output features) x 64 (k), 4 waves in a 2x2 grid,
// each wave a 64x64 block of four v_mfma_f32_32x32x16_bf16 accumulators.
// Both operand tiles are staged through LDS, double buffered: the global loads
// of step k+1 are issued before the MFMAs of step k and written to the other
// buffer afterwards, so one barrier per step suffices.  LDS rows are padded to
// 72 elements (144 B) so the 16-byte fragment reads of 32 consecutive rows
// fall on distinct banks.
#include "dfkv_internal.hpp"

namespace dfkv {

constexpr int TBM = 128, TBN = 128, TBK = 64, TLD = TBK + 8;

__global__ __launch_bounds__(256, 1) void k_tiled(const TiledParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][TBM][TLD];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][TBN][TLD];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.y * TBM, o0 = blockIdx.x * TBN;

    u32x4 ra[4], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i, row = c >> 3, kc = (c & 7) << 3;
            const int n = n0 + row, o = o0 + row;
            ra[i] = n < p.M ? *(const u32x4 *)(p.x + (int64_t)n * p.ldx + k0 + kc) : u32x4{0u, 0u, 0u, 0u};
            rb[i] = o < p.O ? *(const u32x4 *)(p.w + (int64_t)o * p.K + k0 + kc) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i, row = c >> 3, kc = (c & 7) << 3;
            *(u32x4 *)&sA[buf][row][kc] = ra[i];
            *(u32x4 *)&sB[buf][row][kc] = rb[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = p.K / TBK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int fr = lane & 31, fk = (lane >> 5) << 3;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * TBK);
#pragma unroll
        for (int kk = 0; kk < TBK; kk += 16) {
            bf16x8 af[2], bw[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) af[i] = *(const bf16x8 *)&sA[buf][wm * 64 + i * 32 + fr][kk + fk];
#pragma unroll
            for (int j = 0; j < 2; ++j) bw[j] = *(const bf16x8 *)&sB[buf][wn * 64 + j * 32 + fr][kk + fk];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bw[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    // D fragment of 32x32: lane holds column lane%32 and rows 8*(v/4) + 4*(lane/32) + v%4.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int o = o0 + wn * 64 + j * 32 + (lane & 31);
            if (o >= p.O) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int n = n0 + wm * 64 + i * 32 + ((v >> 2) << 3) + ((lane >> 5) << 2) + (v & 3);
                if (n < p.M) p.out[(int64_t)n * p.ldo + o] = f2bf(acc[i][j][v]);
            }
        }
}

hipError_t launch_tiled(const TiledParams &p, hipStream_t s) {
    if (p.M <= 0) return hipSuccess;
    dim3 grid((p.O + TBN - 1) / TBN, (p.M + TBM - 1) / TBM);
    return launch1(k_tiled, grid, dim3(256), s, p);
}

}  // namespace dfkv
