// k_stream.hip -- the weight-streaming GEMMs of the two-kernel projection at
// small batch (M = B*W <= 64 token rows): fc (f and its row statistics) and the
// stacked K/V GEMM (fp32 split partials), one launch each.  The per-workgroup
// work lives in stream_core.hpp.
#include "stream_core.hpp"

namespace dfkv {

// STAGE (K/V GEMM at <= 16 rows): the workgroup first stages g = hidden_norm(f) for its k range in
// LDS -- one global hop loads f, w_hn and the fc tiles' sums of squares together, rinv is reduced
// by one wave per row, and the rounded g is written once -- then streams the weights against it.
template <int NG, int WAVES, int D, int WPE, bool STAGE>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WPE, 8))) void k_stream(
    const StreamParams p) {
    __shared__ float red[stream_red_floats<NG, WAVES>()];
    __shared__ float sh_rinv[16];
    extern __shared__ __attribute__((aligned(16))) uint16_t sh_g[];  // STAGE: [M][kc + 8]
    // the kernel arguments in one round of scalar loads: a field read where the code first needs it
    // is a round trip of its own through the scalar cache, which starts cold in every kernel
    asm volatile("" ::"s"(p.S), "s"(p.M), "s"(p.K), "s"(p.O), "s"(p.nbs), "s"(p.w), "s"(p.w_tiled), "s"(p.x),
                 "s"(p.ldx), "s"(p.out), "s"(p.ss_out), "s"(p.part));
    if constexpr (STAGE) asm volatile("" ::"s"(p.w_hn), "s"(p.ss_in), "s"(p.T_in), "s"(p.eps));
    const int t = (int)blockIdx.y, s = (int)blockIdx.x;   // grid (split, tile)
    stream_tile<NG, WAVES, D, STAGE>(p, t, s, red, sh_g, sh_rinv);
}

template <int NG>
static hipError_t launch_ng(const StreamParams &p, hipStream_t st) {
    const int grid = (p.O / 16) * p.S;
    const dim3 g2((unsigned)p.S, (unsigned)(p.O / 16));   // (split, tile): no division in the kernel
    if constexpr (NG == 1) {
        // fc: one workgroup per CU with a 4-deep ring; above 256 tiles (more than one round) two
        // per CU with a 3-deep ring, so all of them are resident at once (MLA fc, 448 tiles: 52.9 ->
        // 52.5 us measured; the 256-tile dense fc is 0.3 us slower that way)
        if (p.out) {
            if (grid > 256) return launch1(k_stream<1, 8, 3, 4, false>, g2, dim3(512), st, p);
            return launch1(k_stream<1, 8, 4, 2, false>, g2, dim3(512), st, p);
        }
        const size_t shmem = (size_t)p.M * (p.nbs * 128 + 8) * 2;
        // K/V: 3 workgroups per CU (all resident); a 1-deep weight ring keeps the staging prologue
        // free of spills, and 24 waves per CU still keep about 96 KB of loads in flight
        return launch1(k_stream<1, 8, 1, 6, true>, g2, dim3(512), st, p, shmem);
    } else {
        constexpr int D = NG <= 2 ? 2 : 1;
        return launch1(k_stream<NG, 8, D, 2, false>, g2, dim3(512), st, p);
    }
}

hipError_t launch_stream(const StreamParams &p, hipStream_t s) {
    if (p.M <= 0) return hipSuccess;
    switch ((p.M + 15) / 16) {
        case 1: return launch_ng<1>(p, s);
        case 2: return launch_ng<2>(p, s);
        case 3: return launch_ng<3>(p, s);
        case 4: return launch_ng<4>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dfkv
