// k_store.hip -- paged store of the gen tokens' context K/V and the per-request
// advance, in one coalesced launch (TensorRT-LLM PR #20550, section
// TLLM_DFLASH_FUSED_PROLOGUE: rejected-row mask, clamp to the request's
// allocation, page lookup, write to every layer; ctx_len advance with the clamp
// and the dummy-slot reset; bonus token, query/context positions, embedding ids.
// The downstream commit on that page adds seq_lens and requires every pool entry
// outside the step's destinations to stay unchanged).
//
// Layout of the work: one workgroup per token row.  Its threads first agree on
// the row's write predicate (all read the same few request words, served by the
// scalar/L1 path), then copy the row's L layers of K and V (or the MLA latent)
// as 16-byte chunks: consecutive threads move consecutive chunks of one head, so
// both the read of kv and the write into the pool are contiguous 16 B per lane.
// A rejected row returns before touching kv.  The workgroup of token 0 of a
// request also writes that request's advance outputs.
#include "dfkv_internal.hpp"

namespace dfkv {

__device__ __forceinline__ bool row_destination(const StoreParams &p, int r, int i, int row, int64_t &slot) {
    slot = -1;
    if (p.dummy[r]) return false;
    if (!(i < p.n_acc[r])) return false;
    if (p.row_valid && !p.row_valid[row]) return false;
    const int64_t pos = (int64_t)p.ctx_len[r] + i;
    if (pos < 0 || pos >= (int64_t)p.limit[r]) return false;
    const int64_t pidx = pos / p.pg;
    if (pidx >= p.bt_cols) return false;
    const int32_t page = p.bt[(int64_t)r * p.bt_stride + pidx];
    if (page < 0 || page >= p.num_pages) return false;
    slot = (int64_t)page * p.pg + (pos - pidx * p.pg);
    return true;
}

__device__ __forceinline__ void request_advance(const StoreParams &p, int r) {
    const int32_t c = p.ctx_len[r], n = p.n_acc[r], lim = p.limit[r];
    const bool d = p.dummy[r] != 0;
    const int64_t adv = (int64_t)c + n;
    const int32_t ctx_new = d ? 0 : (int32_t)(adv < (int64_t)lim ? adv : (int64_t)lim);
    const int nb = n < 1 ? 1 : (n > p.W ? p.W : n);
    const int32_t bonus = p.acc[(int64_t)r * p.acc_sr + (int64_t)(nb - 1) * p.acc_st];
    for (int j = threadIdx.x; j < p.bs_blk; j += blockDim.x) {
        p.emb[(int64_t)r * p.bs_blk + j] = j == 0 ? bonus : p.mask_id;
        p.q_pos[(int64_t)r * p.bs_blk + j] = ctx_new + j;
    }
    for (int j = threadIdx.x; j < p.W; j += blockDim.x) p.c_pos[(int64_t)r * p.W + j] = (int32_t)((int64_t)c + j);
    if (threadIdx.x == 0) {
        p.bonus[r] = bonus;
        p.ctx_out[r] = ctx_new;
        p.seq_len[r] = ctx_new + p.bs_blk;
    }
}

template <bool STORE, bool ADV>
__global__ __launch_bounds__(256) void k_store_advance(const StoreParams p) {
    int r, i, row;
    if (STORE) {
        row = blockIdx.x;
        r = row / p.W;
        i = row - r * p.W;
    } else {
        r = blockIdx.x;
        i = 0;
        row = r * p.W;
    }
    if (ADV && i == 0) request_advance(p, r);
    if (!STORE) return;

    int64_t slot;
    const bool w = row_destination(p, r, i, row, slot);
    if (threadIdx.x == 0) {
        p.slot[row] = slot;
        p.wmask[row] = w ? 1 : 0;
    }
    if (!w) return;
    const int64_t page = slot / p.pg, off = slot - (slot / p.pg) * p.pg;
    const int64_t dst0 = page * p.sp + off * p.ss;
    const uint16_t *src = p.kv + (int64_t)row * p.kv_ld;
    if (p.kind == DFKV_GQA) {
        const int cph = p.hd >> 3;             // 16-byte chunks per head
        const int cpk = p.nkv * cph;           // chunks per K (or V) half of a layer
        const int total = p.L * 2 * cpk;
        for (int c = threadIdx.x; c < total; c += blockDim.x) {
            const int l = c / (2 * cpk);
            const int rem = c - l * 2 * cpk;
            const int s = rem / cpk;           // 0 = K, 1 = V
            const int rem2 = rem - s * cpk;
            const int h = rem2 / cph;
            const int e = (rem2 - h * cph) << 3;
            const u32x4 v = *(const u32x4 *)(src + (int64_t)l * p.per_layer + s * p.nkv * p.hd + h * p.hd + e);
            uint16_t *base = s ? p.pv[l] : p.pk[l];
            *(u32x4 *)(base + dst0 + (int64_t)h * p.sh + e) = v;
        }
    } else {
        const int cpl = p.per_layer >> 3;
        const int total = p.L * cpl;
        for (int c = threadIdx.x; c < total; c += blockDim.x) {
            const int l = c / cpl;
            const int e = (c - l * cpl) << 3;
            const u32x4 v = *(const u32x4 *)(src + (int64_t)l * p.per_layer + e);
            *(u32x4 *)(p.pk[l] + dst0 + e) = v;
        }
    }
}

hipError_t launch_store_advance(const StoreParams &p, bool store, bool advance, hipStream_t s) {
    const int N = p.B * p.W;
    if (store) {
        if (N == 0) return hipSuccess;
        if (advance) return launch1(k_store_advance<true, true>, dim3(N), dim3(256), s, p);
        return launch1(k_store_advance<true, false>, dim3(N), dim3(256), s, p);
    }
    if (p.B == 0) return hipSuccess;
    return launch1(k_store_advance<false, true>, dim3(p.B), dim3(64), s, p);
}

}  // namespace dfkv
