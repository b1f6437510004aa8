// k_finalize.hip -- the last kernel of a step: k_norm + RoPE, the paged store of
// the gen tokens' context K/V into every layer's pool, and the per-request
// advance, in one launch.
//
// Sources (page titles and sections):
//  * TensorRT-LLM PR #20550 "fuse the decode-step drafter bookkeeping into
//    Triton kernels", section TLLM_DFLASH_FUSED_PROLOGUE: rejected-row mask,
//    clamp to the request's allocation, page lookup, write to every layer; the
//    ctx_len advance with the clamp, the dummy-slot reset and the advertised
//    context length; bonus token, query/context positions, embedding ids.  The
//    downstream commit quoted on that page adds seq_lens and requires pool
//    entries outside the step's destinations to stay unchanged.
//  * TensorRT-LLM PR #13995 "DFlash performance optimizations": commit "fuse
//    cross-layer k_norm" (one RMSNorm over every K head times stacked per-layer
//    weights, one eps) and commit "match RoPE between context and query for
//    YaRN" (context K rotated from the one cos/sin cache).
//
// One workgroup per token row, looping over the drafter layers.  The row's
// stacked projection is read either as fp32 split-K partial sums (summed in split
// order, then rounded to bf16 -- the K/V GEMM output) or as bf16 rows.  With
// `norm`, each K head (GQA) or the latent (MLA) is RMS-normalised by one wave
// (wave-level reduction) and rotated (NeoX pairs held by one lane), the rope
// part of MLA rotated only; V passes through.  The result goes to kv_out
// and, when the row's write predicate holds, to the layer's pool.  Rows whose
// predicate fails never touch the pools.
#include "finalize_common.hpp"

namespace dfkv {

// one element of the row's stacked projection, as fp32 (the bf16-rounded GEMM output)
__device__ __forceinline__ float load_y(const FinalizeParams &p, int row, int64_t col) {
    if (p.part) return part_y(p.part, p.S, p.M, p.O, row, col);
    return bf2f(p.src[(int64_t)row * p.O + col]);
}

// 8 consecutive elements (16 B aligned) of the row, as bf16 bits
__device__ __forceinline__ u32x4 load_y8(const FinalizeParams &p, int row, int64_t col) {
    if (p.part) {
        float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < p.S; ++s) {
            const f32x4 *src = (const f32x4 *)(p.part + ((int64_t)s * p.M + row) * p.O + col);
            const f32x4 lo = src[0], hi = src[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                y[e] += lo[e];
                y[4 + e] += hi[e];
            }
        }
        return u32x4{pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]), pack2(y[6], y[7])};
    }
    return *(const u32x4 *)(p.src + (int64_t)row * p.O + col);
}

constexpr int kFinThreads = 512;  // 8 waves: one K head per wave for up to 8 KV heads

// One workgroup per token row, every drafter layer: the row's destination (request fields, then the
// block-table entry) is looked up once, its loads issued before the first layer's.
__global__ __launch_bounds__(kFinThreads) void k_finalize(const FinalizeParams p) {
    const int L = p.L;
    const int row = blockIdx.x;
    const int r = row / p.W, i = row - (row / p.W) * p.W;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    constexpr int NW = kFinThreads / 64;

    if (p.advance && i == 0) request_advance(p, r);
    int64_t slot = -1;
    const bool w = p.store && row_destination(p, r, i, row, slot);
    if (p.store && tid == 0) {
        p.slot[row] = slot;
        p.wmask[row] = w ? 1 : 0;
    }
    const int64_t dst0 = w ? slot_offset(p, slot) : 0;
    uint16_t *const out_row = p.kv_out ? p.kv_out + (int64_t)row * p.O : nullptr;

    if (!p.norm) {
        // final K/V rows in hand (paged store of a finished projection, or plain rounding of the
        // partial sums): 16-byte chunks of every layer straight through, pool writes only for
        // written rows
        if (!out_row && !w) return;
        const int nch = p.per_layer >> 3;
        for (int c = tid; c < L * nch; c += kFinThreads) {
            const int l = c / nch, e = (c - l * nch) << 3;
            const int64_t lay = (int64_t)l * p.per_layer;
            const u32x4 v = load_y8(p, row, lay + e);
            if (out_row) *(u32x4 *)(out_row + lay + e) = v;
            if (w) {
                if (p.kind == DFKV_GQA) {
                    const int kvh = p.nkv * p.hd;
                    const bool is_v = e >= kvh;
                    const int ee = is_v ? e - kvh : e;
                    const int h = ee / p.hd;
                    *(u32x4 *)((is_v ? p.pv[l] : p.pk[l]) + dst0 + (int64_t)h * p.sh + (ee - h * p.hd)) = v;
                } else {
                    *(u32x4 *)(p.pk[l] + dst0 + e) = v;
                }
            }
        }
        return;
    }

    if (p.kind == DFKV_GQA) {
        const int hd = p.hd, nkv = p.nkv, half = hd >> 1;
        const int kvh = nkv * hd;
        const int vch = kvh >> 3;
        const float *cs = rope_row(p.nr, row);
        // V of every layer straight through (16-byte chunks)
        for (int c = tid; c < L * vch; c += kFinThreads) {
            const int l = c / vch, cc = c - l * vch;
            const int64_t lay = (int64_t)l * p.per_layer;
            const u32x4 v = load_y8(p, row, lay + kvh + (cc << 3));
            const int hh = cc / (hd >> 3), e = (cc - hh * (hd >> 3)) << 3;
            if (out_row) *(u32x4 *)(out_row + lay + kvh + (cc << 3)) = v;
            if (w) *(u32x4 *)(p.pv[l] + dst0 + (int64_t)hh * p.sh + e) = v;
        }
        // K heads of every layer: k_norm then RoPE, one wave per (layer, head)
        for (int item = wave; item < L * nkv; item += NW) {
            const int l = item / nkv, h = item - l * nkv;
            const int64_t lay = (int64_t)l * p.per_layer;
            float a[2] = {0.f, 0.f}, b[2] = {0.f, 0.f};
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const int j = lane + q2 * 64;
                if (j < half) {
                    a[q2] = load_y(p, row, lay + h * hd + j);
                    b[q2] = load_y(p, row, lay + h * hd + j + half);
                }
            }
            uint16_t ka[2], kb[2];
            knorm_rope_head(a, b, hd, p.nr.eps, p.nr.w_knorm + (int64_t)l * hd, cs, lane, ka, kb);
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const int j = lane + q2 * 64;
                if (j < half) {
                    if (out_row) {
                        out_row[lay + h * hd + j] = ka[q2];
                        out_row[lay + h * hd + j + half] = kb[q2];
                    }
                    if (w) {
                        uint16_t *d = p.pk[l] + dst0 + (int64_t)h * p.sh;
                        d[j] = ka[q2];
                        d[j + half] = kb[q2];
                    }
                }
            }
        }
    } else {
        // MLA: one wave per layer normalises the latent and rotates the rope part
        const int R = p.nr.latent, P = p.nr.rope_dim, half = P >> 1;
        const float *cs = rope_row(p.nr, row);
        for (int l = wave; l < L; l += NW) {
            const int64_t lay = (int64_t)l * p.per_layer;
            uint16_t *const out = out_row ? out_row + lay : nullptr;
            float v[16];
#pragma unroll
            for (int q2 = 0; q2 < 16; ++q2) {
                const int e = lane + q2 * 64;
                v[q2] = e < R ? load_y(p, row, lay + e) : 0.f;
            }
            float ra = 0.f, rb = 0.f;
            if (lane < half) {
                ra = load_y(p, row, lay + R + lane);
                rb = load_y(p, row, lay + R + lane + half);
            }
            uint16_t *d = w ? p.pk[l] + dst0 : nullptr;
            const float rinv = latent_rinv(v, R, p.nr.eps);
            const uint16_t *wk = p.nr.w_knorm + (int64_t)l * R;
#pragma unroll
            for (int q2 = 0; q2 < 16; ++q2) {
                const int e = lane + q2 * 64;
                if (e < R) {
                    const uint16_t o = latent_elem(wk[e], v[q2], rinv);
                    if (out) out[e] = o;
                    if (d) d[e] = o;
                }
            }
            if (lane < half) {
                const float c = cs[lane], sn = cs[half + lane];
                uint16_t ka, kb;
                rope_pair(ra, rb, c, sn, ka, kb);
                if (out) {
                    out[R + lane] = ka;
                    out[R + lane + half] = kb;
                }
                if (d) {
                    d[R + lane] = ka;
                    d[R + lane + half] = kb;
                }
            }
        }
    }
}

// GQA with k_norm + RoPE, vectorised: one workgroup of 256 threads per token row; thread t takes
// the row's 16-byte chunks t, t + 256, ..., t + 1024 (K chunks of every layer first, then the V
// chunks).  The row's chunks are loaded first, before anything they wait on: the row's cos/sin
// values and every layer's k_norm weights go to LDS (so no thread holds them in registers across
// the loads, which keeps seven workgroups resident per CU), and the row's destination is looked
// up meanwhile.  A K head of HD elements is HD/8 consecutive lanes of one wave: its sum of squares
// is a butterfly over those lanes, and the NeoX partner of chunk q (elements j and j + HD/2) is the
// lane HD/16 away, whose normalised values come over by lane exchange.  A wave whose chunks are
// all V (or past the row) only copies.  The per-element arithmetic is that of knorm_rope_head;
// only the order in which the squares are summed differs.
constexpr int kFinVThreads = 256;
constexpr int kFinVPer = 5;

template <int HD>
__global__ __launch_bounds__(kFinVThreads) void k_finalize_gqa(const FinalizeParams p) {
    constexpr int half = HD / 2;
    constexpr int qh = HD / 8, hq = qh / 2;   // chunks per head, per half head
    // cos | sin | -sin of the row's position: a first-half chunk rotates with -sin, a second-half
    // chunk with +sin (k = u c + u' s', u' the partner's normalised value)
    __shared__ __attribute__((aligned(16))) float s_cs[HD + half];
    __shared__ __attribute__((aligned(16))) uint16_t s_wk[DFKV_MAX_LAYERS * HD];      // [L][HD]
    // the kernel arguments of the row's path in one round of scalar loads: a field read where the
    // code first needs it is a round trip of its own through the scalar cache, which starts cold in
    // every kernel (the fields the first arithmetic uses pass through the statement, so that it
    // cannot start before it)
    int W = p.W, nkv = p.nkv, L = p.L;
    asm volatile("" : "+s"(W), "+s"(nkv), "+s"(L) : "s"(p.part), "s"(p.src), "s"(p.kv_out), "s"(p.S), "s"(p.M),
                 "s"(p.O), "s"(p.per_layer), "s"(p.store), "s"(p.advance), "s"(p.nr.cos_sin), "s"(p.nr.cache_len),
                 "s"(p.nr.ctx_len_in), "s"(p.nr.width), "s"(p.nr.rope_dim), "s"(p.nr.w_knorm), "s"(p.nr.eps),
                 "s"(p.dummy), "s"(p.n_acc), "s"(p.ctx_len), "s"(p.limit), "s"(p.row_valid), "s"(p.bt),
                 "s"(p.bt_stride), "s"(p.bt_cols), "s"(p.num_pages), "s"(p.pg));
    const int row = blockIdx.x;
    const int r = div_small(row, 1.0f / (float)W), i = row - r * W;   // (row < 2^21)
    const int tid = threadIdx.x;

    const int lch = nkv * qh;               // K (or V) chunks of one layer
    const int kch = L * lch;                // K chunks of the row; as many V chunks follow
    const int nch = 2 * kch;
    // chunk c -> (K or V, layer l, offset rem in the layer's K or V part); cc / lch by a float
    // reciprocal: cc / lch <= 2 * layers <= 64, so the product is within 4e-6 of the quotient while
    // cc + 0.5 keeps it at least 0.5 / lch from an integer
    const float inv_lch = 1.0f / (float)lch;
    auto split = [&](int c, bool &isk, int &l, int &rem) {
        isk = c < kch;
        const int cc = isk ? c : c - kch;
        l = (int)(((float)cc + 0.5f) * inv_lch);
        rem = cc - l * lch;
    };
    // In place (the rows are read from kv_out and written back there), a V chunk is already final:
    // it is only read when the row goes to the pool, and never written back.
    const bool inplace = !p.part && p.kv_out && p.src == p.kv_out;
    u32x4 y[kFinVPer];
    // chunks c0 <= c < c1 of the group at base (the others of the group are left as they are)
    auto load_group = [&](int base, int c0, int c1) {
#pragma unroll
        for (int m = 0; m < kFinVPer; ++m) {
            const int c = base + m * kFinVThreads + tid;
            bool isk;
            int l, rem;
            split(c, isk, l, rem);
            if (c >= c0) y[m] = c < c1 ? load_y8(p, row, (int64_t)l * p.per_layer + (isk ? 0 : p.nkv * HD) + rem * 8)
                                       : u32x4{0u, 0u, 0u, 0u};
        }
    };
    load_group(0, 0, inplace ? kch : nch);

    // the row's cos/sin values (rope_dim = HD floats) and the k_norm weights of every layer
    const float *cs = rope_row(p.nr, row);
    for (int c = tid; c < HD / 4; c += kFinVThreads) {
        const f32x4 v = *(const f32x4 *)(cs + 4 * c);
        *(f32x4 *)(s_cs + 4 * c) = v;
        if (c >= HD / 8) *(f32x4 *)(s_cs + half + 4 * c) = -v;
    }
    for (int c = tid; c < p.L * qh; c += kFinVThreads)
        *(u32x4 *)(s_wk + 8 * c) = *(const u32x4 *)(p.nr.w_knorm + 8 * (int64_t)c);

    if (p.advance && i == 0) request_advance(p, r);
    int64_t slot = -1;
    const bool w = p.store && row_destination(p, r, i, row, slot);
    if (p.store && tid == 0) {
        p.slot[row] = slot;
        p.wmask[row] = w ? 1 : 0;
    }
    const int64_t dst0 = w ? slot_offset(p, slot) : 0;
    uint16_t *const out_row = p.kv_out ? p.kv_out + (int64_t)row * p.O : nullptr;
    const float inv_hd = 1.0f / (float)HD;   // exact: HD is a power of two
    // the chunks this row needs: in place, those past the K part only when the row is stored
    const int cend = inplace && !w ? kch : nch;
    if (inplace && w) load_group(0, kch, nch);
    __syncthreads();

    for (int base = 0;;) {
#pragma unroll
        for (int m = 0; m < kFinVPer; ++m) {
            const int c = base + m * kFinVThreads + tid;
            const bool ok = c < cend;
            bool isk;
            int l, rem;
            split(c, isk, l, rem);
            const int h = rem / qh, q = rem % qh;
            u32x4 o = y[m];
            // wave-uniform: does this wave hold any K chunk?
            if (base + m * kFinVThreads + (tid & ~(kWave - 1)) < kch) {
                // sum of squares over the head's lanes (every lane takes part in the exchanges)
                float v8[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v8[2 * e] = bf_lo(y[m][e]);
                    v8[2 * e + 1] = bf_hi(y[m][e]);
                }
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += v8[e] * v8[e];
                if constexpr (HD == 128) {
                    // a head is one DPP row of 16 lanes: quad sums, then row_ror:4 and :8
                    ss = dpp_add<0xB1>(ss);
                    ss = dpp_add<0x4E>(ss);
                    ss = dpp_add<0x124>(ss);
                    ss = dpp_add<0x128>(ss);
                } else {
#pragma unroll
                    for (int off = hq; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
                }
                const float rinv = __builtin_amdgcn_rsqf(ss * inv_hd + p.nr.eps);
                // normalised values, rounded to bf16, and the partner's
                const u32x4 wk = *(const u32x4 *)(s_wk + l * HD + q * 8);
                uint32_t u2[4], pu2[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    u2[e] = pack2(bf_lo(wk[e]) * (v8[2 * e] * rinv), bf_hi(wk[e]) * (v8[2 * e + 1] * rinv));
                    // the partner chunk is 8 lanes away inside the row of 16: row_ror:8 (HD = 128)
                    pu2[e] = HD == 128 ? (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u2[e], 0x128, 0xF, 0xF, false)
                                       : (uint32_t)__shfl_xor((int)u2[e], hq, kWave);
                }
                if (isk) {
                    const bool first = q < hq;
                    const int j0 = (first ? q : q - hq) * 8;
                    const float *cp = s_cs + j0, *sp = s_cs + (first ? HD : half) + j0;
                    const f32x4 c0 = *(const f32x4 *)cp, c1 = *(const f32x4 *)(cp + 4);
                    const f32x4 s0 = *(const f32x4 *)sp, s1 = *(const f32x4 *)(sp + 4);
                    const float cv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                    const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[e] = pack2(bf_lo(u2[e]) * cv[2 * e] + bf_lo(pu2[e]) * sv[2 * e],
                                     bf_hi(u2[e]) * cv[2 * e + 1] + bf_hi(pu2[e]) * sv[2 * e + 1]);
                }
            }
            if (!ok) continue;
            const int64_t col = (int64_t)l * p.per_layer + (isk ? 0 : p.nkv * HD) + rem * 8;
            if (out_row && (isk || !inplace)) *(u32x4 *)(out_row + col) = o;
            if (w) *(u32x4 *)((isk ? p.pk[l] : p.pv[l]) + dst0 + (int64_t)h * p.sh + q * 8) = o;
        }
        base += kFinVThreads * kFinVPer;
        if (base >= cend) break;
        load_group(base, base, cend);
    }
}

// Advance only: one workgroup per request.
__global__ __launch_bounds__(64) void k_advance(const FinalizeParams p) { request_advance(p, blockIdx.x); }

// Row-wise paged store of prefill-shaped (ragged) rows (the single-latent context scatter the
// TensorRT-LLM PR #20550 page lists, at any row count): row n of request row_req[n] at position
// row_pos[n] is written when 0 <= r < B, 0 <= pos < limit[r], pos/pg < bt_cols and the page is in
// [0, num_pages).  One workgroup per row; every layer's slice moves as 16-byte chunks.
constexpr int kRowThreads = 256;
__global__ __launch_bounds__(kRowThreads) void k_store_rows(const FinalizeParams p) {
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t r = p.row_req[row];
    const int64_t pos = p.row_pos[row];
    int64_t slot = -1;
    if (r >= 0 && r < p.B && pos >= 0 && pos < (int64_t)p.limit[r] && pos / p.pg < p.bt_cols) {
        const int64_t pidx = pos / p.pg;
        const int32_t page = p.bt[(int64_t)r * p.bt_stride + pidx];
        if (page >= 0 && page < p.num_pages) slot = (int64_t)page * p.pg + (pos - pidx * p.pg);
    }
    if (tid == 0) {
        p.slot[row] = slot;
        p.wmask[row] = slot >= 0 ? 1 : 0;
    }
    if (slot < 0) return;
    const int64_t dst0 = slot_offset(p, slot);
    const uint16_t *src = p.src + (int64_t)row * p.O;
    const int nch = p.per_layer >> 3;
    for (int c = tid; c < p.L * nch; c += kRowThreads) {
        const int l = c / nch, e = (c - l * nch) << 3;
        const u32x4 v = *(const u32x4 *)(src + (int64_t)l * p.per_layer + e);
        if (p.kind == DFKV_GQA) {
            const int kvh = p.nkv * p.hd;
            const bool is_v = e >= kvh;
            const int ee = is_v ? e - kvh : e;
            const int h = ee / p.hd;
            *(u32x4 *)((is_v ? p.pv[l] : p.pk[l]) + dst0 + (int64_t)h * p.sh + (ee - h * p.hd)) = v;
        } else {
            *(u32x4 *)(p.pk[l] + dst0 + e) = v;
        }
    }
}

hipError_t launch_store_rows(const FinalizeParams &p, hipStream_t s) {
    if (p.M <= 0) return hipSuccess;
    return launch1(k_store_rows, dim3((unsigned)p.M), dim3(kRowThreads), s, p);
}

hipError_t launch_finalize(const FinalizeParams &p, hipStream_t s) {
    const int64_t N = (int64_t)p.B * p.W;
    if (N == 0) return hipSuccess;
    // the vectorised GQA kernel reads k_norm weights and cos/sin in 16-byte pieces
    if (p.norm && p.kind == DFKV_GQA && ((uintptr_t)p.nr.w_knorm & 15u) == 0 && ((uintptr_t)p.nr.cos_sin & 15u) == 0) {
        if (p.hd == 64) return launch1(k_finalize_gqa<64>, dim3((unsigned)N), dim3(kFinVThreads), s, p);
        if (p.hd == 128) return launch1(k_finalize_gqa<128>, dim3((unsigned)N), dim3(kFinVThreads), s, p);
        if (p.hd == 256) return launch1(k_finalize_gqa<256>, dim3((unsigned)N), dim3(kFinVThreads), s, p);
    }
    return launch1(k_finalize, dim3((unsigned)N), dim3(kFinThreads), s, p);
}

hipError_t launch_advance(const FinalizeParams &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    return launch1(k_advance, dim3(p.B), dim3(64), s, p);
}

}  // namespace dfkv
