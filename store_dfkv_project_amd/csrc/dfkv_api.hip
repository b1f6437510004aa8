// dfkv_api.hip -- the C ABI of libdfkv: host-side validation, workspace
// planning and kernel dispatch.  Every check runs before the first launch, so
// a refused call launches nothing and writes nothing.
#include <string.h>

#include <mutex>

#include "dfkv_internal.hpp"

using namespace dfkv;

// Device scratch of dfkv_step_noalloc: the workspace of a call that cannot allocate.  Each GPU the
// library runs on holds its own copy until the process ends.  Host code never uses this name as an
// address (on the host it is only a stand-in for the symbol); it uses the per-device address that
// scratch_address() looks up.
static __device__ __align__(256) uint8_t scratch[DFKV_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local hipError_t g_last_hip_error = hipSuccess;

dfkv_status hip_status(hipError_t e) {
    if (e == hipSuccess) return DFKV_OK;
    g_last_hip_error = e;
    return DFKV_ERR_HIP;
}

constexpr int kSkinnyMaxRows = 64;   // M = B*W handled by the weight-streaming split-K path
constexpr int kTargetItems = 512;    // K/V GEMM workgroups aimed for (256 CUs x 2)

bool al16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool al4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

int per_layer(const dfkv_geom *g) {
    return g->kind == DFKV_GQA ? 2 * g->n_kv_heads * g->head_dim : g->latent_dim + g->rope_dim;
}
int64_t out_dim(const dfkv_geom *g) { return (int64_t)g->n_layers * per_layer(g); }
int64_t k_in(const dfkv_geom *g) { return (int64_t)g->n_tgt * g->tgt_hidden; }

dfkv_status check_geom(const dfkv_geom *g) {
    if (!g) return DFKV_ERR_NULL;
    if (g->kind != DFKV_GQA && g->kind != DFKV_MLA) return DFKV_ERR_SHAPE;
    if (g->n_tgt <= 0 || g->tgt_hidden <= 0 || g->hidden <= 0 || g->n_layers <= 0) return DFKV_ERR_SHAPE;
    if (g->n_layers > DFKV_MAX_LAYERS) return DFKV_ERR_SHAPE;
    if (g->page_size <= 0 || g->width <= 0 || g->block_size <= 0) return DFKV_ERR_SHAPE;
    if (!(g->eps >= 0.f) || g->eps > 1.f) return DFKV_ERR_SHAPE;
    if (k_in(g) % 128 != 0 || g->hidden % 128 != 0 || k_in(g) > (1 << 20) || g->hidden > (1 << 16))
        return DFKV_ERR_SHAPE;
    if (g->kind == DFKV_GQA) {
        if (g->n_kv_heads <= 0 || g->n_kv_heads > 128) return DFKV_ERR_SHAPE;
        if (g->head_dim != 64 && g->head_dim != 128 && g->head_dim != 256) return DFKV_ERR_SHAPE;
        if (g->rope_dim != g->head_dim) return DFKV_ERR_SHAPE;
    } else {
        if (g->n_kv_heads != 1 || g->head_dim != 0) return DFKV_ERR_SHAPE;
        if (g->latent_dim <= 0 || g->latent_dim % 64 != 0 || g->latent_dim > 1024) return DFKV_ERR_SHAPE;
        if (g->rope_dim <= 0 || g->rope_dim % 2 != 0 || g->rope_dim > 128) return DFKV_ERR_SHAPE;
        if ((g->latent_dim + g->rope_dim) % 64 != 0) return DFKV_ERR_SHAPE;
    }
    if (out_dim(g) > (1 << 20)) return DFKV_ERR_SHAPE;
    return DFKV_OK;
}

// Splits of the K/V GEMM: S divides the number of 128-wide k-blocks, keeps at
// least 8 k-blocks (one per wave) per split when it can, stays within
// kMaxSplitK (and, at <= 16 rows, within the LDS stage of g), and is the
// smallest count giving kTargetItems workgroups.
int choose_kv_splits(int tiles, int kblocks, int64_t M) {
    int best = -1;
    for (int S = 1; S <= kblocks; ++S) {
        if (kblocks % S) continue;
        const int nbs = kblocks / S;
        if (nbs * 128 > kMaxSplitK || (M <= 16 && !stage_fits(M, nbs))) continue;
        if (best > 0 && nbs < 8) break;
        best = S;
        if ((int64_t)tiles * S >= kTargetItems) break;
    }
    return best > 0 ? best : kblocks;
}

// The small-batch K/V kernel's groups: S splits of the K/V GEMM, each a multiple of 8 k-blocks
// (every wave takes the same number of blocks of every tile) whose g fits the LDS stage, times
// groups of ntg 16-feature tiles (ntg <= the tiles of one unit).  Among the choices that fit the resident workgroup slots (one wave of groups,
// all of equal size) it takes the one with the least work on the busiest CU, preferring more
// groups, then fewer splits, on ties.  False when no split qualifies.
bool choose_kv_groups(const dfkv_geom *g, int64_t M, int *S_out, int *ntg_out) {
    const int kb = g->hidden / 128;
    const int T = (int)(out_dim(g) / 16);
    const int tpu = (g->kind == DFKV_GQA ? g->head_dim : per_layer(g)) / 16;
    // The groups are dealt one per CU per round (two resident per CU), so the busiest CU streams
    // ceil(n / CUs) groups of ntg tiles x kb/S k-blocks: minimise that, ties to more groups.
    const int cus = kKvSlots / 2;
    int best_n = 0, best_S = 0, best_ntg = 0;
    int64_t best_cost = 0;
    for (int S = 1; S <= kb; ++S) {
        if (kb % S || (kb / S) % 8 || !stage_fits(M, kb / S)) continue;
        for (int ntg = 1; ntg <= tpu && ntg <= T; ++ntg) {
            if (T % ntg) continue;
            const int n = S * (T / ntg);
            const int64_t cost = (int64_t)((n + cus - 1) / cus) * ntg * (kb / S);
            bool better;
            if (best_n == 0) better = true;
            else if ((n <= kKvSlots) != (best_n <= kKvSlots)) better = n <= kKvSlots;
            else if (n > kKvSlots) better = n < best_n;
            else better = cost < best_cost || (cost == best_cost && n > best_n);
            if (better) {
                best_n = n;
                best_S = S;
                best_ntg = ntg;
                best_cost = cost;
            }
        }
    }
    if (best_n == 0) return false;
    *S_out = best_S;
    *ntg_out = best_ntg;
    return true;
}

// The large-batch fc GEMM is split over k when its output tiles leave most of the 256 CUs idle
// (one workgroup per CU): enough splits to reach about one workgroup per CU, each split at least
// 16 k steps of 64, at most 8 splits.
int choose_fc_splits(int64_t M, int64_t H, int64_t K) {
    const int tiles = gemm_tiles((int)M, (int)H);
    if (tiles >= 192) return 1;
    int S = 256 / tiles;
    S = S < 8 ? S : 8;
    while (S > 1 && K / 64 / S < 16) --S;
    return S < 1 ? 1 : S;
}

struct Plan {
    int64_t M;
    bool skinny;
    bool kvfin;  // k_kvgroups + k_kvfinal run the K/V stage
    int S_kv;
    int S_fc;    // large batch: k splits of the fc GEMM (partials summed by hidden_norm)
    bool kv_w;   // large batch: the K/V GEMM is k_gemm_w (g packed in its token order)
    int ntg;     // k_kvfin: tiles per K/V group
    // bookkeeping area of the small-batch K/V kernels; f [M][H]; small batch: ss [H/16][M] and K/V
    // partials [S][M][O]; large batch: g [M][H] and, when the fc GEMM is split, its partials [S][M][H]
    size_t off_book, off_f, off_g, off_ss, off_part, total;
};

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Per-device address of `scratch`, looked up once per device (hipGetSymbolAddress with that device
// current) and kept.  The device is the stream's (the current device for the null stream).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];

hipError_t scratch_address(hipStream_t s, void **out) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (s) {
        hipDevice_t sd = 0;
        if ((e = hipStreamGetDevice(s, &sd)) != hipSuccess) return e;
        dev = (int)sd;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = ptr;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

dfkv_status make_plan(const dfkv_geom *g, int32_t n_reqs, Plan *pl) {
    dfkv_status st = check_geom(g);
    if (st != DFKV_OK) return st;
    if (n_reqs < 0) return DFKV_ERR_SHAPE;
    const int64_t M = (int64_t)n_reqs * g->width;
    if (M > (1 << 22)) return DFKV_ERR_SHAPE;
    const int64_t H = g->hidden, O = out_dim(g);
    Plan p{};
    p.M = M;
    p.skinny = M <= kSkinnyMaxRows;
    const size_t Mp = M > 0 ? (size_t)M : 1;
    size_t off = 0;
    p.off_book = off; off = up256(off + kv_book_bytes(g->rope_dim));
    p.off_f = off; off = up256(off + Mp * H * 2);
    p.kv_w = !p.skinny && gemm_w_rows((int)O) != 0 && H % 64 == 0;
    p.off_g = off; off = up256(off + (p.kv_w ? (Mp + 63) / 64 * 64 : Mp) * H * 2);
    p.kvfin = M >= 1 && M <= kKvMaxRows && (int64_t)n_reqs * g->block_size <= kKvMaxBlockPositions &&
              choose_kv_groups(g, M, &p.S_kv, &p.ntg);
    if (p.skinny) {
        if (!p.kvfin) p.S_kv = choose_kv_splits((int)(O / 16), (int)(H / 128), M);
        p.off_ss = off;   off = up256(off + (size_t)(H / 16) * Mp * 4);
        p.off_part = off; off = up256(off + (size_t)p.S_kv * Mp * O * 4);
    } else {
        p.S_kv = 1;
        p.S_fc = choose_fc_splits(M, H, k_in(g));
        p.off_ss = 0;
        p.off_part = off;
        if (p.S_fc > 1) off = up256(off + (size_t)p.S_fc * Mp * H * 4);
    }
    p.total = off;
    *pl = p;
    return DFKV_OK;
}

NormRopeGeom nr_geom(const dfkv_geom *g, const void *w_knorm, const int32_t *ctx, const float *cs, int32_t cache_len) {
    NormRopeGeom r{};
    r.kind = g->kind;
    r.n_layers = g->n_layers;
    r.nkv = g->n_kv_heads;
    r.hd = g->head_dim;
    r.latent = g->latent_dim;
    r.rope_dim = g->rope_dim;
    r.per_layer = per_layer(g);
    r.width = g->width;
    r.cache_len = cache_len;
    r.out_dim = (int32_t)out_dim(g);
    r.eps = g->eps;
    r.w_knorm = (const uint16_t *)w_knorm;
    r.ctx_len_in = ctx;
    r.cos_sin = cs;
    return r;
}

// ----- validation shared by the entry points --------------------------------

// The tiled weight copies a call reads (dfkv_pack_stream_weight): 16-byte aligned (LAYOUT), and not
// inside kv_out or the workspace (ALIAS).  `alias` false checks the alignment only.
dfkv_status check_stream_weights(const dfkv_geom *g, const dfkv_weights *w, bool fc, bool kv, bool alias,
                                 const void *kv_out, size_t kv_bytes, const void *ws, size_t ws_bytes) {
    const void *p[2] = {fc ? w->w_fc_stream : nullptr, kv ? w->w_kv_stream : nullptr};
    const size_t n[2] = {(size_t)g->hidden * k_in(g) * 2, (size_t)out_dim(g) * g->hidden * 2};
    for (int i = 0; i < 2; ++i) {
        if (!p[i]) continue;
        if (!alias && !al16(p[i])) return DFKV_ERR_LAYOUT;
        if (alias && (overlap(kv_out, kv_bytes, p[i], n[i]) || overlap(ws, ws_bytes, p[i], n[i])))
            return DFKV_ERR_ALIAS;
    }
    return DFKV_OK;
}

dfkv_status check_project(const dfkv_geom *g, const dfkv_weights *w, const void *hidden, int64_t ld,
                          int32_t n_reqs, const int32_t *ctx, const float *cs, int32_t cache_len, void *kv_out,
                          uint32_t flags, void *ws, size_t ws_bytes, Plan *pl) {
    if (!g || !w) return DFKV_ERR_NULL;
    dfkv_status st = make_plan(g, n_reqs, pl);
    if (st != DFKV_OK) return st;
    const bool fuse = (flags & DFKV_FUSE_NORM_ROPE) != 0;
    if ((flags & ~(uint32_t)DFKV_FUSE_NORM_ROPE) != 0) return DFKV_ERR_SHAPE;
    if (pl->M == 0) return DFKV_OK;
    if (!hidden || !kv_out || !w->w_fc || !w->w_hnorm || !w->w_kv || !ws) return DFKV_ERR_NULL;
    if (fuse && (!w->w_knorm || !ctx || !cs)) return DFKV_ERR_NULL;
    if (fuse && cache_len <= 0) return DFKV_ERR_SHAPE;
    const int64_t K = k_in(g), H = g->hidden, O = out_dim(g), M = pl->M;
    if (ld < K || (ld * 2) % 16 != 0) return DFKV_ERR_LAYOUT;
    if (!al16(hidden) || !al16(kv_out) || !al16(w->w_fc) || !al16(w->w_hnorm) || !al16(w->w_kv) || !al16(ws))
        return DFKV_ERR_LAYOUT;
    if (fuse && (!al4(cs) || ((uintptr_t)w->w_knorm & 1u))) return DFKV_ERR_LAYOUT;
    if (w->w_fc_packed && !al16(w->w_fc_packed)) return DFKV_ERR_LAYOUT;
    if ((st = check_stream_weights(g, w, true, true, false, nullptr, 0, nullptr, 0)) != DFKV_OK) return st;
    if (ws_bytes < pl->total) return DFKV_ERR_WORKSPACE;
    const size_t kv_bytes = (size_t)M * O * 2;
    if (w->w_fc_packed && (overlap(kv_out, kv_bytes, w->w_fc_packed, (size_t)H * K * 2) ||
                           overlap(ws, ws_bytes, w->w_fc_packed, (size_t)H * K * 2)))
        return DFKV_ERR_ALIAS;
    if ((st = check_stream_weights(g, w, true, true, true, kv_out, kv_bytes, ws, ws_bytes)) != DFKV_OK) return st;
    const size_t hid_bytes = (size_t)((M - 1) * ld + K) * 2;
    if (overlap(kv_out, kv_bytes, hidden, hid_bytes) || overlap(kv_out, kv_bytes, ws, ws_bytes) ||
        overlap(kv_out, kv_bytes, w->w_fc, (size_t)H * K * 2) || overlap(kv_out, kv_bytes, w->w_kv, (size_t)O * H * 2) ||
        overlap(kv_out, kv_bytes, w->w_hnorm, (size_t)H * 2) || overlap(ws, ws_bytes, hidden, hid_bytes))
        return DFKV_ERR_ALIAS;
    if (fuse) {
        const size_t kn = (size_t)g->n_layers * (g->kind == DFKV_GQA ? g->head_dim : g->latent_dim) * 2;
        if (overlap(kv_out, kv_bytes, cs, (size_t)cache_len * g->rope_dim * 4) ||
            overlap(kv_out, kv_bytes, w->w_knorm, kn) || overlap(kv_out, kv_bytes, ctx, (size_t)n_reqs * 4))
            return DFKV_ERR_ALIAS;
    }
    return DFKV_OK;
}

dfkv_status check_requests(const dfkv_geom *g, const dfkv_requests *r, bool need_store, bool need_adv) {
    if (!r) return DFKV_ERR_NULL;
    if (r->n_reqs < 0) return DFKV_ERR_SHAPE;
    if (r->n_reqs == 0) return DFKV_OK;
    if (!r->ctx_len_in || !r->n_acc || !r->alloc_limit || !r->is_dummy) return DFKV_ERR_NULL;
    if (need_store) {
        if (!r->block_table) return DFKV_ERR_NULL;
        if (r->bt_cols <= 0 || r->bt_row_stride < r->bt_cols) return DFKV_ERR_LAYOUT;
    }
    if (need_adv) {
        if (!r->accepted_tokens) return DFKV_ERR_NULL;
        if (r->acc_stride_req < 0 || r->acc_stride_tok < 0) return DFKV_ERR_LAYOUT;
    }
    (void)g;
    return DFKV_OK;
}

// Byte extent [lo, hi) of a strided int32 view of n_a x n_b elements.
size_t extent2(int64_t s_a, int64_t n_a, int64_t s_b, int64_t n_b) {
    if (n_a <= 0 || n_b <= 0) return 0;
    return (size_t)(((n_a - 1) * s_a + (n_b - 1) * s_b + 1) * 4);
}

dfkv_status check_pool(const dfkv_geom *g, const dfkv_pool *pool) {
    if (!pool) return DFKV_ERR_NULL;
    if (pool->num_pages < 0) return DFKV_ERR_SHAPE;
    const int64_t sp = pool->stride_page, ss = pool->stride_slot, sh = pool->stride_head;
    if (sp <= 0 || ss <= 0 || sp % 8 || ss % 8) return DFKV_ERR_LAYOUT;
    const int64_t pg = g->page_size;
    if (g->kind == DFKV_GQA) {
        const int64_t hd = g->head_dim, nkv = g->n_kv_heads;
        if (nkv > 1 && (sh <= 0 || sh % 8)) return DFKV_ERR_LAYOUT;
        const bool nhd = sh >= hd && ss >= nkv * sh;     // [page][slot][head][dim]
        const bool hnd = ss >= hd && sh >= pg * ss;      // [page][head][slot][dim]
        if (nkv > 1 ? !(nhd || hnd) : ss < hd) return DFKV_ERR_LAYOUT;
        const int64_t page_extent = (pg - 1) * ss + (nkv - 1) * (nkv > 1 ? sh : 0) + hd;
        if (sp < page_extent) return DFKV_ERR_LAYOUT;
    } else {
        const int64_t row = g->latent_dim + g->rope_dim;
        if (ss < row || sp < (pg - 1) * ss + row) return DFKV_ERR_LAYOUT;
    }
    for (int l = 0; l < g->n_layers; ++l) {
        if (!pool->k[l]) return DFKV_ERR_NULL;
        if (!al16(pool->k[l])) return DFKV_ERR_LAYOUT;
        if (g->kind == DFKV_GQA) {
            if (!pool->v[l]) return DFKV_ERR_NULL;
            if (!al16(pool->v[l])) return DFKV_ERR_LAYOUT;
        }
    }
    return DFKV_OK;
}

size_t pool_bytes(const dfkv_geom *g, const dfkv_pool *pool) { return (size_t)pool->num_pages * pool->stride_page * 2; }

dfkv_status check_store_outputs_n(const dfkv_geom *g, int64_t N, const dfkv_pool *pool, const void *kv,
                                  const int64_t *slot, const uint8_t *wmask) {
    if (N == 0) return DFKV_OK;
    if (!kv || !slot || !wmask) return DFKV_ERR_NULL;
    if (!al16(kv) || ((uintptr_t)slot & 7u)) return DFKV_ERR_LAYOUT;
    const size_t kvb = (size_t)N * out_dim(g) * 2, pb = pool_bytes(g, pool);
    const void *outs[2] = {slot, wmask};
    const size_t outb[2] = {(size_t)N * 8, (size_t)N};
    for (int i = 0; i < 2; ++i) {
        if (overlap(outs[i], outb[i], kv, kvb)) return DFKV_ERR_ALIAS;
        for (int l = 0; l < g->n_layers; ++l) {
            if (overlap(outs[i], outb[i], pool->k[l], pb)) return DFKV_ERR_ALIAS;
            if (g->kind == DFKV_GQA && overlap(outs[i], outb[i], pool->v[l], pb)) return DFKV_ERR_ALIAS;
        }
    }
    if (overlap(slot, outb[0], wmask, outb[1])) return DFKV_ERR_ALIAS;
    for (int l = 0; l < g->n_layers; ++l) {
        if (overlap(kv, kvb, pool->k[l], pb)) return DFKV_ERR_ALIAS;
        if (g->kind == DFKV_GQA && overlap(kv, kvb, pool->v[l], pb)) return DFKV_ERR_ALIAS;
    }
    return DFKV_OK;
}

dfkv_status check_store_outputs(const dfkv_geom *g, const dfkv_requests *r, const dfkv_pool *pool, const void *kv,
                                const int64_t *slot, const uint8_t *wmask) {
    return check_store_outputs_n(g, (int64_t)r->n_reqs * g->width, pool, kv, slot, wmask);
}

dfkv_status check_adv_outputs(const dfkv_geom *g, const dfkv_requests *r, const dfkv_outputs *o) {
    if (!o) return DFKV_ERR_NULL;
    const int64_t B = r->n_reqs;
    if (B == 0) return DFKV_OK;
    if (!o->c_pos || !o->bonus || !o->emb_ids || !o->q_pos || !o->ctx_len_out || !o->seq_len) return DFKV_ERR_NULL;
    const int64_t N = B * g->width, bs = g->block_size;
    const void *outs[6] = {o->c_pos, o->bonus, o->emb_ids, o->q_pos, o->ctx_len_out, o->seq_len};
    const size_t ob[6] = {(size_t)N * 4, (size_t)B * 4, (size_t)(B * bs) * 4, (size_t)(B * bs) * 4, (size_t)B * 4,
                          (size_t)B * 4};
    const void *ins[6] = {r->ctx_len_in, r->n_acc, r->alloc_limit, r->is_dummy, r->accepted_tokens, r->row_valid};
    const size_t ib[6] = {(size_t)B * 4, (size_t)B * 4, (size_t)B * 4, (size_t)B,
                          extent2(r->acc_stride_req, B, r->acc_stride_tok, g->width), (size_t)N};
    for (int i = 0; i < 6; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlap(outs[i], ob[i], ins[j], ib[j])) return DFKV_ERR_ALIAS;
        for (int j = i + 1; j < 6; ++j)
            if (overlap(outs[i], ob[i], outs[j], ob[j])) return DFKV_ERR_ALIAS;
        if (r->block_table && overlap(outs[i], ob[i], r->block_table,
                                      extent2(r->bt_row_stride, B, 1, r->bt_cols)))
            return DFKV_ERR_ALIAS;
    }
    if (o->block_slot) {
        // the block placement reads the block table: it needs one, and overlaps nothing
        if (!r->block_table) return DFKV_ERR_NULL;
        if (((uintptr_t)o->block_slot & 7) != 0) return DFKV_ERR_LAYOUT;
        const size_t bb = (size_t)(B * bs) * 8;
        for (int j = 0; j < 6; ++j)
            if (overlap(o->block_slot, bb, ins[j], ib[j]) || overlap(o->block_slot, bb, outs[j], ob[j]))
                return DFKV_ERR_ALIAS;
        if (overlap(o->block_slot, bb, r->block_table, extent2(r->bt_row_stride, B, 1, r->bt_cols)))
            return DFKV_ERR_ALIAS;
        if (o->slot && overlap(o->block_slot, bb, o->slot, (size_t)N * 8)) return DFKV_ERR_ALIAS;
        if (o->write_mask && overlap(o->block_slot, bb, o->write_mask, (size_t)N)) return DFKV_ERR_ALIAS;
    }
    return DFKV_OK;
}

FinalizeParams fin_params(const dfkv_geom *g, const dfkv_requests *r, const dfkv_pool *pool, const dfkv_outputs *o,
                          int32_t n_reqs) {
    FinalizeParams p;
    memset(&p, 0, sizeof p);
    p.O = (int32_t)out_dim(g);
    p.B = r ? r->n_reqs : n_reqs;
    p.M = p.B * g->width;
    p.W = g->width;
    p.bs_blk = g->block_size;
    p.pg = g->page_size;
    p.L = g->n_layers;
    p.kind = g->kind;
    p.nkv = g->n_kv_heads;
    p.hd = g->head_dim;
    p.per_layer = per_layer(g);
    if (r) {
        p.ctx_len = r->ctx_len_in;
        p.n_acc = r->n_acc;
        p.limit = r->alloc_limit;
        p.dummy = r->is_dummy;
        p.row_valid = r->row_valid;
        p.bt = r->block_table;
        p.bt_stride = r->bt_row_stride;
        p.bt_cols = r->bt_cols;
        p.acc = r->accepted_tokens;
        p.acc_sr = r->acc_stride_req;
        p.acc_st = r->acc_stride_tok;
        p.mask_id = r->mask_token_id;
    }
    if (pool) {
        p.num_pages = pool->num_pages;
        for (int l = 0; l < g->n_layers; ++l) {
            p.pk[l] = (uint16_t *)pool->k[l];
            p.pv[l] = (uint16_t *)pool->v[l];
        }
        p.sp = pool->stride_page;
        p.ss = pool->stride_slot;
        p.sh = pool->stride_head;
    }
    if (o) {
        p.slot = o->slot;
        p.wmask = o->write_mask;
        p.c_pos = o->c_pos;
        p.bonus = o->bonus;
        p.emb = o->emb_ids;
        p.q_pos = o->q_pos;
        p.ctx_out = o->ctx_len_out;
        p.seq_len = o->seq_len;
        p.block_slot = o->block_slot;
    }
    return p;
}

// ----- launches ---------------------------------------------------------------

// The projection, in two stages.
//  fc stage  -- f = bf16(hidden . w_fc^T) into ws.  Small batch: streaming GEMM
//               whose epilogue also writes f's per-16-column sums of squares;
//               above 16 rows (no LDS stage) or 64 rows (tiled GEMM) also
//               g = hidden_norm(f) by its own kernel.
//  K/V stage -- small batch: streaming GEMM (staging g in LDS at <= 16 rows)
//               into fp32 split partials, then the finalize kernel; large batch:
//               tiled GEMM over g into kv_out, then the finalize kernel in place.
// The finalize kernel does k_norm/RoPE (or plain rounding) and, when `fin`
// asks for it, the paged store and the advance.
bool stages_g(const Plan &pl) { return pl.skinny && pl.M <= 16; }

dfkv_status run_fc(const dfkv_geom *g, const dfkv_weights *w, const void *hidden, int64_t ld, void *ws,
                   const Plan &pl, hipStream_t s) {
    if (pl.M == 0) return DFKV_OK;
    char *wsb = (char *)ws;
    const int64_t K = k_in(g), H = g->hidden;
    uint16_t *f = (uint16_t *)(wsb + pl.off_f);
    hipError_t e;
    if (pl.skinny) {
        StreamParams p;
        memset(&p, 0, sizeof p);
        p.w = (const uint16_t *)(w->w_fc_stream ? w->w_fc_stream : w->w_fc);
        p.w_tiled = w->w_fc_stream ? 1 : 0;
        p.x = (const uint16_t *)hidden;
        p.ldx = ld;
        p.M = (int32_t)pl.M;
        p.K = (int32_t)K;
        p.O = (int32_t)H;
        p.S = 1;
        p.nbs = (int32_t)(K / 128);
        p.out = f;
        p.ss_out = (float *)(wsb + pl.off_ss);
        e = launch_stream(p, s);
    } else {
        float *part = pl.S_fc > 1 ? (float *)(wsb + pl.off_part) : nullptr;
        const bool packed = w->w_fc_packed != nullptr;
        GemmParams t{(const uint16_t *)hidden, ld, (const uint16_t *)(packed ? w->w_fc_packed : w->w_fc), f, H, part,
                     (int32_t)pl.M, (int32_t)K, (int32_t)H, (int32_t)pl.S_fc, packed ? 1 : 0};
        e = launch_gemm(t, s);
    }
    if (e != hipSuccess) return hip_status(e);
    if (stages_g(pl)) return DFKV_OK;
    uint16_t *gb = (uint16_t *)(wsb + pl.off_g);
    const float *part = !pl.skinny && pl.S_fc > 1 ? (const float *)(wsb + pl.off_part) : nullptr;
    return hip_status(
        launch_hidden_norm(f, part, pl.S_fc, (const uint16_t *)w->w_hnorm, gb, (int)pl.M, (int)H, g->eps, pl.kv_w, s));
}

dfkv_status run_kvfin(const dfkv_geom *g, const dfkv_weights *w, const int32_t *ctx, const float *cs,
                      int32_t cache_len, void *kv_out, bool fuse, void *ws, const Plan &pl, FinalizeParams fin,
                      hipStream_t s);

dfkv_status run_kv(const dfkv_geom *g, const dfkv_weights *w, const int32_t *ctx, const float *cs, int32_t cache_len,
                   void *kv_out, bool fuse, void *ws, const Plan &pl, FinalizeParams fin, bool need_finalize,
                   hipStream_t s) {
    if (pl.M == 0) return DFKV_OK;
    char *wsb = (char *)ws;
    const int64_t H = g->hidden, O = out_dim(g);
    hipError_t e;
    if (pl.kvfin) return run_kvfin(g, w, ctx, cs, cache_len, kv_out, fuse, ws, pl, fin, s);
    fin.nr = nr_geom(g, w->w_knorm, ctx, cs, cache_len);
    fin.norm = fuse ? 1 : 0;
    fin.kv_out = (uint16_t *)kv_out;
    if (pl.skinny) {
        StreamParams p;
        memset(&p, 0, sizeof p);
        p.w = (const uint16_t *)(w->w_kv_stream ? w->w_kv_stream : w->w_kv);
        p.w_tiled = w->w_kv_stream ? 1 : 0;
        p.ldx = H;
        p.M = (int32_t)pl.M;
        p.K = (int32_t)H;
        p.O = (int32_t)O;
        p.S = pl.S_kv;
        p.nbs = (int32_t)(H / 128 / pl.S_kv);
        p.part = (float *)(wsb + pl.off_part);
        if (stages_g(pl)) {
            p.x = (const uint16_t *)(wsb + pl.off_f);
            p.w_hn = (const uint16_t *)w->w_hnorm;
            p.ss_in = (const float *)(wsb + pl.off_ss);
            p.T_in = (int32_t)(H / 16);
            p.eps = g->eps;
        } else {
            p.x = (const uint16_t *)(wsb + pl.off_g);
        }
        if ((e = launch_stream(p, s)) != hipSuccess) return hip_status(e);
        fin.part = p.part;
        fin.S = pl.S_kv;
        fin.src = nullptr;
        return hip_status(launch_finalize(fin, s));
    }
    const uint16_t *gb = (const uint16_t *)(wsb + pl.off_g);
    GemmParams t2{gb, H, (const uint16_t *)w->w_kv, (uint16_t *)kv_out, O, nullptr, (int32_t)pl.M, (int32_t)H,
                  (int32_t)O, 1};
    if ((e = pl.kv_w ? launch_gemm_w(t2, s) : launch_gemm(t2, s)) != hipSuccess) return hip_status(e);
    if (!fuse && !need_finalize) return DFKV_OK;
    fin.part = nullptr;
    fin.src = (const uint16_t *)kv_out;  // in place: each element is read and written by one thread
    return hip_status(launch_finalize(fin, s));
}

// The K/V stage at <= 16 rows (k_kvgroups then k_kvfinal): hidden_norm, the K/V GEMM, k_norm/RoPE
// into kv_out and, when `fin` asks for them, the paged store and the advance; on f and its
// statistics left in ws by the fc stage.
dfkv_status run_kvfin(const dfkv_geom *g, const dfkv_weights *w, const int32_t *ctx, const float *cs,
                      int32_t cache_len, void *kv_out, bool fuse, void *ws, const Plan &pl, FinalizeParams fin,
                      hipStream_t s) {
    char *wsb = (char *)ws;
    const int64_t H = g->hidden, O = out_dim(g);
    KvParams kp;
    memset(&kp, 0, sizeof kp);
    kp.kv.w = (const uint16_t *)(w->w_kv_stream ? w->w_kv_stream : w->w_kv);
    kp.kv.w_tiled = w->w_kv_stream ? 1 : 0;
    kp.kv.x = (const uint16_t *)(wsb + pl.off_f);
    kp.kv.ldx = H;
    kp.kv.M = (int32_t)pl.M;
    kp.kv.K = (int32_t)H;
    kp.kv.O = (int32_t)O;
    kp.kv.S = pl.S_kv;
    kp.kv.nbs = (int32_t)(H / 128 / pl.S_kv);
    kp.kv.part = (float *)(wsb + pl.off_part);
    kp.kv.w_hn = (const uint16_t *)w->w_hnorm;
    kp.kv.ss_in = (const float *)(wsb + pl.off_ss);
    kp.kv.T_in = (int32_t)(H / 16);
    kp.kv.eps = g->eps;
    fin.nr = nr_geom(g, w->w_knorm, ctx, cs, cache_len);
    fin.norm = fuse ? 1 : 0;
    fin.kv_out = (uint16_t *)kv_out;
    fin.part = kp.kv.part;
    fin.S = pl.S_kv;
    fin.M = (int32_t)pl.M;
    fin.src = nullptr;
    // the kernel reads the pre-step ctx_len once, for RoPE and for the bookkeeping alike
    if ((fin.store || fin.advance) && fin.ctx_len != ctx) return DFKV_ERR_SHAPE;
    kp.fin = fin;
    kp.book = wsb + pl.off_book;
    kp.ntg = pl.ntg;
    kp.n_groups = (int32_t)(O / 16 / pl.ntg) * pl.S_kv;
    kp.unit_cols = g->kind == DFKV_GQA ? g->head_dim : per_layer(g);
    kp.n_units = (int32_t)(O / kp.unit_cols);
    return hip_status(launch_kv(kp, s));
}

dfkv_status run_project(const dfkv_geom *g, const dfkv_weights *w, const void *hidden, int64_t ld, const int32_t *ctx,
                        const float *cs, int32_t cache_len, void *kv_out, bool fuse, void *ws, const Plan &pl,
                        const FinalizeParams &fin, bool need_finalize, hipStream_t s) {
    if (pl.M == 0) return DFKV_OK;
    dfkv_status st = run_fc(g, w, hidden, ld, ws, pl, s);
    if (st != DFKV_OK) return st;
    return run_kv(g, w, ctx, cs, cache_len, kv_out, fuse, ws, pl, fin, need_finalize, s);
}

}  // namespace

extern "C" {

const char *dfkv_status_string(dfkv_status s) {
    switch (s) {
        case DFKV_OK: return "DFKV_OK";
        case DFKV_ERR_NULL: return "DFKV_ERR_NULL: a required pointer is NULL";
        case DFKV_ERR_SHAPE: return "DFKV_ERR_SHAPE: unsupported or inconsistent sizes";
        case DFKV_ERR_LAYOUT: return "DFKV_ERR_LAYOUT: misaligned pointer or bad stride";
        case DFKV_ERR_ALIAS: return "DFKV_ERR_ALIAS: an output overlaps an input";
        case DFKV_ERR_WORKSPACE: return "DFKV_ERR_WORKSPACE: workspace too small";
        case DFKV_ERR_HIP: return "DFKV_ERR_HIP: kernel launch failed";
    }
    return "unknown dfkv_status";
}

const char *dfkv_version(void) { return "libdfkv 0.1 (gfx950)"; }

const char *dfkv_hip_error_string(void) { return hipGetErrorString(g_last_hip_error); }

dfkv_status dfkv_workspace_size(const dfkv_geom *g, int32_t n_reqs, size_t *bytes) {
    if (!g || !bytes) return DFKV_ERR_NULL;
    Plan pl;
    dfkv_status st = make_plan(g, n_reqs, &pl);
    if (st != DFKV_OK) return st;
    *bytes = pl.total;
    return DFKV_OK;
}

dfkv_status dfkv_workspace_init(void *ws, size_t ws_bytes, dfkv_stream_t stream) {
    if (!ws) return DFKV_ERR_NULL;
    if (!al16(ws)) return DFKV_ERR_LAYOUT;
    return hip_status(launch_fill_zero(ws, ws_bytes, (hipStream_t)stream));
}

dfkv_status dfkv_rope_cache_build(const dfkv_rope *rope, float *cos_sin, int32_t cache_len, dfkv_stream_t stream) {
    if (!rope || !cos_sin) return DFKV_ERR_NULL;
    if (rope->rot <= 0 || rope->rot % 2 || rope->rot > 1024 || cache_len <= 0) return DFKV_ERR_SHAPE;
    if (!(rope->theta > 1.0)) return DFKV_ERR_SHAPE;
    if (rope->yarn && (!(rope->factor > 0.0) || !(rope->orig_ctx > 0.0) || !(rope->beta_fast > 0.0) ||
                       !(rope->beta_slow > 0.0)))
        return DFKV_ERR_SHAPE;
    if (!al4(cos_sin)) return DFKV_ERR_LAYOUT;
    return hip_status(launch_rope_cache(*rope, cos_sin, cache_len, (hipStream_t)stream));
}

dfkv_status dfkv_project(const dfkv_geom *g, const dfkv_weights *w, const void *hidden, int64_t hidden_row_stride,
                         int32_t n_reqs, const int32_t *ctx_len_in, const float *cos_sin, int32_t cache_len,
                         void *kv_out, uint32_t flags, void *ws, size_t ws_bytes, dfkv_stream_t stream) {
    Plan pl;
    dfkv_status st = check_project(g, w, hidden, hidden_row_stride, n_reqs, ctx_len_in, cos_sin, cache_len, kv_out,
                                   flags, ws, ws_bytes, &pl);
    if (st != DFKV_OK) return st;
    const FinalizeParams fin = fin_params(g, nullptr, nullptr, nullptr, n_reqs);
    return run_project(g, w, hidden, hidden_row_stride, ctx_len_in, cos_sin, cache_len, kv_out,
                       (flags & DFKV_FUSE_NORM_ROPE) != 0, ws, pl, fin, false, (hipStream_t)stream);
}

dfkv_status dfkv_project_fork(const dfkv_geom *g, const dfkv_weights *w, const void *hidden,
                              int64_t hidden_row_stride, int32_t n_reqs, const int32_t *ctx_len_in,
                              const float *cos_sin, int32_t cache_len, void *kv_out, uint32_t flags, void *ws,
                              size_t ws_bytes, dfkv_stream_t main, dfkv_stream_t aux, void *fork, void *join) {
    Plan pl;
    const bool recorded = (flags & DFKV_FORK_RECORDED) != 0;
    flags &= ~(uint32_t)DFKV_FORK_RECORDED;
    dfkv_status st = check_project(g, w, hidden, hidden_row_stride, n_reqs, ctx_len_in, cos_sin, cache_len, kv_out,
                                   flags, ws, ws_bytes, &pl);
    if (st != DFKV_OK) return st;
    if (!fork || !join) return DFKV_ERR_NULL;
    hipError_t e = recorded ? hipSuccess : hipEventRecord((hipEvent_t)fork, (hipStream_t)main);
    if (e == hipSuccess) e = hipStreamWaitEvent((hipStream_t)aux, (hipEvent_t)fork, 0);
    if (e != hipSuccess) return hip_status(e);
    const FinalizeParams fin = fin_params(g, nullptr, nullptr, nullptr, n_reqs);
    st = run_project(g, w, hidden, hidden_row_stride, ctx_len_in, cos_sin, cache_len, kv_out,
                     (flags & DFKV_FUSE_NORM_ROPE) != 0, ws, pl, fin, false, (hipStream_t)aux);
    if (st != DFKV_OK) return st;
    return hip_status(hipEventRecord((hipEvent_t)join, (hipStream_t)aux));
}

dfkv_status dfkv_block_table_decode(const int32_t *offsets, int64_t off_stride_req, int64_t off_stride_blk,
                                    int32_t n_reqs, int32_t max_blocks, const int32_t *n_tokens, int32_t page_size,
                                    int32_t divisor, int32_t *page_count_out, int32_t *table_out,
                                    int64_t table_row_stride, dfkv_stream_t stream) {
    if (n_reqs < 0 || max_blocks < 0 || page_size <= 0 || divisor <= 0) return DFKV_ERR_SHAPE;
    if (n_reqs == 0) return DFKV_OK;
    if (!n_tokens || !page_count_out || (max_blocks > 0 && (!offsets || !table_out))) return DFKV_ERR_NULL;
    if (off_stride_req < 0 || off_stride_blk < 0 || table_row_stride < max_blocks) return DFKV_ERR_LAYOUT;
    const int64_t B = n_reqs;
    const size_t off_b = max_blocks > 0 ? extent2(off_stride_req, B, off_stride_blk, max_blocks) : 0;
    const size_t tbl_b = max_blocks > 0 ? (size_t)((B - 1) * table_row_stride + max_blocks) * 4 : 0;
    const size_t cnt_b = (size_t)B * 4, nt_b = (size_t)B * 4;
    if (overlap(page_count_out, cnt_b, n_tokens, nt_b) || overlap(page_count_out, cnt_b, offsets, off_b) ||
        overlap(table_out, tbl_b, n_tokens, nt_b) || overlap(table_out, tbl_b, offsets, off_b) ||
        overlap(table_out, tbl_b, page_count_out, cnt_b))
        return DFKV_ERR_ALIAS;
    BtDecodeArgs a{offsets, off_stride_req, off_stride_blk, n_tokens, n_reqs, max_blocks, page_size, divisor,
                   page_count_out, table_out, table_row_stride};
    return hip_status(launch_bt_decode(a, (hipStream_t)stream));
}

dfkv_status dfkv_strict_accept(const int32_t *target, int64_t t_stride_req, int64_t t_stride_tok,
                               const int32_t *draft, int64_t d_stride_req, int64_t d_stride_tok, int32_t n_reqs,
                               int32_t width, int32_t *n_acc_out, int32_t *accepted_out, dfkv_stream_t stream) {
    if (n_reqs < 0 || width < 1) return DFKV_ERR_SHAPE;
    if (n_reqs == 0) return DFKV_OK;
    if (!target || !n_acc_out || !accepted_out || (width > 1 && !draft)) return DFKV_ERR_NULL;
    if (t_stride_req < 0 || t_stride_tok < 0 || d_stride_req < 0 || d_stride_tok < 0) return DFKV_ERR_LAYOUT;
    const int64_t B = n_reqs;
    const size_t t_b = extent2(t_stride_req, B, t_stride_tok, width);
    const size_t d_b = width > 1 ? extent2(d_stride_req, B, d_stride_tok, width - 1) : 0;
    const size_t n_b = (size_t)B * 4, a_b = (size_t)(B * width) * 4;
    if (overlap(n_acc_out, n_b, target, t_b) || overlap(n_acc_out, n_b, draft, d_b) ||
        overlap(accepted_out, a_b, target, t_b) || overlap(accepted_out, a_b, draft, d_b) ||
        overlap(accepted_out, a_b, n_acc_out, n_b))
        return DFKV_ERR_ALIAS;
    AcceptArgs a{target, t_stride_req, t_stride_tok, draft, d_stride_req, d_stride_tok, n_reqs, width, n_acc_out,
                 accepted_out};
    return hip_status(launch_strict_accept(a, (hipStream_t)stream));
}

dfkv_status dfkv_join(dfkv_stream_t main, void *join) {
    if (!join) return DFKV_ERR_NULL;
    return hip_status(hipStreamWaitEvent((hipStream_t)main, (hipEvent_t)join, 0));
}

dfkv_status dfkv_project_fc(const dfkv_geom *g, const dfkv_weights *w, const void *hidden,
                            int64_t hidden_row_stride, int32_t n_reqs, void *ws, size_t ws_bytes,
                            dfkv_stream_t stream) {
    if (!g || !w) return DFKV_ERR_NULL;
    Plan pl;
    dfkv_status st = make_plan(g, n_reqs, &pl);
    if (st != DFKV_OK) return st;
    if (pl.M == 0) return DFKV_OK;
    if (!w->w_fc || !hidden || !ws || !w->w_hnorm) return DFKV_ERR_NULL;
    const int64_t K = k_in(g), H = g->hidden, M = pl.M;
    if (hidden_row_stride < K || (hidden_row_stride * 2) % 16 != 0) return DFKV_ERR_LAYOUT;
    if (!al16(hidden) || !al16(w->w_fc) || !al16(ws) || !al16(w->w_hnorm)) return DFKV_ERR_LAYOUT;
    if (w->w_fc_packed && !al16(w->w_fc_packed)) return DFKV_ERR_LAYOUT;
    if ((st = check_stream_weights(g, w, true, false, false, nullptr, 0, nullptr, 0)) != DFKV_OK) return st;
    if (ws_bytes < pl.total) return DFKV_ERR_WORKSPACE;
    const size_t hid_bytes = (size_t)((M - 1) * hidden_row_stride + K) * 2;
    if (overlap(ws, ws_bytes, hidden, hid_bytes) || overlap(ws, ws_bytes, w->w_fc, (size_t)H * K * 2) ||
        overlap(ws, ws_bytes, w->w_hnorm, (size_t)H * 2) ||
        (w->w_fc_packed && overlap(ws, ws_bytes, w->w_fc_packed, (size_t)H * K * 2)))
        return DFKV_ERR_ALIAS;
    if ((st = check_stream_weights(g, w, true, false, true, nullptr, 0, ws, ws_bytes)) != DFKV_OK) return st;
    return run_fc(g, w, hidden, hidden_row_stride, ws, pl, (hipStream_t)stream);
}

dfkv_status dfkv_pack_fc_weight(const dfkv_geom *g, const void *w_fc, void *w_fc_packed, dfkv_stream_t stream) {
    if (!g || !w_fc || !w_fc_packed) return DFKV_ERR_NULL;
    dfkv_status st = check_geom(g);
    if (st != DFKV_OK) return st;
    if (!al16(w_fc) || !al16(w_fc_packed)) return DFKV_ERR_LAYOUT;
    const int64_t K = k_in(g), H = g->hidden;
    if (overlap(w_fc, (size_t)H * K * 2, w_fc_packed, (size_t)H * K * 2)) return DFKV_ERR_ALIAS;
    return hip_status(launch_pack_rows((const uint16_t *)w_fc, (uint16_t *)w_fc_packed, H, K, (hipStream_t)stream));
}

dfkv_status dfkv_pack_stream_weight(int64_t rows, int64_t cols, const void *w, void *w_stream, dfkv_stream_t stream) {
    if (!w || !w_stream) return DFKV_ERR_NULL;
    if (rows <= 0 || cols <= 0 || rows % 16 != 0 || cols % 128 != 0 || rows > (1 << 24) || cols > (1 << 24))
        return DFKV_ERR_SHAPE;
    if (!al16(w) || !al16(w_stream)) return DFKV_ERR_LAYOUT;
    const size_t bytes = (size_t)rows * (size_t)cols * 2;
    if (overlap(w, bytes, w_stream, bytes)) return DFKV_ERR_ALIAS;
    return hip_status(launch_pack_stream((const uint16_t *)w, (uint16_t *)w_stream, rows, cols, (hipStream_t)stream));
}

dfkv_status dfkv_project_kv(const dfkv_geom *g, const dfkv_weights *w, int32_t n_reqs, const int32_t *ctx_len_in,
                            const float *cos_sin, int32_t cache_len, void *kv_out, uint32_t flags, void *ws,
                            size_t ws_bytes, dfkv_stream_t stream) {
    if (!g || !w) return DFKV_ERR_NULL;
    Plan pl;
    dfkv_status st = make_plan(g, n_reqs, &pl);
    if (st != DFKV_OK) return st;
    if ((flags & ~(uint32_t)DFKV_FUSE_NORM_ROPE) != 0) return DFKV_ERR_SHAPE;
    if (pl.M == 0) return DFKV_OK;
    const bool fuse = (flags & DFKV_FUSE_NORM_ROPE) != 0;
    if (!kv_out || !w->w_hnorm || !w->w_kv || !ws) return DFKV_ERR_NULL;
    if (fuse && (!w->w_knorm || !ctx_len_in || !cos_sin)) return DFKV_ERR_NULL;
    if (fuse && cache_len <= 0) return DFKV_ERR_SHAPE;
    const int64_t H = g->hidden, O = out_dim(g), M = pl.M;
    if (!al16(kv_out) || !al16(w->w_hnorm) || !al16(w->w_kv) || !al16(ws)) return DFKV_ERR_LAYOUT;
    if (fuse && (!al4(cos_sin) || ((uintptr_t)w->w_knorm & 1u))) return DFKV_ERR_LAYOUT;
    if ((st = check_stream_weights(g, w, false, true, false, nullptr, 0, nullptr, 0)) != DFKV_OK) return st;
    if (ws_bytes < pl.total) return DFKV_ERR_WORKSPACE;
    const size_t kv_bytes = (size_t)M * O * 2;
    if (overlap(kv_out, kv_bytes, ws, ws_bytes) || overlap(kv_out, kv_bytes, w->w_kv, (size_t)O * H * 2) ||
        overlap(kv_out, kv_bytes, w->w_hnorm, (size_t)H * 2))
        return DFKV_ERR_ALIAS;
    if ((st = check_stream_weights(g, w, false, true, true, kv_out, kv_bytes, ws, ws_bytes)) != DFKV_OK) return st;
    if (fuse) {
        const size_t kn = (size_t)g->n_layers * (g->kind == DFKV_GQA ? g->head_dim : g->latent_dim) * 2;
        if (overlap(kv_out, kv_bytes, cos_sin, (size_t)cache_len * g->rope_dim * 4) ||
            overlap(kv_out, kv_bytes, w->w_knorm, kn) || overlap(kv_out, kv_bytes, ctx_len_in, (size_t)n_reqs * 4))
            return DFKV_ERR_ALIAS;
    }
    const FinalizeParams fin = fin_params(g, nullptr, nullptr, nullptr, n_reqs);
    return run_kv(g, w, ctx_len_in, cos_sin, cache_len, kv_out, fuse, ws, pl, fin, false, (hipStream_t)stream);
}

dfkv_status dfkv_norm_rope(const dfkv_geom *g, const void *w_knorm, int32_t n_reqs, const int32_t *ctx_len_in,
                           const float *cos_sin, int32_t cache_len, void *kv, dfkv_stream_t stream) {
    dfkv_status st = check_geom(g);
    if (st != DFKV_OK) return st;
    if (n_reqs < 0 || cache_len <= 0) return DFKV_ERR_SHAPE;
    const int64_t N = (int64_t)n_reqs * g->width;
    if (N == 0) return DFKV_OK;
    if (!w_knorm || !ctx_len_in || !cos_sin || !kv) return DFKV_ERR_NULL;
    if (!al16(kv) || !al4(cos_sin) || ((uintptr_t)w_knorm & 1u)) return DFKV_ERR_LAYOUT;
    const size_t kvb = (size_t)N * out_dim(g) * 2;
    const size_t kn = (size_t)g->n_layers * (g->kind == DFKV_GQA ? g->head_dim : g->latent_dim) * 2;
    if (overlap(kv, kvb, cos_sin, (size_t)cache_len * g->rope_dim * 4) || overlap(kv, kvb, w_knorm, kn) ||
        overlap(kv, kvb, ctx_len_in, (size_t)n_reqs * 4))
        return DFKV_ERR_ALIAS;
    FinalizeParams fin = fin_params(g, nullptr, nullptr, nullptr, n_reqs);
    fin.nr = nr_geom(g, w_knorm, ctx_len_in, cos_sin, cache_len);
    fin.norm = 1;
    fin.src = (const uint16_t *)kv;
    fin.kv_out = (uint16_t *)kv;  // in place: each element is read and written by one thread
    return hip_status(launch_finalize(fin, (hipStream_t)stream));
}

dfkv_status dfkv_paged_store(const dfkv_geom *g, const void *kv, const dfkv_requests *req, const dfkv_pool *pool,
                             int64_t *slot_out, uint8_t *write_mask_out, dfkv_stream_t stream) {
    dfkv_status st = check_geom(g);
    if (st != DFKV_OK) return st;
    if ((st = check_requests(g, req, true, false)) != DFKV_OK) return st;
    if (req->n_reqs == 0) return DFKV_OK;
    if ((st = check_pool(g, pool)) != DFKV_OK) return st;
    if ((st = check_store_outputs(g, req, pool, kv, slot_out, write_mask_out)) != DFKV_OK) return st;
    FinalizeParams p = fin_params(g, req, pool, nullptr, 0);
    p.slot = slot_out;
    p.wmask = write_mask_out;
    p.src = (const uint16_t *)kv;
    p.store = 1;
    return hip_status(launch_finalize(p, (hipStream_t)stream));
}

dfkv_status dfkv_paged_store_rows(const dfkv_geom *g, const void *kv, int32_t n_rows, const int32_t *row_req,
                                  const int32_t *row_pos, int32_t n_reqs, const int32_t *alloc_limit,
                                  const int32_t *block_table, int64_t bt_row_stride, int32_t bt_cols,
                                  const dfkv_pool *pool, int64_t *slot_out, uint8_t *write_mask_out,
                                  dfkv_stream_t stream) {
    dfkv_status st = check_geom(g);
    if (st != DFKV_OK) return st;
    if (n_rows < 0 || n_reqs < 0) return DFKV_ERR_SHAPE;
    if (n_rows == 0) return DFKV_OK;
    if (!row_req || !row_pos || (n_reqs > 0 && (!alloc_limit || !block_table))) return DFKV_ERR_NULL;
    if (n_reqs > 0 && (bt_cols <= 0 || bt_row_stride < bt_cols)) return DFKV_ERR_LAYOUT;
    if ((st = check_pool(g, pool)) != DFKV_OK) return st;
    if ((st = check_store_outputs_n(g, n_rows, pool, kv, slot_out, write_mask_out)) != DFKV_OK) return st;
    const size_t nb = (size_t)n_rows * 4, rb = (size_t)n_reqs * 4;
    const size_t bb = n_reqs > 0 ? extent2(bt_row_stride, n_reqs, 1, bt_cols) : 0;
    const void *ins[4] = {row_req, row_pos, alloc_limit, block_table};
    const size_t ib[4] = {nb, nb, rb, bb};
    for (int j = 0; j < 4; ++j)
        if (overlap(slot_out, (size_t)n_rows * 8, ins[j], ib[j]) || overlap(write_mask_out, (size_t)n_rows, ins[j], ib[j]))
            return DFKV_ERR_ALIAS;
    FinalizeParams p = fin_params(g, nullptr, pool, nullptr, 0);
    p.M = n_rows;
    p.B = n_reqs;
    p.limit = alloc_limit;
    p.bt = block_table;
    p.bt_stride = bt_row_stride;
    p.bt_cols = bt_cols;
    p.row_req = row_req;
    p.row_pos = row_pos;
    p.slot = slot_out;
    p.wmask = write_mask_out;
    p.src = (const uint16_t *)kv;
    p.store = 1;
    return hip_status(launch_store_rows(p, (hipStream_t)stream));
}

dfkv_status dfkv_advance(const dfkv_geom *g, const dfkv_requests *req, const dfkv_outputs *out, dfkv_stream_t stream) {
    dfkv_status st = check_geom(g);
    if (st != DFKV_OK) return st;
    if ((st = check_requests(g, req, false, true)) != DFKV_OK) return st;
    if (out && out->block_slot) return DFKV_ERR_SHAPE;   // the placement needs the pool's page count
    if (req->n_reqs == 0) return DFKV_OK;
    if ((st = check_adv_outputs(g, req, out)) != DFKV_OK) return st;
    const FinalizeParams p = fin_params(g, req, nullptr, out, 0);
    return hip_status(launch_advance(p, (hipStream_t)stream));
}

static dfkv_status check_store_advance(const dfkv_geom *g, const void *kv, const dfkv_requests *req,
                                       const dfkv_pool *pool, const dfkv_outputs *out) {
    dfkv_status st = check_geom(g);
    if (st != DFKV_OK) return st;
    if ((st = check_requests(g, req, true, true)) != DFKV_OK) return st;
    if (req->n_reqs == 0) return DFKV_OK;
    if (!out) return DFKV_ERR_NULL;
    if ((st = check_pool(g, pool)) != DFKV_OK) return st;
    if ((st = check_store_outputs(g, req, pool, kv, out->slot, out->write_mask)) != DFKV_OK) return st;
    if ((st = check_adv_outputs(g, req, out)) != DFKV_OK) return st;
    const int64_t N = (int64_t)req->n_reqs * g->width;
    const size_t pb = pool_bytes(g, pool);
    const void *outs[6] = {out->c_pos, out->bonus, out->emb_ids, out->q_pos, out->ctx_len_out, out->seq_len};
    const size_t ob[6] = {(size_t)N * 4, (size_t)req->n_reqs * 4, (size_t)req->n_reqs * g->block_size * 4,
                          (size_t)req->n_reqs * g->block_size * 4, (size_t)req->n_reqs * 4, (size_t)req->n_reqs * 4};
    for (int i = 0; i < 6; ++i) {
        if (overlap(outs[i], ob[i], kv, (size_t)N * out_dim(g) * 2) || overlap(outs[i], ob[i], out->slot, (size_t)N * 8) ||
            overlap(outs[i], ob[i], out->write_mask, (size_t)N))
            return DFKV_ERR_ALIAS;
        for (int l = 0; l < g->n_layers; ++l) {
            if (overlap(outs[i], ob[i], pool->k[l], pb)) return DFKV_ERR_ALIAS;
            if (g->kind == DFKV_GQA && overlap(outs[i], ob[i], pool->v[l], pb)) return DFKV_ERR_ALIAS;
        }
    }
    return DFKV_OK;
}

dfkv_status dfkv_store_advance(const dfkv_geom *g, const void *kv, const dfkv_requests *req, const dfkv_pool *pool,
                               const dfkv_outputs *out, dfkv_stream_t stream) {
    dfkv_status st = check_store_advance(g, kv, req, pool, out);
    if (st != DFKV_OK) return st;
    if (req->n_reqs == 0) return DFKV_OK;
    FinalizeParams p = fin_params(g, req, pool, out, 0);
    p.src = (const uint16_t *)kv;
    p.store = 1;
    p.advance = 1;
    return hip_status(launch_finalize(p, (hipStream_t)stream));
}

dfkv_status dfkv_step(const dfkv_geom *g, const dfkv_weights *w, const void *hidden, int64_t hidden_row_stride,
                      const dfkv_requests *req, const float *cos_sin, int32_t cache_len, void *kv_out,
                      const dfkv_pool *pool, const dfkv_outputs *out, void *ws, size_t ws_bytes, dfkv_stream_t stream) {
    if (!req) return DFKV_ERR_NULL;
    Plan pl;
    dfkv_status st = check_project(g, w, hidden, hidden_row_stride, req->n_reqs, req->ctx_len_in, cos_sin, cache_len,
                                   kv_out, DFKV_FUSE_NORM_ROPE, ws, ws_bytes, &pl);
    if (st != DFKV_OK) return st;
    if ((st = check_store_advance(g, kv_out, req, pool, out)) != DFKV_OK) return st;
    if (req->n_reqs == 0) return DFKV_OK;
    // the bookkeeping outputs must not land in the projection's inputs or workspace either
    const int64_t N = (int64_t)req->n_reqs * g->width;
    const void *outs[8] = {out->slot, out->write_mask, out->c_pos, out->bonus, out->emb_ids, out->q_pos,
                           out->ctx_len_out, out->seq_len};
    const size_t ob[8] = {(size_t)N * 8, (size_t)N, (size_t)N * 4, (size_t)req->n_reqs * 4,
                          (size_t)req->n_reqs * g->block_size * 4, (size_t)req->n_reqs * g->block_size * 4,
                          (size_t)req->n_reqs * 4, (size_t)req->n_reqs * 4};
    const size_t hid_bytes = (size_t)((N - 1) * hidden_row_stride + k_in(g)) * 2;
    for (int i = 0; i < 8; ++i)
        if (overlap(outs[i], ob[i], ws, ws_bytes) || overlap(outs[i], ob[i], hidden, hid_bytes) ||
            overlap(outs[i], ob[i], cos_sin, (size_t)cache_len * g->rope_dim * 4))
            return DFKV_ERR_ALIAS;
    // projection with the finalize kernel doing k_norm/RoPE, the store and the advance
    FinalizeParams fin = fin_params(g, req, pool, out, 0);
    fin.store = 1;
    fin.advance = 1;
    return run_project(g, w, hidden, hidden_row_stride, req->ctx_len_in, cos_sin, cache_len, kv_out, true, ws, pl,
                       fin, true, (hipStream_t)stream);
}

dfkv_status dfkv_step_noalloc(const dfkv_geom *g, const dfkv_weights *w, const void *hidden,
                              int64_t hidden_row_stride, const dfkv_requests *req, const float *cos_sin,
                              int32_t cache_len, void *kv_out, const dfkv_pool *pool, const dfkv_outputs *out,
                              dfkv_stream_t stream) {
    if (!g || !req) return DFKV_ERR_NULL;
    Plan pl;
    dfkv_status st = make_plan(g, req->n_reqs, &pl);
    if (st != DFKV_OK) return st;
    if (pl.total > (size_t)DFKV_NOALLOC_SCRATCH_BYTES) return DFKV_ERR_WORKSPACE;
    void *ws = nullptr;
    const hipError_t e = scratch_address((hipStream_t)stream, &ws);
    if (e != hipSuccess) return hip_status(e);
    // the same validation and kernels as dfkv_step, on this device's scratch (nothing in it needs
    // clearing: every byte a kernel reads there was written earlier in the same call)
    return dfkv_step(g, w, hidden, hidden_row_stride, req, cos_sin, cache_len, kv_out, pool, out, ws,
                     (size_t)DFKV_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
