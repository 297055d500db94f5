// cache.cpp -- the KV cache of include/kivi_cache.h: layout of the stores and
// fp16 residual rings in one caller-owned device buffer, the flush rule, and
// the per-step append / attend / end-of-step calls.  Host code only; the
// kernels are the flush and attend kernels of the library plus the row copy
// in cache.hip.  Every call validates everything before its first launch.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kivi.h"
#include "kivi_cache.h"
#include "kivi_launch.h"

namespace {

constexpr int64_t kMaxTokens = int64_t{1} << 24;      // the attend's 32-bit offsets
constexpr int64_t kMaxSlabs = int64_t{1} << 31;

int64_t align256(int64_t x) { return (x + 255) & ~int64_t{255}; }

struct Layout {
    int64_t slabs, ring, words;
    int64_t kc, ks, kz, vc, vs, vz, kr, vr, kst, vst, total;    // byte offsets / size
};

bool valid(const kivi_cache_config* c) {
    if (!c) return false;
    if (c->layers < 1 || c->layers > KIVI_CACHE_MAX_LAYERS || c->batch < 1 || c->kv_heads < 1) return false;
    if (c->bits != 2 && c->bits != 4) return false;
    // the store geometries: head_dim 128 with groups of 32, 64 or 128 (binary16
    // scale/zero included); any other multiple of 16 up to 256 with groups of
    // 32 and binary32 scale/zero
    const int32_t D = c->head_dim, G = c->group_size;
    if (D == 128) {
        if (G != 32 && G != 64 && G != 128) return false;
    } else if (D < 16 || D > 256 || D % 16 != 0 || G != 32 || c->meta_format != KIVI_META_F32) {
        return false;
    }
    if (c->flush_tokens <= 0 || c->flush_tokens % c->group_size != 0) return false;
    if (c->residual_length < 0 || c->residual_length % c->flush_tokens != 0) return false;
    if (c->store_capacity < 0 || c->store_capacity % c->flush_tokens != 0) return false;
    if (c->meta_format != KIVI_META_F32 && c->meta_format != KIVI_META_F16) return false;
    if (c->bf16 != 0 && c->bf16 != 1) return false;
    if (c->bf16 && c->meta_format != KIVI_META_F32) return false;    // as for the _bf16 flushes
    if (c->store_capacity >= kMaxTokens) return false;
    if (int64_t{c->residual_length} + c->flush_tokens >= kMaxTokens) return false;
    const int64_t slabs = int64_t{c->layers} * c->batch * c->kv_heads;
    return slabs < kMaxSlabs;
}

Layout layout(const kivi_cache_config& c) {
    Layout L;
    L.slabs = int64_t{c.layers} * c.batch * c.kv_heads;
    L.ring = int64_t{c.residual_length} + c.flush_tokens;
    const int64_t kD = c.head_dim;
    L.words = kD * c.bits / 32;
    const int64_t cap = c.store_capacity;
    const int64_t mb = c.meta_format == KIVI_META_F16 ? 2 : 4;     // bytes per scale/zero entry
    int64_t off = 0;
    auto take = [&off](int64_t bytes) { const int64_t at = off; off = align256(off + bytes); return at; };
    L.kc = take(L.slabs * cap * L.words * 4);
    const int64_t G = c.group_size;
    L.ks = take(L.slabs * (cap / G) * kD * mb);
    L.kz = take(L.slabs * (cap / G) * kD * mb);
    L.vc = take(L.slabs * cap * L.words * 4);
    L.vs = take(L.slabs * cap * ((kD + G - 1) / G) * mb);
    L.vz = take(L.slabs * cap * ((kD + G - 1) / G) * mb);
    L.kr = take(L.slabs * L.ring * kD * 2);
    L.vr = take(L.slabs * L.ring * kD * 2);
    L.kst = take(L.slabs * L.ring * kD * 2);      // staging for a prompt chunk's first groups
    L.vst = take(L.slabs * L.ring * kD * 2);
    L.total = off;
    return L;
}

int64_t seq_slabs(const kivi_cache* c) { return int64_t{c->cfg.batch} * c->cfg.kv_heads; }

bool appended(const kivi_cache* c, int layer) { return (c->appended[layer >> 6] >> (layer & 63)) & 1u; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int finish(hipError_t e) { return kivi::hip_status(e); }

// The slabs of one layer as a store of their own.
kivi_store layer_store(const kivi_store& s, int64_t slab0) {
    kivi_store r = s;
    const int64_t meta_bytes = (s.meta_format == KIVI_META_F16 ? 2 : 4) * slab0 * s.meta_bh_stride;
    r.codes = s.codes + slab0 * s.codes_bh_stride;
    r.scale = static_cast<char*>(s.scale) + meta_bytes;
    r.zero = static_cast<char*>(s.zero) + meta_bytes;
    return r;
}

// The flushes of the cache's format.
int flush_keys(const kivi_cache* c, const uint16_t* x, int64_t BH, int64_t S, int64_t stride,
               int64_t dst, hipStream_t stream) {
    return (c->cfg.bf16 ? kivi_quantize_keys_bf16 : kivi_quantize_keys)(x, BH, S, stride, &c->k_store,
                                                                       dst, nullptr, 0, stream);
}
int flush_values(const kivi_cache* c, const uint16_t* x, int64_t BH, int64_t S, int64_t stride,
                 int64_t dst, hipStream_t stream) {
    return (c->cfg.bf16 ? kivi_quantize_values_bf16 : kivi_quantize_values)(x, BH, S, stride, &c->v_store,
                                                                           dst, nullptr, 0, stream);
}

// Quantized tokens of a sequence of S tokens: the whole flush units older
// than the newest R tokens.
int64_t quantized_tokens(const kivi_cache_config& c, int64_t S) {
    if (S < c.residual_length) return 0;
    return (S - c.residual_length) / c.flush_tokens * c.flush_tokens;
}

}  // namespace

extern "C" {

size_t kivi_cache_device_bytes(const kivi_cache_config* cfg) {
    if (!valid(cfg)) return 0;
    return static_cast<size_t>(layout(*cfg).total);
}

int kivi_cache_init(kivi_cache* cache, const kivi_cache_config* cfg, void* device, size_t bytes) {
    if (!cache || !cfg || !device) return KIVI_ERR_NULL;
    if (!valid(cfg)) return KIVI_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(device) & 255u) != 0) return KIVI_ERR_ALIGN;
    const Layout L = layout(*cfg);
    if (bytes < static_cast<size_t>(L.total)) return KIVI_ERR_WORKSPACE;
    char* base = static_cast<char*>(device);
    kivi_cache c = {};
    c.cfg = *cfg;
    const int64_t cap = cfg->store_capacity;
    c.k_store = {reinterpret_cast<uint32_t*>(base + L.kc), base + L.ks, base + L.kz,
                 cap * L.words, (cap / cfg->group_size) * cfg->head_dim, cap,
                 cfg->bits, cfg->group_size, cfg->head_dim, KIVI_KEYS, cfg->meta_format};
    c.v_store = {reinterpret_cast<uint32_t*>(base + L.vc), base + L.vs, base + L.vz,
                 cap * L.words, cap * ((cfg->head_dim + cfg->group_size - 1) / cfg->group_size), cap,
                 cfg->bits, cfg->group_size, cfg->head_dim, KIVI_VALUES, cfg->meta_format};
    c.k_ring = reinterpret_cast<uint16_t*>(base + L.kr);
    c.v_ring = reinterpret_cast<uint16_t*>(base + L.vr);
    c.k_stage = reinterpret_cast<uint16_t*>(base + L.kst);
    c.v_stage = reinterpret_cast<uint16_t*>(base + L.vst);
    c.ring = L.ring;
    *cache = c;
    return KIVI_OK;
}

int kivi_cache_prefill(kivi_cache* cache, const uint16_t* k, const uint16_t* v,
                       int64_t x_bh_stride, int64_t S, hipStream_t stream) {
    if (!cache) return KIVI_ERR_NULL;
    if (!valid(&cache->cfg)) return KIVI_ERR_UNSUPPORTED;
    const int64_t kD = cache->cfg.head_dim;
    const int64_t G = cache->cfg.group_size;
    if (S < 0) return KIVI_ERR_SHAPE;
    for (uint64_t w : cache->appended)
        if (w) return KIVI_ERR_SHAPE;                  // a step is in progress
    const int64_t L0 = cache->length, Q0 = cache->n_quant, R0 = cache->n_res;
    if (S > kMaxTokens || L0 + S >= kMaxTokens) return KIVI_ERR_SHAPE;
    const int64_t L1 = L0 + S;
    const int64_t Q1 = quantized_tokens(cache->cfg, L1);
    if (Q1 > cache->cfg.store_capacity) return KIVI_ERR_SHAPE;
    if (S == 0) return KIVI_OK;
    const int64_t slabs = layout(cache->cfg).slabs;
    if (!k || !v) return KIVI_ERR_NULL;
    if (!aligned16(k) || !aligned16(v) || x_bh_stride % 8 != 0) return KIVI_ERR_ALIGN;
    if (slabs > 1 && x_bh_stride < S * kD) return KIVI_ERR_SHAPE;
    if ((slabs * ((S + cache->ring + 31) / 32) + 3) / 4 >= kMaxSlabs) return KIVI_ERR_SHAPE;
    if (slabs * (S + cache->ring) * (kD / 8) / 256 >= kMaxSlabs) return KIVI_ERR_SHAPE;

    // The flush takes tokens [Q0, Q1).  Its first groups may hold fp16
    // tokens still in the ring (ring rows head, head + 1, ... mod ring) and
    // the chunk's first tokens: tokens [Q0, A_end) with A_end the first group
    // boundary at or past L0 are assembled in the staging rows and flushed
    // from there; the rest, [A_end, Q1), lie in the chunk, start on a group
    // boundary and are flushed from the caller's buffer.  One launch per
    // tensor over all layers for each part.
    uint16_t* kcm = const_cast<uint16_t*>(k);
    uint16_t* vcm = const_cast<uint16_t*>(v);
    const int64_t rs = cache->ring * kD;               // ring / staging slab stride
    int rc = KIVI_OK;
    if (Q1 > Q0) {
        const int64_t a_end = std::min(Q1, (L0 + G - 1) / G * G);
        const int64_t A = a_end - Q0;                  // <= ring: R0 < ring, rounded up to G
        if (A > 0) {
            const int64_t from_ring = std::min(A, R0);
            const kivi::RowGather gk = {{cache->k_stage, rs, 0, 0}, {cache->k_ring, rs, cache->head, cache->ring},
                                        {kcm, x_bh_stride, 0, 0}, from_ring};
            const kivi::RowGather gv = {{cache->v_stage, rs, 0, 0}, {cache->v_ring, rs, cache->head, cache->ring},
                                        {vcm, x_bh_stride, 0, 0}, from_ring};
            rc = finish(kivi::launch_gather_rows(gk, gv, slabs, A, static_cast<int>(kD), stream));
            if (rc == KIVI_OK) rc = flush_keys(cache, cache->k_stage, slabs, A, rs, Q0, stream);
            if (rc == KIVI_OK) rc = flush_values(cache, cache->v_stage, slabs, A, rs, Q0, stream);
            if (rc != KIVI_OK) return rc;
        }
        const int64_t B = Q1 - a_end;
        if (B > 0) {
            const int64_t c0 = a_end - L0;             // chunk row of token a_end
            rc = flush_keys(cache, k + c0 * kD, slabs, B, x_bh_stride, a_end, stream);
            if (rc == KIVI_OK) rc = flush_values(cache, v + c0 * kD, slabs, B, x_bh_stride, a_end, stream);
            if (rc != KIVI_OK) return rc;
        }
    }
    // The fp16 tokens are now [Q1, L1).  Those older than the chunk stay in
    // their ring rows; the ring's head moves past the flushed ones (a
    // multiple of the flush unit, like the ring, so a later flush never
    // wraps), and the chunk's fp16 tokens are written after them.
    const int64_t head1 = (cache->head + (Q1 - Q0)) % cache->ring;
    const int64_t t0 = std::max(L0, Q1);               // first fp16 token that comes from the chunk
    const int64_t n_copy = L1 - t0;
    if (n_copy > 0) {
        const int64_t dst0 = (head1 + (t0 - Q1)) % cache->ring;
        const kivi::RowGather gk = {{cache->k_ring, rs, dst0, cache->ring}, {kcm, x_bh_stride, t0 - L0, 0},
                                    {kcm, x_bh_stride, t0 - L0, 0}, n_copy};
        const kivi::RowGather gv = {{cache->v_ring, rs, dst0, cache->ring}, {vcm, x_bh_stride, t0 - L0, 0},
                                    {vcm, x_bh_stride, t0 - L0, 0}, n_copy};
        rc = finish(kivi::launch_gather_rows(gk, gv, slabs, n_copy, static_cast<int>(kD), stream));
        if (rc != KIVI_OK) return rc;
    }
    cache->length = L1;
    cache->n_quant = Q1;
    cache->n_res = L1 - Q1;
    cache->head = head1;
    return KIVI_OK;
}

int kivi_cache_append(kivi_cache* cache, int32_t layer, const uint16_t* k_new,
                      const uint16_t* v_new, hipStream_t stream) {
    if (!cache) return KIVI_ERR_NULL;
    if (!valid(&cache->cfg)) return KIVI_ERR_UNSUPPORTED;
    const int64_t kD = cache->cfg.head_dim;
    if (layer < 0 || layer >= cache->cfg.layers || appended(cache, layer)) return KIVI_ERR_SHAPE;
    if (cache->n_res >= cache->ring) return KIVI_ERR_SHAPE;        // no free ring row
    if (!k_new || !v_new) return KIVI_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new)) return KIVI_ERR_ALIGN;
    const int64_t slab0 = layer * seq_slabs(cache);
    const int64_t row = (cache->head + cache->n_res) % cache->ring;
    const int64_t rs = cache->ring * kD;
    uint16_t* kn = const_cast<uint16_t*>(k_new);
    uint16_t* vn = const_cast<uint16_t*>(v_new);
    const kivi::RowGather gk = {{cache->k_ring + slab0 * rs, rs, row, 0}, {kn, kD, 0, 0}, {kn, kD, 0, 0}, 1};
    const kivi::RowGather gv = {{cache->v_ring + slab0 * rs, rs, row, 0}, {vn, kD, 0, 0}, {vn, kD, 0, 0}, 1};
    const int rc = finish(kivi::launch_gather_rows(gk, gv, seq_slabs(cache), 1, static_cast<int>(kD), stream));
    if (rc != KIVI_OK) return rc;
    cache->appended[layer >> 6] |= uint64_t{1} << (layer & 63);
    return KIVI_OK;
}

int kivi_cache_attend(const kivi_cache* cache, int32_t layer, const uint16_t* q, int32_t Hq,
                      float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
    if (!cache) return KIVI_ERR_NULL;
    if (!valid(&cache->cfg)) return KIVI_ERR_UNSUPPORTED;
    const int64_t kD = cache->cfg.head_dim;
    if (layer < 0 || layer >= cache->cfg.layers || !appended(cache, layer)) return KIVI_ERR_SHAPE;
    const int64_t slab0 = layer * seq_slabs(cache);
    const kivi_store ks = layer_store(cache->k_store, slab0);
    const kivi_store vs = layer_store(cache->v_store, slab0);
    const int64_t rs = cache->ring * kD;
    return kivi::decode_attend_entry(q, cache->cfg.batch, Hq, cache->cfg.kv_heads, &ks, &vs,
                                     cache->n_quant, cache->k_ring + slab0 * rs,
                                     cache->v_ring + slab0 * rs, rs, cache->n_res + 1, cache->head,
                                     cache->ring, nullptr, nullptr, softmax_scale, out, workspace,
                                     workspace_bytes, stream, cache->cfg.bf16 != 0);
}

int kivi_cache_append_attend(kivi_cache* cache, int32_t layer, const uint16_t* k_new,
                             const uint16_t* v_new, const uint16_t* q, int32_t Hq,
                             float softmax_scale, float* out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    if (!cache) return KIVI_ERR_NULL;
    if (!valid(&cache->cfg)) return KIVI_ERR_UNSUPPORTED;
    const int64_t kD = cache->cfg.head_dim;
    if (layer < 0 || layer >= cache->cfg.layers || appended(cache, layer)) return KIVI_ERR_SHAPE;
    if (cache->n_res >= cache->ring) return KIVI_ERR_SHAPE;        // no free ring row
    if (!k_new || !v_new) return KIVI_ERR_NULL;
    const int64_t slab0 = layer * seq_slabs(cache);
    const kivi_store ks = layer_store(cache->k_store, slab0);
    const kivi_store vs = layer_store(cache->v_store, slab0);
    const int64_t rs = cache->ring * kD;
    const int64_t row = (cache->head + cache->n_res) % cache->ring;
    const int rc = kivi::decode_attend_entry(q, cache->cfg.batch, Hq, cache->cfg.kv_heads, &ks, &vs,
                                             cache->n_quant, cache->k_ring + slab0 * rs,
                                             cache->v_ring + slab0 * rs, rs, cache->n_res + 1, cache->head,
                                             cache->ring, nullptr, nullptr, softmax_scale, out, workspace,
                                             workspace_bytes, stream, cache->cfg.bf16 != 0, false,
                                             k_new, v_new, row);
    if (rc != KIVI_OK) return rc;
    cache->appended[layer >> 6] |= uint64_t{1} << (layer & 63);
    return KIVI_OK;
}

size_t kivi_cache_attend_workspace_bytes(const kivi_cache* cache, int32_t Hq) {
    if (!cache || !valid(&cache->cfg) || Hq <= 0) return 0;
    // An attend plan depends on the token counts only through the number of
    // 32-token steps, ceil(n_quant / 32) + ceil(n_res / 32).  A cache's
    // attends have n_quant <= store_capacity and 1 <= n_res <= ring, so the
    // largest plan over step counts 1 .. steps(capacity) + steps(ring) covers
    // every call the cache can make: at most 2^19 + 2^19 cheap plans.
    const int32_t flags = cache->cfg.bf16 ? KIVI_ATTEND_BF16 : 0;
    const int64_t steps_store = (cache->cfg.store_capacity + 31) / 32;
    const int64_t max_steps = steps_store + (cache->ring + 31) / 32;
    size_t need = 0;
    for (int64_t steps = 1; steps <= max_steps; ++steps) {
        // the same step count as a call with this many store and residual
        // steps, each count within what a call of this cache can pass
        const int64_t sq = std::min(steps, steps_store);
        const size_t b = kivi_decode_attend_workspace_bytes(cache->cfg.batch, Hq, cache->cfg.kv_heads,
                                                            32 * sq, 32 * (steps - sq), cache->cfg.head_dim,
                                                            flags);
        if (b == 0) return 0;
        need = b > need ? b : need;
    }
    return need;
}

int kivi_cache_end_step(kivi_cache* cache, hipStream_t stream) {
    if (!cache) return KIVI_ERR_NULL;
    if (!valid(&cache->cfg)) return KIVI_ERR_UNSUPPORTED;
    const int64_t kD = cache->cfg.head_dim;
    for (int l = 0; l < cache->cfg.layers; ++l)
        if (!appended(cache, l)) return KIVI_ERR_SHAPE;
    const int64_t F = cache->cfg.flush_tokens;
    const int64_t n_res = cache->n_res + 1;
    const bool flush = n_res == cache->ring;
    if (flush && cache->n_quant + F > cache->cfg.store_capacity) return KIVI_ERR_SHAPE;
    int launches = 0;
    if (flush) {
        // the oldest F fp16 tokens of every slab of every layer: ring rows
        // head .. head + F - 1 (head and the ring length are multiples of F)
        const int64_t slabs = layout(cache->cfg).slabs;
        const int64_t rs = cache->ring * kD;
        int rc = flush_keys(cache, cache->k_ring + cache->head * kD, slabs, F, rs, cache->n_quant, stream);
        if (rc == KIVI_OK)
            rc = flush_values(cache, cache->v_ring + cache->head * kD, slabs, F, rs, cache->n_quant, stream);
        if (rc != KIVI_OK) return rc;
        launches = 2;
    }
    cache->length += 1;
    cache->n_res = n_res;
    if (flush) {
        cache->n_quant += F;
        cache->n_res -= F;
        cache->head += F;
        if (cache->head == cache->ring) cache->head = 0;
    }
    for (uint64_t& w : cache->appended) w = 0;
    return launches;
}

}  // extern "C"
