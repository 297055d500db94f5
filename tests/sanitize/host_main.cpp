// host_main.cpp -- drives the C ABI's host code (abi.cpp, cache.cpp,
// plan.cpp) against the launch stand-ins of launch_stubs.cpp, built with
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every "device" buffer is
// a host allocation of exactly the documented size, so a launch whose
// arguments reach outside it is reported.  Three parts:
//   1. valid calls of every entry point at several store geometries: status
//      OK and the expected number of launches;
//   2. invalid and extreme arguments (null, misaligned, negative, 2^62,
//      INT64_MAX sizes and strides): a negative status, nothing launched, and
//      no undefined behaviour in the size arithmetic;
//   3. the decode-loop cache driven through prompt chunks of ragged lengths
//      and decode steps, with every token row carrying its own (slab, token)
//      label: each flush must read exactly tokens [dst_token, dst_token + S)
//      of every slab, each attend must see the newest fp16 tokens in ring
//      order, and the rings must end holding the model's fp16 tail.
// Prints "host checks passed" and exits 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "kivi.h"
#include "kivi_cache.h"
#include "kivi_calib.h"
#include "kivi_launch.h"

namespace kivi {
extern long g_launches;
extern void (*g_on_flush)(bool keys, const FlushArgs& a);
extern void (*g_on_attend)(const AttendArgs& a);
}  // namespace kivi

namespace {

int g_failures = 0;

#define CHECK(cond)                                                                    \
    do {                                                                               \
        if (!(cond)) {                                                                 \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++g_failures;                                                              \
        }                                                                              \
    } while (0)

constexpr int64_t kBig = int64_t{1} << 62;
constexpr int64_t kMax = std::numeric_limits<int64_t>::max();
constexpr int64_t kMin = std::numeric_limits<int64_t>::min();

// Host allocations of exactly n bytes (256-byte aligned, as device memory is).
struct Pool {
    std::vector<void*> blocks;
    void* get(size_t n) {
        void* p = nullptr;
        if (posix_memalign(&p, 256, n ? n : 1) != 0) std::abort();
        std::memset(p, 0, n ? n : 1);
        blocks.push_back(p);
        return p;
    }
    ~Pool() {
        for (void* p : blocks) std::free(p);
    }
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

kivi_store make_store(Pool& pool, int kind, int64_t BH, int64_t cap, int bits, int G, int D, int meta) {
    kivi_store s{};
    const int64_t words = int64_t{D} * bits / 32;
    const int64_t es = meta == KIVI_META_F16 ? 2 : 4;
    const int64_t meta_rows = kind == KIVI_KEYS ? cdiv(cap, G) * D : cap * cdiv(D, G);
    // slab strides in whole 16-byte units, as the ABI requires
    s.codes_bh_stride = cdiv(cap * words, 4) * 4;
    s.meta_bh_stride = cdiv(meta_rows, 16 / es) * (16 / es);
    s.codes = static_cast<uint32_t*>(pool.get(static_cast<size_t>(BH * s.codes_bh_stride * 4)));
    s.scale = pool.get(static_cast<size_t>(BH * s.meta_bh_stride * es));
    s.zero = pool.get(static_cast<size_t>(BH * s.meta_bh_stride * es));
    s.cap = cap;
    s.bits = bits;
    s.group_size = G;
    s.head_dim = D;
    s.kind = kind;
    s.meta_format = meta;
    return s;
}

uint16_t* f16(Pool& pool, int64_t elems) { return static_cast<uint16_t*>(pool.get(static_cast<size_t>(elems * 2))); }

// ---------------------------------------------------------------- part 1
void valid_calls() {
    struct Geo { int D, G, meta, bits; };
    const Geo geos[] = {{128, 32, KIVI_META_F32, 4}, {128, 64, KIVI_META_F32, 2}, {128, 128, KIVI_META_F16, 4},
                        {128, 32, KIVI_META_F16, 2}, {64, 32, KIVI_META_F32, 4}, {96, 32, KIVI_META_F32, 2},
                        {256, 32, KIVI_META_F32, 4}, {16, 32, KIVI_META_F32, 4}};
    for (const Geo& g : geos) {
        Pool pool;
        const int64_t BH = 3, cap = 4 * g.G + 2 * g.G;           // room for a second flush at a group offset
        kivi_store ks = make_store(pool, KIVI_KEYS, BH, cap, g.bits, g.G, g.D, g.meta);
        kivi_store vs = make_store(pool, KIVI_VALUES, BH, cap, g.bits, g.G, g.D, g.meta);
        for (int64_t S : {int64_t{1}, int64_t{g.G} - 1, int64_t{g.G}, int64_t{3 * g.G + 5}}) {
            uint16_t* x = f16(pool, BH * S * g.D);
            uint16_t* rec = f16(pool, BH * S * g.D);
            const long before = kivi::g_launches;
            CHECK(kivi_quantize_keys(x, BH, S, S * g.D, &ks, 0, rec, S * g.D, nullptr) == KIVI_OK);
            CHECK(kivi_quantize_values(x, BH, S, S * g.D, &vs, cap - S, nullptr, 0, nullptr) == KIVI_OK);
            CHECK(kivi_quantize_keys(x, BH, S, S * g.D, &ks, cap - cdiv(S, g.G) * g.G, nullptr, 0, nullptr) == KIVI_OK);
            if (g.meta == KIVI_META_F32) {
                CHECK(kivi_quantize_keys_bf16(x, BH, S, S * g.D, &ks, g.G, rec, S * g.D, nullptr) == KIVI_OK);
                CHECK(kivi_quantize_values_bf16(x, BH, S, S * g.D, &vs, 1, rec, S * g.D, nullptr) == KIVI_OK);
                CHECK(kivi_dequantize_bf16(&ks, BH, cap - S, S, rec, S * g.D, nullptr) == KIVI_OK);
            }
            CHECK(kivi_dequantize(&ks, BH, 0, S, rec, S * g.D, nullptr) == KIVI_OK);
            CHECK(kivi_dequantize(&vs, BH, cap - S, S, rec, S * g.D, nullptr) == KIVI_OK);
            CHECK(kivi::g_launches - before == (g.meta == KIVI_META_F32 ? 8 : 5));
        }
        // attend: B=3 sequences x 1 kv head at every head ratio the ABI takes,
        // store prefix and residual windows of several lengths
        const int64_t B = 3;
        for (int Hq : {1, 2, 4, 8}) {
            for (int64_t nq : {int64_t{0}, int64_t{1}, cap / 2 + 3, cap}) {
                for (int64_t nr : {int64_t{0}, int64_t{1}, int64_t{37}}) {
                    if (nq + nr == 0) continue;
                    const int64_t R = nr > 0 ? nr : 1;
                    uint16_t* q = f16(pool, B * Hq * g.D);
                    uint16_t* kr = f16(pool, B * R * g.D);
                    uint16_t* vr = f16(pool, B * R * g.D);
                    float* out = static_cast<float*>(pool.get(static_cast<size_t>(B * Hq * g.D * 4)));
                    for (int bf = 0; bf < 2; ++bf) {
                        if (bf && g.meta == KIVI_META_F16) continue;
                        const size_t n = kivi_decode_attend_workspace_bytes(B, Hq, 1, nq, nr, g.D,
                                                                            bf ? KIVI_ATTEND_BF16 : 0);
                        CHECK(n > 0);
                        void* ws = pool.get(n);
                        const long before = kivi::g_launches;
                        auto fn = bf ? kivi_decode_attend_bf16 : kivi_decode_attend;
                        CHECK(fn(q, B, Hq, 1, &ks, &vs, nq, kr, vr, R * g.D, nr, 0.125f, out, ws, n, nullptr) == KIVI_OK);
                        CHECK(fn(q, B, Hq, 1, &ks, &vs, nq, kr, vr, R * g.D, nr, 0.125f, out, ws, n - 1, nullptr) ==
                              KIVI_ERR_WORKSPACE);
                        CHECK(kivi::g_launches - before == 1);
                    }
                    // variable lengths: per-sequence counts up to the bounds
                    int32_t* snq = static_cast<int32_t*>(pool.get(B * 4));
                    int32_t* snr = static_cast<int32_t*>(pool.get(B * 4));
                    for (int b = 0; b < B; ++b) {
                        snq[b] = static_cast<int32_t>(nq * b / 2 > nq ? nq : nq * b / 2);
                        snr[b] = static_cast<int32_t>(nr - b > 0 ? nr - b : 0);
                    }
                    const size_t nv = kivi_decode_attend_workspace_bytes(B, Hq, 1, nq, nr, g.D, KIVI_ATTEND_VARLEN);
                    void* wv = pool.get(nv);
                    CHECK(kivi_decode_attend_varlen(q, B, Hq, 1, &ks, &vs, snq, nq, kr, vr, R * g.D, snr, nr, 0.5f,
                                                    out, wv, nv, nullptr) == KIVI_OK);
                    if (g.D == 128 && g.meta == KIVI_META_F32)
                        CHECK(kivi_decode_attend_noalloc(q, B, Hq, 1, &ks, &vs, nq, kr, vr, R * g.D, nr, 0.5f, out,
                                                         nullptr) == KIVI_OK);
                }
            }
        }
    }
    // calibration kernels
    Pool pool;
    void* a = pool.get(1 << 16);
    void* b = pool.get(1 << 16);
    void* sink = pool.get(16);
    CHECK(kivi_calib_copy(a, b, 1 << 16, nullptr) == KIVI_OK);
    CHECK(kivi_calib_read(a, 1 << 16, sink, nullptr) == KIVI_OK);
    CHECK(kivi_calib_write(b, 1 << 16, nullptr) == KIVI_OK);
    CHECK(kivi_calib_mix(a, 1 << 16, b, nullptr) == KIVI_OK);
    CHECK(kivi_calib_mix(a, 48, b, nullptr) == KIVI_OK);
}

// ---------------------------------------------------------------- part 2
void invalid_calls() {
    Pool pool;
    const int64_t BH = 2, cap = 256, D = 128;
    kivi_store ks = make_store(pool, KIVI_KEYS, BH, cap, 4, 32, D, KIVI_META_F32);
    kivi_store vs = make_store(pool, KIVI_VALUES, BH, cap, 4, 32, D, KIVI_META_F32);
    uint16_t* x = f16(pool, BH * cap * D);
    uint16_t* mis = x + 1;                                    // 2-byte aligned only
    const long before = kivi::g_launches;
    // sizes no caller buffer can have: every call below must refuse them
    const int64_t sizes[] = {-1, kMin, kBig, kMax, kMax - 1, kBig + 1, int64_t{1} << 47};
    for (int64_t v : sizes) {
        CHECK(kivi_quantize_keys(x, v, 32, 32 * D, &ks, 0, nullptr, 0, nullptr) < 0);
        CHECK(kivi_quantize_keys(x, BH, v, cap * D, &ks, 0, nullptr, 0, nullptr) < 0);
        CHECK(kivi_quantize_values(x, BH, 32, cap * D, &vs, v, nullptr, 0, nullptr) < 0);
        CHECK(kivi_quantize_values(x, BH, 32, v, &vs, 0, nullptr, 0, nullptr) < 0);
        CHECK(kivi_dequantize(&ks, BH, v, 32, x, 32 * D, nullptr) < 0);
        CHECK(kivi_dequantize(&ks, BH, 0, v, x, cap * D, nullptr) < 0);
        CHECK(kivi_dequantize(&ks, v, 0, 32, x, 32 * D, nullptr) < 0);
        kivi_store bad = ks;
        bad.cap = v;
        CHECK(kivi_quantize_keys(x, BH, 32, 32 * D, &bad, 0, nullptr, 0, nullptr) < 0);
        bad = ks;
        bad.codes_bh_stride = v;
        CHECK(kivi_quantize_keys(x, BH, 32, 32 * D, &bad, 0, nullptr, 0, nullptr) < 0);
        bad = vs;
        bad.meta_bh_stride = v;
        CHECK(kivi_quantize_values(x, BH, 32, 32 * D, &bad, 0, nullptr, 0, nullptr) < 0);
        // attend sizes
        CHECK(kivi_decode_attend_workspace_bytes(v, 32, 8, 1024, 16, 128, 0) == 0 || v > 0);
        CHECK(kivi_decode_attend_workspace_bytes(1, 32, 8, v, 16, 128, 0) == 0 || v > 0);
        float* out = static_cast<float*>(pool.get(64 * D * 4));
        void* ws = pool.get(1 << 20);
        CHECK(kivi_decode_attend(x, v, 4, 1, &ks, &vs, 64, x, x, 64 * D, 16, 0.1f, out, ws, 1 << 20, nullptr) < 0);
        CHECK(kivi_decode_attend(x, 1, 4, 1, &ks, &vs, v, x, x, 64 * D, 16, 0.1f, out, ws, 1 << 20, nullptr) < 0);
        CHECK(kivi_decode_attend(x, 1, 4, 1, &ks, &vs, 64, x, x, 64 * D, v, 0.1f, out, ws, 1 << 20, nullptr) < 0);
        CHECK(kivi_decode_attend(x, 2, 4, 1, &ks, &vs, 64, x, x, v, 16, 0.1f, out, ws, 1 << 20, nullptr) < 0);
        CHECK(kivi_calib_copy(x, x, static_cast<size_t>(v), nullptr) < 0);
        CHECK(kivi_calib_read(x, static_cast<size_t>(v), x, nullptr) < 0);
    }
    // the workspace query at huge sizes is either 0 or a size without wrap-around
    for (int64_t B : {int64_t{1}, int64_t{65535}, kBig, kMax}) {
        for (int64_t nq : {int64_t{1}, int64_t{1} << 24, kBig, kMax}) {
            const size_t n = kivi_decode_attend_workspace_bytes(B, 64, 8, nq, 1, 256, KIVI_ATTEND_VARLEN);
            (void)n;
        }
    }
    // pointers and enums
    CHECK(kivi_quantize_keys(nullptr, BH, 32, 32 * D, &ks, 0, nullptr, 0, nullptr) == KIVI_ERR_NULL);
    CHECK(kivi_quantize_keys(mis, BH, 32, 32 * D, &ks, 0, nullptr, 0, nullptr) == KIVI_ERR_ALIGN);
    CHECK(kivi_quantize_keys(x, BH, 32, 32 * D + 1, &ks, 0, nullptr, 0, nullptr) == KIVI_ERR_ALIGN);
    CHECK(kivi_quantize_keys(x, BH, 32, 32 * D, &ks, 16, nullptr, 0, nullptr) == KIVI_ERR_SHAPE);
    CHECK(kivi_quantize_keys(x, BH, 32, 32 * D, &vs, 0, nullptr, 0, nullptr) == KIVI_ERR_SHAPE);
    CHECK(kivi_quantize_keys(x, BH, 32, 32 * D, nullptr, 0, nullptr, 0, nullptr) == KIVI_ERR_NULL);
    for (int bits : {0, 1, 3, 8, -4}) {
        kivi_store bad = ks;
        bad.bits = bits;
        CHECK(kivi_quantize_keys(x, BH, 32, 32 * D, &bad, 0, nullptr, 0, nullptr) == KIVI_ERR_UNSUPPORTED);
    }
    for (int G : {0, 16, 48, 256, -32}) {
        kivi_store bad = ks;
        bad.group_size = G;
        CHECK(kivi_quantize_keys(x, BH, 32, 32 * D, &bad, 0, nullptr, 0, nullptr) == KIVI_ERR_UNSUPPORTED);
    }
    for (int hd : {0, 8, 100, 272, 512, -128}) {
        kivi_store bad = ks;
        bad.head_dim = hd;
        CHECK(kivi_quantize_keys(x, BH, 32, 32 * D, &bad, 0, nullptr, 0, nullptr) == KIVI_ERR_UNSUPPORTED);
    }
    float* out = static_cast<float*>(pool.get(BH * 8 * D * 4));
    const size_t n = kivi_decode_attend_workspace_bytes(2, 8, 1, 64, 16, 128, 0);
    void* ws = pool.get(n);
    CHECK(kivi_decode_attend(x, 2, 8, 3, &ks, &vs, 64, x, x, 64 * D, 16, 0.1f, out, ws, n, nullptr) == KIVI_ERR_SHAPE);
    CHECK(kivi_decode_attend(x, 2, 16, 1, &ks, &vs, 64, x, x, 64 * D, 16, 0.1f, out, ws, n, nullptr) ==
          KIVI_ERR_UNSUPPORTED);
    CHECK(kivi_decode_attend(x, 2, 8, 1, &ks, &vs, 0, x, x, 64 * D, 0, 0.1f, out, ws, n, nullptr) == KIVI_ERR_SHAPE);
    CHECK(kivi_decode_attend(x, 2, 8, 1, &ks, &vs, 64, x, x, 64 * D, 16, -1.0f, out, ws, n, nullptr) == KIVI_ERR_SHAPE);
    CHECK(kivi_decode_attend(x, 2, 8, 1, &ks, &vs, 64, x, x, 64 * D, 16, 0.0f / 0.0f, out, ws, n, nullptr) ==
          KIVI_ERR_SHAPE);
    CHECK(kivi_decode_attend(x, 2, 8, 1, &ks, &vs, cap + 1, x, x, 64 * D, 16, 0.1f, out, ws, n, nullptr) ==
          KIVI_ERR_SHAPE);
    CHECK(kivi_decode_attend(x, 2, 8, 1, &ks, &vs, 64, x, x, 64 * D, 16, 0.1f, out, nullptr, n, nullptr) ==
          KIVI_ERR_WORKSPACE);
    CHECK(kivi_decode_attend(x, 2, 8, 1, &ks, &vs, 64, x, x, 64 * D, 16, 0.1f, out,
                             static_cast<char*>(ws) + 16, n - 16, nullptr) < 0);
    CHECK(kivi_decode_attend(x, 2, 8, 1, &ks, &vs, 64, x, x, 8 * D, 16, 0.1f, out, ws, n, nullptr) == KIVI_ERR_SHAPE);
    CHECK(kivi_decode_attend_varlen(x, 2, 8, 1, &ks, &vs, nullptr, 64, x, x, 64 * D, nullptr, 16, 0.1f, out, ws, n,
                                    nullptr) == KIVI_ERR_NULL);
    CHECK(kivi_decode_attend_workspace_bytes(2, 8, 1, 64, 16, 100, 0) == 0);
    CHECK(kivi_decode_attend_workspace_bytes(2, 8, 1, 64, 16, 128, 4) == 0);
    CHECK(kivi_calib_copy(x, mis, 64, nullptr) == KIVI_ERR_ALIGN);
    CHECK(kivi_calib_mix(x, 17, x, nullptr) == KIVI_ERR_ALIGN);
    CHECK(kivi_calib_read(nullptr, 64, x, nullptr) == KIVI_ERR_NULL);
    CHECK(kivi::g_launches == before);
    for (int s = -7; s <= 1; ++s) CHECK(kivi_status_string(s) != nullptr);

    // cache configurations at and past every limit
    kivi_cache_config c{};
    c.layers = 2; c.batch = 2; c.kv_heads = 2; c.bits = 4; c.head_dim = 128; c.group_size = 32;
    c.residual_length = 64; c.flush_tokens = 32; c.store_capacity = 1024; c.meta_format = 0; c.bf16 = 0;
    CHECK(kivi_cache_device_bytes(&c) > 0);
    const int32_t i32s[] = {0, -1, std::numeric_limits<int32_t>::max(), std::numeric_limits<int32_t>::min(), 257, 1 << 30};
    for (int32_t v : i32s) {
        for (int field = 0; field < 8; ++field) {
            kivi_cache_config b = c;
            int32_t* f[] = {&b.layers, &b.batch, &b.kv_heads, &b.bits, &b.head_dim, &b.group_size,
                            &b.residual_length, &b.flush_tokens};
            *f[field] = v;
            const size_t bytes = kivi_cache_device_bytes(&b);
            kivi_cache cache;
            if (bytes == 0) {
                CHECK(kivi_cache_init(&cache, &b, x, size_t{1} << 40) < 0);
            }
        }
    }
    for (int64_t v : sizes) {
        kivi_cache_config b = c;
        b.store_capacity = v;
        CHECK(kivi_cache_device_bytes(&b) == 0 || (v > 0 && v < (int64_t{1} << 40)));
    }
    CHECK(kivi_cache_device_bytes(nullptr) == 0);
    CHECK(kivi::g_launches == before);
}

// ---------------------------------------------------------------- part 3
// Token rows carry their identity: element 0 = token index (low 16 bits),
// element 1 = its high bits, element 2 = slab, element 3 = 0 for keys / 1 for
// values, the rest a mix of the three.
void label(uint16_t* row, int64_t slab, int64_t t, int kv, int D) {
    row[0] = static_cast<uint16_t>(t & 0xFFFF);
    row[1] = static_cast<uint16_t>(t >> 16);
    row[2] = static_cast<uint16_t>(slab);
    row[3] = static_cast<uint16_t>(kv);
    for (int d = 4; d < D; ++d) row[d] = static_cast<uint16_t>((t * 31 + slab * 7 + d + kv * 5) & 0xFFFF);
}

bool is_label(const uint16_t* row, int64_t slab, int64_t t, int kv, int D) {
    std::vector<uint16_t> want(static_cast<size_t>(D));
    label(want.data(), slab, t, kv, D);
    return std::memcmp(row, want.data(), static_cast<size_t>(D) * 2) == 0;
}

struct LoopState {
    kivi_cache* cache = nullptr;
    int64_t flushed_keys = 0, flushed_values = 0;   // tokens x slabs seen by flush launches
    int64_t attends = 0;
    int64_t layer = 0;                              // layer of the attend being checked
};
LoopState g_loop;

void on_flush(bool keys, const kivi::FlushArgs& a) {
    const kivi_cache* c = g_loop.cache;
    const int D = c->cfg.head_dim;
    // the flush reads tokens [dst_token, dst_token + S) of every slab, in order
    for (int64_t s = 0; s < a.BH; ++s)
        for (int64_t r = 0; r < a.S; ++r)
            CHECK(is_label(a.x + s * a.x_bh_stride + r * D, s, a.dst_token + r, keys ? 0 : 1, D));
    CHECK(a.dst_token + a.S <= c->cfg.store_capacity);
    (keys ? g_loop.flushed_keys : g_loop.flushed_values) += a.S * a.BH;
}

void on_attend(const kivi::AttendArgs& a) {
    const kivi_cache* c = g_loop.cache;
    const int D = c->cfg.head_dim;
    const int64_t per = int64_t{c->cfg.batch} * c->cfg.kv_heads;
    CHECK(a.n_quant == c->n_quant);
    CHECK(a.n_res == c->n_res + 1);                 // the step's own token included
    for (int64_t s = 0; s < per; ++s) {
        const int64_t slab = g_loop.layer * per + s;
        for (int64_t i = 0; i < a.n_res; ++i) {
            const int64_t row = (a.res_head + i) % a.res_ring;
            // a fused append's token is read from the new rows, not yet the ring
            const bool fresh = a.k_new && i == a.n_res - 1;
            CHECK(is_label(fresh ? a.k_new + s * D : a.k_res + s * a.res_bh_stride + row * D, slab,
                           c->n_quant + i, 0, D));
            CHECK(is_label(fresh ? a.v_new + s * D : a.v_res + s * a.res_bh_stride + row * D, slab,
                           c->n_quant + i, 1, D));
            if (fresh) CHECK(row == a.new_row);
        }
    }
    ++g_loop.attends;
}

int64_t quantized(const kivi_cache_config& c, int64_t L) {
    if (L < c.residual_length) return 0;
    return (L - c.residual_length) / c.flush_tokens * c.flush_tokens;
}

void check_rings(const kivi_cache& c) {
    const int D = c.cfg.head_dim;
    const int64_t slabs = int64_t{c.cfg.layers} * c.cfg.batch * c.cfg.kv_heads;
    CHECK(c.n_quant == quantized(c.cfg, c.length));
    CHECK(c.n_res == c.length - c.n_quant);
    for (int64_t s = 0; s < slabs; ++s)
        for (int64_t i = 0; i < c.n_res; ++i) {
            const int64_t row = (c.head + i) % c.ring;
            CHECK(is_label(c.k_ring + (s * c.ring + row) * D, s, c.n_quant + i, 0, D));
            CHECK(is_label(c.v_ring + (s * c.ring + row) * D, s, c.n_quant + i, 1, D));
        }
}

// schedule: positive = a prompt chunk of that many tokens, negative = that
// many decode steps
void run_cache(const kivi_cache_config& cfg, const std::vector<int64_t>& schedule, int Hq) {
    Pool pool;
    const size_t bytes = kivi_cache_device_bytes(&cfg);
    CHECK(bytes > 0);
    if (bytes == 0) return;
    void* dev = pool.get(bytes);
    kivi_cache c;
    CHECK(kivi_cache_init(&c, &cfg, dev, bytes) == KIVI_OK);
    CHECK(kivi_cache_init(&c, &cfg, dev, bytes - 1) < 0);
    CHECK(kivi_cache_init(&c, &cfg, static_cast<char*>(dev) + 16, bytes) < 0);
    CHECK(kivi_cache_init(&c, &cfg, dev, bytes) == KIVI_OK);
    g_loop = LoopState{};
    g_loop.cache = &c;
    kivi::g_on_flush = on_flush;
    kivi::g_on_attend = on_attend;
    const int D = cfg.head_dim;
    const int64_t per = int64_t{cfg.batch} * cfg.kv_heads;
    const int64_t slabs = cfg.layers * per;
    const size_t wsb = kivi_cache_attend_workspace_bytes(&c, Hq);
    CHECK(wsb > 0);
    void* ws = pool.get(wsb);
    uint16_t* q = f16(pool, cfg.batch * Hq * D);
    float* out = static_cast<float*>(pool.get(static_cast<size_t>(cfg.batch * Hq * D * 4)));
    int64_t expect_flushed = 0;
    for (int64_t ev : schedule) {
        if (ev > 0) {
            // a chunk with a slab stride one token longer than needed
            const int64_t S = ev, stride = (S + 1) * D;
            uint16_t* k = f16(pool, (slabs - 1) * stride + S * D);
            uint16_t* v = f16(pool, (slabs - 1) * stride + S * D);
            for (int64_t s = 0; s < slabs; ++s)
                for (int64_t r = 0; r < S; ++r) {
                    label(k + s * stride + r * D, s, c.length + r, 0, D);
                    label(v + s * stride + r * D, s, c.length + r, 1, D);
                }
            const int64_t q0 = c.n_quant;
            const int rc = kivi_cache_prefill(&c, k, v, stride, S, nullptr);
            CHECK(rc == KIVI_OK);
            if (rc == KIVI_OK) expect_flushed += (c.n_quant - q0) * slabs;
        } else {
            for (int64_t step = 0; step < -ev; ++step) {
                uint16_t* kn = f16(pool, per * D);
                uint16_t* vn = f16(pool, per * D);
                for (int32_t l = 0; l < cfg.layers; ++l) {
                    for (int64_t s = 0; s < per; ++s) {
                        label(kn + s * D, l * per + s, c.length, 0, D);
                        label(vn + s * D, l * per + s, c.length, 1, D);
                    }
                    CHECK(kivi_cache_attend(&c, l, q, Hq, 0.1f, out, ws, wsb, nullptr) == KIVI_ERR_SHAPE);
                    g_loop.layer = l;
                    if (l % 2 == 0) {
                        CHECK(kivi_cache_append(&c, l, kn, vn, nullptr) == KIVI_OK);
                        CHECK(kivi_cache_append(&c, l, kn, vn, nullptr) == KIVI_ERR_SHAPE);
                        CHECK(kivi_cache_append_attend(&c, l, kn, vn, q, Hq, 0.1f, out, ws, wsb, nullptr) ==
                              KIVI_ERR_SHAPE);
                        CHECK(kivi_cache_attend(&c, l, q, Hq, 0.1f, out, ws, wsb, nullptr) == KIVI_OK);
                    } else {
                        // the fused call: a too-small workspace leaves the layer un-appended
                        CHECK(kivi_cache_append_attend(&c, l, kn, vn, q, Hq, 0.1f, out, ws, 16, nullptr) ==
                              KIVI_ERR_WORKSPACE);
                        CHECK(kivi_cache_append_attend(&c, l, kn, vn, q, Hq, 0.1f, out, ws, wsb, nullptr) ==
                              KIVI_OK);
                        CHECK(kivi_cache_append(&c, l, kn, vn, nullptr) == KIVI_ERR_SHAPE);
                    }
                    if (l + 1 < cfg.layers) CHECK(kivi_cache_end_step(&c, nullptr) == KIVI_ERR_SHAPE);
                }
                const int64_t q0 = c.n_quant;
                const int launches = kivi_cache_end_step(&c, nullptr);
                CHECK(launches == (c.n_quant != q0 ? 2 : 0));
                expect_flushed += (c.n_quant - q0) * slabs;
            }
        }
        check_rings(c);
    }
    CHECK(g_loop.flushed_keys == expect_flushed);
    CHECK(g_loop.flushed_values == expect_flushed);
    // a chunk past the capacity is refused and leaves the cache unchanged
    const kivi_cache before = c;
    uint16_t* big = f16(pool, slabs * D);
    CHECK(kivi_cache_prefill(&c, big, big, D, cfg.store_capacity + cfg.residual_length + cfg.flush_tokens, nullptr) < 0);
    CHECK(kivi_cache_prefill(&c, big, big, D, kBig, nullptr) < 0);
    CHECK(kivi_cache_prefill(&c, big, big, D, -1, nullptr) < 0);
    CHECK(std::memcmp(&before, &c, sizeof c) == 0);
    kivi::g_on_flush = nullptr;
    kivi::g_on_attend = nullptr;
}

kivi_cache_config cfg_of(int layers, int batch, int kvh, int bits, int D, int G, int R, int F, int64_t cap, int meta,
                         int bf16) {
    kivi_cache_config c{};
    c.layers = layers; c.batch = batch; c.kv_heads = kvh; c.bits = bits; c.head_dim = D; c.group_size = G;
    c.residual_length = R; c.flush_tokens = F; c.store_capacity = cap; c.meta_format = meta; c.bf16 = bf16;
    return c;
}

void cache_loops() {
    run_cache(cfg_of(2, 2, 2, 4, 128, 32, 64, 32, 1024, 0, 0),
              {45, -3, 1, 100, -40, 77, 31, -2, 200, -5}, 8);
    run_cache(cfg_of(1, 2, 2, 4, 128, 32, 128, 128, 2048, 1, 0), {300, -20, 129, 500, -130}, 8);
    run_cache(cfg_of(2, 1, 2, 2, 128, 32, 0, 32, 512, 0, 1), {33, -1, 64, 95, -40, 7}, 4);
    run_cache(cfg_of(1, 2, 2, 4, 128, 64, 128, 64, 1024, 0, 0), {70, -30, 250, -3, 65}, 8);
    run_cache(cfg_of(1, 1, 2, 4, 96, 32, 64, 32, 512, 0, 0), {50, -20, 90, -5}, 8);
    run_cache(cfg_of(1, 1, 1, 4, 128, 32, 32, 32, 8192, 0, 0), {2048, 2048, 2048, 2048, 17, -2}, 2);
    run_cache(cfg_of(3, 1, 1, 4, 64, 32, 32, 32, 256, 0, 0), {-70, 5, -40}, 8);
}

}  // namespace

int main() {
    valid_calls();
    invalid_calls();
    cache_loops();
    if (g_failures) {
        std::fprintf(stderr, "%d host checks failed\n", g_failures);
        return 1;
    }
    std::printf("host checks passed (%ld launches)\n", kivi::g_launches);
    return 0;
}
