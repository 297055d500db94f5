// abi.cpp -- the C ABI of libkivi (declared in include/kivi.h and
// include/kivi_calib.h): argument validation on the host, then kernel launch
// on the caller's stream.  Validation never calls into HIP, so an error
// return means nothing was enqueued.
#include <cmath>

#include "kivi.h"
#include "kivi_calib.h"
#include "kivi_launch.h"

#include <limits>

namespace {
thread_local int g_last_hip_error = 0;
}  // namespace

namespace kivi {
int hip_status(hipError_t e) {
    if (e == hipSuccess) return KIVI_OK;
    g_last_hip_error = static_cast<int>(e);
    return KIVI_ERR_HIP;
}
}  // namespace kivi

namespace {

constexpr int64_t kD = 128;
constexpr int64_t kMaxBlocks = (int64_t{1} << 31) - 1;
constexpr int64_t kMaxAttendTokens = int64_t{1} << 24;   // attend offsets stay 32-bit
// No buffer reaches past the 47-bit virtual address space a process can map:
// a tensor or store whose extent would is refused before any product of its
// sizes is formed, so the size arithmetic below never overflows.
constexpr int64_t kMaxBytes = int64_t{1} << 47;
constexpr int64_t kMaxStoreTokens = int64_t{1} << 40;
constexpr int64_t kMaxAttendSlabs = 65535;               // B * Hkv: the partial kernel's grid y

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int finish(hipError_t e) { return kivi::hip_status(e); }

int64_t words_per_token(const kivi_store* st) { return int64_t{st->head_dim} * st->bits / 32; }

int64_t meta_rows(const kivi_store* st) {
    const int64_t G = st->group_size, D = st->head_dim;
    return st->kind == KIVI_KEYS ? (st->cap + G - 1) / G * D : st->cap * ((D + G - 1) / G);
}

// Stores take head_dim 128 with groups of 32, 64 or 128 tokens (keys) or
// channels (values), and any other multiple of 16 from 16 to 256 with groups
// of 32 (a token's last value group is ragged when 32 does not divide
// head_dim).  The attend and the decode-loop cache take every such store
// (binary16 scale/zero at head_dim 128 only, see check_store).
bool geometry_ok(int32_t D, int32_t G) {
    if (D == 128) return G == 32 || G == 64 || G == 128;
    return D >= 16 && D <= 256 && D % 16 == 0 && G == 32;
}

bool meta16(const kivi_store* st) { return st->meta_format == KIVI_META_F16; }

// Whether n_slabs slabs of slab_elems elements, stride_elems apart, fit in
// kMaxBytes (all arguments non-negative; no intermediate overflows).
bool extent_ok(int64_t n_slabs, int64_t stride_elems, int64_t slab_elems, int64_t elem_bytes) {
    const int64_t limit = kMaxBytes / elem_bytes;
    if (n_slabs < 0 || stride_elems < 0 || slab_elems < 0 || slab_elems > limit) return false;
    return n_slabs <= 1 || stride_elems <= (limit - slab_elems) / (n_slabs - 1);
}

// Checks a store and that tokens [t0, t0 + n) of slabs [0, BH) lie inside it.
// Binary16 scale/zero are supported at head_dim 128.
int check_store(const kivi_store* st, int kind, int64_t BH, int64_t t0, int64_t n) {
    if (!st) return KIVI_ERR_NULL;
    if (st->kind != KIVI_KEYS && st->kind != KIVI_VALUES) return KIVI_ERR_UNSUPPORTED;
    if (kind >= 0 && st->kind != kind) return KIVI_ERR_SHAPE;
    if (st->bits != 2 && st->bits != 4) return KIVI_ERR_UNSUPPORTED;
    if (!geometry_ok(st->head_dim, st->group_size)) return KIVI_ERR_UNSUPPORTED;
    if (st->meta_format != KIVI_META_F32 && st->meta_format != KIVI_META_F16) return KIVI_ERR_UNSUPPORTED;
    if (meta16(st) && st->head_dim != kD) return KIVI_ERR_UNSUPPORTED;
    if (!st->codes || !st->scale || !st->zero) return KIVI_ERR_NULL;
    if (!aligned16(st->codes) || !aligned16(st->scale) || !aligned16(st->zero)) return KIVI_ERR_ALIGN;
    // slab strides of whole 16-byte units
    if (st->codes_bh_stride % 4 != 0 || st->meta_bh_stride % (meta16(st) ? 8 : 4) != 0) return KIVI_ERR_ALIGN;
    if (st->cap < 0 || st->cap > kMaxStoreTokens || t0 < 0 || n < 0 || t0 > st->cap - n) return KIVI_ERR_SHAPE;
    if (BH < 0 || st->codes_bh_stride < 0 || st->meta_bh_stride < 0) return KIVI_ERR_SHAPE;
    if (BH > 1) {
        if (st->codes_bh_stride < st->cap * words_per_token(st)) return KIVI_ERR_SHAPE;
        if (st->meta_bh_stride < meta_rows(st)) return KIVI_ERR_SHAPE;
    }
    if (!extent_ok(BH, st->codes_bh_stride, st->cap * words_per_token(st), 4) ||
        !extent_ok(BH, st->meta_bh_stride, meta_rows(st), meta16(st) ? 2 : 4)) return KIVI_ERR_SHAPE;
    return KIVI_OK;
}

// 16-bit [BH][S][D] tensor with slab stride `stride` elements.
int check_f16_tensor(const void* p, int64_t BH, int64_t S, int64_t stride, int64_t D = kD) {
    if (!p) return KIVI_ERR_NULL;
    if (!aligned16(p) || stride % 8 != 0) return KIVI_ERR_ALIGN;
    if (BH < 0 || S < 0 || stride < 0 || S > kMaxBytes / 2 / D) return KIVI_ERR_SHAPE;
    if (BH > 1 && stride < S * D) return KIVI_ERR_SHAPE;
    if (!extent_ok(BH, stride, S * D, 2)) return KIVI_ERR_SHAPE;
    return KIVI_OK;
}

int flush(bool keys, bool bf16, const uint16_t* x, int64_t BH, int64_t S, int64_t x_bh_stride,
          const kivi_store* dst, int64_t dst_token, uint16_t* recon, int64_t recon_bh_stride,
          hipStream_t stream) {
    if (BH < 0 || S < 0) return KIVI_ERR_SHAPE;
    int rc = check_store(dst, keys ? KIVI_KEYS : KIVI_VALUES, BH, dst_token, S);
    if (rc != KIVI_OK) return rc;
    if (keys && dst_token % dst->group_size != 0) return KIVI_ERR_SHAPE;
    if (bf16 && meta16(dst)) return KIVI_ERR_UNSUPPORTED;     // binary16 metadata is for fp16 caches
    if (BH == 0 || S == 0) return KIVI_OK;
    if ((rc = check_f16_tensor(x, BH, S, x_bh_stride, dst->head_dim)) != KIVI_OK) return rc;
    if (recon && (rc = check_f16_tensor(recon, BH, S, recon_bh_stride, dst->head_dim)) != KIVI_OK) return rc;
    const int64_t tiles = BH * ((S + 31) / 32);
    if ((tiles + 3) / 4 > kMaxBlocks) return KIVI_ERR_SHAPE;

    kivi::FlushArgs a;
    a.x = x; a.BH = BH; a.S = S; a.x_bh_stride = x_bh_stride;
    a.codes = dst->codes; a.codes_bh_stride = dst->codes_bh_stride;
    a.scale = dst->scale; a.zero = dst->zero; a.meta_bh_stride = dst->meta_bh_stride;
    a.dst_token = dst_token; a.recon = recon; a.recon_bh_stride = recon_bh_stride;
    a.bits = dst->bits;
    a.group = dst->group_size;
    a.head_dim = dst->head_dim;
    a.bf16 = bf16;
    a.meta16 = meta16(dst);
    return finish(keys ? kivi::launch_key_flush(a, stream) : kivi::launch_value_flush(a, stream));
}

}  // namespace

extern "C" {

int kivi_quantize_keys(const uint16_t* x, int64_t BH, int64_t S, int64_t x_bh_stride,
                       const kivi_store* dst, int64_t dst_token,
                       uint16_t* recon, int64_t recon_bh_stride, hipStream_t stream) {
    return flush(true, false, x, BH, S, x_bh_stride, dst, dst_token, recon, recon_bh_stride, stream);
}

int kivi_quantize_keys_bf16(const uint16_t* x, int64_t BH, int64_t S, int64_t x_bh_stride,
                            const kivi_store* dst, int64_t dst_token,
                            uint16_t* recon, int64_t recon_bh_stride, hipStream_t stream) {
    return flush(true, true, x, BH, S, x_bh_stride, dst, dst_token, recon, recon_bh_stride, stream);
}

int kivi_quantize_values(const uint16_t* x, int64_t BH, int64_t S, int64_t x_bh_stride,
                         const kivi_store* dst, int64_t dst_token,
                         uint16_t* recon, int64_t recon_bh_stride, hipStream_t stream) {
    return flush(false, false, x, BH, S, x_bh_stride, dst, dst_token, recon, recon_bh_stride, stream);
}

int kivi_quantize_values_bf16(const uint16_t* x, int64_t BH, int64_t S, int64_t x_bh_stride,
                              const kivi_store* dst, int64_t dst_token,
                              uint16_t* recon, int64_t recon_bh_stride, hipStream_t stream) {
    return flush(false, true, x, BH, S, x_bh_stride, dst, dst_token, recon, recon_bh_stride, stream);
}

static int dequantize(bool bf16, const kivi_store* src, int64_t BH, int64_t token_begin, int64_t n_tokens,
                      uint16_t* out, int64_t out_bh_stride, hipStream_t stream) {
    if (BH < 0 || n_tokens < 0) return KIVI_ERR_SHAPE;
    int rc = check_store(src, -1, BH, token_begin, n_tokens);
    if (rc != KIVI_OK) return rc;
    if (bf16 && meta16(src)) return KIVI_ERR_UNSUPPORTED;
    if (BH == 0 || n_tokens == 0) return KIVI_OK;
    if ((rc = check_f16_tensor(out, BH, n_tokens, out_bh_stride, src->head_dim)) != KIVI_OK) return rc;
    const int64_t tiles = BH * ((n_tokens + 31) / 32);
    if ((tiles + 3) / 4 > kMaxBlocks) return KIVI_ERR_SHAPE;
    kivi::DequantArgs a;
    a.codes = src->codes; a.codes_bh_stride = src->codes_bh_stride;
    a.scale = src->scale; a.zero = src->zero; a.meta_bh_stride = src->meta_bh_stride;
    a.BH = BH; a.t0 = token_begin; a.n = n_tokens; a.out = out; a.out_bh_stride = out_bh_stride;
    a.bits = src->bits; a.kind = src->kind; a.group = src->group_size; a.head_dim = src->head_dim;
    a.bf16 = bf16;
    a.meta16 = meta16(src);
    return finish(kivi::launch_dequantize(a, stream));
}

int kivi_dequantize(const kivi_store* src, int64_t BH, int64_t token_begin, int64_t n_tokens,
                    uint16_t* out, int64_t out_bh_stride, hipStream_t stream) {
    return dequantize(false, src, BH, token_begin, n_tokens, out, out_bh_stride, stream);
}

int kivi_dequantize_bf16(const kivi_store* src, int64_t BH, int64_t token_begin, int64_t n_tokens,
                         uint16_t* out, int64_t out_bh_stride, hipStream_t stream) {
    return dequantize(true, src, BH, token_begin, n_tokens, out, out_bh_stride, stream);
}

size_t kivi_decode_attend_workspace_bytes(int64_t B, int32_t Hq, int32_t Hkv, int64_t n_quant,
                                          int64_t n_res, int32_t head_dim, int32_t flags) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || B > kMaxAttendSlabs / Hkv) return 0;
    if (n_quant < 0 || n_res < 0 || n_quant >= kMaxAttendTokens || n_res >= kMaxAttendTokens ||
        n_quant + n_res == 0) return 0;
    if (head_dim < 16 || head_dim > 256 || head_dim % 16 != 0) return 0;
    if ((flags & ~(KIVI_ATTEND_BF16 | KIVI_ATTEND_VARLEN)) != 0) return 0;
    // exactly the plan the matching call will make
    return kivi::plan_attend(B, Hq, Hkv, n_quant, n_res, (flags & KIVI_ATTEND_VARLEN) != 0, head_dim,
                             (flags & KIVI_ATTEND_BF16) != 0).workspace_bytes;
}

}  // extern "C"

namespace kivi {

// Shared validation and launch of the uniform and variable-length attends
// and of the cache's attend; n_quant / n_res are the uniform counts or the
// per-sequence bounds.  res_ring == 0 means a linear residual window;
// otherwise residual token i of a slab is row (res_head + i) mod res_ring.
int decode_attend_entry(const uint16_t* q, int64_t B, int32_t Hq, int32_t Hkv,
                        const kivi_store* k, const kivi_store* v, int64_t n_quant,
                        const uint16_t* k_res, const uint16_t* v_res, int64_t res_bh_stride,
                        int64_t n_res, int64_t res_head, int64_t res_ring,
                        const int32_t* seq_n_quant, const int32_t* seq_n_res,
                        float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, bool bf16, bool static_scratch,
                        const uint16_t* k_new, const uint16_t* v_new, int64_t new_row) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || n_quant < 0 || n_res < 0) return KIVI_ERR_SHAPE;
    if (Hq % Hkv != 0) return KIVI_ERR_SHAPE;
    const int group = Hq / Hkv;
    if (group != 1 && group != 2 && group != 4 && group != 8) return KIVI_ERR_UNSUPPORTED;
    if (n_quant >= kMaxAttendTokens || n_res >= kMaxAttendTokens) return KIVI_ERR_SHAPE;
    if (n_quant + n_res == 0) return KIVI_ERR_SHAPE;
    if (B > kMaxAttendSlabs / Hkv) return KIVI_ERR_SHAPE;              // B * Hkv slabs <= 65535
    if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return KIVI_ERR_SHAPE;
    const int64_t slabs = B * Hkv;
    int rc = check_store(k, KIVI_KEYS, slabs, 0, n_quant);
    if (rc != KIVI_OK) return rc;
    if ((rc = check_store(v, KIVI_VALUES, slabs, 0, n_quant)) != KIVI_OK) return rc;
    if (k->bits != v->bits) return KIVI_ERR_SHAPE;
    if (k->group_size != v->group_size || k->meta_format != v->meta_format) return KIVI_ERR_UNSUPPORTED;
    // head_dim 128 with any group size; any other store head_dim with groups
    // of 32 (binary16 stores are head_dim 128 only, see check_store)
    const int32_t D = k->head_dim;
    if (v->head_dim != D || !(D == kD || k->group_size == 32)) return KIVI_ERR_UNSUPPORTED;
    if (bf16 && meta16(k)) return KIVI_ERR_UNSUPPORTED;        // bfloat16 stores keep binary32 metadata
    if (B == 0) return KIVI_OK;
    if (!q || !out) return KIVI_ERR_NULL;
    if (!aligned16(q) || !aligned16(out)) return KIVI_ERR_ALIGN;
    if (res_ring < 0 || res_head < 0 || (res_ring > 0 && (res_head >= res_ring || n_res > res_ring)) ||
        (res_ring == 0 && res_head != 0) || res_ring >= kMaxAttendTokens) return KIVI_ERR_SHAPE;
    if (n_res > 0) {
        const int64_t rows = res_ring > 0 ? res_ring : n_res;
        if ((rc = check_f16_tensor(k_res, slabs, rows, res_bh_stride, D)) != KIVI_OK) return rc;
        if ((rc = check_f16_tensor(v_res, slabs, rows, res_bh_stride, D)) != KIVI_OK) return rc;
    }
    if (k_new || v_new) {
        // a fused append: token n_res - 1 comes from row s of k_new / v_new and
        // is written to ring row new_row, which must not hold one of the
        // other n_res - 1 tokens (uniform batches, a ring window only)
        if (!k_new || !v_new) return KIVI_ERR_NULL;
        if (seq_n_quant || seq_n_res || res_ring == 0 || n_res < 1) return KIVI_ERR_SHAPE;
        if (new_row != (res_head + n_res - 1) % res_ring) return KIVI_ERR_SHAPE;
        if ((rc = check_f16_tensor(k_new, slabs, 1, D, D)) != KIVI_OK) return rc;
        if ((rc = check_f16_tensor(v_new, slabs, 1, D, D)) != KIVI_OK) return rc;
    }
    const kivi::AttendPlan plan = kivi::plan_attend(B, Hq, Hkv, n_quant, n_res, seq_n_quant != nullptr, D, bf16);
    if (plan.n_split > kMaxBlocks || slabs > kMaxAttendSlabs || B * Hq > kMaxBlocks) return KIVI_ERR_SHAPE;
    if (static_scratch) {
        // the library's own array: a size check, then its device address
        if (plan.workspace_bytes > kivi::static_attend_scratch_bytes()) return KIVI_ERR_WORKSPACE;
        const hipError_t e = kivi::static_attend_scratch(&workspace);
        if (e != hipSuccess) return finish(e);
        workspace_bytes = kivi::static_attend_scratch_bytes();
    }
    if (!workspace || workspace_bytes < plan.workspace_bytes) return KIVI_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KIVI_ERR_ALIGN;

    kivi::AttendArgs a;
    a.q = q; a.B = B; a.Hq = Hq; a.Hkv = Hkv;
    a.k_codes = k->codes; a.k_scale = k->scale; a.k_zero = k->zero;
    a.v_codes = v->codes; a.v_scale = v->scale; a.v_zero = v->zero;
    a.k_codes_bh_stride = k->codes_bh_stride; a.v_codes_bh_stride = v->codes_bh_stride;
    a.k_meta_bh_stride = k->meta_bh_stride; a.v_meta_bh_stride = v->meta_bh_stride;
    a.n_quant = n_quant;
    a.k_res = n_res > 0 ? k_res : q;     // never read when n_res == 0
    a.v_res = n_res > 0 ? v_res : q;
    a.res_bh_stride = n_res > 0 ? res_bh_stride : 0;
    a.n_res = n_res;
    a.res_head = static_cast<int32_t>(res_head);
    a.res_ring = res_ring > 0 ? static_cast<int32_t>(res_ring) : (1 << 30);
    a.seq_n_quant = seq_n_quant; a.seq_n_res = seq_n_res;
    a.softmax_scale = softmax_scale; a.out = out;
    a.workspace = workspace; a.bits = k->bits; a.group = k->group_size;
    a.meta16 = meta16(k);
    a.bf16 = bf16;
    a.head_dim = D;
    a.k_new = k_new;
    a.v_new = v_new;
    a.new_row = static_cast<int32_t>(new_row);
    return finish(kivi::launch_decode_attend(a, plan, stream));
}

}  // namespace kivi

extern "C" {

int kivi_decode_attend(const uint16_t* q, int64_t B, int32_t Hq, int32_t Hkv,
                       const kivi_store* k, const kivi_store* v, int64_t n_quant,
                       const uint16_t* k_res, const uint16_t* v_res, int64_t res_bh_stride,
                       int64_t n_res, float softmax_scale, float* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return kivi::decode_attend_entry(q, B, Hq, Hkv, k, v, n_quant, k_res, v_res, res_bh_stride,
                                     n_res, 0, 0, nullptr, nullptr, softmax_scale, out, workspace,
                                     workspace_bytes, stream);
}

int kivi_decode_attend_noalloc(const uint16_t* q, int64_t B, int32_t Hq, int32_t Hkv,
                               const kivi_store* k, const kivi_store* v, int64_t n_quant,
                               const uint16_t* k_res, const uint16_t* v_res, int64_t res_bh_stride,
                               int64_t n_res, float softmax_scale, float* out, hipStream_t stream) {
    return kivi::decode_attend_entry(q, B, Hq, Hkv, k, v, n_quant, k_res, v_res, res_bh_stride,
                                     n_res, 0, 0, nullptr, nullptr, softmax_scale, out, nullptr, 0,
                                     stream, false, true);
}

int kivi_decode_attend_varlen(const uint16_t* q, int64_t B, int32_t Hq, int32_t Hkv,
                              const kivi_store* k, const kivi_store* v,
                              const int32_t* n_quant, int64_t max_n_quant,
                              const uint16_t* k_res, const uint16_t* v_res, int64_t res_bh_stride,
                              const int32_t* n_res, int64_t max_n_res, float softmax_scale,
                              float* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    if (B > 0 && (!n_quant || !n_res)) return KIVI_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(n_quant) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(n_res) & 3u) != 0) return KIVI_ERR_ALIGN;
    return kivi::decode_attend_entry(q, B, Hq, Hkv, k, v, max_n_quant, k_res, v_res,
                                     res_bh_stride, max_n_res, 0, 0, n_quant, n_res,
                                     softmax_scale, out, workspace, workspace_bytes, stream);
}

int kivi_decode_attend_bf16(const uint16_t* q, int64_t B, int32_t Hq, int32_t Hkv,
                            const kivi_store* k, const kivi_store* v, int64_t n_quant,
                            const uint16_t* k_res, const uint16_t* v_res, int64_t res_bh_stride,
                            int64_t n_res, float softmax_scale, float* out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return kivi::decode_attend_entry(q, B, Hq, Hkv, k, v, n_quant, k_res, v_res, res_bh_stride,
                                     n_res, 0, 0, nullptr, nullptr, softmax_scale, out, workspace,
                                     workspace_bytes, stream, true);
}

int kivi_decode_attend_varlen_bf16(const uint16_t* q, int64_t B, int32_t Hq, int32_t Hkv,
                                   const kivi_store* k, const kivi_store* v,
                                   const int32_t* n_quant, int64_t max_n_quant,
                                   const uint16_t* k_res, const uint16_t* v_res,
                                   int64_t res_bh_stride, const int32_t* n_res, int64_t max_n_res,
                                   float softmax_scale, float* out, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    if (B > 0 && (!n_quant || !n_res)) return KIVI_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(n_quant) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(n_res) & 3u) != 0) return KIVI_ERR_ALIGN;
    return kivi::decode_attend_entry(q, B, Hq, Hkv, k, v, max_n_quant, k_res, v_res,
                                     res_bh_stride, max_n_res, 0, 0, n_quant, n_res,
                                     softmax_scale, out, workspace, workspace_bytes, stream, true);
}

const char* kivi_status_string(int status) {
    switch (status) {
        case KIVI_OK: return "ok";
        case KIVI_ERR_NULL: return "a required pointer is NULL";
        case KIVI_ERR_SHAPE: return "invalid shape, offset or window";
        case KIVI_ERR_UNSUPPORTED: return "unsupported bits, group size, head dim, kind or head ratio";
        case KIVI_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
        case KIVI_ERR_WORKSPACE: return "attend workspace missing or too small";
        case KIVI_ERR_HIP: return "HIP launch failed (see kivi_last_hip_error)";
        default: return "unknown status";
    }
}

int kivi_last_hip_error(void) { return g_last_hip_error; }

// The calibration kernels take at most one workgroup per 16 KiB: sizes up to
// 2^31 - 1 workgroups (below 2^45 bytes, inside the address space).
static bool calib_size_ok(size_t n_bytes) { return n_bytes / 16384 < static_cast<size_t>(kMaxBlocks); }

int kivi_calib_copy(const void* src, void* dst, size_t n_bytes, hipStream_t stream) {
    if (!src || !dst) return KIVI_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst) || n_bytes % 16 != 0) return KIVI_ERR_ALIGN;
    if (!calib_size_ok(n_bytes)) return KIVI_ERR_SHAPE;
    if (n_bytes == 0) return KIVI_OK;
    return finish(kivi::launch_calib_copy(src, dst, n_bytes, stream));
}

int kivi_calib_read(const void* src, size_t n_bytes, void* sink, hipStream_t stream) {
    if (!src || !sink) return KIVI_ERR_NULL;
    if (!aligned16(src) || !aligned16(sink) || n_bytes % 16 != 0) return KIVI_ERR_ALIGN;
    if (!calib_size_ok(n_bytes)) return KIVI_ERR_SHAPE;
    if (n_bytes == 0) return KIVI_OK;
    return finish(kivi::launch_calib_read(src, n_bytes, static_cast<uint32_t*>(sink), stream));
}

int kivi_calib_write(void* dst, size_t n_bytes, hipStream_t stream) {
    if (!dst) return KIVI_ERR_NULL;
    if (!aligned16(dst) || n_bytes % 16 != 0) return KIVI_ERR_ALIGN;
    if (!calib_size_ok(n_bytes)) return KIVI_ERR_SHAPE;
    if (n_bytes == 0) return KIVI_OK;
    return finish(kivi::launch_calib_write(dst, n_bytes, stream));
}

int kivi_calib_mix(const void* src, size_t n_bytes, void* dst, hipStream_t stream) {
    if (!src || !dst) return KIVI_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst) || n_bytes % 16 != 0) return KIVI_ERR_ALIGN;
    if (!calib_size_ok(n_bytes)) return KIVI_ERR_SHAPE;
    if (n_bytes == 0) return KIVI_OK;
    return finish(kivi::launch_calib_mix(src, n_bytes, dst, stream));
}

}  // extern "C"
