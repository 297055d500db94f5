// launch_stubs.cpp -- host stand-ins for libkivi's kernel launchers, for a
// CPU build of the C ABI's validation code (abi.cpp, cache.cpp, plan.cpp)
// under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Each stand-in reads the first and the last byte of every range the real
// kernel would read or write for its arguments (per slab), so a launch whose
// arguments reach outside the caller's buffers (host allocations of exactly
// the documented sizes in the driver) is reported by AddressSanitizer.  The
// row-gather launch, whose addressing is all host-computed ring arithmetic,
// copies its rows for real.  Nothing here runs on a GPU.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kivi_launch.h"

namespace kivi {

long g_launches = 0;
// Optional checks the driver installs: called with every flush and attend
// launch's arguments before the footprint is read.
void (*g_on_flush)(bool keys, const FlushArgs& a) = nullptr;
void (*g_on_attend)(const AttendArgs& a) = nullptr;

namespace {

volatile unsigned char g_sink;

void touch(const void* p, int64_t bytes) {
    if (bytes <= 0) return;
    const unsigned char* c = static_cast<const unsigned char*>(p);
    g_sink ^= c[0];
    g_sink ^= c[bytes - 1];
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

void flush_footprint(bool keys, const FlushArgs& a) {
    const int64_t D = a.head_dim, W = D * a.bits / 32, es = a.meta16 ? 2 : 4;
    const int64_t NGD = cdiv(D, a.group);
    for (int64_t bh = 0; bh < a.BH; ++bh) {
        touch(a.x + bh * a.x_bh_stride, a.S * D * 2);
        touch(a.codes + bh * a.codes_bh_stride + a.dst_token * W, a.S * W * 4);
        int64_t m0, mn;
        if (keys) {
            m0 = bh * a.meta_bh_stride + a.dst_token / a.group * D;
            mn = (cdiv(a.dst_token + a.S, a.group) - a.dst_token / a.group) * D;
        } else {
            m0 = bh * a.meta_bh_stride + a.dst_token * NGD;
            mn = a.S * NGD;
        }
        touch(static_cast<const char*>(a.scale) + m0 * es, mn * es);
        touch(static_cast<const char*>(a.zero) + m0 * es, mn * es);
        if (a.recon) touch(a.recon + bh * a.recon_bh_stride, a.S * D * 2);
    }
}

}  // namespace

hipError_t launch_key_flush(const FlushArgs& a, hipStream_t) {
    ++g_launches;
    if (g_on_flush) g_on_flush(true, a);
    flush_footprint(true, a);
    return hipSuccess;
}

hipError_t launch_value_flush(const FlushArgs& a, hipStream_t) {
    ++g_launches;
    if (g_on_flush) g_on_flush(false, a);
    flush_footprint(false, a);
    return hipSuccess;
}

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t) {
    ++g_launches;
    const int64_t D = a.head_dim, W = D * a.bits / 32, es = a.meta16 ? 2 : 4;
    const int64_t NGD = cdiv(D, a.group);
    for (int64_t bh = 0; bh < a.BH; ++bh) {
        touch(a.codes + bh * a.codes_bh_stride + a.t0 * W, a.n * W * 4);
        int64_t m0, mn;
        if (a.kind == KIVI_KEYS) {
            m0 = bh * a.meta_bh_stride + a.t0 / a.group * D;
            mn = (cdiv(a.t0 + a.n, a.group) - a.t0 / a.group) * D;
        } else {
            m0 = bh * a.meta_bh_stride + a.t0 * NGD;
            mn = a.n * NGD;
        }
        touch(static_cast<const char*>(a.scale) + m0 * es, mn * es);
        touch(static_cast<const char*>(a.zero) + m0 * es, mn * es);
        touch(a.out + bh * a.out_bh_stride, a.n * D * 2);
    }
    return hipSuccess;
}

hipError_t launch_decode_attend(const AttendArgs& a, const AttendPlan& p, hipStream_t) {
    ++g_launches;
    if (g_on_attend) g_on_attend(a);
    const int64_t D = a.head_dim, W = D * a.bits / 32, es = a.meta16 ? 2 : 4;
    const int64_t NGD = cdiv(D, a.group);
    touch(a.q, a.B * a.Hq * D * 2);
    touch(a.out, a.B * a.Hq * D * 4);
    touch(a.workspace, static_cast<int64_t>(p.workspace_bytes));
    if (a.seq_n_quant) {
        touch(a.seq_n_quant, a.B * 4);
        touch(a.seq_n_res, a.B * 4);
    }
    for (int64_t s = 0; s < a.B * a.Hkv; ++s) {
        const int64_t nq = a.n_quant;
        touch(a.k_codes + s * a.k_codes_bh_stride, nq * W * 4);
        touch(a.v_codes + s * a.v_codes_bh_stride, nq * W * 4);
        touch(static_cast<const char*>(a.k_scale) + s * a.k_meta_bh_stride * es, cdiv(nq, a.group) * D * es);
        touch(static_cast<const char*>(a.k_zero) + s * a.k_meta_bh_stride * es, cdiv(nq, a.group) * D * es);
        touch(static_cast<const char*>(a.v_scale) + s * a.v_meta_bh_stride * es, nq * NGD * es);
        touch(static_cast<const char*>(a.v_zero) + s * a.v_meta_bh_stride * es, nq * NGD * es);
        for (int64_t i = 0; i < a.n_res; ++i) {
            const int64_t row = (a.res_head + i) % a.res_ring;
            touch(a.k_res + s * a.res_bh_stride + row * D, D * 2);
            touch(a.v_res + s * a.res_bh_stride + row * D, D * 2);
        }
        if (a.k_new) {
            // a fused append: the new rows are read and copied into ring row
            // new_row, as the kernel does
            touch(a.k_new + s * D, D * 2);
            touch(a.v_new + s * D, D * 2);
            uint16_t* kd = const_cast<uint16_t*>(a.k_res) + s * a.res_bh_stride + int64_t{a.new_row} * D;
            uint16_t* vd = const_cast<uint16_t*>(a.v_res) + s * a.res_bh_stride + int64_t{a.new_row} * D;
            std::memcpy(kd, a.k_new + s * D, static_cast<size_t>(D) * 2);
            std::memcpy(vd, a.v_new + s * D, static_cast<size_t>(D) * 2);
        }
    }
    return hipSuccess;
}

hipError_t launch_gather_rows(const RowGather& k, const RowGather& v, int64_t slabs, int64_t n_rows, int D,
                              hipStream_t) {
    ++g_launches;
    for (const RowGather* c : {&k, &v}) {
        for (int64_t s = 0; s < slabs; ++s) {
            for (int64_t r = 0; r < n_rows; ++r) {
                const bool from_a = r < c->n_a;
                const RowSpan& src = from_a ? c->a : c->b;
                const int64_t i = src.first + (from_a ? r : r - c->n_a);
                const int64_t srow = src.ring > 0 ? i % src.ring : i;
                const int64_t j = c->dst.first + r;
                const int64_t drow = c->dst.ring > 0 ? j % c->dst.ring : j;
                std::memmove(c->dst.base + s * c->dst.bh_stride + drow * D,
                             src.base + s * src.bh_stride + srow * D, static_cast<size_t>(D) * 2);
            }
        }
    }
    return hipSuccess;
}

hipError_t launch_calib_copy(const void* src, void* dst, size_t n, hipStream_t) {
    ++g_launches;
    touch(src, static_cast<int64_t>(n));
    touch(dst, static_cast<int64_t>(n));
    return hipSuccess;
}

hipError_t launch_calib_read(const void* src, size_t n, uint32_t* sink, hipStream_t) {
    ++g_launches;
    touch(src, static_cast<int64_t>(n));
    touch(sink, 4);
    return hipSuccess;
}

hipError_t launch_calib_write(void* dst, size_t n, hipStream_t) {
    ++g_launches;
    touch(dst, static_cast<int64_t>(n));
    return hipSuccess;
}

hipError_t launch_calib_mix(const void* src, size_t n, void* dst, hipStream_t) {
    ++g_launches;
    touch(src, static_cast<int64_t>(n));
    touch(dst, static_cast<int64_t>(n / 16 * 3 / 8 * 16));
    return hipSuccess;
}

size_t static_attend_scratch_bytes() { return size_t{32} << 20; }

hipError_t static_attend_scratch(void** ptr) {
    static unsigned char* buf = static_cast<unsigned char*>(std::aligned_alloc(256, size_t{32} << 20));
    *ptr = buf;
    return hipSuccess;
}

}  // namespace kivi
