// kivi_launch.h -- host launchers of the libkivi kernels (internal).  The
// C ABI in abi.cpp validates every argument before calling these; they only
// size grids and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kivi.h"

namespace kivi {

struct FlushArgs {
    const uint16_t* x;
    int64_t BH, S, x_bh_stride;
    uint32_t* codes;
    int64_t codes_bh_stride;
    void* scale;                   // float, or binary16 bits when meta16
    void* zero;
    int64_t meta_bh_stride;
    int64_t dst_token;
    uint16_t* recon;               // may be null
    int64_t recon_bh_stride;
    int bits;
    int group;                     // 32, 64 or 128
    int head_dim;                  // 64, 128 or 256
    bool bf16;                     // x and recon hold bfloat16 (else fp16)
    bool meta16;                   // binary16 scale/zero (fp16 x, head_dim 128)
};

struct DequantArgs {
    const uint32_t* codes;
    int64_t codes_bh_stride;
    const void* scale;             // float, or binary16 bits when meta16
    const void* zero;
    int64_t meta_bh_stride;
    int64_t BH, t0, n;
    uint16_t* out;
    int64_t out_bh_stride;
    int bits;
    int kind;                      // KIVI_KEYS or KIVI_VALUES
    int group;                     // 32, 64 or 128
    int head_dim;                  // 64, 128 or 256
    bool bf16;                     // out holds bfloat16 (else fp16)
    bool meta16;                   // binary16 scale/zero (head_dim 128)
};

struct AttendArgs {
    const uint16_t* q;
    int64_t B;
    int Hq, Hkv;
    const uint32_t* k_codes;
    const void* k_scale;           // float, or binary16 bits when meta16
    const void* k_zero;
    const uint32_t* v_codes;
    const void* v_scale;
    const void* v_zero;
    int64_t k_codes_bh_stride, v_codes_bh_stride;
    int64_t k_meta_bh_stride, v_meta_bh_stride;
    int64_t n_quant;               // store tokens (varlen: the per-sequence bound)
    const uint16_t* k_res;
    const uint16_t* v_res;
    int64_t res_bh_stride;
    int64_t n_res;                 // residual tokens (varlen: the per-sequence bound)
    // Residual token i of a slab sits in row (res_head + i) mod res_ring of
    // the slab (a ring of res_ring rows); a linear window has res_head = 0
    // and res_ring >= n_res.
    int32_t res_head, res_ring;
    // Variable-length batches: device int32 [B] per-sequence lengths, each
    // clamped to [0, n_quant] / [0, n_res]; both null for a uniform batch.
    const int32_t* seq_n_quant;
    const int32_t* seq_n_res;
    float softmax_scale;
    float* out;
    void* workspace;
    int bits;
    int group;                     // 32, 64 or 128 (keys and values alike)
    bool meta16;                   // binary16 scale/zero (keys and values alike)
    bool bf16;                     // q, residual and the reconstruction in bfloat16
    int head_dim;                  // 128; others with groups of 32 and binary32 scale/zero
                                   // (q, residual, out and the partials have head_dim channels)
    // Fused append (the decode-loop cache): residual token n_res - 1 of slab s
    // is read from row s of k_new / v_new (head_dim elements each) instead of
    // from the residual window, and the wave that holds that token writes
    // both rows into row new_row of the slab's window (k_res / v_res, which
    // are then the cache's own rings).  No other wave of the launch reads
    // that row.  k_new null: no fused append.
    const uint16_t* k_new = nullptr;
    const uint16_t* v_new = nullptr;
    int32_t new_row = 0;
};

// Three waves per SIMD for the attend at head_dim 64 and 128, fp16 and
// bfloat16 alike (at most 168 VGPRs; four would need 128 and spill), so the
// chip holds 256 CUs x 4 SIMDs x 3 = 3072 of these waves at once.  Each wave
// keeps KIVI_ATTEND_NBUF - 1 steps of loads in flight while it computes one:
// one step (about 6 KiB a wave, 72 KiB a CU) measured faster than two, as
// the streaming read calibration peaked at about 48 KiB in flight per CU and
// slowed with more.  Interleaved on MI355X against two steps in flight at 2
// waves per SIMD: bfloat16 at B=32 x 16384 tokens 164-173 -> 156 us, B=16
// 90 -> 84 us; fp16 B=32 x 2048 31.0 -> 29.4 us, B=32 x 16384 148 -> 147.
// The bfloat16 4-bit instances keep 12 bytes per lane in scratch at 168
// VGPRs and are still faster than at two waves.
#ifndef KIVI_ATTEND_WAVES_PER_SIMD
#define KIVI_ATTEND_WAVES_PER_SIMD 3
#endif
#ifndef KIVI_ATTEND_BF16_WAVES
#define KIVI_ATTEND_BF16_WAVES 3
#endif
constexpr int64_t kWaveSlots = 256 * 4 * KIVI_ATTEND_WAVES_PER_SIMD;
constexpr int64_t kWaveSlotsBF16 = 256 * 4 * KIVI_ATTEND_BF16_WAVES;   // bfloat16, head_dim up to 128
constexpr int64_t kWaveSlotsD256 = 256 * 4 * 2;                         // the head_dim 256 kernels
constexpr int kAttendStep = 32;                 // tokens per wave step (one key group)
constexpr int64_t kMaxStepsPerWave = 64;

// Split of the token axis chosen for an attend shape; the workspace holds
// one (m, l, o[head_dim]) partial per (sequence, query head, split): the o
// rows first, then the (m, l) pairs at ml_offset.
struct AttendPlan {
    int64_t steps_q;               // 32-token steps over store tokens [0, n_quant)
    int64_t steps_per_wave;        // consecutive steps of store-then-residual per wave
    int64_t n_split;               // waves per (sequence, kv head)
    size_t ml_offset;              // bytes from the workspace start to the (m, l) pairs
    size_t workspace_bytes;
};
AttendPlan plan_attend(int64_t B, int Hq, int Hkv, int64_t n_quant, int64_t n_res, bool varlen,
                       int head_dim = 128, bool bf16 = false);

hipError_t launch_key_flush(const FlushArgs& a, hipStream_t stream);
hipError_t launch_value_flush(const FlushArgs& a, hipStream_t stream);
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t stream);
hipError_t launch_decode_attend(const AttendArgs& a, const AttendPlan& p, hipStream_t stream);
// Row copies of the cache (one launch for keys and values): row r < n_rows
// of every slab comes from span a (r < n_a) or from span b (row r - n_a) and
// goes to row r of span dst.  A span's row i is row (first + i) mod ring of
// the slab for a ring (ring > 0), row first + i otherwise; rows hold D
// 16-bit values.
struct RowSpan {
    uint16_t* base;                // slab 0 (read-only for sources)
    int64_t bh_stride;             // elements between slabs
    int64_t first;                 // the span's first row
    int64_t ring;                  // rows of the ring, or 0 for a linear span
};
struct RowGather {
    RowSpan dst, a, b;
    int64_t n_a;
};
hipError_t launch_gather_rows(const RowGather& k, const RowGather& v, int64_t slabs, int64_t n_rows, int D,
                              hipStream_t stream);

// The attend entry point behind kivi_decode_attend(_varlen) and the cache:
// validates on the host, then launches (see abi.cpp).  With static_scratch
// the workspace arguments are ignored and the library's own device array is
// used (kivi_decode_attend_noalloc).
int decode_attend_entry(const uint16_t* q, int64_t B, int32_t Hq, int32_t Hkv,
                        const kivi_store* k, const kivi_store* v, int64_t n_quant,
                        const uint16_t* k_res, const uint16_t* v_res, int64_t res_bh_stride,
                        int64_t n_res, int64_t res_head, int64_t res_ring,
                        const int32_t* seq_n_quant, const int32_t* seq_n_res,
                        float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, bool bf16 = false, bool static_scratch = false,
                        const uint16_t* k_new = nullptr, const uint16_t* v_new = nullptr,
                        int64_t new_row = 0);

// The library-owned attend workspace (noalloc.hip): its size, and its device
// address on the current device (resolved on the first call per device).
size_t static_attend_scratch_bytes();
hipError_t static_attend_scratch(void** ptr);

// KIVI_OK, or KIVI_ERR_HIP after recording e for kivi_last_hip_error.
int hip_status(hipError_t e);

hipError_t launch_calib_copy(const void* src, void* dst, size_t n_bytes, hipStream_t stream);
hipError_t launch_calib_read(const void* src, size_t n_bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_calib_write(void* dst, size_t n_bytes, hipStream_t stream);
hipError_t launch_calib_mix(const void* src, size_t n_bytes, void* dst, hipStream_t stream);

}  // namespace kivi
