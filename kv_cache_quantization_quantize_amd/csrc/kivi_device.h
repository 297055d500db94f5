// kivi_device.h -- device-side helpers shared by the libkivi kernels
// (internal to the library; not part of the C ABI).
//
// Fixed geometry of every kernel here: head_dim 128, group_size 32, wave64.
// A "tile" is 32 consecutive tokens x 128 channels of one bh slab (8 KiB of
// fp16).  Lane l of the wave that owns a tile holds channels 8*(l%16) ..
// 8*(l%16)+7 of tokens tile_start + (l/16) + 4*i, i = 0..7: each token row
// of the tile is read by 16 lanes as one contiguous 256-byte segment, so the
// wave reads the tile as 8 fully coalesced 1 KiB loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace kivi {

constexpr int kHeadDim = 128;
constexpr int kGroup = 32;
constexpr int kLanesPerRow = 16;   // lanes covering one 128-channel token row
constexpr int kRowsPerWave = 4;    // token rows covered by one wave at a time
constexpr int kTokPerLane = 8;     // token rows held by one lane per tile
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = 64 * kWavesPerBlock;

struct h8 {                        // 8 fp16 values as raw bits (one 16 B load)
    uint4 v;
};

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// fp32 -> fp16, round to nearest even (the default rounding mode).
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8]) {
    f[0] = f16_to_f32(v.x & 0xffffu); f[1] = f16_to_f32(v.x >> 16);
    f[2] = f16_to_f32(v.y & 0xffffu); f[3] = f16_to_f32(v.y >> 16);
    f[4] = f16_to_f32(v.z & 0xffffu); f[5] = f16_to_f32(v.z >> 16);
    f[6] = f16_to_f32(v.w & 0xffffu); f[7] = f16_to_f32(v.w >> 16);
}

__device__ __forceinline__ uint4 pack8(const uint32_t (&h)[8]) {
    uint4 v;
    v.x = h[0] | (h[1] << 16);
    v.y = h[2] | (h[3] << 16);
    v.z = h[4] | (h[5] << 16);
    v.w = h[6] | (h[7] << 16);
    return v;
}

// A zero extreme is stored as +0, so the result does not depend on which
// signed zero a reduction kept.
__device__ __forceinline__ float canon_zero(float v) { return v == 0.0f ? 0.0f : v; }

// Code of one element: clip(rint((x - zero) / scale), 0, levels), with code 0
// for a constant group (scale 0).  Two IEEE roundings (subtract, divide),
// then round-half-even.
template <int BITS>
__device__ __forceinline__ uint32_t quant_code(float x, float zero, float scale) {
    constexpr float kLevels = static_cast<float>((1 << BITS) - 1);
    if (scale == 0.0f) return 0u;
    const float t = x - zero;
    const float u = t / scale;
    float r = __builtin_rintf(u);
    r = r < 0.0f ? 0.0f : r;
    r = r > kLevels ? kLevels : r;
    return static_cast<uint32_t>(r);
}

// Reconstruction fp16_rne(fl(fl(q * scale) + zero)) -- two roundings, no FMA.
__device__ __forceinline__ uint32_t recon_f16(uint32_t q, float scale, float zero) {
    const float prod = static_cast<float>(q) * scale;
    const float sum = prod + zero;
    return f32_to_f16(sum);
}

}  // namespace kivi
