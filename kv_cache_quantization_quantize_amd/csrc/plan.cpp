// plan.cpp -- host-side planning of the decode attend: how the token axis of
// every (sequence, kv head) is split over waves, and the workspace the split
// needs (one partial softmax state per split, merged by the combine kernel).
// The VeloxQuant-MLX "Benchmarks" page ("KV-Cache Kernel Roofline: What
// Actually Limits Decode") found its decode kernel bound by how few
// threadgroups it dispatched, not by bandwidth; the split gives every shape
// enough waves to fill the chip.  Host code only, so it builds and is
// checked without a GPU.
#include <algorithm>

#include "kivi_launch.h"

namespace kivi {

// Split of the token axis.  Small problems (no more 32-token steps than the
// chip holds waves) get one step per wave: everything is in flight at once.
// Larger ones get as few whole rounds of kWaveSlots waves as keep a wave at
// most kMaxStepsPerWave steps, with the steps spread evenly, so the last
// round is not a short tail.
AttendPlan plan_attend(int64_t B, int Hq, int Hkv, int64_t n_quant, int64_t n_res, bool varlen,
                       int head_dim, bool bf16) {
    const int64_t pairs = B * Hkv;
    const int64_t steps_q = (n_quant + kAttendStep - 1) / kAttendStep;
    const int64_t steps = steps_q + (n_res + kAttendStep - 1) / kAttendStep;
    const int64_t total = pairs * steps;
    // head_dims other than 64, 128 and 256 run on the kernels of the next of
    // them, with their occupancy
    const int64_t slots = head_dim > 128 ? kWaveSlotsD256 : bf16 ? kWaveSlotsBF16 : kWaveSlots;
    int64_t spw = 1;
    if (total > slots) {
        // A variable-length batch sizes the grid for its longest sequence;
        // the shorter ones leave waves with little or nothing to do, so it
        // gets four times finer splits and the hardware refills the freed
        // slots with the remaining work.
        const int64_t per_round = varlen ? slots * 4 : slots;
        const int64_t rounds = (total + per_round * kMaxStepsPerWave - 1) / (per_round * kMaxStepsPerWave);
        spw = (total + rounds * per_round - 1) / (rounds * per_round);
    }
    // Small and mid-size calls take fewer, longer waves: each wave pays a
    // fixed cost (query load, LDS setup, its partial and its share of the
    // combine), and about 700 waves already keep these sizes at their best.
    // Measured per call on MI355X, fp16, one step of loads in flight (steps
    // per wave -> us): B=1 x 16384 tokens 2 -> 22.0, 6 -> 15.9; B=4 x 2048:
    // 1 -> 13.0, 4 -> 11.9; B=16 x 2048: 3 -> 21.4, 9 -> 17.1; B=4 x 16384:
    // 6 -> 28.8, 9 -> 26.8.  At every fp16 shape the rule below lands within
    // 2% of the best; bfloat16 follows it within 2% but at B=4 x 2048 (13.9
    // against 13.1 us at 3 steps).
    const int64_t longer = (total + 699) / 700;
    spw = std::max(spw, std::min<int64_t>(9, longer));
    AttendPlan p;
    p.steps_q = steps_q;
    p.steps_per_wave = spw;
    p.n_split = (steps + spw - 1) / spw;
    const size_t rows = static_cast<size_t>(B) * static_cast<size_t>(Hq) * static_cast<size_t>(p.n_split);
    p.ml_offset = (rows * head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255);
    p.workspace_bytes = p.ml_offset + rows * 2 * sizeof(float);
    return p;
}

}  // namespace kivi
