// Launch arguments of the decode-attention kernel (wgn_attn.hip), shared by
// the host planner (wgn_api.cpp) and the kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace wgn {

constexpr int32_t ATT_D = 128;          // head dimension this kernel is written for
#ifndef WGN_ATT_SLOTS_PER_WAVE
#define WGN_ATT_SLOTS_PER_WAVE 32
#endif
// Fan-in of the merge tree.  Measured on MI355X: 8 beats 16 and 32 (a merge
// of 32 partials costs a workgroup several microseconds of coherent loads,
// while another tree level costs little more than one ticket).
#ifndef WGN_ATT_FAN_LOG2
#define WGN_ATT_FAN_LOG2 3
#endif
#ifndef WGN_ATT_WAVES
#define WGN_ATT_WAVES 4
#endif
constexpr int32_t ATT_SLOTS_PER_WAVE = WGN_ATT_SLOTS_PER_WAVE;
constexpr int32_t ATT_WAVES = WGN_ATT_WAVES;                      // waves per workgroup
constexpr int32_t ATT_THREADS = 64 * ATT_WAVES;
constexpr int32_t ATT_CHUNK = ATT_WAVES * ATT_SLOTS_PER_WAVE;     // cache slots per workgroup
constexpr int32_t ATT_FAN_LOG2 = WGN_ATT_FAN_LOG2;
constexpr int32_t ATT_FAN = 1 << ATT_FAN_LOG2;  // partials merged by one workgroup
constexpr int32_t ATT_MAX_LEVELS = 9;   // merge levels above the chunks
constexpr int32_t ATT_MAX_GROUP = 8;    // query heads per key/value head
constexpr int32_t ATT_MAX_SLOTS = 1 << 24;

// Floats of one partial result (per key/value head and batch row): the
// weighted value sums acc[G][D], then the running maxima m[G] and the weight
// sums l[G]; padded to 16 bytes.
__host__ __device__ constexpr int32_t att_entry_floats(int32_t G) { return (G * (ATT_D + 2) + 3) & ~3; }

struct AttnArgs {
    const uint16_t *q;        // [B][Hq][D]
    const uint16_t *k_new;    // [B][Hkv][D]
    const uint16_t *v_new;    // [B][Hkv][D]
    uint16_t *k_cache;        // [B][Hkv][slots][D]
    uint16_t *v_cache;        // [B][Hkv][slots][D]
    const int32_t *pos;       // [B]
    uint16_t *out;            // [B][Hq][D]
    // part[L]: partials of level L (L = 0: one per chunk), [B*Hkv][count[L]] entries
    float *part[ATT_MAX_LEVELS];
    // tick[L]: arrival counters of the level-L items (L >= 1), [B*Hkv][count[L]]
    uint32_t *tick[ATT_MAX_LEVELS + 1];
    int32_t count[ATT_MAX_LEVELS + 1];  // items per (batch row, key/value head) at each level
    int32_t top;                        // merge levels; 0: one chunk writes the output itself
    int32_t slots, hq, hkv;
    float scale_log2;                   // score scale times log2(e): weights are 2^(s - m)
};

// Per-level item counts for a cache of `slots` slots; returns the number of
// merge levels, or -1 if more than ATT_MAX_LEVELS would be needed.
inline int32_t att_levels(int32_t slots, int32_t (&count)[ATT_MAX_LEVELS + 1]) {
    for (auto &c : count) c = 0;
    count[0] = (slots + ATT_CHUNK - 1) / ATT_CHUNK;
    int32_t top = 0;
    while (count[top] > 1) {
        if (top == ATT_MAX_LEVELS) return -1;
        count[top + 1] = (count[top] + ATT_FAN - 1) / ATT_FAN;
        ++top;
    }
    return top;
}

hipError_t launch_decode_attention(const AttnArgs &a, int32_t group, int32_t batch, hipStream_t s);

}  // namespace wgn
