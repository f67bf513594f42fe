// Device side of the per-layer expert-slot cache: the table view, the
// lookup of one token by one wave, and the copy of missed blobs by a group
// of workgroups.  Used by the standalone lookup/fill kernels and by the
// decode step that plans and fills on the GPU.
//
// Policy (reading of the pages' "LFU", shilu.ai README translation,
// "推理引擎的工作原理"): a slot's count is 1 on fill and +1 per hit; the
// token's own ids are pinned; misses are taken in rank order; the victim is
// the lowest empty slot, else the unpinned slot with the smallest (count,
// last-use token, slot index).  The LRU option (sh.edu-sjtu.cn, "三件事")
// takes the unpinned slot with the smallest (last-use token, slot index).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tf.h"

// Plain device view of the tables (passed to kernels by value).
struct SlotDev {
    int L, E, S, k;
    int policy;                // TF_SLOT_LFU or TF_SLOT_LRU
    int64_t trace_cap;
    int32_t *slot_of;          // [L][E]  -1 = not cached
    int16_t *expert_of;        // [L][S]  -1 = empty
    uint32_t *count;           // [L][S]
    uint32_t *last;            // [L][S]  last-use token
    uint32_t *tok;             // [L]     tokens seen
    int8_t *trace_hit;         // [L][cap*k]
    int16_t *trace_slot;       // [L][cap*k]
    int32_t *miss_dev;         // [L][1+2k] device alias of the mapped pinned miss list
    int32_t *miss_gpu;         // [L][1+2k] the same list in device memory
    unsigned long long *nfill; // blobs moved by fills planned on the GPU
};

namespace slotk {

template <int CTRL>
__device__ __forceinline__ uint32_t min_dpp(uint32_t x) {
    const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
    return x < y ? x : y;
}

// Smallest value over the wave (every lane gets it): DPP within rows of 16,
// then the four row results.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min_dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v = min_dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v = min_dpp<0x141>(v);   // mirror within 8
    v = min_dpp<0x140>(v);   // mirror within 16
    uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t m1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t m2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t m3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    m = m1 < m ? m1 : m;
    m = m2 < m ? m2 : m;
    return m3 < m ? m3 : m;
}

// Lowest lane whose predicate holds (-1 if none).
__device__ __forceinline__ int first_lane(bool p) {
    const unsigned long long b = __ballot(p);
    return b ? __builtin_ctzll(b) : -1;
}

// One token's lookup of n ids (rank order) in `layer`, by the 64 lanes of
// one wave (call with every lane of that wave, none of any other).  Lane s
// holds slot s's state, lane r the token's rank r; the walk over ranks is
// uniform, each decision a ballot or a wave minimum, so its order is the
// policy's.  ids may sit in LDS or global memory.  Writes the updated
// tables, the miss list (device memory, and the mapped host list when
// host_list), the trace and slots_out (if non-NULL, [n]).  Out-of-range ids
// are clamped (the caller flags them).
__device__ void lookup_wave(const SlotDev &c, int layer, const int32_t *ids, int n,
                            int32_t *slots_out, bool host_list, int lane) {
    const int S = c.S, E = c.E;
    int32_t *slot_of = c.slot_of + (size_t)layer * E;
    int16_t *expert_of = c.expert_of + (size_t)layer * S;
    uint32_t *count = c.count + (size_t)layer * S;
    uint32_t *last = c.last + (size_t)layer * S;
    const bool is_slot = lane < S, is_rank = lane < n;
    int my_ex = is_slot ? expert_of[lane] : 0;
    uint32_t my_cnt = is_slot ? count[lane] : 0u, my_lst = is_slot ? last[lane] : 0u;
    int my_id = 0;
    if (is_rank) {
        my_id = ids[lane];
        my_id = my_id < 0 ? 0 : my_id >= E ? E - 1 : my_id;
    }
    const int my_so = is_rank ? slot_of[my_id] : -1;
    const uint32_t t = c.tok[layer];
    bool my_pin = false;
    // hits first: they are pinned for this token (a repeated hit counts once)
    for (int r = 0; r < n; ++r) {
        const int s = __builtin_amdgcn_readlane(my_so, r);
        if (s >= 0 && lane == s) {
            if (!my_pin) { my_cnt += 1u; my_lst = t; }
            my_pin = true;
        }
    }
    int my_sr = my_so, nm = 0;
    int32_t *miss_g = c.miss_gpu + (size_t)layer * (1 + 2 * c.k);
    int32_t *miss_h = c.miss_dev + (size_t)layer * (1 + 2 * c.k);
    for (int r = 0; r < n; ++r) {
        if (__builtin_amdgcn_readlane(my_so, r) >= 0) continue;   // hit
        const int e = __builtin_amdgcn_readlane(my_id, r);
        const int q = first_lane(lane < r && my_id == e);          // repeated id, filled before
        if (q >= 0) {
            const int s = __builtin_amdgcn_readlane(my_sr, q);
            if (lane == r) my_sr = s;
            continue;
        }
        int v = first_lane(is_slot && my_ex < 0);
        if (v < 0) {
            const bool cand = is_slot && !my_pin;
            if (c.policy == TF_SLOT_LRU) {
                const uint32_t m = wave_min_u32(cand ? my_lst : 0xFFFFFFFFu);
                v = first_lane(cand && my_lst == m);
            } else {
                const uint32_t m = wave_min_u32(cand ? my_cnt : 0xFFFFFFFFu);
                const bool c2 = cand && my_cnt == m;
                const uint32_t m2 = wave_min_u32(c2 ? my_lst : 0xFFFFFFFFu);
                v = first_lane(c2 && my_lst == m2);
            }
            if (v < 0) continue;   // no unpinned slot: S >= n distinct ids rules this out
            const int old = __builtin_amdgcn_readlane(my_ex, v);
            if (lane == 0) slot_of[old] = -1;
        }
        if (lane == v) { my_ex = e; my_cnt = 1u; my_lst = t; my_pin = true; }
        if (lane == r) my_sr = v;
        if (lane == 0) {
            slot_of[e] = v;
            miss_g[1 + 2 * nm] = e;
            miss_g[2 + 2 * nm] = v;
            if (host_list) { miss_h[1 + 2 * nm] = e; miss_h[2 + 2 * nm] = v; }
        }
        ++nm;
    }
    if (is_slot) { expert_of[lane] = (int16_t)my_ex; count[lane] = my_cnt; last[lane] = my_lst; }
    if ((int64_t)t < c.trace_cap && is_rank) {
        c.trace_hit[((size_t)layer * c.trace_cap + t) * c.k + lane] = my_so >= 0 ? 1 : 0;
        c.trace_slot[((size_t)layer * c.trace_cap + t) * c.k + lane] = (int16_t)my_sr;
    }
    if (slots_out && is_rank) slots_out[lane] = my_sr;
    if (lane == 0) {
        miss_g[0] = nm;
        if (host_list) miss_h[0] = nm;
        c.tok[layer] = t + 1;
    }
    if (host_list) __threadfence_system();
}

// Part `part` of `per` workgroups (256 threads) copying miss r of the list
// (16 bytes per lane, four loads in flight per thread).  Ranks past the
// list's length have nothing to do; the first part of rank 0 counts the
// list's blobs.
__device__ __forceinline__ void copy_missed(const int32_t *miss, const uint8_t *host_layer,
                                            uint8_t *slot_layer, size_t stride, int E, int S,
                                            unsigned long long *nfill, int r, int part, int per,
                                            int tid) {
    const int nm = miss[0];
    if (r >= nm) return;
    const int ex = miss[1 + 2 * r], sl = miss[2 + 2 * r];
    if (ex < 0 || ex >= E || sl < 0 || sl >= S) return;   // the lookup writes neither
    if (r == 0 && part == 0 && tid == 0) atomicAdd(nfill, (unsigned long long)nm);
    const uint4 *src = reinterpret_cast<const uint4 *>(host_layer + (size_t)ex * stride);
    uint4 *dst = reinterpret_cast<uint4 *>(slot_layer + (size_t)sl * stride);
    const size_t n16 = stride / 16, step = (size_t)per * 256;
    for (size_t i = (size_t)part * 256 + tid; i < n16; i += 4 * step) {
        // four loads in flight, unconditional (clamped) and in named
        // registers: a conditionally filled array is kept in scratch memory
        const uint4 v0 = src[i], v1 = src[min(i + step, n16 - 1)];
        const uint4 v2 = src[min(i + 2 * step, n16 - 1)], v3 = src[min(i + 3 * step, n16 - 1)];
        dst[i] = v0;
        if (i + step < n16) dst[i + step] = v1;
        if (i + 2 * step < n16) dst[i + 2 * step] = v2;
        if (i + 3 * step < n16) dst[i + 3 * step] = v3;
    }
}

}  // namespace slotk
