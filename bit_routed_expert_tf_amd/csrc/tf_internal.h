// Internal interface between the C ABI (tf_api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tf.h"

// Workspace header words (uint32): device-side flags, the number of expert
// work items of the current step, then one ticket per token and one for the
// whole step (counters that return to zero at the end of every step).
enum { HDR_FLAGS = 0, HDR_NITEMS = 1, HDR_TICKET = 2 };
enum { STAGE_A = 1, STAGE_B = 2, STAGE_C = 4 };
constexpr int KC_BATCH = 8;       // pairs staged per pass in the down/combine kernel
constexpr int MAX_DECODE_T = 16;  // tokens per decode step
constexpr int MAX_TB = 4;         // tokens per expert work item

struct DecodeArgs {
    int d, f, fs, E, k, T, act;
    const uint16_t *x;
    const uint8_t *rq;
    const uint16_t *rs, *rb;
    const uint8_t *shared_blob;
    const uint8_t *pool;
    size_t stride;
    const int16_t *slot_map;     // expert -> slot (NULL: slot = expert)
    const int32_t *forced;       // NULL or [T][k]
    int32_t *ids;
    float *weights;
    double *logits;
    uint16_t *y;
    float *y32;
    uint32_t *hdr;
    int32_t *items;              // [T*k][4] = expert, begin, count, 0
    int32_t *pairs;              // [T*k] pair index t*k+r sorted by (expert, t, r)
    float *h_s;                  // [T][fs]
    float *y_s;                  // [T][d]
    float *h_r;                  // [T*k][f] (or [P][f])
    int a_router_waves, a_shared_waves, b_routed_waves, b_shared_waves;
    int tbx, tbh, kcb;           // tokens per x-staged item, per h-staged item, pairs per C pass
    int topk, do_group;
    // standalone GEMV mode (gemv_slot != NULL): pairs instead of routed items
    const int32_t *gemv_slot, *gemv_token;
    const float *gemv_coef;
    int P;
};

hipError_t tf_launch_decode(const DecodeArgs &a, int which, hipStream_t s);
hipError_t tf_launch_zero(void *p, size_t bytes, hipStream_t s);
