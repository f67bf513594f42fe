// Internal interface between the C ABI (tf_api.cpp) and the kernel files.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tf.h"
#include "tf_slot_dev.h"

// Workspace header words (uint32): device-side flags, the number of expert
// work items of the current step, then one ticket per token and one for the
// whole step (counters that return to zero at the end of every step).  Each
// ticket has a 128-byte line of its own: the router workgroups of all tokens
// take theirs at the same time, and atomics on one line serialise.
enum { HDR_FLAGS = 0, HDR_NITEMS = 1 };
__host__ __device__ constexpr int hdr_ticket(int i) { return 32 + 32 * i; }
// Header bytes of a step of T tokens.
__host__ __device__ constexpr size_t hdr_bytes(int T) { return (size_t)4 * hdr_ticket(T + 1); }
enum { STAGE_A = 1, STAGE_B = 2, STAGE_C = 4 };
constexpr int KC_BATCH = 8;       // pairs staged per pass in the down/combine kernel
constexpr int ROUTER_ROWS = 2;    // router rows per workgroup (two waves per row)
constexpr int RMM_CHUNKS = 6;     // 16-column chunks per wave of the matrix-core router, at most
constexpr int RMM_MAX_KR = (4096 / 16 + 4 * RMM_CHUNKS - 1) / (4 * RMM_CHUNKS);   // its K ranges at d = 4096
// Router workgroups of a step of T tokens over E experts.
__host__ __device__ constexpr int router_blocks(int E, int T) { return ((E + ROUTER_ROWS - 1) / ROUTER_ROWS) * T; }

// Bytes of one hidden row of K values in the global hi/lo layout.
__host__ __device__ constexpr size_t h_row_bytes(int K) { return (size_t)160 * (K >> 5); }
constexpr int MAX_DECODE_T = 16;  // tokens per decode step
constexpr int MAX_PREFILL_T = 128;  // tokens per prefill chunk
constexpr int MAX_TB = 4;         // tokens staged per pass of a gate/up block
constexpr int SLOT_COPY_WGS_PER_BLOB = 16;   // miss copies over PCIe inside a decode step
constexpr int ITEM_INTS = 16;     // ints per expert item record (see group_block)

struct DecodeArgs {
    int d, f, fs, E, k, T, act;
    const uint16_t *x;
    const uint8_t *rq;
    const uint16_t *rs, *rb;
    const uint8_t *shared_blob;
    const uint8_t *pool;
    size_t stride;
    const int32_t *slot_map;     // expert -> slot (NULL: slot = expert)
    const int32_t *forced;       // NULL or [T][k]
    int32_t *ids;
    float *weights;
    double *logits;
    double *part;                // grouped steps: partial logits [nkr][T][E] (NULL otherwise)
    int nkr;                     // their number of K ranges
    uint16_t *y;
    float *y32;
    uint32_t *hdr;
    int32_t *items;              // [items][ITEM_INTS] expert item records
    int32_t *pairs;              // [T*k] pair index t*k+r sorted by (expert, t, r)
    int32_t *g_counts, *g_offsets;  // grouping outputs [E], [E+1] (NULL in layer calls)
    uint4 *xb;                   // grouped steps: x rows in B-operand form (NULL otherwise)
    uint32_t *ctk;               // decode down launch: one ticket per (token, 32-row tile),
                                 // 32 words apart (zero between launches)
    // hidden activations as hi/lo fp16 pair rows (10*K/32 uint4 per row, see
    // tf_decode.hip): shared [T][fs], routed [T*k][f] (or [P][f])
    uint4 *h_s;
    float *y_s;                  // [T][d]
    uint4 *h_r;
    float *y_e;                  // prefill: [T*k][d] p-weighted expert outputs per pair
    // grid partition (256-thread workgroups): stage A = router blocks (four
    // router rows each, per token) then shared gate/up blocks (16 rows, per
    // token sub-batch); stage B = routed gate/up blocks (16 rows of one expert
    // item) then shared down blocks (32 rows, per token sub-batch)
    int a_router_blocks, a_shared_blocks, b_routed_blocks, b_shared_blocks;
    int tbx;                     // tokens per shared gate/up block (<= MAX_TB)
    int tbi;                     // tokens per routed expert item (grouped steps)
    int max_items;               // grouped steps: bound of the step's expert items
    int topk, do_group;
    // standalone GEMV mode (gemv_slot != NULL): pairs instead of routed items
    const int32_t *gemv_slot, *gemv_token;
    const float *gemv_coef;
    int P;
    // slot-cache step planned on the GPU (sc.slot_of != NULL, one token): the
    // router's top-k workgroup also looks the ids up in layer sc_layer of the
    // cache; stage A's first a_copy_blocks workgroups (copy_per per rank of
    // the miss list) copy the missed blobs from sc_host into sc_slots
    SlotDev sc;
    int sc_layer, a_copy_blocks, copy_per;
    const uint8_t *sc_host;
    uint8_t *sc_slots;
};

hipError_t tf_launch_decode(const DecodeArgs &a, int which, hipStream_t s);
// Grouping alone (one workgroup): pairs, item records, counts and offsets.
hipError_t tf_launch_group(const DecodeArgs &a, hipStream_t s);
// Router of a grouped step (T >= 2) on the matrix cores: partial fp64 logits
// over nkr K ranges, then one workgroup per token (top-k, softmax, x in
// B-operand form for decode steps) and the grouping by the last of them.
hipError_t tf_launch_router_grouped(const DecodeArgs &a, hipStream_t s);
// K ranges of the grouped router for d_model d.
int tf_router_nkr(int d);
// Prefill combine: y = y_s + sum over ranks of y_e -> fp16.
hipError_t tf_launch_prefill_combine(const DecodeArgs &a, hipStream_t s);
// Grouped steps (prefill, decode of more than one token) on the matrix cores
// after the router launch (items of at most 16 tokens): gate/up, down and
// the combine.
hipError_t tf_launch_grouped(const DecodeArgs &a, int max_items, hipStream_t s);
// The same for prefill chunks of more than 16 tokens: one workgroup per tile
// of an item of at most 16 tokens (x in B-operand form from the router launch).
hipError_t tf_launch_prefill_tiles(const DecodeArgs &a, int max_items, hipStream_t s);
// Lanes per weight row used by stages A and B for these shapes (8 or 16).
int tf_decode_lpr(const DecodeArgs &a);

// One-shot kernel timer (tf_profile_kernel): take_profile(kernel, &start, &stop)
// returns true once for the armed kernel id and disarms it.
void tf_arm_profile(int kernel, hipEvent_t start, hipEvent_t stop);
bool tf_take_profile(int kernel, hipEvent_t *start, hipEvent_t *stop);

// Launch through hipExtLaunchKernelGGL with the armed events when `kernel` is
// armed, plain hipLaunchKernelGGL otherwise.
#define TF_LAUNCH(kernel_id, fn, grid, block, lds, stream, ...)                            \
    do {                                                                                   \
        hipEvent_t ev0_, ev1_;                                                             \
        if (tf_take_profile(kernel_id, &ev0_, &ev1_))                                      \
            hipExtLaunchKernelGGL(fn, grid, block, lds, stream, ev0_, ev1_, 0, __VA_ARGS__); \
        else                                                                               \
            hipLaunchKernelGGL(fn, grid, block, lds, stream, __VA_ARGS__);                 \
    } while (0)
hipError_t tf_launch_zero(void *p, size_t bytes, hipStream_t s);
hipError_t tf_launch_stream_read(const void *p, size_t bytes, hipStream_t s);
