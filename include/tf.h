/*
 * tf.h -- C ABI of the MI355X (gfx950) q4 MoE-layer hot path.
 *
 * One token of a Mixture-of-Experts decoder layer, as the TurboFieldfare
 * pages describe it (blog.hypho.cn review, "它省的不是模型大小": 128 routed
 * experts per layer, the router picks 8 per token, a dense shared expert
 * always runs; shilu.ai README translation, "概览" table: MLX affine 4-bit
 * weights with group 64 for the shared and routed experts, 8-bit router;
 * "推理引擎的工作原理": router first, then a 16-slot LFU expert cache per
 * layer whose misses are filled while the shared branch runs, then the shared
 * and routed outputs are combined; prefill in chunks of at most 128 tokens).
 *
 * Layer definition (per token t):
 *     l   = W_router x_t                      (8-bit affine, fp64 accumulate)
 *     ids = top-k of l by (logit desc, id asc), in rank order
 *     p   = softmax(l[ids])                   (over the k selected logits)
 *     y_t = shared(x_t) + sum_r p_r * expert_{ids_r}(x_t)
 *     expert(x) = W_down (gelu(W_gate x) (.) (W_up x)),  gelu(z) = z Phi(z)
 *
 * Conventions
 * -----------
 * - Pointers are DEVICE pointers unless the name ends in _host.  Every call
 *   is stream-ordered and asynchronous unless marked [SYNC].
 * - Quantised matrix W[n][k] (affine, group 64): q uint8 [n][k*bits/8]; for
 *   4 bits element j of a row is byte j/2, low nibble when j is even; scale
 *   and bias are IEEE fp16 [n][k/64] (passed as uint16_t); w = scale*q + bias.
 * - Expert blob: gate.q | gate.scale | gate.bias | up.q | up.scale | up.bias |
 *   down.q | down.scale | down.bias, back to back; gate/up are
 *   [d_ff][d_model], down is [d_model][d_ff].  3,345,408 bytes at
 *   d_model=2816, d_ff=704.  Blobs must start 256-byte aligned.
 * - x and y are fp16 (uint16_t) row-major [T][d_model]; y is rounded to
 *   nearest even from an fp32 accumulation (|y| >= 65520 becomes +-inf).
 * - Shapes: d_model, d_ff, d_ff_shared multiples of 64 and <= 4096;
 *   1 <= top_k <= 16; top_k <= n_experts <= 1024.
 * - Argument errors are detected before anything is enqueued and leave no
 *   side effects.  HIP failures return TF_E_HIP.  Asynchronous faults surface
 *   on a later call.  Nothing aborts; no C++ exception crosses the ABI.
 * - T = 0 returns TF_OK with no launches.
 * - Handles and workspaces are not thread-safe: one host thread and one
 *   stream sequence per workspace.  Calls never allocate device memory,
 *   except tf_slot_cache_create.
 * - Workspaces must be zero-filled before first use (tf_workspace_zero);
 *   the library leaves its counters at zero after every completed call.
 *   Counters sit at fixed offsets at the start of a workspace, apart from
 *   the data, so one workspace may serve calls of any token count and any
 *   layer whose workspace size it covers.
 */
#ifndef TF_H
#define TF_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TF_OK = 0,
    TF_E_ARG = 1,     /* NULL pointer, bad count or flag                          */
    TF_E_SHAPE = 2,   /* dimension not supported (see Conventions)                */
    TF_E_ALIGN = 3,   /* pointer misaligned (q rows 16 B, blobs 256 B, ws 256 B)  */
    TF_E_HIP = 4,     /* a HIP runtime call failed; see tf_last_error()           */
    TF_E_NOMEM = 5,   /* workspace too small / allocation failed                  */
    TF_E_STATE = 6    /* handle used out of order (e.g. fill before lookup)       */
} tf_status;

typedef enum { TF_GELU_ERF = 0, TF_GELU_TANH = 1 } tf_act;

/* Device-side error flags a call can record in its workspace (read with
 * tf_workspace_flags).  Kernels clamp the offending ids so that every memory
 * access stays in bounds; outputs of the affected token are unspecified. */
enum { TF_FLAG_ID_RANGE = 1, TF_FLAG_ID_REPEAT = 2 };

/* Thread-local text of the last non-OK return. */
const char *tf_last_error(void);
const char *tf_version(void);

/* Non-owning view of an affine-quantised W[n][k]. */
typedef struct {
    const uint8_t *q;
    const uint16_t *scale;
    const uint16_t *bias;
    int32_t n, k, bits, group;   /* bits 4 or 8, group 64, k % 64 == 0 */
} tf_qmat;

/* Size in bytes of one expert blob (host-only arithmetic): gate, up and down
 * as MLX affine 4-bit matrices with group 64 and one fp16 scale and bias per
 * group (shilu.ai README translation, "概览" table: 4-bit shared and routed
 * experts, group 64).  The blob is the unit the expert cache moves; at the
 * study's shapes 30 x 128 blobs plus the resident core come to about the
 * installed size the pages give (blog.hypho.cn review, "它省的不是模型大小":
 * 14.3 GB installed, 1.35 GB resident shared weights).  Returns 0 when
 * d_model or d_ff is not a positive multiple of 64. */
size_t tf_expert_blob_bytes(int32_t d_model, int32_t d_ff);

/* Split a blob into its three matrix views (host-only pointer arithmetic; the
 * same section layout as tf_expert_blob_bytes).  blob: any pointer, not
 * dereferenced; gate/up/down: caller-owned structs, filled.  TF_E_ARG on a
 * NULL argument, TF_E_SHAPE when d_model or d_ff is not a positive multiple
 * of 64. */
tf_status tf_expert_view(const uint8_t *blob, int32_t d_model, int32_t d_ff,
                         tf_qmat *gate, tf_qmat *up, tf_qmat *down);

/* Zero a workspace with a fill kernel (safe to record in a HIP graph). */
tf_status tf_workspace_zero(void *ws, size_t ws_bytes, hipStream_t s);

/* [SYNC] Read and clear the device-side error flags of a workspace. */
tf_status tf_workspace_flags(void *ws, int32_t *flags_host, hipStream_t s);

/* ---------------------------------------------------------------- router */
/* Router matvec (8-bit affine, products exact in fp32, sums in fp64), then
 * top-k by (logit desc, id asc) and softmax over the k selected logits.
 * The pages: an 8-bit router (shilu.ai README translation, "概览" table)
 * computed on the GPU from resident weights at every layer, whose top-8
 * expert ids the runtime then plans against the layer's expert cache
 * (same page, "推理引擎的工作原理"; blog.hypho.cn review,
 * "它省的不是模型大小": 128 routed experts, 8 chosen per token).  Softmax
 * scope (the k selected logits) and the tie rule (lower id first) are
 * readings; the pages do not state them.
 *   router     : 8-bit tf_qmat [n_experts][d_model]
 *   x          : fp16 [T][d_model]
 *   forced_ids : NULL, or int32 [T][top_k] ids to use instead of the top-k
 *                (p is then the softmax of the router logits at those ids,
 *                in the given order); ids must be distinct and in range --
 *                violations set TF_FLAG_ID_* in the workspace.
 *   ids        : int32 [T][top_k] out, rank order
 *   weights    : fp32 [T][top_k] out
 *   logits     : NULL or fp64 [T][n_experts] out
 *   ws         : workspace of tf_router_workspace_bytes(n_experts, T) bytes */
size_t tf_router_workspace_bytes(int32_t n_experts, int32_t T);
tf_status tf_router_topk(const tf_qmat *router, const uint16_t *x, int32_t T,
                         int32_t top_k, const int32_t *forced_ids, int32_t *ids,
                         float *weights, double *logits, void *ws, size_t ws_bytes,
                         hipStream_t s);

/* ------------------------------------------------------ expert q4 GEMV */
/* The routed expert's fused dequantise-and-multiply: gate and up GEMVs over
 * MLX affine 4-bit weights (group 64, per-group fp16 scale and bias), the
 * activation, then the down GEMV (sh.edu-sjtu.cn article, "三件事": 4-bit
 * experts with group-64 scaling; shilu.ai README translation, "状态和范围":
 * custom quantised-GEMV and MoE kernels).  For each pair p (0 <= p < P):
 *     y32[token[p]] += coef[p] * expert(pool + slot[p]*blob_stride)(x[token[p]])
 * token[] must be non-decreasing (pairs grouped by token); each token's pairs
 * are summed in pair order, so the result is deterministic.  token == NULL
 * means token[p] = p (then T must equal P); coef == NULL means 1.
 * y32 is fp32 [T][d_model], read and written.  P <= 256, T <= 256.
 * ws: tf_gemv_workspace_bytes(d_ff, P) bytes. */
size_t tf_gemv_workspace_bytes(int32_t d_ff, int32_t P);
tf_status tf_expert_q4_gemv(const uint8_t *pool, size_t blob_stride, int32_t d_model,
                            int32_t d_ff, const int32_t *slot, const int32_t *token,
                            const float *coef, int32_t P, const uint16_t *x, int32_t T,
                            float *y32, tf_act act, void *ws, size_t ws_bytes,
                            hipStream_t s);

/* ------------------------------------------------------------ MoE layer */
typedef struct tf_slot_cache tf_slot_cache;   /* opaque, see below */

typedef struct {
    tf_qmat router;              /* 8-bit [n_experts][d_model]               */
    const uint8_t *shared_blob;  /* shared expert, blob layout, d_ff_shared  */
    const uint8_t *pool;         /* n_experts blobs (all-resident) or the
                                    slot pool of a tf_slot_cache             */
    size_t blob_stride;          /* bytes between consecutive blobs          */
    int32_t d_model, d_ff, d_ff_shared, n_experts, top_k;
    int32_t act;                 /* tf_act                                   */
} tf_moe_layer;

/* Workspace for tf_moe_layer_fwd with up to T tokens. */
size_t tf_moe_workspace_bytes(const tf_moe_layer *L, int32_t T);

/* Decode step: T (1..16) independent tokens through one layer, in the order
 * the pages give for each layer (shilu.ai README translation,
 * "推理引擎的工作原理"): the router from resident weights, its top-8 planned
 * against the layer's 16-slot LFU cache, missed experts read in while the
 * resident shared-expert branch runs, then the shared and routed outputs
 * combined (blog.hypho.cn review, "它省的不是模型大小": 128 routed experts,
 * top-8, a dense shared expert).  The combine weights (router softmax, shared
 * branch at weight 1) are the study's layer definition, not the pages'.
 *   x [T][d_model] fp16 in; y [T][d_model] fp16 out; y32 NULL or fp32 out.
 *   ids/weights [T][top_k] out (rank order).
 *   forced_ids NULL or [T][top_k] (see tf_router_topk).
 *   cache NULL: blob of expert e is pool + e*blob_stride (all resident).
 *   cache non-NULL (T must be 1): the layer's routed experts are looked up in
 *     the slot cache; misses are copied from the pinned host pool on `copy`
 *     while the shared branch runs on `compute`.  [SYNC: waits once for the
 *     lookup result to issue the copies.]  With the cache's copy engine set
 *     to TF_SLOT_COPY_DEVICE the whole step runs on `compute` with no host
 *     wait (`copy` is not used): the router's top-k workgroup does the
 *     lookup, and the next launch copies the missed blobs (16 workgroups per
 *     rank of the miss list, over the host pool's device mapping) beside the
 *     shared gate/up.
 * Kernels: router+shared gate/up | (lookup) | routed gate/up + shared down |
 * routed down + combine. */
tf_status tf_moe_layer_fwd(const tf_moe_layer *L, const uint16_t *x, int32_t T,
                           const int32_t *forced_ids, uint16_t *y, float *y32,
                           int32_t *ids, float *weights, tf_slot_cache *cache,
                           int32_t layer, hipStream_t compute, hipStream_t copy,
                           void *ws, size_t ws_bytes);

/* Allocation-free decode step, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, kernels and
 * results as tf_moe_layer_fwd with all experts resident (no slot cache,
 * compute and copy streams both `stream`), but the workspace is the
 * library's own static device scratch of TF_NOALLOC_SCRATCH_BYTES per GPU,
 * held until the process ends.  The call allocates nothing.
 *   TF_E_NOMEM when tf_moe_workspace_bytes(L, T) exceeds the scratch (at
 *   d_model 2816, 128 experts, top-8, every T <= 16 fits; 3.9 MB at T = 16).
 * Every call on a GPU shares that GPU's scratch: calls that overlap on one
 * GPU (other streams, other host threads) race and give undefined results.
 * The scratch is zeroed on a device's first call, and again after a call
 * that returned TF_E_HIP.  The device-side id flags are not reported (no
 * workspace to read them from). */
#define TF_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
tf_status tf_moe_layer_fwd_noalloc(const tf_moe_layer *L, const uint16_t *x, int32_t T,
                                   const int32_t *forced_ids, uint16_t *y, float *y32,
                                   int32_t *ids, float *weights, hipStream_t stream);

/* Prefill: one chunk of T (1..128) tokens through one layer, all experts
 * resident (shilu.ai README translation, "推理引擎的工作原理": prompt prefill
 * in chunks of at most 128 tokens, so that one fetched expert serves several
 * rows).  Tokens are grouped by expert so that each expert's weights are
 * read once per chunk.  x [T][d_model] fp16; y [T][d_model] fp16 out; y32
 * NULL or fp32 [T][d_model] out; ids/weights [T][top_k] out, rank order.
 * ws: tf_prefill_workspace_bytes(L, T) bytes, 256-B aligned, zero-filled
 * before first use.  TF_E_ARG for T outside [0, 128] or a NULL pointer,
 * TF_E_ALIGN, TF_E_NOMEM for a short workspace, TF_E_SHAPE as in
 * tf_moe_layer_fwd; T == 0 enqueues nothing.  Same outputs as T single-token calls (ids bitwise,
 * y within fp32 rounding).  The chunks of one layer are independent: calls
 * on different streams, each with a workspace of its own, may run at once
 * (two chunks in flight overlap one chunk's short router and combine
 * launches with the other's GEMMs) and give bitwise the same results. */
size_t tf_prefill_workspace_bytes(const tf_moe_layer *L, int32_t T);
tf_status tf_moe_prefill_chunk(const tf_moe_layer *L, const uint16_t *x, int32_t T,
                               uint16_t *y, float *y32, int32_t *ids, float *weights,
                               hipStream_t s, void *ws, size_t ws_bytes);

/* Grouping of a chunk's (token, rank) pairs by expert, the step that lets
 * one fetched expert serve several rows of a prefill chunk (shilu.ai README
 * translation, "推理引擎的工作原理").  tf_moe_prefill_chunk and batched
 * tf_moe_layer_fwd run the same code after their top-k; this call runs it
 * alone on given ids.
 *   ids     [T][top_k] int32 device, in [0, n_experts) and distinct within a
 *           token (ids out of range are clamped; a repeated id leaves the
 *           outputs unspecified but in range).
 *   counts  [n_experts] int32 device out: pairs per expert.
 *   offsets [n_experts + 1] int32 device out: exclusive prefix sums of counts.
 *   pairs   [T * top_k] int32 device out: pair index t*top_k + r, sorted by
 *           (expert, t, r); expert e owns pairs[offsets[e] .. offsets[e+1]).
 * 1 <= top_k <= 16, top_k <= n_experts <= 1024, T <= 128 (TF_E_SHAPE);
 * T == 0 returns TF_OK with no launch.  One workgroup, stream-ordered.
 * ws: tf_group_workspace_bytes(n_experts, T, top_k) bytes, 256-B aligned. */
size_t tf_group_workspace_bytes(int32_t n_experts, int32_t T, int32_t top_k);
tf_status tf_group_by_expert(const int32_t *ids, int32_t T, int32_t top_k, int32_t n_experts,
                             int32_t *counts, int32_t *offsets, int32_t *pairs, void *ws,
                             size_t ws_bytes, hipStream_t s);

/* ------------------------------------------------------------ attention */
/* Decode attention of one new token (shilu.ai README translation, "状态和范围":
 * fp16 key/value storage, a bounded ring for the sliding-window layers and
 * linear storage for the full-attention layers, exact split-K/V decode
 * attention).  Per query head h, with key/value head g = h / (H / G):
 * scores s = scale * q_h . k over the tokens the layer sees, p = softmax(s),
 * out_h = sum p v.  The call first stores the new token's key and value:
 * ring != 0 keeps the last S tokens (token pos in slot pos % S; the layer
 * sees min(pos + 1, S) tokens); ring == 0 keeps token pos in slot pos
 * (pos < S; the layer sees pos + 1 tokens).
 *   q            [H][D] fp16 device (already normalised and rotated).
 *   k_new, v_new [G][D] fp16 device: the new token's key and value.
 *   k_cache, v_cache [G][S][D] fp16 device, caller-owned; slot pos (or
 *                pos % S) is written, the others only read.
 *   out          [H][D] fp32 device.
 *   ws           tf_attn_workspace_bytes(H, D, S) bytes, 256-B aligned.
 * D in {64, 128, 256}; H = G, 2G or 4G, H <= 1024; 1 <= S <= 2^20
 * (TF_E_SHAPE); pos >= 0, pos < S without the ring, scale > 0 (TF_E_ARG);
 * q, k/v and the caches 16-B aligned (TF_E_ALIGN).  Two launches,
 * stream-ordered: per (32-slot chunk, key/value head) the chunk's softmax
 * statistics and weighted values, then their exact merge per query head. */
size_t tf_attn_workspace_bytes(int32_t H, int32_t D, int32_t S);
tf_status tf_attn_decode(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                         uint16_t *k_cache, uint16_t *v_cache, int32_t H, int32_t G, int32_t D,
                         int32_t S, int32_t pos, int32_t ring, float scale, float *out, void *ws,
                         size_t ws_bytes, hipStream_t s);

/* ------------------------------------------------------------ sampling */
/* Next-token ids from rows of logits (shilu.ai README translation,
 * "向模型输入 prompt": the temperature, Top-K and Top-P knobs; temperature 0
 * gives greedy output).  Per row t:
 *   1. the top_k largest logits, ties to the lower id, NaN ranked as -inf;
 *   2. their softmax at `temperature`, in fp64, every sum taken
 *      sequentially in rank order;
 *   3. keep the shortest rank prefix whose cumulative probability is >= top_p;
 *   4. ids[t] = the first kept rank whose cumulative probability exceeds
 *      u[t] * (the kept cumulative probability).
 * temperature == 0: ids[t] = the largest logit's id (u may be NULL).
 *   logits [T][V] fp32 device, rows contiguous, 4-B aligned.
 *   u      [T] fp64 device, each in [0, 1) (the caller's random draws).
 *   ids    [T] int32 device out.
 *   ws     tf_sample_workspace_bytes(V, T, top_k) bytes, 256-B aligned: 64
 *          keys per 4096-logit slice of every row (512 * T * ceil(V / 4096)
 *          bytes).  Calls that share a workspace must not overlap.
 * 1 <= top_k <= 64, top_k <= V <= 262144 (TF_E_SHAPE); 0 <= T <= 4096,
 * temperature >= 0, 0 < top_p <= 1 (TF_E_ARG).  T == 0 returns TF_OK with no
 * launch.  Two launches, stream-ordered. */
size_t tf_sample_workspace_bytes(int32_t V, int32_t T, int32_t top_k);
tf_status tf_sample(const float *logits, int32_t V, int32_t T, float temperature, int32_t top_k,
                    float top_p, const double *u, int32_t *ids, void *ws, size_t ws_bytes,
                    hipStream_t s);

/* ------------------------------------------------------------ profiling */
/* Kernel ids of the hot path (for tf_profile_kernel). */
enum {
    TF_KERNEL_ROUTER_SHARED_GATEUP = 1,      /* decode A: router + top-k + shared gate/up;
                                                decode steps of 2-16 tokens and the router
                                                alone: router rows + top-k (+ grouping);
                                                prefill chunks: the router GEMM           */
    TF_KERNEL_ROUTED_GATEUP_SHARED_DOWN = 2, /* decode B: routed gate/up + shared down    */
    TF_KERNEL_DOWN_COMBINE = 4,              /* decode C: routed down + combine -> y      */
    TF_KERNEL_PREFILL_DOWN = 8,              /* prefill: shared and per-item down (MFMA)  */
    TF_KERNEL_PREFILL_COMBINE = 16,          /* prefill: y_s + sum of y_e -> y            */
    TF_KERNEL_PREFILL_GATEUP = 32,           /* prefill: shared and per-item gate/up (MFMA) */
    TF_KERNEL_GROUP = 64,                    /* tf_group_by_expert                        */
    TF_KERNEL_SAMPLE_PART = 128,             /* tf_sample: per-slice 64 largest keys      */
    TF_KERNEL_SAMPLE_FINAL = 256,            /* tf_sample: row merge, softmax, draw       */
    TF_KERNEL_ATTN_CHUNK = 512,              /* tf_attn_decode: per-chunk partials        */
    TF_KERNEL_ATTN_COMBINE = 1024,           /* tf_attn_decode: merge per query head      */
    TF_KERNEL_ROUTER_TOPK = 2048             /* grouped steps: per-token top-k + grouping  */
};
/* Arm a one-shot timer: the next launch, by this host thread, of the named
 * kernel goes through hipExtLaunchKernel with `start` recorded when the
 * kernel begins and `stop` when it ends, on the stream it runs on.  Events
 * must be created with timing enabled; hipEventElapsedTime(start, stop) is
 * then the kernel's own duration.  Create them with hipEventDisableSystemFence:
 * a default event's system-scope cache write-back and invalidate slows the
 * timed kernel (measured: 10.3 against 8.5 us for the routed decode kernel).
 * Pass kernel 0 to disarm. */
tf_status tf_profile_kernel(int32_t kernel, hipEvent_t start, hipEvent_t stop);
/* Read `bytes` (a multiple of 16; p 16-byte aligned, device memory) once with
 * the GEMVs' load pattern -- 16 bytes per lane, each wave's load covering
 * whole 128-byte lines -- and write nothing: the kernel of known traffic
 * against which memory counters of the GEMV kernels are scaled.  The
 * kernel's name contains "k_stream_read".  TF_E_ARG on a bad pointer or
 * size. */
tf_status tf_profile_stream_read(const void *p, size_t bytes, hipStream_t s);

/* ------------------------------------------------------------ slot cache */
/* Per-layer LFU expert cache in HBM (shilu.ai README translation,
 * "推理引擎的工作原理"; sh.edu-sjtu.cn, "三件事").  Policy: a slot's count is
 * 1 on fill and +1 per hit; the token's own ids are pinned; misses are
 * handled in rank order; the victim is the lowest empty slot, else the
 * unpinned slot with the smallest (count, last-use token, slot index); every
 * layer starts empty.
 *   slot_pool        : device [n_layers][n_slots][blob_stride] bytes (caller-owned)
 *   host_pool_pinned : pinned host [n_layers][n_experts][blob_stride] bytes
 *                      (caller-owned, hipHostMalloc)
 *   trace_cap        : tokens per layer recorded in the hit/slot trace (0 = off)
 * The handle owns only its small device tables, a mapped pinned miss list,
 * the trace and two events. */
tf_status tf_slot_cache_create(int32_t n_layers, int32_t n_experts, int32_t n_slots,
                               int32_t top_k, size_t blob_stride, uint8_t *slot_pool,
                               const uint8_t *host_pool_pinned, int64_t trace_cap,
                               tf_slot_cache **out);
void tf_slot_cache_destroy(tf_slot_cache *c);
/* Look up one token's ids (device int32 [n]) in `layer`'s cache: updates
 * the LFU state, writes slots (device int32 [n]) and the miss list, records
 * the lookup event.  Asynchronous. */
tf_status tf_slot_cache_lookup(tf_slot_cache *c, int32_t layer, const int32_t *ids,
                               int32_t n, int32_t *slots, hipStream_t compute);
/* [SYNC] Wait for the last lookup of `layer`, copy each missed blob from the
 * host pool (or a prefetch buffer) into its slot on `copy` (see the copy
 * engine below), then record `filled` (may be NULL) on `copy`.
 * *n_miss_host receives the count.  With TF_SLOT_COPY_DEVICE the call does
 * not wait: `copy` waits for the lookup on the GPU, one kernel reads the
 * miss list from device memory and moves the blobs, and *n_miss_host
 * receives -1 (the count stays on the GPU; tf_slot_cache_trace has it). */
tf_status tf_slot_cache_fill(tf_slot_cache *c, int32_t layer, hipStream_t copy,
                             hipEvent_t filled, int32_t *n_miss_host);
/* [SYNC] Copy `layer`'s trace (hit flag, slot per token and rank) to the host.
 * hit_host / slot_host hold cap entries; *len receives the entries written. */
tf_status tf_slot_cache_trace(tf_slot_cache *c, int32_t layer, int8_t *hit_host,
                              int16_t *slot_host, int64_t cap, int64_t *len);
/* [SYNC] Empty every layer and clear the traces. */
tf_status tf_slot_cache_reset(tf_slot_cache *c);
/* Total bytes copied host->device by fills since create/reset (misses served
 * from a prefetch buffer are device copies and do not count).  [SYNC once a
 * TF_SLOT_COPY_DEVICE fill has run: those fills count on the GPU.]  -1 on a
 * NULL cache or a failed read. */
int64_t tf_slot_cache_bytes_filled(const tf_slot_cache *c);

/* Speculative fill (shengyayun.com AI newsletter of 2026-07-30, "事件与背景"
 * item 一: read-ahead with parallel reads and a small expert cache hide the
 * SSD latency; here host-to-device copies of predicted experts run ahead of
 * the layer's lookup).
 * set_prefetch: give the cache n_buffers (0..16; 0 turns prefetch off)
 * expert-sized device buffers per layer, [n_layers][n_buffers][blob_stride]
 * bytes, 256-B aligned, caller-owned.  Synchronises the device.
 * prefetch: for each predicted id (host int32 [n], each in [0, n_experts))
 * that is neither resident in `layer` (as the fills so far left it) nor
 * already in a buffer, copy its blob from the host pool into a free buffer
 * on `copy` (ids past the last free buffer are dropped; one launch for all
 * of them, or one hipMemcpyAsync each, see the copy engine below).
 * *n_issued (may be NULL) receives the number of copies.  The layer's next
 * fill takes each miss found in a buffer as a device copy from it (after the
 * prefetch copies, whatever stream they ran on) and frees every buffer of
 * the layer; predictions never change the cache's hit/miss sequence.
 * TF_E_STATE without buffers or between a lookup and its fill.
 * prefetch_stats: host->device bytes of prefetch copies, buffers used by a
 * fill, buffers freed unused (any pointer may be NULL). */
tf_status tf_slot_cache_set_prefetch(tf_slot_cache *c, uint8_t *buffers, int32_t n_buffers);
tf_status tf_slot_cache_prefetch(tf_slot_cache *c, int32_t layer, const int32_t *ids_host,
                                 int32_t n, hipStream_t copy, int32_t *n_issued);
tf_status tf_slot_cache_prefetch_stats(const tf_slot_cache *c, int64_t *h2d_bytes, int64_t *used,
                                       int64_t *wasted);

/* How fills and prefetches move blobs on the copy stream.
 * TF_SLOT_COPY_KERNEL (the default when hipHostGetDevicePointer maps the
 * host pool): one kernel launch per fill or prefetch reads every blob of the
 * call over PCIe through the mapping (16 workgroups per blob).
 * TF_SLOT_COPY_DMA (the default otherwise): one hipMemcpyAsync per blob.
 * TF_SLOT_COPY_DEVICE: the fill is planned on the GPU too, with no host
 * round trip.  tf_slot_cache_fill: the copy stream waits for the lookup, and
 * one kernel of k x 16 workgroups reads the layer's miss list from device
 * memory and copies the missed blobs over the mapping; the next lookup of
 * the layer waits on the GPU for that fill.  tf_moe_layer_fwd: the lookup
 * and the copies join the step's own launches (see there).  No prefetch
 * with it (it keeps no host view of the slots).
 * Device copies out of prefetch buffers always run as a kernel.  TF_E_STATE
 * asks for a kernel engine on an unmapped pool, for the device engine with
 * prefetch buffers set, or for any change between a lookup and its fill;
 * TF_E_ARG for an unknown engine. */
typedef enum {
    TF_SLOT_COPY_DMA = 0, TF_SLOT_COPY_KERNEL = 1, TF_SLOT_COPY_DEVICE = 2
} tf_slot_copy_engine;
tf_status tf_slot_cache_set_copy_engine(tf_slot_cache *c, int32_t engine);

/* Eviction rule of later lookups (every layer).  TF_SLOT_LFU (the default,
 * the pages' word): victim = unpinned slot with the smallest (count,
 * last-use token, slot index).  TF_SLOT_LRU (the sh.edu-sjtu.cn article's
 * gloss of the same cache, "三件事": the longest-unused slot goes): victim =
 * unpinned slot with the smallest (last-use token, slot index).  Hits, pins
 * and empty slots work the same in both.  Meant to be set right after create
 * or reset; TF_E_ARG for an unknown policy. */
typedef enum { TF_SLOT_LFU = 0, TF_SLOT_LRU = 1 } tf_slot_policy;
tf_status tf_slot_cache_set_policy(tf_slot_cache *c, int32_t policy);

#ifdef __cplusplus
}
#endif
#endif /* TF_H */
