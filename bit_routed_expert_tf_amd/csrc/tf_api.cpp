// C ABI of the q4 MoE-layer hot path (declared in include/tf.h).
//
// This file validates arguments, lays out workspaces and enqueues the
// kernels; it never allocates device memory on the hot path and never
// throws across the ABI.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "tf_internal.h"
#include "tf_layer.h"
#include "tf_slot.h"

namespace {

thread_local std::string g_err;

tf_status fail(tf_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

tf_status hip_fail(hipError_t e, const char *what) {
    return fail(TF_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

inline size_t up256(size_t n) { return (n + 255) & ~size_t(255); }
inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool dim_ok(int32_t v) { return v >= 64 && v <= 4096 && v % 64 == 0; }

tf_status check_qmat(const tf_qmat *m, int bits, int n, int k, const char *what) {
    if (!m || !m->q || !m->scale || !m->bias) return fail(TF_E_ARG, "%s: NULL matrix", what);
    if (m->bits != bits || m->group != 64) return fail(TF_E_SHAPE, "%s: need %d-bit, group 64", what, bits);
    if (m->n != n || m->k != k) return fail(TF_E_SHAPE, "%s: shape [%d][%d], want [%d][%d]", what, m->n, m->k, n, k);
    if (!aligned(m->q, 16)) return fail(TF_E_ALIGN, "%s: q not 16-byte aligned", what);
    if (!aligned(m->scale, 2) || !aligned(m->bias, 2)) return fail(TF_E_ALIGN, "%s: scale/bias misaligned", what);
    return TF_OK;
}

tf_status check_layer(const tf_moe_layer *L) {
    if (!L) return fail(TF_E_ARG, "layer is NULL");
    if (!dim_ok(L->d_model) || !dim_ok(L->d_ff) || !dim_ok(L->d_ff_shared))
        return fail(TF_E_SHAPE, "d_model/d_ff/d_ff_shared must be multiples of 64 in [64, 4096]");
    if (L->top_k < 1 || L->top_k > 16) return fail(TF_E_SHAPE, "top_k must be in [1, 16]");
    if (L->n_experts < L->top_k || L->n_experts > 1024)
        return fail(TF_E_SHAPE, "n_experts must be in [top_k, 1024]");
    if (L->act != TF_GELU_ERF && L->act != TF_GELU_TANH) return fail(TF_E_ARG, "unknown activation");
    tf_status st = check_qmat(&L->router, 8, L->n_experts, L->d_model, "router");
    if (st) return st;
    if (!L->shared_blob || !L->pool) return fail(TF_E_ARG, "shared_blob/pool is NULL");
    if (!aligned(L->shared_blob, 256) || !aligned(L->pool, 256))
        return fail(TF_E_ALIGN, "blobs must be 256-byte aligned");
    if (L->blob_stride < tf_expert_blob_bytes(L->d_model, L->d_ff) || L->blob_stride % 256)
        return fail(TF_E_ALIGN, "blob_stride must be >= the blob size and a multiple of 256");
    return TF_OK;
}

// Counters (flags, tickets) sit at the start of every workspace, at offsets
// that depend on nothing but the entry point: sized for the most tokens a
// call takes and, for the decode down launch's tickets, the widest d_model.
// Data regions never overlap them, so a workspace stays valid when it is
// reused for another token count or another layer shape (every completed
// call leaves its counters at zero).
constexpr size_t kHdrBytes = (hdr_bytes(MAX_PREFILL_T) + 255) & ~size_t(255);
constexpr size_t kCtkBytes = (size_t)128 * (4096 / 32);   // one token's down tiles

// Decode workspace layout (offsets in bytes).
struct WsLayout {
    size_t hdr, logits, part, items, pairs, hs, ys, hr, xb, ye, ctk, total;
};

WsLayout decode_layout(int d, int f, int fs, int E, int k, int T) {
    WsLayout w{};
    size_t o = 0;
    w.hdr = o; o += kHdrBytes;
    w.ctk = o; o += kCtkBytes;             // decode down tile tickets (one token)
    w.logits = o; o += up256((size_t)8 * T * E);
    w.part = o; o += T > MAX_DECODE_T ? up256((size_t)8 * tf_router_nkr(d) * T * E) : 0;   // prefill chunks
    w.items = o; o += up256((size_t)4 * ITEM_INTS * T * k);
    w.pairs = o; o += up256((size_t)4 * T * k);
    w.hs = o; o += up256(h_row_bytes(fs) * T);
    w.ys = o; o += up256((size_t)4 * T * d);
    w.hr = o; o += up256(h_row_bytes(f) * T * k);
    w.xb = o; o += up256((size_t)16 * tfk::xb_row_u4(d) * T);
    w.ye = o; o += up256((size_t)4 * T * k * d);           // decode: per-pair down rows
    w.total = o;
    return w;
}

template <typename T> T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

void fill_common(DecodeArgs &a, const tf_moe_layer *L, int T) {
    memset(&a, 0, sizeof a);
    a.d = L->d_model; a.f = L->d_ff; a.fs = L->d_ff_shared;
    a.E = L->n_experts; a.k = L->top_k; a.T = T; a.act = L->act;
    a.rq = L->router.q; a.rs = L->router.scale; a.rb = L->router.bias;
    a.shared_blob = L->shared_blob; a.pool = L->pool; a.stride = L->blob_stride;
    a.tbx = T < MAX_TB ? T : MAX_TB;
    a.tbi = MAX_TB;   // decode: items of up to MAX_TB tokens, one pass each
    a.topk = 1;
}

// Workspace of a grouped step (prefill, decode of T >= 2): the decode layout
// plus the per-pair down outputs y_e fp32 [T*k][d].
size_t grouped_ws_bytes(const tf_moe_layer *L, int T) {
    const WsLayout w = decode_layout(L->d_model, L->d_ff, L->d_ff_shared, L->n_experts, L->top_k, T);
    return w.total + up256((size_t)4 * T * L->top_k * L->d_model);
}

// Grouped step of T >= 2 tokens, all experts resident (shilu.ai README
// translation, "推理引擎的工作原理": a chunk's tokens share each fetched
// expert).  Arguments are checked by the caller.
//   A  router rows + top-k per token, grouping into items of <= 4 tokens
//   B  gate/up on the matrix cores: shared expert per 4 tokens, routed
//      expert per item -> h_s, h_r
//   C  down on the matrix cores -> y_s, y_e per pair
//   D  y = y_s + sum over ranks of y_e, fp16
hipError_t grouped_step(const tf_moe_layer *L, const uint16_t *x, int T, const int32_t *forced,
                        uint16_t *y, float *y32, int32_t *ids, float *weights, void *ws,
                        hipStream_t s) {
    const WsLayout w = decode_layout(L->d_model, L->d_ff, L->d_ff_shared, L->n_experts, L->top_k, T);
    DecodeArgs a;
    fill_common(a, L, T);
    a.x = x; a.forced = forced; a.ids = ids; a.weights = weights; a.y = y; a.y32 = y32;
    a.hdr = at<uint32_t>(ws, w.hdr);
    a.logits = at<double>(ws, w.logits);
    a.items = at<int32_t>(ws, w.items);
    a.pairs = at<int32_t>(ws, w.pairs);
    a.h_s = at<uint4>(ws, w.hs);
    a.y_s = at<float>(ws, w.ys);
    a.h_r = at<uint4>(ws, w.hr);
    a.y_e = at<float>(ws, w.total);
    a.do_group = 1;
    // decode steps (T <= 16): persistent units of up to four tokens; prefill
    // chunks: tiles of up to 16 tokens; both read x in B-operand form, staged
    // by the router launch
    const bool tiles = T > MAX_DECODE_T;
    a.xb = at<uint4>(ws, w.xb);
    a.tbi = tiles ? 16 : 4;
    const int P = T * a.k;
    const int max_items = P < a.E + P / a.tbi ? P : a.E + P / a.tbi;
    a.max_items = max_items;
    hipError_t e;
    if (tiles) {
        // prefill chunks: the router on the matrix cores (two launches; at 128
        // tokens 21 against 39 us for the fused router launch)
        a.part = at<double>(ws, w.part);
        a.nkr = tf_router_nkr(a.d);
        e = tf_launch_router_grouped(a, s);
    } else {
        // decode steps: one fused launch of router rows, top-k and grouping
        // (at 16 tokens 10.7 against 16.1 us for the two-launch router)
        a.a_router_blocks = router_blocks(a.E, T);
        e = tf_launch_decode(a, STAGE_A, s);
    }
    if (e == hipSuccess)
        e = tiles ? tf_launch_prefill_tiles(a, max_items, s) : tf_launch_grouped(a, max_items, s);
    return e;
}

}  // namespace

void tf_set_error(const char *msg) { g_err = msg; }

extern "C" {

const char *tf_last_error(void) { return g_err.c_str(); }
const char *tf_version(void) { return "tf-moe-mi355x 0.1 (gfx950)"; }

size_t tf_expert_blob_bytes(int32_t d_model, int32_t d_ff) {
    if (d_model <= 0 || d_ff <= 0 || d_model % 64 || d_ff % 64) return 0;
    const size_t mq = (size_t)d_model * d_ff / 2, ms = (size_t)d_model * d_ff / 64 * 2;
    return 3 * (mq + 2 * ms);
}

tf_status tf_expert_view(const uint8_t *blob, int32_t d_model, int32_t d_ff, tf_qmat *gate,
                         tf_qmat *up, tf_qmat *down) {
    if (!blob || !gate || !up || !down) return fail(TF_E_ARG, "NULL argument");
    if (d_model <= 0 || d_ff <= 0 || d_model % 64 || d_ff % 64)
        return fail(TF_E_SHAPE, "d_model and d_ff must be positive multiples of 64");
    const size_t mq = (size_t)d_model * d_ff / 2, ms = (size_t)d_model * d_ff / 64 * 2;
    const uint8_t *p = blob;
    tf_qmat *m[3] = {gate, up, down};
    for (int i = 0; i < 3; ++i) {
        m[i]->q = p; p += mq;
        m[i]->scale = reinterpret_cast<const uint16_t *>(p); p += ms;
        m[i]->bias = reinterpret_cast<const uint16_t *>(p); p += ms;
        m[i]->n = i < 2 ? d_ff : d_model;
        m[i]->k = i < 2 ? d_model : d_ff;
        m[i]->bits = 4;
        m[i]->group = 64;
    }
    return TF_OK;
}

tf_status tf_workspace_zero(void *ws, size_t ws_bytes, hipStream_t s) {
    if (!ws || ws_bytes % 4) return fail(TF_E_ARG, "workspace NULL or size not a multiple of 4");
    hipError_t e = tf_launch_zero(ws, ws_bytes, s);
    return e == hipSuccess ? TF_OK : hip_fail(e, "zero kernel");
}

tf_status tf_workspace_flags(void *ws, int32_t *flags_host, hipStream_t s) {
    if (!ws || !flags_host) return fail(TF_E_ARG, "NULL argument");
    uint32_t v = 0;
    hipError_t e = hipMemcpyAsync(&v, ws, 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "reading workspace flags");
    *flags_host = (int32_t)v;
    e = tf_launch_zero(ws, 4, s);
    return e == hipSuccess ? TF_OK : hip_fail(e, "clearing workspace flags");
}

// The router's counters: sized for the largest T it takes (see kHdrBytes).
static size_t router_hdr_bytes(int32_t) { return up256(hdr_bytes(4096)); }

size_t tf_router_workspace_bytes(int32_t n_experts, int32_t T) {
    if (n_experts <= 0 || T <= 0) return 256;
    return router_hdr_bytes(T) + up256((size_t)8 * T * n_experts);
}

tf_status tf_router_topk(const tf_qmat *router, const uint16_t *x, int32_t T, int32_t top_k,
                         const int32_t *forced_ids, int32_t *ids, float *weights, double *logits,
                         void *ws, size_t ws_bytes, hipStream_t s) {
    if (T < 0 || T > 4096) return fail(TF_E_ARG, "T must be in [0, 4096]");
    if (T == 0) return TF_OK;
    if (!router) return fail(TF_E_ARG, "router is NULL");
    const int E = router->n, d = router->k;
    if (!dim_ok(d)) return fail(TF_E_SHAPE, "d_model must be a multiple of 64 in [64, 4096]");
    if (top_k < 1 || top_k > 16 || E < top_k || E > 1024)
        return fail(TF_E_SHAPE, "need 1 <= top_k <= 16 and top_k <= n_experts <= 1024");
    tf_status st = check_qmat(router, 8, E, d, "router");
    if (st) return st;
    if (!x || !ids || !weights || !ws) return fail(TF_E_ARG, "NULL x/ids/weights/ws");
    if (!aligned(x, 16) || !aligned(ws, 256)) return fail(TF_E_ALIGN, "x 16-byte / ws 256-byte alignment");
    if (ws_bytes < tf_router_workspace_bytes(E, T)) return fail(TF_E_NOMEM, "workspace too small");
    DecodeArgs a;
    memset(&a, 0, sizeof a);
    a.d = d; a.E = E; a.k = top_k; a.T = T;
    a.x = x; a.rq = router->q; a.rs = router->scale; a.rb = router->bias;
    a.forced = forced_ids; a.ids = ids; a.weights = weights;
    a.hdr = at<uint32_t>(ws, 0);
    a.logits = logits ? logits : at<double>(ws, router_hdr_bytes(T));
    a.a_router_blocks = router_blocks(E, T);
    a.topk = 1;
    a.do_group = 0;
    a.f = a.fs = 64;
    hipError_t e = tf_launch_decode(a, STAGE_A, s);
    return e == hipSuccess ? TF_OK : hip_fail(e, "router launch");
}

size_t tf_gemv_workspace_bytes(int32_t d_ff, int32_t P) {
    if (d_ff <= 0 || P <= 0) return 256;
    return 256 + up256(h_row_bytes(d_ff) * P);
}

tf_status tf_expert_q4_gemv(const uint8_t *pool, size_t blob_stride, int32_t d_model,
                            int32_t d_ff, const int32_t *slot, const int32_t *token,
                            const float *coef, int32_t P, const uint16_t *x, int32_t T,
                            float *y32, tf_act act, void *ws, size_t ws_bytes, hipStream_t s) {
    if (P < 0 || P > 256 || T < 0 || T > 256) return fail(TF_E_ARG, "P and T must be in [0, 256]");
    if (P == 0 || T == 0) return TF_OK;
    if (!dim_ok(d_model) || !dim_ok(d_ff)) return fail(TF_E_SHAPE, "d_model/d_ff: multiples of 64 in [64, 4096]");
    if (!pool || !slot || !x || !y32 || !ws) return fail(TF_E_ARG, "NULL pool/slot/x/y32/ws");
    if (!token && T != P) return fail(TF_E_ARG, "token == NULL requires T == P");
    if (act != TF_GELU_ERF && act != TF_GELU_TANH) return fail(TF_E_ARG, "unknown activation");
    if (!aligned(pool, 256) || blob_stride % 256 || blob_stride < tf_expert_blob_bytes(d_model, d_ff))
        return fail(TF_E_ALIGN, "pool 256-byte aligned, stride a multiple of 256 >= blob size");
    if (!aligned(x, 16) || !aligned(y32, 16) || !aligned(ws, 256)) return fail(TF_E_ALIGN, "x/y32/ws alignment");
    if (ws_bytes < tf_gemv_workspace_bytes(d_ff, P)) return fail(TF_E_NOMEM, "workspace too small");
    DecodeArgs a;
    memset(&a, 0, sizeof a);
    a.d = d_model; a.f = d_ff; a.fs = d_model; a.E = 1; a.k = 1; a.T = T; a.act = act;
    a.x = x; a.pool = pool; a.stride = blob_stride;
    a.y32 = y32;
    a.hdr = at<uint32_t>(ws, 0);
    a.h_r = at<uint4>(ws, 256);
    a.gemv_slot = slot; a.gemv_token = token; a.gemv_coef = coef; a.P = P;
    a.tbx = 1; a.tbi = 1;
    a.b_routed_blocks = P * (d_ff / (2 * (64 / tf_decode_lpr(a))));
    hipError_t e = tf_launch_decode(a, STAGE_B | STAGE_C, s);
    return e == hipSuccess ? TF_OK : hip_fail(e, "gemv launch");
}

tf_status tf_profile_stream_read(const void *p, size_t bytes, hipStream_t s) {
    if (!p || bytes % 16 || ((uintptr_t)p & 15)) return fail(TF_E_ARG, "16-byte aligned pointer and size");
    hipError_t e = tf_launch_stream_read(p, bytes, s);
    return e == hipSuccess ? TF_OK : hip_fail(e, "stream-read kernel");
}

tf_status tf_profile_kernel(int32_t kernel, hipEvent_t start, hipEvent_t stop) {
    if (kernel != 0 && ((!start || !stop) || (kernel & (kernel - 1)) || kernel > 4096))
        return fail(TF_E_ARG, "one kernel id and two events, or kernel 0 to disarm");
    tf_arm_profile(kernel, start, stop);
    return TF_OK;
}

size_t tf_moe_workspace_bytes(const tf_moe_layer *L, int32_t T) {
    if (!L || T <= 0) return 0;
    if (T >= 2) return grouped_ws_bytes(L, T);
    return decode_layout(L->d_model, L->d_ff, L->d_ff_shared, L->n_experts, L->top_k, T).total;
}

tf_status tf_moe_layer_fwd(const tf_moe_layer *L, const uint16_t *x, int32_t T,
                           const int32_t *forced_ids, uint16_t *y, float *y32, int32_t *ids,
                           float *weights, tf_slot_cache *cache, int32_t layer,
                           hipStream_t compute, hipStream_t copy, void *ws, size_t ws_bytes) {
    if (T < 0 || T > MAX_DECODE_T) return fail(TF_E_ARG, "T must be in [0, %d]", MAX_DECODE_T);
    if (T == 0) return TF_OK;
    tf_status st = check_layer(L);
    if (st) return st;
    if (!x || !y || !ids || !weights || !ws) return fail(TF_E_ARG, "NULL x/y/ids/weights/ws");
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 256) || (y32 && !aligned(y32, 16)))
        return fail(TF_E_ALIGN, "x/y/y32 16-byte, ws 256-byte alignment");
    const size_t need = tf_moe_workspace_bytes(L, T);
    if (ws_bytes < need) return fail(TF_E_NOMEM, "workspace too small (%zu < %zu)", ws_bytes, need);
    if (cache) {
        if (T != 1) return fail(TF_E_ARG, "the slot-cache path takes one token per call");
        st = tf_slot_check_layer(cache, L, layer);
        if (st) return st;
    }
    hipError_t e;
    if (T >= 2) {   // several tokens: grouped by expert, as a prefill chunk
        e = grouped_step(L, x, T, forced_ids, y, y32, ids, weights, ws, compute);
        return e == hipSuccess ? TF_OK : hip_fail(e, "grouped decode launch");
    }
    const WsLayout w = decode_layout(L->d_model, L->d_ff, L->d_ff_shared, L->n_experts, L->top_k, T);

    DecodeArgs a;
    fill_common(a, L, T);
    a.x = x; a.forced = forced_ids; a.ids = ids; a.weights = weights; a.y = y; a.y32 = y32;
    a.hdr = at<uint32_t>(ws, w.hdr);
    a.logits = at<double>(ws, w.logits);
    a.items = at<int32_t>(ws, w.items);
    a.pairs = at<int32_t>(ws, w.pairs);
    a.h_s = at<uint4>(ws, w.hs);
    a.y_s = at<float>(ws, w.ys);
    a.h_r = at<uint4>(ws, w.hr);
    a.y_e = at<float>(ws, w.ye);
    a.ctk = at<uint32_t>(ws, w.ctk);
    a.do_group = 1;
    // T == 1: one item per rank; else items of up to tbi pairs of one expert
    // (at most E + T*k/tbi of them)
    const int max_items = T == 1 ? a.k
                          : (T * a.k < a.E + T * a.k / a.tbi ? T * a.k : a.E + T * a.k / a.tbi);
    const int n_router = router_blocks(a.E, T);
    // rows per workgroup: gate/up 2*RPW, shared down 4*RPW (RPW = 64 / lanes per row)
    const int rpw = 64 / tf_decode_lpr(a);
    const int n_shared_a = (a.fs / (2 * rpw)) * ((T + a.tbx - 1) / a.tbx);
    const int n_routed_b = (a.f / (2 * rpw)) * max_items;
    const int n_shared_b = (a.d / (4 * rpw)) * T;   // one token per shared-down block

    if (!cache) {
        a.a_router_blocks = n_router;
        a.a_shared_blocks = n_shared_a;
        a.b_routed_blocks = n_routed_b;
        a.b_shared_blocks = n_shared_b;
        e = tf_launch_decode(a, STAGE_A | STAGE_B | STAGE_C, compute);
        return e == hipSuccess ? TF_OK : hip_fail(e, "decode launch");
    }

    if (tf_slot_device_engine(cache)) {
        // Planned and filled on the GPU, all on `compute`: router + top-k +
        // lookup | miss copies beside the shared gate/up | routed gate/up +
        // shared down | routed down + combine.
        SlotFused sf;
        st = tf_slot_fused_begin(cache, layer, compute, &sf);
        if (st) return st;
        a.sc = sf.d;
        a.sc_layer = layer;
        a.sc_host = sf.host_layer;
        a.sc_slots = sf.slot_layer;
        a.a_router_blocks = n_router;
        e = tf_launch_decode(a, STAGE_A, compute);
        if (e != hipSuccess) return hip_fail(e, "router launch");
        a.a_router_blocks = 0;
        a.a_shared_blocks = n_shared_a;
        a.copy_per = SLOT_COPY_WGS_PER_BLOB;
        a.a_copy_blocks = a.k * a.copy_per;
        e = tf_launch_decode(a, STAGE_A, compute);
        if (e != hipSuccess) return hip_fail(e, "copy + shared-branch launch");
        a.a_shared_blocks = 0;
        a.a_copy_blocks = 0;
        a.slot_map = tf_slot_map(cache, layer);
        a.pool = tf_slot_pool(cache, layer);
        a.b_routed_blocks = n_routed_b;
        a.b_shared_blocks = n_shared_b;
        e = tf_launch_decode(a, STAGE_B | STAGE_C, compute);
        return e == hipSuccess ? TF_OK : hip_fail(e, "routed launch");
    }

    // Slot-cache path: router -> lookup -> shared branch (runs while the host
    // waits for the miss list and the copies run) -> routed experts.
    a.a_router_blocks = n_router;
    e = tf_launch_decode(a, STAGE_A, compute);
    if (e != hipSuccess) return hip_fail(e, "router launch");
    st = tf_slot_cache_lookup(cache, layer, ids, L->top_k, nullptr, compute);
    if (st) return st;
    a.a_router_blocks = 0;
    a.a_shared_blocks = n_shared_a;
    a.b_routed_blocks = 0;
    a.b_shared_blocks = n_shared_b;
    e = tf_launch_decode(a, STAGE_A | STAGE_B, compute);
    if (e != hipSuccess) return hip_fail(e, "shared-branch launch");
    hipEvent_t filled = tf_slot_fill_event(cache);
    int32_t nmiss = 0;
    st = tf_slot_cache_fill(cache, layer, copy, filled, &nmiss);
    if (st) return st;
    e = hipStreamWaitEvent(compute, filled, 0);
    if (e != hipSuccess) return hip_fail(e, "waiting for the fill");
    a.slot_map = tf_slot_map(cache, layer);
    a.pool = tf_slot_pool(cache, layer);
    a.b_routed_blocks = n_routed_b;
    a.b_shared_blocks = 0;
    e = tf_launch_decode(a, STAGE_B | STAGE_C, compute);
    return e == hipSuccess ? TF_OK : hip_fail(e, "routed launch");
}

}  // extern "C"

// ------------------------------------------------ allocation-free decode
// Scratch of tf_moe_layer_fwd_noalloc: a file-scope device array, one copy
// per GPU for the life of the process.  Host code never uses its name as an
// address; each device's address comes from hipGetSymbolAddress with that
// device current.
static __device__ __align__(256) unsigned char scratch[TF_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
bool g_scratch_clean[kMaxDevices];

// This device's scratch address (set up on the device's first call: the
// symbol address, then the whole array zeroed on `s`).  Returns NULL with
// the error recorded.
void *device_scratch(hipStream_t s, tf_status *st) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) { *st = hip_fail(e, "hipGetDevice"); return nullptr; }
    if (dev < 0 || dev >= kMaxDevices) { *st = fail(TF_E_STATE, "device %d out of range", dev); return nullptr; }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) { *st = hip_fail(e, "hipGetSymbolAddress(scratch)"); return nullptr; }
        g_scratch_ptr[dev] = p;
        g_scratch_clean[dev] = false;
    }
    if (!g_scratch_clean[dev]) {   // first use, or after a call that failed mid-way
        e = tf_launch_zero(g_scratch_ptr[dev], TF_NOALLOC_SCRATCH_BYTES, s);
        if (e != hipSuccess) { *st = hip_fail(e, "clearing the scratch"); return nullptr; }
        g_scratch_clean[dev] = true;
    }
    *st = TF_OK;
    return g_scratch_ptr[dev];
}

void scratch_dirty() {
    int dev = -1;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        g_scratch_clean[dev] = false;
    }
}
}  // namespace

extern "C" {

tf_status tf_moe_layer_fwd_noalloc(const tf_moe_layer *L, const uint16_t *x, int32_t T,
                                   const int32_t *forced_ids, uint16_t *y, float *y32,
                                   int32_t *ids, float *weights, hipStream_t stream) {
    if (T < 0 || T > MAX_DECODE_T) return fail(TF_E_ARG, "T must be in [0, %d]", MAX_DECODE_T);
    if (T == 0) return TF_OK;
    tf_status st = check_layer(L);
    if (st) return st;
    const size_t need = tf_moe_workspace_bytes(L, T);
    if (need > TF_NOALLOC_SCRATCH_BYTES)
        return fail(TF_E_NOMEM, "this step needs %zu bytes of scratch, more than the %zu the "
                    "allocation-free entry point holds (use tf_moe_layer_fwd with a workspace)",
                    need, (size_t)TF_NOALLOC_SCRATCH_BYTES);
    void *ws = device_scratch(stream, &st);
    if (!ws) return st;
    st = tf_moe_layer_fwd(L, x, T, forced_ids, y, y32, ids, weights, nullptr, 0, stream, stream,
                          ws, TF_NOALLOC_SCRATCH_BYTES);
    if (st == TF_E_HIP) scratch_dirty();   // counters may be left set: clear on the next call
    return st;
}

}  // extern "C"

extern "C" {

size_t tf_prefill_workspace_bytes(const tf_moe_layer *L, int32_t T) {
    if (!L || T <= 0) return 0;
    return grouped_ws_bytes(L, T);
}

// Chunked prefill (shilu.ai README translation, "推理引擎的工作原理": chunks
// of at most 128 tokens, so each fetched expert serves several rows): the
// grouped step, whose every expert's weights are read once per chunk.
tf_status tf_moe_prefill_chunk(const tf_moe_layer *L, const uint16_t *x, int32_t T, uint16_t *y,
                               float *y32, int32_t *ids, float *weights, hipStream_t s, void *ws,
                               size_t ws_bytes) {
    if (T < 0 || T > MAX_PREFILL_T) return fail(TF_E_ARG, "T must be in [0, %d]", MAX_PREFILL_T);
    if (T == 0) return TF_OK;
    tf_status st = check_layer(L);
    if (st) return st;
    if (!x || !y || !ids || !weights || !ws) return fail(TF_E_ARG, "NULL x/y/ids/weights/ws");
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 256) || (y32 && !aligned(y32, 16)))
        return fail(TF_E_ALIGN, "x/y/y32 16-byte, ws 256-byte alignment");
    if (ws_bytes < tf_prefill_workspace_bytes(L, T)) return fail(TF_E_NOMEM, "workspace too small");
    if (T == 1)   // a single token is a decode step
        return tf_moe_layer_fwd(L, x, 1, nullptr, y, y32, ids, weights, nullptr, 0, s, s, ws,
                                ws_bytes);
    const hipError_t e = grouped_step(L, x, T, nullptr, y, y32, ids, weights, ws, s);
    return e == hipSuccess ? TF_OK : hip_fail(e, "prefill launch");
}

// Grouping alone: the same block the prefill and batched decode steps run
// after their top-k, here on caller ids (shilu.ai README translation,
// "推理引擎的工作原理").  Workspace: a 256-B header, then the item records.
size_t tf_group_workspace_bytes(int32_t n_experts, int32_t T, int32_t top_k) {
    if (n_experts <= 0 || T <= 0 || top_k <= 0) return 256;
    return 256 + up256((size_t)4 * ITEM_INTS * ((size_t)n_experts + (size_t)T * top_k));
}

tf_status tf_group_by_expert(const int32_t *ids, int32_t T, int32_t top_k, int32_t n_experts,
                             int32_t *counts, int32_t *offsets, int32_t *pairs, void *ws,
                             size_t ws_bytes, hipStream_t s) {
    if (T < 0 || T > MAX_PREFILL_T) return fail(TF_E_SHAPE, "T must be in [0, %d]", MAX_PREFILL_T);
    if (T == 0) return TF_OK;
    if (top_k < 1 || top_k > 16 || n_experts < top_k || n_experts > 1024)
        return fail(TF_E_SHAPE, "need 1 <= top_k <= 16 and top_k <= n_experts <= 1024");
    if (!ids || !counts || !offsets || !pairs || !ws) return fail(TF_E_ARG, "NULL ids/counts/offsets/pairs/ws");
    if (!aligned(ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(pairs, 4) ||
        !aligned(ws, 256))
        return fail(TF_E_ALIGN, "int32 arrays 4-byte, ws 256-byte alignment");
    if (ws_bytes < tf_group_workspace_bytes(n_experts, T, top_k)) return fail(TF_E_NOMEM, "workspace too small");
    DecodeArgs a;
    memset(&a, 0, sizeof a);
    a.E = n_experts; a.k = top_k; a.T = T;
    a.ids = const_cast<int32_t *>(ids);   // read only by the grouping
    a.pairs = pairs;
    a.g_counts = counts; a.g_offsets = offsets;
    a.hdr = at<uint32_t>(ws, 0);
    a.items = at<int32_t>(ws, 256);
    a.tbi = 16;   // items of <= 16 tokens, as in a prefill chunk
    hipError_t e = tf_launch_group(a, s);
    return e == hipSuccess ? TF_OK : hip_fail(e, "grouping launch");
}

}  // extern "C"
