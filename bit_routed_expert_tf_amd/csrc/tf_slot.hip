// Per-layer LFU expert-slot cache: device tables, lookup kernel and the
// host-driven miss fill.
//
// The pages' runtime keeps 16 expert slots per layer, plans hits and misses
// on the CPU from the router's top-8, and fills misses with bounded parallel
// reads into GPU-visible buffers while the GPU runs the shared expert
// (shilu.ai README translation, "推理引擎的工作原理"; sh.edu-sjtu.cn, "三件事").
// Here the plan runs on the GPU right after the router (one wave, no host
// round trip), the miss list lands in mapped pinned host memory, and the host
// turns it into one hipMemcpyAsync per miss from a pinned host pool on a copy
// stream; the shared-expert kernels are already queued on the compute stream
// and run meanwhile.
//
// Policy (reading of "LFU"): a slot's count is 1 on fill and +1 per hit; the
// token's own ids are pinned; misses are taken in rank order; the victim is
// the lowest empty slot, else the unpinned slot with the smallest
// (count, last-use token, slot index); every layer starts empty.  The LRU
// option (the sh.edu-sjtu.cn article's gloss, "三件事") takes the unpinned
// slot with the smallest (last-use token, slot index) instead.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "tf_slot.h"

// Plain device view of the tables (passed to the lookup kernel by value).
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
};

struct tf_slot_cache {
    SlotDev d;
    size_t stride;
    uint8_t *slot_pool;
    const uint8_t *host_pool;
    void *dev;                 // one device allocation for all tables
    int32_t *miss_host;        // [L][1+2k]: n, (expert, slot)*
    std::vector<hipEvent_t> ev_lookup;
    std::vector<int> pending;
    hipEvent_t ev_fill;
    int64_t bytes_filled;
};

namespace {

__global__ void k_fill16(int16_t *p, size_t n, int16_t v) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// One token's lookup for one layer; a single lane walks the policy so that
// the order of every decision is exactly the policy's order.
__global__ __launch_bounds__(64) void k_lookup(SlotDev c, int layer, const int32_t *ids,
                                               int n, int32_t *slots_out, uint32_t *flags) {
    if (threadIdx.x != 0) return;
    const int S = c.S, E = c.E;
    int32_t *slot_of = c.slot_of + (size_t)layer * E;
    int16_t *expert_of = c.expert_of + (size_t)layer * S;
    uint32_t *count = c.count + (size_t)layer * S;
    uint32_t *last = c.last + (size_t)layer * S;
    int32_t *miss = c.miss_dev + (size_t)layer * (1 + 2 * c.k);
    const uint32_t t = c.tok[layer];
    int e_r[16], s_r[16];
    bool hit[16];
    uint32_t pinned = 0, fl = 0;
    for (int r = 0; r < n; ++r) {
        int e = ids[r];
        if (e < 0 || e >= E) { fl |= TF_FLAG_ID_RANGE; e = e < 0 ? 0 : E - 1; }
        for (int q = 0; q < r; ++q)
            if (e_r[q] == e) fl |= TF_FLAG_ID_REPEAT;
        e_r[r] = e;
        const int s = slot_of[e];
        hit[r] = s >= 0;
        s_r[r] = s;
        if (s >= 0) {               // hits first: they are pinned for this token
            bool seen = (pinned >> s) & 1u;
            if (!seen) { count[s] += 1; last[s] = t; }
            pinned |= 1u << s;
        }
    }
    int nm = 0;
    for (int r = 0; r < n; ++r) {
        if (hit[r]) continue;
        const int e = e_r[r];
        if (slot_of[e] >= 0) {      // repeated id already filled for this token
            s_r[r] = slot_of[e];
            continue;
        }
        int v = -1;
        for (int s = 0; s < S; ++s)
            if (expert_of[s] < 0) { v = s; break; }
        if (v < 0) {
            for (int s = 0; s < S; ++s) {
                if ((pinned >> s) & 1u) continue;
                const bool lt = c.policy == TF_SLOT_LRU
                                    ? last[s] < last[v]
                                    : count[s] < count[v] || (count[s] == count[v] && last[s] < last[v]);
                if (v < 0 || lt) v = s;
            }
            slot_of[expert_of[v]] = -1;
        }
        expert_of[v] = (int16_t)e;
        slot_of[e] = v;
        count[v] = 1;
        last[v] = t;
        pinned |= 1u << v;
        s_r[r] = v;
        miss[1 + 2 * nm] = e;
        miss[2 + 2 * nm] = v;
        ++nm;
    }
    miss[0] = nm;
    if ((int64_t)t < c.trace_cap) {
        int8_t *th = c.trace_hit + ((size_t)layer * c.trace_cap + t) * c.k;
        int16_t *ts = c.trace_slot + ((size_t)layer * c.trace_cap + t) * c.k;
        for (int r = 0; r < n; ++r) { th[r] = hit[r] ? 1 : 0; ts[r] = (int16_t)s_r[r]; }
    }
    if (slots_out)
        for (int r = 0; r < n; ++r) slots_out[r] = s_r[r];
    if (fl && flags) atomicOr(flags, fl);
    c.tok[layer] = t + 1;
    __threadfence_system();
}

}  // namespace

void tf_set_error(const char *msg);   // tf_api.cpp

namespace {
tf_status fail(tf_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    tf_set_error(buf);
    return st;
}
inline size_t up256(size_t n) { return (n + 255) & ~size_t(255); }
}  // namespace

tf_status tf_slot_check_layer(const tf_slot_cache *c, const tf_moe_layer *L, int32_t layer) {
    if (layer < 0 || layer >= c->d.L) return fail(TF_E_ARG, "layer %d out of range", layer);
    if (L->n_experts != c->d.E || L->top_k != c->d.k || L->blob_stride != c->stride)
        return fail(TF_E_SHAPE, "layer shape does not match the slot cache");
    return TF_OK;
}

hipEvent_t tf_slot_fill_event(tf_slot_cache *c) { return c->ev_fill; }
const int32_t *tf_slot_map(const tf_slot_cache *c, int32_t layer) {
    return c->d.slot_of + (size_t)layer * c->d.E;
}
const uint8_t *tf_slot_pool(const tf_slot_cache *c, int32_t layer) {
    return c->slot_pool + (size_t)layer * c->d.S * c->stride;
}

static tf_status reset_tables(tf_slot_cache *c) {
    // slot_of (int32) and expert_of (int16) to -1: both are all-ones bit patterns
    const size_t n16 = 2 * (size_t)c->d.L * c->d.E + (size_t)c->d.L * c->d.S;
    hipLaunchKernelGGL(k_fill16, dim3(256), dim3(256), 0, 0,
                       reinterpret_cast<int16_t *>(c->d.slot_of), n16, (int16_t)-1);
    hipError_t e = hipGetLastError();
    const size_t zbytes = (size_t)c->d.L * c->d.S * 8 + (size_t)c->d.L * 4;   // count, last, tok
    if (e == hipSuccess) e = tf_launch_zero(c->d.count, (zbytes + 3) & ~size_t(3), 0);
    if (e == hipSuccess && c->d.trace_cap) {
        const size_t tb = (size_t)c->d.L * c->d.trace_cap * c->d.k;
        e = tf_launch_zero(c->d.trace_hit, up256(tb) + up256(2 * tb), 0);
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(TF_E_HIP, "slot cache reset: %s", hipGetErrorString(e));
    memset(c->miss_host, 0, sizeof(int32_t) * c->d.L * (1 + 2 * c->d.k));
    for (auto &p : c->pending) p = 0;
    c->bytes_filled = 0;
    return TF_OK;
}

extern "C" {

tf_status tf_slot_cache_create(int32_t n_layers, int32_t n_experts, int32_t n_slots,
                               int32_t top_k, size_t blob_stride, uint8_t *slot_pool,
                               const uint8_t *host_pool_pinned, int64_t trace_cap,
                               tf_slot_cache **out) {
    if (!out) return fail(TF_E_ARG, "out is NULL");
    *out = nullptr;
    if (n_layers < 1 || n_layers > 1024) return fail(TF_E_ARG, "n_layers must be in [1, 1024]");
    if (top_k < 1 || top_k > 16) return fail(TF_E_SHAPE, "top_k must be in [1, 16]");
    if (n_experts < top_k || n_experts > 1024) return fail(TF_E_SHAPE, "n_experts must be in [top_k, 1024]");
    if (n_slots < top_k || n_slots > 32 || n_slots > n_experts)
        return fail(TF_E_ARG, "n_slots must be in [top_k, min(32, n_experts)]");
    if (!slot_pool || !host_pool_pinned) return fail(TF_E_ARG, "NULL pool");
    if (blob_stride == 0 || blob_stride % 256 || ((uintptr_t)slot_pool & 255))
        return fail(TF_E_ALIGN, "slot pool 256-byte aligned, stride a multiple of 256");
    if (trace_cap < 0) return fail(TF_E_ARG, "trace_cap must be >= 0");
    tf_slot_cache *c = new (std::nothrow) tf_slot_cache();
    if (!c) return fail(TF_E_NOMEM, "host allocation failed");
    c->d.L = n_layers; c->d.E = n_experts; c->d.S = n_slots; c->d.k = top_k;
    c->stride = blob_stride; c->slot_pool = slot_pool; c->host_pool = host_pool_pinned;
    c->d.trace_cap = trace_cap;
    const size_t o_slot_of = 0;
    const size_t o_expert_of = o_slot_of + 4 * (size_t)n_layers * n_experts;
    const size_t o_count = up256(o_expert_of + 2 * (size_t)n_layers * n_slots);
    const size_t o_last = o_count + 4 * (size_t)n_layers * n_slots;
    const size_t o_tok = o_last + 4 * (size_t)n_layers * n_slots;
    const size_t o_th = up256(o_tok + 4 * (size_t)n_layers);
    const size_t tb = (size_t)n_layers * trace_cap * top_k;
    const size_t o_ts = o_th + up256(tb);
    const size_t total = o_ts + up256(2 * tb) + 256;
    hipError_t e = hipMalloc(&c->dev, total);
    if (e != hipSuccess) { delete c; return fail(TF_E_NOMEM, "device tables: %s", hipGetErrorString(e)); }
    char *b = static_cast<char *>(c->dev);
    c->d.slot_of = reinterpret_cast<int32_t *>(b + o_slot_of);
    c->d.expert_of = reinterpret_cast<int16_t *>(b + o_expert_of);
    c->d.count = reinterpret_cast<uint32_t *>(b + o_count);
    c->d.last = reinterpret_cast<uint32_t *>(b + o_last);
    c->d.tok = reinterpret_cast<uint32_t *>(b + o_tok);
    c->d.trace_hit = reinterpret_cast<int8_t *>(b + o_th);
    c->d.trace_slot = reinterpret_cast<int16_t *>(b + o_ts);
    e = hipHostMalloc(reinterpret_cast<void **>(&c->miss_host),
                      sizeof(int32_t) * n_layers * (1 + 2 * top_k), hipHostMallocMapped);
    if (e != hipSuccess) {
        (void)hipFree(c->dev);
        delete c;
        return fail(TF_E_NOMEM, "pinned miss list: %s", hipGetErrorString(e));
    }
    e = hipHostGetDevicePointer(reinterpret_cast<void **>(&c->d.miss_dev), c->miss_host, 0);
    c->ev_lookup.assign(n_layers, nullptr);
    c->pending.assign(n_layers, 0);
    for (int l = 0; l < n_layers && e == hipSuccess; ++l)
        e = hipEventCreateWithFlags(&c->ev_lookup[l], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_fill, hipEventDisableTiming);
    if (e != hipSuccess) {
        tf_slot_cache_destroy(c);
        return fail(TF_E_HIP, "slot cache events: %s", hipGetErrorString(e));
    }
    tf_status st = reset_tables(c);
    if (st) { tf_slot_cache_destroy(c); return st; }
    *out = c;
    return TF_OK;
}

void tf_slot_cache_destroy(tf_slot_cache *c) {
    if (!c) return;
    (void)hipDeviceSynchronize();
    for (auto ev : c->ev_lookup)
        if (ev) (void)hipEventDestroy(ev);
    if (c->ev_fill) (void)hipEventDestroy(c->ev_fill);
    if (c->miss_host) (void)hipHostFree(c->miss_host);
    if (c->dev) (void)hipFree(c->dev);
    delete c;
}

tf_status tf_slot_cache_lookup(tf_slot_cache *c, int32_t layer, const int32_t *ids, int32_t n,
                               int32_t *slots, hipStream_t compute) {
    if (!c || !ids) return fail(TF_E_ARG, "NULL cache/ids");
    if (layer < 0 || layer >= c->d.L) return fail(TF_E_ARG, "layer %d out of range", layer);
    if (n != c->d.k) return fail(TF_E_ARG, "n must equal top_k (%d)", c->d.k);
    if (c->pending[layer]) return fail(TF_E_STATE, "layer %d: previous lookup not filled", layer);
    hipLaunchKernelGGL(k_lookup, dim3(1), dim3(64), 0, compute, c->d, layer, ids, n, slots,
                       static_cast<uint32_t *>(nullptr));
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(c->ev_lookup[layer], compute);
    if (e != hipSuccess) return fail(TF_E_HIP, "lookup: %s", hipGetErrorString(e));
    c->pending[layer] = 1;
    return TF_OK;
}

tf_status tf_slot_cache_fill(tf_slot_cache *c, int32_t layer, hipStream_t copy, hipEvent_t filled,
                             int32_t *n_miss_host) {
    if (!c) return fail(TF_E_ARG, "NULL cache");
    if (layer < 0 || layer >= c->d.L) return fail(TF_E_ARG, "layer %d out of range", layer);
    if (!c->pending[layer]) return fail(TF_E_STATE, "layer %d: fill without a lookup", layer);
    hipError_t e = hipEventSynchronize(c->ev_lookup[layer]);
    if (e != hipSuccess) return fail(TF_E_HIP, "waiting for lookup: %s", hipGetErrorString(e));
    c->pending[layer] = 0;
    const int32_t *m = c->miss_host + (size_t)layer * (1 + 2 * c->d.k);
    const int nm = m[0];
    if (nm < 0 || nm > c->d.k) return fail(TF_E_STATE, "corrupt miss list (%d)", nm);
    for (int i = 0; i < nm && e == hipSuccess; ++i) {
        const int ex = m[1 + 2 * i], sl = m[2 + 2 * i];
        if (ex < 0 || ex >= c->d.E || sl < 0 || sl >= c->d.S) return fail(TF_E_STATE, "corrupt miss entry");
        uint8_t *dst = c->slot_pool + ((size_t)layer * c->d.S + sl) * c->stride;
        const uint8_t *src = c->host_pool + ((size_t)layer * c->d.E + ex) * c->stride;
        e = hipMemcpyAsync(dst, src, c->stride, hipMemcpyHostToDevice, copy);
    }
    if (e == hipSuccess && filled) e = hipEventRecord(filled, copy);
    if (e != hipSuccess) return fail(TF_E_HIP, "fill: %s", hipGetErrorString(e));
    c->bytes_filled += (int64_t)nm * (int64_t)c->stride;
    if (n_miss_host) *n_miss_host = nm;
    return TF_OK;
}

tf_status tf_slot_cache_trace(tf_slot_cache *c, int32_t layer, int8_t *hit_host,
                              int16_t *slot_host, int64_t cap, int64_t *len) {
    if (!c || !len) return fail(TF_E_ARG, "NULL argument");
    if (layer < 0 || layer >= c->d.L) return fail(TF_E_ARG, "layer %d out of range", layer);
    uint32_t tok = 0;
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(&tok, c->d.tok + layer, 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(TF_E_HIP, "trace: %s", hipGetErrorString(e));
    int64_t n = (int64_t)(tok < (uint64_t)c->d.trace_cap ? tok : c->d.trace_cap) * c->d.k;
    if (n > cap) n = cap;
    if (n > 0 && hit_host)
        e = hipMemcpy(hit_host, c->d.trace_hit + (size_t)layer * c->d.trace_cap * c->d.k, n,
                      hipMemcpyDeviceToHost);
    if (e == hipSuccess && n > 0 && slot_host)
        e = hipMemcpy(slot_host, c->d.trace_slot + (size_t)layer * c->d.trace_cap * c->d.k, 2 * n,
                      hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(TF_E_HIP, "trace copy: %s", hipGetErrorString(e));
    *len = n;
    return TF_OK;
}

tf_status tf_slot_cache_reset(tf_slot_cache *c) {
    if (!c) return fail(TF_E_ARG, "NULL cache");
    return reset_tables(c);
}

int64_t tf_slot_cache_bytes_filled(const tf_slot_cache *c) { return c ? c->bytes_filled : -1; }

tf_status tf_slot_cache_set_policy(tf_slot_cache *c, int32_t policy) {
    if (!c) return fail(TF_E_ARG, "NULL cache");
    if (policy != TF_SLOT_LFU && policy != TF_SLOT_LRU) return fail(TF_E_ARG, "unknown policy %d", policy);
    c->d.policy = policy;
    return TF_OK;
}

}  // extern "C"
