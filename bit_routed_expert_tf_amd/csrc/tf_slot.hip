// Per-layer LFU expert-slot cache: device tables, lookup kernel and the
// host-driven miss fill.
//
// The pages' runtime keeps 16 expert slots per layer, plans hits and misses
// on the CPU from the router's top-8, and fills misses with bounded parallel
// reads into GPU-visible buffers while the GPU runs the shared expert
// (shilu.ai README translation, "推理引擎的工作原理"; sh.edu-sjtu.cn, "三件事").
// Here the plan runs on the GPU right after the router (one wave, no host
// round trip), the miss list lands in mapped pinned host memory, and the host
// turns it into one copy launch over all the misses (a kernel reading the
// pinned host pool through its device mapping; or one hipMemcpyAsync per
// miss) on a copy stream; the shared-expert kernels are already queued on
// the compute stream and run meanwhile.  Optionally the host copies the
// experts it predicts for a layer into per-layer buffers ahead of that
// layer's lookup (speculative fill, after the pages' read-ahead); the fill
// then takes each predicted miss from its buffer.  Predictions never change
// the hit/miss sequence.  With the device copy engine the host is out of the
// loop: the lookup also leaves the miss list in device memory, and a copy
// kernel queued behind the lookup on the copy stream reads it and moves the
// missed blobs.
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
#include "tf_slot_dev.h"

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
    // speculative fill (tf_slot_cache_prefetch)
    uint8_t *pf_pool = nullptr;          // device [L][P][stride] (caller-owned)
    int P = 0;                           // buffers per layer (0 = off)
    std::vector<int16_t> mirror;         // [L][S] expert per slot as the fills left it
    std::vector<int32_t> pf;             // [L][P] expert in each buffer (-1 free)
    std::vector<hipEvent_t> ev_pf;       // [L] after the layer's latest prefetch copies
    std::vector<hipEvent_t> ev_done;     // [L] after the layer's latest fill copies
    int64_t pf_bytes = 0, pf_used = 0, pf_wasted = 0;
    const uint8_t *host_dev = nullptr;   // device mapping of host_pool (NULL: DMA only)
    int engine = TF_SLOT_COPY_KERNEL;   // DMA when the host pool has no mapping
    std::vector<hipEvent_t> ev_dfill;    // [L] after the layer's latest device-initiated fill
    std::vector<char> dfill_pending;     // [L] that fill may still run
    bool dfill_any = false;              // some fill ran with TF_SLOT_COPY_DEVICE
};

namespace {

__global__ void k_fill16(int16_t *p, size_t n, int16_t v) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// Blob copies by a kernel: blob blockIdx.y, the x workgroups of a blob
// striding over it in 16-byte units, four loads in flight per thread.  The
// sources are device blobs (prefetch buffers) or blobs of the pinned host
// pool read over PCIe through its device mapping (the kernel copy engine):
// one launch moves all of a call's blobs, where one DMA copy per 3.3 MB blob
// pays a fixed cost each (39 GB/s for such copies back to back, against
// 54-56 GB/s for large ones).  On an idle GPU four workgroups per host blob
// already reach the PCIe rate; beside the decode kernels sixteen do (fewer
// starve, more crowd the decode kernels).
constexpr int MAX_COPIES = 32;
struct BlobCopies {
    const uint4 *src[MAX_COPIES];
    uint4 *dst[MAX_COPIES];
};
__device__ __forceinline__ void copy_blob(const uint4 *src, uint4 *dst, size_t n16) {
    const size_t step = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += 4 * step) {
        uint4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (i + j * step < n16) v[j] = src[i + j * step];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (i + j * step < n16) dst[i + j * step] = v[j];
    }
}
__global__ __launch_bounds__(256) void k_copy_blobs(BlobCopies c, size_t n16) {
    copy_blob(c.src[blockIdx.y], c.dst[blockIdx.y], n16);
}

// Fill of one layer planned on the GPU: the miss list the lookup left in
// device memory says which blobs to move, so the copy starts as soon as the
// lookup ends, with no host round trip.  Miss blockIdx.y of the list.
__global__ __launch_bounds__(256) void k_fill_listed(const int32_t *miss, const uint8_t *host_layer,
                                                     uint8_t *slot_layer, size_t stride, int E, int S,
                                                     unsigned long long *nfill) {
    slotk::copy_missed(miss, host_layer, slot_layer, stride, E, S, nfill, blockIdx.y, blockIdx.x,
                       gridDim.x, threadIdx.x);
}

// One token's lookup for one layer (one wave), the miss list also in the
// mapped host memory for the host-driven fills.
__global__ __launch_bounds__(64) void k_lookup(SlotDev c, int layer, const int32_t *ids, int n,
                                               int32_t *slots_out) {
    slotk::lookup_wave(c, layer, ids, n, slots_out, true, threadIdx.x);
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
bool tf_slot_device_engine(const tf_slot_cache *c) { return c->engine == TF_SLOT_COPY_DEVICE; }

tf_status tf_slot_fused_begin(tf_slot_cache *c, int32_t layer, hipStream_t compute, SlotFused *out) {
    if (c->pending[layer]) return fail(TF_E_STATE, "layer %d: previous lookup not filled", layer);
    if (c->dfill_pending[layer]) {   // a standalone fill may still read the layer's miss list
        const hipError_t e = hipStreamWaitEvent(compute, c->ev_dfill[layer], 0);
        if (e != hipSuccess) return fail(TF_E_HIP, "slot step: %s", hipGetErrorString(e));
        c->dfill_pending[layer] = 0;
    }
    out->d = c->d;
    out->host_layer = c->host_dev + (size_t)layer * c->d.E * c->stride;
    out->slot_layer = c->slot_pool + (size_t)layer * c->d.S * c->stride;
    c->dfill_any = true;
    return TF_OK;
}
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
    // count, last, tok, the device miss lists and the fill counter
    const size_t zbytes = reinterpret_cast<char *>(c->d.nfill + 1) - reinterpret_cast<char *>(c->d.count);
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
    c->mirror.assign((size_t)c->d.L * c->d.S, -1);
    c->pf.assign((size_t)c->d.L * c->P, -1);
    c->pf_bytes = c->pf_used = c->pf_wasted = 0;
    c->dfill_any = false;
    for (auto &p : c->dfill_pending) p = 0;
    return TF_OK;
}

// Host-pool blob (layer, expert) as seen by a kernel.
static const uint4 *host_blob_dev(const tf_slot_cache *c, int layer, int ex) {
    if (!c->host_dev) return nullptr;
    return reinterpret_cast<const uint4 *>(c->host_dev + ((size_t)layer * c->d.E + ex) * c->stride);
}

// One k_copy_blobs launch for n blobs (n <= MAX_COPIES) with `per_blob`
// workgroups each.
static hipError_t launch_copies(const tf_slot_cache *c, const BlobCopies &bc, int n, int per_blob,
                                hipStream_t s) {
    if (!n) return hipSuccess;
    hipLaunchKernelGGL(k_copy_blobs, dim3(per_blob, n), dim3(256), 0, s, bc, c->stride / 16);
    return hipGetLastError();
}
constexpr int HOST_WGS_PER_BLOB = 16;   // PCIe reads: about 1 MB in flight per blob
constexpr int DEV_WGS_PER_BLOB = 64;    // HBM copies

// n host-to-device DMA copies of one blob each on `copy`.
static hipError_t dma_copies(const tf_slot_cache *c, uint8_t *const *dst, const uint8_t *const *src,
                             int n, hipStream_t copy) {
    hipError_t e = hipSuccess;
    for (int j = 0; j < n && e == hipSuccess; ++j)
        e = hipMemcpyAsync(dst[j], src[j], c->stride, hipMemcpyHostToDevice, copy);
    return e;
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
    const size_t o_miss = o_tok + 4 * (size_t)n_layers;
    const size_t o_nfill = (o_miss + 4 * (size_t)n_layers * (1 + 2 * top_k) + 7) & ~size_t(7);
    const size_t o_th = up256(o_nfill + 8);
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
    c->d.miss_gpu = reinterpret_cast<int32_t *>(b + o_miss);
    c->d.nfill = reinterpret_cast<unsigned long long *>(b + o_nfill);
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
    if (e == hipSuccess) {
        void *hd = nullptr;   // kernels read the host pool through its mapping when it has one
        if (hipHostGetDevicePointer(&hd, const_cast<uint8_t *>(host_pool_pinned), 0) == hipSuccess)
            c->host_dev = static_cast<const uint8_t *>(hd);
        else
            (void)hipGetLastError();
        if (!c->host_dev) c->engine = TF_SLOT_COPY_DMA;
    }
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
    for (auto ev : c->ev_pf)
        if (ev) (void)hipEventDestroy(ev);
    for (auto ev : c->ev_done)
        if (ev) (void)hipEventDestroy(ev);
    for (auto ev : c->ev_dfill)
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
    if (c->dfill_pending.size() && c->dfill_pending[layer]) {   // its miss list is still being read
        const hipError_t w = hipStreamWaitEvent(compute, c->ev_dfill[layer], 0);
        if (w != hipSuccess) return fail(TF_E_HIP, "lookup: %s", hipGetErrorString(w));
        c->dfill_pending[layer] = 0;
    }
    hipLaunchKernelGGL(k_lookup, dim3(1), dim3(64), 0, compute, c->d, layer, ids, n, slots);
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
    if (c->engine == TF_SLOT_COPY_DEVICE) {
        // the copy stream waits for the lookup on the GPU; the kernel reads the list itself
        hipError_t e = hipStreamWaitEvent(copy, c->ev_lookup[layer], 0);
        const size_t lay = (size_t)layer;
        if (e == hipSuccess) {
            hipLaunchKernelGGL(k_fill_listed, dim3(HOST_WGS_PER_BLOB, c->d.k), dim3(256), 0, copy,
                               c->d.miss_gpu + lay * (1 + 2 * c->d.k), c->host_dev + lay * c->d.E * c->stride,
                               c->slot_pool + lay * c->d.S * c->stride, c->stride, c->d.E, c->d.S, c->d.nfill);
            e = hipGetLastError();
        }
        if (e == hipSuccess) e = hipEventRecord(c->ev_dfill[layer], copy);
        if (e == hipSuccess && filled) e = hipEventRecord(filled, copy);
        if (e != hipSuccess) return fail(TF_E_HIP, "device fill: %s", hipGetErrorString(e));
        c->pending[layer] = 0;
        c->dfill_pending[layer] = 1;
        c->dfill_any = true;
        if (n_miss_host) *n_miss_host = -1;
        return TF_OK;
    }
    hipError_t e = hipEventSynchronize(c->ev_lookup[layer]);
    if (e != hipSuccess) return fail(TF_E_HIP, "waiting for lookup: %s", hipGetErrorString(e));
    c->pending[layer] = 0;
    const int32_t *m = c->miss_host + (size_t)layer * (1 + 2 * c->d.k);
    const int nm = m[0];
    if (nm < 0 || nm > c->d.k) return fail(TF_E_STATE, "corrupt miss list (%d)", nm);
    int32_t *pf = c->P ? c->pf.data() + (size_t)layer * c->P : nullptr;
    const bool kern = c->engine == TF_SLOT_COPY_KERNEL;
    BlobCopies dc, hc;
    int ndc = 0, nhc = 0, nh = 0;
    uint8_t *hdst[16];
    const uint8_t *hsrc[16];
    int64_t h2d = 0;
    for (int i = 0; i < nm && e == hipSuccess; ++i) {
        const int ex = m[1 + 2 * i], sl = m[2 + 2 * i];
        if (ex < 0 || ex >= c->d.E || sl < 0 || sl >= c->d.S) return fail(TF_E_STATE, "corrupt miss entry");
        c->mirror[(size_t)layer * c->d.S + sl] = (int16_t)ex;
        uint8_t *dst = c->slot_pool + ((size_t)layer * c->d.S + sl) * c->stride;
        int b = -1;
        for (int q = 0; q < c->P; ++q)
            if (pf[q] == ex) { b = q; break; }
        if (b >= 0) {   // speculatively filled: a device copy from its buffer
            dc.src[ndc] = reinterpret_cast<const uint4 *>(c->pf_pool + ((size_t)layer * c->P + b) * c->stride);
            dc.dst[ndc] = reinterpret_cast<uint4 *>(dst);
            ++ndc;
            pf[b] = -2;   // used
            ++c->pf_used;
        } else {
            if (kern) {
                hc.src[nhc] = host_blob_dev(c, layer, ex);
                hc.dst[nhc] = reinterpret_cast<uint4 *>(dst);
                ++nhc;
            } else {
                hdst[nh] = dst;
                hsrc[nh] = c->host_pool + ((size_t)layer * c->d.E + ex) * c->stride;
                ++nh;
            }
            h2d += (int64_t)c->stride;
        }
    }
    if (e == hipSuccess) e = launch_copies(c, hc, nhc, HOST_WGS_PER_BLOB, copy);
    if (e == hipSuccess) e = dma_copies(c, hdst, hsrc, nh, copy);
    if (ndc && e == hipSuccess) {   // after the prefetch copies, wherever they ran
        e = hipStreamWaitEvent(copy, c->ev_pf[layer], 0);
        if (e == hipSuccess) e = launch_copies(c, dc, ndc, DEV_WGS_PER_BLOB, copy);
    }
    for (int q = 0; q < c->P; ++q) {   // buffers serve one lookup
        if (pf[q] >= 0) ++c->pf_wasted;
        pf[q] = -1;
    }
    if (e == hipSuccess && c->P) e = hipEventRecord(c->ev_done[layer], copy);
    if (e == hipSuccess && filled) e = hipEventRecord(filled, copy);
    if (e != hipSuccess) return fail(TF_E_HIP, "fill: %s", hipGetErrorString(e));
    c->bytes_filled += h2d;
    if (n_miss_host) *n_miss_host = nm;
    return TF_OK;
}

tf_status tf_slot_cache_set_prefetch(tf_slot_cache *c, uint8_t *buffers, int32_t n_buffers) {
    if (!c) return fail(TF_E_ARG, "NULL cache");
    if (n_buffers < 0 || n_buffers > 16) return fail(TF_E_ARG, "n_buffers must be in [0, 16]");
    if (n_buffers && c->engine == TF_SLOT_COPY_DEVICE)
        return fail(TF_E_STATE, "prefetch needs a host-driven copy engine");
    if (n_buffers && !buffers) return fail(TF_E_ARG, "NULL buffers");
    if ((uintptr_t)buffers & 255) return fail(TF_E_ALIGN, "buffers 256-byte aligned");
    hipError_t e = hipSuccess;
    if (n_buffers && c->ev_pf.empty()) {
        c->ev_pf.assign(c->d.L, nullptr);
        c->ev_done.assign(c->d.L, nullptr);
        for (int l = 0; l < c->d.L && e == hipSuccess; ++l) {
            e = hipEventCreateWithFlags(&c->ev_pf[l], hipEventDisableTiming);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_done[l], hipEventDisableTiming);
        }
        if (e != hipSuccess) return fail(TF_E_HIP, "prefetch events: %s", hipGetErrorString(e));
    }
    e = hipDeviceSynchronize();   // no copy into the old buffers is in flight
    if (e != hipSuccess) return fail(TF_E_HIP, "set_prefetch: %s", hipGetErrorString(e));
    c->pf_pool = n_buffers ? buffers : nullptr;
    c->P = n_buffers;
    c->pf.assign((size_t)c->d.L * c->P, -1);
    return TF_OK;
}

tf_status tf_slot_cache_prefetch(tf_slot_cache *c, int32_t layer, const int32_t *ids_host, int32_t n,
                                 hipStream_t copy, int32_t *n_issued) {
    if (!c) return fail(TF_E_ARG, "NULL cache");
    if (layer < 0 || layer >= c->d.L) return fail(TF_E_ARG, "layer %d out of range", layer);
    if (!c->P) return fail(TF_E_STATE, "no prefetch buffers (tf_slot_cache_set_prefetch)");
    if (n < 0 || n > 1024 || (n && !ids_host)) return fail(TF_E_ARG, "need 0 <= n <= 1024 ids");
    for (int i = 0; i < n; ++i)
        if (ids_host[i] < 0 || ids_host[i] >= c->d.E) return fail(TF_E_ARG, "id %d out of range", ids_host[i]);
    if (c->pending[layer]) return fail(TF_E_STATE, "layer %d: lookup not yet filled", layer);
    // the previous fill's device copies out of these buffers come first
    hipError_t e = hipStreamWaitEvent(copy, c->ev_done[layer], 0);
    const int16_t *mir = c->mirror.data() + (size_t)layer * c->d.S;
    int32_t *pf = c->pf.data() + (size_t)layer * c->P;
    const bool kern = c->engine == TF_SLOT_COPY_KERNEL;
    BlobCopies hc;
    uint8_t *hdst[16];
    const uint8_t *hsrc[16];
    int issued = 0;
    for (int i = 0; i < n && e == hipSuccess; ++i) {
        const int ex = ids_host[i];
        bool skip = false;
        for (int s = 0; s < c->d.S && !skip; ++s) skip = mir[s] == ex;    // resident
        for (int q = 0; q < c->P && !skip; ++q) skip = pf[q] == ex;       // already fetched
        if (skip) continue;
        int b = -1;
        for (int q = 0; q < c->P; ++q)
            if (pf[q] == -1) { b = q; break; }
        if (b < 0) break;   // every buffer holds a prediction
        uint8_t *dst = c->pf_pool + ((size_t)layer * c->P + b) * c->stride;
        hc.src[issued] = host_blob_dev(c, layer, ex);
        hc.dst[issued] = reinterpret_cast<uint4 *>(dst);
        hdst[issued] = dst;
        hsrc[issued] = c->host_pool + ((size_t)layer * c->d.E + ex) * c->stride;
        pf[b] = ex;
        c->pf_bytes += (int64_t)c->stride;
        ++issued;
    }
    if (e == hipSuccess)
        e = kern ? launch_copies(c, hc, issued, HOST_WGS_PER_BLOB, copy) : dma_copies(c, hdst, hsrc, issued, copy);
    if (e == hipSuccess && issued) e = hipEventRecord(c->ev_pf[layer], copy);
    if (e != hipSuccess) return fail(TF_E_HIP, "prefetch: %s", hipGetErrorString(e));
    if (n_issued) *n_issued = issued;
    return TF_OK;
}

tf_status tf_slot_cache_set_copy_engine(tf_slot_cache *c, int32_t engine) {
    if (!c) return fail(TF_E_ARG, "NULL cache");
    if (engine != TF_SLOT_COPY_DMA && engine != TF_SLOT_COPY_KERNEL && engine != TF_SLOT_COPY_DEVICE)
        return fail(TF_E_ARG, "unknown copy engine %d", engine);
    if (engine != TF_SLOT_COPY_DMA && !c->host_dev)
        return fail(TF_E_STATE, "the host pool has no device mapping");
    if (engine == TF_SLOT_COPY_DEVICE && c->P)
        return fail(TF_E_STATE, "the device copy engine does not take prefetch buffers");
    for (int l = 0; l < c->d.L; ++l)
        if (c->pending[l]) return fail(TF_E_STATE, "layer %d: lookup not yet filled", l);
    if (engine == TF_SLOT_COPY_DEVICE && c->ev_dfill.empty()) {
        hipError_t e = hipSuccess;
        c->ev_dfill.assign(c->d.L, nullptr);
        for (int l = 0; l < c->d.L && e == hipSuccess; ++l)
            e = hipEventCreateWithFlags(&c->ev_dfill[l], hipEventDisableTiming);
        if (e != hipSuccess) return fail(TF_E_HIP, "fill events: %s", hipGetErrorString(e));
        c->dfill_pending.assign(c->d.L, 0);
    }
    if (c->engine == TF_SLOT_COPY_DEVICE && engine != TF_SLOT_COPY_DEVICE && c->dfill_any)
        c->mirror.assign(c->mirror.size(), -1);   // device fills kept no host view: assume nothing resident
    c->engine = engine;
    return TF_OK;
}

tf_status tf_slot_cache_prefetch_stats(const tf_slot_cache *c, int64_t *h2d_bytes, int64_t *used,
                                       int64_t *wasted) {
    if (!c) return fail(TF_E_ARG, "NULL cache");
    if (h2d_bytes) *h2d_bytes = c->pf_bytes;
    if (used) *used = c->pf_used;
    if (wasted) *wasted = c->pf_wasted;
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

int64_t tf_slot_cache_bytes_filled(const tf_slot_cache *c) {
    if (!c) return -1;
    if (!c->dfill_any) return c->bytes_filled;
    unsigned long long n = 0;   // device-initiated fills count their blobs on the GPU
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(&n, c->d.nfill, sizeof n, hipMemcpyDeviceToHost) != hipSuccess)
        return -1;
    return c->bytes_filled + (int64_t)n * (int64_t)c->stride;
}

tf_status tf_slot_cache_set_policy(tf_slot_cache *c, int32_t policy) {
    if (!c) return fail(TF_E_ARG, "NULL cache");
    if (policy != TF_SLOT_LFU && policy != TF_SLOT_LRU) return fail(TF_E_ARG, "unknown policy %d", policy);
    c->d.policy = policy;
    return TF_OK;
}

}  // extern "C"
