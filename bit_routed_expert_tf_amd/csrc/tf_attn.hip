// Decode attention of one new token over an fp16 key/value store (shilu.ai
// README translation, "状态和范围": fp16 KV storage, a bounded ring for the
// sliding-window layers and linear storage for the full-attention layers,
// exact split-K/V decode attention).
//
// Store: k_cache, v_cache [G][S][D] fp16.  A sliding-window layer keeps its
// last S tokens in a ring (token p in slot p % S); a full layer keeps token p
// in slot p (p < S).  Before the ring wraps, slot = token in both, and after
// it every slot holds one of the last S tokens, so the tokens a layer sees
// are always slots [0, min(pos + 1, S)) -- attention does not depend on
// their order.
//
// Two launches:
//   k_attn_chunk    grid (chunks of CH slots, G; CH = 64 when the layer sees
//                   more than 2,048 tokens, else 32): one workgroup per chunk
//                   of one key/value head serves all R = H / G query heads of
//                   it from one read of the chunk's keys and values.  The chunk
//                   holding the new token's slot writes k_new / v_new there
//                   and uses them directly.  Out: per query head the chunk's
//                   score maximum m, sum of exp(s - m), and sum of
//                   exp(s - m) v (fp32).
//   k_attn_combine  per (query head, 32 columns): the exact merge
//                   M = max m_c, L = sum l_c e^(m_c - M),
//                   out = sum o_c e^(m_c - M) / L, taken as an online merge
//                   over chunk groups.
// Scores are fp32 sums of exact fp16 products (fdot2); exp and the sums are
// fp32.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>

#include "tf_device.h"
#include "tf_internal.h"

void tf_set_error(const char *msg);   // tf_api.cpp

namespace {

using namespace tfk;

constexpr int WGS = 256;
constexpr int LONG_SEEN = 2048;        // above this many seen tokens, 64-slot chunks

tf_status fail(tf_status st, const char *fmt, ...) {
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    tf_set_error(buf);
    return st;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ float h2f_lo(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFF)); }
__device__ __forceinline__ float h2f_hi(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16)); }

// 8-element fp16 dot product, fp32 accumulation of exact products.
__device__ __forceinline__ float dot8(uint4 a, uint4 b) {
    float s = __builtin_amdgcn_fdot2(as_h2(a.x), as_h2(b.x), 0.f, false);
    s = __builtin_amdgcn_fdot2(as_h2(a.y), as_h2(b.y), s, false);
    s = __builtin_amdgcn_fdot2(as_h2(a.z), as_h2(b.z), s, false);
    return __builtin_amdgcn_fdot2(as_h2(a.w), as_h2(b.w), s, false);
}

// Partial results of one chunk: per (g, chunk, r) the max, the sum and D sums.
struct Parts {
    float *m, *l, *o;   // [G][NC][R], [G][NC][R], [G][NC][R][D]
};

// D: head dim; R: query heads per key/value head.  Thread t holds column
// block cb = t % CPR (8 fp16 of a row) of rows r0 + RPI * i.
template <int D, int R, int CH>
__global__ __launch_bounds__(WGS) void k_attn_chunk(const uint16_t *q, const uint16_t *k_new,
                                                    const uint16_t *v_new, uint16_t *k_cache,
                                                    uint16_t *v_cache, int S, int n_valid,
                                                    int new_slot, float scale, int NC, Parts P) {
    constexpr int CPR = D / 8, RPI = WGS / CPR, IT = CH / RPI;
    static_assert(CH % RPI == 0 && R <= 4, "layout");
    __shared__ float sc[R][CH];
    __shared__ float red[RPI][R][D];
    const int c = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
    const int cb = tid % CPR, r0 = tid / CPR;
    const size_t row0 = (size_t)g * S;
    const uint4 *kc = reinterpret_cast<const uint4 *>(k_cache) + row0 * CPR;
    const uint4 *vc = reinterpret_cast<const uint4 *>(v_cache) + row0 * CPR;
    // every key and value block of this thread in flight at once
    uint4 kv[IT], vv[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int j = c * CH + r0 + RPI * i;
        const int jj = j < n_valid ? j : 0;
        kv[i] = kc[(size_t)jj * CPR + cb];
        vv[i] = vc[(size_t)jj * CPR + cb];
    }
    uint4 qv[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        qv[r] = reinterpret_cast<const uint4 *>(q)[(size_t)(g * R + r) * CPR + cb];
    const uint4 kn = reinterpret_cast<const uint4 *>(k_new)[(size_t)g * CPR + cb];
    const uint4 vn = reinterpret_cast<const uint4 *>(v_new)[(size_t)g * CPR + cb];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        if (c * CH + r0 + RPI * i == new_slot) {   // the new token: use and store it
            kv[i] = kn;
            vv[i] = vn;
            reinterpret_cast<uint4 *>(k_cache)[(row0 + new_slot) * CPR + cb] = kn;
            reinterpret_cast<uint4 *>(v_cache)[(row0 + new_slot) * CPR + cb] = vn;
        }
    }
    // scores: partial dots over this thread's 8 columns, summed over the CPR
    // threads of the row (consecutive lanes)
    float part[IT][R];
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int r = 0; r < R; ++r) part[i][r] = dot8(qv[r], kv[i]);
#pragma unroll
    for (int off = 1; off < CPR; off <<= 1)
#pragma unroll
        for (int i = 0; i < IT; ++i)
#pragma unroll
            for (int r = 0; r < R; ++r) part[i][r] += __shfl_xor(part[i][r], off, 64);
    if (cb == 0) {
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int jl = r0 + RPI * i;
            const bool ok = c * CH + jl < n_valid;
#pragma unroll
            for (int r = 0; r < R; ++r) sc[r][jl] = ok ? part[i][r] * scale : -INFINITY;
        }
    }
    lds_barrier();
    // chunk softmax statistics: wave r handles query head r (CH <= 64 lanes)
    const int lane = tid & 63, w = tid >> 6;
    if (w < R) {
        const float s = lane < CH ? sc[w][lane] : -INFINITY;
        float m = s;
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        const float p = lane < CH ? __expf(s - m) : 0.f;
        float l = p;
        for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off, 64);
        if (lane < CH) sc[w][lane] = p;
        if (lane == 0) {
            const size_t pi = ((size_t)g * NC + c) * R + w;
            P.m[pi] = m;
            P.l[pi] = l;
        }
    }
    lds_barrier();
    // weighted values: this thread's 8 columns over its rows, then summed over
    // the RPI row groups through LDS
    float acc[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int jl = r0 + RPI * i;
        const uint32_t w4[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float p = sc[r][jl];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[r][2 * e] = fmaf(p, h2f_lo(w4[e]), acc[r][2 * e]);
                acc[r][2 * e + 1] = fmaf(p, h2f_hi(w4[e]), acc[r][2 * e + 1]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[r0][r][cb * 8 + e] = acc[r][e];
    lds_barrier();
    for (int x = tid; x < R * D; x += WGS) {
        const int r = x / D, d = x % D;
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < RPI; ++k) s += red[k][r][d];
        P.o[(((size_t)g * NC + c) * R + r) * D + d] = s;
    }
}

// Merge of the NC chunk results of query head h = g * R + r over 32 of its
// columns (grid (D / 32, H)): thread (d, cg) runs an online merge over the
// chunks c = cg, cg + 8, ... (running maximum, rescaled sum and column
// value), 16 (above 64 chunks) or 4 chunks' loads at a time, then the 8
// chunk groups merge through LDS:
// M = max m_c, L = sum l_c e^(m_c - M), out = sum o_c e^(m_c - M) / L.
constexpr int CMB_D = 32, CMB_G = WGS / CMB_D;
template <int CMB_U>   // chunks per thread in flight: 16 above 64 chunks, else 4
__global__ __launch_bounds__(WGS) void k_attn_combine(int D, int R, int NC, Parts P, float *out) {
    __shared__ float sm[CMB_G][CMB_D], sl[CMB_G][CMB_D], so[CMB_G][CMB_D];
    const int h = blockIdx.y, g = h / R, r = h % R;
    const int dl = threadIdx.x % CMB_D, cg = threadIdx.x / CMB_D;
    const int d = blockIdx.x * CMB_D + dl;
    float m = -INFINITY, l = 0.f, o = 0.f;
    for (int c0 = cg; c0 < NC; c0 += CMB_U * CMB_G) {
        float mc[CMB_U], lc[CMB_U], oc[CMB_U];
#pragma unroll
        for (int u = 0; u < CMB_U; ++u) {   // CMB_U chunks' loads in flight
            const int c = c0 + u * CMB_G;
            const size_t pi = ((size_t)g * NC + (c < NC ? c : 0)) * R + r;
            mc[u] = c < NC ? P.m[pi] : -INFINITY;
            lc[u] = c < NC ? P.l[pi] : 0.f;
            oc[u] = c < NC ? P.o[pi * D + d] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < CMB_U; ++u) {
            const float mn = fmaxf(m, mc[u]);
            if (mn == -INFINITY) continue;
            const float a = __expf(m - mn), b = __expf(mc[u] - mn);
            l = l * a + lc[u] * b;
            o = o * a + oc[u] * b;
            m = mn;
        }
    }
    sm[cg][dl] = m;
    sl[cg][dl] = l;
    so[cg][dl] = o;
    lds_barrier();
    if (cg == 0) {
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < CMB_G; ++k) M = fmaxf(M, sm[k][dl]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int k = 0; k < CMB_G; ++k) {
            const float f = sm[k][dl] == -INFINITY ? 0.f : __expf(sm[k][dl] - M);
            L = fmaf(sl[k][dl], f, L);
            O = fmaf(so[k][dl], f, O);
        }
        out[(size_t)h * D + d] = O / L;
    }
}

int chunk_slots(int n_valid) { return n_valid > LONG_SEEN ? 64 : 32; }
size_t chunks(int n, int ch) { return ((size_t)n + ch - 1) / ch; }
size_t up256(size_t n) { return (n + 255) & ~size_t(255); }

template <int D, int CH>
hipError_t launch_chunks(int R, dim3 grid, const uint16_t *q, const uint16_t *kn, const uint16_t *vn,
                         uint16_t *kc, uint16_t *vc, int S, int n_valid, int slot, float scale, int NC,
                         Parts P, hipStream_t s) {
    switch (R) {
    case 1: TF_LAUNCH(TF_KERNEL_ATTN_CHUNK, (k_attn_chunk<D, 1, CH>), grid, dim3(WGS), 0, s, q, kn, vn, kc, vc, S, n_valid, slot, scale, NC, P); break;
    case 2: TF_LAUNCH(TF_KERNEL_ATTN_CHUNK, (k_attn_chunk<D, 2, CH>), grid, dim3(WGS), 0, s, q, kn, vn, kc, vc, S, n_valid, slot, scale, NC, P); break;
    case 4: TF_LAUNCH(TF_KERNEL_ATTN_CHUNK, (k_attn_chunk<D, 4, CH>), grid, dim3(WGS), 0, s, q, kn, vn, kc, vc, S, n_valid, slot, scale, NC, P); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

extern "C" {

size_t tf_attn_workspace_bytes(int32_t H, int32_t D, int32_t S) {
    if (H <= 0 || D <= 0 || S <= 0) return 256;
    const size_t n = (size_t)H * chunks(S, 32);   // the most chunks a call on this store uses
    return 2 * up256(4 * n) + up256(4 * n * D);
}

tf_status tf_attn_decode(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                         uint16_t *k_cache, uint16_t *v_cache, int32_t H, int32_t G, int32_t D,
                         int32_t S, int32_t pos, int32_t ring, float scale, float *out, void *ws,
                         size_t ws_bytes, hipStream_t s) {
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !out || !ws)
        return fail(TF_E_ARG, "NULL argument");
    if (D != 64 && D != 128 && D != 256) return fail(TF_E_SHAPE, "D must be 64, 128 or 256");
    if (G < 1 || H < G || H % G || (H / G != 1 && H / G != 2 && H / G != 4) || H > 1024)
        return fail(TF_E_SHAPE, "H must be G, 2G or 4G (H <= 1024)");
    if (S < 1 || S > (1 << 20)) return fail(TF_E_SHAPE, "S must be in [1, 2^20]");
    if (pos < 0 || (!ring && pos >= S)) return fail(TF_E_ARG, "pos must be >= 0 (and < S for a linear store)");
    if (!(scale > 0.f)) return fail(TF_E_ARG, "scale must be > 0");
    const uintptr_t a = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_new) |
                        reinterpret_cast<uintptr_t>(v_new) | reinterpret_cast<uintptr_t>(k_cache) |
                        reinterpret_cast<uintptr_t>(v_cache);
    if ((a & 15) || (reinterpret_cast<uintptr_t>(ws) & 255))
        return fail(TF_E_ALIGN, "q, k/v and caches 16-byte, ws 256-byte aligned");
    if (ws_bytes < tf_attn_workspace_bytes(H, D, S)) return fail(TF_E_NOMEM, "workspace too small");
    const int R = H / G;
    const int n_valid = pos + 1 < S ? pos + 1 : S;
    const int slot = ring ? pos % S : pos;
    const int ch = chunk_slots(n_valid);
    const int NC = (int)chunks(n_valid, ch);
    const size_t n = (size_t)H * chunks(S, 32);
    Parts P;
    P.m = reinterpret_cast<float *>(ws);
    P.l = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(ws) + up256(4 * n));
    P.o = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(ws) + 2 * up256(4 * n));
    const dim3 grid(NC, G);
    hipError_t e;
#define TF_ATTN_CHUNKS(DD, CC) \
    launch_chunks<DD, CC>(R, grid, q, k_new, v_new, k_cache, v_cache, S, n_valid, slot, scale, NC, P, s)
    if (ch == 64) {
        switch (D) {
        case 64: e = TF_ATTN_CHUNKS(64, 64); break;
        case 128: e = TF_ATTN_CHUNKS(128, 64); break;
        default: e = TF_ATTN_CHUNKS(256, 64); break;
        }
    } else {
        switch (D) {
        case 64: e = TF_ATTN_CHUNKS(64, 32); break;
        case 128: e = TF_ATTN_CHUNKS(128, 32); break;
        default: e = TF_ATTN_CHUNKS(256, 32); break;
        }
    }
#undef TF_ATTN_CHUNKS
    if (e == hipSuccess) {
        if (NC > 64)
            TF_LAUNCH(TF_KERNEL_ATTN_COMBINE, k_attn_combine<16>, dim3(D / CMB_D, H), dim3(WGS), 0, s, D, R, NC, P, out);
        else
            TF_LAUNCH(TF_KERNEL_ATTN_COMBINE, k_attn_combine<4>, dim3(D / CMB_D, H), dim3(WGS), 0, s, D, R, NC, P, out);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return fail(TF_E_HIP, "attention launch: %s", hipGetErrorString(e));
    return TF_OK;
}

}  // extern "C"
