// Next-token sampling after the stack, on the GPU (shilu.ai README
// translation, "向模型输入 prompt": temperature, Top-K and Top-P knobs,
// defaults 0.2 / 64 / 0.95, temperature 0 for greedy output).
//
// Steps (the order is a reading; the pages give only the knobs): the top_k
// largest logits of the row, ties to the lower id and NaN ranked as -inf; their
// softmax at the temperature, in fp64 with every sum sequential in rank
// order; the shortest rank prefix whose cumulative probability reaches
// top_p; then the first kept rank whose cumulative probability exceeds u
// times the kept total, u in [0, 1) given per row by the caller.
//
// Selection works on 64-bit keys: the fp32 logit mapped to an unsigned key
// that orders as the value (-0 as +0, NaN as -inf) in the high word and the
// complement of the id in the low word, so the keys of a row are distinct and
// a larger key is a larger logit or the same logit with a lower id.  Key 0
// (below every logit) pads.  Two launches:
//   k_sample_part   one workgroup per 4096-logit slice of a row: the slice's
//                   64 largest keys, sorted, into the workspace;
//   k_sample_final  one workgroup per row: the 64 largest keys of the (at
//                   most 64) slice lists, then the softmax, nucleus and draw
//                   over the first top_k.
// Sorting uses two steps of Batcher's bitonic network on lists of 64 keys
// held one per lane: a sort of each list across the lanes, and the top-64
// merge of two descending lists A and B -- the lane-wise maximum of A and B
// reversed holds the 64 largest keys of both as a bitonic sequence, which six
// compare-exchange rounds sort.  A merge tree takes many lists to one.
// The slice kernel first bounds its 64th largest key from below: the 128
// thread pairs hold 32 keys each, and the 64th largest of the 128 pair maxima
// is at most the 64th largest key.  When at most 512 keys reach that bound
// (about 90 of 4096 for logits in random order) only they are sorted, as
// eight lists; otherwise all 64 lists are.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>

#include "tf_device.h"
#include "tf_internal.h"

void tf_set_error(const char *msg);   // tf_api.cpp

namespace {

using namespace tfk;

constexpr int WGS = 256;             // threads per workgroup (4 waves)
constexpr int PER = 16;              // lists (registers) per wave
constexpr int SLICE = WGS * PER;     // keys per workgroup
constexpr int LIST = 64;             // keys per list (the lane index)
constexpr int MAXK = 64;             // largest top_k
constexpr int MAX_SLICES = 64;       // slices per row (the final kernel's lists)

void tf_sample_error(const char *fmt, ...) {
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    tf_set_error(buf);
}

__device__ __forceinline__ uint64_t logit_key(float v, uint32_t id) {
    uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
    if (v != v) u = 0xFF800000u;                      // NaN ranks as -inf
    const uint32_t k = (u >> 31) ? ~u : (u | 0x80000000u);
    return ((uint64_t)k << 32) | (0xFFFFFFFFu - id);
}
__device__ __forceinline__ float key_value(uint64_t key) {
    const uint32_t k = (uint32_t)(key >> 32);
    return __uint_as_float((k >> 31) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ uint32_t key_id(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)key; }

__device__ __forceinline__ uint64_t join(uint32_t lo, uint32_t hi) { return ((uint64_t)hi << 32) | lo; }

// The key of lane (lane ^ J).
template <int J>
__device__ __forceinline__ uint64_t lane_xor(uint64_t v) {
    const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
    if constexpr (J == 1 || J == 2) {
        constexpr int ctrl = J == 1 ? 0xB1 : 0x4E;    // quad_perm [1,0,3,2] / [2,3,0,1]
        return join((uint32_t)__builtin_amdgcn_update_dpp(0, lo, ctrl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_update_dpp(0, hi, ctrl, 0xF, 0xF, false));
    } else if constexpr (J < 32) {
        constexpr int pat = 0x1F | (J << 10);          // swizzle bit mode: lane ^ J within 32
        return join((uint32_t)__builtin_amdgcn_ds_swizzle(lo, pat),
                    (uint32_t)__builtin_amdgcn_ds_swizzle(hi, pat));
    } else {
        const int addr = (int)((__lane_id() ^ J) << 2);
        return join((uint32_t)__builtin_amdgcn_ds_bpermute(addr, lo),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(addr, hi));
    }
}

// One compare-exchange round at distance J on all n lists: a lane keeps the
// larger key of its pair when take_max.
template <int J, int N>
__device__ __forceinline__ void cx(uint64_t (&v)[N], int n, bool take_max) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (i < n) {
            const uint64_t p = lane_xor<J>(v[i]);
            v[i] = ((v[i] > p) == take_max) ? v[i] : p;
        }
    }
}

// Sort every list of v descending across the lanes.
template <int N>
__device__ __forceinline__ void sort_lists(uint64_t (&v)[N]) {
    const int x = (int)__lane_id();
#define TF_SORT_STAGE(SIZE)                                                     \
    {                                                                           \
        const bool desc = !(x & (SIZE));                                        \
        if constexpr ((SIZE) >= 64) cx<32>(v, N, !(x & 32) == desc);          \
        if constexpr ((SIZE) >= 32) cx<16>(v, N, !(x & 16) == desc);          \
        if constexpr ((SIZE) >= 16) cx<8>(v, N, !(x & 8) == desc);            \
        if constexpr ((SIZE) >= 8) cx<4>(v, N, !(x & 4) == desc);             \
        if constexpr ((SIZE) >= 4) cx<2>(v, N, !(x & 2) == desc);             \
        cx<1>(v, N, !(x & 1) == desc);                                        \
    }
    TF_SORT_STAGE(2) TF_SORT_STAGE(4) TF_SORT_STAGE(8) TF_SORT_STAGE(16) TF_SORT_STAGE(32)
    TF_SORT_STAGE(64)
#undef TF_SORT_STAGE
}

// v[i] = the 64 largest keys of descending lists v[i] and v[i + n], sorted
// descending, for i < n.
template <int N>
__device__ __forceinline__ void merge_half(uint64_t (&v)[N], int n) {
    const int x = (int)__lane_id();
    const int rev = (x ^ 63) << 2;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (i < n) {
            const uint64_t b = v[i + n];
            const uint64_t r = join((uint32_t)__builtin_amdgcn_ds_bpermute(rev, (int)(uint32_t)b),
                                    (uint32_t)__builtin_amdgcn_ds_bpermute(rev, (int)(uint32_t)(b >> 32)));
            v[i] = v[i] > r ? v[i] : r;
        }
    }
    cx<32>(v, n, !(x & 32));
    cx<16>(v, n, !(x & 16));
    cx<8>(v, n, !(x & 8));
    cx<4>(v, n, !(x & 4));
    cx<2>(v, n, !(x & 2));
    cx<1>(v, n, !(x & 1));
}

// The 64 largest keys of the four waves' descending lists `mine`, sorted
// descending, in wave 0 (lane = rank).  Other waves get 0.
__device__ uint64_t merge_waves(uint64_t mine, uint64_t (&lists)[4][LIST]) {
    const int lane = (int)__lane_id(), w = threadIdx.x >> 6;
    lists[w][lane] = mine;
    lds_barrier();
    if (w != 0) return 0;
    uint64_t q[4] = {lists[0][lane], lists[1][lane], lists[2][lane], lists[3][lane]};
    merge_half(q, 2);
    merge_half(q, 1);
    return q[0];
}

// The 64 largest keys of the workgroup's 64 descending lists (v: 16 per
// wave), sorted descending, in wave 0 (lane = rank).  Other waves get 0.
__device__ uint64_t merge_all(uint64_t (&v)[PER], uint64_t (&lists)[4][LIST]) {
    merge_half(v, 8);
    merge_half(v, 4);
    merge_half(v, 2);
    merge_half(v, 1);
    return merge_waves(v[0], lists);
}

struct SliceLds {
    uint64_t gmax[128];          // thread-pair maxima
    uint64_t surv[8 * LIST];     // keys at or above the bound (when at most 512)
    uint64_t lists[4][LIST];     // merge_all's hand-off
    uint64_t tau;
    int wcnt[4];                 // keys at or above the bound per wave
};

// The 64 largest of the workgroup's 4096 keys (v: 16 per thread), sorted,
// in wave 0 (lane = rank); other waves get 0.
__device__ uint64_t slice_top(uint64_t (&v)[PER], SliceLds &L) {
    const int tid = threadIdx.x, lane = (int)__lane_id(), w = tid >> 6;
    uint64_t m = v[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) m = v[i] > m ? v[i] : m;
    const uint64_t mp = lane_xor<1>(m);
    if (!(lane & 1)) L.gmax[tid >> 1] = m > mp ? m : mp;
    lds_barrier();
    if (tid < 128) {   // tau: the pair maximum with fewer than 64 above it
        const uint64_t g0 = L.gmax[tid];
        int gt = 0, ge = 0;
        for (int j = 0; j < 128; j += 8) {
            uint64_t g[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) g[q] = L.gmax[j + q];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                gt += (int)(g[q] > g0);
                ge += (int)(g[q] >= g0);
            }
        }
        if (gt < LIST && ge >= LIST) L.tau = g0;
    }
    lds_barrier();
    const uint64_t tau = L.tau;
    uint64_t bal[PER];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        bal[i] = __ballot(v[i] >= tau && v[i] != 0);
        cnt += __popcll(bal[i]);
    }
    if (lane == 0) L.wcnt[w] = cnt;
    lds_barrier();
    const int S = L.wcnt[0] + L.wcnt[1] + L.wcnt[2] + L.wcnt[3];
    if (S > 8 * LIST) {   // uniform: sort everything
        sort_lists(v);
        return merge_all(v, L.lists);
    }
    int base = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) base += q < w ? L.wcnt[q] : 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const uint64_t mb = bal[i];
        if ((mb >> lane) & 1) {
            const int pos = base + (int)__builtin_amdgcn_mbcnt_hi(
                                       (uint32_t)(mb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mb, 0u));
            L.surv[pos] = v[i];
        }
        base += __popcll(mb);
    }
    for (int j = tid; j < 8 * LIST; j += WGS)   // pad to eight lists
        if (j >= S) L.surv[j] = 0;
    lds_barrier();
    uint64_t q[2] = {L.surv[2 * w * LIST + lane], L.surv[(2 * w + 1) * LIST + lane]};
    sort_lists(q);
    merge_half(q, 1);
    return merge_waves(q[0], L.lists);
}

// One 4096-logit slice of one row: its 64 largest keys, sorted -> cand.
__global__ __launch_bounds__(WGS) void k_sample_part(const float *logits, int V, int nb,
                                                     uint64_t *cand) {
    __shared__ SliceLds L;
    const int b = blockIdx.x, t = blockIdx.y;
    const int lane = (int)__lane_id(), w = threadIdx.x >> 6;
    const float *row = logits + (size_t)t * V + (size_t)b * SLICE;
    const int n = min(SLICE, V - b * SLICE);
    float f[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int j = (w * PER + i) * LIST + lane;
        f[i] = j < n ? row[j] : 0.f;
    }
    uint64_t v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int j = (w * PER + i) * LIST + lane;
        v[i] = j < n ? logit_key(f[i], (uint32_t)(b * SLICE + j)) : 0ull;
    }
    const uint64_t top = slice_top(v, L);
    if (w == 0) cand[((size_t)t * nb + b) * LIST + lane] = top;
}

// Lane r's value of v (r uniform).
__device__ __forceinline__ double lane_read(double v, int r) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, r);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), r);
    return __longlong_as_double((long long)join(lo, hi));
}

// One row: the 64 largest keys of its slice lists, then the draw among the
// first k.
__global__ __launch_bounds__(WGS) void k_sample_final(const uint64_t *cand, int nb, int k,
                                                      double temperature, double top_p,
                                                      const double *u, int32_t *ids) {
    __shared__ uint64_t lists[4][LIST];
    const int t = blockIdx.x;
    const int lane = (int)__lane_id(), w = threadIdx.x >> 6;
    const double ut = temperature != 0.0 ? u[t] : 0.0;
    const uint64_t *c = cand + (size_t)t * nb * LIST;
    uint64_t v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int l = w * PER + i;
        v[i] = l < nb ? c[l * LIST + lane] : 0ull;
    }
    const uint64_t key = merge_all(v, lists);   // wave 0: lane r holds rank r
    if (w != 0) return;
    if (temperature == 0.0) {
        if (lane == 0) ids[t] = (int32_t)key_id(key);
        return;
    }
    // softmax at the temperature (fp64): the exps and quotients in parallel,
    // the sum and the cumulative sum in rank order through lane reads
    const bool act = lane < k;
    const double l0 = lane_read((double)key_value(key), 0);
    const double e = act ? exp(((double)key_value(key) - l0) / temperature) : 0.0;
    double s = 0.0;
    for (int r = 0; r < k; ++r) s += lane_read(e, r);
    const double q = e / s;
    double acc = 0.0, cum = 0.0;
    for (int r = 0; r < k; ++r) {
        acc += lane_read(q, r);
        cum = lane == r ? acc : cum;
    }
    const uint64_t reach = __ballot(act && cum >= top_p);
    const int keep = reach ? __ffsll((unsigned long long)reach) : k;   // kept ranks
    const double target = ut * lane_read(cum, keep - 1);
    const uint64_t over = __ballot(lane < keep && cum > target);
    const int pick = over ? __ffsll((unsigned long long)over) - 1 : keep - 1;
    const uint64_t chosen = join((uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key, pick),
                                 (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(key >> 32), pick));
    if (lane == 0) ids[t] = (int32_t)key_id(chosen);
}

size_t slices(int V) { return ((size_t)V + SLICE - 1) / SLICE; }

}  // namespace

extern "C" {

size_t tf_sample_workspace_bytes(int32_t V, int32_t T, int32_t top_k) {
    (void)top_k;
    if (V <= 0 || T <= 0) return 256;
    return (size_t)T * slices(V) * LIST * 8;
}

tf_status tf_sample(const float *logits, int32_t V, int32_t T, float temperature, int32_t top_k,
                    float top_p, const double *u, int32_t *ids, void *ws, size_t ws_bytes,
                    hipStream_t s) {
    if (T < 0 || T > 4096) { tf_sample_error("T must be in [0, 4096]"); return TF_E_ARG; }
    if (T == 0) return TF_OK;
    if (!logits || !ids || !ws || (temperature != 0.f && !u)) {
        tf_sample_error("NULL logits, ids or ws, or NULL u with a nonzero temperature");
        return TF_E_ARG;
    }
    if (top_k < 1 || top_k > MAXK || V < top_k) {
        tf_sample_error("need 1 <= top_k <= %d and top_k <= V", MAXK);
        return TF_E_SHAPE;
    }
    if (slices(V) > (size_t)MAX_SLICES) {
        tf_sample_error("V must be at most %d", MAX_SLICES * SLICE);
        return TF_E_SHAPE;
    }
    if (!(temperature >= 0.f) || !(top_p > 0.f && top_p <= 1.f)) {
        tf_sample_error("need temperature >= 0 and 0 < top_p <= 1");
        return TF_E_ARG;
    }
    if ((reinterpret_cast<uintptr_t>(logits) & 3) || (reinterpret_cast<uintptr_t>(ws) & 255)) {
        tf_sample_error("logits 4-byte, ws 256-byte alignment");
        return TF_E_ALIGN;
    }
    if (ws_bytes < tf_sample_workspace_bytes(V, T, top_k)) {
        tf_sample_error("workspace too small");
        return TF_E_NOMEM;
    }
    const int nb = (int)slices(V);
    uint64_t *cand = reinterpret_cast<uint64_t *>(ws);
    TF_LAUNCH(TF_KERNEL_SAMPLE_PART, k_sample_part, dim3(nb, T), dim3(WGS), 0, s, logits, V, nb, cand);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) {
        TF_LAUNCH(TF_KERNEL_SAMPLE_FINAL, k_sample_final, dim3(T), dim3(WGS), 0, s, cand, nb, top_k,
                  (double)temperature, (double)top_p, u, ids);
        e = hipGetLastError();
    }
    if (e != hipSuccess) {
        tf_sample_error("sampling launch: %s", hipGetErrorString(e));
        return TF_E_HIP;
    }
    return TF_OK;
}

}  // extern "C"
