// Decode-path kernels of the q4 MoE layer for gfx950 (CDNA4).
//
// One decode step of T <= 16 tokens through one layer is three launches on
// one stream (the shilu.ai README translation, "推理引擎的工作原理", orders
// the work as router -> shared branch (overlapping the expert fetch) ->
// routed experts -> combine):
//
//   A  router rows (8-bit, fp64 sums) + shared gate/up (q4)     depends on x
//      the last router wave of a token does its top-k + softmax; the last
//      token's top-k wave groups the (token, rank) pairs by expert
//   B  routed gate/up (q4, per expert group) + shared down (q4)  needs ids, h_s
//   C  routed down (q4) summed over the token's ranks + y_s -> fp16 y
//
// Every wave owns an 8-row tile: lanes 8r..8r+7 share row r, lane s reads the
// 16-byte chunks s, s+8, s+16, ... of the row, so each load instruction moves
// eight full 128-byte lines.  Activations are staged per wave in LDS in the
// (e0,e4)(e1,e5)(e2,e6)(e3,e7) pairing that the nibble unpack produces (see
// tf_device.h).  No float atomics: every sum has a fixed order, so repeated
// runs are bitwise identical.
#include "tf_device.h"
#include "tf_internal.h"

using namespace tfk;

namespace {

struct Mat {
    const uint8_t *q;
    const uint16_t *s;
    const uint16_t *b;
};

__device__ __forceinline__ void blob_mats(const uint8_t *blob, int d, int f, Mat &g, Mat &u,
                                          Mat &dn) {
    const size_t qb = (size_t)f * d / 2, sb = (size_t)f * (d / 64) * 2;
    const size_t dqb = (size_t)d * f / 2, dsb = (size_t)d * (f / 64) * 2;
    const uint8_t *p = blob;
    g.q = p; p += qb;
    g.s = reinterpret_cast<const uint16_t *>(p); p += sb;
    g.b = reinterpret_cast<const uint16_t *>(p); p += sb;
    u.q = p; p += qb;
    u.s = reinterpret_cast<const uint16_t *>(p); p += sb;
    u.b = reinterpret_cast<const uint16_t *>(p); p += sb;
    dn.q = p; p += dqb;
    dn.s = reinterpret_cast<const uint16_t *>(p); p += dsb;
    dn.b = reinterpret_cast<const uint16_t *>(p);
}

__device__ __forceinline__ const uint8_t *expert_blob(const DecodeArgs &a, int e) {
    const int slot = a.slot_map ? (int)a.slot_map[e] : e;
    return a.pool + (size_t)slot * a.stride;
}

// Loads of one 8-row tile of a q4 matrix with K columns: chunk j of lane
// (r, s) is half-group hg = 8j + s of row row0 + r.  Scale and bias of the
// chunk's group are packed into one word (scale low, bias high).
template <int J>
__device__ __forceinline__ void load_tile(const Mat &m, int row0, int K, int lane, uint4 (&q)[J],
                                          uint32_t (&sb)[J]) {
    const int H = K >> 5, G = K >> 6;
    const int r = lane >> 3, s = lane & 7;
    const uint4 *qrow = reinterpret_cast<const uint4 *>(m.q + (size_t)(row0 + r) * (K >> 1));
    const uint16_t *srow = m.s + (size_t)(row0 + r) * G;
    const uint16_t *brow = m.b + (size_t)(row0 + r) * G;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int hg = 8 * j + s;
        if (hg < H) {
            q[j] = qrow[hg];
            sb[j] = (uint32_t)srow[hg >> 1] | ((uint32_t)brow[hg >> 1] << 16);
        } else {
            q[j] = make_uint4(0, 0, 0, 0);
            sb[j] = 0;
        }
    }
}

// Partial dot product of the lane's chunks against a staged fp16 row.
template <int J>
__device__ __forceinline__ float tile_dot_x(const uint4 (&q)[J], const uint32_t (&sb)[J],
                                            const uint4 *xp, const float *xs, int H, int lane) {
    const int s = lane & 7;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int hg = 8 * j + s;
        if (hg < H) {
            const float D = q4_chunk_dot(q[j], xp + hg, xp + H + hg, xp + 2 * H + hg,
                                         xp + 3 * H + hg, 0.f);
            const float sc = h2f((uint16_t)(sb[j] & 0xFFFF)), bi = h2f((uint16_t)(sb[j] >> 16));
            acc = fmaf(sc, D, fmaf(fmaf(-1024.f, sc, bi), xs[hg], acc));
        }
    }
    return acc;
}

// Same against a staged hi/lo pair of fp16 rows (fp32 activation).
template <int J>
__device__ __forceinline__ float tile_dot_hl(const uint4 (&q)[J], const uint32_t (&sb)[J],
                                             const uint4 *hp, const uint4 *lp, const float *xs,
                                             int H, int lane) {
    const int s = lane & 7;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int hg = 8 * j + s;
        if (hg < H) {
            float D = q4_chunk_dot(q[j], hp + hg, hp + H + hg, hp + 2 * H + hg, hp + 3 * H + hg,
                                   0.f);
            D = q4_chunk_dot(q[j], lp + hg, lp + H + hg, lp + 2 * H + hg, lp + 3 * H + hg, D);
            const float sc = h2f((uint16_t)(sb[j] & 0xFFFF)), bi = h2f((uint16_t)(sb[j] >> 16));
            acc = fmaf(sc, D, fmaf(fmaf(-1024.f, sc, bi), xs[hg], acc));
        }
    }
    return acc;
}

// LDS footprint of one staged fp16 row / hi-lo row of K values (bytes).
__host__ __device__ constexpr int x_stage_bytes(int K) { return (2 * K + 4 * (K >> 5) + 15) & ~15; }
__host__ __device__ constexpr int h_stage_bytes(int K) { return (4 * K + 4 * (K >> 5) + 15) & ~15; }

__device__ __forceinline__ void x_stage_ptrs(unsigned char *base, int K, int i, uint4 *&xp,
                                             float *&xs) {
    unsigned char *p = base + (size_t)i * x_stage_bytes(K);
    xp = reinterpret_cast<uint4 *>(p);
    xs = reinterpret_cast<float *>(p + 2 * K);
}

__device__ __forceinline__ void h_stage_ptrs(unsigned char *base, int K, int i, uint4 *&hp,
                                             uint4 *&lp, float *&xs) {
    unsigned char *p = base + (size_t)i * h_stage_bytes(K);
    hp = reinterpret_cast<uint4 *>(p);
    lp = reinterpret_cast<uint4 *>(p + 2 * K);
    xs = reinterpret_cast<float *>(p + 4 * K);
}

__device__ __forceinline__ uint32_t ld_acquire_u32(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- top-k
// Top-k of token t by (logit desc, id asc), or the forced ids; softmax in
// fp64 over the k selected logits (max-subtracted).  One wave.
__device__ void topk_token(const DecodeArgs &a, int t, int lane, unsigned char *lds) {
    double *l = reinterpret_cast<double *>(lds);
    int *sel = reinterpret_cast<int *>(l + a.E);
    __syncthreads();
    for (int i = lane; i < a.E; i += WAVE) {
        const double v = __hip_atomic_load(a.logits + (size_t)t * a.E + i, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        l[i] = (v != v) ? -__builtin_inf() : v;   // NaN ranks last
    }
    __syncthreads();
    if (a.forced) {
        uint32_t flags = 0;
        if (lane < a.k) {
            int id = a.forced[(size_t)t * a.k + lane];
            if (id < 0 || id >= a.E) {
                flags |= TF_FLAG_ID_RANGE;
                id = id < 0 ? 0 : a.E - 1;
            }
            sel[lane] = id;
        }
        __syncthreads();
        if (lane < a.k)
            for (int r = 0; r < lane; ++r)
                if (sel[r] == sel[lane]) flags |= TF_FLAG_ID_REPEAT;
        if (flags) atomicOr(a.hdr + HDR_FLAGS, flags);
    } else {
        // k rounds of a wave-wide argmax over the untaken candidates
        uint32_t taken = 0;   // bit c: candidate lane + 64c taken
        for (int r = 0; r < a.k; ++r) {
            double bv = -__builtin_inf();
            int bi = 0x7FFFFFFF;
            for (int c = 0, i = lane; i < a.E; ++c, i += WAVE) {
                if (taken & (1u << c)) continue;
                const double v = l[i];
                if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
            }
#pragma unroll
            for (int o = 1; o < WAVE; o <<= 1) {
                const double ov = __shfl_xor(bv, o);
                const int oi = __shfl_xor(bi, o);
                if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
            }
            if ((bi & (WAVE - 1)) == lane) taken |= 1u << (bi / WAVE);
            if (lane == 0) sel[r] = bi;
        }
    }
    __syncthreads();
    if (lane == 0) {
        double m = l[sel[0]];
        for (int r = 1; r < a.k; ++r) m = fmax(m, l[sel[r]]);
        double p[16], s = 0.0;
        for (int r = 0; r < a.k; ++r) { p[r] = exp(l[sel[r]] - m); s += p[r]; }
        for (int r = 0; r < a.k; ++r) {
            a.ids[(size_t)t * a.k + r] = sel[r];
            a.weights[(size_t)t * a.k + r] = (float)(p[r] / s);
        }
    }
}

// Group the T*k (token, rank) pairs by expert: pairs sorted by (expert,
// token, rank); items hold at most a.tbx pairs of one expert.  One wave.
__device__ void group_pairs(const DecodeArgs &a, int lane, unsigned char *lds) {
    const int P = a.T * a.k;
    int *pid = reinterpret_cast<int *>(lds);
    int *sorted = pid + P;
    __syncthreads();
    for (int p = lane; p < P; p += WAVE)
        pid[p] = (int)__hip_atomic_load(reinterpret_cast<const uint32_t *>(a.ids) + p,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    for (int p = lane; p < P; p += WAVE) {
        const int e = pid[p];
        int pos = 0;
        for (int q = 0; q < P; ++q) pos += (pid[q] < e) | ((pid[q] == e) & (q < p));
        sorted[pos] = p;
    }
    __syncthreads();
    if (lane == 0) {
        int n = 0;
        for (int i = 0; i < P;) {
            const int e = pid[sorted[i]];
            int j = i + 1;
            while (j < P && j - i < a.tbx && pid[sorted[j]] == e) ++j;
            int *it = a.items + 4 * n;
            it[0] = e; it[1] = i; it[2] = j - i; it[3] = 0;
            ++n;
            i = j;
        }
        a.hdr[HDR_NITEMS] = (uint32_t)n;
    }
    for (int p = lane; p < P; p += WAVE) a.pairs[p] = sorted[p];
}

// ----------------------------------------------------------- router wave
// Logit of expert e for token t: sum over 16-element chunks of
// s_g * sum_i q_i x_i + b_g * sum_i x_i, products and sums in fp64.
__device__ void router_wave(const DecodeArgs &a, int bid, int lane, unsigned char *lds) {
    const int t = bid / a.E, e = bid - t * a.E;
    const int d = a.d, NC = d >> 4, G = d >> 6;
    constexpr int JR = 4;   // d <= 4096
    uint4 qv[JR];
    double sv[JR], bv[JR];
    const uint4 *qrow = reinterpret_cast<const uint4 *>(a.rq + (size_t)e * d);
#pragma unroll
    for (int j = 0; j < JR; ++j) {
        const int c = lane + WAVE * j;
        if (c < NC) {
            qv[j] = qrow[c];
            sv[j] = (double)h2f(a.rs[(size_t)e * G + (c >> 2)]);
            bv[j] = (double)h2f(a.rb[(size_t)e * G + (c >> 2)]);
        }
    }
    double *xd = reinterpret_cast<double *>(lds);
    double *x16 = xd + d;
    const uint4 *xv = reinterpret_cast<const uint4 *>(a.x + (size_t)t * d);
    for (int c = lane; c < NC; c += WAVE) {
        const uint4 v0 = xv[2 * c], v1 = xv[2 * c + 1];
        const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double lo = (double)h2f((uint16_t)(w[i] & 0xFFFF));
            const double hi = (double)h2f((uint16_t)(w[i] >> 16));
            xd[16 * c + 2 * i] = lo;
            xd[16 * c + 2 * i + 1] = hi;
            s += lo + hi;
        }
        x16[c] = s;
    }
    __syncthreads();
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < JR; ++j) {
        const int c = lane + WAVE * j;
        if (c < NC) {
            const uint32_t w[4] = {qv[j].x, qv[j].y, qv[j].z, qv[j].w};
            const double *xx = xd + 16 * c;
            double D = 0.0;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                D = fma((double)((w[i >> 2] >> (8 * (i & 3))) & 0xFF), xx[i], D);
            acc = fma(sv[j], D, fma(bv[j], x16[c], acc));
        }
    }
    acc = wave_sum_f64(acc);
    if (lane == 0) a.logits[(size_t)t * a.E + e] = acc;
    if (!a.topk) return;

    // last router wave of token t: top-k (+ grouping when it is the last token)
    __threadfence();
    uint32_t old = 0;
    if (lane == 0) old = atomicAdd(a.hdr + HDR_TICKET + t, 1u);
    old = __shfl(old, 0);
    if (old != (uint32_t)(a.E - 1)) return;
    __threadfence();
    if (lane == 0) a.hdr[HDR_TICKET + t] = 0;
    topk_token(a, t, lane, lds);
    if (!a.do_group) return;
    __threadfence();
    old = 0;
    if (lane == 0) old = atomicAdd(a.hdr + HDR_TICKET + a.T, 1u);
    old = __shfl(old, 0);
    if (old != (uint32_t)(a.T - 1)) return;
    __threadfence();
    if (lane == 0) a.hdr[HDR_TICKET + a.T] = 0;
    group_pairs(a, lane, lds);
}

// ----------------------------------------------- shared gate/up wave
template <int J>
__device__ void shared_gateup_wave(const DecodeArgs &a, int bid, int lane, unsigned char *lds) {
    const int tiles = a.fs / TILE_ROWS;
    const int tile = bid % tiles, sb = bid / tiles;
    const int t0 = sb * a.tbx, nt = min(a.tbx, a.T - t0);
    const int row0 = tile * TILE_ROWS, H = a.d >> 5;
    Mat g, u, dn;
    blob_mats(a.shared_blob, a.d, a.fs, g, u, dn);
    uint4 qg[J], qu[J];
    uint32_t sg[J], su[J];
    load_tile<J>(g, row0, a.d, lane, qg, sg);
    load_tile<J>(u, row0, a.d, lane, qu, su);
    for (int i = 0; i < nt; ++i) {
        uint4 *xp; float *xs;
        x_stage_ptrs(lds, a.d, i, xp, xs);
        stage_x_f16(a.x + (size_t)(t0 + i) * a.d, a.d, xp, xs, lane);
    }
    __syncthreads();
    for (int i = 0; i < nt; ++i) {
        uint4 *xp; float *xs;
        x_stage_ptrs(lds, a.d, i, xp, xs);
        const float gv = row8_sum(tile_dot_x<J>(qg, sg, xp, xs, H, lane));
        const float uv = row8_sum(tile_dot_x<J>(qu, su, xp, xs, H, lane));
        if ((lane & 7) == 0)
            a.h_s[(size_t)(t0 + i) * a.fs + row0 + (lane >> 3)] = gelu_f(gv, a.act) * uv;
    }
}

// ---------------------------------------------- routed gate/up wave
template <int J>
__device__ void routed_gateup_wave(const DecodeArgs &a, int bid, int lane, unsigned char *lds) {
    const int tiles = a.f / TILE_ROWS;
    const int item = bid / tiles, tile = bid - item * tiles;
    int e, begin, cnt;
    if (a.gemv_slot) {               // standalone GEMV: item = pair
        if (item >= a.P) return;
        e = a.gemv_slot[item]; begin = item; cnt = 1;
    } else {
        if (item >= (int)a.hdr[HDR_NITEMS]) return;
        const int *it = a.items + 4 * item;
        e = it[0]; begin = it[1]; cnt = it[2];
    }
    const int row0 = tile * TILE_ROWS, H = a.d >> 5;
    Mat g, u, dn;
    blob_mats(expert_blob(a, e), a.d, a.f, g, u, dn);
    uint4 qg[J], qu[J];
    uint32_t sg[J], su[J];
    load_tile<J>(g, row0, a.d, lane, qg, sg);
    load_tile<J>(u, row0, a.d, lane, qu, su);
    int prow[4], tok[4];
    for (int i = 0; i < cnt; ++i) {
        if (a.gemv_slot) {
            prow[i] = begin + i;
            tok[i] = a.gemv_token ? a.gemv_token[begin + i] : begin + i;
        } else {
            prow[i] = a.pairs[begin + i];
            tok[i] = prow[i] / a.k;
        }
        uint4 *xp; float *xs;
        x_stage_ptrs(lds, a.d, i, xp, xs);
        stage_x_f16(a.x + (size_t)tok[i] * a.d, a.d, xp, xs, lane);
    }
    __syncthreads();
    for (int i = 0; i < cnt; ++i) {
        uint4 *xp; float *xs;
        x_stage_ptrs(lds, a.d, i, xp, xs);
        const float gv = row8_sum(tile_dot_x<J>(qg, sg, xp, xs, H, lane));
        const float uv = row8_sum(tile_dot_x<J>(qu, su, xp, xs, H, lane));
        if ((lane & 7) == 0)
            a.h_r[(size_t)prow[i] * a.f + row0 + (lane >> 3)] = gelu_f(gv, a.act) * uv;
    }
}

// ------------------------------------------------- shared down wave
template <int J>
__device__ void shared_down_wave(const DecodeArgs &a, int bid, int lane, unsigned char *lds) {
    const int tiles = a.d / TILE_ROWS;
    const int tile = bid % tiles, sb = bid / tiles;
    const int t0 = sb * a.tbh, nt = min(a.tbh, a.T - t0);
    const int row0 = tile * TILE_ROWS, H = a.fs >> 5;
    Mat g, u, dn;
    blob_mats(a.shared_blob, a.d, a.fs, g, u, dn);
    uint4 q[J];
    uint32_t sbw[J];
    load_tile<J>(dn, row0, a.fs, lane, q, sbw);
    for (int i = 0; i < nt; ++i) {
        uint4 *hp, *lp; float *xs;
        h_stage_ptrs(lds, a.fs, i, hp, lp, xs);
        stage_h_f32(a.h_s + (size_t)(t0 + i) * a.fs, 1.f, a.fs, hp, lp, xs, lane);
    }
    __syncthreads();
    for (int i = 0; i < nt; ++i) {
        uint4 *hp, *lp; float *xs;
        h_stage_ptrs(lds, a.fs, i, hp, lp, xs);
        const float v = row8_sum(tile_dot_hl<J>(q, sbw, hp, lp, xs, H, lane));
        if ((lane & 7) == 0) a.y_s[(size_t)(t0 + i) * a.d + row0 + (lane >> 3)] = v;
    }
}

template <int J>
__global__ __launch_bounds__(64) void k_stage_a(DecodeArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int bid = blockIdx.x, lane = threadIdx.x;
    if (bid < a.a_router_waves)
        router_wave(a, bid, lane, lds);
    else
        shared_gateup_wave<J>(a, bid - a.a_router_waves, lane, lds);
}

template <int J>
__global__ __launch_bounds__(64) void k_stage_b(DecodeArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int bid = blockIdx.x, lane = threadIdx.x;
    if (bid < a.b_routed_waves)
        routed_gateup_wave<J>(a, bid, lane, lds);
    else
        shared_down_wave<J>(a, bid - a.b_routed_waves, lane, lds);
}

// ------------------------------------------- routed down + combine wave
// y[t][row] = base[t][row] + sum over the token's pairs (in order) of
//             W_down,e (coef * h_pair)[row]
template <int J>
__global__ __launch_bounds__(64) void k_stage_c(DecodeArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int lane = threadIdx.x;
    const int tiles = a.d / TILE_ROWS;
    const int t = blockIdx.x / tiles, tile = blockIdx.x - t * tiles;
    const int row0 = tile * TILE_ROWS, H = a.f >> 5;
    int lo, hi;
    if (a.gemv_slot) {
        if (a.gemv_token) {           // first pair with token >= t, and > t
            int l0 = 0, h0 = a.P;
            while (l0 < h0) { const int m = (l0 + h0) >> 1; if (a.gemv_token[m] < t) l0 = m + 1; else h0 = m; }
            lo = l0;
            h0 = a.P;
            while (l0 < h0) { const int m = (l0 + h0) >> 1; if (a.gemv_token[m] <= t) l0 = m + 1; else h0 = m; }
            hi = l0;
        } else {
            lo = t; hi = t + 1;
        }
    } else {
        lo = t * a.k; hi = lo + a.k;
    }
    float acc = 0.f;
    for (int p0 = lo; p0 < hi; p0 += a.kcb) {
        const int np = min(a.kcb, hi - p0);
        if (p0 != lo) __syncthreads();
        for (int i = 0; i < np; ++i) {
            const int p = p0 + i;
            const float c = a.gemv_slot ? (a.gemv_coef ? a.gemv_coef[p] : 1.f) : a.weights[p];
            uint4 *hp, *lp; float *xs;
            h_stage_ptrs(lds, a.f, i, hp, lp, xs);
            stage_h_f32(a.h_r + (size_t)p * a.f, c, a.f, hp, lp, xs, lane);
        }
        Mat g, u, dn;
        uint4 q[J], qn[J];
        uint32_t sb[J], sbn[J];
        const int e0 = a.gemv_slot ? a.gemv_slot[p0] : a.ids[p0];
        blob_mats(expert_blob(a, e0), a.d, a.f, g, u, dn);
        load_tile<J>(dn, row0, a.f, lane, q, sb);
        __syncthreads();
        for (int i = 0; i < np; ++i) {
            if (i + 1 < np) {         // issue the next expert's rows before this one's math
                const int p = p0 + i + 1;
                const int e = a.gemv_slot ? a.gemv_slot[p] : a.ids[p];
                blob_mats(expert_blob(a, e), a.d, a.f, g, u, dn);
                load_tile<J>(dn, row0, a.f, lane, qn, sbn);
            }
            uint4 *hp, *lp; float *xs;
            h_stage_ptrs(lds, a.f, i, hp, lp, xs);
            acc += tile_dot_hl<J>(q, sb, hp, lp, xs, H, lane);
#pragma unroll
            for (int j = 0; j < J; ++j) { q[j] = qn[j]; sb[j] = sbn[j]; }
        }
    }
    acc = row8_sum(acc);
    if ((lane & 7) == 0) {
        const size_t o = (size_t)t * a.d + row0 + (lane >> 3);
        if (a.gemv_slot) {
            a.y32[o] = a.y32[o] + acc;
        } else {
            const float y = a.y_s[o] + acc;
            if (a.y32) a.y32[o] = y;
            a.y[o] = f2h(y);
        }
    }
}

__global__ __launch_bounds__(256) void k_zero(uint32_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

template <int J>
hipError_t launch_abc(const DecodeArgs &a, int which, hipStream_t s) {
    if (which & STAGE_A) {
        const int n = a.a_router_waves + a.a_shared_waves;
        if (n) {
            // router x staging, then (reusing it) top-k and grouping scratch
            const int lds_r = max(max(8 * a.d + 8 * (a.d >> 4), 8 * a.E + 4 * 16),
                                  a.do_group ? 8 * a.T * a.k : 0);
            const int lds_s = a.a_shared_waves ? a.tbx * x_stage_bytes(a.d) : 0;
            hipLaunchKernelGGL(k_stage_a<J>, dim3(n), dim3(64), max(lds_r, lds_s), s, a);
        }
    }
    if (which & STAGE_B) {
        const int n = a.b_routed_waves + a.b_shared_waves;
        if (n) {
            const int lds_r = a.b_routed_waves ? a.tbx * x_stage_bytes(a.d) : 0;
            const int lds_s = a.b_shared_waves ? a.tbh * h_stage_bytes(a.fs) : 0;
            hipLaunchKernelGGL(k_stage_b<J>, dim3(n), dim3(64), max(lds_r, lds_s), s, a);
        }
    }
    if (which & STAGE_C) {
        const int n = a.T * (a.d / TILE_ROWS);
        if (n) {
            const int lds = a.kcb * h_stage_bytes(a.f);
            hipLaunchKernelGGL(k_stage_c<J>, dim3(n), dim3(64), lds, s, a);
        }
    }
    return hipGetLastError();
}

}  // namespace

// J = chunks per lane = ceil(K / 256) for the largest K among d, f, fs.
hipError_t tf_launch_decode(const DecodeArgs &a, int which, hipStream_t s) {
    int K = a.d;
    if (a.f > K) K = a.f;
    if (a.fs > K) K = a.fs;
    const int J = (K + 255) / 256;
    switch (J) {
        case 1: return launch_abc<1>(a, which, s);
        case 2: return launch_abc<2>(a, which, s);
        case 3: return launch_abc<3>(a, which, s);
        case 4: return launch_abc<4>(a, which, s);
        case 5: case 6: return launch_abc<6>(a, which, s);
        case 7: case 8: return launch_abc<8>(a, which, s);
        case 9: case 10: case 11: return launch_abc<11>(a, which, s);
        case 12: return launch_abc<12>(a, which, s);
        default: return launch_abc<16>(a, which, s);
    }
}

hipError_t tf_launch_zero(void *p, size_t bytes, hipStream_t s) {
    const size_t n = bytes / 4;
    if (!n) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<uint32_t *>(p), n);
    return hipGetLastError();
}
