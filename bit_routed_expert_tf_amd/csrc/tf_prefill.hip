// Prefill GEMMs of the q4 MoE layer on the gfx950 matrix cores.
//
// A prefill chunk has at most 128 tokens, so one fetched expert serves
// several rows (shilu.ai README translation, "推理引擎的工作原理").  With
// about 8 tokens per routed expert and all tokens on the shared expert, the
// vector path is bound by its ALU, so these GEMMs use
// v_mfma_f32_16x16x32_f16 (D[16 rows][16 tokens] += A[16][32] B[32][16]):
//
//   A  16 weight rows x 32 k: the 4-bit codes as exact fp16 integers.  One
//      AND-OR against the exponent pattern of 1024.0 gives 1024+q (low
//      nibble) or 1024+16q (high nibble, left in place); one packed add of
//      -1024, or one packed multiply-add by 1/16 and -64, turns that into q.
//      Every step is exact.
//   B  32 k x 16 tokens: activations staged in LDS in the pairing the unpack
//      produces, (e0,e4)(e1,e5)(e2,e6)(e3,e7), so A's and B's per-lane k
//      orders agree.
//
// Lane l feeds row (or token) l % 16 with k block l / 16.  Lane block b of
// step t takes k = 64g + 16b + 8t + [0, 8), so the two steps of group g
// cover its 64 columns exactly and the group's sum D_g = sum_k q x is
// complete before its scale and bias apply:
//     y += s_g * D_g + b_g * X_g,      X_g = sum of the group's activations.
// Products are exact, sums fp32.  Down projections read the hidden rows as
// hi/lo fp16 pairs: one MFMA for each.
//
// Work: a block owns 32 rows of gate and of up (gate/up: waves 0/1 gate,
// 2/3 up) or 64 rows of down, for one tile of at most 16 tokens -- an expert
// item (routed) or 16 consecutive tokens (shared).  K goes through LDS in
// chunks of 8 groups; each lane's weight codes stream through an 8-group
// register ring that runs one chunk ahead.
#include "tf_device.h"
#include "tf_internal.h"
#include "tf_layer.h"

using namespace tfk;

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int MM_TOK = 16;   // tokens per tile (the MFMA's N)
constexpr int KCH = 8;       // groups per staged K chunk (512 columns)

// The 8 codes of one word as exact fp16 integers, in the pair order above
// (plain expressions: the compiler forms v_and_or_b32 and may interleave
// the unpacks with the LDS reads and MFMAs of neighbouring groups).
__device__ __forceinline__ half8 unpack_q(uint32_t v) {
    const h2_t lo_off = {(_Float16)-1024.f, (_Float16)-1024.f};
    const h2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2_t hi_off = {(_Float16)-64.f, (_Float16)-64.f};
    const uint32_t v8 = v >> 8;
    const h2_t a = __builtin_bit_cast(h2_t, (v & M_LO) | MAGIC) + lo_off;      // (e0,e4)
    const h2_t b = __builtin_bit_cast(h2_t, (v & M_HI) | MAGIC) * sixteenth + hi_off;  // (e1,e5)
    const h2_t c = __builtin_bit_cast(h2_t, (v8 & M_LO) | MAGIC) + lo_off;     // (e2,e6)
    const h2_t d = __builtin_bit_cast(h2_t, (v8 & M_HI) | MAGIC) * sixteenth + hi_off; // (e3,e7)
    const u32x4 w = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                     __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
    return __builtin_bit_cast(half8, w);
}

__device__ __forceinline__ half8 as_half8(uint4 v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    return __builtin_bit_cast(half8, w);
}

__device__ __forceinline__ f32x4 mfma(half8 a, half8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// LDS of one block (bytes): token lists, staged activations (hi and, for
// down projections, lo), half-group sums, scale/bias table, gate/up results.
struct MMLds {
    int src[MM_TOK], dst[MM_TOK];
    float coef[MM_TOK];
    int nt;
    // rows padded by one element: the 16 tokens a B-operand read touches
    // then fall on different LDS banks
    uint4 xs[2][MM_TOK][4 * 2 * KCH + 1];   // [hi/lo][token][8-value block of the chunk]
    float xh[MM_TOK][2 * KCH + 1];          // [token][half-group of the chunk]
    uint32_t sbt[KCH][64];               // [group of the chunk][row]: scale | bias << 16
    float out[2][32][MM_TOK];            // gate/up results
};

// One tile: DOWN = false -> gate/up rows [32 rt, +32) of the expert with
// blob `blob` (F rows, K = d) into hidden rows; DOWN = true -> down rows
// [64 rt, +64) (d rows, K = F) into fp32 output rows.
template <bool DOWN>
__device__ void mm_tile(const DecodeArgs &a, const uint8_t *blob, int F, int rt, MMLds &L,
                        const uint16_t *x, const uint4 *hsrc, uint4 *hdst, float *ydst) {
    const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
    const int j = lane & 15, b = lane >> 4;
    const int d = a.d;
    const int K = DOWN ? F : d, G = K >> 6, H = K >> 5;
    Mat mg, mu, md;
    blob_mats(blob, d, F, mg, mu, md);
    const Mat &mm = DOWN ? md : ((w >> 1) ? mu : mg);
    const int r0 = DOWN ? 64 * rt + 16 * w : 32 * rt + 16 * (w & 1);   // first row of the wave
    const uint8_t *qrow = mm.q + (size_t)(r0 + j) * (K >> 1) + 8 * b;
    // 8-group ring of this lane's codes (8 bytes per group), one chunk ahead
    uint2 rb[KCH];
#pragma unroll
    for (int i = 0; i < KCH; ++i)
        rb[i] = *reinterpret_cast<const uint2 *>(qrow + 32 * min(i, G - 1));
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int nt = L.nt;
    const int nch = (G + KCH - 1) / KCH;
    // Staging of chunk c: thread (token tj, half-group hh) moves 32 values;
    // loads into registers first (prefetch), LDS stores later, so that the
    // next chunk's loads fly while this chunk computes.  Their loads are
    // issued before the chunk's ring loads: waiting for them never waits
    // for the weights.
    const int tj = tid >> 4, hh = tid & 15;
    const int src = L.src[min(tj, nt - 1)];
    struct Pre { uint4 hv[4], lv[DOWN ? 4 : 1]; float2 ps[DOWN ? 4 : 1]; uint32_t sb[2]; };
    auto fetch = [&](Pre &P, int c) {
        const int HG = 2 * KCH * c + hh, hg = min(HG, H - 1);
        if (!DOWN) {
            const uint4 *xr = reinterpret_cast<const uint4 *>(x + (size_t)src * d);
#pragma unroll
            for (int m = 0; m < 4; ++m) P.hv[m] = xr[4 * hg + m];
        } else {
            const uint4 *hr = hsrc + (size_t)src * 10 * H;
#pragma unroll
            for (int m = 0; m < 4; ++m) { P.hv[m] = hr[m * H + hg]; P.lv[DOWN ? m : 0] = hr[4 * H + m * H + hg]; }
            const float2 *ps = reinterpret_cast<const float2 *>(hr + 8 * H + 2 * hg);
#pragma unroll
            for (int m = 0; m < 4; ++m) P.ps[DOWN ? m : 0] = ps[m];
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int e = tid + 256 * q, gl = e >> 6, row = e & 63, g = min(KCH * c + gl, G - 1);
            const Mat &ms = DOWN ? md : (row < 32 ? mg : mu);
            const int rr = DOWN ? 64 * rt + row : 32 * rt + (row & 31);
            P.sb[q] = (uint32_t)ms.s[(size_t)rr * G + g] | ((uint32_t)ms.b[(size_t)rr * G + g] << 16);
        }
    };
    auto store = [&](const Pre &P, int c) {
        const bool ok = 2 * KCH * c + hh < H;
        float sum = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint4 v = ok ? P.hv[m] : make_uint4(0, 0, 0, 0);
            if (!DOWN) {
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sum += h2f((uint16_t)(w4[e] & 0xFFFF)) + h2f((uint16_t)(w4[e] >> 16));
                L.xs[0][tj][4 * hh + m] = pair_halves(v);
            } else {
                L.xs[0][tj][4 * hh + m] = v;
                L.xs[1][tj][4 * hh + m] = ok ? P.lv[DOWN ? m : 0] : make_uint4(0, 0, 0, 0);
            }
        }
        if (DOWN && ok) sum = ((P.ps[0].x + P.ps[DOWN ? 1 : 0].x) + P.ps[DOWN ? 2 : 0].x) + P.ps[DOWN ? 3 : 0].x;
        L.xh[tj][hh] = sum;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int e = tid + 256 * q, gl = e >> 6, row = e & 63;
            L.sbt[gl][row] = KCH * c + gl < G ? P.sb[q] : 0u;
        }
    };
    Pre P;
    fetch(P, 0);
    store(P, 0);
    const int trow = DOWN ? 16 * w : 16 * (w & 1) + 32 * (w >> 1);   // wave's rows in sbt
    for (int c = 0; c < nch; ++c) {
        __syncthreads();   // chunk c is staged
        const bool more = c + 1 < nch;   // uniform
        if (more) fetch(P, c + 1);
#pragma unroll
        for (int gi = 0; gi < KCH; ++gi) {
            const uint2 wv = rb[gi];
            rb[gi] = *reinterpret_cast<const uint2 *>(qrow + 32 * min(KCH * (c + 1) + gi, G - 1));
            const half8 a0 = unpack_q(wv.x), a1 = unpack_q(wv.y);
            f32x4 D = {0.f, 0.f, 0.f, 0.f};
            D = mfma(a0, as_half8(L.xs[0][j][8 * gi + 2 * b]), D);
            D = mfma(a1, as_half8(L.xs[0][j][8 * gi + 2 * b + 1]), D);
            if (DOWN) {
                D = mfma(a0, as_half8(L.xs[1][j][8 * gi + 2 * b]), D);
                D = mfma(a1, as_half8(L.xs[1][j][8 * gi + 2 * b + 1]), D);
            }
            const uint4 sb4 = *reinterpret_cast<const uint4 *>(&L.sbt[gi][trow + 4 * b]);
            const float Xg = L.xh[j][2 * gi] + L.xh[j][2 * gi + 1];
            const uint32_t s4[4] = {sb4.x, sb4.y, sb4.z, sb4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[r] = fmaf(h2f((uint16_t)(s4[r] & 0xFFFF)), D[r],
                              fmaf(h2f((uint16_t)(s4[r] >> 16)), Xg, acc[r]));
        }
        if (more) {
            __syncthreads();   // everyone is done reading chunk c
            store(P, c + 1);
        }
    }
    if (DOWN) {   // lane (token j, rows 4b + r)
        if (j < nt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) ydst[(size_t)L.dst[j] * d + r0 + 4 * b + r] = acc[r];
        }
        return;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) L.out[w >> 1][16 * (w & 1) + 4 * b + r][j] = acc[r];
    __syncthreads();
    if (tid < 4 * MM_TOK) {   // (token, 8-row block): h = coef * gelu(g) * u
        const int tj = tid >> 2, sub = tid & 3;
        if (tj < nt) {
            float ev[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                ev[q] = L.coef[tj] * (gelu_f(L.out[0][8 * sub + q][tj], a.act) *
                                      L.out[1][8 * sub + q][tj]);
            hs_produce(hdst + (size_t)L.dst[tj] * (10 * (F >> 5)), F, 4 * rt + sub, ev);
        }
    }
}

// Token list of a tile: routed item (expert, up to 16 pairs) or 16 shared
// tokens.  Returns the expert (-1: the shared expert, -2: nothing to do).
__device__ int mm_tokens(const DecodeArgs &a, bool routed, bool down, int tile, MMLds &L) {
    const int tid = threadIdx.x;
    int e = -1;
    if (routed) {
        if (tile >= (int)ld_dev(a.hdr + HDR_NITEMS)) return -2;
        const uint4 it = ld_dev(reinterpret_cast<const uint4 *>(a.items + ITEM_INTS * tile));
        e = (int)it.x;
        if (tid == 0) L.nt = (int)it.z;
        if (tid < MM_TOK) {
            const int pr = ld_dev(a.pairs + (int)it.y + min(tid, (int)it.z - 1));
            L.src[tid] = down ? pr : pr / a.k;
            L.dst[tid] = pr;
            L.coef[tid] = ld_dev(a.weights + pr);
        }
    } else {
        const int t0 = tile * MM_TOK;
        if (tid == 0) L.nt = min(MM_TOK, a.T - t0);
        if (tid < MM_TOK) {
            L.src[tid] = L.dst[tid] = min(t0 + tid, a.T - 1);
            L.coef[tid] = 1.f;
        }
    }
    __syncthreads();
    return e;
}

// Gate/up of the shared expert (blocks [0, a_shared_blocks)) and of the
// routed expert items (the rest).
__global__ __launch_bounds__(256, 2) void k_mm_gateup(DecodeArgs a) {
    __shared__ MMLds L;
    int b = blockIdx.x;
    const bool routed = b >= a.a_shared_blocks;
    if (routed) b -= a.a_shared_blocks;
    const int F = routed ? a.f : a.fs, tiles = F / 32;
    const int e = mm_tokens(a, routed, false, b / tiles, L);
    if (e == -2) return;
    mm_tile<false>(a, routed ? expert_blob(a, e) : a.shared_blob, F, b % tiles, L, a.x, nullptr,
                   routed ? a.h_r : a.h_s, nullptr);
}

// Down of the shared expert (-> y_s) and of the routed expert items (-> y_e).
__global__ __launch_bounds__(256, 2) void k_mm_down(DecodeArgs a) {
    __shared__ MMLds L;
    int b = blockIdx.x;
    const bool routed = b >= a.b_shared_blocks;
    if (routed) b -= a.b_shared_blocks;
    const int F = routed ? a.f : a.fs, tiles = a.d / 64;
    const int e = mm_tokens(a, routed, true, b / tiles, L);
    if (e == -2) return;
    mm_tile<true>(a, routed ? expert_blob(a, e) : a.shared_blob, F, b % tiles, L, nullptr,
                  routed ? a.h_r : a.h_s, nullptr, routed ? a.y_e : a.y_s);
}

}  // namespace

// Prefill after the router launch (top-k and grouping into items of at
// most 16 tokens): gate/up, down, then the combine.
hipError_t tf_launch_prefill_mfma(const DecodeArgs &a0, int max_items, hipStream_t s) {
    DecodeArgs a = a0;
    const int ttiles = (a.T + MM_TOK - 1) / MM_TOK;
    a.a_shared_blocks = ttiles * (a.fs / 32);
    const int n_gu = a.a_shared_blocks + max_items * (a.f / 32);
    TF_LAUNCH(TF_KERNEL_PREFILL_GATEUP, k_mm_gateup, dim3(n_gu), dim3(WG), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.b_shared_blocks = ttiles * (a.d / 64);
    const int n_dn = a.b_shared_blocks + max_items * (a.d / 64);
    TF_LAUNCH(TF_KERNEL_PREFILL_DOWN, k_mm_down, dim3(n_dn), dim3(WG), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return tf_launch_prefill_combine(a, s);
}
