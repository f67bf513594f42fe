// Device helpers shared by the decode and prefill kernels: the expert blob
// layout, the hi/lo hidden-row format and the LDS staging sizes.
#pragma once
#include "tf_device.h"
#include "tf_internal.h"

namespace tfk {

constexpr int WG = 256;   // threads per workgroup (four waves)

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
    const int slot = a.slot_map ? a.slot_map[e] : e;
    return a.pool + (size_t)slot * a.stride;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// LDS stage layouts (bytes): fp16 row  = pairs [4H] uint4 + S [H] float2
//                            hi/lo row = hi [4H] uint4 + lo [4H] uint4 + S [H] float2
__host__ __device__ constexpr int xst_bytes(int K) { return 72 * (K >> 5); }
__host__ __device__ constexpr int hst_bytes(int K) { return 136 * (K >> 5); }

// Producer side: the 8 values of rows 8*blk .. 8*blk+7 of one hidden row of
// length K go to the global hi/lo row `dst` (10H uint4).
__device__ __forceinline__ void hs_produce(uint4 *dst, int K, int blk, const float (&e)[8]) {
    const int H = K >> 5;
    float hi[8], lo[8], xe = 0.f, xo = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        hi[q] = (float)(_Float16)e[q];
        lo[q] = (float)(_Float16)(e[q] - hi[q]);
        if (q & 1) xo += hi[q] + lo[q];
        else xe += hi[q] + lo[q];
    }
    const int hg = blk >> 2, m = blk & 3;
    dst[m * H + hg] = make_uint4(pack_h2(hi[0], hi[4]), pack_h2(hi[1], hi[5]),
                                 pack_h2(hi[2], hi[6]), pack_h2(hi[3], hi[7]));
    dst[4 * H + m * H + hg] = make_uint4(pack_h2(lo[0], lo[4]), pack_h2(lo[1], lo[5]),
                                         pack_h2(lo[2], lo[6]), pack_h2(lo[3], lo[7]));
    reinterpret_cast<float2 *>(dst + 8 * H + 2 * hg)[m] =
        make_float2(xe + xo, fmaf(1024.f, xe, 64.f * xo));
}

// An fp16 pair divided by 16 (exact unless the result is subnormal).
__device__ __forceinline__ uint32_t div16(uint32_t p) {
    const h2_t v = __builtin_bit_cast(h2_t, p) * h2_t{(_Float16)0.0625f, (_Float16)0.0625f};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float hsum2(uint32_t p) {
    return h2f((uint16_t)(p & 0xFFFF)) + h2f((uint16_t)(p >> 16));
}

// Activation rows in the grouped kernels' B-operand form: per pair of code
// words (16 values) the even elements and the odd elements divided by 16,
// each as (e0,e4)(e2,e6) of both words (32 bytes), then one (X, C) float2
// per group of 64: X = sum of the values, C = 1024 (sum of the even values +
// sum of the odd values / 16).  Row size in uint4.
__host__ __device__ constexpr int xb_row_u4(int d) { return (2 * d + 8 * (d / 64) + 15) / 16; }

// Values 16 wp .. 16 wp + 15 (v0: the first eight) into word pair wp of an
// activation row; X and C get their share of the group sums.
__device__ __forceinline__ void xb_produce(uint4 v0, uint4 v1, uint4 *row, int wp, float &X,
                                           float &C) {
    const uint4 p0 = pair_halves(v0), p1 = pair_halves(v1);
    const uint4 ev = make_uint4(p0.x, p0.z, p1.x, p1.z);
    const uint4 od = make_uint4(div16(p0.y), div16(p0.w), div16(p1.y), div16(p1.w));
    row[2 * wp] = ev;
    row[2 * wp + 1] = od;
    X = ((hsum2(p0.x) + hsum2(p0.z)) + (hsum2(p0.y) + hsum2(p0.w))) +
        ((hsum2(p1.x) + hsum2(p1.z)) + (hsum2(p1.y) + hsum2(p1.w)));
    C = 1024.f * (((hsum2(ev.x) + hsum2(ev.y)) + (hsum2(ev.z) + hsum2(ev.w))) +
                  ((hsum2(od.x) + hsum2(od.y)) + (hsum2(od.z) + hsum2(od.w))));
}

}  // namespace tfk
