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

}  // namespace tfk
