// Device helpers shared by the gfx950 kernels of the q4 MoE layer.
//
// Arithmetic form of the quantised dot product.  A weight is
// w = s*q + b with q a 4-bit code and (s, b) the fp16 scale and bias of its
// group of 64 (shilu.ai README translation, "概览": MLX affine 4-bit, group
// 64).  Over one half-group of 32 elements
//     sum_i w_i x_i = s * sum_i q_i x_i + b * sum_i x_i .
// The nibbles are turned into fp16 values 1024+q with one AND-OR against the
// exponent pattern 0x6400 (1024.0 has an ulp of 1, so the 4-bit code lands
// exactly in the low mantissa bits), two codes per 32-bit register, and fed
// to v_dot2_f32_f16 against fp16 pairs of x.  That yields
//     D = sum_i (1024 + q_i) x_i = sum_i q_i x_i + 1024 X,
// so the half-group contributes  s*D + (b - 1024 s) * X  with X = sum_i x_i
// precomputed once per token.  Products are exact in fp32 (11 x 11 bits);
// only the fp32 sums round.
//
// Register pairing.  One 32-bit word of codes holds elements e0..e7 (low
// nibble first).  Masking with 0x000F000F after shifts of 0/4/8/12 gives the
// pairs (e0,e4) (e1,e5) (e2,e6) (e3,e7); the activation is staged in LDS in
// the same pairing, so no shuffle is needed in the inner loop.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tfk {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr int TILE_ROWS = 8;      // rows per wave tile
constexpr int LANES_PER_ROW = 8;  // lanes cooperating on one row
constexpr int MAX_J = 16;         // half-group chunks per lane (K <= 4096)

__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);   // v_cvt_f16_f32, RNE
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b),
                                  c, false);
}

// D = sum over the 32 codes of one 16-byte chunk of (1024+q) * x, with the
// activation pairs xp[m] (m = 0..3) staged for the four code words.
__device__ __forceinline__ float q4_chunk_dot(const uint4 q, const uint4 *xp0, const uint4 *xp1,
                                              const uint4 *xp2, const uint4 *xp3, float acc) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    const uint4 *xs[4] = {xp0, xp1, xp2, xp3};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint4 X = *xs[m];
        const uint32_t v = w[m];
        acc = dot2((v & 0x000F000Fu) | 0x64006400u, X.x, acc);
        acc = dot2(((v >> 4) & 0x000F000Fu) | 0x64006400u, X.y, acc);
        acc = dot2(((v >> 8) & 0x000F000Fu) | 0x64006400u, X.z, acc);
        acc = dot2(((v >> 12) & 0x000F000Fu) | 0x64006400u, X.w, acc);
    }
    return acc;
}

// Sum over the 8 lanes of a row group (lanes 8r..8r+7).
__device__ __forceinline__ float row8_sum(float v) {
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

// Pair eight fp16 values (four words, low half first) as (e0,e4) (e1,e5)
// (e2,e6) (e3,e7).
__device__ __forceinline__ uint4 pair_halves(uint4 v) {
    uint4 p;
    p.x = (v.x & 0xFFFFu) | (v.z << 16);
    p.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    p.z = (v.y & 0xFFFFu) | (v.w << 16);
    p.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return p;
}

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    return (uint32_t)f2h(lo) | ((uint32_t)f2h(hi) << 16);
}

// Stage one fp16 activation row x[K] into LDS:
//   xp[(m*H + hg)]  (uint4) : the four pair words for code word m of half-group hg
//   xs[hg]          (float) : X = sum of the 32 values of half-group hg
// H = K/32.  All 64 lanes must call (shuffles inside).
__device__ __forceinline__ void stage_x_f16(const uint16_t *__restrict__ x, int K, uint4 *xp,
                                            float *xs, int lane) {
    const int H = K >> 5, NB = K >> 3;
    const uint4 *xv = reinterpret_cast<const uint4 *>(x);
    for (int b0 = 0; b0 < NB; b0 += WAVE) {
        const int b = b0 + lane;
        const bool ok = b < NB;
        uint4 v = ok ? xv[b] : make_uint4(0, 0, 0, 0);
        float s = 0.f;
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s += h2f((uint16_t)(w[i] & 0xFFFF)) + h2f((uint16_t)(w[i] >> 16));
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        if (ok) {
            const int hg = b >> 2, m = b & 3;
            xp[m * H + hg] = pair_halves(v);
            if (m == 0) xs[hg] = s;
        }
    }
}

// Stage one fp32 activation row h[K] scaled by c as a hi/lo pair of fp16 rows
// (h*c = hi + lo + O(2^-22 |h*c|)) in the same pairing, plus
// xs[hg] = sum over the half-group of (float)hi + (float)lo.
__device__ __forceinline__ void stage_h_f32(const float *__restrict__ h, float c, int K,
                                            uint4 *hp, uint4 *lp, float *xs, int lane) {
    const int H = K >> 5, NB = K >> 3;
    const float4 *hv = reinterpret_cast<const float4 *>(h);
    for (int b0 = 0; b0 < NB; b0 += WAVE) {
        const int b = b0 + lane;
        const bool ok = b < NB;
        float e[8];
        if (ok) {
            const float4 a = hv[2 * b], d = hv[2 * b + 1];
            e[0] = a.x; e[1] = a.y; e[2] = a.z; e[3] = a.w;
            e[4] = d.x; e[5] = d.y; e[6] = d.z; e[7] = d.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = 0.f;
        }
        float hi[8], lo[8], s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = e[i] * c;
            hi[i] = (float)(_Float16)v;
            lo[i] = (float)(_Float16)(v - hi[i]);
            s += hi[i] + lo[i];
        }
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        if (ok) {
            const int hg = b >> 2, m = b & 3;
            hp[m * H + hg] = make_uint4(pack_h2(hi[0], hi[4]), pack_h2(hi[1], hi[5]),
                                        pack_h2(hi[2], hi[6]), pack_h2(hi[3], hi[7]));
            lp[m * H + hg] = make_uint4(pack_h2(lo[0], lo[4]), pack_h2(lo[1], lo[5]),
                                        pack_h2(lo[2], lo[6]), pack_h2(lo[3], lo[7]));
            if (m == 0) xs[hg] = s;
        }
    }
}

__device__ __forceinline__ float gelu_f(float z, int tanh_form) {
    if (tanh_form) {
        const float c = 0.7978845608028654f;
        return 0.5f * z * (1.f + tanhf(c * (z + 0.044715f * z * z * z)));
    }
    return 0.5f * z * (1.f + erff(z * 0.7071067811865476f));
}

}  // namespace tfk
