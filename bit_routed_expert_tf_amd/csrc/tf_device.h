// Device helpers shared by the gfx950 kernels of the q4 MoE layer.
//
// Arithmetic form of the quantised dot product.  A weight is
// w = s*q + b with q a 4-bit code and (s, b) the fp16 scale and bias of its
// group of 64 (shilu.ai README translation, "概览": MLX affine 4-bit, group
// 64).  Over a half-group of 32 elements
//     sum_i w_i x_i = s * sum_i q_i x_i + b * X,      X = sum_i x_i .
// Codes become fp16 values with one AND-OR against the exponent pattern
// 0x6400 (1024.0, whose ulp is 1): an even element (low nibble) lands as
// 1024+q, an odd element (high nibble, left where it is) as 1024+16q.  Two
// codes share a 32-bit register and go through v_dot2_f32_f16 against fp16
// pairs of the activation, the even ones into De and the odd ones into Do:
//     De + Do/16 = sum_i q_i x_i + C,   C = 1024 X_even + 64 X_odd,
// so the half-group contributes  s * (De - C + Do/16) + b * X, with X and C
// computed once per activation row.  Every product is exact in fp32 (11-bit
// by 11-bit significands); only the fp32 sums round.
//
// Register pairing.  One 32-bit word of codes holds elements e0..e7 (low
// nibble first).  Masks 0x000F000F / 0x00F000F0 on the word and on the word
// shifted right by 8 give the pairs (e0,e4) (e1,e5) (e2,e6) (e3,e7); the
// activation is staged in the same pairing.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tfk {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr uint32_t M_LO = 0x000F000Fu, M_HI = 0x00F000F0u, MAGIC = 0x64006400u;

__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);   // v_cvt_f16_f32, round to nearest even
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b),
                                  c, false);
}

// The nibble unpack is an ordered asm statement: it keeps each chunk's
// unpack (and so its dot products) in place instead of letting the
// scheduler sink all dot products to the end of the unrolled loop (which
// keeps every unpacked word live and spills), and it gets v_and_or_b32 with
// the masks in registers (VOP3 cannot take the literals directly).
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t m, uint32_t c) {
    uint32_t r;
    asm volatile("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "v"(m), "s"(c));
    return r;
}

// acc += a.lo * b.lo + a.hi * b.hi  (fp16 pairs, fp32 accumulate).  Always
// the compiler builtin, never asm: the compiler must see the dot product to
// insert the wait states it needs after a VALU write of its operands.
__device__ __forceinline__ float dot2c(uint32_t a, uint32_t b, float acc) {
    return dot2(a, b, acc);
}

// Materialise a value here (an empty ordered asm): pins the computations
// feeding it before every later ordered asm statement.
__device__ __forceinline__ void pin(float &a, float &b) { asm volatile("" : "+v"(a), "+v"(b)); }

// One 16-byte chunk (32 codes of one half-group) against activation pair
// words X[m] (m = 0..3, one uint4 per code word): accumulates De and Do.
__device__ __forceinline__ void q4_chunk(const uint4 q, const uint4 X0, const uint4 X1,
                                         const uint4 X2, const uint4 X3, float &de, float &dd) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    const uint4 X[4] = {X0, X1, X2, X3};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t v = w[m], v8 = v >> 8;
        de = dot2c(and_or(v, M_LO, MAGIC), X[m].x, de);
        dd = dot2c(and_or(v, M_HI, MAGIC), X[m].y, dd);
        de = dot2c(and_or(v8, M_LO, MAGIC), X[m].z, de);
        dd = dot2c(and_or(v8, M_HI, MAGIC), X[m].w, dd);
        pin(de, dd);
    }
}

// Device-coherent accesses (agent-scope relaxed atomics: coherent across the
// XCDs' L2 caches).  Data one workgroup writes and another workgroup of the
// same launch reads goes through these; the writer waits for its stores
// (stores_done) before it takes a ticket, so the hand-off needs no
// cache-wide write-back or invalidation.
template <typename T>
__device__ __forceinline__ T ld_dev(const T *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_dev(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte values as two 8-byte halves (each half is single-copy atomic).
__device__ __forceinline__ uint4 ld_dev(const uint4 *p) {
    const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
    const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32));
}
__device__ __forceinline__ void st_dev(uint4 *p, uint4 v) {
    uint64_t *q = reinterpret_cast<uint64_t *>(p);
    __hip_atomic_store(q, (uint64_t)v.x | ((uint64_t)v.y << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, (uint64_t)v.z | ((uint64_t)v.w << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Data an earlier launch on the stream wrote (expert ids, router weights,
// item records): plain loads.  The kernel boundary already makes those
// writes visible, and a plain load can be served by this XCD's L2 -- when
// every workgroup of a launch reads the same few words, one miss per L2
// fetches them instead of one device-coherent request per workgroup.
template <typename T>
__device__ __forceinline__ T ld_prev(const T *p) {
    return *p;
}

// This thread's stores have completed; also a compiler barrier for memory
// operations.
__device__ __forceinline__ void stores_done() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
}
// Workgroup barrier after this thread's LDS writes have completed.  The
// explicit LDS-counter wait matters: without it the compiler may reach the
// barrier with LDS stores still in flight, and a wave past the barrier has
// been seen to read stale LDS data.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited on
    __syncthreads();
}

// DPP lane moves (row = 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const long long b = __builtin_bit_cast(long long, v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xFFFFFFFF), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned)lo);
}
// Inclusive prefix sum over the wave by DPP moves: within rows of 16 by
// shifts of 1, 2, 4, 8 (lanes before the row start add 0), then the totals
// of rows 0 and 2 into rows 1 and 3, then that of rows 0-1 into rows 2-3.
__device__ __forceinline__ int wave_scan_incl(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <-> 7-i within 8
constexpr int DPP_MIRROR = 0x140;       // lane i <-> 15-i within 16

// Sum over the 8 lanes of a row group (lanes 8r..8r+7); every lane of the
// group gets the sum.
__device__ __forceinline__ float row8_sum(float v) {
    v += dpp_f<DPP_XOR1>(v);
    v += dpp_f<DPP_XOR2>(v);
    v += dpp_f<DPP_HALF_MIRROR>(v);
    return v;
}

// Sum over the whole wave in fp64, returned in every lane (fixed order:
// within rows of 16 by DPP, then rows 0+1 and 2+3, then the two halves).
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_d<DPP_XOR1>(v);
    v += dpp_d<DPP_XOR2>(v);
    v += dpp_d<DPP_HALF_MIRROR>(v);
    v += dpp_d<DPP_MIRROR>(v);
    const long long b = __builtin_bit_cast(long long, v);
    double r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFF), 16 * i);
        const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 16 * i);
        r[i] = __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned)lo);
    }
    return (r[0] + r[1]) + (r[2] + r[3]);
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

__device__ __forceinline__ float gelu_f(float z, int tanh_form) {
    if (tanh_form) {
        const float c = 0.7978845608028654f;
        return 0.5f * z * (1.f + tanhf(c * (z + 0.044715f * z * z * z)));
    }
    return 0.5f * z * (1.f + erff(z * 0.7071067811865476f));
}

}  // namespace tfk
