// Grouped q4 GEMMs of the MoE layer on the gfx950 matrix cores: prefill
// chunks and decode steps of more than one token.
//
// Once a step's (token, rank) pairs are grouped by expert, one fetched
// expert serves all of its tokens (shilu.ai README translation,
// "推理引擎的工作原理").  The work is cut into units: 32 rows of gate and of
// up (gate/up launch) or 64 rows of down (down launch) of one expert for up
// to four of its tokens -- an expert item of the grouping, or four tokens of
// the shared expert.  An expert with more tokens has several items; their
// weight reads after the first are cache hits.
//
// MFMA: v_mfma_f32_16x16x32_f16, D[16 rows][16 columns] += A[16][32] B[32][16].
// A (weights).  One AND-OR with the exponent pattern of 1024.0 turns a code
// word into fp16 1024+q (low nibbles: even elements) or 1024+16q (high
// nibbles: odd elements, left in place).  Low-nibble values of two words
// form one A operand, high-nibble values another; nothing else is done to
// the codes.
// B (activations).  Staged in LDS per pair of words as the activations of
// the even elements and, for the odd elements, the activations divided by
// 16 (exact in fp16 short of the subnormal range), in the order the AND-OR
// produces: (e0,e4)(e2,e6) of each word.  So for one group and column
//     D = sum_even (1024+q) x + sum_odd (1024+16q) (x/16)
//       = sum q x + C,   C = 1024 (sum_even x + sum_odd x/16),
// with every product exact in fp32.  The accumulator starts at -C, and the
// group's scale and bias apply once: y += s D + b X, X = the group's sum of x.
// Down projections read the hidden rows as hi + lo fp16 parts, each through
// its own pair of MFMAs, so h keeps 22 significant bits.
// Columns.  Column c is token c / 4 of group slot c % 4; lane block b (lanes
// 16b..16b+15) feeds k-block b of A and B with the codes of slot b's group,
// so one round of MFMAs covers four groups and the scale/bias epilogue runs
// once per round.  B lanes of the other slots read a zero block.  At the end
// the four slot columns of a token are summed (DPP), in a fixed order.
//
// Streaming.  A workgroup is persistent: it takes units blockIdx.x,
// blockIdx.x + gridDim.x, ...  K goes through LDS in chunks of 16 groups
// (gate/up) or 4 (down) (activations, and scale/bias as fp32); each lane
// holds its codes of one chunk in registers.  Loads run one chunk ahead
// regardless of unit boundaries: the last chunk of a unit loads the first
// chunk of the next (whose item record was loaded when the unit began), so a
// unit's start-up and epilogue overlap the next unit's loads.
#include "tf_device.h"
#include "tf_internal.h"
#include "tf_layer.h"

using namespace tfk;

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int UT = 4;     // tokens per unit

// Hidden rows between the grouped gate/up and down launches, F values:
// word pairs (16 values) of 64 bytes [part hi: even | odd/16][part lo:
// even | odd/16], then one (X, C) float2 per 8-value block (the consumer adds
// a group's eight in a fixed order).
__host__ __device__ constexpr int mq_row_u4(int F) { return F / 4 + F / 16; }

// The masks and the exponent pattern live in registers (Masks), so that each
// value is one v_and_or_b32 (its VOP3 encoding takes no literal operands).
struct Masks {
    uint32_t lo, hi, magic;
};
__device__ __forceinline__ Masks masks() {
    Masks k = {M_LO, M_HI, MAGIC};
    asm volatile("" : "+v"(k.lo), "+v"(k.hi), "+v"(k.magic));
    return k;
}
__device__ __forceinline__ half8 codes_lo(const Masks &k, uint32_t w0, uint32_t w1) {
    const u32x4 v = {(w0 & k.lo) | k.magic, ((w0 >> 8) & k.lo) | k.magic, (w1 & k.lo) | k.magic,
                     ((w1 >> 8) & k.lo) | k.magic};
    return __builtin_bit_cast(half8, v);
}
__device__ __forceinline__ half8 codes_hi(const Masks &k, uint32_t w0, uint32_t w1) {
    const u32x4 v = {(w0 & k.hi) | k.magic, ((w0 >> 8) & k.hi) | k.magic, (w1 & k.hi) | k.magic,
                     ((w1 >> 8) & k.hi) | k.magic};
    return __builtin_bit_cast(half8, v);
}
__device__ __forceinline__ half8 as_half8(uint4 v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    return __builtin_bit_cast(half8, w);
}
__device__ __forceinline__ f32x4 mfma(half8 a, half8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// indexed through memory).
template <typename T>
__device__ __forceinline__ T pick4(int i, T v0, T v1, T v2, T v3) {
    return i == 0 ? v0 : i == 1 ? v1 : i == 2 ? v2 : v3;
}

// KC groups per staged K chunk.
template <int PARTS, int KC>
struct GLds {
    // the chunk's activations: [token][word pair][part][even | odd/16], one
    // 16-byte entry each; rows padded so that the tokens of a B read fall on
    // different banks
    // (two buffers: chunk c is read from buffer c % 2 while chunk c + 1 is
    // staged into the other, so one barrier per chunk suffices)
    uint4 xs[2][UT][KC * 4 * PARTS * 2 + 1];
    float2 xc[2][UT][KC + 1];   // (X, C) per token and group of the chunk
    float2 sb[2][KC][64 + 4];   // (scale, bias) per group and row of the block
    float out[2][32][UT + 1];   // gate and up sums of a unit
    uint4 zero[2 * PARTS];      // B operand of the columns a lane block does not feed
    uint4 rec[2][3];            // item record of the next unit, by unit parity
};

// Item record as loaded (expert, begin, count, -, pairs[4], weights[4]).
struct Rec {
    uint4 r0, r1, r2;
};

// One unit: the expert blob, routed or shared, its hidden size, the row
// tile, its chunk count and up to four (source row, destination row,
// coefficient) slots.
struct Unit {
    const uint8_t *blob;
    int routed, F, rt, nt, nch;
    int s0, s1, s2, s3;       // source rows
    int d0, d1, d2, d3;       // destination rows
    float c0, c1, c2, c3;     // coefficients
};

// Unit u of a launch: shared units first (token quads x row tiles), then
// routed units (items x row tiles).  The chunk count is even (two buffers
// alternate; an odd count gets an empty chunk).
template <bool DOWN, int KC, int DEPTH>
__device__ Unit unit_of(const DecodeArgs &a, int u, const Rec &rc, int ns, int tiles_s,
                        int tiles_r) {
    Unit U;
    if (u < ns) {
        const int qd = u / tiles_s;
        U.blob = a.shared_blob;
        U.routed = 0;
        U.F = a.fs;
        U.rt = u - qd * tiles_s;
        U.nt = min(UT, a.T - UT * qd);
        U.s0 = U.d0 = min(UT * qd, a.T - 1);
        U.s1 = U.d1 = min(UT * qd + 1, a.T - 1);
        U.s2 = U.d2 = min(UT * qd + 2, a.T - 1);
        U.s3 = U.d3 = min(UT * qd + 3, a.T - 1);
        U.c0 = U.c1 = U.c2 = U.c3 = 1.f;
    } else {
        const int v = u - ns, item = v / tiles_r;
        U.blob = expert_blob(a, min(max((int)rc.r0.x, 0), a.E - 1));
        U.routed = 1;
        U.F = a.f;
        U.rt = v - item * tiles_r;
        U.nt = min(UT, max((int)rc.r0.z, 1));
        const int pmax = a.T * a.k - 1;
        // slots past the count repeat the first pair
        const int p0 = min(max((int)rc.r1.x, 0), pmax);
        const int p1 = U.nt > 1 ? min(max((int)rc.r1.y, 0), pmax) : p0;
        const int p2 = U.nt > 2 ? min(max((int)rc.r1.z, 0), pmax) : p0;
        const int p3 = U.nt > 3 ? min(max((int)rc.r1.w, 0), pmax) : p0;
        U.d0 = p0; U.d1 = p1; U.d2 = p2; U.d3 = p3;
        U.s0 = DOWN ? p0 : p0 / a.k;
        U.s1 = DOWN ? p1 : p1 / a.k;
        U.s2 = DOWN ? p2 : p2 / a.k;
        U.s3 = DOWN ? p3 : p3 / a.k;
        U.c0 = __uint_as_float(rc.r2.x);
        U.c1 = __uint_as_float(rc.r2.y);
        U.c2 = __uint_as_float(rc.r2.z);
        U.c3 = __uint_as_float(rc.r2.w);
    }
    const int nc = ((DOWN ? U.F : a.d) / 64 + KC - 1) / KC;
    U.nch = DEPTH == 2 ? (nc + 1) & ~1 : nc;
    return U;
}

// Persistent grouped GEMM.  DOWN = false: gate/up rows [32 rt, +32) (K = d)
// into hidden rows h = coef * gelu(g) * u; DOWN = true: down rows [64 rt, +64)
// (K = F) into fp32 rows (y_s per token, y_e per pair).
// Pipeline: chunk c computes from LDS (staged at the end of chunk c - 1) and
// from code ring c % 2 (loaded during chunk c - 2); it loads chunk c + 2 into
// ring c % 2 and staging registers c % 2, and stages chunk c + 1 (loaded
// during chunk c - 1) into LDS.  Chunk positions past a unit's end belong to
// the next unit of this workgroup.
template <bool DOWN, int KC, int DEPTH>
__device__ void grouped(const DecodeArgs &a, GLds<DOWN ? 2 : 1, KC> &L) {
    constexpr int PARTS = DOWN ? 2 : 1;
    constexpr int NR = KC / 4;        // rounds of four groups per chunk
    constexpr int XW = KC / 8;        // gate/up staging: uint4 per lane per chunk
    constexpr int HW = KC / 4;        // down staging: uint4 per lane per chunk
    constexpr int SW = KC / 4;        // scale/bias entries per thread per chunk
    static_assert(!DOWN || 8 * KC <= 64, "one lane per 8-value block partial of a chunk");
    static_assert(DOWN || KC % 8 == 0, "gate/up staging copies whole uint4 per lane");
    const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
    const int j = lane & 15, b = lane >> 4;
    const int d = a.d;
    const int tiles_s = DOWN ? d / 64 : a.fs / 32, tiles_r = DOWN ? d / 64 : a.f / 32;
    const int ns = ((a.T + UT - 1) / UT) * tiles_s;
    const int grid = (int)gridDim.x;
    int u = blockIdx.x;

    // the item record of unit v (a valid record when v is not routed; past
    // the step's items, a stale record of the workspace that no unit uses).
    // The address takes an opaque zero, so the values stay in vector
    // registers and nothing waits for them before their first use.
    auto load_rec = [&](int v) {
        int z = 0;
        asm volatile("" : "+v"(z));
        const int item = min(max(v - ns, 0) / tiles_r, a.max_items - 1) + z;
        const uint4 *p = reinterpret_cast<const uint4 *>(a.items + ITEM_INTS * item);
        Rec r;
        r.r0 = ld_prev(p);
        r.r1 = ld_prev(p + 1);
        r.r2 = ld_prev(p + 2);
        return r;
    };
    // a loaded record, used here: an ordered empty asm keeps what follows at
    // this point (not hoisted next to the loads); then the fields move to
    // scalar registers
    auto settle = [](Rec r) {
        asm volatile("" : "+v"(r.r0.x), "+v"(r.r0.y), "+v"(r.r0.z), "+v"(r.r0.w),
                          "+v"(r.r1.x), "+v"(r.r1.y), "+v"(r.r1.z), "+v"(r.r1.w),
                          "+v"(r.r2.x), "+v"(r.r2.y), "+v"(r.r2.z), "+v"(r.r2.w));
        r.r0.x = uniform(r.r0.x); r.r0.z = uniform(r.r0.z);
        r.r1.x = uniform(r.r1.x); r.r1.y = uniform(r.r1.y);
        r.r1.z = uniform(r.r1.z); r.r1.w = uniform(r.r1.w);
        r.r2.x = uniform(r.r2.x); r.r2.y = uniform(r.r2.y);
        r.r2.z = uniform(r.r2.z); r.r2.w = uniform(r.r2.w);
        return r;
    };
    // Per-unit streaming bases, all uniform and selected by value: the wave's
    // code matrix, the scale/bias arrays of block rows [0, 32) and [32, 64),
    // and the activation row of the token this wave stages (tj = wave; every
    // lane loads, non-stagers a valid row they then ignore, so that no load
    // sits behind a branch).
    const int tj = w, li = lane;
    struct Str {
        const uint8_t *q;
        const uint16_t *s0, *b0, *s1, *b1;
        const uint4 *srow;
        int rt, G, nt, F;
    };
    auto mkstr = [&](const Unit &U) {
        Str S;
        Mat mg, mu, md;
        blob_mats(U.blob, d, U.F, mg, mu, md);
        S.G = (DOWN ? U.F : d) >> 6;
        S.rt = U.rt;
        S.nt = U.nt;
        S.F = U.F;
        S.q = DOWN ? md.q : ((w >> 1) ? mu.q : mg.q);
        S.s0 = DOWN ? md.s : mg.s;
        S.b0 = DOWN ? md.b : mg.b;
        S.s1 = DOWN ? md.s : mu.s;
        S.b1 = DOWN ? md.b : mu.b;
        const int src = pick4(min(tj, U.nt - 1), U.s0, U.s1, U.s2, U.s3);
        if (!DOWN) S.srow = a.xb + (size_t)src * xb_row_u4(d);
        else S.srow = (U.routed ? a.h_r : a.h_s) + (size_t)src * mq_row_u4(U.F);
        return S;
    };
    auto sel = [](bool c, const Str &x, const Str &y) {
        Str r;
        r.q = c ? x.q : y.q;
        r.s0 = c ? x.s0 : y.s0; r.b0 = c ? x.b0 : y.b0;
        r.s1 = c ? x.s1 : y.s1; r.b1 = c ? x.b1 : y.b1;
        r.srow = c ? x.srow : y.srow;
        r.rt = c ? x.rt : y.rt; r.G = c ? x.G : y.G; r.nt = c ? x.nt : y.nt; r.F = c ? x.F : y.F;
        return r;
    };
    // this lane's codes of chunk c: group KC c + 4 rho + b of round rho, 32
    // bytes each, of row r0 + j
    auto qload = [&](uint4 (&q)[2 * NR], const Str &S, int c, int rho) {
        const int r0 = DOWN ? 64 * S.rt + 16 * w : 32 * S.rt + 16 * (w & 1);
        const int g = min(KC * c + 4 * rho + b, S.G - 1);
        const uint8_t *p = S.q + (size_t)(r0 + j) * (32 * S.G) + 32 * g;
        q[2 * rho] = *reinterpret_cast<const uint4 *>(p);
        q[2 * rho + 1] = *reinterpret_cast<const uint4 *>(p + 16);
    };
    // staging loads of chunk c into registers (activation rows are already in
    // B-operand form: these are copies)
    struct Pre {
        uint4 v[DOWN ? HW : XW];
        float2 xc;
        uint32_t sbw[SW];
    };
    auto fetch = [&](Pre &P, const Str &S, int c) {
        if (!DOWN) {   // uint4 8 KC c + XW li + i; (X, C) of group KC c + li
#pragma unroll
            for (int i = 0; i < XW; ++i) P.v[i] = S.srow[min(8 * KC * c + XW * li + i, d / 8 - 1)];
            P.xc = reinterpret_cast<const float2 *>(S.srow + d / 8)[min(KC * c + (li & (KC - 1)), S.G - 1)];
        } else {       // uint4 16 KC c + HW li + i; (X, C) of 8-value block 8 KC c + li
            const int HU = S.F / 4;
#pragma unroll
            for (int i = 0; i < HW; ++i) P.v[i] = S.srow[min(16 * KC * c + HW * li + i, HU - 1)];
            P.xc = reinterpret_cast<const float2 *>(S.srow + HU)[min(8 * KC * c + (li & (8 * KC - 1)), S.F / 8 - 1)];
        }
        // entry e = tid + 256 qq: block row e / KC, group KC c + e % KC; rows
        // [0, 32) from s0/b0, [32, 64) from s1/b1 (down: one matrix)
        const int g = min(KC * c + tid % KC, S.G - 1);
#pragma unroll
        for (int qq = 0; qq < SW; ++qq) {
            const int rr = tid / KC + 256 / KC * qq;
            if (DOWN || qq < SW / 2) {
                const int row = (DOWN ? 64 * S.rt : 32 * S.rt) + rr;
                P.sbw[qq] = (uint32_t)S.s0[row * S.G + g] | ((uint32_t)S.b0[row * S.G + g] << 16);
            } else {
                const int row = 32 * S.rt + rr - 32;
                P.sbw[qq] = (uint32_t)S.s1[row * S.G + g] | ((uint32_t)S.b1[row * S.G + g] << 16);
            }
        }
    };
    auto store = [&](const Pre &P, const Str &S, int c, int nb) {
        const bool stager = tj < S.nt;   // uniform per wave
        if (!DOWN) {
            if (stager) {
#pragma unroll
                for (int i = 0; i < XW; ++i)
                    L.xs[nb][tj][XW * li + i] =
                        8 * KC * c + XW * li + i < d / 8 ? P.v[i] : make_uint4(0, 0, 0, 0);
                if (li < KC)
                    L.xc[nb][tj][li] = KC * c + li < S.G ? P.xc : make_float2(0.f, 0.f);
            }
        } else {
            const int HU = S.F / 4;
            float X = 0.f, C = 0.f;
            if (stager) {
#pragma unroll
                for (int i = 0; i < HW; ++i)
                    L.xs[nb][tj][HW * li + i] =
                        16 * KC * c + HW * li + i < HU ? P.v[i] : make_uint4(0, 0, 0, 0);
            }
            if (li < 8 * KC && 8 * KC * c + li < S.F / 8) { X = P.xc.x; C = P.xc.y; }
            // a group's eight block partials, in a fixed order
            X += __shfl_xor(X, 1);
            C += __shfl_xor(C, 1);
            X += __shfl_xor(X, 2);
            C += __shfl_xor(C, 2);
            X += __shfl_xor(X, 4);
            C += __shfl_xor(C, 4);
            if (stager && li < 8 * KC && !(li & 7)) L.xc[nb][tj][li >> 3] = make_float2(X, C);
        }
#pragma unroll
        for (int qq = 0; qq < SW; ++qq) {
            const int rr = tid / KC + 256 / KC * qq, gl = tid % KC;
            const uint32_t v = KC * c + gl < S.G ? P.sbw[qq] : 0u;
            L.sb[nb][gl][rr] = make_float2(h2f((uint16_t)(v & 0xFFFF)), h2f((uint16_t)(v >> 16)));
        }
    };

    // this lane's column: token tc of slot sc
    const int tc = j >> 2, sc = j & 3;
    const Masks km = masks();
    // the first record is read together with the item count
    const Rec rec0 = load_rec(u);
    const int n_items = (int)ld_prev(a.hdr + HDR_NITEMS);
    const int n_units = ns + n_items * tiles_r;
    if (u >= n_units) return;
    if (tid < 2 * PARTS) L.zero[tid] = make_uint4(0, 0, 0, 0);
    Unit cur = unit_of<DOWN, KC, DEPTH>(a, u, settle(rec0), ns, tiles_s, tiles_r);
    Str scu = mkstr(cur);
    uint4 qa[2 * NR], qb[DEPTH == 2 ? 2 * NR : 1];
#pragma unroll
    for (int rho = 0; rho < NR; ++rho) qload(qa, scu, 0, rho);
    Pre Pa, Pb;
    int buf = 0;   // LDS buffer the current chunk is read from
    fetch(Pa, scu, 0);
    store(Pa, scu, 0, 0);
    if (DEPTH == 2) {
        uint4 (&q2)[2 * NR] = *reinterpret_cast<uint4 (*)[2 * NR]>(DEPTH == 2 ? qb : qa);
#pragma unroll
        for (int rho = 0; rho < NR; ++rho) qload(q2, scu, 1, rho);
        fetch(Pb, scu, 1);
    }
    // Records: the next unit's sits in LDS slot par (read when this unit's
    // last two chunks start); the one after is loaded into registers a unit
    // ahead and moved to the other slot at that same point, where a wait
    // for it costs nothing extra.  (Copying loaded registers at the unit
    // boundary would wait for every load in flight.)
    int par = 0;
    {
        const Rec r = load_rec(u + grid);
        if (tid == 0) L.rec[0][0] = r.r0;
        if (tid == 1) L.rec[0][1] = r.r1;
        if (tid == 2) L.rec[0][2] = r.r2;
    }
    lds_barrier();   // the slot is read before the first chunk's barrier when nch == 2
    Rec rnn = load_rec(u + 2 * grid);
    for (;;) {
        const int un = u + grid;
        const bool more = un < n_units;
        Unit nxt = cur;
        Str snx = scu;
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        const bool feeds = tc < cur.nt && sc == b;
        // One chunk: compute from LDS and ring q; load position c + DEPTH
        // into q and Pf; stage position c + 1 from Ps (DEPTH 1: Pf is Ps,
        // staged after its loads land).
        auto chunk = [&](int c, uint4 (&q)[2 * NR], Pre &Pf, const Pre &Ps) {
            lds_barrier();   // chunk c is staged
            const bool n1 = c + 1 >= cur.nch, n2 = c + DEPTH >= cur.nch;
            const Str s1 = sel(n1, snx, scu), s2 = sel(n2, snx, scu);
            const int c1 = n1 ? c + 1 - cur.nch : c + 1;
            const int c2 = n2 ? c + DEPTH - cur.nch : c + DEPTH;
            fetch(Pf, s2, c2);
#pragma unroll
            for (int rho = 0; rho < NR; ++rho) {
                const int gc = 4 * rho + sc;   // the column's group in the chunk
                const float2 xc = L.xc[buf][tc][gc];
                f32x4 D = {-xc.y, -xc.y, -xc.y, -xc.y};
#pragma unroll
                for (int sg = 0; sg < 4; ++sg) {
                    const uint4 v = q[2 * rho + (sg >> 1)];
                    const uint32_t w0 = (sg & 1) ? v.z : v.x, w1 = (sg & 1) ? v.w : v.y;
                    const half8 al = codes_lo(km, w0, w1), ah = codes_hi(km, w0, w1);
                    const int m = 4 * (4 * rho + b) + sg;   // word pair fed by lane block b
                    const uint4 *bp = feeds ? &L.xs[buf][tc][m * 2 * PARTS] : L.zero;
#pragma unroll
                    for (int p = 0; p < PARTS; ++p) {
                        D = mfma(al, as_half8(bp[2 * p]), D);
                        D = mfma(ah, as_half8(bp[2 * p + 1]), D);
                    }
                }
                qload(q, s2, c2, rho);
                const float4 s01 = *reinterpret_cast<const float4 *>(&L.sb[buf][gc][16 * w + 4 * b]);
                const float4 s23 = *reinterpret_cast<const float4 *>(&L.sb[buf][gc][16 * w + 4 * b + 2]);
                y[0] = fmaf(s01.x, D[0], fmaf(s01.y, xc.x, y[0]));
                y[1] = fmaf(s01.z, D[1], fmaf(s01.w, xc.x, y[1]));
                y[2] = fmaf(s23.x, D[2], fmaf(s23.y, xc.x, y[2]));
                y[3] = fmaf(s23.z, D[3], fmaf(s23.w, xc.x, y[3]));
                // the round's epilogue completes here (an ordered empty asm
                // reading y), so no round's D stays live to the end
                asm volatile("" : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]));
            }
            // the other buffer: every wave finished reading it before this
            // chunk's barrier
            store(Ps, s1, c1, buf ^ 1);
            buf ^= 1;
        };
        for (int c = 0; c < cur.nch; c += DEPTH) {
            if (c + DEPTH == cur.nch && more) {   // no loads in here
                Rec rn;
                rn.r0 = L.rec[par][0];
                rn.r1 = L.rec[par][1];
                rn.r2 = L.rec[par][2];
                nxt = unit_of<DOWN, KC, DEPTH>(a, un, settle(rn), ns, tiles_s, tiles_r);
                snx = mkstr(nxt);
                if (tid == 0) L.rec[par ^ 1][0] = rnn.r0;
                if (tid == 1) L.rec[par ^ 1][1] = rnn.r1;
                if (tid == 2) L.rec[par ^ 1][2] = rnn.r2;
            }
            if (DEPTH == 2) {
                uint4 (&q2)[2 * NR] = *reinterpret_cast<uint4 (*)[2 * NR]>(DEPTH == 2 ? qb : qa);
                chunk(c, qa, Pa, Pb);
                chunk(c + 1, q2, Pb, Pa);
            } else {
                chunk(c, qa, Pa, Pa);
            }
        }
        // a token's four slot columns are neighbouring lanes: sum them
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            y[r] += dpp_f<DPP_XOR1>(y[r]);
            y[r] += dpp_f<DPP_XOR2>(y[r]);
        }
        const bool owner = sc == 0 && tc < cur.nt;
        if (DOWN) {   // rows 64 rt + 16 w + 4b .. +3 of token tc
            if (owner) {
                float *yd = cur.routed ? a.y_e : a.y_s;
                *reinterpret_cast<float4 *>(yd + (size_t)pick4(tc, cur.d0, cur.d1, cur.d2, cur.d3) * d +
                                            64 * cur.rt + 16 * w + 4 * b) = make_float4(y[0], y[1], y[2], y[3]);
            }
        } else {
            if (owner) {
#pragma unroll
                for (int r = 0; r < 4; ++r) L.out[w >> 1][16 * (w & 1) + 4 * b + r][tc] = y[r];
            }
            lds_barrier();
            // wave w: 8-row block w of the unit; lane (token t, row i) of it:
            // h = coef * gelu(g) * u, split into hi + lo fp16 parts
            const int t = (lane >> 3) & (UT - 1), i = lane & 7;
            const bool ok = lane < 8 * UT && t < cur.nt;
            const float cf = pick4(t, cur.c0, cur.c1, cur.c2, cur.c3);
            const float e = ok ? cf * (gelu_f(L.out[0][8 * w + i][t], a.act) * L.out[1][8 * w + i][t]) : 0.f;
            const float eh = (float)(_Float16)e, el = (float)(_Float16)(e - eh);
            // lane i < 4 packs elements (i, i + 4): even i as they are, odd i
            // divided by 16 -- words (e0,e4)(e2,e6) | (e1,e5)(e3,e7)
            const float ph = __shfl_xor(eh, 4), pl = __shfl_xor(el, 4);
            uint32_t wh = pack_h2(eh, ph), wl = pack_h2(el, pl);
            if (i & 1) { wh = div16(wh); wl = div16(wl); }
            float C = i < 4 ? hsum2(wh) + hsum2(wl) : 0.f;
            float X = e;
            X += __shfl_xor(X, 1);
            C += __shfl_xor(C, 1);
            X += __shfl_xor(X, 2);
            C += __shfl_xor(C, 2);
            X += __shfl_xor(X, 4);
            if (ok && i < 4) {
                const int F = cur.F, wg = 4 * cur.rt + w;   // 8-value block of the hidden row
                uint4 *row = (cur.routed ? a.h_r : a.h_s) +
                             (size_t)pick4(t, cur.d0, cur.d1, cur.d2, cur.d3) * mq_row_u4(F);
                uint32_t *wd = reinterpret_cast<uint32_t *>(row) + 16 * (wg >> 1) + 2 * (wg & 1) +
                               4 * (i & 1) + (i >> 1);
                wd[0] = wh;
                wd[8] = wl;
                if (i == 0) reinterpret_cast<float2 *>(row + F / 4)[wg] = make_float2(X, 1024.f * C);
            }
        }
        if (!more) break;
        u = un;
        cur = nxt;
        scu = snx;
        par ^= 1;
        rnn = load_rec(u + 2 * grid);
    }
}

constexpr int KC_GU = 16, KC_DN = 4;  // groups per staged chunk
constexpr int DEPTH = 1;              // chunks loaded ahead

__global__ __launch_bounds__(256, 2) void k_gu(DecodeArgs a) {
    __shared__ GLds<1, KC_GU> L;
    grouped<false, KC_GU, DEPTH>(a, L);
}

__global__ __launch_bounds__(256, 4) void k_dn(DecodeArgs a) {
    __shared__ GLds<2, KC_DN> L;
    grouped<true, KC_DN, DEPTH>(a, L);
}

}  // namespace

// After the router launch (top-k and grouping into items of at most four
// tokens): gate/up, down, then the combine.  Persistent grids of at most two
// (gate/up) and four (down) workgroups per compute unit: gate/up measured
// 53.5, 52.0, 49.3 and 64.6 us per 16-token layer at four, three, two and
// one per unit, down 36.0 at four against 46.0 at two.
hipError_t tf_launch_grouped(const DecodeArgs &a, int max_items, hipStream_t s) {
    const int quads = (a.T + UT - 1) / UT;
    const int cap_gu = 2 * 256, cap = 4 * 256;
    const int n_gu = quads * (a.fs / 32) + max_items * (a.f / 32);
    TF_LAUNCH(TF_KERNEL_PREFILL_GATEUP, k_gu, dim3(n_gu < cap_gu ? n_gu : cap_gu), dim3(WG), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_dn = (quads + max_items) * (a.d / 64);
    TF_LAUNCH(TF_KERNEL_PREFILL_DOWN, k_dn, dim3(n_dn < cap ? n_dn : cap), dim3(WG), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return tf_launch_prefill_combine(a, s);
}
