// Grouped q4 GEMMs of the MoE layer on the gfx950 matrix cores for prefill
// chunks (more than 16 tokens): one workgroup per tile of up to 16 tokens.
// (Decode steps of 2..16 tokens use the persistent kernels of
// tf_grouped.hip, whose 4-token units suit their few tokens per expert.)
//
// Once a step's (token, rank) pairs are grouped by expert, one fetched
// expert serves all of its tokens (shilu.ai README translation,
// "推理引擎的工作原理").  A tile is one expert item (up to 16 of its tokens)
// or up to 16 tokens of the shared expert; its rows go through
// v_mfma_f32_16x16x32_f16 (D[16 rows][16 columns] += A[16][32] B[32][16]).
//
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
//
// Columns.  Lane block b (lanes 16b..16b+15) feeds k-block b of A and B.
// A tile of n tokens uses GS = 4, 2 or 1 group slots (n <= 4, <= 8, <= 16):
// column c is token c / GS of slot c % GS, and lane block b feeds slot
// b / (4 / GS), so one round of MFMAs covers GS groups at once and the
// per-group scale/bias epilogue runs once per round.  B lanes of the other
// slots read a zero block.  At the end the GS slot columns of a token are
// summed (DPP), in a fixed order.
//
// Work.  A workgroup owns 32 rows of gate and of up (waves 0/1 gate, 2/3 up)
// or 64 rows of down, for one tile.  K goes through LDS in chunks of KC_GU / KC_DN groups
// (activations and scale/bias as fp32), loaded into registers one chunk
// ahead; each lane's codes (64 bytes per chunk) are reloaded for the next
// chunk as soon as a round has used them.
#include "tf_device.h"
#include "tf_internal.h"
#include "tf_layer.h"

using namespace tfk;

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int TT = 16;    // tokens per tile (the MFMA's N)
constexpr int KC_GU = 8;  // groups per staged K chunk: gate/up (512 columns of d)
constexpr int KC_DN = 4;  // down (256 columns of d_ff; 704 = 11 groups)

// Hidden rows between the grouped gate/up and down launches, F values:
// word pairs (16 values) of 64 bytes [part hi: even | odd/16][part lo:
// even | odd/16], then one (X, C) float2 per half-group (32 values).
__host__ __device__ constexpr int mq_row_u4(int F) { return F / 4 + F / 64; }

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
// An fp16 pair divided by 16 (exact unless the result is subnormal).
__device__ __forceinline__ uint32_t div16(uint32_t p) {
    const h2_t v = __builtin_bit_cast(h2_t, p) * h2_t{(_Float16)0.0625f, (_Float16)0.0625f};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float hsum2(uint32_t p) {
    return h2f((uint16_t)(p & 0xFFFF)) + h2f((uint16_t)(p >> 16));
}

template <int PARTS, int R, int KC>
struct MQLds {
    int src[TT], dst[TT];
    float coef[TT];
    int nt;
    // the chunk's activations: [token][word pair][part][even | odd/16], one
    // 16-byte entry each; rows padded so that the 16 tokens of a B read fall
    // on different banks
    uint4 xs[TT][KC * 4 * PARTS * 2 + 1];
    float2 xc[TT][KC + 1];      // (X, C) per token and group of the chunk
    float2 sb[R][KC][64 + 4];   // (scale, bias) per row tile, group and row of the block
    uint4 zero[2 * PARTS];      // B operand of the columns a lane block does not feed
};

// R row tiles rt0 .. rt0 + nrt - 1 (nrt <= R) of one item.  DOWN = false:
// gate/up rows [32 rt, +32) of the expert (F rows, K = d) into hidden rows;
// DOWN = true: down rows [64 rt, +64) (d rows, K = F) into fp32 output rows.
// Each K chunk of the tokens' activations is staged once for all R tiles,
// and each B operand read from LDS feeds R MFMAs.  Tiles past nrt repeat
// the last one and store nothing.  hsrc: the activation rows, already in
// B-operand form (gate/up: x rows as the router launch left them,
// xb_row_u4(d) uint4 each; down: hidden rows, mq_row_u4(F) uint4 each).
template <bool DOWN, int GS, int R, int KC>
__device__ void mq_tile(const DecodeArgs &a, const uint8_t *blob, int F, int rt0, int nrt,
                        MQLds<DOWN ? 2 : 1, R, KC> &L, int nt, const uint4 *hsrc, uint4 *hdst,
                        float *ydst) {
    constexpr int PARTS = DOWN ? 2 : 1;
    constexpr int NRND = KC / GS;    // rounds per chunk
    constexpr int XU = DOWN ? KC : KC / 2;   // staged uint4 per thread per chunk
    constexpr int SBQ = KC / 4;      // scale/bias entries per thread per chunk and tile
    static_assert(KC % 4 == 0 && KC <= 8, "rounds of four groups; 16 threads per token row");
    constexpr int BPS = 4 / GS;      // lane blocks per slot
    const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
    const int j = lane & 15, b = lane >> 4;
    const int d = a.d, K = DOWN ? F : d, G = K >> 6;
    Mat mg, mu, md;
    blob_mats(blob, d, F, mg, mu, md);
    const Mat &mm = DOWN ? md : ((w >> 1) ? mu : mg);
    int rts[R], r0s[R];   // row tile, first row of the wave
    const uint8_t *qrow[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        rts[i] = rt0 + min(i, nrt - 1);
        r0s[i] = DOWN ? 64 * rts[i] + 16 * w : 32 * rts[i] + 16 * (w & 1);
        qrow[i] = mm.q + (size_t)(r0s[i] + j) * (K >> 1);
    }

    // This lane's code bytes of tile i, chunk c, round rho: slot group and
    // words of lane block b (GS 4: the whole group; 2: half of it; 1: a
    // quarter).
    uint4 q[R][4];
    auto qload = [&](int i, int c, int rho) {
        if (GS == 4) {
            const int g = min(KC * c + 4 * rho + b, G - 1);
            q[i][2 * rho] = *reinterpret_cast<const uint4 *>(qrow[i] + 32 * g);
            q[i][2 * rho + 1] = *reinterpret_cast<const uint4 *>(qrow[i] + 32 * g + 16);
        } else if (GS == 2) {
            const int g = min(KC * c + 2 * rho + (b >> 1), G - 1);
            q[i][rho] = *reinterpret_cast<const uint4 *>(qrow[i] + 32 * g + 16 * (b & 1));
        } else {
            const int g = min(KC * c + rho, G - 1);
            const uint2 v = *reinterpret_cast<const uint2 *>(qrow[i] + 32 * g + 8 * b);
            if (rho & 1) { q[i][rho >> 1].z = v.x; q[i][rho >> 1].w = v.y; }
            else { q[i][rho >> 1].x = v.x; q[i][rho >> 1].y = v.y; }
        }
    };
    // words (w0, w1) of step sg of round rho of tile i
    auto words = [&](int i, int rho, int sg, uint32_t &w0, uint32_t &w1) {
        if (GS == 4) {
            const uint4 v = q[i][2 * rho + (sg >> 1)];
            w0 = (sg & 1) ? v.z : v.x;
            w1 = (sg & 1) ? v.w : v.y;
        } else if (GS == 2) {
            const uint4 v = q[i][rho];
            w0 = sg ? v.z : v.x;
            w1 = sg ? v.w : v.y;
        } else {
            const uint4 v = q[i][rho >> 1];
            w0 = (rho & 1) ? v.z : v.x;
            w1 = (rho & 1) ? v.w : v.y;
        }
    };

    // Staging: thread (token tj, sub) copies uint4 sub + 16 i of the chunk's
    // row (4 for gate/up, 8 for down; neighbouring lanes, neighbouring LDS
    // entries); loads into registers one chunk ahead (fetch), LDS stores after
    // the compute.
    const int tj = tid >> 4, sub = tid & 15;
    const bool stager = tj < nt;
    const int srow = L.src[min(tj, nt - 1)];
    const int HU = F / 4;   // word-pair uint4 of a hidden row (DOWN)
    struct Pre {
        uint4 v[XU];
        float2 xc;
        uint32_t sbw[R][SBQ];
    };
    // (every lane loads, non-stagers a valid row they then ignore: the loads
    // take no branch, so each wait counts only the loads it needs)
    auto fetch = [&](Pre &P, int c) {
        if (!DOWN) {   // uint4 sub + 16 i of the chunk's x row in B-operand form; (X, C) of group sub / 2
            const uint4 *xr = hsrc + (size_t)srow * xb_row_u4(d);
#pragma unroll
            for (int i = 0; i < XU; ++i) P.v[i] = xr[min(8 * KC * c + sub + 16 * i, d / 8 - 1)];
            P.xc = reinterpret_cast<const float2 *>(xr + d / 8)[min(KC * c + (sub >> 1), G - 1)];
        } else {
            const uint4 *hr = hsrc + (size_t)srow * mq_row_u4(F);
#pragma unroll
            for (int i = 0; i < XU; ++i) P.v[i] = hr[min(16 * KC * c + sub + 16 * i, HU - 1)];
            P.xc = reinterpret_cast<const float2 *>(hr + HU)[min(2 * KC * c + sub, F / 32 - 1)];
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
#pragma unroll
            for (int qq = 0; qq < SBQ; ++qq) {
                const int e = tid + 256 * qq, rr = e / KC, g = min(KC * c + e % KC, G - 1);
                const Mat &ms = DOWN ? md : (rr < 32 ? mg : mu);
                const int row = DOWN ? 64 * rts[i] + rr : 32 * rts[i] + (rr & 31);
                P.sbw[i][qq] =
                    (uint32_t)ms.s[(size_t)row * G + g] | ((uint32_t)ms.b[(size_t)row * G + g] << 16);
            }
        }
    };
    auto store = [&](const Pre &P, int c) {
        if (!DOWN) {   // copies: the router launch staged x in this form
            if (stager) {
#pragma unroll
                for (int i = 0; i < XU; ++i)
                    L.xs[tj][sub + 16 * i] =
                        8 * KC * c + sub + 16 * i < d / 8 ? P.v[i] : make_uint4(0, 0, 0, 0);
                if (!(sub & 1) && (sub >> 1) < KC)
                    L.xc[tj][sub >> 1] = KC * c + (sub >> 1) < G ? P.xc : make_float2(0.f, 0.f);
            }
        } else {
            float X = 0.f, C = 0.f;
            if (stager) {
#pragma unroll
                for (int i = 0; i < XU; ++i)
                    L.xs[tj][sub + 16 * i] =
                        16 * KC * c + sub + 16 * i < HU ? P.v[i] : make_uint4(0, 0, 0, 0);
                if (sub < 2 * KC && 2 * KC * c + sub < F / 32) { X = P.xc.x; C = P.xc.y; }
            }
            // the two halves of a group: lanes sub and sub ^ 1 (whole wave active)
            const float X2 = X + __shfl_xor(X, 1), C2 = C + __shfl_xor(C, 1);
            if (stager && !(sub & 1) && (sub >> 1) < KC) L.xc[tj][sub >> 1] = make_float2(X2, C2);
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
#pragma unroll
            for (int qq = 0; qq < SBQ; ++qq) {
                const int e = tid + 256 * qq, rr = e / KC, gl = e % KC;
                const uint32_t v = KC * c + gl < G ? P.sbw[i][qq] : 0u;
                L.sb[i][gl][rr] = make_float2(h2f((uint16_t)(v & 0xFFFF)), h2f((uint16_t)(v >> 16)));
            }
        }
    };

    // this lane's column: token tc of slot group sc; whether its B entries
    // are real (its lane block feeds its slot) or the zero block
    const int tc = j / GS, sc = j % GS;
    const bool col_ok = tc < nt;
    const bool feeds = col_ok && (GS == 1 || sc == b / BPS);
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int rho = 0; rho < NRND; ++rho) qload(i, 0, rho);
    Pre P;
    fetch(P, 0);
    store(P, 0);
    f32x4 y[R];
#pragma unroll
    for (int i = 0; i < R; ++i) y[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nch = (G + KC - 1) / KC;
    const uint4 *xrow = &L.xs[tc][0];
    const Masks km = masks();
    for (int c = 0; c < nch; ++c) {
        lds_barrier();   // chunk c is staged
        // the next chunk's loads; after the last chunk the last one again
        // (cache hits), so that no load sits behind a branch
        const int cn = min(c + 1, nch - 1);
        fetch(P, cn);
#pragma unroll
        for (int rho = 0; rho < NRND; ++rho) {
            const int gc = GS * rho + sc;   // the column's group in the chunk
            const float2 xc = L.xc[tc][gc];
            f32x4 D[R];
#pragma unroll
            for (int i = 0; i < R; ++i) D[i] = f32x4{-xc.y, -xc.y, -xc.y, -xc.y};
#pragma unroll
            for (int sg = 0; sg < GS; ++sg) {
                // the word pair lane block b feeds in this step
                const int m = GS == 4 ? 4 * (4 * rho + b) + sg
                            : GS == 2 ? 4 * (2 * rho + (b >> 1)) + 2 * (b & 1) + sg
                                      : 4 * rho + b;
                const uint4 *bp = feeds ? xrow + m * 2 * PARTS : L.zero;
                uint4 bv[2 * PARTS];
#pragma unroll
                for (int p = 0; p < 2 * PARTS; ++p) bv[p] = bp[p];
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    uint32_t w0, w1;
                    words(i, rho, sg, w0, w1);
                    const half8 al = codes_lo(km, w0, w1), ah = codes_hi(km, w0, w1);
#pragma unroll
                    for (int p = 0; p < PARTS; ++p) {
                        D[i] = mfma(al, as_half8(bv[2 * p]), D[i]);
                        D[i] = mfma(ah, as_half8(bv[2 * p + 1]), D[i]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < R; ++i) {
                qload(i, cn, rho);
                const float4 s01 = *reinterpret_cast<const float4 *>(&L.sb[i][gc][16 * w + 4 * b]);
                const float4 s23 = *reinterpret_cast<const float4 *>(&L.sb[i][gc][16 * w + 4 * b + 2]);
                y[i][0] = fmaf(s01.x, D[i][0], fmaf(s01.y, xc.x, y[i][0]));
                y[i][1] = fmaf(s01.z, D[i][1], fmaf(s01.w, xc.x, y[i][1]));
                y[i][2] = fmaf(s23.x, D[i][2], fmaf(s23.y, xc.x, y[i][2]));
                y[i][3] = fmaf(s23.z, D[i][3], fmaf(s23.w, xc.x, y[i][3]));
                // the round's epilogue completes here (an ordered empty asm
                // reading y), so no round's D stays live to the end of the chunk
                asm volatile("" : "+v"(y[i][0]), "+v"(y[i][1]), "+v"(y[i][2]), "+v"(y[i][3]));
            }
        }
        lds_barrier();   // everyone is done reading chunk c
        store(P, cn);
    }
    // a token's slot columns are neighbouring lanes: sum them
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (GS >= 2) y[i][r] += dpp_f<DPP_XOR1>(y[i][r]);
            if (GS == 4) y[i][r] += dpp_f<DPP_XOR2>(y[i][r]);
        }
    const bool owner = col_ok && sc == 0;
    if (DOWN) {   // rows r0 + 4b .. +3 of token tc
        if (owner) {
#pragma unroll
            for (int i = 0; i < R; ++i)
                if (i < nrt)
                    *reinterpret_cast<float4 *>(ydst + (size_t)L.dst[tc] * d + r0s[i] + 4 * b) =
                        make_float4(y[i][0], y[i][1], y[i][2], y[i][3]);
        }
        return;
    }
    // gate and up sums, in the activation area once every wave is done with it
    float(*out)[32][TT + 1] = reinterpret_cast<float(*)[32][TT + 1]>(&L.xs[0][0]);
#pragma unroll
    for (int i = 0; i < R; ++i) {
        if (i >= nrt) break;   // uniform
        lds_barrier();
        if (owner) {
#pragma unroll
            for (int r = 0; r < 4; ++r) out[w >> 1][16 * (w & 1) + 4 * b + r][tc] = y[i][r];
        }
        lds_barrier();
        if (tid < 64) {   // thread (token, 8-row block): h = coef * gelu(g) * u
            const int t = tid >> 2, s4 = tid & 3;
            const bool ok = t < nt;
            float hh[8], hl[8], X = 0.f, C = 0.f;
#pragma unroll
            for (int e8 = 0; e8 < 8; ++e8) {
                const float e = ok ? L.coef[t] * (gelu_f(out[0][8 * s4 + e8][t], a.act) *
                                                  out[1][8 * s4 + e8][t])
                                   : 0.f;
                hh[e8] = (float)(_Float16)e;
                hl[e8] = (float)(_Float16)(e - hh[e8]);
                X += e;
            }
            // even elements as they are, odd ones divided by 16, in the pair
            // order (e0,e4)(e2,e6) | (e1,e5)(e3,e7)
            const uint2 he = make_uint2(pack_h2(hh[0], hh[4]), pack_h2(hh[2], hh[6]));
            const uint2 ho = make_uint2(div16(pack_h2(hh[1], hh[5])), div16(pack_h2(hh[3], hh[7])));
            const uint2 le = make_uint2(pack_h2(hl[0], hl[4]), pack_h2(hl[2], hl[6]));
            const uint2 lo = make_uint2(div16(pack_h2(hl[1], hl[5])), div16(pack_h2(hl[3], hl[7])));
            C = ((hsum2(he.x) + hsum2(he.y)) + (hsum2(ho.x) + hsum2(ho.y))) +
                ((hsum2(le.x) + hsum2(le.y)) + (hsum2(lo.x) + hsum2(lo.y)));
            C *= 1024.f;
            X += __shfl_xor(X, 1);
            X += __shfl_xor(X, 2);
            C += __shfl_xor(C, 1);
            C += __shfl_xor(C, 2);
            if (ok) {
                const int wg = 4 * rts[i] + s4;   // word of the hidden row
                uint4 *row = hdst + (size_t)L.dst[t] * mq_row_u4(F);
                uint2 *u2 = reinterpret_cast<uint2 *>(row) + 8 * (wg >> 1) + (wg & 1);
                u2[0] = he;
                u2[2] = ho;
                u2[4] = le;
                u2[6] = lo;
                if (s4 == 0) reinterpret_cast<float2 *>(row + F / 4)[rts[i]] = make_float2(X, C);
            }
        }
    }
}

// Token list of a tile: routed item (expert, up to 16 pairs) or 16 shared
// tokens.  Returns the expert (-1: the shared expert, -2: nothing to do).
template <int PARTS, int R, int KC>
__device__ int mq_tokens(const DecodeArgs &a, bool routed, bool down, int tile,
                          MQLds<PARTS, R, KC> &L) {
    const int tid = threadIdx.x;
    int e = -1;
    if (tid < 2 * PARTS) L.zero[tid] = make_uint4(0, 0, 0, 0);
    if (routed) {
        if (tile >= (int)ld_prev(a.hdr + HDR_NITEMS)) return -2;
        const uint4 it = ld_prev(reinterpret_cast<const uint4 *>(a.items + ITEM_INTS * tile));
        e = (int)it.x;
        if (tid == 0) L.nt = min((int)it.z, TT);
        if (tid < TT) {
            const int pr = ld_prev(a.pairs + (int)it.y + min(tid, (int)it.z - 1));
            L.src[tid] = down ? pr : pr / a.k;
            L.dst[tid] = pr;
            L.coef[tid] = ld_prev(a.weights + pr);
        }
    } else {
        const int t0 = tile * TT;
        if (tid == 0) L.nt = min(TT, a.T - t0);
        if (tid < TT) {
            L.src[tid] = L.dst[tid] = min(t0 + tid, a.T - 1);
            L.coef[tid] = 1.f;
        }
    }
    lds_barrier();
    return e;
}

// Row tiles per workgroup (each staged activation chunk serves them all) and
// the residency that leaves room for their registers.  At 128 tokens: gate/up
// 115 us at one tile, 124 at two; down 64.5 at two, 66.5 at four.
constexpr int RT_GU = 1, RT_DN = 2;
constexpr int occ(int r) { return r == 1 ? 4 : r == 2 ? 3 : 2; }

// Gate/up of the shared expert (blocks [0, a_shared_blocks)) and of the
// routed expert items (the rest); a workgroup takes RT_GU row tiles of one
// item.
__global__ __launch_bounds__(256, occ(RT_GU)) void k_mq_gateup(DecodeArgs a) {
    __shared__ MQLds<1, RT_GU, KC_GU> L;
    int b = blockIdx.x;
    const bool routed = b >= a.a_shared_blocks;
    if (routed) b -= a.a_shared_blocks;
    const int F = routed ? a.f : a.fs, tiles = F / 32, wpi = (tiles + RT_GU - 1) / RT_GU;
    const int e = mq_tokens(a, routed, false, b / wpi, L);
    if (e == -2) return;
    const int nt = uniform(L.nt);
    const int rt0 = (b % wpi) * RT_GU, nrt = min(RT_GU, tiles - rt0);
    const uint8_t *blob = routed ? expert_blob(a, e) : a.shared_blob;
    uint4 *dst = routed ? a.h_r : a.h_s;
    if (nt <= 4) mq_tile<false, 4, RT_GU, KC_GU>(a, blob, F, rt0, nrt, L, nt, a.xb, dst, nullptr);
    else if (nt <= 8) mq_tile<false, 2, RT_GU, KC_GU>(a, blob, F, rt0, nrt, L, nt, a.xb, dst, nullptr);
    else mq_tile<false, 1, RT_GU, KC_GU>(a, blob, F, rt0, nrt, L, nt, a.xb, dst, nullptr);
}

// Down of the shared expert (-> y_s) and of the routed expert items (-> y_e);
// a workgroup takes RT_DN row tiles of one item.
__global__ __launch_bounds__(256, occ(RT_DN)) void k_mq_down(DecodeArgs a) {
    __shared__ MQLds<2, RT_DN, KC_DN> L;
    int b = blockIdx.x;
    const bool routed = b >= a.b_shared_blocks;
    if (routed) b -= a.b_shared_blocks;
    const int F = routed ? a.f : a.fs, tiles = a.d / 64, wpi = (tiles + RT_DN - 1) / RT_DN;
    const int e = mq_tokens(a, routed, true, b / wpi, L);
    if (e == -2) return;
    const int nt = uniform(L.nt);
    const int rt0 = (b % wpi) * RT_DN, nrt = min(RT_DN, tiles - rt0);
    const uint8_t *blob = routed ? expert_blob(a, e) : a.shared_blob;
    const uint4 *src = routed ? a.h_r : a.h_s;
    float *dst = routed ? a.y_e : a.y_s;
    if (nt <= 4) mq_tile<true, 4, RT_DN, KC_DN>(a, blob, F, rt0, nrt, L, nt, src, nullptr, dst);
    else if (nt <= 8) mq_tile<true, 2, RT_DN, KC_DN>(a, blob, F, rt0, nrt, L, nt, src, nullptr, dst);
    else mq_tile<true, 1, RT_DN, KC_DN>(a, blob, F, rt0, nrt, L, nt, src, nullptr, dst);
}

}  // namespace

// Prefill chunks: after the router launch (top-k and grouping into items of
// at most 16 tokens): gate/up, down, then the combine.
hipError_t tf_launch_prefill_tiles(const DecodeArgs &a0, int max_items, hipStream_t s) {
    DecodeArgs a = a0;
    const int ttiles = (a.T + TT - 1) / TT;
    const int wpi_s = (a.fs / 32 + RT_GU - 1) / RT_GU, wpi_r = (a.f / 32 + RT_GU - 1) / RT_GU;
    a.a_shared_blocks = ttiles * wpi_s;
    const int n_gu = a.a_shared_blocks + max_items * wpi_r;
    TF_LAUNCH(TF_KERNEL_PREFILL_GATEUP, k_mq_gateup, dim3(n_gu), dim3(WG), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int wpi_d = (a.d / 64 + RT_DN - 1) / RT_DN;
    a.b_shared_blocks = ttiles * wpi_d;
    const int n_dn = a.b_shared_blocks + max_items * wpi_d;
    TF_LAUNCH(TF_KERNEL_PREFILL_DOWN, k_mq_down, dim3(n_dn), dim3(WG), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return tf_launch_prefill_combine(a, s);
}
