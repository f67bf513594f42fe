// Decode-path kernels of the q4 MoE layer for gfx950 (CDNA4).
//
// One decode step of T <= 16 tokens through one layer is three launches on
// one stream, in the order the shilu.ai README translation
// ("推理引擎的工作原理") gives for the runtime: router, shared branch,
// routed experts, combine.
//
//   A  router rows (8-bit, fp64 sums) + shared gate/up (q4) -> h_s
//      The last router workgroup of a token runs its top-k and softmax; for
//      T > 1 the last token's top-k workgroup groups (token, rank) pairs by
//      expert so that each expert's weights are read once per step.
//   B  routed gate/up (q4, per expert item) -> h_r = p * gelu(g) * u
//      + shared down (q4) -> y_s
//   C  routed down (q4) over the token's pairs + y_s -> fp16 y
//
// Workgroups are 256 threads (4 waves).  Every wave owns an 8-row tile of one
// matrix: lanes 8r..8r+7 share row r and lane s reads the 16-byte chunks s,
// s+8, s+16, ... of that row, so each load instruction moves eight whole
// 128-byte lines.  Each workgroup issues its activation loads first and its
// weight loads second, all before any of them is consumed; loads are
// straight-line (out-of-range chunks read a clamped address and get a zero
// scale), so the compiler's in-order load counter lets chunk j be consumed
// as soon as it lands.  Activations live in LDS in the (e0,e4)(e1,e5)(e2,e6)
// (e3,e7) pairing the nibble unpack produces; the hidden activations h are
// written by their producers already split into hi/lo fp16 pairs, so the
// consumers only copy them.  No float atomics: every sum has a fixed order,
// so repeated runs are bitwise identical.
#include "tf_device.h"
#include "tf_internal.h"
#include "tf_layer.h"

using namespace tfk;

namespace {

// ----------------------------------------------------------- weight tile
// RPW = 64/LPR rows of one q4 matrix with K columns per wave: lane (r, s)
// (r = lane / LPR, s = lane % LPR) reads half-group chunks hg = LPR*j + s of
// row row0 + r.  Out-of-range chunks read the row's last chunk and are
// disabled through a zero scale/bias word.
template <int LPR, int J>
struct Tile {
    uint4 q[J];
    uint4 sv, bv;   // lane l < RPW*G/8: uint4 l of the tile's scales / biases
};

// Scale/bias loads are issued before the code loads, so that storing them to
// LDS does not wait for the codes.  The RPW rows' scales are RPW*G contiguous
// fp16 values (RPW*G/8 uint4; RPW*G is a multiple of 8 by the launch rule).
template <int LPR, int J>
__device__ __forceinline__ void tile_load_sb(Tile<LPR, J> &t, const Mat &m, int row0, int K,
                                             int lane) {
    constexpr int RPW = WAVE / LPR;
    const int G = K >> 6, NS = RPW * G / 8;
    const int l = min(lane, NS - 1);
    t.sv = reinterpret_cast<const uint4 *>(m.s + (size_t)row0 * G)[l];
    t.bv = reinterpret_cast<const uint4 *>(m.b + (size_t)row0 * G)[l];
}

template <int LPR, int J>
__device__ __forceinline__ void tile_load_q(Tile<LPR, J> &t, const Mat &m, int row0, int K,
                                            int lane) {
    const int H = K >> 5;
    const int r = lane / LPR, s = lane % LPR;
    const uint4 *qrow = reinterpret_cast<const uint4 *>(m.q + (size_t)(row0 + r) * (K >> 1));
#pragma unroll
    for (int j = 0; j < J; ++j) t.q[j] = qrow[min(LPR * j + s, H - 1)];
}

// Interleave the tile's scales and biases into LDS words (scale | bias<<16),
// [RPW][G].
template <int LPR, int J>
__device__ __forceinline__ void tile_store_sb(const Tile<LPR, J> &t, uint32_t *lsb, int G,
                                              int lane) {
    constexpr int RPW = WAVE / LPR;
    if (lane < RPW * G / 8) {
        const uint32_t s4[4] = {t.sv.x, t.sv.y, t.sv.z, t.sv.w};
        const uint32_t b4[4] = {t.bv.x, t.bv.y, t.bv.z, t.bv.w};
        uint4 o0, o1;
        o0.x = (s4[0] & 0xFFFFu) | (b4[0] << 16); o0.y = (s4[0] >> 16) | (b4[0] & 0xFFFF0000u);
        o0.z = (s4[1] & 0xFFFFu) | (b4[1] << 16); o0.w = (s4[1] >> 16) | (b4[1] & 0xFFFF0000u);
        o1.x = (s4[2] & 0xFFFFu) | (b4[2] << 16); o1.y = (s4[2] >> 16) | (b4[2] & 0xFFFF0000u);
        o1.z = (s4[3] & 0xFFFFu) | (b4[3] << 16); o1.w = (s4[3] >> 16) | (b4[3] & 0xFFFF0000u);
        reinterpret_cast<uint4 *>(lsb)[2 * lane] = o0;
        reinterpret_cast<uint4 *>(lsb)[2 * lane + 1] = o1;
    }
}

// Sum over the LPR lanes of a row group; every lane of the group gets it.
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
    v += dpp_f<DPP_XOR1>(v);
    v += dpp_f<DPP_XOR2>(v);
    v += dpp_f<DPP_HALF_MIRROR>(v);
    if (LPR == 16) v += dpp_f<DPP_MIRROR>(v);
    return v;
}

// Partial dot product of the lane's chunks with one staged activation row:
// P = pair words [4][H] (uint4), S = (X, C) per half-group.  With LO, a
// second pair row (the low part of a hi/lo split) is added into the same sums.
// The compiler barrier keeps each chunk's LDS reads next to their use
// (bounded register use; other waves on the SIMD hide the LDS latency), and
// each chunk waits only for its own code load.
template <bool LO>
struct Act {
    uint4 x[4], xl[LO ? 4 : 1];
    float2 xc;
    uint32_t sbw;
};

template <bool LO>
__device__ __forceinline__ void act_read(Act<LO> &A, const uint32_t *lsb, int G, const uint4 *P,
                                         const uint4 *PL, const float2 *S, int H, int r, int hg0) {
    const int hg = min(hg0, H - 1);
#pragma unroll
    for (int m = 0; m < 4; ++m) A.x[m] = P[m * H + hg];
    if (LO) {
#pragma unroll
        for (int m = 0; m < 4; ++m) A.xl[LO ? m : 0] = PL[m * H + hg];
    }
    A.xc = S[hg];
    A.sbw = hg0 < H ? lsb[r * G + (hg >> 1)] : 0u;
}

template <bool LO>
__device__ __forceinline__ float act_dot(const Act<LO> &A, uint4 q, float acc) {
    float de = 0.f, dd = 0.f;
    q4_chunk(q, A.x[0], A.x[1], A.x[2], A.x[3], de, dd);
    if (LO) q4_chunk(q, A.xl[0], A.xl[LO ? 1 : 0], A.xl[LO ? 2 : 0], A.xl[LO ? 3 : 0], de, dd);
    const float sc = h2f((uint16_t)(A.sbw & 0xFFFF)), bi = h2f((uint16_t)(A.sbw >> 16));
    return fmaf(sc, fmaf(dd, 0.0625f, de - A.xc.y), fmaf(bi, A.xc.x, acc));
}

template <int LPR, int J, bool LO>
__device__ __forceinline__ float tile_dot(const Tile<LPR, J> &t, const uint32_t *lsb, int G,
                                          const uint4 *P, const uint4 *PL, const float2 *S, int H,
                                          int lane) {
    const int r = lane / LPR, s = lane % LPR;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        Act<LO> cur;
        act_read<LO>(cur, lsb, G, P, PL, S, H, r, LPR * j + s);
        asm volatile("" ::: "memory");
        acc = act_dot<LO>(cur, t.q[j], acc);
        __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
}

// ------------------------------------------------------- fp16 x staging
// Up to 4 rows (row i at rp[i]) of K fp16 values, 8-value blocks, thread t
// takes blocks t, t+256, ...: loads first (xs_load), processing later
// (xs_store) so that weight loads can be issued in between.
template <int MAXI>
struct XStage {
    uint4 v[MAXI];
};

__device__ __forceinline__ const uint16_t *pick4(const uint16_t *const (&rp)[4], int row) {
    return row == 0 ? rp[0] : row == 1 ? rp[1] : row == 2 ? rp[2] : rp[3];
}

template <int MAXI>
__device__ __forceinline__ void xs_load(XStage<MAXI> &X, const uint16_t *const (&rp)[4],
                                        int rows, int K, int tid) {
    const int NB = K >> 3, NT = rows * NB;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const int bb = min(tid + WG * i, NT - 1);
        const int row = bb / NB, b = bb - row * NB;
        X.v[i] = reinterpret_cast<const uint4 *>(pick4(rp, row))[b];
    }
}

template <int MAXI>
__device__ __forceinline__ void xs_store(const XStage<MAXI> &X, int rows, int K,
                                         unsigned char *base, int tid) {
    const int H = K >> 5, NB = K >> 3, NT = rows * NB, sb = xst_bytes(K);
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const int bb = tid + WG * i;
        if (WG * i < NT) {   // uniform: all lanes run the quad sums
            const uint32_t w4[4] = {X.v[i].x, X.v[i].y, X.v[i].z, X.v[i].w};
            float xe = 0.f, xo = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xe += h2f((uint16_t)(w4[e] & 0xFFFF));
                xo += h2f((uint16_t)(w4[e] >> 16));
            }
            xe += dpp_f<DPP_XOR1>(xe);
            xe += dpp_f<DPP_XOR2>(xe);
            xo += dpp_f<DPP_XOR1>(xo);
            xo += dpp_f<DPP_XOR2>(xo);
            if (bb < NT) {
                const int row = bb / NB, b = bb - row * NB, hg = b >> 2, m = b & 3;
                unsigned char *st = base + (size_t)row * sb;
                reinterpret_cast<uint4 *>(st)[m * H + hg] = pair_halves(X.v[i]);
                if (m == 0)
                    reinterpret_cast<float2 *>(st + 64 * H)[hg] =
                        make_float2(xe + xo, fmaf(1024.f, xe, 64.f * xo));
            }
        }
    }
}

// --------------------------------------------------- hi/lo h staging
// Global hi/lo row (written by producers): 10H uint4 = hi [4H] | lo [4H] |
// per half-group four partial (X, C) pairs, one per 8-value block.  The
// consumer copies the pair words and adds the four partials in order.
template <int MAXI, int MAXS>
struct HStage {
    uint4 v[MAXI];
    uint4 s0[MAXS], s1[MAXS];
};

template <int MAXI, int MAXS>
__device__ __forceinline__ void hs_load(HStage<MAXI, MAXS> &Hs, const uint4 *src, int rows, int K,
                                        int tid) {
    const int H = K >> 5, NC = rows * 8 * H, NS = rows * H;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const int c = min(tid + WG * i, NC - 1);
        const int row = c / (8 * H), o = c - row * 8 * H;
        Hs.v[i] = src[(size_t)row * 10 * H + o];
    }
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
        const int c = min(tid + WG * i, NS - 1);
        const int row = c / H, hg = c - row * H;
        const uint4 *p = src + (size_t)row * 10 * H + 8 * H + 2 * hg;
        Hs.s0[i] = p[0];
        Hs.s1[i] = p[1];
    }
}

template <int MAXI, int MAXS>
__device__ __forceinline__ void hs_store(const HStage<MAXI, MAXS> &Hs, int rows, int K,
                                         unsigned char *base, int tid) {
    const int H = K >> 5, NC = rows * 8 * H, NS = rows * H, sb = hst_bytes(K);
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const int c = tid + WG * i;
        if (c < NC) {
            const int row = c / (8 * H), o = c - row * 8 * H;
            reinterpret_cast<uint4 *>(base + (size_t)row * sb)[o] = Hs.v[i];
        }
    }
#pragma unroll
    for (int i = 0; i < MAXS; ++i) {
        const int c = tid + WG * i;
        if (c < NS) {
            const int row = c / H, hg = c - row * H;
            const uint4 a = Hs.s0[i], b = Hs.s1[i];
            const float X = ((__uint_as_float(a.x) + __uint_as_float(a.z)) + __uint_as_float(b.x)) +
                            __uint_as_float(b.z);
            const float C = ((__uint_as_float(a.y) + __uint_as_float(a.w)) + __uint_as_float(b.y)) +
                            __uint_as_float(b.w);
            reinterpret_cast<float2 *>(base + (size_t)row * sb + 128 * H)[hg] = make_float2(X, C);
        }
    }
}

// ------------------------------------------------------------------ top-k
// Top-k of token t by (logit desc, id asc) -- or the forced ids -- and the
// softmax over the k selected logits (max-subtracted differences in fp64,
// exponentials in fp32, normalised in fp64).  Whole WG.
//
// Selection is exact on the fp64 logits, through 64-bit keys that order as
// the logits do (NaN taken as -inf, -0 as +0).  Every candidate counts the
// keys above its own, g(i) = #{j : key_j > key_i}: P threads per candidate
// each scan a contiguous share of the keys (LDS reads that every lane of the
// wave shares), and the P counts are added by lane moves.  Without exact
// ties the g of the k largest are 0 .. k-1, one candidate each, and g(i) is
// the rank; each selected candidate also counts itself into its rank's slot,
// so a tie (two candidates with the same g, a slot below k with a count
// other than one) is seen, and then every candidate counts again by the full
// rule rank(i) = g(i) + #{j < i : key_j == key_i}.
__host__ __device__ constexpr int topk_lds_bytes(int E) {
    return 8 * E + 8 * E + 4 * 16 + 4 * 16 + 16;
}

// Unsigned key ordered as the double (NaN excluded; -0 taken as +0).
__device__ __forceinline__ uint64_t order_key(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v == 0.0 ? 0.0 : v);
    return (u >> 63) ? ~u : (u | (1ull << 63));
}

// Keys above key_i among keys [j0, j1) (pairs of keys per LDS read; j0 even);
// with TIES, also the keys equal to key_i at positions below i.
template <bool TIES>
__device__ __forceinline__ int count_above(const uint64_t *key, int j0, int j1, uint64_t ki, int i) {
    int r = 0;
    int j = j0;
    for (; j + 8 <= j1; j += 8) {
        ulonglong2 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const ulonglong2 *>(key + j + 2 * u);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            r += (int)(v[u].x > ki) + (int)(v[u].y > ki);
            if (TIES) r += (int)((v[u].x == ki) & (j + 2 * u < i)) + (int)((v[u].y == ki) & (j + 2 * u + 1 < i));
        }
    }
    for (; j < j1; ++j) {
        const uint64_t kj = key[j];
        r += (int)(kj > ki);
        if (TIES) r += (int)((kj == ki) & (j < i));
    }
    return r;
}

// x of token t in the grouped kernels' B-operand form (whole WG; d <= 4096:
// one word pair per thread).
__device__ void xb_load(const DecodeArgs &a, int t, int tid, uint4 &xv0, uint4 &xv1) {
    const uint4 *xrow = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.d);
    if (tid < (a.d >> 4)) {
        xv0 = xrow[2 * tid];
        xv1 = xrow[2 * tid + 1];
    }
}
__device__ void xb_store(const DecodeArgs &a, int t, int tid, uint4 xv0, uint4 xv1) {
    const int d = a.d, NC = d >> 4;
    uint4 *row = a.xb + (size_t)t * xb_row_u4(d);
    float X = 0.f, C = 0.f;
    if (tid < NC) xb_produce(xv0, xv1, row, tid, X, C);
    // a group is four word pairs: lanes 4g .. 4g+3
    X += dpp_f<DPP_XOR1>(X);
    C += dpp_f<DPP_XOR1>(C);
    X += dpp_f<DPP_XOR2>(X);
    C += dpp_f<DPP_XOR2>(C);
    if (tid < NC && !(tid & 3)) reinterpret_cast<float2 *>(row + d / 8)[tid >> 2] = make_float2(X, C);
}
__device__ void xb_row(const DecodeArgs &a, int t, int tid) {
    uint4 xv0 = make_uint4(0, 0, 0, 0), xv1 = xv0;
    xb_load(a, t, tid, xv0, xv1);
    xb_store(a, t, tid, xv0, xv1);
}

// PART: the logits are the partial sums of an earlier launch (a.part), else
// single values written in this launch (a.logits).
template <bool PART>
__device__ void topk_block(const DecodeArgs &a, int t, int tid, unsigned char *lds, bool xb = false,
                           uint4 xv0 = {}, uint4 xv1 = {}) {
    const int E = a.E;
    uint64_t *key = reinterpret_cast<uint64_t *>(lds);        // [E] (16-byte aligned)
    double *l = reinterpret_cast<double *>(key + E);          // [E] logits
    int *sel = reinterpret_cast<int *>(l + E);                // [16] id of each rank
    int *hits = sel + 16;                                     // [16] candidates per rank
    int *tie = hits + 16;                                     // a rank below k not held once
    lds_barrier();   // the caller's LDS (router partial sums) is no longer read
    if (tid < 16) { sel[tid] = 0; hits[tid] = 0; }
    if (tid == 0) *tie = 0;
    for (int i = tid; i < E; i += WG) {
        double v;
        if (PART) {   // partial logits of an earlier launch, added in K-range order
            double pv[RMM_MAX_KR];   // all in flight at once
#pragma unroll
            for (int r = 0; r < RMM_MAX_KR; ++r)
                pv[r] = ld_prev(a.part + ((size_t)min(r, a.nkr - 1) * a.T + t) * E + i);
            v = 0.0;
#pragma unroll
            for (int r = 0; r < RMM_MAX_KR; ++r)
                if (r < a.nkr) v += pv[r];
        } else {
            v = ld_dev(a.logits + (size_t)t * E + i);
        }
        if (v != v) v = -__builtin_inf();   // NaN ranks last
        l[i] = v;
        key[i] = order_key(v);
    }
    if (xb) xb_store(a, t, tid, xv0, xv1);   // x has arrived with the logits
    lds_barrier();
    if (a.forced) {
        uint32_t fl = 0;
        if (tid < a.k) {
            int id = a.forced[(size_t)t * a.k + tid];
            if (id < 0 || id >= a.E) { fl |= TF_FLAG_ID_RANGE; id = id < 0 ? 0 : a.E - 1; }
            sel[tid] = id;
        }
        lds_barrier();
        if (tid < a.k)
            for (int r = 0; r < tid; ++r)
                if (sel[r] == sel[tid]) fl |= TF_FLAG_ID_REPEAT;
        if (fl) atomicOr(a.hdr + HDR_FLAGS, fl);
    } else {
        // P threads per candidate (adjacent lanes), P in {1, 2, 4}; candidates
        // beyond WG / P are taken in further rounds
        const int P = E <= 64 ? 4 : E <= 128 ? 2 : 1;
        const int part = tid & (P - 1), per = ((E + P - 1) / P + 1) & ~1;
        const int j0 = min(E, part * per), j1 = min(E, j0 + per);
        for (int c0 = 0; c0 < E; c0 += WG / P) {
            const int c = c0 + tid / P, cc = min(c, E - 1);
            int g = count_above<false>(key, j0, j1, key[cc], cc);
            if (P >= 2) g += __builtin_amdgcn_update_dpp(0, g, DPP_XOR1, 0xF, 0xF, false);
            if (P >= 4) g += __builtin_amdgcn_update_dpp(0, g, DPP_XOR2, 0xF, 0xF, false);
            if (c < E && part == 0 && g < a.k) {
                sel[g] = c;
                atomicAdd(&hits[g], 1);
            }
        }
        lds_barrier();
        if (tid < a.k && hits[tid] != 1) *tie = 1;
        lds_barrier();
        if (*tie) {   // exact ties: rank by the full rule
            for (int c0 = 0; c0 < E; c0 += WG / P) {
                const int c = c0 + tid / P, cc = min(c, E - 1);
                int r = count_above<true>(key, j0, j1, key[cc], cc);
                if (P >= 2) r += __builtin_amdgcn_update_dpp(0, r, DPP_XOR1, 0xF, 0xF, false);
                if (P >= 4) r += __builtin_amdgcn_update_dpp(0, r, DPP_XOR2, 0xF, 0xF, false);
                if (c < E && part == 0 && r < a.k) sel[r] = c;
            }
        }
    }
    lds_barrier();
    if (tid < WAVE) {   // lane r < k: rank r (k <= 16)
        const int r = tid, id = sel[min(r, a.k - 1)];
        const double v = l[id];
        // the largest selected logit (rank 0 without forced ids; any order is
        // exact for a maximum)
        double m = r < a.k ? v : -__builtin_inf();
        m = fmax(m, dpp_d<DPP_XOR1>(m));
        m = fmax(m, dpp_d<DPP_XOR2>(m));
        m = fmax(m, dpp_d<DPP_HALF_MIRROR>(m));
        m = fmax(m, dpp_d<DPP_MIRROR>(m));
        const double e = r < a.k ? (double)expf((float)(v - m)) : 0.0;
        // the sum in rank order, every lane adding the same sequence
        const long long eb = __builtin_bit_cast(long long, e);
        double s = 0.0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int lo = __builtin_amdgcn_readlane((int)(eb & 0xFFFFFFFF), q);
            const int hi = __builtin_amdgcn_readlane((int)(eb >> 32), q);
            if (q < a.k) s += __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned)lo);
        }
        if (r < a.k) {
            st_dev(a.ids + (size_t)t * a.k + r, (int32_t)id);
            st_dev(a.weights + (size_t)t * a.k + r, (float)(e / s));
        }
    }
}

// Group the T*k (token, rank) pairs by expert, sorted by (expert, token,
// rank): items of at most a.tbi consecutive pairs of one expert (shilu.ai
// README translation, "推理引擎的工作原理": a chunk's rows share each fetched
// expert).  An item record is ITEM_INTS ints: expert, first sorted
// position, count, 0, then -- for its first MAX_TB pairs -- the pair indices
// and their router weights, so a gate/up block learns everything it needs
// in one load.  Token t's pair with expert e lands at
// offs[e] + #{t' < t that selected e}, counted on a per-expert bit mask over
// the tokens (T <= 128) and the exclusive prefix of its words' counts, so the
// order never depends on thread timing.
// The ids and weights are read once (one round trip); the sorted order is
// built in LDS, where positions start out holding their own index, so
// repeated ids (flagged by the top-k) can never leave an out-of-range pair
// behind, and is written out at the end.  Whole WG.
constexpr int GROUP_PPT = (MAX_PREFILL_T * 16 + WG - 1) / WG;   // pairs per thread, at most
constexpr int GROUP_MAX_NW = (MAX_PREFILL_T + 31) / 32;          // mask words per expert, at most
__host__ __device__ constexpr int group_lds_bytes(int E, int T) {
    return 8 * E * ((T + 31) >> 5) + 12 * E + 8 * 4 + 4 * T * 16;
}

__device__ void group_block(const DecodeArgs &a, int tid, unsigned char *lds) {
    const int P = a.T * a.k, E = a.E, NW = (a.T + 31) >> 5;
    const int lane = tid & 63, w = tid >> 6;
    uint32_t *mask = reinterpret_cast<uint32_t *>(lds);       // [E][NW]
    int *pref = reinterpret_cast<int *>(mask + E * NW);       // [E][NW] pairs in earlier words
    int *cnt = pref + E * NW;                                 // [E]
    int *offs = cnt + E;                                      // [E]
    int *iidx = offs + E;                                     // [E] item index
    int *wsum = iidx + E;                                     // [4][2]
    int *pl = wsum + 8;                                       // [P] sorted pair order
    // this thread's pairs p = tid + WG j: expert and router weight
    int pe[GROUP_PPT];
    float pw[GROUP_PPT];
    // (loads from clamped positions, all in flight at once)
    int ev[GROUP_PPT];
#pragma unroll
    for (int j = 0; j < GROUP_PPT; ++j) {
        const int pc = min(tid + WG * j, P - 1);
        ev[j] = (int)ld_dev(a.ids + pc);
        pw[j] = a.weights ? ld_dev(a.weights + pc) : 0.f;
    }
    int pt[GROUP_PPT];   // the pairs' tokens
#pragma unroll
    for (int j = 0; j < GROUP_PPT; ++j) {
        pe[j] = min(max(ev[j], 0), E - 1);
        pt[j] = WG * j < P ? (tid + WG * j) / a.k : 0;   // (rounds beyond P: uniform skips)
    }
    const int tsh = __builtin_ctz(a.tbi);   // a power of two
    lds_barrier();
    for (int i = tid; i < E * NW; i += WG) mask[i] = 0;
    for (int i = tid; i < P; i += WG) pl[i] = i;
    lds_barrier();
#pragma unroll
    for (int j = 0; j < GROUP_PPT; ++j)
        if (tid + WG * j < P) atomicOr(&mask[pe[j] * NW + (pt[j] >> 5)], 1u << (pt[j] & 31));
    lds_barrier();
    // counts, and exclusive scans of the counts and of the item counts;
    // thread tid owns experts [tid*per, tid*per + per)
    const int per = (E + WG - 1) / WG, e0 = tid * per, e1 = min(E, e0 + per);
    int sc = 0, sn = 0;
    for (int e = e0; e < e1; ++e) {
        uint32_t m[GROUP_MAX_NW];
#pragma unroll
        for (int q = 0; q < GROUP_MAX_NW; ++q) m[q] = q < NW ? mask[e * NW + q] : 0u;
        int c = 0;
#pragma unroll
        for (int q = 0; q < GROUP_MAX_NW; ++q) {
            if (q < NW) pref[e * NW + q] = c;
            c += __popc(m[q]);
        }
        cnt[e] = c;
        sc += c;
        sn += (c + a.tbi - 1) >> tsh;
    }
    const int ic = wave_scan_incl(sc), in = wave_scan_incl(sn);
    if (lane == WAVE - 1) { wsum[2 * w] = ic; wsum[2 * w + 1] = in; }
    lds_barrier();
    int oc = ic - sc, on = in - sn;
    for (int q = 0; q < w; ++q) { oc += wsum[2 * q]; on += wsum[2 * q + 1]; }
    for (int e = e0; e < e1; ++e) {
        offs[e] = oc;
        iidx[e] = on;
        oc += cnt[e];
        on += (cnt[e] + a.tbi - 1) >> tsh;
    }
    if (tid == WG - 1) st_dev(a.hdr + HDR_NITEMS, (uint32_t)on);
    if (a.g_counts) {
        for (int e = e0; e < e1; ++e) {
            st_dev(a.g_counts + e, (int32_t)cnt[e]);
            st_dev(a.g_offsets + e, (int32_t)offs[e]);
        }
        if (tid == WG - 1) st_dev(a.g_offsets + E, (int32_t)oc);   // the total
    }
    lds_barrier();
    for (int e = tid; e < E; e += WG) {
        const int c = cnt[e], o = offs[e], ii = iidx[e];
        for (int q = 0; q < c; q += a.tbi)
            st_dev(reinterpret_cast<uint4 *>(a.items + ITEM_INTS * (ii + (q >> tsh))),
                   make_uint4((uint32_t)e, (uint32_t)(o + q), (uint32_t)min(a.tbi, c - q), 0u));
    }
    // a pair's rank within its expert: earlier words' pairs + the bits below
    // its token; every LDS read of the thread's pairs before the first use
    int rk[GROUP_PPT], po[GROUP_PPT], pi[GROUP_PPT];
#pragma unroll
    for (int j = 0; j < GROUP_PPT; ++j) {
        rk[j] = po[j] = pi[j] = 0;
        if (WG * j < P) {
            const int e = pe[j], t = pt[j], wq = e * NW + min(t >> 5, NW - 1);
            rk[j] = pref[wq] + __popc(mask[wq] & ((1u << (t & 31)) - 1u));
            po[j] = offs[e];
            pi[j] = iidx[e];
        }
    }
#pragma unroll
    for (int j = 0; j < GROUP_PPT; ++j) {
        const int p = tid + WG * j, r = rk[j];
        if (p < P) {
            const int pos = po[j] + r;
            if (pos < P) pl[pos] = p;
            const int slot = r & (a.tbi - 1);
            if (slot < MAX_TB) {
                int32_t *rec = a.items + ITEM_INTS * (pi[j] + (r >> tsh));
                st_dev(rec + 4 + slot, (int32_t)p);
                st_dev(reinterpret_cast<float *>(rec) + 8 + slot, pw[j]);
            }
        }
    }
    lds_barrier();
    for (int i = tid; i < P; i += WG) st_dev(a.pairs + i, (int32_t)pl[i]);
}

// After a token's top-k in a grouped step: the step's ticket; the last
// token's workgroup groups the pairs by expert.  With xb, the token's x in
// B-operand form is stored while the ticket is out (the grouping does not
// read it, so the ticket need not wait for those stores).
__device__ void group_after_topk(const DecodeArgs &a, int t, int tid, unsigned char *lds,
                                 bool xb = false, uint4 xv0 = {}, uint4 xv1 = {}) {
    stores_done();
    lds_barrier();
    if (tid == 0) {
        const uint32_t old = atomicAdd(a.hdr + hdr_ticket(a.T), 1u);
        reinterpret_cast<int *>(lds)[0] = old == (uint32_t)(a.T - 1);
    }
    if (xb) xb_store(a, t, tid, xv0, xv1);
    lds_barrier();
    if (!reinterpret_cast<int *>(lds)[0]) return;
    if (tid == 0) st_dev(a.hdr + hdr_ticket(a.T), 0u);
    group_block(a, tid, lds);
}

// ----------------------------------------------------- grouped router
// Router logits of a grouped step on the matrix cores, in fp64:
// l[t][e] = sum_k w[e][k] x[t][k] with w = s q + b dequantised exactly in fp64
// (s q has at most 19 significant bits and every term is a multiple of
// 2^-24 below 2^24, so the sum is exact) and x exact; every product is
// exact, only the fp64 sums round.  v_mfma_f64_16x16x4_f64 takes A[e][k]
// from lane l as A[l % 16][l / 16] and B[k][t] as B[l / 16][l % 16], and
// leaves D[l / 16 + 4 r][l % 16] in slot r of lane l (rows interleaved, unlike
// the fp32 16x16 layout).  The k index of a step is free: lane (i, kq) feeds
// columns 16 c + 4 kq + s of chunk c in step s, so it reads just its own four
// consecutive codes (one word) and x values (two words) of each chunk.
// Workgroup: a tile of 16 experts x 16 tokens over one of nkr K ranges, the
// range split in four between the waves; the wave sums are added in wave
// order and the ranges' partial logits part[kr][t][e] in range order by the
// top-k.
typedef double v4d __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_router_mm(DecodeArgs a) {
    __shared__ v4d red[3][64];
    const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
    // token tile fastest: workgroup b runs on XCD b mod 8, so with eight
    // token tiles every tile's partial logits stay in one XCD's L2, the one
    // its tokens' top-k workgroups run on
    const int ebn = (a.E + 15) >> 4, ntb = (a.T + 15) >> 4;
    int b = blockIdx.x;
    const int tb = b % ntb;
    b /= ntb;
    const int eb = b % ebn, kr = b / ebn;
    const int d = a.d, NC = d >> 4, G = d >> 6;   // 16-column chunks, groups
    const int pidx = 4 * kr + w, parts = 4 * a.nkr;
    const int c0 = (int)((long)NC * pidx / parts), c1 = (int)((long)NC * (pidx + 1) / parts);
    const int i = lane & 15, kq = lane >> 4;
    const int e = min(16 * eb + i, a.E - 1), t = min(16 * tb + i, a.T - 1);   // clamped: not stored
    const uint8_t *qrow = a.rq + (size_t)e * d + 4 * kq;
    const uint16_t *srow = a.rs + (size_t)e * G, *brow = a.rb + (size_t)e * G;
    const uint16_t *xrow = a.x + (size_t)t * d + 4 * kq;
    v4d acc = {0.0, 0.0, 0.0, 0.0};
    // a wave's chunks (at most RMM_CHUNKS, see tf_router_nkr): every load in
    // flight before the first MFMA
    uint32_t qv[RMM_CHUNKS];
    uint2 xv[RMM_CHUNKS];
    uint16_t sh[RMM_CHUNKS], bh[RMM_CHUNKS];
#pragma unroll
    for (int u = 0; u < RMM_CHUNKS; ++u) {
        const int c = min(c0 + u, NC - 1);
        qv[u] = *reinterpret_cast<const uint32_t *>(qrow + 16 * c);
        xv[u] = *reinterpret_cast<const uint2 *>(xrow + 16 * c);
        sh[u] = srow[c >> 2];
        bh[u] = brow[c >> 2];
    }
#pragma unroll
    for (int u = 0; u < RMM_CHUNKS; ++u) {
        if (c0 + u >= c1) break;   // uniform
        const double sc = (double)h2f(sh[u]), bi = (double)h2f(bh[u]);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const uint32_t code = (qv[u] >> (8 * s4)) & 0xFFu;
            const uint16_t xh = (uint16_t)((s4 < 2 ? xv[u].x : xv[u].y) >> (16 * (s4 & 1)));
            const double wv = fma(sc, (double)code, bi);
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(wv, (double)h2f(xh), acc, 0, 0, 0);
        }
    }
    if (w > 0) red[w - 1][lane] = acc;
    lds_barrier();
    if (w == 0) {
        const v4d s = ((acc + red[0][lane]) + red[1][lane]) + red[2][lane];
        const int tt = 16 * tb + i;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ee = 16 * eb + kq + 4 * r;
            if (tt < a.T && ee < a.E) a.part[((size_t)kr * a.T + tt) * a.E + ee] = s[r];
        }
    }
}

// One workgroup per token of a grouped step: x in B-operand form (decode
// steps), top-k and softmax from the partial logits, then the grouping by
// the last token's workgroup.
__global__ __launch_bounds__(256) void k_router_topk(DecodeArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    // token t of tile t / 16 on that tile's XCD (see k_router_mm) when the
    // tiles are full
    const int ntb = a.T >> 4, b = blockIdx.x, tid = threadIdx.x;
    const int t = (a.T & 15) ? b : (b % ntb) * 16 + b / ntb;
    // the x loads go out with the top-k's logit loads
    uint4 xv0 = make_uint4(0, 0, 0, 0), xv1 = xv0;
    if (a.xb) xb_load(a, t, tid, xv0, xv1);
    topk_block<true>(a, t, tid, lds, a.xb && !a.do_group, xv0, xv1);
    if (a.do_group) group_after_topk(a, t, tid, lds, a.xb != nullptr, xv0, xv1);
}

// ------------------------------------------------------------- router
// ------------------------------------------------------------- router
// ROUTER_ROWS router rows per workgroup, two waves per row: lane r of a row
// (0..127) takes the 16-element chunks r and r + 128, reading its codes and
// its x straight into registers.  Logit of expert e: sum over chunks of
// s_g * sum_i q_i x_i + b_g * sum_i x_i, products exact and every sum in
// fp64 (per lane over its chunks, then over the wave, then the two waves).
__device__ void router_block(const DecodeArgs &a, int b, int tid, unsigned char *lds) {
    const int lane = tid & 63, w = uniform(tid >> 6);
    const int nrb = (a.E + ROUTER_ROWS - 1) / ROUTER_ROWS;
    const int t = b / nrb, e0 = (b - t * nrb) * ROUTER_ROWS, e = e0 + (w >> 1);
    const int d = a.d, NC = d >> 4, G = d >> 6;
    constexpr int JR = 2;   // d <= 4096: at most 256 chunks over a row's 128 lanes
    const bool row_ok = e < a.E;
    const int er = row_ok ? e : 0;
    const int rl = (w & 1) * WAVE + lane;
    const uint4 *qrow = reinterpret_cast<const uint4 *>(a.rq + (size_t)er * d);
    const uint4 *xrow = reinterpret_cast<const uint4 *>(a.x + (size_t)t * d);
    uint4 qv[JR], x0[JR], x1[JR];
    uint32_t sbw[JR];
#pragma unroll
    for (int j = 0; j < JR; ++j) {
        const int c = min(rl + 2 * WAVE * j, NC - 1);
        qv[j] = qrow[c];
        x0[j] = xrow[2 * c];
        x1[j] = xrow[2 * c + 1];
        sbw[j] = (uint32_t)a.rs[(size_t)er * G + (c >> 2)] |
                 ((uint32_t)a.rb[(size_t)er * G + (c >> 2)] << 16);
    }
    double *part = reinterpret_cast<double *>(lds);   // [4] wave sums
    int *flag = reinterpret_cast<int *>(part + 4);
    if (a.xb && b == t * nrb) xb_row(a, t, tid);   // the token's first router workgroup
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < JR; ++j) {
        const int c0 = rl + 2 * WAVE * j;
        const uint32_t w4[4] = {qv[j].x, qv[j].y, qv[j].z, qv[j].w};
        const uint32_t w8[8] = {x0[j].x, x0[j].y, x0[j].z, x0[j].w, x1[j].x, x1[j].y, x1[j].z, x1[j].w};
        double D = 0.0, s16 = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double v0 = (double)h2f((uint16_t)(w8[i] & 0xFFFF));
            const double v1 = (double)h2f((uint16_t)(w8[i] >> 16));
            s16 += v0 + v1;
            D = fma((double)((w4[i >> 1] >> (16 * (i & 1))) & 0xFF), v0, D);
            D = fma((double)((w4[i >> 1] >> (16 * (i & 1) + 8)) & 0xFF), v1, D);
        }
        const uint32_t sw = (c0 < NC && row_ok) ? sbw[j] : 0u;
        acc = fma((double)h2f((uint16_t)(sw & 0xFFFF)), D, fma((double)h2f((uint16_t)(sw >> 16)), s16, acc));
    }
    acc = wave_sum_f64(acc);
    if (lane == 0) part[w] = acc;
    lds_barrier();
    if (tid < ROUTER_ROWS && e0 + tid < a.E)
        st_dev(a.logits + (size_t)t * a.E + e0 + tid, part[2 * tid] + part[2 * tid + 1]);
    stores_done();
    lds_barrier();
    if (tid == 0) {
        const uint32_t old = atomicAdd(a.hdr + hdr_ticket(t), 1u);
        *flag = old == (uint32_t)(nrb - 1);
    }
    lds_barrier();
    if (!*flag) return;
    if (tid == 0) st_dev(a.hdr + hdr_ticket(t), 0u);
    topk_block<false>(a, t, tid, lds);
    if (a.do_group && a.T > 1) group_after_topk(a, t, tid, lds);
    if (a.sc.slot_of && tid < WAVE) {   // one token: the slot lookup of its ids (rank order)
        const int *sel = reinterpret_cast<const int *>(lds + 16 * (size_t)a.E);
        slotk::lookup_wave(a.sc, a.sc_layer, sel, a.k, nullptr, false, tid);
    }
}

// ------------------------------------------------------- gate/up block
// 2*RPW output rows of (gate, up): waves 0/1 gate rows [0, RPW) / [RPW,
// 2 RPW), waves 2/3 the same up rows; h = coef * gelu(g) * u, written as
// hi/lo rows.  routed == false: the shared expert for tokens
// [b / tiles * tbx, +tbx) -> h_s; routed == true: expert item b / tiles ->
// h_r[pair].  An item has at most MAX_TB tokens, staged together.
template <int LPR, int J, bool routed>
__device__ void gateup_block(const DecodeArgs &a, int b, int tid, unsigned char *lds) {
    constexpr int RPW = WAVE / LPR, RWG = 2 * RPW;
    const int lane = tid & 63, w = uniform(tid >> 6);
    const int F = routed ? a.f : a.fs;
    const int tiles = F / RWG;
    const int item = b / tiles, rb = b - item * tiles;
    const int d = a.d, H = d >> 5, G = d >> 6;
    float *gu = reinterpret_cast<float *>(lds);                      // [4*RPW][MAX_TB]
    float *hv = gu + 4 * RPW * MAX_TB;                               // [MAX_TB][RWG]
    uint32_t *lsb = reinterpret_cast<uint32_t *>(hv + RWG * MAX_TB); // [4][RPW*G]
    unsigned char *xst = reinterpret_cast<unsigned char *>(lsb + 4 * RPW * G);

    // the item: expert e and nt token slots; slot i -> x row, output row, coef
    // (mode 0: shared, tokens base + i; 1: a single slot; 3: item pairs from
    // the item record)
    int nt, e = 0, base = 0, mode, row1 = 0, xrow1 = 0;
    float coef1 = 1.f;
    int rp4[MAX_TB] = {0, 0, 0, 0};
    float cf4[MAX_TB] = {0.f, 0.f, 0.f, 0.f};
    if (!routed) {
        base = item * a.tbx;
        nt = min(a.tbx, a.T - base);
        mode = 0;
    } else if (a.gemv_slot) {
        if (item >= a.P) return;
        nt = 1;
        mode = 1;
        e = a.gemv_slot[item];
        row1 = item;
        coef1 = a.gemv_coef ? a.gemv_coef[item] : 1.f;
        xrow1 = a.gemv_token ? a.gemv_token[item] : item;
    } else if (a.T == 1) {
        if (item >= a.k) return;
        nt = 1;
        mode = 1;
        e = ld_prev(a.ids + item);
        row1 = item;
        coef1 = ld_prev(a.weights + item);
    } else {
        if (item >= (int)ld_prev(a.hdr + HDR_NITEMS)) return;
        // at most MAX_TB pairs: all of them are in the item record
        const uint4 *rec = reinterpret_cast<const uint4 *>(a.items + ITEM_INTS * item);
        const uint4 it = ld_prev(rec), pp = ld_prev(rec + 1), cc = ld_prev(rec + 2);
        e = (int)it.x;
        nt = min((int)it.z, MAX_TB);
        const int pmax = a.T * a.k - 1;
        rp4[0] = min((int)pp.x, pmax); rp4[1] = min((int)pp.y, pmax);
        rp4[2] = min((int)pp.z, pmax); rp4[3] = min((int)pp.w, pmax);
        cf4[0] = __uint_as_float(cc.x); cf4[1] = __uint_as_float(cc.y);
        cf4[2] = __uint_as_float(cc.z); cf4[3] = __uint_as_float(cc.w);
        mode = 3;
    }
    int prow[MAX_TB];
    float coef[MAX_TB];
    const uint16_t *rp[4];
    auto rows = [&](int s0, int ns) {
#pragma unroll
        for (int i = 0; i < MAX_TB; ++i) {
            const int si = s0 + min(i, ns - 1);
            int xr = xrow1, orow = row1;
            float c = coef1;
            if (mode == 0) {
                xr = orow = base + si;
                c = 1.f;
            } else if (mode == 3) {
                const int pr = si == 0 ? rp4[0] : si == 1 ? rp4[1] : si == 2 ? rp4[2] : rp4[3];
                xr = pr / a.k;
                orow = pr;
                c = si == 0 ? cf4[0] : si == 1 ? cf4[1] : si == 2 ? cf4[2] : cf4[3];
            }
            prow[i] = orow;
            coef[i] = c;
            rp[i] = a.x + (size_t)xr * d;
        }
    };
    Mat g, u, dn;
    blob_mats(routed ? expert_blob(a, e) : a.shared_blob, d, F, g, u, dn);
    Tile<LPR, J> tl;
    const Mat &mm = (w >> 1) ? u : g;
    const int row0 = rb * RWG + RPW * (w & 1);
    const int xsb = xst_bytes(d);
    // compute one pass of ns tokens from the staged rows and write their h
    auto finish = [&](int ns) {
        auto one = [&](int i) {
            const unsigned char *st = xst + (size_t)i * xsb;
            const float v = row_sum<LPR>(tile_dot<LPR, J, false>(
                tl, lsb + w * RPW * G, G, reinterpret_cast<const uint4 *>(st), nullptr,
                reinterpret_cast<const float2 *>(st + 64 * H), H, lane));
            if (lane % LPR == 0) gu[(w * RPW + lane / LPR) * MAX_TB + i] = v;
        };
        if (ns == 1) {
            one(0);   // straight line: chunk j waits only for its own load
        } else {
            for (int i = 0; i < ns; ++i) one(i);
        }
        lds_barrier();
        if (tid < RWG * ns) {
            const int row = tid % RWG, i = tid / RWG;
            const int half = row / RPW, rr = row % RPW;
            const float gv = gu[(half * RPW + rr) * MAX_TB + i];
            const float uv = gu[((2 + half) * RPW + rr) * MAX_TB + i];
            hv[i * RWG + row] = gelu_f(gv, a.act) * uv;
        }
        lds_barrier();
        if (tid < (RWG / 8) * ns) {
            const int i = tid / (RWG / 8), sub = tid % (RWG / 8);
            const float c = coef[0] * (i == 0) + coef[1] * (i == 1) + coef[2] * (i == 2) +
                            coef[3] * (i == 3);
            const int pr = i == 0 ? prow[0] : i == 1 ? prow[1] : i == 2 ? prow[2] : prow[3];
            float ev[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) ev[q] = c * hv[i * RWG + 8 * sub + q];
            uint4 *dst = (routed ? a.h_r : a.h_s) + (size_t)pr * (10 * (F >> 5));
            hs_produce(dst, F, rb * (RWG / 8) + sub, ev);
        }
    };
    // first pass: activation loads, then weight loads, then activation processing
    XStage<(J * LPR + 15) / 16> X;   // <= 4 rows of d/8 <= 4*J*LPR blocks over 256 threads
    const int ns0 = min(MAX_TB, nt);
    rows(0, ns0);
    xs_load(X, rp, ns0, d, tid);
    tile_load_sb<LPR, J>(tl, mm, row0, d, lane);
    tile_load_q<LPR, J>(tl, mm, row0, d, lane);
    xs_store(X, ns0, d, xst, tid);
    tile_store_sb(tl, lsb + w * RPW * G, G, lane);
    lds_barrier();
    finish(ns0);
}

// --------------------------------------------------------- shared down
// 4*RPW output rows (RPW per wave) of the shared down projection for tokens
// b / tiles: y_s[t][row].
template <int LPR, int J>
__device__ void shared_down_block(const DecodeArgs &a, int b, int tid, unsigned char *lds) {
    constexpr int RPW = WAVE / LPR;
    const int lane = tid & 63, w = uniform(tid >> 6);
    const int tiles = a.d / (4 * RPW);
    const int t0 = b / tiles, rb = b - t0 * tiles;
    const int K = a.fs, H = K >> 5, G = K >> 6;
    uint32_t *lsb = reinterpret_cast<uint32_t *>(lds);               // [4][RPW*G]
    unsigned char *hst = reinterpret_cast<unsigned char *>(lsb + 4 * RPW * G);
    HStage<(J * LPR + 31) / 32, (J * LPR + 255) / 256> Hs;   // 1 row: 8H copies, H sums
    hs_load(Hs, a.h_s + (size_t)t0 * 10 * H, 1, K, tid);
    Mat g, u, dn;
    blob_mats(a.shared_blob, a.d, a.fs, g, u, dn);
    const int row0 = rb * 4 * RPW + RPW * w;
    Tile<LPR, J> tl;
    tile_load_sb<LPR, J>(tl, dn, row0, K, lane);
    tile_load_q<LPR, J>(tl, dn, row0, K, lane);
    hs_store(Hs, 1, K, hst, tid);
    tile_store_sb(tl, lsb + w * RPW * G, G, lane);
    lds_barrier();
    auto one = [&](int i) {
        const float v = row_sum<LPR>(tile_dot<LPR, J, true>(
            tl, lsb + w * RPW * G, G, reinterpret_cast<const uint4 *>(hst),
            reinterpret_cast<const uint4 *>(hst + 64 * H),
            reinterpret_cast<const float2 *>(hst + 128 * H), H, lane));
        if (lane % LPR == 0) a.y_s[(size_t)(t0 + i) * a.d + row0 + lane / LPR] = v;
    };
    one(0);
}

template <int LPR, int J>
__global__ __launch_bounds__(256, 4) void k_stage_a(DecodeArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x;
    int b = blockIdx.x;
    if (b < a.a_copy_blocks) {   // the slot-cache miss copies, first so that they start first
        const int r = b / a.copy_per;
        slotk::copy_missed(a.sc.miss_gpu + (size_t)a.sc_layer * (1 + 2 * a.k), a.sc_host, a.sc_slots,
                           a.stride, a.E, a.sc.S, a.sc.nfill, r, b - r * a.copy_per, a.copy_per, tid);
        return;
    }
    b -= a.a_copy_blocks;
    if (b < a.a_router_blocks)
        router_block(a, b, tid, lds);
    else
        gateup_block<LPR, J, false>(a, b - a.a_router_blocks, tid, lds);
}

// A router launch with no other roles (grouped steps, the router alone):
// router rows, and the top-k and grouping that their last workgroups run, at
// a fraction of k_stage_a's registers, so that every workgroup is resident
// at once.
__global__ __launch_bounds__(256) void k_router_rows(DecodeArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    router_block(a, blockIdx.x, threadIdx.x, lds);
}

template <int LPR, int J>
__global__ __launch_bounds__(256, 4) void k_stage_b(DecodeArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int b = blockIdx.x, tid = threadIdx.x;
    if (b < a.b_routed_blocks)
        gateup_block<LPR, J, true>(a, b, tid, lds);
    else
        shared_down_block<LPR, J>(a, b - a.b_routed_blocks, tid, lds);
}

// ---------------------------------------------- routed down + combine
// One 8-row output tile of one token (8 lanes per row); the token's pairs
// are split across the four waves (pairs w and w+4 of each pass of up to 8),
// and the waves' partial sums are added in wave order.  Layer: y = y_s + sum
// -> fp16 (and y32); standalone GEMV: y32 += sum.
template <int JF>
__global__ __launch_bounds__(256, 4) void k_stage_c(DecodeArgs a) {
    constexpr int LPR = 8;
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
    const int tiles = a.d >> 3;
    const int t = blockIdx.x / tiles, tile = blockIdx.x - t * tiles;
    const int row0 = tile * 8, K = a.f, H = K >> 5, G = K >> 6;
    float *part = reinterpret_cast<float *>(lds);                  // [4][8]
    uint32_t *lsb = reinterpret_cast<uint32_t *>(part + 32);       // [4 waves][2][8*G]
    unsigned char *hst = reinterpret_cast<unsigned char *>(lsb + 8 * 8 * G);
    const int hsb = hst_bytes(K);
    int lo, hi;
    if (a.gemv_slot) {
        if (a.gemv_token) {   // pairs are grouped by token: binary search
            int l0 = 0, h0 = a.P;
            while (l0 < h0) { const int mid = (l0 + h0) >> 1; if (a.gemv_token[mid] < t) l0 = mid + 1; else h0 = mid; }
            lo = l0;
            h0 = a.P;
            while (l0 < h0) { const int mid = (l0 + h0) >> 1; if (a.gemv_token[mid] <= t) l0 = mid + 1; else h0 = mid; }
            hi = l0;
        } else {
            lo = t; hi = t + 1;
        }
    } else {
        lo = t * a.k; hi = lo + a.k;
    }
    float acc = 0.f;
    for (int p0 = lo; p0 < hi; p0 += KC_BATCH) {
        const int np = min(KC_BATCH, hi - p0);
        const int pa = min(p0 + w, hi - 1), pb = min(p0 + w + 4, hi - 1);
        const bool va = w < np, vb = w + 4 < np;
        const int ea = a.gemv_slot ? a.gemv_slot[pa] : a.ids[pa];
        const int eb = a.gemv_slot ? a.gemv_slot[pb] : a.ids[pb];
        if (p0 != lo) lds_barrier();   // the previous pass is done with LDS
        HStage<(JF * 8 * 8 * 8 + 255) / 256, (JF * 8 * 8 + 255) / 256> Hs;   // 8 rows
        hs_load(Hs, a.h_r + (size_t)p0 * 10 * H, np, K, tid);
        Mat ga, ua, da, gb, ub, db;
        Tile<LPR, JF> ta, tb;
        blob_mats(expert_blob(a, ea), a.d, a.f, ga, ua, da);
        blob_mats(expert_blob(a, eb), a.d, a.f, gb, ub, db);
        tile_load_sb<LPR, JF>(ta, da, row0, K, lane);
        tile_load_sb<LPR, JF>(tb, db, row0, K, lane);
        tile_load_q<LPR, JF>(ta, da, row0, K, lane);
        tile_load_q<LPR, JF>(tb, db, row0, K, lane);
        hs_store(Hs, np, K, hst, tid);
        tile_store_sb(ta, lsb + (w * 2) * 8 * G, G, lane);
        tile_store_sb(tb, lsb + (w * 2 + 1) * 8 * G, G, lane);
        lds_barrier();
        if (va) {
            const unsigned char *st = hst + (size_t)(pa - p0) * hsb;
            acc += tile_dot<LPR, JF, true>(ta, lsb + (w * 2) * 8 * G, G,
                                           reinterpret_cast<const uint4 *>(st),
                                           reinterpret_cast<const uint4 *>(st + 64 * H),
                                           reinterpret_cast<const float2 *>(st + 128 * H), H,
                                           lane);
        }
        if (vb) {
            const unsigned char *st = hst + (size_t)(pb - p0) * hsb;
            acc += tile_dot<LPR, JF, true>(tb, lsb + (w * 2 + 1) * 8 * G, G,
                                           reinterpret_cast<const uint4 *>(st),
                                           reinterpret_cast<const uint4 *>(st + 64 * H),
                                           reinterpret_cast<const float2 *>(st + 128 * H), H,
                                           lane);
        }
    }
    acc = row_sum<LPR>(acc);
    if ((lane & 7) == 0) part[w * 8 + (lane >> 3)] = acc;
    lds_barrier();
    if (tid < 8) {
        const float sum = ((part[tid] + part[8 + tid]) + part[16 + tid]) + part[24 + tid];
        const size_t o = (size_t)t * a.d + row0 + tid;
        if (a.gemv_slot) {
            a.y32[o] = a.y32[o] + sum;
        } else {
            const float y = a.y_s[o] + sum;
            if (a.y32) a.y32[o] = y;
            a.y[o] = f2h(y);
        }
    }
}

// ------------------------------------------------ routed down, decode step
// Layer decode (not the standalone GEMV): one workgroup per (pair, 32-row
// tile), a wave per 8 rows (8 lanes per row); the pair's hidden row is
// staged once (it already carries the router weight).  Each workgroup
// stores its rows of y_e[pair]; the last of the token's k pairs to finish a
// tile (a ticket) forms y = y_s + sum over ranks of y_e in rank order ->
// fp16 (and y32).
template <int JF>
__global__ __launch_bounds__(256, 4) void k_stage_c1(DecodeArgs a) {
    constexpr int LPR = 8, RPW = 64 / LPR;
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
    const int tiles = a.d >> 5;
    const int pair = blockIdx.x / tiles, tile = blockIdx.x - pair * tiles, t = pair / a.k;
    const int row0 = 32 * tile + RPW * w, K = a.f, H = K >> 5, G = K >> 6;
    uint32_t *lsb = reinterpret_cast<uint32_t *>(lds);                    // [4 waves][RPW * G]
    unsigned char *hst = reinterpret_cast<unsigned char *>(lsb + 4 * RPW * G);
    int *flag = reinterpret_cast<int *>(hst + hst_bytes(K));
    HStage<(JF * 64 + 255) / 256, (JF * 8 + 255) / 256> Hs;
    hs_load(Hs, a.h_r + (size_t)pair * 10 * H, 1, K, tid);
    Mat g, u, dn;
    blob_mats(expert_blob(a, a.ids[pair]), a.d, a.f, g, u, dn);
    Tile<LPR, JF> tl;
    tile_load_sb<LPR, JF>(tl, dn, row0, K, lane);
    tile_load_q<LPR, JF>(tl, dn, row0, K, lane);
    hs_store(Hs, 1, K, hst, tid);
    tile_store_sb(tl, lsb + w * RPW * G, G, lane);
    lds_barrier();
    const float v = row_sum<LPR>(tile_dot<LPR, JF, true>(
        tl, lsb + w * RPW * G, G, reinterpret_cast<const uint4 *>(hst),
        reinterpret_cast<const uint4 *>(hst + 64 * H), reinterpret_cast<const float2 *>(hst + 128 * H),
        H, lane));
    if (lane % LPR == 0) st_dev(a.y_e + (size_t)pair * a.d + row0 + lane / LPR, v);
    stores_done();
    lds_barrier();
    uint32_t *tk = a.ctk + 32 * (t * tiles + tile);
    if (tid == 0) {
        const uint32_t old = atomicAdd(tk, 1u);
        *flag = old == (uint32_t)(a.k - 1);
    }
    lds_barrier();
    if (!*flag) return;
    if (tid == 0) st_dev(tk, 0u);
    if (tid < 32) {
        const size_t o = (size_t)t * a.d + 32 * tile + tid;
        // every rank's value in flight at once, then added in rank order
        float yv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            yv[r] = ld_dev(a.y_e + (size_t)(t * a.k + min(r, a.k - 1)) * a.d + 32 * tile + tid);
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (r < a.k) sum += yv[r];
        const float y = a.y_s[o] + sum;
        if (a.y32) a.y32[o] = y;
        a.y[o] = f2h(y);
    }
}

// ------------------------------------------------------ prefill combine
// Combine: y[t] = y_s[t] + sum over ranks r of y_e[t*k + r], in rank order,
// then fp16 round to nearest even (and the fp32 value when asked).
__global__ __launch_bounds__(256) void k_pf_combine(DecodeArgs a) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)a.T * a.d) return;
    const size_t t = i / a.d, c = i - t * a.d;
    // every rank's value in flight at once, then added in rank order
    float yv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) yv[r] = a.y_e[(t * a.k + min(r, a.k - 1)) * a.d + c];
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        if (r < a.k) s += yv[r];
    const float y = a.y_s[i] + s;
    if (a.y32) a.y32[i] = y;
    a.y[i] = f2h(y);
}

__global__ __launch_bounds__(256) void k_group(DecodeArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    group_block(a, threadIdx.x, lds);
}

// Read-only stream with the GEMVs' load pattern (16 bytes per lane, each
// wave's load instruction covering whole 128-byte lines), for calibrating
// memory counters: XOR of every word, stored only if it equals a value no
// real input produces, so no load can be dropped.
__global__ __launch_bounds__(256) void k_stream_read(const uint4 *p, size_t n16, uint32_t *sink) {
    uint32_t acc = 0;
    const size_t step = (size_t)gridDim.x * 256 * 4;
    for (size_t i = (size_t)blockIdx.x * 1024 + threadIdx.x; i < n16; i += step) {
        uint4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = i + 256 * j < n16 ? p[i + 256 * j] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    if (acc == 0x9e3779b9u && sink) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void k_zero(uint32_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// LDS bytes of each stage (mirrors the device layouts above).
int gateup_lds(const DecodeArgs &a, int lpr, int rows) {
    const int rpw = 64 / lpr;
    return 4 * 4 * rpw * MAX_TB + 4 * 2 * rpw * MAX_TB + 4 * 4 * rpw * (a.d >> 6) +
           rows * xst_bytes(a.d);
}

int lds_a(const DecodeArgs &a, int lpr) {
    int r = 0;
    if (a.a_router_blocks) {
        const int route = 8 * 4 + 16;   // wave sums and the ticket flag
        const int topk = topk_lds_bytes(a.E);
        const int group = a.do_group ? group_lds_bytes(a.E, a.T) : 0;
        r = max(route, max(topk, group));
    }
    int s = 0;
    if (a.a_shared_blocks) s = gateup_lds(a, lpr, min(a.tbx, MAX_TB));
    return max(r, s);
}

int lds_b(const DecodeArgs &a, int lpr) {
    const int rpw = 64 / lpr;
    int r = 0, s = 0;
    if (a.b_routed_blocks) r = gateup_lds(a, lpr, a.T > 1 && !a.gemv_slot ? min(a.T, MAX_TB) : 1);
    if (a.b_shared_blocks) s = 4 * 4 * rpw * (a.fs >> 6) + hst_bytes(a.fs);
    return max(r, s);
}

int lds_c(const DecodeArgs &a) {
    return 4 * 32 + 4 * 8 * 8 * (a.f >> 6) + KC_BATCH * hst_bytes(a.f);
}
int lds_c1(const DecodeArgs &a) { return 4 * 4 * 8 * (a.f >> 6) + hst_bytes(a.f) + 16; }

template <int LPR, int J>
hipError_t launch_ab(const DecodeArgs &a, int which, hipStream_t s) {
    if (which & STAGE_A) {
        const int n = a.a_copy_blocks + a.a_router_blocks + a.a_shared_blocks;
        if (n && n == a.a_router_blocks)
            TF_LAUNCH(TF_KERNEL_ROUTER_SHARED_GATEUP, k_router_rows, dim3(n), dim3(WG), lds_a(a, LPR), s, a);
        else if (n)
            TF_LAUNCH(TF_KERNEL_ROUTER_SHARED_GATEUP, (k_stage_a<LPR, J>), dim3(n), dim3(WG),
                      lds_a(a, LPR), s, a);
    }
    if (which & STAGE_B) {
        const int n = a.b_routed_blocks + a.b_shared_blocks;
        if (n)
            TF_LAUNCH(TF_KERNEL_ROUTED_GATEUP_SHARED_DOWN, (k_stage_b<LPR, J>), dim3(n), dim3(WG),
                      lds_b(a, LPR), s, a);
    }
    return hipGetLastError();
}

template <int JF>
hipError_t launch_c(const DecodeArgs &a, hipStream_t s) {
    if (!a.gemv_slot) {   // layer decode: per (pair, 32-row tile), last pair combines
        const int n = a.T * a.k * (a.d >> 5);
        if (n) TF_LAUNCH(TF_KERNEL_DOWN_COMBINE, k_stage_c1<JF>, dim3(n), dim3(WG), lds_c1(a), s, a);
        return hipGetLastError();
    }
    const int n = a.T * (a.d >> 3);
    if (n) TF_LAUNCH(TF_KERNEL_DOWN_COMBINE, k_stage_c<JF>, dim3(n), dim3(WG), lds_c(a), s, a);
    return hipGetLastError();
}

thread_local int g_prof_kernel = 0;
thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;

}  // namespace

#define TF_J_SWITCH(J, CALL)                         \
    switch (J) {                                     \
        case 1: CALL(1); break;                      \
        case 2: CALL(2); break;                      \
        case 3: CALL(3); break;                      \
        case 4: CALL(4); break;                      \
        case 5: case 6: CALL(6); break;              \
        case 7: case 8: CALL(8); break;              \
        case 9: case 10: case 11: CALL(11); break;   \
        case 12: CALL(12); break;                    \
        default: CALL(16); break;                    \
    }

void tf_arm_profile(int kernel, hipEvent_t start, hipEvent_t stop) {
    g_prof_kernel = kernel;
    g_prof_start = start;
    g_prof_stop = stop;
}

bool tf_take_profile(int kernel, hipEvent_t *start, hipEvent_t *stop) {
    if (!g_prof_kernel || g_prof_kernel != kernel) return false;
    *start = g_prof_start;
    *stop = g_prof_stop;
    g_prof_kernel = 0;
    return true;
}

// Stages A/B: 16 lanes per row when every K they read has an even number of
// 64-groups (so 4 rows of scales fill whole 16-byte loads), else 8;
// J = 16-byte chunks per lane = ceil(K / (32 * LPR)) for the larger K.
// Stage C: 8 lanes per row, J = ceil(d_ff / 256).
int tf_decode_lpr(const DecodeArgs &a) {
    return ((a.d >> 6) % 2 == 0 && (a.fs >> 6) % 2 == 0) ? 16 : 8;
}

hipError_t tf_launch_decode(const DecodeArgs &a, int which, hipStream_t s) {
    hipError_t e = hipSuccess;
    if (which & (STAGE_A | STAGE_B)) {
        const int K = a.d > a.fs ? a.d : a.fs;
        if (tf_decode_lpr(a) == 16) {
            const int J = (K + 511) / 512;
#define TF_CALL_AB(JJ) e = launch_ab<16, JJ>(a, which, s)
            TF_J_SWITCH(J, TF_CALL_AB)
#undef TF_CALL_AB
        } else {
            const int J = (K + 255) / 256;
#define TF_CALL_AB(JJ) e = launch_ab<8, JJ>(a, which, s)
            TF_J_SWITCH(J, TF_CALL_AB)
#undef TF_CALL_AB
        }
        if (e != hipSuccess) return e;
    }
    if (which & STAGE_C) {
        const int J = (a.f + 255) / 256;
#define TF_CALL_C(JJ) e = launch_c<JJ>(a, s)
        TF_J_SWITCH(J, TF_CALL_C)
#undef TF_CALL_C
    }
    return e;
}

int tf_router_nkr(int d) {
    // K ranges of four waves each, every wave at most RMM_CHUNKS 16-column chunks
    return (d / 16 + 4 * RMM_CHUNKS - 1) / (4 * RMM_CHUNKS);
}

hipError_t tf_launch_router_grouped(const DecodeArgs &a, hipStream_t s) {
    const int tiles = ((a.E + 15) / 16) * ((a.T + 15) / 16);
    TF_LAUNCH(TF_KERNEL_ROUTER_SHARED_GATEUP, k_router_mm, dim3(tiles * a.nkr), dim3(WG), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int lds = max(topk_lds_bytes(a.E), a.do_group ? group_lds_bytes(a.E, a.T) : 0);
    TF_LAUNCH(TF_KERNEL_ROUTER_TOPK, k_router_topk, dim3(a.T), dim3(WG), lds, s, a);
    return hipGetLastError();
}

hipError_t tf_launch_group(const DecodeArgs &a, hipStream_t s) {
    TF_LAUNCH(TF_KERNEL_GROUP, k_group, dim3(1), dim3(WG), group_lds_bytes(a.E, a.T), s, a);
    return hipGetLastError();
}

// Prefill: y = y_s + sum over ranks of y_e -> fp16.
hipError_t tf_launch_prefill_combine(const DecodeArgs &a, hipStream_t s) {
    const size_t n = (size_t)a.T * a.d;
    TF_LAUNCH(TF_KERNEL_PREFILL_COMBINE, k_pf_combine, dim3((unsigned)((n + 255) / 256)), dim3(WG), 0,
              s, a);
    return hipGetLastError();
}

hipError_t tf_launch_stream_read(const void *p, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    if (!n16) return hipSuccess;
    size_t blocks = (n16 + 1023) / 1024;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint4 *>(p), n16, (uint32_t *)nullptr);
    return hipGetLastError();
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
