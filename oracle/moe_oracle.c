/*
 * fp64 CPU oracle for the q4 MoE layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the smoke check and the benchmark's cpu_baseline leg load this
 * library.  It shares no code, header or table with the HIP path.
 *
 * What it computes (the plain definition, in fp64):
 *   affine dequantisation  w = scale * q + bias, q unsigned, group of 64
 *     (sh.edu-sjtu.cn article, section "三件事": MLX affine 4-bit, group-64
 *      scaling, 8-bit router; shilu.ai README translation, "状态和范围")
 *   quantised mat-vec      y_r = sum_i w_ri * x_i
 *   GELU                   gelu(z) = z * Phi(z) = 0.5 z (1 + erf(z / sqrt 2))
 *   expert FFN             W_down (gelu(W_gate x) (.) (W_up x))
 *   top-k                  (logit descending, id ascending), ids in rank order
 *   softmax                over the k selected logits, max-subtracted
 * Each weight is dequantised on the fly to fp64; s*q+b is exact in fp64 for
 * every fp16 s, b and q <= 255, and so is the fp16 -> fp64 cast of x.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC moe_oracle.c -lm -o liboracle.so
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* IEEE 754 binary16 -> binary64, written from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 is
 * zero/subnormal (value = f * 2^-24), exponent 31 is inf/NaN. */
double orc_half_to_double(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return s ? -v : v;
}

void orc_halves_to_double(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_half_to_double(h[i]);
}

/* Code of element j of one row: 4-bit -> byte j/2, low nibble for even j. */
static inline unsigned code_at(const uint8_t *row, int j, int bits)
{
    if (bits == 8) return row[j];
    uint8_t b = row[j >> 1];
    return (j & 1) ? (b >> 4) : (b & 15);
}

/* Dequantised weight W[r][j] in fp64. */
double orc_weight(const uint8_t *q, const uint16_t *scale, const uint16_t *bias,
                  int n, int k, int bits, int r, int j)
{
    (void)n;
    int ng = k / 64, g = j / 64;
    const uint8_t *row = q + (int64_t)r * k * bits / 8;
    double s = orc_half_to_double(scale[(int64_t)r * ng + g]);
    double b = orc_half_to_double(bias[(int64_t)r * ng + g]);
    return s * (double)code_at(row, j, bits) + b;
}

/* y[r] = sum_j W[r][j] * x[j], every weight dequantised to fp64 on the fly.
 * Rows are independent; OpenMP splits them across threads. */
void orc_qmatvec(const uint8_t *q, const uint16_t *scale, const uint16_t *bias,
                 int n, int k, int bits, const double *x, double *y)
{
    int ng = k / 64;
    #pragma omp parallel for schedule(static)
    for (int r = 0; r < n; ++r) {
        const uint8_t *row = q + (int64_t)r * k * bits / 8;
        double acc = 0.0;
        for (int g = 0; g < ng; ++g) {
            /* one scale and one bias per group of 64 elements */
            double s = orc_half_to_double(scale[(int64_t)r * ng + g]);
            double b = orc_half_to_double(bias[(int64_t)r * ng + g]);
            for (int j = 64 * g; j < 64 * g + 64; ++j) {
                double w = s * (double)code_at(row, j, bits) + b;
                acc += w * x[j];
            }
        }
        y[r] = acc;
    }
}

double orc_gelu(double z, int tanh_form)
{
    if (tanh_form) {
        const double c = sqrt(2.0 / M_PI);
        return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
    }
    return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));
}

/* Selection of the k largest logits: ids ordered by (logit descending,
 * id ascending).  A plain selection sort over an index array, so that exact
 * ties fall to the lowest id. */
void orc_topk(const double *logits, int E, int k, int32_t *ids)
{
    int *idx = (int *)malloc(sizeof(int) * E);
    for (int i = 0; i < E; ++i) idx[i] = i;
    for (int a = 0; a < k; ++a) {
        int best = a;
        for (int b = a + 1; b < E; ++b) {
            double lb = logits[idx[b]], lbest = logits[idx[best]];
            if (lb > lbest || (lb == lbest && idx[b] < idx[best])) best = b;
        }
        int t = idx[a]; idx[a] = idx[best]; idx[best] = t;
        ids[a] = idx[a];
    }
    free(idx);
}

/* p_i = exp(l_i - max) / sum_j exp(l_j - max) over the k given logits. */
void orc_softmax(const double *l, int k, double *p)
{
    double m = l[0];
    for (int i = 1; i < k; ++i) if (l[i] > m) m = l[i];
    double s = 0.0;
    for (int i = 0; i < k; ++i) { p[i] = exp(l[i] - m); s += p[i]; }
    for (int i = 0; i < k; ++i) p[i] /= s;
}

/* One expert (or the shared branch): y = W_d (gelu(W_g x) (.) (W_u x)).
 * gate/up are [f][d], down is [d][f]; h (optional, [f]) receives the hidden
 * activation. */
void orc_expert_ffn(const uint8_t *gq, const uint16_t *gs, const uint16_t *gb,
                    const uint8_t *uq, const uint16_t *us, const uint16_t *ub,
                    const uint8_t *dq, const uint16_t *ds, const uint16_t *db,
                    int d, int f, int tanh_form, const double *x, double *y,
                    double *h_out)
{
    double *g = (double *)malloc(sizeof(double) * f);
    double *u = (double *)malloc(sizeof(double) * f);
    orc_qmatvec(gq, gs, gb, f, d, 4, x, g);
    orc_qmatvec(uq, us, ub, f, d, 4, x, u);
    for (int i = 0; i < f; ++i) g[i] = orc_gelu(g[i], tanh_form) * u[i];
    orc_qmatvec(dq, ds, db, d, f, 4, g, y);
    if (h_out) memcpy(h_out, g, sizeof(double) * f);
    free(g);
    free(u);
}

/* Expert from a blob laid out as gate.q|gate.scale|gate.bias|up.*|down.*
 * (the byte order of one routed expert). */
void orc_expert_blob(const uint8_t *blob, int d, int f, int tanh_form,
                     const double *x, double *y, double *h_out)
{
    int64_t qb = (int64_t)f * d / 2, sb = (int64_t)f * (d / 64) * 2;
    int64_t dqb = (int64_t)d * f / 2, dsb = (int64_t)d * (f / 64) * 2;
    const uint8_t *p = blob;
    const uint8_t *gq = p; p += qb;
    const uint16_t *gs = (const uint16_t *)p; p += sb;
    const uint16_t *gb = (const uint16_t *)p; p += sb;
    const uint8_t *uq = p; p += qb;
    const uint16_t *us = (const uint16_t *)p; p += sb;
    const uint16_t *ub = (const uint16_t *)p; p += sb;
    const uint8_t *dq = p; p += dqb;
    const uint16_t *ds = (const uint16_t *)p; p += dsb;
    const uint16_t *db = (const uint16_t *)p;
    orc_expert_ffn(gq, gs, gb, uq, us, ub, dq, ds, db, d, f, tanh_form, x, y, h_out);
}

/*
 * One token through one MoE layer:
 *   l   = W_router x                                    (8-bit, fp64)
 *   ids = top-k(l) or the forced ids                    (rank order)
 *   p   = softmax(l[ids])
 *   y   = shared(x) + sum_k p_k expert_{ids_k}(x)       (rank order, fp64)
 * pool holds E expert blobs at `stride` bytes; forced may be NULL.
 * Returns 0, or -1 if a forced id is out of range or repeated.
 */
int orc_moe_token(const uint8_t *rq, const uint16_t *rs, const uint16_t *rb,
                  const uint8_t *shared_blob, const uint8_t *pool, int64_t stride,
                  int d, int E, int k, int f, int fs, int tanh_form,
                  const uint16_t *x16, const int32_t *forced,
                  double *y, int32_t *ids, double *p, double *logits_out)
{
    double *x = (double *)malloc(sizeof(double) * d);
    double *l = (double *)malloc(sizeof(double) * E);
    double *ye = (double *)malloc(sizeof(double) * d);
    double lsel[64];
    int rc = 0;
    orc_halves_to_double(x16, d, x);
    orc_qmatvec(rq, rs, rb, E, d, 8, x, l);
    if (logits_out) memcpy(logits_out, l, sizeof(double) * E);
    if (forced) {
        for (int a = 0; a < k; ++a) {
            if (forced[a] < 0 || forced[a] >= E) rc = -1;
            for (int b = 0; b < a; ++b) if (forced[a] == forced[b]) rc = -1;
            ids[a] = forced[a];
        }
        if (rc) goto done;
    } else {
        orc_topk(l, E, k, ids);
    }
    for (int a = 0; a < k; ++a) lsel[a] = l[ids[a]];
    orc_softmax(lsel, k, p);
    orc_expert_blob(shared_blob, d, fs, tanh_form, x, y, NULL);
    for (int a = 0; a < k; ++a) {
        orc_expert_blob(pool + (int64_t)ids[a] * stride, d, f, tanh_form, x, ye, NULL);
        for (int i = 0; i < d; ++i) y[i] += p[a] * ye[i];
    }
done:
    free(x);
    free(l);
    free(ye);
    return rc;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of later calls (n >= 1); for timing the oracle on fewer cores. */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
