/*
 * CPU oracle for the output-centric ("warp decode") MoE decode layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code,
 * header, table or helper with the HIP library: it is a plain, slow,
 * obviously correct restatement of what the layer computes, in FP64.
 *
 * What the layer computes (Cursor, "warp decode" blog post):
 *   - "How the two kernels work", first paragraph: for one token and one of
 *     its routed experts, an intermediate neuron takes the dot products of
 *     that neuron's gate row and up row with the token's activation vector;
 *     MXFP8 weights are converted to FP32 as they are read.
 *   - same section, second paragraph: the neuron's value is SiLU(gate) x up,
 *     written once.
 *   - same section, third and fourth paragraphs: one output dimension of one
 *     token walks the token's top-k experts' down-projection rows against the
 *     intermediate and folds each expert's routing weight into one running
 *     sum; the weighted top-k combination is part of that projection.
 *   - "Accuracy improvement": activations stay BF16 and accumulators FP32.
 *
 * The oracle evaluates exactly that definition in FP64 (products and sums of
 * dequantised E4M3 x E8M0 weights with bf16 activations), rounds the stored
 * intermediate h and output y to bf16 once each, round to nearest even,
 * directly from FP64.  The GPU is free to accumulate in FP32 in any order.
 *
 * The "conventional path" emulation at the bottom follows "Accuracy
 * improvement" (BF16 activations converted to MXFP8 and back) and "Eliminating
 * buffers" (a BF16 per-expert output buffer that is combined afterwards); it
 * exists only to check the direction of the accuracy claim.
 *
 * orc_route, at the end, is the top-k router step in front of the layer (the
 * pages give no router details; the reading is stated there).
 *
 * Format facts used (OCP 8-bit floating point and OCP Microscaling v1.0
 * specifications, not on the pages): E4M3 has 1 sign, 4 exponent (bias 7) and
 * 3 mantissa bits, no infinities, NaN = S.1111.111; E8M0 is an unsigned
 * biased exponent, value 2^(v-127), with 0xFF = NaN.
 *
 * Error returns: 0 = ok, -1 = null pointer, -2 = bad shape (or a logit that
 * is not finite), -3 = expert id outside [0, E).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BLOCK 32

/* ------------------------------------------------------------------ */
/* Scalar definitions                                                  */
/* ------------------------------------------------------------------ */

/* E4M3 code -> value (exact in FP64). */
double orc_e4m3(uint8_t q)
{
    int s = q >> 7, e = (q >> 3) & 15, m = q & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);            /* subnormal: m/8 * 2^(1-7) */
    else
        mag = ldexp((double)(8 + m), e - 10);  /* (1 + m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* E8M0 code -> value 2^(v-127) (exact in FP64), 0xFF is NaN. */
double orc_e8m0(uint8_t v)
{
    if (v == 255)
        return NAN;
    return ldexp(1.0, (int)v - 127);
}

/* bf16 bit pattern -> value (exact). */
double orc_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* FP64 -> bf16 bit pattern, round to nearest, ties to even, in one step
 * (no intermediate FP32 rounding).  bf16 has 8 significant bits and FP32's
 * exponent range: normal binades [2^-126, 2^128), subnormal spacing 2^-133.
 * Magnitudes that round to 2^128 or beyond become infinity; NaN -> 0x7FC0. */
uint16_t orc_bf16_rne(double v)
{
    uint16_t sign;
    double a, spacing, r;
    int ex;
    float f;
    uint32_t u;
    if (isnan(v))
        return 0x7FC0;
    sign = signbit(v) ? 0x8000 : 0;
    a = fabs(v);
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    frexp(a, &ex);                 /* a = m * 2^ex, m in [0.5, 1): binade 2^(ex-1) */
    if (ex - 1 < -126)
        spacing = ldexp(1.0, -133);
    else
        spacing = ldexp(1.0, ex - 1 - 7);
    r = nearbyint(a / spacing) * spacing;   /* a / spacing is exact (power of two) */
    if (r >= ldexp(1.0, 128))
        return sign | 0x7F80;
    f = (float)r;                  /* exact: r has <= 8 significant bits in range */
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

double orc_silu(double g)
{
    return g / (1.0 + exp(-g));
}

/* ------------------------------------------------------------------ */
/* One output of each kernel                                           */
/* ------------------------------------------------------------------ */

/* Dequantised weight (row r of expert e, column c) of a [E, R, C] MXFP8 tensor. */
static double weight_at(const uint8_t *q, const uint8_t *s, long R, long C, long e, long r, long c)
{
    long row = e * R + r;
    return orc_e4m3(q[row * C + c]) * orc_e8m0(s[row * (C / ORC_BLOCK) + c / ORC_BLOCK]);
}

/* Gate and up pre-activations G, U of neuron n for token b, slot j. */
static void gate_up_one(const uint16_t *x, const int32_t *ids,
                        const uint8_t *wg, const uint8_t *sg, const uint8_t *wu, const uint8_t *su,
                        long H, long I, long k, long b, long j, long n, double *G, double *U)
{
    long e = ids[b * k + j], c;
    double g = 0.0, u = 0.0;
    for (c = 0; c < H; ++c) {
        double xv = orc_bf16_value(x[b * H + c]);
        g += weight_at(wg, sg, I, H, e, n, c) * xv;
        u += weight_at(wu, su, I, H, e, n, c) * xv;
    }
    *G = g;
    *U = u;
}

/* Weighted sum over the k routed experts for output o of token b (unrounded). */
static double down_one(const uint16_t *h, const int32_t *ids, const float *tw,
                       const uint8_t *wd, const uint8_t *sd,
                       long H, long I, long k, long b, long o)
{
    long j, i;
    double y = 0.0;
    for (j = 0; j < k; ++j) {
        long e = ids[b * k + j];
        double dot = 0.0;
        for (i = 0; i < I; ++i)
            dot += weight_at(wd, sd, H, I, e, o, i) * orc_bf16_value(h[(b * k + j) * I + i]);
        y += (double)tw[b * k + j] * dot;
    }
    return y;
}

static int check_shape(int B, int H, int I, int E, int k)
{
    if (B < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || k > E)
        return -2;
    if (H % ORC_BLOCK || I % ORC_BLOCK)
        return -2;
    return 0;
}

static int check_ids(const int32_t *ids, int B, int E, int k)
{
    long t;
    for (t = 0; t < (long)B * k; ++t)
        if (ids[t] < 0 || ids[t] >= E)
            return -3;
    return 0;
}

int orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Full tensors                                                        */
/* ------------------------------------------------------------------ */

/* h[b,j,n] = bf16(SiLU(G) * U) for every (b, j, n).  Optional FP64 outputs
 * G, U and the unrounded product Hx (each [B,k,I]) may be NULL. */
int orc_gate_up(const uint16_t *x, const int32_t *ids,
                const uint8_t *wg, const uint8_t *sg, const uint8_t *wu, const uint8_t *su,
                uint16_t *h_out, double *G_out, double *U_out, double *Hx_out,
                int B, int H, int I, int E, int k)
{
    long total, t;
    int rc;
    if (!x || !ids || !wg || !sg || !wu || !su || !h_out)
        return -1;
    if ((rc = check_shape(B, H, I, E, k)) || (rc = check_ids(ids, B, E, k)))
        return rc;
    total = (long)B * k * I;
#pragma omp parallel for schedule(dynamic, 64)
    for (t = 0; t < total; ++t) {
        long n = t % I, j = (t / I) % k, b = t / ((long)I * k);
        double G, U, hv;
        gate_up_one(x, ids, wg, sg, wu, su, H, I, k, b, j, n, &G, &U);
        hv = orc_silu(G) * U;
        h_out[t] = orc_bf16_rne(hv);
        if (G_out) G_out[t] = G;
        if (U_out) U_out[t] = U;
        if (Hx_out) Hx_out[t] = hv;
    }
    return 0;
}

/* y[b,o] = bf16(sum_j w[b,j] * (Wd[ids[b,j], o, :] . h[b,j,:])).  Optional
 * unrounded FP64 output Y_out [B,H] may be NULL. */
int orc_down(const uint16_t *h, const int32_t *ids, const float *tw,
             const uint8_t *wd, const uint8_t *sd,
             uint16_t *y_out, double *Y_out,
             int B, int H, int I, int E, int k)
{
    long total, t;
    int rc;
    if (!h || !ids || !tw || !wd || !sd || !y_out)
        return -1;
    if ((rc = check_shape(B, H, I, E, k)) || (rc = check_ids(ids, B, E, k)))
        return rc;
    total = (long)B * H;
#pragma omp parallel for schedule(dynamic, 64)
    for (t = 0; t < total; ++t) {
        long o = t % H, b = t / H;
        double Y = down_one(h, ids, tw, wd, sd, H, I, k, b, o);
        y_out[t] = orc_bf16_rne(Y);
        if (Y_out) Y_out[t] = Y;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Conventional expert-centric path, numerically emulated               */
/* ------------------------------------------------------------------ */

/* MX quantise-dequantise of n values (n % 32 == 0) in place, blocks of 32:
 * shared exponent floor(log2(block max |v|)) - 8, element = nearest E4M3
 * value (ties to even) of v / 2^shared, saturated to +-448. */
static double e4m3_round(double a)  /* a >= 0, already saturated to <= 448 */
{
    int ex;
    double spacing;
    if (a == 0.0)
        return 0.0;
    frexp(a, &ex);
    if (ex - 1 < -6)
        spacing = ldexp(1.0, -9);
    else
        spacing = ldexp(1.0, ex - 1 - 3);
    return nearbyint(a / spacing) * spacing;
}

void orc_mx_fake_quant(double *v, long n)
{
    long blk, i;
    for (blk = 0; blk < n / ORC_BLOCK; ++blk) {
        double *p = v + blk * ORC_BLOCK, amax = 0.0, X;
        int ex;
        for (i = 0; i < ORC_BLOCK; ++i)
            if (fabs(p[i]) > amax)
                amax = fabs(p[i]);
        if (amax == 0.0)
            continue;
        frexp(amax, &ex);
        X = ldexp(1.0, ex - 1 - 8);
        for (i = 0; i < ORC_BLOCK; ++i) {
            double a = fabs(p[i]) / X;
            if (a > 448.0)
                a = 448.0;
            a = e4m3_round(a) * X;
            p[i] = signbit(p[i]) ? -a : a;
        }
    }
}

/* y_conv[b,o] for the conventional path: x quantised to MXFP8 (blocks along H);
 * h = bf16(SiLU(G) * U) then quantised to MXFP8 (blocks along I); per-expert
 * outputs rounded to bf16 (the per-expert buffer); weighted combine rounded to
 * bf16.  Y_out (unrounded combine, FP64) may be NULL. */
int orc_conventional(const uint16_t *x, const int32_t *ids, const float *tw,
                     const uint8_t *wg, const uint8_t *sg, const uint8_t *wu, const uint8_t *su,
                     const uint8_t *wd, const uint8_t *sd,
                     uint16_t *y_out, double *Y_out,
                     int B, int H, int I, int E, int k)
{
    long b;
    int rc;
    if (!x || !ids || !tw || !wg || !sg || !wu || !su || !wd || !sd || !y_out)
        return -1;
    if ((rc = check_shape(B, H, I, E, k)) || (rc = check_ids(ids, B, E, k)))
        return rc;
#pragma omp parallel for schedule(dynamic, 1)
    for (b = 0; b < B; ++b) {
        double *xq = malloc(sizeof(double) * H);
        double *hq = malloc(sizeof(double) * I);
        double *acc = calloc(H, sizeof(double));
        long c, j, n, o, i;
        for (c = 0; c < H; ++c)
            xq[c] = orc_bf16_value(x[b * H + c]);
        orc_mx_fake_quant(xq, H);
        for (j = 0; j < k; ++j) {
            long e = ids[b * k + j];
            for (n = 0; n < I; ++n) {
                double g = 0.0, u = 0.0;
                for (c = 0; c < H; ++c) {
                    g += weight_at(wg, sg, I, H, e, n, c) * xq[c];
                    u += weight_at(wu, su, I, H, e, n, c) * xq[c];
                }
                hq[n] = orc_bf16_value(orc_bf16_rne(orc_silu(g) * u));
            }
            orc_mx_fake_quant(hq, I);
            for (o = 0; o < H; ++o) {
                double d = 0.0;
                for (i = 0; i < I; ++i)
                    d += weight_at(wd, sd, H, I, e, o, i) * hq[i];
                acc[o] += (double)tw[b * k + j] * orc_bf16_value(orc_bf16_rne(d));
            }
        }
        for (o = 0; o < H; ++o) {
            y_out[b * H + o] = orc_bf16_rne(acc[o]);
            if (Y_out) Y_out[b * H + o] = acc[o];
        }
        free(xq);
        free(hq);
        free(acc);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Router step in front of the layer                                   */
/* ------------------------------------------------------------------ */

/* The pages route each token to a few of many experts ("The traditional MoE
 * path": 8 of 128 in one layer) and give no router details.  The reading
 * used here, the plainest top-k router: from one FP32 logit per expert,
 * token b keeps the k largest logits, largest first, the lower expert id
 * first among equal logits; its routing weights are the softmax of all E
 * logits restricted to the k kept experts and renormalised to sum to one
 * (FP64 throughout).  Logits must be finite (-2 otherwise); B = 0 is a valid
 * empty batch. */
int orc_route(const float *logits, int32_t *ids_out, double *w_out, int B, int E, int k)
{
    long b, i;
    int j;
    if (!logits || !ids_out || !w_out)
        return -1;
    if (B < 0 || E <= 0 || k <= 0 || k > E)
        return -2;
    for (i = 0; i < (long)B * E; ++i)
        if (!isfinite(logits[i]))
            return -2;
    for (b = 0; b < B; ++b) {
        const float *l = logits + b * E;
        char *taken = calloc((size_t)E, 1);
        double m = -INFINITY, z = 0.0, s = 0.0;
        if (!taken)
            return -1;
        /* selection: k times, the best expert not yet taken */
        for (j = 0; j < k; ++j) {
            long best = -1;
            for (i = 0; i < E; ++i)
                if (!taken[i] && (best < 0 || (double)l[i] > (double)l[best]))
                    best = i;   /* strict >: an equal logit later in the list loses */
            taken[best] = 1;
            ids_out[b * k + j] = (int32_t)best;
        }
        /* softmax over all E experts, then renormalised over the kept k */
        for (i = 0; i < E; ++i)
            if ((double)l[i] > m)
                m = l[i];
        for (i = 0; i < E; ++i)
            z += exp((double)l[i] - m);
        for (j = 0; j < k; ++j)
            s += exp((double)l[ids_out[b * k + j]] - m) / z;
        for (j = 0; j < k; ++j)
            w_out[b * k + j] = exp((double)l[ids_out[b * k + j]] - m) / z / s;
        free(taken);
    }
    return 0;
}
