/*
 * ftmoe_oracle.c -- plain, slow CPU oracle for the NVFP4-weight mixture-of-experts
 * layer (router, top-k, renormalised weights, clamped-SwiGLU experts, down
 * projection, weighted combine and gated shared expert).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no source, header,
 * table or helper with the HIP library; the two meet only in the seeded input
 * arrays that the tests hand to both.
 *
 * The "omp parallel for" pragmas only spread independent rows (each with its
 * own serial sum) over threads in a second build used to time the oracle on
 * every host core; the checker is the plain build, where they are ignored, and
 * the two give identical bits.
 *
 * Every function computes the plain definition, one element at a time, in
 * IEEE binary64 (products of the fp32/bf16/e2m1/e4m3 operands are exact in
 * binary64), and rounds once at the end where a narrower type is stored.
 *
 * Sources of the definitions:
 *  - FreeToken fork PR #84 (page 1), bullet on #631: the NVFP4 MoE decode GEMV on
 *    the per-token path of each MoE layer; bullet on #578: NVFP4 prefill experts
 *    dequantised by bit placement.
 *  - FreeToken commit log (page 2): the 288-expert NVFP4 MoE entry; the
 *    clamped-SwiGLU entry; the 512-routed-expert top-10 entry with a gated shared
 *    expert; the router / shared-gate kernel entry; the top-k entry (k not a
 *    power of two).
 *  - NVFP4 codec: e2m1 element codes (OCP Microscaling Formats v1.0, FP4 E2M1),
 *    one e4m3 scale per 16 consecutive K elements (OCP 8-bit Floating Point,
 *    E4M3: bias 7, no infinities, S.1111.111 is NaN), one fp32 global scale per
 *    tensor.  The dequantised weight is fp32(fp32(e2m1 x e4m3) x global).
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *  - the low nibble of a code byte holds the even K index;
 *  - w13 stacks gate rows [0, I) over up rows [I, 2I); per-expert global scales
 *    are stored as [gate, up, down];
 *  - router logits are accumulated in binary64 in index order, plus the optional
 *    bias, and rounded once to fp32; top-k orders by (logit desc, index asc), a
 *    NaN logit ranks below every number;
 *  - routing weights are the softmax over the selected logits (equal, in exact
 *    arithmetic, to a softmax over all experts renormalised over the top-k),
 *    evaluated in binary64 and stored as fp32; the layer combines with the
 *    stored fp32 weights;
 *  - clamped SwiGLU is silu(min(g, gate_max)) * clamp(u, -up_absmax, up_absmax)
 *    with silu(z) = z / (1 + exp(-z)); plain SwiGLU is silu(g) * u; comparisons
 *    are written so that a NaN propagates;
 *  - the expert intermediate h is kept unrounded (binary64 here);
 *  - the shared expert's gate is sigmoid(sum_h gs[h] * x[h]);
 *  - the output is bf16, rounded to nearest-even once from the binary64 sum
 *    sum_i w_i * o_i + gamma * o_shared (routed slots in rank order, then the
 *    shared expert).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the row loops use: 1 in the plain build. */
int32_t or_threads(void)
{
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- codecs -- */

/* e2m1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * Normal (e > 0): 2^(e-1) * (1 + m/2).  Subnormal (e == 0): m * 0.5. */
double or_e2m1(uint32_t code)
{
    uint32_t s = (code >> 3) & 1u;
    uint32_t e = (code >> 1) & 3u;
    uint32_t m = code & 1u;
    double mag;
    if (e == 0)
        mag = 0.5 * (double)m;
    else
        mag = ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* e4m3 (OCP FP8 E4M3): sign bit 7, exponent bits 6..3 (bias 7), mantissa 2..0.
 * S.1111.111 is NaN; there are no infinities.  Subnormal: m/8 * 2^-6. */
double or_e4m3(uint32_t byte)
{
    uint32_t s = (byte >> 7) & 1u;
    uint32_t e = (byte >> 3) & 15u;
    uint32_t m = byte & 7u;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* One dequantised NVFP4 weight: fp32(fp32(e2m1 * e4m3) * g).
 * The inner product has at most 2 + 4 significant bits and an exponent inside
 * fp32's normal range, so its conversion to fp32 is exact; the product with the
 * fp32 global scale is exact in binary64 and rounds once (to nearest-even) when
 * converted to fp32, which is the correctly rounded fp32 multiplication. */
float or_dequant_value(uint32_t code, uint32_t scale_byte, float g)
{
    float p = (float)(or_e2m1(code) * or_e4m3(scale_byte));
    return (float)((double)p * (double)g);
}

/* Code of element k of a row: byte k/2 of the row, low nibble for even k. */
static uint32_t row_code(const uint8_t *row_codes, int64_t k)
{
    uint8_t b = row_codes[k / 2];
    return (k % 2 == 0) ? (uint32_t)(b & 0x0F) : (uint32_t)(b >> 4);
}

/* Dequantise a [rows, K] NVFP4 matrix stored as codes [rows, K/2] and scales
 * [rows, K/16] (row-major) with global scale g, into fp32 out[rows, K]. */
void or_dequant_matrix(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                       float g, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint8_t *rc = codes + r * (K / 2);
        const uint8_t *rs = scales + r * (K / 16);
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = or_dequant_value(row_code(rc, k), rs[k / 16], g);
    }
}

/* bf16 -> binary64 (exact). */
double or_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* binary64 -> bf16, round to nearest, ties to even, in one step (no detour
 * through fp32, which could round twice).  bf16 has 8 significant bits, normal
 * exponents down to -126 and subnormals spaced 2^-133. */
uint16_t or_bf16_from_double(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    int ex;
    frexp(a, &ex);           /* a in [2^(ex-1), 2^ex) */
    int q = ex - 1 - 7;      /* exponent of one unit in the last place */
    if (q < -133)
        q = -133;
    double r = ldexp(nearbyint(ldexp(a, -q)), q); /* default rounding: nearest-even */
    const double bf16_max = ldexp(255.0, 120);     /* 0x7F7F = (2 - 2^-7) * 2^127 */
    if (r > bf16_max)
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;      /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFFu));
}

/* ---------------------------------------------------------------- router -- */

/* logits[t, e] = fp32( sum_h W[e, h] * x[t, h]  (+ bias[e]) ), binary64 sum in
 * index order.  x is bf16 [T, H]; W fp32 [E, H]; bias fp32 [E] or NULL. */
void or_router_logits(int64_t T, int32_t E, int32_t H, const uint16_t *x, const float *W,
                      const float *bias, float *logits)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int32_t h = 0; h < H; ++h)
                acc += (double)W[(int64_t)e * H + h] * or_bf16_to_double(x[t * H + h]);
            if (bias)
                acc += (double)bias[e];
            logits[t * E + e] = (float)acc;
        }
    }
}

/* Rank key: a NaN logit ranks below every number (it is kept, not skipped). */
static int ranks_above(float a, int32_t ia, float b, int32_t ib)
{
    int an = isnan(a), bn = isnan(b);
    if (an || bn) {
        if (an && bn)
            return ia < ib;
        return bn; /* the number ranks above the NaN */
    }
    if (a != b)
        return a > b;
    return ia < ib;
}

/* Top-k by (logit descending, index ascending), emitted in that order, and the
 * softmax of the selected logits in binary64, stored as fp32. */
void or_topk(int64_t T, int32_t E, int32_t k, const float *logits, int32_t *ids, float *w)
{
    char *taken = (char *)malloc((size_t)E);
    double *d = (double *)malloc(sizeof(double) * (size_t)k);
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int32_t i = 0; i < k; ++i) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || ranks_above(l[e], e, l[best], best))
                    best = e;
            }
            taken[best] = 1;
            ids[t * k + i] = best;
        }
        double top = (double)l[ids[t * k]];
        double sum = 0.0;
        for (int32_t i = 0; i < k; ++i) {
            d[i] = exp((double)l[ids[t * k + i]] - top);
            sum += d[i];
        }
        for (int32_t i = 0; i < k; ++i)
            w[t * k + i] = (float)(d[i] / sum);
    }
    free(taken);
    free(d);
}

/* ------------------------------------------------------------ activations -- */

double or_silu(double z) { return z / (1.0 + exp(-z)); }

/* act 0: silu(g) * u.  act 1: silu(min(g, gate_max)) * clamp(u, -up_absmax, up_absmax). */
double or_swiglu(int32_t act, double g, double u, double gate_max, double up_absmax)
{
    if (act == 1) {
        if (g > gate_max)
            g = gate_max;
        if (u > up_absmax)
            u = up_absmax;
        if (u < -up_absmax)
            u = -up_absmax;
    }
    return or_silu(g) * u;
}

/* ---------------------------------------------------------------- experts -- */

/* One expert's MLP on one token, from its dequantised fp32 matrices:
 *   gate_r = sum_h Wg[r, h] x_h,  up_r = sum_h Wu[r, h] x_h,
 *   h_r = swiglu(gate_r, up_r),   o_c = sum_r Wd[c, r] h_r.
 * wg, wu: [I, H]; wd: [H, I] (fp32, already dequantised); x: binary64 [H]. */
static void expert_forward(int32_t H, int32_t I, const float *wg, const float *wu, const float *wd,
                           int32_t act, double gate_max, double up_absmax, const double *x,
                           double *hbuf, double *o)
{
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < I; ++r) {
        double g = 0.0, u = 0.0;
        for (int32_t h = 0; h < H; ++h) {
            g += (double)wg[(int64_t)r * H + h] * x[h];
            u += (double)wu[(int64_t)r * H + h] * x[h];
        }
        hbuf[r] = or_swiglu(act, g, u, gate_max, up_absmax);
    }
#pragma omp parallel for schedule(static)
    for (int32_t c = 0; c < H; ++c) {
        double acc = 0.0;
        for (int32_t r = 0; r < I; ++r)
            acc += (double)wd[(int64_t)c * I + r] * hbuf[r];
        o[c] = acc;
    }
}

/* Dequantise expert e of a canonical NVFP4 expert bank into wg, wu [I, H] and
 * wd [H, I].  Bank layout: w13 codes [n][2I][H/2], w13 scales [n][2I][H/16],
 * w2 codes [n][H][I/2], w2 scales [n][H][I/16], global scales [n][3]. */
static void dequant_expert(int32_t H, int32_t I, int64_t e, const uint8_t *w13c,
                           const uint8_t *w13s, const uint8_t *w2c, const uint8_t *w2s,
                           const float *gsc, float *wg, float *wu, float *wd)
{
    int64_t rows13 = 2 * (int64_t)I;
    const uint8_t *c13 = w13c + e * rows13 * (H / 2);
    const uint8_t *s13 = w13s + e * rows13 * (H / 16);
    or_dequant_matrix(c13, s13, I, H, gsc[e * 3 + 0], wg);
    or_dequant_matrix(c13 + (int64_t)I * (H / 2), s13 + (int64_t)I * (H / 16), I, H,
                      gsc[e * 3 + 1], wu);
    or_dequant_matrix(w2c + e * (int64_t)H * (I / 2), w2s + e * (int64_t)H * (I / 16), H, I,
                      gsc[e * 3 + 2], wd);
}

/* One expert's output o[H] for one token x (bf16 [H]).  Exported for tests. */
void or_expert_output(int32_t H, int32_t I, int64_t e, const uint8_t *w13c, const uint8_t *w13s,
                      const uint8_t *w2c, const uint8_t *w2s, const float *gsc, int32_t act,
                      float gate_max, float up_absmax, const uint16_t *x, double *o)
{
    float *wg = (float *)malloc(sizeof(float) * (size_t)I * H);
    float *wu = (float *)malloc(sizeof(float) * (size_t)I * H);
    float *wd = (float *)malloc(sizeof(float) * (size_t)I * H);
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *hb = (double *)malloc(sizeof(double) * (size_t)I);
    for (int32_t h = 0; h < H; ++h)
        xd[h] = or_bf16_to_double(x[h]);
    dequant_expert(H, I, e, w13c, w13s, w2c, w2s, gsc, wg, wu, wd);
    expert_forward(H, I, wg, wu, wd, act, gate_max, up_absmax, xd, hb, o);
    free(wg); free(wu); free(wd); free(xd); free(hb);
}

/* ------------------------------------------------------------------ layer -- */

/* The whole MoE layer for T tokens.
 *   Routed bank: E experts of intermediate size I (canonical layout above).
 *   Shared expert (optional, Is > 0): one expert of intermediate size Is in the
 *   same layout, gated by sigmoid(sum_h sgate[h] x[h]).
 *   Routing: if ids_in/w_in are given they are used as the routes; otherwise the
 *   router logits, top-k and weights are computed here (and written to
 *   ids_out / w_out when those are non-NULL).
 * Outputs: y bf16 [T, H]; y64 (optional) the binary64 value before rounding. */
int32_t or_moe_layer(int32_t E, int32_t H, int32_t I, int32_t k, int32_t act, float gate_max,
                     float up_absmax, int64_t T, const uint16_t *x, const float *Wr,
                     const float *bias, const uint8_t *w13c, const uint8_t *w13s,
                     const uint8_t *w2c, const uint8_t *w2s, const float *gsc, int32_t Is,
                     const uint8_t *s13c, const uint8_t *s13s, const uint8_t *s2c,
                     const uint8_t *s2s, const float *sgsc, const uint16_t *sgate,
                     const int32_t *ids_in, const float *w_in, int32_t *ids_out, float *w_out,
                     double *y64, uint16_t *y)
{
    if (E <= 0 || H <= 0 || I <= 0 || k <= 0 || k > E || T < 0 || H % 16 || I % 16 ||
        (Is > 0 && Is % 16))
        return -1;
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1) * k);
    float *wts = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1) * k);
    if (ids_in && w_in) {
        memcpy(ids, ids_in, sizeof(int32_t) * (size_t)T * k);
        memcpy(wts, w_in, sizeof(float) * (size_t)T * k);
    } else {
        float *logits = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1) * E);
        or_router_logits(T, E, H, x, Wr, bias, logits);
        or_topk(T, E, k, logits, ids, wts);
        free(logits);
    }
    if (ids_out)
        memcpy(ids_out, ids, sizeof(int32_t) * (size_t)T * k);
    if (w_out)
        memcpy(w_out, wts, sizeof(float) * (size_t)T * k);

    int32_t Imax = (Is > I) ? Is : I;
    float *wg = (float *)malloc(sizeof(float) * (size_t)Imax * H);
    float *wu = (float *)malloc(sizeof(float) * (size_t)Imax * H);
    float *wd = (float *)malloc(sizeof(float) * (size_t)Imax * H);
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *hb = (double *)malloc(sizeof(double) * (size_t)Imax);
    double *o = (double *)malloc(sizeof(double) * (size_t)H);
    double *acc = (double *)malloc(sizeof(double) * (size_t)H);

    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h) {
            xd[h] = or_bf16_to_double(x[t * H + h]);
            acc[h] = 0.0;
        }
        for (int32_t i = 0; i < k; ++i) {
            int64_t e = ids[t * k + i];
            dequant_expert(H, I, e, w13c, w13s, w2c, w2s, gsc, wg, wu, wd);
            expert_forward(H, I, wg, wu, wd, act, gate_max, up_absmax, xd, hb, o);
            double wi = (double)wts[t * k + i];
            for (int32_t h = 0; h < H; ++h)
                acc[h] += wi * o[h];
        }
        if (Is > 0) {
            double z = 0.0;
            for (int32_t h = 0; h < H; ++h)
                z += or_bf16_to_double(sgate[h]) * xd[h];
            double gamma = 1.0 / (1.0 + exp(-z));
            dequant_expert(H, Is, 0, s13c, s13s, s2c, s2s, sgsc, wg, wu, wd);
            expert_forward(H, Is, wg, wu, wd, act, gate_max, up_absmax, xd, hb, o);
            for (int32_t h = 0; h < H; ++h)
                acc[h] += gamma * o[h];
        }
        for (int32_t h = 0; h < H; ++h) {
            if (y64)
                y64[t * H + h] = acc[h];
            if (y)
                y[t * H + h] = or_bf16_from_double(acc[h]);
        }
    }
    free(ids); free(wts); free(wg); free(wu); free(wd);
    free(xd); free(hb); free(o); free(acc);
    return 0;
}

/* ------------------------------------------------- expert-slot indirection -- */

/* The layer with its routed experts held in a bank of expert SLOTS (FreeToken fork
 * PR #84, page 1, the interleaved A/B table: the production configuration keeps
 * 2100 expert slots and reports expert-cache misses per token; FreeToken commit
 * log, page 2: the expert banks plan their residency).
 *   slot_of[e] is the slot of the bank holding expert e's weights, or any value
 *   outside [0, n_slots) when expert e is not resident.  Routing is unchanged
 *   (it reads only the router).  Reading taken here: a selected expert that is not
 *   resident contributes nothing to y, its routing weight is kept (the others are
 *   not renormalised), and its id is reported in miss[t * k + i] (-1 when the
 *   expert of that place is resident), so that the caller can page it in and
 *   recompute.  The bank (w13c .. gsc) is a canonical bank of n_slots experts. */
int32_t or_moe_layer_slots(int32_t E, int32_t H, int32_t I, int32_t k, int32_t act,
                           float gate_max, float up_absmax, int64_t T, const uint16_t *x,
                           const float *Wr, const float *bias, int32_t n_slots,
                           const int32_t *slot_of, const uint8_t *w13c, const uint8_t *w13s,
                           const uint8_t *w2c, const uint8_t *w2s, const float *gsc, int32_t Is,
                           const uint8_t *s13c, const uint8_t *s13s, const uint8_t *s2c,
                           const uint8_t *s2s, const float *sgsc, const uint16_t *sgate,
                           int32_t *ids_out, float *w_out, int32_t *miss, double *y64,
                           uint16_t *y)
{
    if (E <= 0 || H <= 0 || I <= 0 || k <= 0 || k > E || T < 0 || H % 16 || I % 16 ||
        n_slots <= 0 || !slot_of || (Is > 0 && Is % 16))
        return -1;
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1) * k);
    float *wts = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1) * k);
    float *logits = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1) * E);
    or_router_logits(T, E, H, x, Wr, bias, logits);
    or_topk(T, E, k, logits, ids, wts);
    free(logits);
    if (ids_out)
        memcpy(ids_out, ids, sizeof(int32_t) * (size_t)T * k);
    if (w_out)
        memcpy(w_out, wts, sizeof(float) * (size_t)T * k);

    int32_t Imax = (Is > I) ? Is : I;
    float *wg = (float *)malloc(sizeof(float) * (size_t)Imax * H);
    float *wu = (float *)malloc(sizeof(float) * (size_t)Imax * H);
    float *wd = (float *)malloc(sizeof(float) * (size_t)Imax * H);
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *hb = (double *)malloc(sizeof(double) * (size_t)Imax);
    double *o = (double *)malloc(sizeof(double) * (size_t)H);
    double *acc = (double *)malloc(sizeof(double) * (size_t)H);

    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h) {
            xd[h] = or_bf16_to_double(x[t * H + h]);
            acc[h] = 0.0;
        }
        for (int32_t i = 0; i < k; ++i) {
            int32_t e = ids[t * k + i];
            int32_t s = slot_of[e];
            int resident = (s >= 0 && s < n_slots);
            if (miss)
                miss[t * k + i] = resident ? -1 : e;
            if (!resident)
                continue;
            dequant_expert(H, I, s, w13c, w13s, w2c, w2s, gsc, wg, wu, wd);
            expert_forward(H, I, wg, wu, wd, act, gate_max, up_absmax, xd, hb, o);
            double wi = (double)wts[t * k + i];
            for (int32_t h = 0; h < H; ++h)
                acc[h] += wi * o[h];
        }
        if (Is > 0) {
            double z = 0.0;
            for (int32_t h = 0; h < H; ++h)
                z += or_bf16_to_double(sgate[h]) * xd[h];
            double gamma = 1.0 / (1.0 + exp(-z));
            dequant_expert(H, Is, 0, s13c, s13s, s2c, s2s, sgsc, wg, wu, wd);
            expert_forward(H, Is, wg, wu, wd, act, gate_max, up_absmax, xd, hb, o);
            for (int32_t h = 0; h < H; ++h)
                acc[h] += gamma * o[h];
        }
        for (int32_t h = 0; h < H; ++h) {
            if (y64)
                y64[t * H + h] = acc[h];
            if (y)
                y[t * H + h] = or_bf16_from_double(acc[h]);
        }
    }
    free(ids); free(wts); free(wg); free(wu); free(wd);
    free(xd); free(hb); free(o); free(acc);
    return 0;
}

/* ----------------------------------------------------------- block-fp8 codec -- */

/* The second routed-expert codec of the 512-expert layer (FreeToken commit log,
 * page 2: the entry with 512 NVFP4 / block-fp8 routed experts, and its fp8 scale-bank
 * padding rule).  The pages do not give the block shape; reading taken here: each
 * weight is one OCP e4m3 byte, and each 128 x 128 block of a [rows, K] matrix
 * (rows r..r+127, columns c..c+127) shares one fp32 scale; a matrix dimension that is
 * not a multiple of 128 ends in a partial block that still has its own scale, so the
 * scale bank is [ceil(rows/128)][ceil(K/128)].  There is no separate global scale.
 * The dequantised weight is fp32(e4m3 * scale): one rounding of the exact product
 * (4 significant bits times 24 fit in binary64). */
#define OR_FP8_BLOCK 128

float or_fp8_dequant_value(uint32_t byte, float scale)
{
    return (float)(or_e4m3(byte) * (double)scale);
}

/* codes u8 [rows, K], scales f32 [ceil(rows/128), ceil(K/128)] -> fp32 out [rows, K]. */
void or_fp8_dequant_matrix(const uint8_t *codes, const float *scales, int64_t rows, int64_t K,
                           float *out)
{
    int64_t kb = (K + OR_FP8_BLOCK - 1) / OR_FP8_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < K; ++c)
            out[r * K + c] = or_fp8_dequant_value(codes[r * K + c],
                                                  scales[(r / OR_FP8_BLOCK) * kb + c / OR_FP8_BLOCK]);
}

/* Expert e of a canonical block-fp8 bank: w13 codes [n][2I][H] (gate rows 0..I-1,
 * then up), w13 scales [n][ceil(2I/128)][ceil(H/128)], w2 codes [n][H][I], w2 scales
 * [n][ceil(H/128)][ceil(I/128)].  With I % 128 == 0 no scale block straddles gate and
 * up. */
static void dequant_expert_fp8(int32_t H, int32_t I, int64_t e, const uint8_t *w13c,
                               const float *w13s, const uint8_t *w2c, const float *w2s,
                               float *wg, float *wu, float *wd)
{
    int64_t rb13 = (2 * (int64_t)I + OR_FP8_BLOCK - 1) / OR_FP8_BLOCK;
    int64_t kb13 = ((int64_t)H + OR_FP8_BLOCK - 1) / OR_FP8_BLOCK;
    int64_t rb2 = ((int64_t)H + OR_FP8_BLOCK - 1) / OR_FP8_BLOCK;
    int64_t kb2 = ((int64_t)I + OR_FP8_BLOCK - 1) / OR_FP8_BLOCK;
    const uint8_t *c13 = w13c + e * 2 * (int64_t)I * H;
    const float *s13 = w13s + e * rb13 * kb13;
    or_fp8_dequant_matrix(c13, s13, I, H, wg);
    or_fp8_dequant_matrix(c13 + (int64_t)I * H, s13 + ((int64_t)I / OR_FP8_BLOCK) * kb13, I, H,
                          wu);
    or_fp8_dequant_matrix(w2c + e * (int64_t)H * I, w2s + e * rb2 * kb2, H, I, wd);
}

/* The whole layer with block-fp8 routed experts and (when Is > 0) a block-fp8 shared
 * expert; everything else as or_moe_layer (routes computed here).  Needs
 * I % 128 == 0 and Is % 128 == 0. */
int32_t or_moe_layer_fp8(int32_t E, int32_t H, int32_t I, int32_t k, int32_t act,
                         float gate_max, float up_absmax, int64_t T, const uint16_t *x,
                         const float *Wr, const float *bias, const uint8_t *w13c,
                         const float *w13s, const uint8_t *w2c, const float *w2s, int32_t Is,
                         const uint8_t *s13c, const float *s13s, const uint8_t *s2c,
                         const float *s2s, const uint16_t *sgate, int32_t *ids_out,
                         float *w_out, double *y64, uint16_t *y)
{
    if (E <= 0 || H <= 0 || I <= 0 || k <= 0 || k > E || T < 0 || I % OR_FP8_BLOCK ||
        (Is > 0 && Is % OR_FP8_BLOCK))
        return -1;
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1) * k);
    float *wts = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1) * k);
    float *logits = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1) * E);
    or_router_logits(T, E, H, x, Wr, bias, logits);
    or_topk(T, E, k, logits, ids, wts);
    free(logits);
    if (ids_out)
        memcpy(ids_out, ids, sizeof(int32_t) * (size_t)T * k);
    if (w_out)
        memcpy(w_out, wts, sizeof(float) * (size_t)T * k);

    int32_t Imax = (Is > I) ? Is : I;
    float *wg = (float *)malloc(sizeof(float) * (size_t)Imax * H);
    float *wu = (float *)malloc(sizeof(float) * (size_t)Imax * H);
    float *wd = (float *)malloc(sizeof(float) * (size_t)Imax * H);
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *hb = (double *)malloc(sizeof(double) * (size_t)Imax);
    double *o = (double *)malloc(sizeof(double) * (size_t)H);
    double *acc = (double *)malloc(sizeof(double) * (size_t)H);
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h) {
            xd[h] = or_bf16_to_double(x[t * H + h]);
            acc[h] = 0.0;
        }
        for (int32_t i = 0; i < k; ++i) {
            dequant_expert_fp8(H, I, ids[t * k + i], w13c, w13s, w2c, w2s, wg, wu, wd);
            expert_forward(H, I, wg, wu, wd, act, gate_max, up_absmax, xd, hb, o);
            double wi = (double)wts[t * k + i];
            for (int32_t h = 0; h < H; ++h)
                acc[h] += wi * o[h];
        }
        if (Is > 0) {
            double z = 0.0;
            for (int32_t h = 0; h < H; ++h)
                z += or_bf16_to_double(sgate[h]) * xd[h];
            double gamma = 1.0 / (1.0 + exp(-z));
            dequant_expert_fp8(H, Is, 0, s13c, s13s, s2c, s2s, wg, wu, wd);
            expert_forward(H, Is, wg, wu, wd, act, gate_max, up_absmax, xd, hb, o);
            for (int32_t h = 0; h < H; ++h)
                acc[h] += gamma * o[h];
        }
        for (int32_t h = 0; h < H; ++h) {
            if (y64)
                y64[t * H + h] = acc[h];
            if (y)
                y[t * H + h] = or_bf16_from_double(acc[h]);
        }
    }
    free(ids); free(wts); free(wg); free(wu); free(wd);
    free(xd); free(hb); free(o); free(acc);
    return 0;
}

/* ------------------------------------------------ fp8 per-tensor W8A8 linear -- */

/* FreeToken commit log (page 2), the paragraph on row-wise FP8 scaled matrix products:
 * the fused per-tensor-FP8 projections (q/k/v parts stacked along the output rows)
 * run as W8A8 products, either one row-wise-scaled GEMM or, as a fallback, one
 * tensor-wise GEMM per part over its row slice, the parts found from the run-lengths
 * of the per-row weight scales.  Readings taken here: activations are quantised per
 * tensor with scale s_x = amax|x| / 448 (fp32 division) and codes
 * e4m3(x / s_x) (the quotient in fp32, then round to the nearest e4m3 value, ties to
 * the even code, magnitudes above 448 saturating to 448; s_x = 1 for an all-zero x);
 * y[m, n] = bf16( s_x * s_w[n] * sum_k e4m3(xq[m, k]) * e4m3(w[n, k]) ), where s_w[n]
 * is the scale of the part holding row n.  The e4m3 x e4m3 products have at most 8
 * significant bits, so the sum is exact in binary64 for K < 2^17. */

/* fp32 value -> e4m3 byte: the nearest of the 254 finite e4m3 values by exhaustive
 * search (ties to the code with an even mantissa), saturating at +-448; NaN -> 0x7F. */
uint32_t or_e4m3_encode(float v)
{
    if (isnan(v))
        return 0x7F;
    double a = fabs((double)v);
    uint32_t sign = signbit(v) ? 0x80u : 0u;
    uint32_t best = 0;
    double best_d = INFINITY;
    for (uint32_t b = 0; b < 0x7F; ++b) { /* magnitudes 0 .. 448 */
        double d = fabs(or_e4m3(b) - a);
        if (d < best_d || (d == best_d && (b & 1u) == 0u)) {
            best_d = d;
            best = b;
        }
    }
    return sign | best;
}

/* Per-tensor activation quantisation: s_x and the codes of x (bf16 [M, K]). */
void or_fp8_quantize(int64_t M, int64_t K, const uint16_t *x, uint8_t *codes, float *scale)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < M * K; ++i) {
        float a = (float)fabs(or_bf16_to_double(x[i]));
        if (a > amax)
            amax = a;
    }
    float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    *scale = s;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M * K; ++i) {
        float q = (float)or_bf16_to_double(x[i]) / s;
        codes[i] = (uint8_t)or_e4m3_encode(q);
    }
}

/* y = bf16( s_x * s_w[n] * sum_k e4m3(xq[m,k]) e4m3(w[n,k]) ), binary64 throughout;
 * xq [M, K], w [N, K] e4m3 bytes, w_scale fp32 [N]; y64 (optional) the unrounded value. */
void or_fp8_linear(int64_t M, int64_t N, int64_t K, const uint8_t *xq, float s_x,
                   const uint8_t *w, const float *w_scale, double *y64, uint16_t *y)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += or_e4m3(xq[m * K + k]) * or_e4m3(w[n * K + k]);
            double v = acc * (double)s_x * (double)w_scale[n];
            if (y64)
                y64[m * N + n] = v;
            if (y)
                y[m * N + n] = or_bf16_from_double(v);
        }
    }
}

/* ------------------------------------------------ extend attention, KV cache -- */

/* FreeToken fork PR #84 (page 1), the bullet on the extend-attention kernel of the
 * NVFP4 KV-cache step: new (extend) query tokens attend to a cached prefix held as a
 * 16-bit, fp8 or NVFP4 cache, and to the new tokens themselves; the quantised-cache
 * tile applies the fp8 scales to the dot outputs, and the check is against a
 * dequantised-cache reference with head dims 64 and 128, prefixes 37, 200 and 1000,
 * and windows 0 and 100.  This is that reference, written out plainly in binary64.
 * Readings taken here:
 *  - one sequence; q [n_new][Hq][d], new keys / values [n_new][Hkv][d] (bf16); query
 *    head h reads kv head h / (Hq / Hkv);
 *  - cache of `prefix` positions, [prefix][Hkv][d] per K and V:
 *      format 0: bf16;
 *      format 1: e4m3 bytes, one fp32 scale per tensor (k_scale, v_scale);
 *      format 2: NVFP4: e2m1 codes [prefix][Hkv][d/2] (low nibble = even element),
 *                one e4m3 scale per 16 elements [prefix][Hkv][d/16], and one fp32
 *                scale per tensor (k_scale, v_scale);
 *    a cached value is code (x block scale) x tensor scale, exact in binary64;
 *  - positions: cache entry j is at j, new token t at prefix + t; query t sees key
 *    position p iff p <= prefix + t and (window == 0 or prefix + t - p < window);
 *  - scores (q . k) / sqrt(d), softmax over the visible keys, out = sum p v / sum p,
 *    rounded once to bf16. */
static double kv_value(int32_t format, const void *codes, const uint8_t *bscale, float tscale,
                       int64_t pos, int32_t Hkv, int32_t d, int32_t kh, int32_t i)
{
    int64_t row = pos * Hkv + kh;
    if (format == 0)
        return or_bf16_to_double(((const uint16_t *)codes)[row * d + i]);
    if (format == 1)
        return or_e4m3(((const uint8_t *)codes)[row * d + i]) * (double)tscale;
    uint8_t b = ((const uint8_t *)codes)[row * (d / 2) + i / 2];
    uint32_t c = (i % 2 == 0) ? (uint32_t)(b & 0x0F) : (uint32_t)(b >> 4);
    return or_e2m1(c) * or_e4m3(bscale[row * (d / 16) + i / 16]) * (double)tscale;
}

int32_t or_attn_extend(int32_t n_new, int32_t prefix, int32_t Hq, int32_t Hkv, int32_t d,
                       int32_t window, const uint16_t *q, const uint16_t *k_new,
                       const uint16_t *v_new, int32_t format, const void *k_cache,
                       const void *v_cache, const uint8_t *k_bscale, const uint8_t *v_bscale,
                       float k_scale, float v_scale, double *out64, uint16_t *out)
{
    if (n_new < 0 || prefix < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || d % 16 ||
        window < 0 || format < 0 || format > 2)
        return -1;
    int32_t group = Hq / Hkv;
    int64_t P = (int64_t)prefix + n_new;
    double scale = 1.0 / sqrt((double)d);
#pragma omp parallel for collapse(2) schedule(static)
    for (int32_t t = 0; t < n_new; ++t) {
        for (int32_t h = 0; h < Hq; ++h) {
            int32_t kh = h / group;
            int64_t qpos = (int64_t)prefix + t;
            double *s = (double *)malloc(sizeof(double) * (size_t)(P > 0 ? P : 1));
            double smax = -INFINITY;
            for (int64_t p = 0; p < P; ++p) {
                int visible = p <= qpos && (window == 0 || qpos - p < window);
                if (!visible) {
                    s[p] = -INFINITY;
                    continue;
                }
                double dot = 0.0;
                for (int32_t i = 0; i < d; ++i) {
                    double kv = p < prefix
                                    ? kv_value(format, k_cache, k_bscale, k_scale, p, Hkv, d, kh, i)
                                    : or_bf16_to_double(k_new[((p - prefix) * Hkv + kh) * d + i]);
                    dot += or_bf16_to_double(q[((int64_t)t * Hq + h) * d + i]) * kv;
                }
                s[p] = dot * scale;
                if (s[p] > smax)
                    smax = s[p];
            }
            double l = 0.0;
            for (int64_t p = 0; p < P; ++p) {
                s[p] = (s[p] == -INFINITY) ? 0.0 : exp(s[p] - smax);
                l += s[p];
            }
            for (int32_t i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int64_t p = 0; p < P; ++p) {
                    if (s[p] == 0.0)
                        continue;
                    double vv = p < prefix
                                    ? kv_value(format, v_cache, v_bscale, v_scale, p, Hkv, d, kh, i)
                                    : or_bf16_to_double(v_new[((p - prefix) * Hkv + kh) * d + i]);
                    acc += s[p] * vv;
                }
                double o = acc / l;
                int64_t idx = ((int64_t)t * Hq + h) * d + i;
                if (out64)
                    out64[idx] = o;
                if (out)
                    out[idx] = or_bf16_from_double(o);
            }
            free(s);
        }
    }
    return 0;
}
