/* oracle_check.c -- runs every entry point of the CPU oracle (oracle/ftmoe_oracle.c)
 * on small random layers, built with the address and undefined-behaviour
 * sanitizers by tests/test_sanitizers.py: shapes with and without a shared expert,
 * k = 1 and k = E, given routes, NaN and signed-zero logits, a NaN block scale and
 * zero tokens.  Only memory safety and defined behaviour are checked here (the
 * numbers are pinned elsewhere).  Prints "ok" and exits 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double or_e2m1(uint32_t code);
double or_e4m3(uint32_t byte);
float or_dequant_value(uint32_t code, uint32_t scale_byte, float g);
void or_dequant_matrix(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                       float g, float *out);
double or_bf16_to_double(uint16_t b);
uint16_t or_bf16_from_double(double v);
void or_router_logits(int64_t T, int32_t E, int32_t H, const uint16_t *x, const float *W,
                      const float *bias, float *logits);
void or_topk(int64_t T, int32_t E, int32_t k, const float *logits, int32_t *ids, float *w);
double or_swiglu(int32_t act, double g, double u, double gate_max, double up_absmax);
void or_expert_output(int32_t H, int32_t I, int64_t e, const uint8_t *w13c, const uint8_t *w13s,
                      const uint8_t *w2c, const uint8_t *w2s, const float *gsc, int32_t act,
                      float gate_max, float up_absmax, const uint16_t *x, double *o);
int32_t or_moe_layer(int32_t E, int32_t H, int32_t I, int32_t k, int32_t act, float gate_max,
                     float up_absmax, int64_t T, const uint16_t *x, const float *Wr,
                     const float *bias, const uint8_t *w13c, const uint8_t *w13s,
                     const uint8_t *w2c, const uint8_t *w2s, const float *gsc, int32_t Is,
                     const uint8_t *s13c, const uint8_t *s13s, const uint8_t *s2c,
                     const uint8_t *s2s, const float *sgsc, const uint16_t *sgate,
                     const int32_t *ids_in, const float *w_in, int32_t *ids_out, float *w_out,
                     double *y64, uint16_t *y);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (uint32_t)(g_state >> 16);
}

static void *fill_bytes(size_t n)
{
    uint8_t *p = (uint8_t *)malloc(n ? n : 1);
    for (size_t i = 0; i < n; ++i)
        p[i] = (uint8_t)rnd();
    return p;
}

static uint8_t *scales(size_t n)
{
    uint8_t *p = (uint8_t *)malloc(n ? n : 1);
    for (size_t i = 0; i < n; ++i)
        p[i] = (uint8_t)((3 + rnd() % 7) << 3); /* 2^-4 .. 2^2 */
    return p;
}

static float *normal_f32(size_t n, float sd)
{
    float *p = (float *)malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i)
        p[i] = sd * ((float)(rnd() % 20001) / 10000.0f - 1.0f);
    return p;
}

static uint16_t *tokens(size_t n)
{
    uint16_t *p = (uint16_t *)malloc(sizeof(uint16_t) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) {
        float f = (float)(rnd() % 20001) / 5000.0f - 2.0f;
        uint32_t u;
        memcpy(&u, &f, 4);
        p[i] = (uint16_t)(u >> 16);
    }
    return p;
}

static int run_layer(int E, int H, int I, int k, int act, int64_t T, int Is, int given,
                     int nan_scale, int special_router)
{
    uint8_t *w13c = fill_bytes((size_t)E * 2 * I * H / 2), *w13s = scales((size_t)E * 2 * I * H / 16);
    uint8_t *w2c = fill_bytes((size_t)E * H * I / 2), *w2s = scales((size_t)E * H * I / 16);
    float *gsc = normal_f32((size_t)E * 3, 1.0f), *wr = normal_f32((size_t)E * H, 0.02f);
    uint8_t *s13c = NULL, *s13s = NULL, *s2c = NULL, *s2s = NULL;
    float *sg = NULL;
    uint16_t *sgate = NULL;
    if (nan_scale)
        w13s[1] = 0x7F; /* e4m3 NaN */
    if (special_router && E > 3) {
        memset(wr, 0, sizeof(float) * H);           /* +0 logits */
        wr[H + 3] = NAN;                             /* NaN logits */
        for (int h = 0; h < H; ++h) wr[2 * H + h] = -0.0f;
    }
    if (Is > 0) {
        s13c = fill_bytes((size_t)2 * Is * H / 2);
        s13s = scales((size_t)2 * Is * H / 16);
        s2c = fill_bytes((size_t)H * Is / 2);
        s2s = scales((size_t)H * Is / 16);
        sg = normal_f32(3, 1.0f);
        sgate = tokens((size_t)H);
    }
    uint16_t *x = tokens((size_t)T * H);
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T ? T : 1) * k);
    float *w = (float *)malloc(sizeof(float) * (size_t)(T ? T : 1) * k);
    double *y64 = (double *)malloc(sizeof(double) * (size_t)(T ? T : 1) * H);
    uint16_t *y = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(T ? T : 1) * H);
    int32_t *ids_in = NULL;
    float *w_in = NULL;
    if (given) {
        ids_in = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T ? T : 1) * k);
        w_in = (float *)malloc(sizeof(float) * (size_t)(T ? T : 1) * k);
        for (int64_t i = 0; i < T * k; ++i) {
            ids_in[i] = (int32_t)((i * 7 + 3) % E);
            w_in[i] = 1.0f / (float)k;
        }
    }
    int rc = or_moe_layer(E, H, I, k, act, 7.0f, 7.0f, T, x, wr, NULL, w13c, w13s, w2c, w2s, gsc,
                          Is, s13c, s13s, s2c, s2s, sg, sgate, ids_in, w_in, ids, w, y64, y);
    if (T > 0) {
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
        or_expert_output(H, I, E - 1, w13c, w13s, w2c, w2s, gsc, act, 7.0f, 7.0f, x, o);
        free(o);
        float *lg = (float *)malloc(sizeof(float) * (size_t)T * E);
        or_router_logits(T, E, H, x, wr, gsc /* any E floats as a bias */, lg);
        or_topk(T, E, k, lg, ids, w);
        free(lg);
    }
    free(w13c); free(w13s); free(w2c); free(w2s); free(gsc); free(wr);
    free(s13c); free(s13s); free(s2c); free(s2s); free(sg); free(sgate);
    free(x); free(ids); free(w); free(y64); free(y); free(ids_in); free(w_in);
    return rc;
}

int main(void)
{
    for (uint32_t c = 0; c < 16; ++c)
        (void)or_e2m1(c);
    for (uint32_t b = 0; b < 256; ++b)
        for (uint32_t c = 0; c < 16; ++c)
            (void)or_dequant_value(c, b, 0.75f);
    double specials[] = {0.0, -0.0, 1e-300, -1e-300, 3.4e38, 1e39, -1e39, NAN, INFINITY, 1.0 / 3.0};
    for (unsigned i = 0; i < sizeof specials / sizeof specials[0]; ++i) {
        uint16_t b = or_bf16_from_double(specials[i]);
        (void)or_bf16_to_double(b);
        (void)or_swiglu(1, specials[i], specials[i], 7.0, 7.0);
        (void)or_swiglu(0, specials[i], -specials[i], 7.0, 7.0);
    }
    int bad = 0;
    bad |= run_layer(8, 256, 128, 2, 0, 1, 0, 0, 0, 0);      /* tiny workload shape */
    bad |= run_layer(12, 256, 128, 10, 1, 3, 128, 0, 0, 0);  /* shared expert */
    bad |= run_layer(6, 256, 64, 6, 1, 2, 0, 0, 0, 0);       /* k = E */
    bad |= run_layer(9, 128, 32, 1, 1, 4, 64, 0, 1, 0);      /* k = 1, NaN scale */
    bad |= run_layer(16, 256, 64, 4, 1, 5, 0, 1, 0, 0);      /* given routes */
    bad |= run_layer(20, 256, 64, 16, 1, 2, 0, 0, 0, 1);     /* zero / NaN logits */
    bad |= run_layer(8, 256, 128, 2, 1, 0, 64, 0, 0, 0);     /* zero tokens */
    if (or_moe_layer(0, 256, 128, 2, 1, 7.0f, 7.0f, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                     NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                     NULL) != -1)
        bad = 1; /* bad shapes are rejected before any access */
    if (bad) {
        printf("a layer call failed\n");
        return 1;
    }
    printf("ok\n");
    return 0;
}
