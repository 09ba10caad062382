/* Drives every entry point of the C oracle on small inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize.py):
 * any out-of-bounds access, use of uninitialised heap memory through a bad
 * index, signed overflow or invalid shift aborts the run.  Also checks a few
 * properties cheaply (weights sum to one, the permutation and its inverse).
 * Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double k3o_e2m1(int code);
double k3o_e8m0(int s);
double k3o_silu(double z);
void k3o_mx_dequant(long rows, long cols, const uint8_t *codes, const uint8_t *scales, double *out);
void k3o_router_logits(int T, int E, int d, const float *x, const float *wr, double *logits);
void k3o_select_topk(int T, int E, int k, const double *key, int32_t *idx);
void k3o_topk_weights(int T, int E, int k, const double *logits, const int32_t *idx, double *w);
void k3o_sigmoid(long n, const double *l, double *s);
void k3o_sigmoid_weights(int T, int E, int k, const double *scores, const int32_t *idx, double *w);
int k3o_permute(int T, int E, int k, const int32_t *idx, int32_t *counts, int32_t *offsets, int32_t *perm_pair,
                int32_t *row_of_pair);
void k3o_mx_quantize(long nblocks, const double *v, uint8_t *codes, uint8_t *scales);
void k3o_gateup(int d, int f, const double *x, const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                const uint8_t *us, double *h, double *g_out, double *u_out);
void k3o_down(int d, int f, const double *h, const uint8_t *dc, const uint8_t *ds, double *o);

static uint32_t rng = 12345u;
static uint32_t next_u32(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 17;
    rng ^= rng << 5;
    return rng;
}
static double next_unit(void) { return (next_u32() >> 8) * (1.0 / 16777216.0) * 2.0 - 1.0; }

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            return 1;                                                     \
        }                                                                 \
    } while (0)

int main(void)
{
    enum { T = 7, E = 16, K = 3, D = 256, F = 128 };
    for (int c = 0; c < 16; ++c) CHECK(!isnan(k3o_e2m1(c)));
    for (int s = 0; s < 255; ++s) CHECK(k3o_e8m0(s) > 0.0);
    CHECK(isnan(k3o_e8m0(255)));
    CHECK(k3o_silu(-800.0) <= 0.0 && k3o_silu(800.0) == 800.0);

    /* router: one all-zero token (all logits tie) and two equal router rows */
    float *x = malloc(sizeof(float) * T * D), *wr = malloc(sizeof(float) * E * D);
    for (int i = 0; i < T * D; ++i) x[i] = (float)next_unit();
    for (int i = 0; i < E * D; ++i) wr[i] = (float)(next_unit() / 16.0);
    memset(x + 2 * D, 0, sizeof(float) * D);
    memcpy(wr + 9 * D, wr + 4 * D, sizeof(float) * D);
    double *logits = malloc(sizeof(double) * T * E), *w = malloc(sizeof(double) * T * K);
    int32_t *idx = malloc(sizeof(int32_t) * T * K);
    k3o_router_logits(T, E, D, x, wr, logits);
    k3o_select_topk(T, E, K, logits, idx);
    k3o_topk_weights(T, E, K, logits, idx, w);
    for (int t = 0; t < T; ++t) {
        double sum = 0.0;
        for (int j = 0; j < K; ++j) sum += w[t * K + j];
        CHECK(fabs(sum - 1.0) < 1e-12);
    }
    CHECK(idx[2 * K] == 0 && idx[2 * K + 1] == 1 && idx[2 * K + 2] == 2); /* ties: the lowest indices */
    double *sc = malloc(sizeof(double) * T * E);
    k3o_sigmoid((long)T * E, logits, sc);
    k3o_select_topk(T, E, K, sc, idx);
    k3o_sigmoid_weights(T, E, K, sc, idx, w);

    /* grouping, and its refusal of a repeated expert */
    int32_t counts[E], offsets[E + 1], perm[T * K], row_of[T * K];
    CHECK(k3o_permute(T, E, K, idx, counts, offsets, perm, row_of) == 0);
    CHECK(offsets[E] == T * K);
    for (int p = 0; p < T * K; ++p) CHECK(perm[row_of[p]] == p);
    int32_t bad[T * K];
    memcpy(bad, idx, sizeof(bad));
    bad[1] = bad[0];
    CHECK(k3o_permute(T, E, K, bad, counts, offsets, perm, row_of) == -1);
    bad[1] = E;
    CHECK(k3o_permute(T, E, K, bad, counts, offsets, perm, row_of) == -1);

    /* MX weights with scale bytes 0..252 and zero / -0 code blocks; one expert's FFN */
    const long gbytes = (long)F * D / 2, gsb = (long)F * D / 32;
    uint8_t *gc = malloc(gbytes), *uc = malloc(gbytes), *dc = malloc(gbytes);
    uint8_t *gs = malloc(gsb), *us = malloc(gsb), *ds = malloc(gsb);
    for (long i = 0; i < gbytes; ++i) {
        gc[i] = (uint8_t)next_u32();
        uc[i] = (uint8_t)next_u32();
        dc[i] = (uint8_t)next_u32();
    }
    for (long i = 0; i < gsb; ++i) {
        gs[i] = (uint8_t)(i % 253);
        us[i] = (uint8_t)(100 + i % 40);
        ds[i] = (uint8_t)(110 + i % 30);
    }
    memset(gc, 0x00, 16);  /* an all-zero block */
    memset(uc, 0x88, 16);  /* an all -0 block */
    double *xd = malloc(sizeof(double) * D), *h = malloc(sizeof(double) * F), *o = malloc(sizeof(double) * D);
    double *g = malloc(sizeof(double) * F), *u = malloc(sizeof(double) * F);
    for (int i = 0; i < D; ++i) xd[i] = next_unit();
    k3o_gateup(D, F, xd, gc, gs, uc, us, h, g, u);
    k3o_gateup(D, F, xd, gc, gs, uc, us, h, NULL, NULL);
    k3o_down(D, F, h, dc, ds, o);
    double *dq = malloc(sizeof(double) * F * D);
    k3o_mx_dequant(F, D, gc, gs, dq);
    CHECK(dq[0] == 0.0);

    /* the activation quantiser: ordinary values, amax edges, zeros, subnormals */
    enum { NB = 6 };
    double v[NB * 32];
    for (int i = 0; i < NB * 32; ++i) v[i] = next_unit() * 100.0;
    for (int i = 0; i < 32; ++i) v[32 + i] = 0.0;
    for (int i = 0; i < 32; ++i) v[64 + i] = (i & 1) ? -0.0 : 1e-310;
    v[96] = 6.0 * ldexp(1.0, 120);
    v[128] = ldexp(1.0, -130);
    uint8_t qc[NB * 16], qs[NB];
    k3o_mx_quantize(NB, v, qc, qs);
    for (int i = 0; i < 16; ++i) CHECK(qc[16 + i] == 0);

    free(x); free(wr); free(logits); free(w); free(idx); free(sc);
    free(gc); free(uc); free(dc); free(gs); free(us); free(ds);
    free(xd); free(h); free(o); free(g); free(u); free(dq);
    printf("oracle driver ok\n");
    return 0;
}
