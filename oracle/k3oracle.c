/*
 * k3oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU statement of what the routed-expert MoE layer
 * computes.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library; the product path never does.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * Sources (the pages describe the "kimi-k3-in-c" CPU engine):
 *   [DD]  fiv.co.kr, "kimi-k3-in-c deep dive" (Korean)
 *   [RL]  repolode.com, "FareedKhan-dev/kimi-k3-in-c" (Portuguese)
 *   [HR]  hotrepo.ai, "FareedKhan-dev/kimi-k3-in-c" (Chinese)
 *   [YP]  yunpan.plus, "176KB pure-C inference engine ... Kimi K3" (Chinese)
 *
 * Every dot product below is evaluated in fp64 with a strictly sequential
 * (ascending index) reduction, so results do not depend on the OpenMP
 * thread count.  OpenMP only splits independent rows / tokens.
 *
 * Functions whose result has no independent pin are marked "parity unpinned"
 * in their comment; at present every exported function has pins (see tests).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ O1 --- */
/* E2M1 magnitudes by the low three bits of a 4-bit code; bit 3 is the sign.
 * [DD] "four reductions", first reduction (MXFP4 note): the format holds only
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives.  [DD] glossary, "MXFP4". */
static const double E2M1_MAGNITUDE[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double k3o_e2m1(int code)
{
    double m = E2M1_MAGNITUDE[code & 7];
    return (code & 8) ? -m : m;
}

/* E8M0 shared exponent: value = 2^(s - 127).  [DD] "four reductions", MXFP4
 * note: value = E2M1[nibble] x 2^(scale - 127), one 8-bit scale per 32 values.
 * s = 255 is NaN in the OCP MX format and is outside the layer's contract. */
double k3o_e8m0(int s)
{
    if (s == 255) return NAN;
    return ldexp(1.0, s - 127);
}

/* Element i of one MX row: code from byte i/2 (even element in the low
 * nibble), scale from byte i/32.  The nibble order is not stated on the pages
 * ([DD] exercises only warn that flipping it is silently wrong); the low-
 * nibble-first order is the OCP MX packing. */
static double mx_element(const uint8_t *codes, const uint8_t *scales, long i)
{
    int byte = codes[i >> 1];
    int code = (i & 1) ? (byte >> 4) : (byte & 15);
    return k3o_e2m1(code) * k3o_e8m0(scales[i >> 5]);
}

/* Explicit dequantisation of a [rows][cols] MX matrix into fp64 (the pages'
 * k3_mxfp4_dequant, [DD] exercises).  Used only to cross-check the on-code
 * dot products below against a dense matmul. */
void k3o_mx_dequant(long rows, long cols, const uint8_t *codes,
                    const uint8_t *scales, double *out)
{
    #pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r)
        for (long i = 0; i < cols; ++i)
            out[r * cols + i] = mx_element(codes + r * (cols / 2),
                                           scales + r * (cols / 32), i);
}

/* Dot product of MX row r (length n) with an fp64 vector, ascending i: each
 * weight is decoded on the fly from its nibble and its block's scale, and the
 * matrix is never expanded ([DD] "four reductions", MXFP4 note; [YP] section
 * 02, computing on MXFP4 directly). */
static double mx_row_dot(const uint8_t *codes, const uint8_t *scales, long n,
                         const double *v)
{
    double acc = 0.0;
    for (long b = 0; b < n / 32; ++b) {
        double sc = k3o_e8m0(scales[b]);
        for (long i = 32 * b; i < 32 * b + 32; ++i) {
            int byte = codes[i >> 1];
            int code = (i & 1) ? (byte >> 4) : (byte & 15);
            acc += (k3o_e2m1(code) * sc) * v[i];
        }
    }
    return acc;
}

/* ------------------------------------------------------------------ O2 --- */
/* Router logits l[t][e] = sum_i x[t][i] * Wr[e][i] in fp64 (each fp32 x fp32
 * product is exact in fp64).  The router is named k3_router on [DD] (study
 * plan, week 4); 16 of 896 experts are chosen per token ([DD] glossary "MoE",
 * [RL] "O que e?"). */
void k3o_router_logits(int T, int E, int d, const float *x, const float *wr,
                       double *logits)
{
    #pragma omp parallel for schedule(static)
    for (long te = 0; te < (long)T * E; ++te) {
        long t = te / E, e = te % E;
        double acc = 0.0;
        for (long i = 0; i < d; ++i)
            acc += (double)x[t * d + i] * (double)wr[e * d + i];
        logits[te] = acc;
    }
}

/* ------------------------------------------------------------------ O3 --- */
/* Top-k selection: the first k experts of the order "key descending, then
 * expert index ascending".  The pages do not state a tie rule; ties go to the
 * lower expert index.  Written as k rounds of "pick the best not yet taken",
 * which is exactly the first k entries of that full order. */
void k3o_select_topk(int T, int E, int k, const double *key, int32_t *idx)
{
    #pragma omp parallel for schedule(static)
    for (long t = 0; t < T; ++t) {
        const double *kt = key + t * (long)E;
        char *taken = (char *)calloc((size_t)E, 1);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || kt[e] > kt[best]) best = e; /* strict: lower e wins ties */
            }
            taken[best] = 1;
            idx[t * (long)k + j] = best;
        }
        free(taken);
    }
}

/* ------------------------------------------------------------------ O4 --- */
/* Combine weights: the literal full softmax over all E logits, then the k
 * selected probabilities renormalised to sum to one.  (The pages' own router
 * uses sigmoid scores -- [DD] invariant #5 -- the layer measured here uses
 * softmax with renormalised top-k weights.) */
void k3o_topk_weights(int T, int E, int k, const double *logits,
                      const int32_t *idx, double *w)
{
    #pragma omp parallel for schedule(static)
    for (long t = 0; t < T; ++t) {
        const double *lt = logits + t * (long)E;
        double mx = lt[0];
        for (int e = 1; e < E; ++e) if (lt[e] > mx) mx = lt[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) z += exp(lt[e] - mx);
        double sel = 0.0;
        for (int j = 0; j < k; ++j) sel += exp(lt[idx[t * k + j]] - mx) / z;
        for (int j = 0; j < k; ++j)
            w[t * k + j] = (exp(lt[idx[t * k + j]] - mx) / z) / sel;
    }
}

/* Sigmoid scores (the pages' router: each expert scored by a sigmoid of its
 * logit, [DD] invariant #5 and the MoE-routing study-plan row), in the form
 * that never overflows: 1/(1+e^-l) for l >= 0, e^l/(1+e^l) below. */
void k3o_sigmoid(long n, const double *l, double *s)
{
    for (long i = 0; i < n; ++i) {
        const double v = l[i];
        if (v >= 0.0) {
            s[i] = 1.0 / (1.0 + exp(-v));
        } else {
            const double ev = exp(v);
            s[i] = ev / (1.0 + ev);
        }
    }
}

/* Sigmoid combine weights: the chosen experts' scores, renormalised to sum
 * to one (the pages weight by the bias-free scores; the renormalisation is
 * the reading taken, as for softmax). */
void k3o_sigmoid_weights(int T, int E, int k, const double *scores, const int32_t *idx, double *w)
{
    for (long t = 0; t < T; ++t) {
        const double *st = scores + t * (long)E;
        double sum = 0.0;
        for (int j = 0; j < k; ++j) sum += st[idx[t * k + j]];
        for (int j = 0; j < k; ++j) w[t * k + j] = st[idx[t * k + j]] / sum;
    }
}

/* ------------------------------------------------------------------ O5 --- */
/* Grouping of token-expert pairs by expert (the pages' k3_moe runs "the
 * selected experts"; [DD] study plan week 4).  counts[e] = number of tokens
 * that chose e; offsets = exclusive prefix sum (E+1 entries); rows of expert e
 * hold its tokens in ascending t; perm_pair[row] = t*k + j; row_of_pair is the
 * inverse.  Returns -1 (and writes nothing useful) if an index is out of range
 * or repeated within one token. */
int k3o_permute(int T, int E, int k, const int32_t *idx, int32_t *counts,
                int32_t *offsets, int32_t *perm_pair, int32_t *row_of_pair)
{
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (long t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = idx[t * k + j];
            if (e < 0 || e >= E) return -1;
            for (int j2 = 0; j2 < j; ++j2)
                if (idx[t * k + j2] == e) return -1;
            counts[e]++;
        }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    long row = 0;
    for (int e = 0; e < E; ++e)
        for (long t = 0; t < T; ++t)
            for (int j = 0; j < k; ++j)
                if (idx[t * k + j] == e) {
                    perm_pair[row] = (int32_t)(t * k + j);
                    row_of_pair[t * k + j] = (int32_t)row;
                    ++row;
                }
    return 0;
}

/* ------------------------------------------------------------------ O8 --- */
/* MXFP4 quantiser for one 32-element block, the OCP MX v1.0 conversion (the
 * pages give only the decode direction, [DD] MXFP4 note):
 *   amax = max |v|;  amax == 0  -> scale byte 0, every code sign-only;
 *   else e = floor(log2 amax) - 2 (2 = largest E2M1 exponent),
 *        scale byte = clamp(e + 127, 0, 254);
 *   m_i = |v_i| / 2^(byte-127), rounded to the nearest of
 *        {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even index, saturating at 6;
 *   code = sign(v_i) << 3 | index.
 * Decisions are exact: scaling by a power of two and comparing with the
 * midpoints involve no rounding for any fp32 input. */
static int e2m1_index_rne(double m)
{
    /* midpoints between consecutive magnitudes and the index on each side */
    static const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
    for (int i = 0; i < 7; ++i) {
        if (m < mid[i]) return i;
        if (m == mid[i]) return (i % 2 == 0) ? i : i + 1; /* tie -> even index */
    }
    return 7; /* m > 5: nearest is 6 (and saturation beyond 6) */
}

void k3o_mx_quantize(long nblocks, const double *v, uint8_t *codes,
                     uint8_t *scales)
{
    #pragma omp parallel for schedule(static)
    for (long b = 0; b < nblocks; ++b) {
        const double *vb = v + 32 * b;
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) if (fabs(vb[i]) > amax) amax = fabs(vb[i]);
        int byte = 0;
        if (amax > 0.0) {
            int ex;
            frexp(amax, &ex);            /* amax = f * 2^ex, f in [0.5, 1) */
            int e = (ex - 1) - 2;        /* floor(log2 amax) - emax(E2M1) */
            byte = e + 127;
            if (byte < 0) byte = 0;
            if (byte > 254) byte = 254;
        }
        scales[b] = (uint8_t)byte;
        for (int i = 0; i < 32; i += 2) {
            int c[2];
            for (int h = 0; h < 2; ++h) {
                double x = vb[i + h];
                int idx = 0;
                if (amax > 0.0) idx = e2m1_index_rne(ldexp(fabs(x), 127 - byte));
                c[h] = (signbit(x) ? 8 : 0) | idx;
            }
            codes[16 * b + i / 2] = (uint8_t)(c[0] | (c[1] << 4));
        }
    }
}

/* ------------------------------------------------------------------ O6 --- */
/* Logistic function in the form that never overflows: 1/(1+e^-z) for z >= 0,
 * e^z/(1+e^z) for z < 0. */
static double sigmoid(double z)
{
    if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
    double ez = exp(z);
    return ez / (1.0 + ez);
}

double k3o_silu(double z) { return z * sigmoid(z); }

/* Gate/up half of one expert's SwiGLU FFN on MX weights:
 * g_r = Wg[r,:] . x,  u_r = Wu[r,:] . x,  h_r = silu(g_r) * u_r.
 * Wg, Wu are [f][d] MX matrices (32-blocks along d).  Optional g, u outputs. */
void k3o_gateup(int d, int f, const double *x,
                const uint8_t *gc, const uint8_t *gs,
                const uint8_t *uc, const uint8_t *us,
                double *h, double *g_out, double *u_out)
{
    #pragma omp parallel for schedule(static)
    for (long r = 0; r < f; ++r) {
        double g = mx_row_dot(gc + r * (d / 2), gs + r * (d / 32), d, x);
        double u = mx_row_dot(uc + r * (d / 2), us + r * (d / 32), d, x);
        h[r] = k3o_silu(g) * u;
        if (g_out) g_out[r] = g;
        if (u_out) u_out[r] = u;
    }
}

/* Down half: o_c = Wd[c,:] . h, Wd is a [d][f] MX matrix (32-blocks along f). */
void k3o_down(int d, int f, const double *h, const uint8_t *dc,
              const uint8_t *ds, double *o)
{
    #pragma omp parallel for schedule(static)
    for (long c = 0; c < d; ++c)
        o[c] = mx_row_dot(dc + c * (f / 2), ds + c * (f / 32), f, h);
}

/* Convenience: set the number of OpenMP threads (no-op without OpenMP). */
void k3o_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Convenience: number of threads OpenMP will use (0 when built without it). */
int k3o_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
