/*
 * asf_oracle.c -- plain, slow, obviously correct CPU reference (fp64) for the
 * activation-sparse ReLU FFN decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library and never touches a GPU.
 *
 * Sources (pages are cited by title and section):
 *   [ZH]  "LLM模型之PowerInfer1.0" (blog notes on PowerInfer 1.0 + DejaVu appendix)
 *   [VI]  "PowerInfer: Nhanh Large Language Model với GPU Tiêu dùng"
 *   [ES]  "Técnicas dispersas para una aceleración 100X en la inferencia de
 *          modelos de lenguaje grandes"
 *
 * Conventions
 *   - Weights arrive in their original (nn.Linear) layouts:
 *       W_up, W_gate [f][d], W_down [d][f], P1 [H][d], P2 [f][H].
 *     wtype 0 = IEEE binary32, wtype 1 = IEEE binary16 (raw bits).
 *   - Every weight is widened exactly to double; fp32 inputs (x, biases) too.
 *   - All arithmetic is double; sums run in ascending index order.
 *   - Parity pins for every function live in tests/ (closed forms, brute force,
 *     library cross-checks, the worked example of [ZH] §3.2 / [ES]).
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fPIC -shared [-fopenmp]
 * OpenMP only splits independent output elements across threads; it never
 * changes the order of any single sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------------
 * IEEE-754 binary16 -> double, written from the format's definition:
 *   sign (1 bit) | exponent e (5 bits, bias 15) | fraction m (10 bits)
 *   e == 0       : subnormal, value = m * 2^-24 (signed zero when m == 0)
 *   e == 31      : infinity (m == 0) or NaN (m != 0)
 *   otherwise    : value = (1024 + m) * 2^(e - 25)
 * ------------------------------------------------------------------------- */
double orc_half_to_double(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 31;
    int m = bits & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = (m == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

static double wval(const void *w, int wtype, size_t idx)
{
    if (wtype == 1)
        return orc_half_to_double(((const uint16_t *)w)[idx]);
    return (double)((const float *)w)[idx];
}

static double opt_f32(const float *v, size_t idx)
{
    return v ? (double)v[idx] : 0.0;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------------------
 * Predictor: a two-layer MLP X-H-O per FFN layer ([ZH] §1 "自适应" and
 * appendix "DejaVu": one two-layer MLP scores the MLP neurons; each output is
 * a binary decision through a sigmoid).
 *
 *   h_k = max(0, c1_k + sum_j P1[k][j] x_j)           k < H
 *   s_i = c2_i + sum_k P2[i][k] h_k                    i < f (original ids)
 *   active_i = (s_i > theta)
 *
 * The hidden nonlinearity is not stated on the pages: ReLU is taken.  The
 * per-output sigmoid decision sigmoid(s) > 0.5 is the logit test s > 0, so
 * theta is a logit threshold (default 0); a tie s == theta is inactive.
 *
 * x: [B][d] fp32.  Outputs (each nullable): h [B][H], s [B][f], act [B][f].
 * ------------------------------------------------------------------------- */
int orc_predict(int d, int f, int H, int wtype,
                const void *P1, const float *c1,
                const void *P2, const float *c2,
                double theta, const float *x, int B,
                double *h_out, double *s_out, uint8_t *act_out)
{
    if (d <= 0 || f <= 0 || H <= 0 || B < 0 || !P1 || !P2 || (B > 0 && !x))
        return -1;
    double *h = (double *)malloc(sizeof(double) * (size_t)H);
    if (!h)
        return -2;
    for (int b = 0; b < B; ++b) {
        const float *xb = x + (size_t)b * d;
        int k;
#pragma omp parallel for schedule(static)
        for (k = 0; k < H; ++k) {
            double acc = opt_f32(c1, k);
            for (int j = 0; j < d; ++j)
                acc += wval(P1, wtype, (size_t)k * d + j) * (double)xb[j];
            h[k] = acc > 0.0 ? acc : 0.0;
        }
        if (h_out)
            memcpy(h_out + (size_t)b * H, h, sizeof(double) * (size_t)H);
        int i;
#pragma omp parallel for schedule(static)
        for (i = 0; i < f; ++i) {
            double acc = opt_f32(c2, i);
            for (int kk = 0; kk < H; ++kk)
                acc += wval(P2, wtype, (size_t)i * H + kk) * h[kk];
            if (s_out)
                s_out[(size_t)b * f + i] = acc;
            if (act_out)
                act_out[(size_t)b * f + i] = (uint8_t)(acc > theta);
        }
    }
    free(h);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Union of per-token active sets for batched decode: neuron i is in U when any
 * token of the batch activates it (the "joint activation" whose density grows
 * with batch size, [ES] "Impacto del tamaño del lote").
 * ------------------------------------------------------------------------- */
void orc_union(int B, int f, const uint8_t *act, uint8_t *u_out)
{
    for (int i = 0; i < f; ++i) {
        uint8_t u = 0;
        for (int b = 0; b < B; ++b)
            u |= act[(size_t)b * f + i] ? 1 : 0;
        u_out[i] = u;
    }
}

/* ---------------------------------------------------------------------------
 * Neuron table ([ZH] §4.2, [VI] "Đặt vị trí và Quản lý Nơ-ron"): the stored
 * (physical) order of neurons differs from their original position, and a
 * table maps each stored slot back to its original id: perm[slot] = id.
 *
 * Hot-first order: neurons sorted by impact v_i = f_i, the profiled
 * activation frequency ([ZH] §5.2, Eq. 1), largest first; equal counts keep
 * the smaller original id first.
 * ------------------------------------------------------------------------- */
static const int64_t *g_sort_counts;

static int cmp_hot_first(const void *a, const void *b)
{
    int32_t ia = *(const int32_t *)a, ib = *(const int32_t *)b;
    int64_t ca = g_sort_counts[ia], cb = g_sort_counts[ib];
    if (ca != cb)
        return ca > cb ? -1 : 1;
    return ia < ib ? -1 : (ia > ib ? 1 : 0);
}

int orc_hot_first_table(int f, const int64_t *counts, int32_t *perm_out)
{
    if (f < 0 || (f > 0 && (!counts || !perm_out)))
        return -1;
    for (int i = 0; i < f; ++i)
        perm_out[i] = i;
    g_sort_counts = counts;
    qsort(perm_out, (size_t)f, sizeof(int32_t), cmp_hot_first);
    g_sort_counts = NULL;
    return 0;
}

/* Activation counting (the offline profiler's monitor of [ZH] §5.1): add one
 * to a neuron's count for every token on which it is active. */
void orc_count_activations(int B, int f, const uint8_t *act, int64_t *counts)
{
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < f; ++i)
            counts[i] += act[(size_t)b * f + i] ? 1 : 0;
}

/* Canonical active list: walk the stored slots in ascending order and emit
 * the original id of every slot whose neuron is active.  Returns the count. */
int orc_active_list(int f, const int32_t *perm, const uint8_t *active_by_id,
                    int32_t *ids_out)
{
    int n = 0;
    for (int slot = 0; slot < f; ++slot) {
        int32_t id = perm ? perm[slot] : slot;
        if (active_by_id[id])
            ids_out[n++] = id;
    }
    return n;
}

/* ---------------------------------------------------------------------------
 * FFN over a neuron set S ([ZH] §2.1 Fig. 1; [ZH] "其他" Q3 on AXPY):
 *
 *   plain : a_i = max(0, b1_i + W_up[i] . x)
 *   gated : a_i = max(0, b1_i + W_gate[i] . x) * (W_up[i] . x)
 *   y_m   = r_m + b2_m + sum_{i in S} a_i * W_down[m][i]
 *
 * FC1 is a dot product of the input with neuron row i; FC2 adds a_i times
 * column i of W_down (the AXPY form).  Neurons outside S contribute nothing.
 * The gated form (ReLU in place of SiLU on the gate) is not on the pages; it
 * is the plainest ReLU variant of a gated FFN.  Biases are not on the pages
 * either: b1 / b2 are optional (NULL = 0).  r is an optional residual input
 * (NULL = 0) used when layers are chained.
 *
 * Batch B > 1 with S = the union of the tokens' sets: every token computes
 * every neuron of S (union reading).  If token_act ([B][f], by original id)
 * is given, token b instead keeps a_{b,i} only where token_act[b][i] is set
 * (per-token masked reading).
 *
 * S is any list of distinct original ids; it is sorted so every sum runs in
 * ascending original id.  a_out [B][nS] (nullable) receives a in that sorted
 * order.  y_out [B][d].
 * ------------------------------------------------------------------------- */
static int cmp_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return x < y ? -1 : (x > y ? 1 : 0);
}

int orc_ffn(int d, int f, int wtype, int gated,
            const void *W_up, const void *W_gate, const float *b1,
            const void *W_down, const float *b2, const float *resid,
            const float *x, int B, const int32_t *S, int nS,
            const uint8_t *token_act, double *a_out, double *y_out)
{
    if (d <= 0 || f <= 0 || B < 0 || nS < 0 || nS > f || !W_up || !W_down ||
        (gated && !W_gate) || (nS > 0 && !S) || (B > 0 && (!x || !y_out)))
        return -1;
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nS > 0 ? nS : 1));
    double *a = (double *)malloc(sizeof(double) * (size_t)(nS > 0 ? nS : 1));
    if (!ids || !a) {
        free(ids);
        free(a);
        return -2;
    }
    if (nS > 0)
        memcpy(ids, S, sizeof(int32_t) * (size_t)nS);
    qsort(ids, (size_t)nS, sizeof(int32_t), cmp_i32);
    for (int t = 0; t < nS; ++t) {
        if (ids[t] < 0 || ids[t] >= f || (t > 0 && ids[t] == ids[t - 1])) {
            free(ids);
            free(a);
            return -3;
        }
    }
    for (int b = 0; b < B; ++b) {
        const float *xb = x + (size_t)b * d;
        int t;
#pragma omp parallel for schedule(static)
        for (t = 0; t < nS; ++t) {
            int i = ids[t];
            double ai;
            if (gated) {
                double g = opt_f32(b1, i), u = 0.0;
                for (int j = 0; j < d; ++j) {
                    g += wval(W_gate, wtype, (size_t)i * d + j) * (double)xb[j];
                    u += wval(W_up, wtype, (size_t)i * d + j) * (double)xb[j];
                }
                ai = (g > 0.0 ? g : 0.0) * u;
            } else {
                double z = opt_f32(b1, i);
                for (int j = 0; j < d; ++j)
                    z += wval(W_up, wtype, (size_t)i * d + j) * (double)xb[j];
                ai = z > 0.0 ? z : 0.0;
            }
            if (token_act && !token_act[(size_t)b * f + i])
                ai = 0.0;
            a[t] = ai;
        }
        if (a_out)
            memcpy(a_out + (size_t)b * nS, a, sizeof(double) * (size_t)nS);
        int m;
#pragma omp parallel for schedule(static)
        for (m = 0; m < d; ++m) {
            double acc = opt_f32(resid ? resid + (size_t)b * d : NULL, m) + opt_f32(b2, m);
            for (int tt = 0; tt < nS; ++tt)
                acc += a[tt] * wval(W_down, wtype, (size_t)m * f + ids[tt]);
            y_out[(size_t)b * d + m] = acc;
        }
    }
    free(ids);
    free(a);
    return 0;
}

/* Dense FFN: the same FFN over every neuron (S = all f), the computation the
 * sparse path is compared with ([ES] "Viabilidad": ReLU saves FLOPs relative
 * to the full FC1 -> ReLU -> FC2). */
int orc_dense_ffn(int d, int f, int wtype, int gated,
                  const void *W_up, const void *W_gate, const float *b1,
                  const void *W_down, const float *b2, const float *resid,
                  const float *x, int B, double *y_out)
{
    int32_t *all = (int32_t *)malloc(sizeof(int32_t) * (size_t)(f > 0 ? f : 1));
    if (!all)
        return -2;
    for (int i = 0; i < f; ++i)
        all[i] = i;
    int rc = orc_ffn(d, f, wtype, gated, W_up, W_gate, b1, W_down, b2, resid,
                     x, B, all, f, NULL, NULL, y_out);
    free(all);
    return rc;
}

/* True mask of a token: the neurons whose FC1 result is nonzero after ReLU,
 * i.e. pre-activation (gate pre-activation when gated) strictly above zero.
 * act_out [B][f] by original id; pre_out [B][f] nullable. */
int orc_true_mask(int d, int f, int wtype, int gated,
                  const void *W_up, const void *W_gate, const float *b1,
                  const float *x, int B, double *pre_out, uint8_t *act_out)
{
    if (d <= 0 || f <= 0 || B < 0 || !W_up || (gated && !W_gate))
        return -1;
    const void *W = gated ? W_gate : W_up;
    for (int b = 0; b < B; ++b) {
        const float *xb = x + (size_t)b * d;
        int i;
#pragma omp parallel for schedule(static)
        for (i = 0; i < f; ++i) {
            double z = opt_f32(b1, i);
            for (int j = 0; j < d; ++j)
                z += wval(W, wtype, (size_t)i * d + j) * (double)xb[j];
            if (pre_out)
                pre_out[(size_t)b * f + i] = z;
            act_out[(size_t)b * f + i] = (uint8_t)(z > 0.0);
        }
    }
    return 0;
}
