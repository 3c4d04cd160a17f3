/* Driver that runs every function of the C oracle on small inputs in buffers
 * of exactly the documented sizes, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py): an access past
 * any buffer, a use after free, a leak or undefined arithmetic aborts it.
 * Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_half_to_double(uint16_t bits);
int orc_predict(int d, int f, int H, int wtype, const void *P1, const float *c1, const void *P2,
                const float *c2, double theta, const float *x, int B, double *h_out,
                double *s_out, uint8_t *act_out);
void orc_union(int B, int f, const uint8_t *act, uint8_t *u_out);
int orc_hot_first_table(int f, const int64_t *counts, int32_t *perm_out);
void orc_count_activations(int B, int f, const uint8_t *act, int64_t *counts);
int orc_active_list(int f, const int32_t *perm, const uint8_t *active_by_id, int32_t *ids_out);
int orc_ffn(int d, int f, int wtype, int gated, const void *W_up, const void *W_gate,
            const float *b1, const void *W_down, const float *b2, const float *resid,
            const float *x, int B, const int32_t *S, int nS, const uint8_t *token_act,
            double *a_out, double *y_out);
int orc_dense_ffn(int d, int f, int wtype, int gated, const void *W_up, const void *W_gate,
                  const float *b1, const void *W_down, const float *b2, const float *resid,
                  const float *x, int B, double *y_out);
int orc_true_mask(int d, int f, int wtype, int gated, const void *W_up, const void *W_gate,
                  const float *b1, const float *x, int B, double *pre_out, uint8_t *act_out);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static double rnd(void) /* xorshift64*, uniform in [-1, 1) */
{
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (double)((g_state * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0;
}

/* a weight matrix of n elements, binary32 or binary16 (the bits of a value
 * that binary16 holds exactly: k / 1024 with |k| < 1024) */
static void *weights(int wtype, size_t n)
{
    if (wtype == 0) {
        float *w = malloc(n * sizeof(float));
        for (size_t i = 0; i < n; ++i)
            w[i] = (float)rnd();
        return w;
    }
    uint16_t *w = malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) {
        int k = (int)(rnd() * 1023.0);
        float v = (float)k / 1024.0f;
        /* binary16 of v: exponent and fraction written out for |v| in [2^-10, 1) */
        uint16_t bits = 0;
        if (k != 0) {
            int a = k < 0 ? -k : k, e = 0;
            while ((a << e) < 1024)
                ++e;
            bits = (uint16_t)(((25 - e - 10) << 10) | (((a << e) - 1024) & 1023));
            if (k < 0)
                bits |= 0x8000;
        }
        (void)v;
        w[i] = bits;
    }
    return w;
}

static float *vec(size_t n)
{
    float *v = malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i)
        v[i] = (float)rnd();
    return v;
}

static int fail(const char *what)
{
    fprintf(stderr, "oracle check failed: %s\n", what);
    return 1;
}

int main(void)
{
    for (uint32_t b = 0; b < 65536; ++b) {
        volatile double v = orc_half_to_double((uint16_t)b);
        (void)v;
    }
    const int d = 24, f = 37, H = 10, B = 3;
    for (int wtype = 0; wtype < 2; ++wtype) {
        for (int gated = 0; gated < 2; ++gated) {
            void *P1 = weights(wtype, (size_t)H * d), *P2 = weights(wtype, (size_t)f * H);
            void *Wu = weights(wtype, (size_t)f * d), *Wd = weights(wtype, (size_t)d * f);
            void *Wg = gated ? weights(wtype, (size_t)f * d) : NULL;
            float *c1 = vec(H), *c2 = vec(f), *b1 = vec(f), *b2 = vec(d), *x = vec((size_t)B * d);
            float *r = vec((size_t)B * d);
            double *h = malloc(sizeof(double) * B * H), *s = malloc(sizeof(double) * B * f);
            uint8_t *act = malloc((size_t)B * f), *u = malloc(f);
            int64_t *cnt = calloc(f, sizeof(int64_t));
            int32_t *perm = malloc(sizeof(int32_t) * f), *ids = malloc(sizeof(int32_t) * f);
            double *y = malloc(sizeof(double) * B * d), *yd = malloc(sizeof(double) * B * d);
            double *pre = malloc(sizeof(double) * B * f);
            uint8_t *tm = malloc((size_t)B * f);
            if (orc_predict(d, f, H, wtype, P1, c1, P2, c2, 0.0, x, B, h, s, act) != 0)
                return fail("predict");
            orc_union(B, f, act, u);
            orc_count_activations(B, f, act, cnt);
            if (orc_hot_first_table(f, cnt, perm) != 0)
                return fail("hot_first_table");
            int n = orc_active_list(f, perm, u, ids);
            double *a = malloc(sizeof(double) * B * (n > 0 ? n : 1));
            if (orc_ffn(d, f, wtype, gated, Wu, Wg, b1, Wd, b2, r, x, B, ids, n, act, a, y) != 0)
                return fail("ffn");
            if (orc_ffn(d, f, wtype, gated, Wu, Wg, NULL, Wd, NULL, NULL, x, B, ids, n, NULL,
                        NULL, y) != 0)
                return fail("ffn without biases");
            if (n >= 2) {
                int32_t saved = ids[1];
                ids[1] = ids[0];
                if (orc_ffn(d, f, wtype, gated, Wu, Wg, b1, Wd, b2, NULL, x, B, ids, n, NULL,
                            NULL, y) != -3)
                    return fail("a repeated id is refused");
                ids[1] = f;
                if (orc_ffn(d, f, wtype, gated, Wu, Wg, b1, Wd, b2, NULL, x, B, ids, n, NULL,
                            NULL, y) != -3)
                    return fail("an id out of range is refused");
                ids[1] = saved;
            }
            if (orc_dense_ffn(d, f, wtype, gated, Wu, Wg, b1, Wd, b2, r, x, B, yd) != 0)
                return fail("dense_ffn");
            if (orc_true_mask(d, f, wtype, gated, Wu, Wg, b1, x, B, pre, tm) != 0)
                return fail("true_mask");
            for (int t = 0; t < B; ++t) {
                /* the FFN over the token's true set is the dense FFN */
                int m = orc_active_list(f, NULL, tm + (size_t)t * f, ids);
                if (orc_ffn(d, f, wtype, gated, Wu, Wg, b1, Wd, b2, r + (size_t)t * d,
                            x + (size_t)t * d, 1, ids, m, NULL, NULL, y) != 0)
                    return fail("ffn over the true set");
                if (memcmp(y, yd + (size_t)t * d, sizeof(double) * d) != 0)
                    return fail("true set equals dense");
            }
            free(a);
            free(P1); free(P2); free(Wu); free(Wd); free(Wg);
            free(c1); free(c2); free(b1); free(b2); free(x); free(r);
            free(h); free(s); free(act); free(u); free(cnt); free(perm); free(ids);
            free(y); free(yd); free(pre); free(tm);
        }
    }
    printf("ok\n");
    return 0;
}
