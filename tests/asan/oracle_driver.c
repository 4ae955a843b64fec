/*
 * oracle_driver.c -- drives every function of the CPU oracle through small
 * inputs and its edge cases (empty rows, all -inf rows, NULL selections,
 * masks, lengths of zero, grouped heads), built with AddressSanitizer and
 * UndefinedBehaviorSanitizer.  A few invariants are checked on the way
 * (softmax rows sum to 1, one visible key gives its value row); the
 * oracle's real pins live in the Python test suite.  Exit status 0 when
 * every expectation holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_softmax_rows(const float *x, int64_t ld, int64_t cols, const int64_t *sel, int64_t nsel,
                        double *y, double *row_max, double *row_sum);
int oracle_online_normalizer(const double *s, int64_t n, double *m_steps, double *l_steps);
int oracle_summary(const double *s, const double *v, int64_t n, int64_t d, double *m_out, double *l_out,
                   double *o_tilde);
int oracle_merge(const float *part_m, const float *part_l, const float *part_o, int64_t rows, int64_t splits,
                 int64_t d, double *o, double *lse);
int oracle_attention(const float *q, const float *k, const float *v, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nk, int64_t d, const int32_t *seqlens_q, const int32_t *seqlens_k,
                     double scale, int causal, const int64_t *sel, int64_t nsel, double *o, double *lse);
int oracle_merge_lse(const double *o_a, const double *lse_a, const double *o_b, const double *lse_b,
                     int64_t rows, int64_t d, double *o, double *lse);
int oracle_attention_bwd(const float *q, const float *k, const float *v, const float *dout, int64_t B,
                         int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, const int32_t *seqlens_q,
                         const int32_t *seqlens_k, double scale, int causal, double *dq, double *dk,
                         double *dv);

static int failures = 0;
#define EXPECT(cond)                                                                       \
    do {                                                                                   \
        if (!(cond)) {                                                                     \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                                    \
        }                                                                                  \
    } while (0)

static uint64_t state = 88172645463325252ull;
static float frand(void) {   /* xorshift64, uniform in [-2, 2) */
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (float)((double)(state >> 11) / 9007199254740992.0 * 4.0 - 2.0);
}

int main(void) {
    /* softmax: ragged rows, an all -inf row, a row with one finite entry */
    enum { R = 4, C = 7, LD = 9 };
    float x[R * LD];
    for (int i = 0; i < R * LD; ++i) x[i] = frand();
    for (int c = 0; c < C; ++c) x[1 * LD + c] = -INFINITY;
    for (int c = 1; c < C; ++c) x[2 * LD + c] = -INFINITY;
    double y[R * C], mx[R], sm[R];
    EXPECT(oracle_softmax_rows(x, LD, C, NULL, R, y, mx, sm) == 0);
    for (int r = 0; r < R; ++r) {
        double s = 0;
        for (int c = 0; c < C; ++c) s += y[r * C + c];
        EXPECT(r == 1 ? (s == 0.0 && isinf(mx[r]) && sm[r] == 0.0) : fabs(s - 1.0) < 1e-14);
    }
    int64_t sel[2] = {3, 0};
    EXPECT(oracle_softmax_rows(x, LD, C, sel, 2, y, NULL, NULL) == 0);
    EXPECT(oracle_softmax_rows(x, LD, 0, NULL, R, y, mx, sm) == 0);
    EXPECT(oracle_softmax_rows(x, 3, C, NULL, R, y, mx, sm) != 0);      /* ld < cols */

    /* the recurrence and the summary, including an empty set */
    double s[6] = {2, 5, 1, 7, -INFINITY, 3}, ms[6], ls[6];
    EXPECT(oracle_online_normalizer(s, 6, ms, ls) == 0);
    EXPECT(ms[3] == 7.0 && ls[0] == 1.0);
    EXPECT(oracle_online_normalizer(NULL, 0, NULL, NULL) == 0);
    double v[6 * 3], m1, l1, o1[3];
    for (int i = 0; i < 18; ++i) v[i] = frand();
    EXPECT(oracle_summary(s, v, 6, 3, &m1, &l1, o1) == 0);
    EXPECT(oracle_summary(s, v, 0, 3, &m1, &l1, o1) == 0 && isinf(m1) && l1 == 0.0);

    /* merge of piece summaries, with an all-empty row */
    enum { MR = 3, MS = 4, MD = 5 };
    float pm[MR * MS], pl[MR * MS], po[MR * MS * MD];
    for (int i = 0; i < MR * MS; ++i) {
        pm[i] = frand();
        pl[i] = 1.0f + 0.25f * frand();
    }
    for (int i = 0; i < MR * MS * MD; ++i) po[i] = frand();
    for (int c = 0; c < MS; ++c) pm[0 * MS + c] = -INFINITY;
    pm[1 * MS + 2] = -INFINITY;
    double om[MR * MD], lm[MR];
    EXPECT(oracle_merge(pm, pl, po, MR, MS, MD, om, lm) == 0);
    EXPECT(isinf(lm[0]) && om[0] == 0.0 && isfinite(lm[1]));

    /* attention: grouped heads, causal, lengths (one of them 0), selections */
    enum { B = 2, HQ = 4, HKV = 2, NQ = 5, NK = 6, D = 3 };
    float q[B * HQ * NQ * D], k[B * HKV * NK * D], vv[B * HKV * NK * D], dout[B * HQ * NQ * D];
    for (int i = 0; i < B * HQ * NQ * D; ++i) {
        q[i] = frand();
        dout[i] = frand();
    }
    for (int i = 0; i < B * HKV * NK * D; ++i) {
        k[i] = frand();
        vv[i] = frand();
    }
    int32_t lq[B] = {5, 0}, lk[B] = {1, 6};
    double o[B * HQ * NQ * D], lse[B * HQ * NQ];
    EXPECT(oracle_attention(q, k, vv, B, HQ, HKV, NQ, NK, D, lq, lk, 0.5, 1, NULL, B * HQ * NQ, o, lse) == 0);
    /* batch 0 sees key 0 only: every live row of head h is v[kv head][0] */
    for (int h = 0; h < HQ; ++h)
        for (int i = 0; i < NQ; ++i)
            for (int c = 0; c < D; ++c)
                EXPECT(o[((0 * HQ + h) * NQ + i) * D + c] == (double)vv[((0 * HKV + h / 2) * NK + 0) * D + c]);
    for (int t = HQ * NQ; t < 2 * HQ * NQ; ++t) EXPECT(isinf(lse[t]));          /* batch 1: Lq = 0 */
    int64_t asel[3] = {7, 0, 39};
    EXPECT(oracle_attention(q, k, vv, B, HQ, HKV, NQ, NK, D, NULL, NULL, 0.5, 0, asel, 3, o, lse) == 0);
    EXPECT(oracle_attention(q, k, vv, B, 3, HKV, NQ, NK, D, NULL, NULL, 0.5, 0, NULL, 1, o, lse) != 0);

    /* log-sum-exp merge with an empty piece */
    double oa[2 * 3] = {1, 2, 3, 4, 5, 6}, la[2] = {0.5, -INFINITY};
    double ob[2 * 3] = {6, 5, 4, 3, 2, 1}, lb[2] = {-INFINITY, -INFINITY};
    double oo[2 * 3], lo[2];
    EXPECT(oracle_merge_lse(oa, la, ob, lb, 2, 3, oo, lo) == 0);
    EXPECT(lo[0] == 0.5 && oo[0] == 1.0 && isinf(lo[1]) && oo[3] == 0.0);

    /* backward: causal with lengths, grouped heads */
    double dq[B * HQ * NQ * D], dk[B * HKV * NK * D], dv[B * HKV * NK * D];
    int32_t lq2[B] = {5, 3}, lk2[B] = {6, 2};
    EXPECT(oracle_attention_bwd(q, k, vv, dout, B, HQ, HKV, NQ, NK, D, lq2, lk2, 0.5, 1, dq, dk, dv) == 0);
    for (int c = 0; c < D; ++c) EXPECT(dk[((1 * HKV + 0) * NK + 5) * D + c] == 0.0);   /* key past Lk */
    EXPECT(oracle_attention_bwd(q, k, vv, dout, B, HQ, HKV, NQ, NK, D, NULL, NULL, 0.5, 0, dq, dk, dv) == 0);

    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("oracle driver: all expectations hold\n");
    return 0;
}
