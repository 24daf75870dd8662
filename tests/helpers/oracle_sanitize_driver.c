/*
 * Host-only driver for a sanitizer build of the CPU oracle (test infrastructure): the
 * oracle's C source is compiled into this program with AddressSanitizer and
 * UndefinedBehaviorSanitizer, and every entry point runs on small seeded inputs that
 * include the edge cases (masked, NaN and empty rows; K = 0; one particle; degenerate
 * weights; an exhausted block pool; shared and unshared prefixes).  Exit status 0 and a
 * final "ok" line mean no sanitizer report.
 */
#include "../../oracle/smcsd_oracle.c"

#include <stdio.h>

static uint64_t lcg_state = 88172645463325252ull;
static double rnd(void)
{
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(lcg_state >> 11) * (1.0 / 9007199254740992.0);
}
static float nrm(void) { return (float)(2.0 * rnd() - 1.0) * 2.5f; }
static uint16_t to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

static void fill(float *f32, uint16_t *b16, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        f32[i] = nrm();
        b16[i] = to_bf16(f32[i]);
    }
}

static void run_verify(int nseq, int K, int64_t V, int masked)
{
    const int R = 2 * K + 1;
    int64_t nt = (int64_t)nseq * (K + 1) * V, nd = (int64_t)nseq * (K > 0 ? K : 1) * V;
    float *tf = malloc(sizeof(float) * nt), *df = malloc(sizeof(float) * nd);
    uint16_t *tb = malloc(2 * nt), *db = malloc(2 * nd);
    fill(tf, tb, nt);
    fill(df, db, nd);
    if (masked) {
        for (int64_t v = 0; v < V; ++v) tf[v] = -INFINITY;        /* sequence 0 row 0: empty */
        tf[(int64_t)(K > 0 ? 1 : 0) * V] = NAN;                     /* a NaN logit             */
        for (int64_t i = 0; i < nt; i += 3) tb[i] = 0xFF80;         /* -inf in bf16            */
    }
    int32_t *tok = malloc(sizeof(int32_t) * nseq * (K > 0 ? K : 1));
    for (int i = 0; i < nseq * K; ++i) tok[i] = (int32_t)(rnd() * (double)V);
    if (masked && K > 1) {                                           /* out-of-vocabulary tokens */
        tok[0] = (int32_t)V + 5;
        tok[1] = -1;
    }
    int64_t *idx = malloc(sizeof(int64_t) * nseq);
    for (int s = 0; s < nseq; ++s) idx[s] = 5 * s + 1;
    double *lw = calloc(nseq, sizeof(double)), *lwo = malloc(sizeof(double) * nseq);
    double *lq_in = malloc(sizeof(double) * nseq * (K > 0 ? K : 1));
    for (int i = 0; i < nseq * K; ++i) lq_in[i] = -3.0 * rnd();
    int32_t *otok = malloc(sizeof(int32_t) * nseq * (K + 1)), *num = malloc(sizeof(int32_t) * nseq);
    double *lp = malloc(sizeof(double) * nseq * (K + 1)), *lq = malloc(sizeof(double) * nseq * (K > 0 ? K : 1));
    double *lse = malloc(sizeof(double) * nseq * R), *u = malloc(sizeof(double) * nseq);
    double *mg = malloc(sizeof(double) * nseq), *mg2 = malloc(sizeof(double) * nseq);
    int32_t st = 0;
    for (int dt = 0; dt < 2; ++dt) {
        const void *t = dt ? (const void *)tb : (const void *)tf;
        const void *d = dt ? (const void *)db : (const void *)df;
        for (int rule = 0; rule < 2; ++rule) {
            orc_verify_smc(t, d, dt, V, nseq, idx, K, tok, 0.8, 1.0, 7, 3, lw, NULL, rule, lwo, otok, lp,
                           lq, lse, u, mg, &st);
            orc_verify_smc(t, d, dt, V, nseq, idx, K, tok, 1.0, 4.0, 7, 3, lw, lq_in, rule, lwo, otok,
                           lp, lq, lse, u, mg, &st);
        }
        orc_verify_sps(t, d, dt, V, nseq, idx, K, tok, 1.3, 9, 4, otok, num, lp, lq, lse, mg, mg2, &st);
        orc_draft_sample(t, dt, V, nseq, idx, 2, 0.9, 11, 5, otok, lp, mg, &st);
        orc_race_sample(t, dt, V, nseq, idx, 1.1, 13, 6, otok, mg);
    }
    /* SpS with identical rows and every draft token masked in both: empty residuals */
    for (int i = 0; i < nseq * K; ++i)
        if (tok[i] < 0 || tok[i] >= V) tok[i] = 0;
    for (int s = 0; s < nseq; ++s)
        for (int k = 0; k < K; ++k) {
            float *tr = tf + ((int64_t)s * (K + 1) + k) * V, *dr = df + ((int64_t)s * K + k) * V;
            memcpy(dr, tr, sizeof(float) * V);
            tr[tok[s * K + k]] = -INFINITY;
            dr[tok[s * K + k]] = -INFINITY;
        }
    orc_verify_sps(tf, df, 0, V, nseq, idx, K, tok, 1.0, 9, 4, otok, num, lp, lq, lse, mg, mg2, &st);
    free(tf); free(df); free(tb); free(db); free(tok); free(idx); free(lw); free(lwo); free(lq_in);
    free(otok); free(num); free(lp); free(lq); free(lse); free(u); free(mg); free(mg2);
}

static void run_resample(int B, int N)
{
    float *lw = malloc(sizeof(float) * B * N);
    for (int i = 0; i < B * N; ++i) lw[i] = nrm() * 3.0f;
    if (B > 1) lw[N] = NAN;                           /* prompt 1: degenerate */
    if (B > 2)
        for (int n = 0; n < N; ++n) lw[2 * N + n] = -INFINITY;
    double *lwo = malloc(sizeof(double) * B * N), *ess = malloc(sizeof(double) * B);
    double *me = malloc(sizeof(double) * B), *mp = malloc(sizeof(double) * B * N);
    int32_t *anc = malloc(sizeof(int32_t) * B * N), *res = malloc(sizeof(int32_t) * B), st = 0;
    orc_resample(lw, B, N, 0.5, 3, 1, lwo, anc, ess, res, me, mp, &st);
    orc_resample(lw, B, N, 2.0, 3, 2, lwo, anc, ess, res, me, mp, &st);
    free(lw); free(lwo); free(ess); free(me); free(mp); free(anc); free(res);
}

static void run_kv(int B, int N, int bs, int ctx0, int R, int rounds, int shared, int P_short)
{
    const int S = B * N;
    const int M = (ctx0 + (rounds + 2) * R + bs - 1) / bs;
    const int P = P_short ? S * ((ctx0 + bs - 1) / bs) / (shared ? N : 1) + 3 : S * M;
    int32_t *T = malloc(sizeof(int32_t) * S * M), *rc = calloc(P, sizeof(int32_t));
    int32_t *fl = malloc(sizeof(int32_t) * P), top = P, *cow = malloc(sizeof(int32_t) * S * 3), ncow = 0;
    int32_t *anc = malloc(sizeof(int32_t) * S), *res = malloc(sizeof(int32_t) * B), st = 0;
    for (int i = 0; i < S * M; ++i) T[i] = -1;
    for (int i = 0; i < P; ++i) fl[i] = P - 1 - i;
    const int nb0 = (ctx0 + bs - 1) / bs;
    for (int b = 0; b < B; ++b)
        for (int n = 0; n < N; ++n)
            for (int s = 0; s < nb0; ++s) {
                int32_t blk;
                if (shared && n > 0) {
                    blk = T[(b * N) * M + s];
                } else {
                    blk = fl[--top];
                }
                T[(b * N + n) * M + s] = blk;
                rc[blk] += 1;
            }
    int64_t L = ctx0;
    for (int i = 0; i < S; ++i) anc[i] = i % N;
    for (int b = 0; b < B; ++b) res[b] = 0;
    orc_kv_reassign(anc, res, B, N, T, M, bs, L, R, rc, fl, &top, P, cow, &ncow, &st);
    for (int r = 0; r < rounds; ++r) {
        L += R;
        for (int b = 0; b < B; ++b) {
            res[b] = rnd() < 0.7;
            int a = 0;
            for (int n = 0; n < N; ++n) {          /* non-decreasing, as systematic resampling gives */
                while (a < N - 1 && rnd() < 0.4) ++a;
                anc[b * N + n] = a;
            }
        }
        orc_kv_reassign(anc, res, B, N, T, M, bs, L, R, rc, fl, &top, P, cow, &ncow, &st);
    }
    if (L + 2 * R <= (int64_t)M * bs) {
        /* an ancestor outside [0, N) and a corrupt free-stack entry at the top */
        L += R;
        for (int b = 0; b < B; ++b) res[b] = 1;
        anc[N - 1] = N + 3;
        if (top > 0) fl[top - 1] = P + 100;
        orc_kv_reassign(anc, res, B, N, T, M, bs, L, R, rc, fl, &top, P, cow, &ncow, &st);
    }
    free(T); free(rc); free(fl); free(cow); free(anc); free(res);
}

int main(void)
{
    uint32_t c[4] = {1, 2, 3, 4}, k[2] = {5, 6}, o[4];
    orc_philox4x32_10(c, k, o);
    volatile double acc = orc_uniform(1, 2, 3, 4, 3) + orc_race_clock(1, 2, 3, 12345);
    (void)acc;
    run_verify(3, 0, 5, 0);
    run_verify(4, 1, 1, 0);
    run_verify(5, 3, 37, 1);
    run_verify(2, 4, 2000, 0);
    run_resample(1, 1);
    run_resample(3, 5);
    run_resample(4, 64);
    run_kv(2, 4, 4, 10, 3, 6, 0, 0);
    run_kv(3, 5, 4, 13, 3, 6, 1, 0);
    run_kv(2, 16, 16, 40, 5, 8, 1, 0);
    run_kv(2, 4, 4, 10, 3, 6, 0, 1);               /* the pool runs out: NOSPACE */
    printf("ok\n");
    return 0;
}
