/*
 * smcsd_oracle.c - plain, slow CPU oracle for the SMC-SD verify / resample / KV
 * pointer-exchange path.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The GPU product path never calls it, and
 * it shares no code, header, table or constant generator with the HIP sources.
 *
 * Arithmetic: every floating-point step is fp64, every sum runs in ascending index
 * order with a plain loop.  bf16 and fp32 inputs are widened exactly to fp64.
 *
 * Sources, cited by page title and section:
 *   [SMC]  "Faster LLM Inference via Sequential Monte Carlo" - the two gist.science
 *          explainers of the SMC-SD paper (Chinese page: section 2 methodology
 *          "core flow" and "system optimisation design", section 3 theory;
 *          Spanish page: "Resumen Tecnico" section 2 Metodologia, section 3).
 *   [SpS]  "Accelerating-Large-Language-Model-Decoding-with-Speculative-Sampling"
 *          (mengman.github.io notes): section 1 Introduction (the three-step SpS
 *          loop) and section 4.2 Modified Rejection Sampling.
 *   [Philox] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *          1, 2, 3", SC'11 - the Philox4x32 bijection with 10 rounds.
 *   [ERSD] "Speculative Sampling via Exponential Races" (paper summary page):
 *          key design, the exponential race - only the race as a sampling rule is
 *          used here (the one-pass bonus variant), not ERSD's verify.
 *
 * The pages leave several steps open (the weight formula beyond "target/draft
 * ratio", the ESS formula, the resampling scheme, the RNG, the block-table rules).
 * The readings taken are stated at each function and collected in the design notes.
 *
 * Parity unpinned: none - every function here is checked by the CPU test suite
 * against closed forms, library routines, brute-force enumeration or invariants.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* status bits (the values documented for the library's device status word) */
#define ORC_ST_NAN_INPUT 1
#define ORC_ST_EMPTY_ROW 2
#define ORC_ST_NOSPACE 4
#define ORC_ST_DEGENERATE_WEIGHTS 8
#define ORC_ST_BAD_INPUT 16 /* a token, ancestor or block id out of range: never read */

/* RNG stream tags (counter word 3) */
#define ORC_TAG_BONUS 1u
#define ORC_TAG_RESAMPLE 2u
#define ORC_TAG_SPS_ACCEPT 3u
#define ORC_TAG_SPS_FINAL 4u
#define ORC_TAG_DRAFT 5u
#define ORC_TAG_RACE 6u

/* bonus-token rules of the SMC verify */
#define ORC_BONUS_CDF 0
#define ORC_BONUS_RACE 1

int orc_version(void) { return 1; }

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* [Philox] Philox4x32-10.  One round multiplies counter words 0 and 2 by the   */
/* two round multipliers (full 64-bit products), then forms the new counter from */
/* the high halves xor'ed with the other two words and the key, and the low      */
/* halves.  The key is advanced by the two Weyl increments between rounds.       */
/* ------------------------------------------------------------------------- */
void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint32_t mult0 = 0xD2511F53u, mult1 = 0xCD9E8D57u;
    const uint32_t weyl0 = 0x9E3779B9u, weyl1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += weyl0;
            k1 += weyl1;
        }
        uint64_t prod0 = (uint64_t)mult0 * (uint64_t)c0;
        uint64_t prod1 = (uint64_t)mult1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
        uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Counter convention (a reading; the pages name no RNG): key = (seed low word,
 * seed high word), counter = (stream index, round t low word, round t high word,
 * tag).  A uniform is the top 24 bits of one output word times 2^-24, which is exact
 * in fp32 and fp64 and lies in [0, 1). */
double orc_uniform(uint64_t seed, uint32_t index, uint64_t t, uint32_t tag, int word)
{
    uint32_t ctr[4] = {index, (uint32_t)t, (uint32_t)(t >> 32), tag};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return (double)(out[word & 3] >> 8) * (1.0 / 16777216.0);
}

/* ------------------------------------------------------------------------- */
/* element access: dtype 0 = fp32, 1 = bf16 (upper half of an fp32)            */
/* ------------------------------------------------------------------------- */
static double load_elem(const void *row, int dtype, int64_t v)
{
    if (dtype == 0) {
        return (double)((const float *)row)[v];
    } else {
        uint32_t bits = (uint32_t)((const uint16_t *)row)[v] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
}

static const void *row_ptr(const void *base, int dtype, int64_t row, int64_t V)
{
    size_t esz = dtype == 0 ? 4 : 2;
    return (const char *)base + (size_t)row * (size_t)V * esz;
}

/* ------------------------------------------------------------------------- */
/* [SMC] Score step.  The target scores every drafted position; the log-       */
/* probability of a token is its tempered logit minus the row's log-normaliser:  */
/*   z_v = l_v / T,  LSE = max_v z_v + ln sum_v exp(z_v - max_v z_v).            */
/* A NaN or +inf logit sets NAN_INPUT; a row with no finite logit sets            */
/* EMPTY_ROW (-inf marks a masked token with probability 0).                     */
/* ------------------------------------------------------------------------- */
double orc_row_lse(const void *row, int dtype, int64_t V, double T, int32_t *status)
{
    double zmax = -INFINITY;
    int bad = 0;
    for (int64_t v = 0; v < V; ++v) {
        double z = load_elem(row, dtype, v) / T;
        if (isnan(z) || z == INFINITY) bad = 1;
        else if (z > zmax) zmax = z;
    }
    if (bad) {
        *status |= ORC_ST_NAN_INPUT;
        return NAN;
    }
    if (zmax == -INFINITY) {
        *status |= ORC_ST_EMPTY_ROW;
        return -INFINITY;
    }
    double s = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        double z = load_elem(row, dtype, v) / T;
        s += exp(z - zmax);
    }
    return zmax + log(s);
}

/* Inverse CDF over a probability row p_v = exp(z_v - lse), ascending vocabulary
 * order: the first v with F_v = sum_{w<=v} p_w > u (strict).  If rounding leaves
 * F_{V-1} <= u the last token with p_v > 0 is returned.  *margin receives the
 * distance from u to the nearest CDF value bracketing the decision. */
static int32_t inverse_cdf_row(const void *row, int dtype, int64_t V, double T, double lse,
                               double u, double *margin)
{
    double F = 0.0;
    int32_t last_pos = -1;
    for (int64_t v = 0; v < V; ++v) {
        double p = exp(load_elem(row, dtype, v) / T - lse);
        double Fprev = F;
        F += p;
        if (p > 0.0) last_pos = (int32_t)v;
        if (F > u) {
            double a = u - Fprev, b = F - u;
            *margin = a < b ? a : b;
            return (int32_t)v;
        }
    }
    *margin = 0.0;
    return last_pos;
}

/* ------------------------------------------------------------------------- */
/* [ERSD] key design: an exponential race.  Every token v starts an independent */
/* exponential clock of rate p_v; the first to finish, argmin_v E_v / p_v with    */
/* E_v ~ Exp(1), is a draw from p (the minimum of independent exponentials is     */
/* attained at v with probability p_v / sum_w p_w).  With p_v proportional to    */
/* exp(z_v) the rule reads argmax_v (z_v - ln E_v): no normaliser is needed, so   */
/* one pass over the row decides it.                                              */
/* The clock of token v (a reading; the pages fix no generator): word v mod 4 of  */
/* the Philox block with counter (index, t low, t high, RACE | (v div 4) << 8);   */
/* u_v = (floor(w / 2^9) + 1/2) * 2^-23, strictly inside (0, 1) and exact in fp32; */
/* E_v = -ln u_v.                                                                 */
/* ------------------------------------------------------------------------- */
double orc_race_clock(uint64_t seed, uint32_t index, uint64_t t, int64_t v)
{
    uint32_t ctr[4] = {index, (uint32_t)t, (uint32_t)(t >> 32),
                       ORC_TAG_RACE | ((uint32_t)(v >> 2) << 8)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    double u = ((double)(out[v & 3] >> 9) + 0.5) / 8388608.0;
    return -log(u);
}

/* The race over one row: the token with the largest z_v - ln E_v among the finite
 * z_v (a -inf logit never finishes; NaN is reported by the row's LSE).  Equal keys
 * go to the smaller id.  *margin receives the gap between the two largest keys
 * (+inf with a single finite logit); -1 if no logit is finite. */
static int32_t race_row(const void *row, int dtype, int64_t V, double T, uint64_t seed,
                        uint32_t index, uint64_t t, double *margin)
{
    double best = -INFINITY, second = -INFINITY;
    int32_t arg = -1;
    for (int64_t v = 0; v < V; ++v) {
        double z = load_elem(row, dtype, v) / T;
        if (!(z > -INFINITY) || isnan(z)) continue;
        double key = z - log(orc_race_clock(seed, index, t, v));
        if (key > best) {
            second = best;
            best = key;
            arg = (int32_t)v;
        } else if (key > second) {
            second = key;
        }
    }
    *margin = arg < 0 ? 0.0 : best - second;
    return arg;
}

/* The race for nrows rows (rows [nrows, V]); rng_index[r] is row r's stream. */
int orc_race_sample(const void *rows, int dtype, int64_t V, int nrows, const int64_t *rng_index,
                    double T, uint64_t seed, uint64_t t, int32_t *tokens, double *margin)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r)
        tokens[r] = race_row(row_ptr(rows, dtype, r, V), dtype, V, T, seed,
                             (uint32_t)rng_index[r], t, &margin[r]);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* [SMC] One verify round for nseq sequences (SMC mode).                       */
/*   Score:    LSE of the K+1 target rows and the K draft rows (tempered).       */
/*   Gather:   logp_k = z^t_k[x_k] - LSE^t_k,  logq_k = z^d_k[x_k] - LSE^d_k.    */
/*   Bonus:    one extra token per sequence from the target row K by inverse    */
/*             CDF with u = U(seed; g, t, BONUS) (bonus_rule CDF), or by the      */
/*             exponential race above (bonus_rule RACE); logp_K = its log-prob.   */
/*   Reweight: lw += sum_{k<K} (alpha*logp_k - logq_k) + (alpha-1)*logp_K.       */
/*             alpha = 1 gives the plain target/draft ratio; the bonus is drawn  */
/*             from the target, so it contributes (alpha-1)*logp_K (power mode). */
/*   Output:   tokens = (x_0 .. x_{K-1}, bonus) - always K+1 tokens per round.   */
/* Layout: tgt [nseq, K+1, V], drf [nseq, K, V], draft_tokens [nseq, K];         */
/* rng_index[s] is the global sequence index g used as the RNG stream index.    */
/* lse is [nseq, 2K+1]: target rows 0..K then draft rows 0..K-1.                 */
/* ------------------------------------------------------------------------- */
int orc_verify_smc(const void *tgt, const void *drf, int dtype, int64_t V, int nseq,
                   const int64_t *rng_index, int K, const int32_t *draft_tokens, double T,
                   double alpha, uint64_t seed, uint64_t t, const double *lw_in,
                   const double *logq_in, int bonus_rule, double *lw_out, int32_t *tokens,
                   double *logp,
                   double *logq, double *lse, double *bonus_u, double *margin, int32_t *status)
{
    const int R = 2 * K + 1;
    const int64_t nrows = (int64_t)nseq * R;
    int32_t st = 0;

    /* Score: every row's log-normaliser (rows are independent).  With logq_in (the
       draft's log-probabilities emitted when it sampled) the draft rows are not read. */
#pragma omp parallel for schedule(dynamic, 1) reduction(| : st)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t s = r / R;
        int k = (int)(r % R);
        if (k > K && logq_in) {
            lse[r] = NAN;
            continue;
        }
        const void *row = k <= K ? row_ptr(tgt, dtype, s * (K + 1) + k, V)
                                 : row_ptr(drf, dtype, s * K + (k - K - 1), V);
        int32_t rst = 0;
        lse[r] = orc_row_lse(row, dtype, V, T, &rst);
        st |= rst;
    }

    int32_t bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int s = 0; s < nseq; ++s) {
        const double *L = lse + (int64_t)s * R;
        double incr = 0.0;
        for (int k = 0; k < K; ++k) {
            int32_t x = draft_tokens[(int64_t)s * K + k];
            const void *trow = row_ptr(tgt, dtype, (int64_t)s * (K + 1) + k, V);
            double lp = NAN, lq = NAN;
            if (x < 0 || x >= V) {
                /* a draft token outside the vocabulary is flagged, never read */
                bad |= ORC_ST_BAD_INPUT;
            } else {
                lp = load_elem(trow, dtype, x) / T - L[k];
                lq = logq_in ? logq_in[(int64_t)s * K + k]
                             : load_elem(row_ptr(drf, dtype, (int64_t)s * K + k, V), dtype, x) / T -
                                   L[K + 1 + k];
            }
            logp[(int64_t)s * (K + 1) + k] = lp;
            logq[(int64_t)s * K + k] = lq;
            tokens[(int64_t)s * (K + 1) + k] = x;
            incr += alpha * lp - lq;
        }
        /* Bonus token from the target's distribution at position K */
        double u = orc_uniform(seed, (uint32_t)rng_index[s], t, ORC_TAG_BONUS, 0);
        const void *brow = row_ptr(tgt, dtype, (int64_t)s * (K + 1) + K, V);
        double m = 0.0;
        int32_t bonus = -1;
        double lpK = NAN;
        if (isfinite(L[K])) {
            if (bonus_rule == ORC_BONUS_RACE)
                bonus = race_row(brow, dtype, V, T, seed, (uint32_t)rng_index[s], t, &m);
            else
                bonus = inverse_cdf_row(brow, dtype, V, T, L[K], u, &m);
            lpK = load_elem(brow, dtype, bonus) / T - L[K];
        }
        tokens[(int64_t)s * (K + 1) + K] = bonus;
        logp[(int64_t)s * (K + 1) + K] = lpK;
        incr += (alpha - 1.0) * lpK;
        lw_out[s] = lw_in[s] + incr;
        bonus_u[s] = u;
        margin[s] = m;
    }
    *status |= st | bad;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* [SpS] Modified rejection verify on the same tempered p and q.               */
/* For k = 0..K-1: r_k = U(seed; g, t, SPS_ACCEPT | (k/4)<<8, word k mod 4);    */
/* keep x_k iff r_k < p_k(x_k)/q_k(x_k).  At the first rejection k* the        */
/* replacement is drawn from the residual max(0, p_{k*} - q_{k*}) renormalised  */
/* (inverse CDF with u = U(seed; g, t, SPS_FINAL)); the output stops there      */
/* (k*+1 tokens).  If all K are kept, a bonus is drawn from p_K with the same u */
/* (K+1 tokens).  A residual of total mass 0 falls back to p_{k*}.               */
/* tokens [nseq, K+1] is padded with -1 after num_tokens.                        */
/* logp[s, K] is the target log-probability of the last emitted token at its     */
/* position.  margin_accept[s] = min |r_k - ratio_k| over the tests made;        */
/* margin_final[s] = distance of u to the nearest bracketing (normalised) CDF.    */
/* ------------------------------------------------------------------------- */
/* ------------------------------------------------------------------------- */
/* [SMC] Extend step, draft side: the draft model proposes each token from its  */
/* own tempered distribution (core flow, "Extend").  One row per sequence at one */
/* draft position pos: x = min{v : sum_{w<=v} softmax(z)_w > u} with z = l / T   */
/* and u = U(seed; g, t, DRAFT | pos << 8) (a reading: inverse CDF in ascending  */
/* id order, the same rule as the bonus token), and log q(x) = z_x - LSE(z), the */
/* value the verify's reweighting needs, so the verify can skip the draft rows.  */
/* margin[r] = distance from u to the nearest CDF boundary of the choice.       */
/* ------------------------------------------------------------------------- */
int orc_draft_sample(const void *rows, int dtype, int64_t V, int nrows, const int64_t *rng_index,
                     int pos, double T, uint64_t seed, uint64_t t, int32_t *tokens, double *logq,
                     double *margin, int32_t *status)
{
    int32_t st = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : st)
    for (int r = 0; r < nrows; ++r) {
        const void *row = row_ptr(rows, dtype, r, V);
        int32_t rst = 0;
        double L = orc_row_lse(row, dtype, V, T, &rst);
        st |= rst;
        double u = orc_uniform(seed, (uint32_t)rng_index[r], t,
                               ORC_TAG_DRAFT | ((uint32_t)pos << 8), 0);
        double m = 0.0;
        int32_t x = -1;
        if (isfinite(L)) x = inverse_cdf_row(row, dtype, V, T, L, u, &m);
        tokens[r] = x;
        logq[r] = x >= 0 ? load_elem(row, dtype, x) / T - L : NAN;
        margin[r] = m;
    }
    *status |= st;
    return 0;
}

int orc_verify_sps(const void *tgt, const void *drf, int dtype, int64_t V, int nseq,
                   const int64_t *rng_index, int K, const int32_t *draft_tokens, double T,
                   uint64_t seed, uint64_t t, int32_t *tokens, int32_t *num_tokens, double *logp,
                   double *logq, double *lse, double *margin_accept, double *margin_final,
                   int32_t *status)
{
    const int R = 2 * K + 1;
    const int64_t nrows = (int64_t)nseq * R;
    int32_t st = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : st)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t s = r / R;
        int k = (int)(r % R);
        const void *row = k <= K ? row_ptr(tgt, dtype, s * (K + 1) + k, V)
                                 : row_ptr(drf, dtype, s * K + (k - K - 1), V);
        int32_t rst = 0;
        lse[r] = orc_row_lse(row, dtype, V, T, &rst);
        st |= rst;
    }

    int32_t bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int s = 0; s < nseq; ++s) {
        const double *L = lse + (int64_t)s * R;
        const uint32_t g = (uint32_t)rng_index[s];
        double macc = INFINITY;
        int kstar = K;
        for (int k = 0; k < K; ++k) {
            int32_t x = draft_tokens[(int64_t)s * K + k];
            const void *trow = row_ptr(tgt, dtype, (int64_t)s * (K + 1) + k, V);
            const void *drow = row_ptr(drf, dtype, (int64_t)s * K + k, V);
            if (x < 0 || x >= V) {   /* flagged, never read; its ratio is NaN: rejected */
                bad |= ORC_ST_BAD_INPUT;
                logp[(int64_t)s * (K + 1) + k] = NAN;
                logq[(int64_t)s * K + k] = NAN;
                continue;
            }
            logp[(int64_t)s * (K + 1) + k] = load_elem(trow, dtype, x) / T - L[k];
            logq[(int64_t)s * K + k] = load_elem(drow, dtype, x) / T - L[K + 1 + k];
        }
        for (int k = 0; k < K; ++k) {
            double lp = logp[(int64_t)s * (K + 1) + k];
            double lq = logq[(int64_t)s * K + k];
            double ratio = exp(lp - lq);
            double r = orc_uniform(seed, g, t, ORC_TAG_SPS_ACCEPT | ((uint32_t)(k / 4) << 8), k % 4);
            double d = fabs(r - ratio);
            if (d < macc) macc = d;
            if (!(r < ratio)) {
                kstar = k;
                break;
            }
        }
        for (int k = 0; k <= K; ++k) tokens[(int64_t)s * (K + 1) + k] = -1;
        for (int k = 0; k < kstar; ++k)
            tokens[(int64_t)s * (K + 1) + k] = draft_tokens[(int64_t)s * K + k];

        double u = orc_uniform(seed, g, t, ORC_TAG_SPS_FINAL, 0);
        int32_t tok = -1;
        double mfin = 0.0;
        const void *prow = row_ptr(tgt, dtype, (int64_t)s * (K + 1) + kstar, V);
        if (kstar < K) {
            const void *qrow = row_ptr(drf, dtype, (int64_t)s * K + kstar, V);
            double Rm = 0.0;
            for (int64_t v = 0; v < V; ++v) {
                double p = exp(load_elem(prow, dtype, v) / T - L[kstar]);
                double q = exp(load_elem(qrow, dtype, v) / T - L[K + 1 + kstar]);
                double rho = p - q > 0.0 ? p - q : 0.0;
                Rm += rho;
            }
            if (Rm > 0.0) {
                double F = 0.0;
                int32_t last_pos = -1;
                for (int64_t v = 0; v < V; ++v) {
                    double p = exp(load_elem(prow, dtype, v) / T - L[kstar]);
                    double q = exp(load_elem(qrow, dtype, v) / T - L[K + 1 + kstar]);
                    double rho = p - q > 0.0 ? p - q : 0.0;
                    double Fprev = F;
                    F += rho;
                    if (rho > 0.0) last_pos = (int32_t)v;
                    if (F > u * Rm) {
                        double a = u - Fprev / Rm, b = F / Rm - u;
                        mfin = a < b ? a : b;
                        tok = (int32_t)v;
                        break;
                    }
                }
                if (tok < 0) tok = last_pos;
            } else if (isfinite(L[kstar])) {
                tok = inverse_cdf_row(prow, dtype, V, T, L[kstar], u, &mfin);
            }
        } else if (isfinite(L[K])) {
            tok = inverse_cdf_row(prow, dtype, V, T, L[K], u, &mfin);
        }
        tokens[(int64_t)s * (K + 1) + kstar] = tok;
        num_tokens[s] = kstar + 1;
        logp[(int64_t)s * (K + 1) + K] =
            tok >= 0 ? load_elem(prow, dtype, tok) / T - L[kstar] : NAN;
        margin_accept[s] = macc;
        margin_final[s] = mfin;
    }
    *status |= st | bad;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* [SMC] Resample step, per prompt b.                                          */
/* ESS (a reading; the pages name it only): with m = max_n lw_n and            */
/* w_n = exp(lw_n - m), ESS = (sum w)^2 / sum w^2, clamped to [1, N].            */
/* Resample iff ESS < tau*N (strict; the pages say "below the threshold").     */
/* Scheme (a reading): systematic.  u0 = U(seed; b, t, RESAMPLE); with          */
/* C_j = (sum_{i<=j} w_i) / sum w, particle i takes the ancestor                */
/* a_i = min{ j : C_j > (i + u0)/N } (clamped to N-1), so high-weight particles  */
/* are duplicated and low-weight ones dropped; the log-weights then restart at  */
/* 0 (uniform).  Without resampling a_i = i and the weights carry over.         */
/* A prompt whose weights are all zero (max lw not finite) sets                  */
/* DEGENERATE_WEIGHTS and keeps identity ancestors, ess = 0.                     */
/* margin_ess[b] = |ESS - tau*N| / N; margin_pos[b, i] = distance from          */
/* (i+u0)/N to the nearest of C_{a_i - 1}, C_{a_i} (INFINITY if not resampled). */
/* ------------------------------------------------------------------------- */
int orc_resample(const float *lw_in, int B, int N, double tau, uint64_t seed, uint64_t t,
                 double *lw_out, int32_t *ancestors, double *ess, int32_t *resampled,
                 double *margin_ess, double *margin_pos, int32_t *status)
{
    double *w = (double *)malloc(sizeof(double) * (size_t)N);
    double *C = (double *)malloc(sizeof(double) * (size_t)N);
    if (!w || !C) {
        free(w);
        free(C);
        return -1;
    }
    for (int b = 0; b < B; ++b) {
        const float *lw = lw_in + (int64_t)b * N;
        double m = -INFINITY;
        int has_nan = 0;
        for (int n = 0; n < N; ++n) {
            double x = (double)lw[n];
            if (isnan(x)) has_nan = 1;
            else if (x > m) m = x;
        }
        for (int n = 0; n < N; ++n) {
            lw_out[(int64_t)b * N + n] = (double)lw[n];
            ancestors[(int64_t)b * N + n] = n;
            margin_pos[(int64_t)b * N + n] = INFINITY;
        }
        if (has_nan || !isfinite(m)) {
            *status |= ORC_ST_DEGENERATE_WEIGHTS;
            ess[b] = 0.0;
            resampled[b] = 0;
            margin_ess[b] = INFINITY;
            continue;
        }
        double s1 = 0.0, s2 = 0.0;
        for (int n = 0; n < N; ++n) {
            w[n] = exp((double)lw[n] - m);
            s1 += w[n];
            s2 += w[n] * w[n];
        }
        double e = s1 * s1 / s2;
        if (e < 1.0) e = 1.0;
        if (e > (double)N) e = (double)N;
        ess[b] = e;
        margin_ess[b] = fabs(e - tau * (double)N) / (double)N;
        int do_res = e < tau * (double)N;
        resampled[b] = do_res;
        if (!do_res) continue;

        double u0 = orc_uniform(seed, (uint32_t)b, t, ORC_TAG_RESAMPLE, 0);
        double acc = 0.0;
        for (int j = 0; j < N; ++j) {
            acc += w[j];
            C[j] = acc / s1;
        }
        for (int i = 0; i < N; ++i) {
            double pos = ((double)i + u0) / (double)N;
            int a = N - 1;
            for (int j = 0; j < N; ++j) {
                if (C[j] > pos) {
                    a = j;
                    break;
                }
            }
            ancestors[(int64_t)b * N + i] = a;
            double lo = a > 0 ? pos - C[a - 1] : INFINITY;
            double hi = C[a] - pos;
            double mg = fabs(lo) < fabs(hi) ? fabs(lo) : fabs(hi);
            margin_pos[(int64_t)b * N + i] = mg;
        }
        for (int n = 0; n < N; ++n) lw_out[(int64_t)b * N + n] = 0.0;
    }
    free(w);
    free(C);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* [SMC] KV cache at resampling: pointer exchange with reference counts and     */
/* prefixes shared across particles, with no KV data copied (system            */
/* optimisation design / Gestion de Cache).  The rules below are readings; the  */
/* pages give only the principle.                                                */
/*                                                                               */
/* State: tables [B*N, M_cap] block ids (-1 = unallocated); every sequence has   */
/* positions [0, L) allocated in slots [0, ceil(L/bs)).  rc [P] counts table     */
/* references; the free stack is free_list[0 .. top) with its top at top-1.      */
/*                                                                               */
/* Phase 1, prompts with resampled[b] = 1:                                       */
/*   c_j = #{i : a_i = j};  rc[T_j[s]] += c_j - 1 for every allocated slot s of  */
/*   the old table j (all increments before any decrement, so a block that      */
/*   stays referenced never reaches 0); blocks whose count reaches 0 are freed; */
/*   then T'_i = T_{a_i} (slot values only - no KV data moves).                 */
/* Freed blocks of the whole call are pushed in descending id order, so the next */
/* pops return ascending ids.                                                    */
/* Phase 2, all prompts: reserve positions [L, L+R).  With the tables after     */
/* phase 1, a sequence whose partial tail block (slot floor(L/bs), when L mod bs */
/* != 0) is also held by a higher-index sequence of the same prompt (so the     */
/* block is shared: the highest holder keeps it) does copy-on-write: pop d,     */
/* rc[old] -= 1, rc[d] = 1, T'[g][slot] = d, and emit                           */
/* (old, d, L mod bs) - the caller copies those L mod bs token entries.  Then    */
/* every slot in [ceil(L/bs), ceil((L+R)/bs)) pops a fresh block with rc = 1.     */
/* Pops run in ascending (sequence, slot) order.  An empty stack sets NOSPACE    */
/* and leaves that slot as it was (-1, or the shared block for a COW).           */
/* ------------------------------------------------------------------------- */
static int cmp_desc_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x < y) - (x > y);
}

int orc_kv_reassign(const int32_t *ancestors, const int32_t *resampled, int B, int N,
                    int32_t *tables, int M_cap, int bs, int64_t L, int R, int32_t *rc,
                    int32_t *free_list, int32_t *free_top, int P, int32_t *cow,
                    int32_t *cow_count, int32_t *status)
{
    const int S = B * N;
    const int nb_old = (int)((L + bs - 1) / bs);
    const int nb_new = (int)((L + R + bs - 1) / bs);
    if (nb_new > M_cap) return -1;
    int32_t *cnt = (int32_t *)calloc((size_t)N, sizeof(int32_t));
    int32_t *old = (int32_t *)malloc(sizeof(int32_t) * (size_t)N * (size_t)(nb_old > 0 ? nb_old : 1));
    int32_t *freed = (int32_t *)malloc(sizeof(int32_t) * ((size_t)S * (size_t)(nb_old > 0 ? nb_old : 1) + 1));
    int32_t *needs_cow = (int32_t *)calloc((size_t)S, sizeof(int32_t));
    if (!cnt || !old || !freed || !needs_cow) {
        free(cnt); free(old); free(freed); free(needs_cow);
        return -1;
    }
    int nfreed = 0;
    int32_t bad = 0;

    /* phase 1.  Indices are checked before use (the library's error convention: an
       ancestor outside [0, N) leaves its prompt unexchanged; a block id outside [0, P) in
       an exchanged table - a slot a NOSPACE call could not fill holds -1 - changes no
       count; both set BAD_INPUT) */
    for (int b = 0; b < B; ++b) {
        if (!resampled[b]) continue;
        const int32_t *a = ancestors + (int64_t)b * N;
        int32_t *T = tables + (int64_t)b * N * M_cap;
        int valid = 1;
        for (int i = 0; i < N; ++i)
            if (a[i] < 0 || a[i] >= N) valid = 0;
        if (!valid) {
            bad |= ORC_ST_BAD_INPUT;
            continue;
        }
        for (int j = 0; j < N; ++j)
            for (int s = 0; s < nb_old; ++s) {
                int32_t blk = T[(int64_t)j * M_cap + s];
                if (blk < 0 || blk >= P) bad |= ORC_ST_BAD_INPUT;
            }
        for (int j = 0; j < N; ++j) cnt[j] = 0;
        for (int i = 0; i < N; ++i) cnt[a[i]] += 1;
        for (int j = 0; j < N; ++j)
            if (cnt[j] > 1)
                for (int s = 0; s < nb_old; ++s) {
                    int32_t blk = T[(int64_t)j * M_cap + s];
                    if (blk >= 0 && blk < P) rc[blk] += cnt[j] - 1;
                }
        for (int j = 0; j < N; ++j)
            if (cnt[j] == 0)
                for (int s = 0; s < nb_old; ++s) {
                    int32_t blk = T[(int64_t)j * M_cap + s];
                    if (blk < 0 || blk >= P) continue;
                    rc[blk] -= 1;
                    if (rc[blk] == 0) freed[nfreed++] = blk;
                }
        for (int j = 0; j < N; ++j)
            for (int s = 0; s < nb_old; ++s) old[(int64_t)j * nb_old + s] = T[(int64_t)j * M_cap + s];
        for (int i = 0; i < N; ++i)
            for (int s = 0; s < nb_old; ++s)
                T[(int64_t)i * M_cap + s] = old[(int64_t)a[i] * nb_old + s];
    }
    qsort(freed, (size_t)nfreed, sizeof(int32_t), cmp_desc_i32);
    int top = *free_top;
    for (int f = 0; f < nfreed; ++f) free_list[top++] = freed[f];

    /* phase 2: copy-on-write decisions from the post-phase-1 state */
    const int tail_partial = (L % bs) != 0;
    const int ts = (int)(L / bs);
    if (tail_partial) {
        for (int g = 0; g < S; ++g) {
            int b = g / N;
            int32_t blk = tables[(int64_t)g * M_cap + ts];
            if (blk >= P) bad |= ORC_ST_BAD_INPUT;
            if (blk < 0 || blk >= P) continue;
            for (int h = g + 1; h < (b + 1) * N; ++h)
                if (tables[(int64_t)h * M_cap + ts] == blk) {
                    needs_cow[g] = 1;
                    break;
                }
        }
    }
    int ncow = 0;
    for (int g = 0; g < S; ++g) {
        int32_t *Tg = tables + (int64_t)g * M_cap;
        if (needs_cow[g]) {
            if (top > 0) {
                /* a popped id outside [0, P) (a corrupt free stack) is flagged: the copy
                   is listed with destination -1 and nothing else changes */
                int32_t d = free_list[--top];
                int32_t o = Tg[ts];
                int ok = d >= 0 && d < P;
                if (ok) {
                    rc[o] -= 1;
                    rc[d] = 1;
                    Tg[ts] = d;
                } else {
                    bad |= ORC_ST_BAD_INPUT;
                }
                cow[3 * ncow + 0] = o;
                cow[3 * ncow + 1] = ok ? d : -1;
                cow[3 * ncow + 2] = (int32_t)(L % bs);
                ncow++;
            } else {
                *status |= ORC_ST_NOSPACE;
            }
        }
        for (int s = nb_old; s < nb_new; ++s) {
            if (top > 0) {
                int32_t d = free_list[--top];
                if (d < 0 || d >= P) {      /* flagged; the slot keeps its value */
                    bad |= ORC_ST_BAD_INPUT;
                    continue;
                }
                rc[d] = 1;
                Tg[s] = d;
            } else {
                *status |= ORC_ST_NOSPACE;
            }
        }
    }
    *free_top = top;
    *cow_count = ncow;
    *status |= bad;
    free(cnt); free(old); free(freed); free(needs_cow);
    return 0;
}
