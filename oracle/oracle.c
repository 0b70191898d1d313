/*
 * oracle.c -- plain, slow, obviously correct CPU implementation of the
 * per-token sampling chain and of the raw-logit logprobs.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU-baseline leg call it; the product path never does.  It shares no code
 * with the HIP library.  Sources are listed in oracle.h.
 *
 * Every step follows the plain definition of what the pages describe, in
 * the pages' order: sanitise -> penalties -> top_k (full sort) -> min_p ->
 * top_p -> temperature -> Philox draw.  No blocking, no fusion, no early exit.
 * Floating point: the pages fix fp32 for the logits, for the penalties and
 * for the min_p threshold (they print it with logf); the cuts and the draw
 * after that are taken in fp64.  Build with -ffp-contract=off.
 *
 * Readings where the pages are silent (each one is pinned by a test):
 *   R1  NaN logits count as -inf, +inf as FLT_MAX, before and after penalties.
 *   R2  penalty of a token seen c > 0 times in the window:
 *         y = (x <= 0) ? x * repeat : x / repeat;  y = y - (c * freq + present)
 *       each op rounded to fp32.  The pages give the repeat rule and say the
 *       presence term is boolean; the frequency term scaling with c is the
 *       plainest reading of a frequency penalty.
 *   R3  the window is the last min(penalty_last_n, hlen) ids of the row's
 *       history (all of it for penalty_last_n < 0); ids outside [0, V) are
 *       ignored.
 *   R4  k_eff = min(top_k, V); greedy rows (temperature <= 0) keep k_eff = 1.
 *   R5  top_p: cumulative fp64 softmax of the min_p survivors, n = first j+1
 *       with cum_j >= top_p.  A head of -inf (all logits masked) keeps n = 1.
 *   R6  draw: counter words (lo, hi, 0, 0), key words (lo, hi) of the seed,
 *       u = x0 * 2^-32, token = first j with cdf_j > u (cdf_{n-1} = 1).
 *   R7  logprobs: an allowed list with no entries means no restriction; if
 *       every logit of the domain is -inf the domain is taken as uniform.
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------- Philox4x32-10 [SC11, section 3 "Philox"] ---------------- */

/* One Philox round: two 32x32->64 products, the high halves XORed with the
 * other two counter words and the round key, the low halves passed through. */
static void philox_round(uint32_t c[4], const uint32_t k[2])
{
    const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k[0];
    const uint32_t n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
}

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {               /* Weyl key schedule between rounds */
            k[0] += 0x9E3779B9u;
            k[1] += 0xBB67AE85u;
        }
        philox_round(c, k);
    }
    for (int i = 0; i < 4; ++i) out[i] = c[i];
}

/* ---------------- the sampling chain ---------------- */

static float sanitize(float v)     /* R1 */
{
    if (isnan(v)) return -INFINITY;
    if (v == INFINITY) return FLT_MAX;
    return v;
}

typedef struct { float y; int32_t i; } scored;

/* Total order of [P19] "The sampled chain is one block per token": larger
 * logit first, equal logits by lower index (a serial scan with strict >). */
static int by_logit_then_index(const void *pa, const void *pb)
{
    const scored *a = (const scored *)pa, *b = (const scored *)pb;
    if (a->y > b->y) return -1;
    if (a->y < b->y) return 1;
    return (a->i < b->i) ? -1 : (a->i > b->i);
}

int oracle_penalised_row(const float *x, int64_t V, const oracle_row_params *p,
                         const int32_t *hist, int64_t hlen, float *y)
{
    if (V <= 0) return -1;
    for (int64_t i = 0; i < V; ++i) y[i] = sanitize(x[i]);

    /* [P19] "min_p and the penalties": counts over the last penalty_last_n
     * tokens of the request; a request without a history row is neutral. */
    if (p->history_row < 0 || hist == NULL || hlen <= 0) return 0;
    int64_t n_eff = (p->penalty_last_n < 0) ? hlen
                  : (p->penalty_last_n < hlen ? p->penalty_last_n : hlen);   /* R3 */
    if (n_eff <= 0) return 0;
    const int32_t *w = hist + (hlen - n_eff);

    int32_t *count = (int32_t *)calloc((size_t)V, sizeof(int32_t));
    if (!count) return -1;
    for (int64_t j = 0; j < n_eff; ++j)
        if (w[j] >= 0 && w[j] < V) count[w[j]] += 1;

    for (int64_t i = 0; i < V; ++i) {
        const int32_t c = count[i];
        if (c <= 0) continue;
        float v = y[i];
        /* repeat: divide a positive logit, multiply a non-positive one */
        v = (v <= 0.0f) ? v * p->penalty_repeat : v / p->penalty_repeat;
        /* frequency scales with the count, presence is charged once (R2) */
        float t = (float)c * p->penalty_freq;
        t = t + p->penalty_present;
        v = v - t;
        y[i] = sanitize(v);
    }
    free(count);
    return 0;
}

/* Temperature and the inverse CDF at u over the first n kept logits y[0..n)
 * (R6): weights exp((y_i - y_0) / T) in fp64, cdf_j their normalised running
 * sum, the pick is the first j with cdf_j > u (cdf_{n-1} = 1).  Bit j of
 * *edges is set when |cdf_j - u| < 1e-6 for j < n - 1: there another correct
 * fp64 evaluation may pick j + 1 instead of j or the other way round. */
int oracle_draw_on_prefix(const float *y, int n, float temperature, double u, uint64_t *edges)
{
    *edges = 0;
    int pick = n - 1;
    if (n > 1) {
        const double y0 = (double)y[0];
        const double T = (double)temperature;
        double z = 0.0;
        for (int i = 0; i < n; ++i) z += exp(((double)y[i] - y0) / T);
        double run = 0.0;
        for (int j = 0; j < n - 1; ++j) {
            run += exp(((double)y[j] - y0) / T);
            const double cj = run / z;
            if (fabs(cj - u) < 1e-6) *edges |= 1ull << j;
            if (cj > u) { pick = j; break; }
        }
    }
    return pick;
}

/* The chain after the penalties, over a domain of nd candidates already in
 * the selection order (s sorted by logit desc, index asc). */
static void chain_on_sorted(const scored *s, int64_t nd, const oracle_row_params *p,
                            int32_t *token, int32_t counts[3],
                            int32_t kept_ids[64], float kept_logits[64],
                            uint32_t *x0, double *u, int32_t *flags)
{
    const int greedy = !(p->temperature > 0.0f);
    /* top_k: the first k_eff of the domain under the total order (R4) */
    const int64_t kk = greedy ? 1 : p->top_k;
    const int k_eff = (int)(kk < nd ? kk : nd);

    for (int i = 0; i < 64; ++i) { kept_ids[i] = -1; kept_logits[i] = -INFINITY; }
    for (int i = 0; i < k_eff; ++i) { kept_ids[i] = s[i].i; kept_logits[i] = s[i].y; }
    *flags = 0;
    *x0 = 0;
    *u = 0.0;

    if (!greedy) {
        /* the row's draw word (R6); taken even when the domain is empty */
        const uint32_t ctr[4] = {(uint32_t)p->counter, (uint32_t)(p->counter >> 32), 0u, 0u};
        const uint32_t key[2] = {(uint32_t)p->seed, (uint32_t)(p->seed >> 32)};
        uint32_t out[4];
        oracle_philox4x32_10(ctr, key, out);
        *x0 = out[0];
        *u = (double)out[0] * (1.0 / 4294967296.0);
    }
    if (nd == 0) {                                      /* R11: nothing to sample */
        *token = -1;
        counts[0] = counts[1] = counts[2] = 0;
        return;
    }
    if (greedy) {                                       /* argmax, no draw */
        *token = s[0].i;
        counts[0] = counts[1] = counts[2] = 1;
        return;
    }

    /* min_p [P19 "min_p and the penalties"]: keep the prefix whose logit is
     * at least head + logf(min_p), computed in fp32; the head always stays. */
    const float lnp = logf(p->min_p);                   /* min_p = 0 -> -inf */
    const float thr = s[0].y + lnp;
    int m = 0;
    while (m < k_eff && s[m].y >= thr) ++m;
    if (m < 1) m = 1;

    /* top_p over the min_p survivors, fp64 (R5). */
    int n = m;
    const double y0 = (double)s[0].y;
    if (s[0].y == -INFINITY) {
        n = 1;
    } else if (!((double)p->top_p >= 1.0)) {
        double z = 0.0;
        for (int i = 0; i < m; ++i) z += exp((double)s[i].y - y0);
        double run = 0.0;
        n = m;
        for (int j = 0; j < m; ++j) {
            run += exp((double)s[j].y - y0);
            const double cj = run / z;
            if (j < m - 1 && fabs(cj - (double)p->top_p) < 1e-6) *flags |= ORACLE_FLAG_TOP_P_EDGE;
            if (cj >= (double)p->top_p) { n = j + 1; break; }
        }
        if (n < 1) n = 1;
    }

    /* temperature, then the inverse CDF at u (R6). */
    float yk[64];
    for (int i = 0; i < n; ++i) yk[i] = s[i].y;
    uint64_t edges = 0;
    const int pick = oracle_draw_on_prefix(yk, n, p->temperature, *u, &edges);
    if (edges) *flags |= ORACLE_FLAG_DRAW_EDGE;
    *token = s[pick].i;
    counts[0] = k_eff;
    counts[1] = m;
    counts[2] = n;
}

int oracle_sample_row_masked(const float *x, int64_t V, const oracle_row_params *p,
                             const int32_t *hist, int64_t hlen,
                             const int32_t *allowed, int64_t n_allowed,
                             int32_t *token, int32_t counts[3],
                             int32_t kept_ids[64], float kept_logits[64],
                             uint32_t *x0, double *u, int32_t *flags)
{
    if (V <= 0) return -1;
    const int greedy = !(p->temperature > 0.0f);       /* NaN refused by callers */
    if (!greedy && (p->top_k < 1 || p->top_k > 64)) return -1;

    float *y = (float *)malloc((size_t)V * sizeof(float));
    scored *s = (scored *)malloc((size_t)V * sizeof(scored));
    unsigned char *in_d = (unsigned char *)calloc((size_t)V, 1);
    if (!y || !s || !in_d) { free(y); free(s); free(in_d); return -1; }
    if (oracle_penalised_row(x, V, p, hist, hlen, y) != 0) {
        free(y); free(s); free(in_d);
        return -1;
    }
    /* R11: a non-empty allowed list restricts the candidates to its distinct
     * in-range ids; an empty list leaves the whole vocabulary. */
    if (allowed != NULL && n_allowed > 0) {
        for (int64_t j = 0; j < n_allowed; ++j)
            if (allowed[j] >= 0 && allowed[j] < V) in_d[allowed[j]] = 1;
    } else {
        memset(in_d, 1, (size_t)V);
    }
    int64_t nd = 0;
    for (int64_t i = 0; i < V; ++i)
        if (in_d[i]) { s[nd].y = y[i]; s[nd].i = (int32_t)i; ++nd; }
    qsort(s, (size_t)nd, sizeof(scored), by_logit_then_index);
    chain_on_sorted(s, nd, p, token, counts, kept_ids, kept_logits, x0, u, flags);
    free(y); free(s); free(in_d);
    return 0;
}

int oracle_sample_row(const float *x, int64_t V, const oracle_row_params *p,
                      const int32_t *hist, int64_t hlen,
                      int32_t *token, int32_t counts[3],
                      int32_t kept_ids[64], float kept_logits[64],
                      uint32_t *x0, double *u, int32_t *flags)
{
    return oracle_sample_row_masked(x, V, p, hist, hlen, NULL, 0, token, counts, kept_ids,
                                    kept_logits, x0, u, flags);
}

/* Speculative verify windows [P19 "What changed": the emitted tokens are the
 * target's own samples; P559 "Not done (yet)": a sampled row is accepted when
 * its pick equals the draft].  Row j of a window holds the target's sample
 * after the first j drafts; draft[r] is the proposal that row r's sample is
 * compared with.  A window emits 1 + the number of leading rows (before its
 * last) whose sample equals its draft (R12). */
int oracle_accept_windows(const int32_t *token, int64_t B, int32_t window,
                          const int32_t *draft, int32_t *accepted)
{
    if (window < 1 || B % window != 0) return -1;
    for (int64_t w = 0; w < B / window; ++w) {
        const int64_t r0 = w * window;
        int32_t a = 0;
        while (a < window - 1 && token[r0 + a] == draft[r0 + a]) ++a;
        accepted[w] = a + 1;
    }
    return 0;
}

int oracle_sample_tokens(const float *logits, int64_t B, int64_t V, int64_t ld,
                         const oracle_row_params *params,
                         const int32_t *history, int64_t H, int64_t ldh,
                         const int32_t *hist_len,
                         int32_t *token, int32_t *counts, int32_t *kept_ids,
                         float *kept_logits, uint32_t *x0, double *u, int32_t *flags)
{
    for (int64_t r = 0; r < B; ++r) {
        const oracle_row_params *p = &params[r];
        const int32_t *h = NULL;
        int64_t hl = 0;
        if (p->history_row >= 0) {
            if (history == NULL || p->history_row >= H) return -1;
            h = history + (int64_t)p->history_row * ldh;
            hl = hist_len[p->history_row];
        }
        int rc = oracle_sample_row(logits + r * ld, V, p, h, hl, &token[r], &counts[3 * r],
                                   &kept_ids[64 * r], &kept_logits[64 * r], &x0[r], &u[r],
                                   &flags[r]);
        if (rc != 0) return rc;
    }
    return 0;
}

/* ---------------- logprobs [P3200 "Approach"], [P1916 "What changed"] ----
 * The model's own distribution: log-softmax of the raw logits, before the
 * penalties, temperature and the draw; with allowed ids, renormalised over
 * exactly those ids [P3200 "Problem and result"]. */
int oracle_token_logprobs_row(const float *x, int64_t V, int32_t token, int32_t top_n,
                              const int32_t *allowed, int64_t n_allowed,
                              double *token_lp, int32_t *top_ids, double *top_lp)
{
    if (V <= 0 || top_n < 0) return -1;
    unsigned char *in_d = (unsigned char *)calloc((size_t)V, 1);
    scored *s = (scored *)malloc((size_t)V * sizeof(scored));
    if (!in_d || !s) { free(in_d); free(s); return -1; }

    if (allowed != NULL && n_allowed > 0) {             /* R7 */
        for (int64_t j = 0; j < n_allowed; ++j)
            if (allowed[j] >= 0 && allowed[j] < V) in_d[allowed[j]] = 1;
    } else {
        memset(in_d, 1, (size_t)V);
    }

    int64_t nd = 0;
    double mx = -INFINITY;
    for (int64_t i = 0; i < V; ++i) {
        if (!in_d[i]) continue;
        const float v = sanitize(x[i]);
        s[nd].y = v;
        s[nd].i = (int32_t)i;
        ++nd;
        if ((double)v > mx) mx = (double)v;
    }

    double L;                                           /* log of the partition sum */
    if (nd == 0) {
        L = INFINITY;                                   /* empty domain: nothing has mass */
    } else if (mx == -INFINITY) {
        L = log((double)nd);                            /* R7: uniform; lp = 0 - L */
    } else {
        double z = 0.0;
        for (int64_t j = 0; j < nd; ++j) z += exp((double)s[j].y - mx);
        L = mx + log(z);
    }
    /* shifted logit of a member: x - L, or -L in the all -inf case */
#define LP_OF(v) ((mx == -INFINITY) ? -L : ((double)(v) - L))

    *token_lp = -INFINITY;
    if (token >= 0 && token < V && in_d[token])
        *token_lp = LP_OF(sanitize(x[token]));

    qsort(s, (size_t)nd, sizeof(scored), by_logit_then_index);
    for (int32_t j = 0; j < top_n; ++j) {
        if (j < nd) { top_ids[j] = s[j].i; top_lp[j] = LP_OF(s[j].y); }
        else        { top_ids[j] = -1;     top_lp[j] = -INFINITY; }
    }
#undef LP_OF
    free(in_d);
    free(s);
    return 0;
}
