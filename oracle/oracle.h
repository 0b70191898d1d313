/*
 * oracle.h -- plain CPU oracle for the per-token sampling chain.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path includes, links or
 * calls this code: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the HIP
 * library; both sides were written independently from the pages below.
 *
 * Sources (cited by page title and section):
 *   [P19]   "#19 serve: per-request temperature/top_p/top_k/min_p/penalties
 *           sampling", sections "What changed" and "Verification".
 *   [P3200] "#3200 [Engine] OpenAI logprobs / top_logprobs / allowed_token_ids
 *           for the CUDA/HIP engine", "Problem and result", "Approach", "Limits".
 *   [P1916] "#1916 OpenAI logprobs on /v1/chat/completions for the CUDA/HIP
 *           engine", "What changed".
 *   [SC11]  Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 *           1, 2, 3", SC'11 -- the Philox4x32-10 block function.
 */
#ifndef RTS_ORACLE_H
#define RTS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Per-row sampling request, the oracle's own definition. */
typedef struct {
    float    temperature;     /* <= 0: greedy */
    int32_t  top_k;           /* sampled rows: 1..64 */
    float    top_p;           /* (0, 1]; >= 1 disables the cut */
    float    min_p;           /* [0, 1]; 0 disables the cut */
    float    penalty_repeat;  /* 1 = neutral */
    float    penalty_freq;    /* 0 = neutral */
    float    penalty_present; /* 0 = neutral */
    int32_t  penalty_last_n;  /* -1 whole history, 0 off, > 0 window length */
    int32_t  history_row;     /* -1 none, else a row of the history matrix */
    int32_t  pad_;
    uint64_t seed;
    uint64_t counter;
} oracle_row_params;

/* Flags reported per row: where two correct floating-point implementations
 * may take a different branch. */
#define ORACLE_FLAG_TOP_P_EDGE 1  /* a cumulative top_p sum within 1e-6 of top_p */
#define ORACLE_FLAG_DRAW_EDGE  2  /* the uniform draw within 1e-6 of a CDF step */

/* Philox4x32-10 block function [SC11]: out = philox(ctr, key). */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* The sampling chain on one row of V logits.
 *   hist/hlen: the row's full history (the window is its tail); may be NULL/0.
 *   kept_ids/kept_logits: 64 entries each, padded with -1 / -INFINITY.
 *   counts: (k_eff, m, n) -- kept after top_k, after min_p, after top_p.
 *   u: the uniform draw (0 for greedy rows).  Returns 0, or -1 on bad input. */
int oracle_sample_row(const float *x, int64_t V, const oracle_row_params *p,
                      const int32_t *hist, int64_t hlen,
                      int32_t *token, int32_t counts[3],
                      int32_t kept_ids[64], float kept_logits[64],
                      uint32_t *x0, double *u, int32_t *flags);

/* The chain with the candidates restricted to the distinct in-range ids of
 * `allowed` (n_allowed > 0; R11): k_eff = min(top_k, |D|); an empty D gives
 * token -1 and counts (0, 0, 0).  n_allowed = 0 is oracle_sample_row. */
int oracle_sample_row_masked(const float *x, int64_t V, const oracle_row_params *p,
                             const int32_t *hist, int64_t hlen,
                             const int32_t *allowed, int64_t n_allowed,
                             int32_t *token, int32_t counts[3],
                             int32_t kept_ids[64], float kept_logits[64],
                             uint32_t *x0, double *u, int32_t *flags);

/* Verify windows of `window` consecutive rows (B a multiple of it):
 * accepted[w] = 1 + the number of leading rows r of window w, before its
 * last, with token[r] == draft[r] (R12). */
int oracle_accept_windows(const int32_t *token, int64_t B, int32_t window,
                          const int32_t *draft, int32_t *accepted);

/* The draw alone (temperature, then the inverse CDF at u) over the first n
 * kept logits y[0..n), n in 1..64; returns the picked position.  Bit j of
 * *edges marks |cdf_j - u| < 1e-6 (a flagged draw, where another correct
 * fp64 evaluation may pick position j + 1 instead of j, or j instead of
 * j + 1). */
int oracle_draw_on_prefix(const float *y, int n, float temperature, double u, uint64_t *edges);

/* Penalised and sanitised logits of one row (the chain's first two steps). */
int oracle_penalised_row(const float *x, int64_t V, const oracle_row_params *p,
                         const int32_t *hist, int64_t hlen, float *y);

/* B rows at once: logits [B][ld], history [H][ldh] with lengths hist_len[H]. */
int oracle_sample_tokens(const float *logits, int64_t B, int64_t V, int64_t ld,
                         const oracle_row_params *params,
                         const int32_t *history, int64_t H, int64_t ldh,
                         const int32_t *hist_len,
                         int32_t *token, int32_t *counts, int32_t *kept_ids,
                         float *kept_logits, uint32_t *x0, double *u, int32_t *flags);

/* Log-softmax of the raw (sanitised) logits over the domain D -- all of
 * [0, V), or the distinct in-range ids of `allowed` when n_allowed > 0.
 * token_lp is -INFINITY when token is not in D; top_ids/top_lp hold the first
 * top_n members of D by (logit desc, index asc), padded with (-1, -INFINITY). */
int oracle_token_logprobs_row(const float *x, int64_t V, int32_t token, int32_t top_n,
                              const int32_t *allowed, int64_t n_allowed,
                              double *token_lp, int32_t *top_ids, double *top_lp);

#ifdef __cplusplus
}
#endif
#endif
