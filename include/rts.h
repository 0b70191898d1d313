/*
 * rts.h -- C ABI of the MI355X (gfx950) per-token sampler.
 *
 * For each of B rows of fp32 head logits the library runs the sampling chain
 * of page "#19 serve: per-request temperature/top_p/top_k/min_p/penalties
 * sampling" (section "What changed"):
 *   penalties (repeat / frequency / presence over a history window, looked up
 *   through a per-chunk token bitmap) -> top_k (k in 1..64, kept in
 *   descending order, ties to the lowest index) -> min_p cut -> top_p cut ->
 *   temperature -> Philox4x32-10 draw keyed by (seed, counter);
 * and the logprobs of page "#3200 [Engine] OpenAI logprobs / top_logprobs /
 * allowed_token_ids for the CUDA/HIP engine" (sections "Problem and result",
 * "Approach", "Limits"): log-softmax of the raw logits with up to 20 top
 * entries, optionally renormalised over a list of allowed ids.
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are HIP device memory; "host" are host memory
 *    read before the call returns.  The caller owns every buffer; the library
 *    allocates nothing and keeps no pointer after returning.
 *  - Work is enqueued on `stream` and runs asynchronously; outputs are valid
 *    once the stream has reached that point.  A workspace may not be used by
 *    two calls that can run at the same time.
 *  - Return value: RTS_OK, or a negative RTS_E* code.  All argument checks
 *    run before anything is enqueued, so a failed call writes nothing.
 *    rts_last_error() names the offending row and field (per thread).
 *  - Device-resident ids (history rows, allowed lists, tokens) are not
 *    validated: ids outside [0, V) are ignored as the pages' semantics
 *    require no host round trip (rts_sample_extras.ignored_ids counts the
 *    ones a sampling call ignored).
 */
#ifndef RTS_H
#define RTS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RTS_OK 0
#define RTS_EINVAL (-1)  /* a bad shape, pointer or per-row parameter   */
#define RTS_ENOSPC (-2)  /* the workspace is smaller than required      */
#define RTS_EDEVICE (-3) /* a HIP launch error                          */

#define RTS_MAX_TOP_K 64 /* top_k limit of sampled rows (#19, "A persistent per-request draw counter") */
#define RTS_KEPT 64      /* entries per row of kept_ids / kept_logits          */
#define RTS_MAX_TOP_N 20 /* top_logprobs limit (#3200, "Problem and result")   */
#define RTS_MAX_WINDOW 65535 /* longest penalty window, in ids                  */
#define RTS_MAX_V (1LL << 30) /* largest vocabulary: ids and chunk offsets stay in 32-bit arithmetic */

/*
 * Per-row request (#19, "What changed": the per-request paragraph lists the
 * keys; the counter paragraph makes the counter the caller's).  56 bytes.
 */
typedef struct rts_row_params {
    float temperature;     /* <= 0: greedy (argmax of the penalised logits); else finite > 0 */
    int32_t top_k;         /* sampled rows: 1..64, else RTS_EINVAL; ignored for greedy rows  */
    float top_p;           /* (0, 1]; 1 disables the cut                                     */
    float min_p;           /* [0, 1]; 0 disables the cut                                     */
    float penalty_repeat;  /* finite > 0; 1 = neutral                                        */
    float penalty_freq;    /* finite; 0 = neutral                                            */
    float penalty_present; /* finite; 0 = neutral                                            */
    int32_t penalty_last_n;/* -1: whole history row, 0: no penalties, > 0: window length     */
    int32_t history_row;   /* -1: none (neutral path), else a row index into `history`       */
    int32_t reserved;      /* must be 0                                                      */
    uint64_t seed;         /* Philox key (low word, high word)                               */
    uint64_t counter;      /* Philox counter (low word, high word, 0, 0); caller-owned       */
} rts_row_params;

/*
 * Raw-logit logprobs computed in the same pass over the logits as the draw
 * (#3200, "Approach": the reported distribution is the model's own, taken
 * before penalties and temperature).  Given to rts_sample_tokens, it asks for
 * what rts_token_logprobs would report, unrestricted, for the tokens that
 * call samples, without reading the logits a second time.
 *   top_n     0..20 entries of top_ids / top_lp per row.
 *   reserved  must be 0.
 *   token_lp  device f32 [B]: logprob of the sampled token.
 *   top_ids   device int32 [B][top_n]; top_lp device f32 [B][top_n]: the
 *             row's largest raw logits in (logit desc, index asc) order and
 *             their logprobs.  Both may be NULL when top_n = 0.
 * Optionally, the same values renormalised over allowed_token_ids (#3200,
 * "Problem and result": the distribution over exactly the listed ids), as
 * rts_token_logprobs reports them for these lists and the sampled tokens.
 * The lists do not restrict sampling (rts_sample_extras.allowed does).
 *   allowed           device int32 ids, row r owning allowed[allowed_off[r]
 *                     .. allowed_off[r+1]); NULL for none (then the four
 *                     fields below must be NULL too).  Repeated ids count
 *                     once and ids outside [0, V) are ignored; a row with
 *                     an empty list reports the unrestricted values.
 *   allowed_off       host int64 [B+1], non-decreasing, allowed_off[0] >= 0.
 *   allowed_token_lp  device f32 [B]: the sampled token's renormalised
 *                     logprob, -inf when the token is not listed.
 *   allowed_top_ids / allowed_top_lp  device [B][top_n]: the top listed
 *                     ids; NULL allowed when top_n = 0.
 * When no row also has an rts_sample_extras list and every list holds at
 * most 2,048 ids, these are computed by extra workgroups of the sampling
 * launch, overlapped with it.  Otherwise a second launch computes them after
 * the draw, as rts_token_logprobs does (lists longer than 2,048 ids then need
 * V <= 2^19; RTS_EINVAL before anything is enqueued).
 */
typedef struct rts_logprob_request {
    int32_t top_n;
    int32_t reserved;
    float *token_lp;
    int32_t *top_ids;
    float *top_lp;
    const int32_t *allowed;
    const int64_t *allowed_off;
    float *allowed_token_lp;
    int32_t *allowed_top_ids;
    float *allowed_top_lp;
} rts_logprob_request;

/*
 * Speculative verify windows and masked sampling for rts_sample_tokens.
 *   window      rows per verify window (1..64), 0 for none; B must be a
 *               multiple of it.  Rows r0 .. r0+window-1 hold the target's
 *               logits after 0, 1, ... drafts of one sequence (#19, "What
 *               changed": the emitted tokens are the target's own samples;
 *               #559, "Not done (yet)": a sampled row is accepted when its
 *               pick equals the draft).
 *   reserved    must be 0.
 *   draft       device int32 [B] when window > 0: draft[r] is the proposal
 *               row r's sample is compared with (ignored on each window's
 *               last row).
 *   accepted    device int32 [B / window] when window > 0: the number of
 *               target tokens the window emits, 1 + the number of leading
 *               rows whose sample equals their draft.
 *   allowed     device int32 ids, row r owning allowed[allowed_off[r] ..
 *               allowed_off[r+1]), or NULL.  A row with a non-empty range
 *               samples only among its distinct ids in [0, V) (the sampler
 *               masked by allowed_token_ids): k_eff = min(top_k, that count),
 *               and with none in range the row's token is -1 and its counts
 *               are 0.  The fused logprobs stay unrestricted.
 *   allowed_off host int64 [B+1], non-decreasing, allowed_off[0] >= 0,
 *               allowed_off[B] < 2^31.
 *   ignored_ids device uint32 [1], or NULL.  The call adds the number of
 *               device-resident ids it read and ignored because they lie
 *               outside [0, V): history ids in the window of a row whose
 *               penalties apply, and allowed ids of masked rows, each
 *               occurrence once per row.  Ids are not validated otherwise
 *               (that would need a host round trip); this word lets a
 *               caller notice bad ids without one.
 */
typedef struct rts_sample_extras {
    int32_t window;
    int32_t reserved;
    const int32_t *draft;
    int32_t *accepted;
    const int32_t *allowed;
    const int64_t *allowed_off;
    uint32_t *ignored_ids;
} rts_sample_extras;

/* Bytes of workspace that calls with up to B rows of V logits need
 * (both entry points).  *bytes is set on RTS_OK. */
int rts_workspace_bytes(int64_t B, int64_t V, size_t *bytes);

/* Prepare a fresh workspace (zero its counters) on `stream`.  A workspace
 * that was zero-filled by the caller needs no call; the library returns its
 * counters to zero at the end of every call. */
int rts_workspace_init(void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * The sampling chain over B rows.
 *   logits      device fp32 [B][ld], row-major, ld >= V; 0 < V <= 2^30.  ld = 0
 *               makes every row read row 0: several parameter sets (several
 *               samples, a sampled and a greedy pass) over one distribution.
 *   params      host [B].
 *   history     device int32 [H][ldh] or NULL when no row names one; row h
 *               holds history_len[h] ids, oldest first.  The window of a row
 *               is the last min(penalty_last_n, history_len) ids of its
 *               history row (all of them for penalty_last_n = -1), at most
 *               RTS_MAX_WINDOW ids.  Rows of a verify window may share one
 *               history row (#19, "What changed", the penalties paragraph).
 *   history_len host int32 [H].
 * Outputs (device; all but `token` may be NULL):
 *   token       int32 [B]      the sampled id (greedy: the argmax).
 *   counts      int32 [B][3]   (k_eff, kept after min_p, kept after top_p).
 *   kept_ids    int32 [B][64]  the top_k sequence, padded with -1.
 *   kept_logits f32 [B][64]    its penalised logits, padded with -inf.
 *   philox_x0   uint32 [B]     first Philox output word (0 for greedy rows).
 *   counters    device uint64 [B] or NULL.  NULL: row r draws with
 *               params[r].counter.  Otherwise row r draws with counters[r]
 *               (params[r].counter is ignored) and the call adds
 *               counter_stride to counters[r] (every row, greedy ones too),
 *               so a captured HIP graph that replays the call draws fresh
 *               numbers on every replay instead of repeating them (page
 *               "#19 ...", "Problem": a captured sampler would replay the same
 *               draws forever; "A persistent per-request draw counter").
 *   lp          host, or NULL for no logprobs: see rts_logprob_request.
 *   ex          host, or NULL: verify windows and allowed-id masks, see
 *               rts_sample_extras.
 * Errors: RTS_EINVAL for B < 0, V out of range, 0 < ld < V, NULL logits/token,
 * a row with NaN or infinite temperature, top_k outside 1..64 on a sampled
 * row, top_p outside (0, 1], min_p outside [0, 1], penalty_repeat <= 0 or
 * non-finite penalties, history_row >= H or set without history, a window
 * longer than RTS_MAX_WINDOW, reserved != 0, an lp request with top_n
 * outside 0..20, reserved != 0, a NULL output it needs, bad allowed offsets,
 * allowed_* fields without allowed, or lists that need V <= 2^19, extras with a
 * window outside 0..64 or not dividing B, missing draft / accepted, or bad
 * allowed offsets, or history offsets (history_row * ldh + length) of 2^31
 * or more; RTS_ENOSPC for a short
 * workspace; RTS_EDEVICE if a launch fails.  B = 0 is a no-op.
 */
int rts_sample_tokens(const float *logits, int64_t B, int64_t V, int64_t ld,
                      const rts_row_params *params,
                      const int32_t *history, int64_t H, int64_t ldh,
                      const int32_t *history_len,
                      int32_t *token, int32_t *counts, int32_t *kept_ids,
                      float *kept_logits, uint32_t *philox_x0,
                      uint64_t *counters, int64_t counter_stride,
                      const rts_logprob_request *lp, const rts_sample_extras *ex,
                      void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * rts_sample_tokens for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, outputs, errors and results are those of
 * rts_sample_tokens without `workspace` / `ws_bytes`: the scratch memory
 * comes from one static device array inside the library,
 * rts_noalloc_scratch_bytes() bytes (16 MiB) per GPU, held by every GPU the
 * library runs on until the process ends.  The call allocates nothing.
 *  - Calls whose rows need more scratch than that (rts_workspace_bytes(B, V)
 *    above it; 64 rows fit V <= 394,240) return RTS_ENOSPC before anything
 *    is enqueued, with rts_last_error() giving both sizes.
 *  - The first call on a device looks the array up for that device and
 *    enqueues one small kernel on `stream` that zeroes its counters; every
 *    call leaves them zeroed for the next.
 *  - Every call on one GPU shares that GPU's array: calls that can overlap on
 *    one GPU (two streams, two host threads) race and must be serialised by
 *    the caller.
 */
size_t rts_noalloc_scratch_bytes(void);
int rts_sample_tokens_noalloc(const float *logits, int64_t B, int64_t V, int64_t ld,
                              const rts_row_params *params,
                              const int32_t *history, int64_t H, int64_t ldh,
                              const int32_t *history_len,
                              int32_t *token, int32_t *counts, int32_t *kept_ids,
                              float *kept_logits, uint32_t *philox_x0,
                              uint64_t *counters, int64_t counter_stride,
                              const rts_logprob_request *lp, const rts_sample_extras *ex,
                              hipStream_t stream);

/*
 * Log-softmax of the raw logits (before penalties and temperature), per row:
 * the OpenAI logprobs and top_logprobs of page "#3200 [Engine] OpenAI
 * logprobs / top_logprobs / allowed_token_ids for the CUDA/HIP engine"
 * ("Problem and result": up to 20 alternatives per token, and with
 * allowed_token_ids a distribution renormalised over exactly the listed ids;
 * "Approach": the values are the model's own distribution, taken from the
 * head logits before the sampling chain), which page "#1916 OpenAI logprobs
 * on /v1/chat/completions for the CUDA/HIP engine" ("What changed") takes
 * from the same head logits as the sampled token.
 *   logits      device fp32 [B][ld] as above; NaN counts as -inf, +inf as
 *               the largest finite float.
 *   tokens      device int32 [B]: the ids whose logprob is reported.
 *   top_n       0..20 entries of top_ids / top_lp per row.
 *   allowed     device int32 ids, row r owning allowed[allowed_off[r] ..
 *               allowed_off[r+1]); NULL for no restriction.  A row with an
 *               empty range is unrestricted; duplicates count once; ids
 *               outside [0, V) are ignored.  Lists longer than 2,048 ids need
 *               V <= 2^19 (a vocabulary bitmap in LDS); shorter ones take a
 *               hash set past that size.
 *   allowed_off host int64 [B+1], non-decreasing, allowed_off[0] >= 0.
 * Outputs (device): token_lp f32 [B] (-inf when the token is outside the
 * row's domain), top_ids int32 [B][top_n] and top_lp f32 [B][top_n], the
 * domain's largest logits in (logit desc, index asc) order, padded with
 * (-1, -inf).  top_ids/top_lp may be NULL when top_n = 0.
 */
int rts_token_logprobs(const float *logits, int64_t B, int64_t V, int64_t ld,
                       const int32_t *tokens, int32_t top_n,
                       const int32_t *allowed, const int64_t *allowed_off,
                       float *token_lp, int32_t *top_ids, float *top_lp,
                       void *workspace, size_t ws_bytes, hipStream_t stream);

/* Static description of an error code. */
const char *rts_strerror(int code);

/* Text of the last error raised on the calling thread ("" if none). */
const char *rts_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
