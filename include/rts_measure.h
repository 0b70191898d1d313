/*
 * rts_measure.h -- measurement entry points of librts.so, beside the product
 * ABI in rts.h.  Neither is part of the sampling path: they exist so the
 * single-pass sampler can be timed against the designs it replaces and
 * against a bare read of the same bytes.  Conventions (device / host
 * pointers, streams, error codes, rts_last_error) are those of rts.h.
 */
#ifndef RTS_MEASURE_H
#define RTS_MEASURE_H

#include "rts.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The pages' earlier designs of the same chain, kept as measured ablations of
 * rts_sample_tokens (#19, "What changed", the one-block-per-token and the
 * min_p-and-penalties paragraphs).  Same outputs, bit for bit:
 *   RTS_PRIOR_THREAD   one thread per row: top_k as k sequential
 *                      full-vocabulary scans (the design the pages replaced);
 *   RTS_PRIOR_BLOCK    one workgroup per row: k argmax rounds, each a wave
 *                      then workgroup reduction over the whole row; penalty
 *                      counts through a per-row token bitmap in LDS, a
 *                      flagged id scanning the window;
 *   RTS_PRIOR_RECOUNT  the same with every id scanning the window (the naive
 *                      O(k * V * window) recount the bitmap replaced).
 * Arguments as in rts_sample_tokens (host counters only, no logprobs, no
 * extras); V <= 2^20.  The kernels reread the row k times: they exist to be
 * measured against the single-pass kernel, not to be used.
 */
#define RTS_PRIOR_THREAD 1
#define RTS_PRIOR_BLOCK 2
#define RTS_PRIOR_RECOUNT 3
int rts_sample_tokens_prior(int design, const float *logits, int64_t B, int64_t V, int64_t ld,
                            const rts_row_params *params,
                            const int32_t *history, int64_t H, int64_t ldh,
                            const int32_t *history_len,
                            int32_t *token, int32_t *counts, int32_t *kept_ids,
                            float *kept_logits, uint32_t *philox_x0,
                            void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * A plain streaming read of the rows, the measuring stick for the sampler's
 * bandwidth: the same grid, chunking, 16-byte loads and row-major layout as
 * rts_sample_tokens over the same B rows, with only a maximum taken per
 * chunk and no selection, merge or draw.  Its duration is the practical
 * floor of any one-pass kernel over those bytes.
 *   logits     device fp32 [B][ld] as in rts_sample_tokens.
 *   chunk_max  device fp32 [B][ceil(V / 1024)]; row r's first C entries
 *              receive its chunk maxima (C = the sampler's chunk count for
 *              this B and V), NaN ignored.
 * Errors: RTS_EINVAL for bad shapes or NULL pointers; RTS_EDEVICE if the
 * launch fails.  B = 0 is a no-op.
 */
int rts_read_rows(const float *logits, int64_t B, int64_t V, int64_t ld, float *chunk_max,
                  hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
