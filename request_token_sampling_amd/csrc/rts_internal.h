// rts_internal.h -- launch descriptors shared by the C-ABI host code and the
// kernels.  Per-row parameters travel in the kernel-argument block, so a call
// needs no host-to-device copy and no staging buffer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// the C ABI's argument structs (include/rts.h)
struct rts_row_params;
struct rts_logprob_request;
struct rts_sample_extras;

namespace rts {

constexpr int kBlock = 256;          // threads per workgroup: four 64-lane waves
constexpr int kRowsPerLaunch = 64;   // rows whose parameters fit one argument block
constexpr int kMinChunk = 1024;      // smallest chunk of a row handled by one workgroup
constexpr int kMaxK = 64;            // largest top_k
constexpr int kMaxTopN = 20;         // largest top_logprobs
// Five waves per SIMD (VGPRs <= 96) keep five 256-thread workgroups resident
// per CU, 1,280 on the chip: a 40-row batch of 31 chunks fits in one round.
constexpr int kMinWavesPerSimd = 5;

// Workspace layout (bytes from its start):
//   [0, 8192)      sampling tickets, one per row slot of a launch, each on a
//                  128-byte line of its own: a row's chunks all hit one
//                  ticket, and rows sharing a line would queue behind each
//                  other's atomics
//   [8192, 16384)  logprob tickets, laid out the same way
//   [16384, 24576) verify-window tickets, one per window slot of a launch
//   then, for every row slot of a launch: chunk candidate keys (64 per chunk),
//   raw-logit top-K keys (20 per chunk) and (max, sum) partials (one per chunk)
constexpr int kTicketStride = 32;  // uint32 words between two row slots' tickets
constexpr size_t kTicketRegion = (size_t)kRowsPerLaunch * kTicketStride * 4u;
constexpr size_t kTicketBytes = 3 * kTicketRegion;

// Static LDS of the allowed-ids kernels besides their dynamic bitmap / list.
constexpr size_t kAllowedStaticLds = 10240;
// Rows whose allowed list holds at most kAllowedFast ids gather their members
// once into registers (kAllowedPerThread per thread); longer lists walk the
// bitmap in every pass.
constexpr int kAllowedPerThread = 16;
constexpr int kAllowedFast = kAllowedPerThread * kBlock;
// A sampling call that also renormalises its logprobs over allowed lists does
// it in the same launch when every list holds at most kRenormMax ids: one
// extra workgroup per row gathers the list (kRenormPerThread ids a thread)
// and drops repeats with a kRenormSlots-entry hash table in LDS.
constexpr int kRenormPerThread = 8;
constexpr int kRenormMax = kRenormPerThread * kBlock;
constexpr int kRenormSlots = 2 * kRenormMax;
// SampleRow.pack bit: the row's allowed list renormalises its logprobs and
// does not restrict its candidates.
constexpr uint32_t kPackRenorm = 1u << 25;

inline int64_t max_chunks(int64_t V) { return (V + kMinChunk - 1) / kMinChunk; }
inline size_t keys_bytes_per_row(int64_t V) { return (size_t)max_chunks(V) * kMaxK * 8u; }
inline size_t partial_bytes_per_row(int64_t V) { return (size_t)max_chunks(V) * 8u; }
inline size_t rawkeys_bytes_per_row(int64_t V) { return (size_t)max_chunks(V) * kMaxTopN * 8u; }

struct WsLayout {
    size_t keys, raw, partials, total;
};

inline WsLayout ws_layout(int64_t rows_ws, int64_t V)
{
    WsLayout l;
    const size_t r = (size_t)(rows_ws > 0 ? rows_ws : 1);
    l.keys = kTicketBytes;
    l.raw = l.keys + r * keys_bytes_per_row(V);
    l.partials = l.raw + r * rawkeys_bytes_per_row(V);
    l.total = (l.partials + r * partial_bytes_per_row(V) + 255u) & ~(size_t)255u;
    return l;
}

// Per-row sampling parameters after host-side checking (56 bytes).
struct SampleRow {
    uint64_t seed;
    uint64_t counter;
    int32_t hist_off;      // element offset of the window's first id in `history`
    int32_t allowed_off;   // first id of the row's allowed list in `allowed`
    float lnp;             // logf(min_p); -inf for min_p = 0
    float top_p;
    float temperature;
    float rep;
    float freq;
    float present;
    uint32_t pack;         // bits 0..15 window length, 16..22 k_eff, 24 greedy, 25 kPackRenorm
    int32_t allowed_cnt;   // 0: every id is a candidate
};
static_assert(sizeof(SampleRow) == 56, "argument block layout");

struct SampleArgs {
    const float *logits;   // row 0 of this launch
    int64_t ld;
    const int32_t *history;
    uint64_t *keys;        // workspace: per row slot nchunks * k_eff keys
    uint32_t *tickets;
    int32_t *token;        // outputs, row 0 of this launch
    int32_t *counts;
    int32_t *kept_ids;
    float *kept_logits;
    uint32_t *philox_x0;
    uint64_t *counters;     // device-resident counters (NULL: use row[].counter)
    int64_t counter_stride; // added to counters[] by every call
    int32_t V;
    int32_t nchunks;
    int32_t keys_stride;   // keys per row slot in the workspace
    int32_t rows;
    int32_t early_xcds;    // 1: work only on blockIdx % 8 < 2 (see logical_block)
    int32_t lp_topn;       // raw-logit logprobs in the same pass: top entries (0..20)
    int32_t lp_on;         // 1: compute the raw logprobs of the sampled token
    int32_t raw_stride;    // raw top-K keys per row slot in the workspace
    int32_t partial_stride;
    int32_t lpa_blocks;    // trailing workgroups that renormalise over allowed lists (0: none)
    uint64_t *raw_keys;    // workspace: per row slot nchunks * lp_topn keys
    uint64_t *partials;    // workspace: per row slot nchunks (max, sum) pairs
    float *lp_token;       // outputs, row 0 of this launch
    int32_t *lp_ids;
    float *lp_top;
    const int32_t *allowed;  // candidate lists of masked rows (row[].allowed_off/cnt)
    const int32_t *draft;    // verify windows: draft id per row, row 0 of this launch
    int32_t *accepted;       // tokens emitted per window, window 0 of this launch
    uint32_t *wtickets;      // workspace: one ticket per window slot
    uint32_t *ignored;       // device count of ids read and ignored (outside [0, V)), or NULL
    int32_t window;          // rows per verify window; 0: none
    int32_t chunk_major;     // 1: rows share one logits row; a chunk's rows share an XCD
    float *lpa_token;        // logprobs over allowed lists (NULL: not asked), row 0 of this launch
    int32_t *lpa_ids;
    float *lpa_top;
    uint64_t *lpa_w;         // workspace: one rendezvous word per row slot, 128 bytes apart
    SampleRow row[kRowsPerLaunch];
};
// HIP passes at most 4 KiB of kernel arguments.
static_assert(sizeof(SampleArgs) <= 4096, "kernel argument block");


struct LogprobRow {
    int64_t allowed_off;   // first id of the row's list in `allowed`
    int64_t allowed_cnt;   // 0: unrestricted
    int32_t row;           // row index within the launch's logits / outputs
    int32_t pad;
};

struct LogprobArgs {
    const float *logits;
    int64_t ld;
    const int32_t *tokens;
    const int32_t *allowed;
    uint64_t *keys;
    float2 *partials;
    uint32_t *tickets;
    float *token_lp;
    int32_t *top_ids;
    float *top_lp;
    int32_t V;
    int32_t nchunks;
    int32_t keys_stride;
    int32_t partial_stride;
    int32_t top_n;
    int32_t rows;
    int32_t early_xcds;
    int32_t pad_;
    LogprobRow row[kRowsPerLaunch];
};

// Launches with at most this many workgroups of work run on XCDs 0-1 only.
constexpr int kEarlyXcdWork = 64;

// Grid for `work` workgroups, padded for early-XCD placement when it applies.
__host__ __device__ inline unsigned grid_for(int work, int early)
{
    return early ? (unsigned)(((work + 1) / 2) * 8) : (unsigned)work;
}

// XCDs a launch's work is spread over (logical_block): 2 for early-XCD launches.
__host__ __device__ inline int xcds_used(int early) { return early ? 2 : 8; }

// Logical workgroups of a sampling launch.  Chunk-major launches (rows that
// share one logits row) pad the chunk count to a multiple of the XCDs used.
__host__ __device__ inline int sample_work(int rows, int nchunks, int early, int chunk_major)
{
    if (!chunk_major) return rows * nchunks;
    const int P = xcds_used(early);
    return rows * ((nchunks + P - 1) / P) * P;
}

// A workspace handed out after a call's arguments are checked (the static
// scratch of rts_sample_tokens_noalloc); returns an RTS_* code.
typedef int (*WorkspaceProvider)(void **workspace, hipStream_t stream);

// The body of rts_sample_tokens (rts_api.cpp), shared with the allocation-
// free entry point, and the thread's rts_last_error text.
int sample_tokens_impl(const float *logits, int64_t B, int64_t V, int64_t ld,
                       const ::rts_row_params *params,
                       const int32_t *history, int64_t H, int64_t ldh,
                       const int32_t *history_len,
                       int32_t *token, int32_t *counts, int32_t *kept_ids,
                       float *kept_logits, uint32_t *philox_x0,
                       uint64_t *counters, int64_t counter_stride,
                       const ::rts_logprob_request *lp, const ::rts_sample_extras *ex,
                       void *workspace, size_t ws_bytes, WorkspaceProvider get_ws,
                       hipStream_t stream);
int set_error(int code, const char *fmt, ...);
void clear_last_error();

// Launchers (return a hipError_t as int).
int launch_sample(const SampleArgs &a, int ept, bool vec, hipStream_t s);
int launch_logprobs_full(const LogprobArgs &a, int ept, bool vec, hipStream_t s);
// Kernels for restricted rows: a hash set (lists of <= kRenormMax ids, any V),
// or a vocabulary bitmap gathering at once (<= kAllowedFast ids) or walking it.
constexpr int kAllowedHash = 1;
constexpr int kAllowedFastBitmap = 2;
constexpr int kAllowedWide = 3;
int launch_logprobs_allowed(const LogprobArgs &a, size_t lds_bytes, int kind, hipStream_t s);
int launch_zero_u32(uint32_t *p, size_t n, hipStream_t s);

// The pages' earlier designs (rts_sample_tokens_prior): one thread per row,
// one workgroup per row with k argmax rounds, and the latter with the
// per-candidate penalty recount instead of the bitmap.
constexpr int PRIOR_THREAD = 1;
constexpr int PRIOR_BLOCK = 2;
constexpr int PRIOR_RECOUNT = 3;
int launch_prior(const SampleArgs &a, int design, size_t lds_bytes, hipStream_t s);
int launch_read_rows(const float *x, int rows, int V, int64_t ld, int nchunks, int out_stride,
                     float *out, int ept, bool vec, bool early, hipStream_t s);

}  // namespace rts
