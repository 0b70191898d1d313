// rts_api.cpp -- the C ABI declared in include/rts.h and include/rts_measure.h: argument checks, the
// per-launch argument blocks, chunk sizing and the launches.  Every check
// runs before anything is enqueued, so a refused call writes nothing (page
// "#19 serve: per-request temperature/top_p/top_k/min_p/penalties sampling",
// "What changed": a sampled request outside top_k 1..64 is refused rather
// than left to write a stale token, and a bad sampling value is refused
// rather than silently changed).
#include "rts.h"
#include "rts_measure.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "rts_internal.h"

static_assert(rts::PRIOR_THREAD == RTS_PRIOR_THREAD && rts::PRIOR_BLOCK == RTS_PRIOR_BLOCK &&
                  rts::PRIOR_RECOUNT == RTS_PRIOR_RECOUNT,
              "design numbers of the C ABI and the kernels");

namespace {

thread_local char g_last_error[512];

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_last_error[0] = '\0'; }

// Rows per launch and elements per thread.  A launch covers up to 64 rows;
// each workgroup covers a chunk of 256 * ept elements.  A smaller chunk
// shortens the per-workgroup selection (its ballot compaction takes one step
// per element a thread holds) while the row merge grows with the chunks per
// row, and a grid larger than the chip holds at once (five workgroups per CU)
// runs in two rounds.  So the chunk is the smallest with at most 64 chunks
// per row whose grid still fits one round; when none does, the largest
// (8,192 elements).  Measured on MI355X at V = 248,320: one row read as two
// parameter rows 10.0 -> 9.45 us and a 5-row window 12.4 -> 12.0 us at 4,096
// elements against 8,192; 2,048 was slower for both (9.66, 12.0 at 4,096 and
// 11.0 us at 1,024 for the former); 40 rows stay at 8,192.
constexpr int64_t kMaxChunksPerRow = 64;
constexpr int64_t kResidentWorkgroups = 5 * 256;

int choose_ept(int64_t rows, int64_t V)
{
    static const int opts[4] = {4, 8, 16, 32};
    for (int i = 0; i < 4; ++i) {
        const int64_t ch = (int64_t)rts::kBlock * opts[i];
        const int64_t nch = (V + ch - 1) / ch;
        if (nch <= kMaxChunksPerRow && rows * nch <= kResidentWorkgroups) return opts[i];
    }
    return 32;
}

int64_t chunks_for(int64_t V, int ept)
{
    const int64_t ch = (int64_t)rts::kBlock * ept;
    return (V + ch - 1) / ch;
}

bool is_vec_ok(const float *p, int64_t ld)
{
    return (reinterpret_cast<uintptr_t>(p) % 16u) == 0u && (ld % 4) == 0;
}

size_t max_lds_per_block()
{
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 65536;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        return 65536;
    return (size_t)v;
}

// Every row's parameters (and its history window), before anything is
// enqueued; returns RTS_OK or the error of the first bad row.
int check_rows(int64_t B, const rts_row_params *params, const int32_t *history, int64_t H,
               int64_t ldh, const int32_t *history_len)
{
    for (int64_t r = 0; r < B; ++r) {
        const rts_row_params &p = params[r];
        const long long rr = (long long)r;
        if (std::isnan(p.temperature) || std::isinf(p.temperature))
            return fail(RTS_EINVAL, "row %lld: temperature is not finite", rr);
        const bool greedy = !(p.temperature > 0.0f);
        if (!greedy && (p.top_k < 1 || p.top_k > RTS_MAX_TOP_K))
            return fail(RTS_EINVAL, "row %lld: top_k = %d outside 1..64 on a sampled row", rr, p.top_k);
        if (!(p.top_p > 0.0f && p.top_p <= 1.0f))
            return fail(RTS_EINVAL, "row %lld: top_p = %g outside (0, 1]", rr, (double)p.top_p);
        if (!(p.min_p >= 0.0f && p.min_p <= 1.0f))
            return fail(RTS_EINVAL, "row %lld: min_p = %g outside [0, 1]", rr, (double)p.min_p);
        if (!(p.penalty_repeat > 0.0f) || std::isinf(p.penalty_repeat))
            return fail(RTS_EINVAL, "row %lld: penalty_repeat = %g must be finite > 0", rr,
                        (double)p.penalty_repeat);
        if (!std::isfinite(p.penalty_freq) || !std::isfinite(p.penalty_present))
            return fail(RTS_EINVAL, "row %lld: penalty_freq / penalty_present not finite", rr);
        if (p.penalty_last_n < -1)
            return fail(RTS_EINVAL, "row %lld: penalty_last_n = %d < -1", rr, p.penalty_last_n);
        if (p.history_row < -1)
            return fail(RTS_EINVAL, "row %lld: history_row = %d < -1", rr, p.history_row);
        if (p.reserved != 0) return fail(RTS_EINVAL, "row %lld: reserved field is not 0", rr);
        if (p.history_row >= 0) {
            if (history == nullptr || history_len == nullptr)
                return fail(RTS_EINVAL, "row %lld: history_row set without history", rr);
            if (p.history_row >= H)
                return fail(RTS_EINVAL, "row %lld: history_row = %d >= H = %lld", rr,
                            p.history_row, (long long)H);
            const int32_t hl = history_len[p.history_row];
            if (hl < 0 || hl > ldh)
                return fail(RTS_EINVAL, "history row %d: length %d outside [0, ldh = %lld]",
                            p.history_row, hl, (long long)ldh);
            if ((int64_t)p.history_row * ldh + hl > 0x7FFFFFFFLL)
                return fail(RTS_EINVAL, "row %lld: history offset of 2^31 ids or more", rr);
            const int64_t n_eff = p.penalty_last_n < 0 ? hl
                                  : (p.penalty_last_n < hl ? p.penalty_last_n : hl);
            if (n_eff > RTS_MAX_WINDOW)
                return fail(RTS_EINVAL, "row %lld: penalty window of %lld ids > %d", rr,
                            (long long)n_eff, RTS_MAX_WINDOW);
        }
    }

    return RTS_OK;
}

// The kernel's view of one checked row.
void pack_row(rts::SampleRow &s, const rts_row_params &p, int64_t V, const int32_t *history_len,
              int64_t ldh, int32_t allowed_off, int32_t allowed_cnt)
{
    const bool greedy = !(p.temperature > 0.0f);
    const int64_t k_eff = greedy ? 1 : (p.top_k < V ? p.top_k : V);
    int64_t n_eff = 0, hist_off = 0;
    const bool neutral = p.penalty_repeat == 1.0f && p.penalty_freq == 0.0f &&
                         p.penalty_present == 0.0f;
    if (p.history_row >= 0 && !neutral) {
        const int32_t hl = history_len[p.history_row];
        n_eff = p.penalty_last_n < 0 ? hl : (p.penalty_last_n < hl ? p.penalty_last_n : hl);
        hist_off = (int64_t)p.history_row * ldh + (hl - n_eff);
    }
    s.seed = p.seed;
    s.counter = p.counter;
    s.hist_off = (int32_t)hist_off;
    s.allowed_off = allowed_off;
    s.allowed_cnt = allowed_cnt;
    s.lnp = logf(p.min_p);
    s.top_p = p.top_p;
    s.temperature = p.temperature;
    s.rep = p.penalty_repeat;
    s.freq = p.penalty_freq;
    s.present = p.penalty_present;
    s.pack = (uint32_t)n_eff | ((uint32_t)k_eff << 16) | (greedy ? (1u << 24) : 0u);
}

// Per-row offsets into an id list: off[0] >= 0 and never decreasing.
int check_offsets(int64_t B, const int64_t *off, const char *what)
{
    if (off[0] < 0) return fail(RTS_EINVAL, "%s[0] < 0", what);
    for (int64_t r = 0; r < B; ++r)
        if (off[r + 1] < off[r]) return fail(RTS_EINVAL, "%s decreases at row %lld", what, (long long)r);
    return RTS_OK;
}

// The bitmap kernels for allowed lists keep a vocabulary bitmap in LDS: true
// when it fits (V <= 2^19).  Lists of up to kRenormMax ids also have the
// hash-set kernel, which needs no bitmap; longer ones need the bitmap.
bool bitmap_fits(int64_t V)
{
    const size_t bitmap_bytes = (size_t)((V + 31) / 32) * 4u;
    const size_t max_lds = V > (1 << 19) ? 0 : max_lds_per_block();
    return bitmap_bytes + rts::kAllowedStaticLds <= max_lds;
}

int refuse_long_lists(int64_t V)
{
    return fail(RTS_EINVAL, "allowed lists of more than %d ids need V <= 2^19 (V = %lld)",
                rts::kRenormMax, (long long)V);
}

// The launches of rts_token_logprobs once its arguments are checked.  Rows
// with an empty list take the full-row reducer, unless `restricted_only`
// leaves them out.  Restricted rows take the bitmap kernels when the bitmap
// fits (gather-once up to kAllowedFast ids, else walking the bitmap; measured
// faster than the hash set on 1,000-id lists), else the hash-set kernel
// (lists of up to kRenormMax ids, checked by the caller).  ld = 0 makes every
// row read row 0.
int enqueue_logprobs(const float *logits, int64_t B, int64_t V, int64_t ld, const int32_t *tokens,
                     int32_t top_n, const int32_t *allowed, const int64_t *allowed_off,
                     float *token_lp, int32_t *top_ids, float *top_lp, void *workspace,
                     bool restricted_only, hipStream_t stream)
{
    const bool bitmap = bitmap_fits(V);
    const size_t bitmap_bytes = (size_t)((V + 31) / 32) * 4u;
    bool any_restricted = false;
    if (allowed != nullptr)
        for (int64_t r = 0; r < B && !any_restricted; ++r)
            any_restricted = allowed_off[r + 1] > allowed_off[r];

    char *ws = static_cast<char *>(workspace);
    rts::LogprobArgs base;
    std::memset(&base, 0, sizeof base);
    base.logits = logits;
    base.ld = ld;
    base.tokens = tokens;
    base.allowed = allowed;
    const int64_t rows_ws = B < rts::kRowsPerLaunch ? B : rts::kRowsPerLaunch;
    const rts::WsLayout L = rts::ws_layout(rows_ws, V);
    base.keys = reinterpret_cast<uint64_t *>(ws + L.keys);
    base.tickets = reinterpret_cast<uint32_t *>(ws + rts::kTicketRegion);
    base.token_lp = token_lp;
    base.top_ids = top_ids;
    base.top_lp = top_lp;
    base.V = (int32_t)V;
    base.keys_stride = (int32_t)(rts::keys_bytes_per_row(V) / 8u);
    base.partial_stride = (int32_t)rts::max_chunks(V);
    base.top_n = top_n;
    base.partials = reinterpret_cast<float2 *>(ws + L.partials);

    // kind 0: unrestricted rows (full-row reducer); then rts::kAllowedHash,
    // kAllowedFastBitmap and kAllowedWide.  Each kind in launches of up to 64 rows.
    for (int kind = restricted_only ? 1 : 0; kind <= rts::kAllowedWide; ++kind) {
        if (kind > 0 && !any_restricted) break;
        rts::LogprobArgs a = base;
        int n = 0;
        auto flush = [&]() -> int {
            if (n == 0) return 0;
            a.rows = n;
            int e;
            if (kind == 0) {
                const bool vec = is_vec_ok(logits, ld);
                int ept = choose_ept(n, V);
                if (!vec && ept > 16) ept = 16;  // as for sampling: the scalar-load form spills at 32
                a.nchunks = (int32_t)chunks_for(V, ept);
                a.early_xcds = n * a.nchunks <= rts::kEarlyXcdWork ? 1 : 0;
                e = rts::launch_logprobs_full(a, ept, vec, stream);
            } else {
                e = rts::launch_logprobs_allowed(a, bitmap_bytes, kind, stream);
            }
            n = 0;
            return e;
        };
        for (int64_t r = 0; r < B; ++r) {
            const int64_t cnt = allowed ? allowed_off[r + 1] - allowed_off[r] : 0;
            const int row_kind = cnt == 0  ? 0
                                 : !bitmap ? rts::kAllowedHash
                                 : cnt <= rts::kAllowedFast ? rts::kAllowedFastBitmap
                                                            : rts::kAllowedWide;
            if (row_kind != kind) continue;
            rts::LogprobRow &lr = a.row[n++];
            lr.row = (int32_t)r;
            lr.allowed_off = allowed ? allowed_off[r] : 0;
            lr.allowed_cnt = cnt;
            lr.pad = 0;
            if (n == rts::kRowsPerLaunch) {
                const int e = flush();
                if (e != 0)
                    return fail(RTS_EDEVICE, "logprob launch: %s", hipGetErrorString((hipError_t)e));
            }
        }
        const int e = flush();
        if (e != 0) return fail(RTS_EDEVICE, "logprob launch: %s", hipGetErrorString((hipError_t)e));
    }
    return RTS_OK;
}

}  // namespace

namespace rts {

int set_error(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

void clear_last_error() { clear_error(); }

// rts_sample_tokens once its error state is cleared.  With get_ws, the
// workspace comes from it, asked only after every argument has been checked
// (so a refused call touches no device); `workspace` is then ignored.
int sample_tokens_impl(const float *logits, int64_t B, int64_t V, int64_t ld,
                       const rts_row_params *params,
                       const int32_t *history, int64_t H, int64_t ldh,
                       const int32_t *history_len,
                       int32_t *token, int32_t *counts, int32_t *kept_ids,
                       float *kept_logits, uint32_t *philox_x0,
                       uint64_t *counters, int64_t counter_stride,
                       const rts_logprob_request *lp, const rts_sample_extras *ex,
                       void *workspace, size_t ws_bytes, WorkspaceProvider get_ws,
                       hipStream_t stream)
{
    if (B < 0) return fail(RTS_EINVAL, "B = %lld < 0", (long long)B);
    if (B == 0) return RTS_OK;
    if (B >= 0x7FFFFFFFLL) return fail(RTS_EINVAL, "B = %lld too large", (long long)B);
    if (V <= 0 || V > RTS_MAX_V) return fail(RTS_EINVAL, "V = %lld outside 1..2^30", (long long)V);
    // ld = 0: every row reads logits row 0 (several parameter sets over one
    // distribution, e.g. several samples of one request)
    if (ld != 0 && ld < V)
        return fail(RTS_EINVAL, "ld = %lld is neither 0 nor >= V = %lld", (long long)ld, (long long)V);
    if (logits == nullptr) return fail(RTS_EINVAL, "logits is NULL");
    if (params == nullptr) return fail(RTS_EINVAL, "params is NULL");
    if (token == nullptr) return fail(RTS_EINVAL, "token is NULL");
    if (workspace == nullptr && get_ws == nullptr) return fail(RTS_EINVAL, "workspace is NULL");
    if (H < 0 || ldh < 0) return fail(RTS_EINVAL, "H = %lld, ldh = %lld", (long long)H, (long long)ldh);
    if (lp != nullptr) {
        if (lp->top_n < 0 || lp->top_n > RTS_MAX_TOP_N)
            return fail(RTS_EINVAL, "lp->top_n = %d outside 0..20", lp->top_n);
        if (lp->reserved != 0) return fail(RTS_EINVAL, "lp->reserved is not 0");
        if (lp->token_lp == nullptr) return fail(RTS_EINVAL, "lp->token_lp is NULL");
        if (lp->top_n > 0 && (lp->top_ids == nullptr || lp->top_lp == nullptr))
            return fail(RTS_EINVAL, "lp->top_ids / lp->top_lp are NULL with top_n = %d", lp->top_n);
        if (lp->allowed != nullptr) {
            if (lp->allowed_off == nullptr) return fail(RTS_EINVAL, "lp->allowed without allowed_off");
            if (lp->allowed_token_lp == nullptr)
                return fail(RTS_EINVAL, "lp->allowed_token_lp is NULL with lp->allowed");
            if (lp->top_n > 0 && (lp->allowed_top_ids == nullptr || lp->allowed_top_lp == nullptr))
                return fail(RTS_EINVAL, "lp->allowed_top_ids / allowed_top_lp are NULL with top_n = %d",
                            lp->top_n);
            if (const int e = check_offsets(B, lp->allowed_off, "lp->allowed_off")) return e;
        } else if (lp->allowed_off != nullptr || lp->allowed_token_lp != nullptr ||
                   lp->allowed_top_ids != nullptr || lp->allowed_top_lp != nullptr) {
            return fail(RTS_EINVAL, "lp->allowed_* outputs or offsets without lp->allowed");
        }
    }
    const int window = ex ? ex->window : 0;
    const int32_t *allowed = ex ? ex->allowed : nullptr;
    const int64_t *allowed_off = ex ? ex->allowed_off : nullptr;
    if (ex != nullptr) {
        if (ex->reserved != 0) return fail(RTS_EINVAL, "ex->reserved is not 0");
        if (window < 0 || window > rts::kRowsPerLaunch)
            return fail(RTS_EINVAL, "ex->window = %d outside 0..64", window);
        if (window > 0 && B % window != 0)
            return fail(RTS_EINVAL, "B = %lld is not a multiple of ex->window = %d", (long long)B,
                        window);
        if (window > 0 && (ex->draft == nullptr || ex->accepted == nullptr))
            return fail(RTS_EINVAL, "ex->draft / ex->accepted are NULL with window = %d", window);
        if (allowed != nullptr) {
            if (allowed_off == nullptr) return fail(RTS_EINVAL, "ex->allowed without allowed_off");
            if (const int e = check_offsets(B, allowed_off, "allowed_off")) return e;
            if (allowed_off[B] > 0x7FFFFFFFLL)
                return fail(RTS_EINVAL, "allowed_off[B] = %lld >= 2^31", (long long)allowed_off[B]);
        }
    }
    size_t need = 0;
    rts_workspace_bytes(B, V, &need);
    if (ws_bytes < need)
        return fail(RTS_ENOSPC, "workspace of %zu bytes, %zu needed", ws_bytes, need);

    // Logprobs renormalised over allowed lists: in the sampling launch itself
    // when no row also has a candidate list and every list is short enough;
    // else by the allowed-id logprob kernels after it, on the sampled tokens.
    const int32_t *lpa = lp ? lp->allowed : nullptr;
    const int64_t *lpa_off = lpa ? lp->allowed_off : nullptr;
    int64_t lpa_max = 0;
    bool lpa_fused = false;
    if (lpa != nullptr) {
        for (int64_t r = 0; r < B; ++r)
            if (lpa_off[r + 1] - lpa_off[r] > lpa_max) lpa_max = lpa_off[r + 1] - lpa_off[r];
        lpa_fused = allowed == nullptr && lpa_max <= rts::kRenormMax && lpa_off[B] <= 0x7FFFFFFFLL;
        if (!lpa_fused && lpa_max > rts::kRenormMax && !bitmap_fits(V)) return refuse_long_lists(V);
    }

    // Check every row before enqueuing anything.
    if (const int e = check_rows(B, params, history, H, ldh, history_len)) return e;
    if (get_ws != nullptr)
        if (const int e = get_ws(&workspace, stream)) return e;

    char *ws = static_cast<char *>(workspace);
    const rts::WsLayout L = rts::ws_layout(B < rts::kRowsPerLaunch ? B : rts::kRowsPerLaunch, V);
    // A launch covers whole verify windows.
    const int64_t per_launch = window > 0 ? (rts::kRowsPerLaunch / window) * window
                                          : rts::kRowsPerLaunch;
    for (int64_t r0 = 0; r0 < B; r0 += per_launch) {
        const int rows = (int)((B - r0) < per_launch ? (B - r0) : per_launch);
        const bool vec = is_vec_ok(logits + r0 * ld, ld);
        int ept = choose_ept(rows, V);
        // rows read element by element keep 4,096-element chunks: at 8,192 the
        // scalar-load variant spills registers
        if (!vec && ept > 16) ept = 16;
        rts::SampleArgs a;
        std::memset(&a, 0, sizeof a);
        a.logits = logits + r0 * ld;
        a.ld = ld;
        a.history = history;
        a.keys = reinterpret_cast<uint64_t *>(ws + L.keys);
        a.tickets = reinterpret_cast<uint32_t *>(ws);
        a.token = token + r0;
        a.counts = counts ? counts + 3 * r0 : nullptr;
        a.kept_ids = kept_ids ? kept_ids + rts::kMaxK * r0 : nullptr;
        a.kept_logits = kept_logits ? kept_logits + rts::kMaxK * r0 : nullptr;
        a.philox_x0 = philox_x0 ? philox_x0 + r0 : nullptr;
        a.counters = counters ? counters + r0 : nullptr;
        a.counter_stride = counter_stride;
        a.V = (int32_t)V;
        a.nchunks = (int32_t)chunks_for(V, ept);
        a.keys_stride = (int32_t)(rts::keys_bytes_per_row(V) / 8u);
        a.rows = rows;
        a.chunk_major = (ld == 0 && rows > 1) ? 1 : 0;
        a.early_xcds = rts::sample_work(rows, a.nchunks, 1, a.chunk_major) <= rts::kEarlyXcdWork ? 1 : 0;
        a.allowed = allowed;
        a.ignored = ex ? ex->ignored_ids : nullptr;
        if (window > 0) {
            a.window = window;
            a.draft = ex->draft + r0;
            a.accepted = ex->accepted + r0 / window;
            a.wtickets = reinterpret_cast<uint32_t *>(ws + 2 * rts::kTicketRegion);
        }
        if (lp != nullptr) {
            a.lp_on = 1;
            a.lp_topn = lp->top_n;
            a.raw_keys = reinterpret_cast<uint64_t *>(ws + L.raw);
            a.raw_stride = (int32_t)(rts::rawkeys_bytes_per_row(V) / 8u);
            a.partials = reinterpret_cast<uint64_t *>(ws + L.partials);
            a.partial_stride = (int32_t)rts::max_chunks(V);
            a.lp_token = lp->token_lp + r0;
            a.lp_ids = lp->top_n > 0 ? lp->top_ids + r0 * lp->top_n : nullptr;
            a.lp_top = lp->top_n > 0 ? lp->top_lp + r0 * lp->top_n : nullptr;
        }
        if (lpa != nullptr) {
            // rows without a list get the unrestricted values here; with the
            // allowed-id kernels, listed rows are overwritten after the launch
            a.lpa_token = lp->allowed_token_lp + r0;
            a.lpa_ids = lp->top_n > 0 ? lp->allowed_top_ids + r0 * lp->top_n : nullptr;
            a.lpa_top = lp->top_n > 0 ? lp->allowed_top_lp + r0 * lp->top_n : nullptr;
            // the first 8 bytes of each logprob ticket line: the row's exchange
            // word (zero between calls, like the tickets)
            a.lpa_w = reinterpret_cast<uint64_t *>(ws + rts::kTicketRegion);
            if (lpa_fused && lpa_max > 0) {
                a.allowed = lpa;
                a.lpa_blocks = rows;  // after the sampling grid, one per row
            }
        }
        for (int i = 0; i < rows; ++i) {
            if (a.lpa_blocks > 0) {
                const int64_t c = lpa_off[r0 + i + 1] - lpa_off[r0 + i];
                pack_row(a.row[i], params[r0 + i], V, history_len, ldh, (int32_t)lpa_off[r0 + i],
                         (int32_t)c);
                if (c > 0) a.row[i].pack |= rts::kPackRenorm;
            } else {
                pack_row(a.row[i], params[r0 + i], V, history_len, ldh,
                         allowed ? (int32_t)allowed_off[r0 + i] : 0,
                         allowed ? (int32_t)(allowed_off[r0 + i + 1] - allowed_off[r0 + i]) : 0);
            }
        }
        const int e = rts::launch_sample(a, ept, vec, stream);
        if (e != 0)
            return fail(RTS_EDEVICE, "sample launch (rows %lld..%lld): %s", (long long)r0,
                        (long long)(r0 + rows - 1), hipGetErrorString((hipError_t)e));
    }
    if (lpa != nullptr && !lpa_fused && lpa_max > 0)
        return enqueue_logprobs(logits, B, V, ld, token, lp->top_n, lpa, lpa_off,
                                lp->allowed_token_lp, lp->allowed_top_ids, lp->allowed_top_lp,
                                workspace, true, stream);
    return RTS_OK;
}

}  // namespace rts

extern "C" {

const char *rts_strerror(int code)
{
    switch (code) {
    case RTS_OK: return "ok";
    case RTS_EINVAL: return "invalid argument";
    case RTS_ENOSPC: return "workspace too small";
    case RTS_EDEVICE: return "HIP launch error";
    default: return "unknown error";
    }
}

const char *rts_last_error(void) { return g_last_error; }

int rts_workspace_bytes(int64_t B, int64_t V, size_t *bytes)
{
    clear_error();
    if (bytes == nullptr) return fail(RTS_EINVAL, "bytes is NULL");
    if (B < 0) return fail(RTS_EINVAL, "B = %lld < 0", (long long)B);
    if (V <= 0 || V > RTS_MAX_V) return fail(RTS_EINVAL, "V = %lld outside 1..2^30", (long long)V);
    const int64_t rows = B < rts::kRowsPerLaunch ? B : rts::kRowsPerLaunch;
    *bytes = rts::ws_layout(rows, V).total;
    return RTS_OK;
}

int rts_workspace_init(void *workspace, size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    if (workspace == nullptr) return fail(RTS_EINVAL, "workspace is NULL");
    if (ws_bytes < rts::kTicketBytes) return fail(RTS_ENOSPC, "workspace of %zu bytes", ws_bytes);
    const int e = rts::launch_zero_u32(static_cast<uint32_t *>(workspace),
                                       rts::kTicketBytes / 4u, stream);
    if (e != 0) return fail(RTS_EDEVICE, "zero kernel: %s", hipGetErrorString((hipError_t)e));
    return RTS_OK;
}

int rts_sample_tokens(const float *logits, int64_t B, int64_t V, int64_t ld,
                      const rts_row_params *params,
                      const int32_t *history, int64_t H, int64_t ldh,
                      const int32_t *history_len,
                      int32_t *token, int32_t *counts, int32_t *kept_ids,
                      float *kept_logits, uint32_t *philox_x0,
                      uint64_t *counters, int64_t counter_stride,
                      const rts_logprob_request *lp, const rts_sample_extras *ex,
                      void *workspace, size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    return rts::sample_tokens_impl(logits, B, V, ld, params, history, H, ldh, history_len, token,
                                   counts, kept_ids, kept_logits, philox_x0, counters,
                                   counter_stride, lp, ex, workspace, ws_bytes, nullptr, stream);
}

int rts_token_logprobs(const float *logits, int64_t B, int64_t V, int64_t ld,
                       const int32_t *tokens, int32_t top_n,
                       const int32_t *allowed, const int64_t *allowed_off,
                       float *token_lp, int32_t *top_ids, float *top_lp,
                       void *workspace, size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    if (B < 0) return fail(RTS_EINVAL, "B = %lld < 0", (long long)B);
    if (B == 0) return RTS_OK;
    if (B >= 0x7FFFFFFFLL) return fail(RTS_EINVAL, "B = %lld too large", (long long)B);
    if (V <= 0 || V > RTS_MAX_V) return fail(RTS_EINVAL, "V = %lld outside 1..2^30", (long long)V);
    if (ld < V) return fail(RTS_EINVAL, "ld = %lld < V = %lld", (long long)ld, (long long)V);
    if (logits == nullptr || tokens == nullptr || token_lp == nullptr)
        return fail(RTS_EINVAL, "logits, tokens and token_lp must not be NULL");
    if (top_n < 0 || top_n > RTS_MAX_TOP_N)
        return fail(RTS_EINVAL, "top_n = %d outside 0..20", top_n);
    if (top_n > 0 && (top_ids == nullptr || top_lp == nullptr))
        return fail(RTS_EINVAL, "top_ids / top_lp are NULL with top_n = %d", top_n);
    if (allowed != nullptr && allowed_off == nullptr)
        return fail(RTS_EINVAL, "allowed without allowed_off");
    if (workspace == nullptr) return fail(RTS_EINVAL, "workspace is NULL");
    size_t need = 0;
    rts_workspace_bytes(B, V, &need);
    if (ws_bytes < need)
        return fail(RTS_ENOSPC, "workspace of %zu bytes, %zu needed", ws_bytes, need);

    // Restricted rows: the bitmap kernels where V <= 2^19, else the hash-set
    // kernel, which takes lists of up to kRenormMax ids.
    if (allowed != nullptr) {
        if (const int e = check_offsets(B, allowed_off, "allowed_off")) return e;
        bool any_long = false;
        for (int64_t r = 0; r < B; ++r)
            if (allowed_off[r + 1] - allowed_off[r] > rts::kRenormMax) any_long = true;
        if (any_long && !bitmap_fits(V)) return refuse_long_lists(V);
    }
    return enqueue_logprobs(logits, B, V, ld, tokens, top_n, allowed, allowed_off, token_lp, top_ids,
                            top_lp, workspace, false, stream);
}

int rts_sample_tokens_prior(int design, const float *logits, int64_t B, int64_t V, int64_t ld,
                            const rts_row_params *params,
                            const int32_t *history, int64_t H, int64_t ldh,
                            const int32_t *history_len,
                            int32_t *token, int32_t *counts, int32_t *kept_ids,
                            float *kept_logits, uint32_t *philox_x0,
                            void *workspace, size_t ws_bytes, hipStream_t stream)
{
    clear_error();
    if (design < RTS_PRIOR_THREAD || design > RTS_PRIOR_RECOUNT)
        return fail(RTS_EINVAL, "design = %d outside 1..3", design);
    if (B < 0) return fail(RTS_EINVAL, "B = %lld < 0", (long long)B);
    if (B == 0) return RTS_OK;
    if (B >= 0x7FFFFFFFLL) return fail(RTS_EINVAL, "B = %lld too large", (long long)B);
    if (V <= 0 || V > (1 << 20)) return fail(RTS_EINVAL, "V = %lld out of (0, 2^20]", (long long)V);
    if (ld < V) return fail(RTS_EINVAL, "ld = %lld < V = %lld", (long long)ld, (long long)V);
    if (logits == nullptr || params == nullptr || token == nullptr || workspace == nullptr)
        return fail(RTS_EINVAL, "logits, params, token and workspace must not be NULL");
    if (H < 0 || ldh < 0) return fail(RTS_EINVAL, "H = %lld, ldh = %lld", (long long)H, (long long)ldh);
    size_t need = 0;
    rts_workspace_bytes(B, V, &need);
    if (ws_bytes < need)
        return fail(RTS_ENOSPC, "workspace of %zu bytes, %zu needed", ws_bytes, need);
    if (const int e = check_rows(B, params, history, H, ldh, history_len)) return e;
    // the row's penalty bitmap lives in LDS beside the selection's own
    const size_t lds = design == RTS_PRIOR_RECOUNT ? 0 : (size_t)((V + 31) / 32) * 4u;
    if (lds + rts::kAllowedStaticLds > max_lds_per_block())
        return fail(RTS_EINVAL, "V = %lld: the penalty bitmap does not fit in LDS", (long long)V);

    char *ws = static_cast<char *>(workspace);
    for (int64_t r0 = 0; r0 < B; r0 += rts::kRowsPerLaunch) {
        const int rows = (int)((B - r0) < rts::kRowsPerLaunch ? (B - r0) : rts::kRowsPerLaunch);
        rts::SampleArgs a;
        std::memset(&a, 0, sizeof a);
        a.logits = logits + r0 * ld;
        a.ld = ld;
        a.history = history;
        a.tickets = reinterpret_cast<uint32_t *>(ws);
        a.token = token + r0;
        a.counts = counts ? counts + 3 * r0 : nullptr;
        a.kept_ids = kept_ids ? kept_ids + rts::kMaxK * r0 : nullptr;
        a.kept_logits = kept_logits ? kept_logits + rts::kMaxK * r0 : nullptr;
        a.philox_x0 = philox_x0 ? philox_x0 + r0 : nullptr;
        a.V = (int32_t)V;
        a.rows = rows;
        for (int i = 0; i < rows; ++i) pack_row(a.row[i], params[r0 + i], V, history_len, ldh, 0, 0);
        const int e = rts::launch_prior(a, design, lds, stream);
        if (e != 0) return fail(RTS_EDEVICE, "prior-design launch: %s", hipGetErrorString((hipError_t)e));
    }
    return RTS_OK;
}

int rts_read_rows(const float *logits, int64_t B, int64_t V, int64_t ld, float *chunk_max,
                  hipStream_t stream)
{
    clear_error();
    if (B < 0) return fail(RTS_EINVAL, "B = %lld < 0", (long long)B);
    if (B == 0) return RTS_OK;
    if (B >= 0x7FFFFFFFLL) return fail(RTS_EINVAL, "B = %lld too large", (long long)B);
    if (V <= 0 || V > RTS_MAX_V) return fail(RTS_EINVAL, "V = %lld outside 1..2^30", (long long)V);
    if (ld < V) return fail(RTS_EINVAL, "ld = %lld < V = %lld", (long long)ld, (long long)V);
    if (logits == nullptr || chunk_max == nullptr)
        return fail(RTS_EINVAL, "logits and chunk_max must not be NULL");
    const int out_stride = (int)rts::max_chunks(V);
    for (int64_t r0 = 0; r0 < B; r0 += rts::kRowsPerLaunch) {
        const int rows = (int)((B - r0) < rts::kRowsPerLaunch ? (B - r0) : rts::kRowsPerLaunch);
        const bool vec = is_vec_ok(logits + r0 * ld, ld);
        int ept = choose_ept(rows, V);
        if (!vec && ept > 16) ept = 16;  // the sampler's chunking
        const int nchunks = (int)chunks_for(V, ept);
        const int e = rts::launch_read_rows(logits + r0 * ld, rows, (int)V, ld, nchunks, out_stride,
                                            chunk_max + r0 * out_stride, ept, vec,
                                            rows * nchunks <= rts::kEarlyXcdWork, stream);
        if (e != 0) return fail(RTS_EDEVICE, "read launch: %s", hipGetErrorString((hipError_t)e));
    }
    return RTS_OK;
}

}  // extern "C"
