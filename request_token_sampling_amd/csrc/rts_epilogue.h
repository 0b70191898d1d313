// rts_epilogue.h -- device code shared by the sampling kernels: the penalty
// of one id, the cuts and the draw on a merged kept sequence, and the
// verify-window acceptance.
#pragma once

#include "rts_select.h"

namespace rts {

constexpr int kPackedWindow = 33;  // windows this long or shorter take window_step_packed

// What the row's merging workgroup writes through, read from the kernel's
// argument block in one place.  The compiler otherwise issues a scalar load
// of each pointer next to its first store and waits for it there, so the
// tail of every row paid about nine scalar round trips one after another;
// read while the merge's loads are in flight and held in registers (the
// empty asm makes each value opaque, so it is not re-read at its use), they
// cost nothing on the tail.
// (The pointers carry the global address space: made opaque, they would
// otherwise lose it and every store would take the flat path.)
#define RTS_GLOBAL __attribute__((address_space(1)))
struct RowOut {
    RTS_GLOBAL int32_t *token;
    RTS_GLOBAL int32_t *counts;
    RTS_GLOBAL int32_t *kept_ids;
    RTS_GLOBAL float *kept_logits;
    RTS_GLOBAL uint32_t *philox_x0;
    RTS_GLOBAL uint64_t *counters;
    int64_t counter_stride;
    RTS_GLOBAL uint32_t *tickets;
    RTS_GLOBAL const int32_t *draft;
    RTS_GLOBAL int32_t *accepted;
    RTS_GLOBAL uint32_t *wtickets;
    int32_t window;
};

__device__ __forceinline__ RowOut row_out(const SampleArgs &a)
{
    RowOut o{(RTS_GLOBAL int32_t *)a.token,        (RTS_GLOBAL int32_t *)a.counts,
             (RTS_GLOBAL int32_t *)a.kept_ids,     (RTS_GLOBAL float *)a.kept_logits,
             (RTS_GLOBAL uint32_t *)a.philox_x0,   (RTS_GLOBAL uint64_t *)a.counters,
             a.counter_stride,                     (RTS_GLOBAL uint32_t *)a.tickets,
             (RTS_GLOBAL const int32_t *)a.draft,  (RTS_GLOBAL int32_t *)a.accepted,
             (RTS_GLOBAL uint32_t *)a.wtickets,    a.window};
    asm volatile("" : "+s"(o.token), "+s"(o.counts), "+s"(o.kept_ids), "+s"(o.kept_logits),
                      "+s"(o.philox_x0), "+s"(o.counters), "+s"(o.counter_stride));
    asm volatile("" : "+s"(o.tickets), "+s"(o.draft), "+s"(o.accepted), "+s"(o.wtickets),
                      "+s"(o.window));
    return o;
}

// llama.cpp-style penalty of an id seen c > 0 times in the window: the repeat
// penalty divides a positive logit and multiplies a non-positive one, the
// frequency term scales with the count and the presence term is charged once.
// Every operation is rounded to fp32 (the build disables contraction).
__device__ __forceinline__ float penalize(float v, uint32_t c, float rep, float freq,
                                          float present)
{
    v = (v <= 0.0f) ? v * rep : v / rep;
    float t = (float)c * freq;
    t = t + present;
    v = v - t;
    return sanitize(v);
}

// Verify windows (page "#19 ...", "What changed": the emitted tokens are the
// target's own samples; page "#559 ...", "Not done (yet)": a sampled row is
// accepted when its pick equals the draft).  Run by wave 0 of a row's merging
// workgroup once the row's token is known: the window's last row to get here
// counts the leading rows whose token equals their draft and writes the
// number of tokens the window emits (the first mismatch among all rows but
// the last, plus one; the window's size when there is none).
//
// Windows of up to 33 rows: each row adds 2^32 (one arrival) plus, if its
// token equals its draft, 2^r (r its place; the last row's bit is never
// read) to the window's 64-bit word with one device-scope atomic, so the
// last arrival reads every row's outcome from the value the atomic returns;
// no token is published and nothing else is read.
__device__ __forceinline__ void window_step_packed(const RowOut &a, int slot, int32_t tok,
                                                   int32_t draft)
{
    if (lane_id() != 0) return;
    const int w = slot / a.window, r = slot - w * a.window;
    const uint64_t add = (1ull << 32) | ((r < a.window - 1 && tok == draft) ? (1ull << r) : 0ull);
    RTS_GLOBAL uint64_t *word = reinterpret_cast<RTS_GLOBAL uint64_t *>(&a.wtickets[w * kTicketStride]);
    const uint64_t old =
        __hip_atomic_fetch_add(word, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((old >> 32) != (uint64_t)(a.window - 1)) return;
    const uint32_t rows = (uint32_t)(a.window - 1);  // rows whose match decides
    const uint32_t span = rows >= 32u ? 0xFFFFFFFFu : ((1u << rows) - 1u);
    const uint32_t miss = ~(uint32_t)(old + add) & span;
    a.accepted[w] = miss ? __ffs(miss) : a.window;
    __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next launch
}

// Longer windows: the row's token is published, then a ticket, and the last
// row reads every row's token back.
__device__ __forceinline__ void window_step(const RowOut &a, int slot, int32_t tok)
{
    const int lane = lane_id();
    const int w = slot / a.window;
    uint32_t last = 0u;
    if (lane == 0) {
        wait_stores_complete();
        const uint32_t old = __hip_atomic_fetch_add(&a.wtickets[w * kTicketStride], 1u,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = (old == (uint32_t)a.window - 1u) ? 1u : 0u;
    }
    if (lane_u32(last, 0) == 0u) return;
    const int r0 = w * a.window;
    bool miss = false;
    if (lane < a.window - 1) {
        const int32_t t = (r0 + lane == slot) ? tok
                          : __hip_atomic_load(&a.token[r0 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        miss = t != a.draft[r0 + lane];
    }
    const uint64_t b = __ballot(miss);
    if (lane == 0) {
        a.accepted[w] = b ? __ffsll((unsigned long long)b) : a.window;
        a.wtickets[w * kTicketStride] = 0u;
    }
}

// The cuts and the draw, run by wave 0 of the row's last workgroup on the
// merged kept sequence sm.sel[0..k).  Leaves the sampled token in sm.flag.
__device__ __forceinline__ void epilogue(const RowOut &a, const SampleRow &R, SelectSmem &sm,
                                         int slot, int k, bool greedy, uint64_t ctr, uint32_t x0)
{
    const int lane = lane_id();
    // a verify window's draft for this row, loaded now so the cuts hide it
    const int32_t draft = (a.window > 0 && a.window <= kPackedWindow) ? a.draft[slot] : 0;
    const uint64_t key = (lane < k) ? sm.sel[lane] : 0ull;
    const bool valid = key != 0ull;
    const int32_t id = valid ? (int32_t)key_index(key) : -1;
    const float y = valid ? key_logit(key) : -INFINITY;
    if (a.kept_ids) a.kept_ids[(int64_t)slot * kMaxK + lane] = id;
    if (a.kept_logits) a.kept_logits[(int64_t)slot * kMaxK + lane] = y;
    // The kept sequence holds k keys, or fewer when a row's allowed ids are
    // fewer than k (zero keys sort last); an empty one samples nothing.
    k = __popcll(__ballot(valid));

    const float y0 = lane_f32(y, 0);
    int m = k > 0 ? 1 : 0, n = m, pick = 0;
    if (!greedy && k > 0) {
        // min_p: keep the prefix with logit >= head + logf(min_p), in fp32.
        const float thr = y0 + R.lnp;
        m = __popcll(__ballot(lane < k && y >= thr));
        m = m < 1 ? 1 : m;
        // The weights are fp64 exponentials of y - y0: untempered for top_p,
        // tempered for the draw.  Each is computed only where it can be used
        // (top_p < 1; more than one min_p survivor), both before the cuts so
        // the two chains overlap, and a temperature of 1 reuses the
        // untempered one (dy / 1 is dy exactly).
        const double dy = (double)y - (double)y0;
        const bool head_masked = (y0 == -INFINITY);
        const bool use_top_p = !head_masked && !(R.top_p >= 1.0f);
        const bool same_w = use_top_p && R.temperature == 1.0f;
        double d = 0.0, w = 0.0;
        if (use_top_p) d = (lane < m) ? exp(dy) : 0.0;
        if (!head_masked && m > 1 && !same_w) w = (lane < m) ? exp(dy / (double)R.temperature) : 0.0;
        // top_p: shortest prefix of the min_p survivors whose fp64 softmax
        // mass reaches top_p; a masked head (-inf) keeps one candidate.
        // Both inclusive scans run before the top_p cut is known, so their
        // chains overlap: lane j of a DPP scan only adds lanes below it, so
        // the tempered sums of the lanes below the cut are the same whether
        // the lanes past it hold their weights or zeros; with a temperature
        // of 1 the draw reuses the untempered scan.
        double Sd = 0.0, Sw = 0.0;
        if (use_top_p) Sd = wave_scan_f64(lane < m ? d : 0.0);
        if (!head_masked && m > 1 && !same_w) Sw = wave_scan_f64(w);  // w is 0 past m
        n = m;
        if (head_masked) {
            n = 1;
        } else if (use_top_p) {
            const double Z = lane_f64(Sd, m - 1);
            const uint64_t b = __ballot(lane < m && Sd / Z >= (double)R.top_p);
            n = b ? __ffsll((unsigned long long)b) : m;
        }
        // temperature, then the draw: u = x0 / 2^32 against the tempered CDF.
        const double u = (double)x0 * (1.0 / 4294967296.0);
        pick = n - 1;
        if (n > 1) {
            const double S = same_w ? Sd : Sw;
            const double Z = lane_f64(S, n - 1);
            const uint64_t b = __ballot(lane < n - 1 && S / Z > u);
            if (b) pick = __ffsll((unsigned long long)b) - 1;
        }
    }
    const int32_t tok = lane_i32(id, pick);
    if (lane == 0) {
        sm.flag = (uint32_t)tok;
        if (a.window > kPackedWindow)  // read by the window's last row
            __hip_atomic_store(&a.token[slot], tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else a.token[slot] = tok;
        if (a.counts) {
            a.counts[3 * (int64_t)slot + 0] = k;
            a.counts[3 * (int64_t)slot + 1] = m;
            a.counts[3 * (int64_t)slot + 2] = n;
        }
        if (a.philox_x0) a.philox_x0[slot] = x0;
        if (a.counters) a.counters[slot] = ctr + (uint64_t)a.counter_stride;
        a.tickets[slot * kTicketStride] = 0u;  // ready for the next launch on this workspace
    }
    if (a.window > kPackedWindow) window_step(a, slot, tok);
    else if (a.window > 0) window_step_packed(a, slot, tok, draft);
}

// The same for callers that have not read the outputs ahead.
__device__ __forceinline__ void epilogue(const SampleArgs &a, const SampleRow &R, SelectSmem &sm,
                                         int slot, int k, bool greedy, uint64_t ctr, uint32_t x0)
{
    epilogue(row_out(a), R, sm, slot, k, greedy, ctr, x0);
}

}  // namespace rts
