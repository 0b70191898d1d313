// rts_select.h -- exact top-k selection building blocks for one workgroup.
//
// The selection of page "#19 serve: per-request temperature/top_p/top_k/
// min_p/penalties sampling" ("What changed", the one-block-per-token
// paragraph) is k argmax rounds over the row: the kept sequence is the k best
// (value, index) pairs, values descending, ties to the lowest index.  Here a
// row is split into chunks, one per workgroup, and each chunk is read from
// HBM once:
//   1. every lane keeps its elements in registers and takes their maximum;
//   2. t = the k-th largest of the 256 lane maxima is a lower bound of the
//      chunk's k-th value (k lanes each hold an element >= t);
//   3. the elements >= t (about k of them on smooth data) are compacted into
//      LDS with wavefront ballots, no atomics;
//   4. each survivor's rank among the survivors is counted; ranks < k are the
//      chunk's exact top-k in order.
// If a wave's LDS region overflows (massive ties, adversarial data), the
// chunk falls back to the pages' k argmax rounds, but over the register-
// resident chunk rather than over HBM.
#pragma once

#include "rts_device.h"

namespace rts {

constexpr int kCap = 128;  // LDS candidate slots per wave

struct SelectSmem {
    uint32_t lane_keys[kBlock];
    uint32_t wave_cnt[4];
    uint32_t flag;
    uint32_t pad;
    uint64_t red[4];
    uint64_t cand[4 * kCap];
    uint64_t sel[kMaxK];
    uint16_t part[4][4 * kCap];  // partial ranks, one row per wave
};

// Destinations of a selection: the workspace (device-coherent stores, read by
// another workgroup) or LDS.
struct ToWorkspace {
    uint64_t *p;
    __device__ void put(int i, uint64_t v) const { publish_u64(p + i, v); }
};
struct ToLds {
    uint64_t *p;
    __device__ void put(int i, uint64_t v) const { p[i] = v; }
};

// Each wave pads its region with zero keys up to a multiple of 8 (zero never
// outranks a real key), so the rank loop reads eight keys per step.
__device__ __forceinline__ void pad_region(SelectSmem &sm, int wave, uint32_t cnt)
{
    const int lane = lane_id();
    const uint32_t end = (cnt + 7u) & ~7u;
    if (cnt <= (uint32_t)kCap && cnt + (uint32_t)lane < end)
        sm.cand[wave * kCap + cnt + lane] = 0ull;
}

// Key at flat position f of the compacted candidates (regions in wave order).
__device__ __forceinline__ uint64_t cand_at(const SelectSmem &sm, const uint32_t (&cnt)[4],
                                            uint32_t f)
{
    uint32_t w = 0;
    if (f >= cnt[0]) {
        f -= cnt[0]; w = 1;
        if (f >= cnt[1]) {
            f -= cnt[1]; w = 2;
            if (f >= cnt[2]) { f -= cnt[2]; w = 3; }
        }
    }
    return sm.cand[w * kCap + f];
}

// Rank of every compacted candidate; writes the ones ranked below k to
// out[rank] and zero-fills out[n..k) when fewer survived.  Each wave counts,
// for every candidate, the larger keys in its own region only (eight LDS
// reads per step); a barrier later the four partial counts are summed.
// Requires every wave count <= kCap and padded regions.  Ends without a barrier.
template <typename Out>
__device__ __forceinline__ void rank_candidates(SelectSmem &sm, int k, Out out)
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const uint32_t cnt[4] = {sm.wave_cnt[0], sm.wave_cnt[1], sm.wave_cnt[2], sm.wave_cnt[3]};
    const uint32_t n = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    const uint64_t *cw = sm.cand + wave * kCap;
    const uint32_t end = (cnt[wave] + 7u) & ~7u;
    for (uint32_t f = lane; f < n; f += 64) {
        const uint64_t key = cand_at(sm, cnt, f);
        uint32_t r = 0;
        for (uint32_t j = 0; j < end; j += 8) {
            uint64_t c[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) c[u] = cw[j + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) r += (c[u] > key) ? 1u : 0u;
        }
        sm.part[wave][f] = (uint16_t)r;
    }
    __syncthreads();
    for (uint32_t f = tid; f < n; f += kBlock) {
        const uint32_t rank = (uint32_t)sm.part[0][f] + sm.part[1][f] + sm.part[2][f] + sm.part[3][f];
        if (rank < (uint32_t)k) out.put((int)rank, cand_at(sm, cnt, f));
    }
    for (int r = (int)n + tid; r < k; r += kBlock) out.put(r, 0ull);
}

__device__ __forceinline__ bool any_overflow(const SelectSmem &sm)
{
    return (sm.wave_cnt[0] > (uint32_t)kCap) | (sm.wave_cnt[1] > (uint32_t)kCap) |
           (sm.wave_cnt[2] > (uint32_t)kCap) | (sm.wave_cnt[3] > (uint32_t)kCap);
}

// Block-wide maximum of one u64 per thread.  Ends after a barrier.
__device__ __forceinline__ uint64_t block_max_u64(SelectSmem &sm, uint64_t v)
{
    v = lane_u64(wave_scan_max_u64(v), 63);
    if (lane_id() == 0) sm.red[threadIdx.x >> 6] = v;
    __syncthreads();
    uint64_t m = sm.red[0];
    m = sm.red[1] > m ? sm.red[1] : m;
    m = sm.red[2] > m ? sm.red[2] : m;
    m = sm.red[3] > m ? sm.red[3] : m;
    __syncthreads();
    return m;
}

// Chunk selection over register-resident values.  v[e] holds the (already
// transformed) value of element idx = base + (e/4)*1024 + tid*4 + e%4, or NaN
// for "no element".  Writes the chunk's top-k keys in order to out[0..k).
template <int EPT>
__device__ __forceinline__ void chunk_topk(SelectSmem &sm, const float (&v)[EPT], int64_t base,
                                           int k, uint64_t *out_keys)
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const ToWorkspace out{out_keys};

    float lmax = __builtin_nanf("");
#pragma unroll
    for (int e = 0; e < EPT; ++e) lmax = fmaxf(lmax, v[e]);

    if (k == 1) {
        // Argmax: the lane's first element equal to its maximum (elements are
        // in increasing index order), then a block maximum of the keys.
        int first = 0;
#pragma unroll
        for (int e = EPT - 1; e >= 0; --e) first = (v[e] == lmax) ? e : first;
        uint64_t key = 0;
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            if (e == first && lmax == lmax)
                key = cand_key(lmax, (uint32_t)(base + (e >> 2) * 1024 + tid * 4 + (e & 3)));
        key = block_max_u64(sm, key);
        if (tid == 0) out.put(0, key);
        return;
    }

    sm.lane_keys[tid] = (lmax != lmax) ? 0u : value_key(lmax);
    __syncthreads();

    const uint32_t lk[4] = {sm.lane_keys[lane], sm.lane_keys[lane + 64],
                            sm.lane_keys[lane + 128], sm.lane_keys[lane + 192]};
    const float tf = key_threshold(kth_largest_key_256<16>(lk, k));

    const uint64_t below = lanes_below_mask();
    uint64_t *wc = sm.cand + wave * kCap;
    uint32_t wcnt = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const bool c = v[e] >= tf;
        const uint64_t m = __ballot(c);
        if (m) {
            const uint32_t pos = wcnt + (uint32_t)__popcll(m & below);
            if (c && pos < (uint32_t)kCap)
                wc[pos] = cand_key(v[e], (uint32_t)(base + (e >> 2) * 1024 + tid * 4 + (e & 3)));
            wcnt += (uint32_t)__popcll(m);
        }
    }
    if (lane == 0) sm.wave_cnt[wave] = wcnt;
    pad_region(sm, wave, wcnt);
    __syncthreads();

    if (!any_overflow(sm)) {
        rank_candidates(sm, k, out);
        return;
    }
    // Fallback: k argmax rounds over the registers, each taking the best key
    // strictly below the previous pick.
    uint64_t prev = ~0ull;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            if (v[e] == v[e]) {
                const uint64_t key =
                    cand_key(v[e], (uint32_t)(base + (e >> 2) * 1024 + tid * 4 + (e & 3)));
                best = (key < prev && key > best) ? key : best;
            }
        }
        best = block_max_u64(sm, best);
        if (tid == 0) out.put(r, best);
        prev = best;
    }
}

// Top-k of a list of n published keys (0 = no element), written in order to
// sm.sel[0..k).  Used by the row merge.  The first kCache keys of every thread
// are loaded in one batch and kept in registers; longer lists are re-read in
// batches of the same size.  Ends after a barrier.
constexpr int kCache = 16;

__device__ __forceinline__ void load_batch(const uint64_t *list, int n, int first,
                                           uint64_t (&kv)[kCache])
{
#pragma unroll
    for (int i = 0; i < kCache; ++i) {
        const int f = first + i * kBlock + (int)threadIdx.x;
        kv[i] = (f < n) ? read_published_u64(list + f) : 0ull;
    }
}

__device__ __forceinline__ void list_topk(SelectSmem &sm, const uint64_t *list, int n, int k)
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    constexpr int kSpan = kCache * kBlock;

    uint64_t kr[kCache];
    load_batch(list, n, 0, kr);
    uint64_t lm = 0;
#pragma unroll
    for (int i = 0; i < kCache; ++i) lm = kr[i] > lm ? kr[i] : lm;
    for (int first = kSpan; first < n; first += kSpan) {
        uint64_t t[kCache];
        load_batch(list, n, first, t);
#pragma unroll
        for (int i = 0; i < kCache; ++i) lm = t[i] > lm ? t[i] : lm;
    }
    if (k == 1) {
        lm = block_max_u64(sm, lm);
        if (tid == 0) sm.sel[0] = lm;
        __syncthreads();
        return;
    }
    sm.lane_keys[tid] = (uint32_t)(lm >> 32);
    __syncthreads();
    const uint32_t lk[4] = {sm.lane_keys[lane], sm.lane_keys[lane + 64],
                            sm.lane_keys[lane + 128], sm.lane_keys[lane + 192]};
    const uint64_t t64 = (uint64_t)kth_largest_key_256<16>(lk, k) << 32;

    const uint64_t below = lanes_below_mask();
    uint64_t *wc = sm.cand + wave * kCap;
    uint32_t wcnt = 0;
    auto compact = [&](const uint64_t (&kv)[kCache]) {
#pragma unroll
        for (int i = 0; i < kCache; ++i) {
            const bool c = kv[i] != 0ull && kv[i] >= t64;
            const uint64_t m = __ballot(c);
            if (m) {
                const uint32_t pos = wcnt + (uint32_t)__popcll(m & below);
                if (c && pos < (uint32_t)kCap) wc[pos] = kv[i];
                wcnt += (uint32_t)__popcll(m);
            }
        }
    };
    compact(kr);
    for (int first = kSpan; first < n; first += kSpan) {
        uint64_t t[kCache];
        load_batch(list, n, first, t);
        compact(t);
    }
    if (lane == 0) sm.wave_cnt[wave] = wcnt;
    pad_region(sm, wave, wcnt);
    __syncthreads();

    if (!any_overflow(sm)) {
        rank_candidates(sm, k, ToLds{sm.sel});
        __syncthreads();
        return;
    }
    uint64_t prev = ~0ull;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
        for (int first = 0; first < n; first += kSpan) {
            uint64_t t[kCache];
            load_batch(list, n, first, t);
#pragma unroll
            for (int i = 0; i < kCache; ++i) best = (t[i] < prev && t[i] > best) ? t[i] : best;
        }
        best = block_max_u64(sm, best);
        if (tid == 0) sm.sel[r] = best;
        prev = best;
    }
    __syncthreads();
}

}  // namespace rts
