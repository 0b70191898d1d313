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
};

// Rank of every compacted candidate; writes the ones ranked below k to
// out[rank] (global or LDS) and zero-fills out[n..k) when fewer survived.
// Requires every wave count <= kCap.  Ends without a barrier.
template <typename OutT>
__device__ __forceinline__ void rank_candidates(SelectSmem &sm, int k, OutT *out)
{
    const int tid = threadIdx.x;
    const uint32_t c0 = sm.wave_cnt[0], c1 = sm.wave_cnt[1], c2 = sm.wave_cnt[2],
                   c3 = sm.wave_cnt[3];
    const uint32_t n = c0 + c1 + c2 + c3;
    for (uint32_t f = tid; f < n; f += kBlock) {
        uint32_t j = f, w = 0;
        if (j >= c0) {
            j -= c0; w = 1;
            if (j >= c1) {
                j -= c1; w = 2;
                if (j >= c2) { j -= c2; w = 3; }
            }
        }
        const uint64_t key = sm.cand[w * kCap + j];
        uint32_t rank = 0;
        const uint32_t cnt[4] = {c0, c1, c2, c3};
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            const uint64_t *cw = sm.cand + w2 * kCap;
            for (uint32_t j2 = 0; j2 < cnt[w2]; ++j2) rank += (cw[j2] > key) ? 1u : 0u;
        }
        if (rank < (uint32_t)k) out[rank] = (OutT)key;
    }
    for (int r = (int)n + tid; r < k; r += kBlock) out[r] = (OutT)0;
}

__device__ __forceinline__ bool any_overflow(const SelectSmem &sm)
{
    return (sm.wave_cnt[0] > (uint32_t)kCap) | (sm.wave_cnt[1] > (uint32_t)kCap) |
           (sm.wave_cnt[2] > (uint32_t)kCap) | (sm.wave_cnt[3] > (uint32_t)kCap);
}

// Block-wide maximum of one u64 per thread.  Ends after a barrier.
__device__ __forceinline__ uint64_t block_max_u64(SelectSmem &sm, uint64_t v)
{
    v = wave_max_u64(v);
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
                                           int k, uint64_t *out)
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;

    float lmax = __builtin_nanf("");
#pragma unroll
    for (int e = 0; e < EPT; ++e) lmax = fmaxf(lmax, v[e]);
    sm.lane_keys[tid] = (lmax != lmax) ? 0u : value_key(lmax);
    __syncthreads();

    const uint32_t lk[4] = {sm.lane_keys[lane], sm.lane_keys[lane + 64],
                            sm.lane_keys[lane + 128], sm.lane_keys[lane + 192]};
    const float tf = key_threshold(kth_largest_key_256<24>(lk, k));

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
        if (tid == 0) out[r] = best;
        prev = best;
    }
}

// Top-k of a list of n keys in global memory (0 = no element), written in
// order to sm.sel[0..k).  Used by the row merge.  Ends after a barrier.
__device__ __forceinline__ void list_topk(SelectSmem &sm, const uint64_t *list, int n, int k)
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int rounds = (n + kBlock - 1) / kBlock;

    uint64_t lm = 0;
    for (int i = 0; i < rounds; ++i) {
        const int f = tid + i * kBlock;
        if (f < n) {
            const uint64_t kv = list[f];
            lm = kv > lm ? kv : lm;
        }
    }
    sm.lane_keys[tid] = (uint32_t)(lm >> 32);
    __syncthreads();
    const uint32_t lk[4] = {sm.lane_keys[lane], sm.lane_keys[lane + 64],
                            sm.lane_keys[lane + 128], sm.lane_keys[lane + 192]};
    const uint64_t t64 = (uint64_t)kth_largest_key_256<32>(lk, k) << 32;

    const uint64_t below = lanes_below_mask();
    uint64_t *wc = sm.cand + wave * kCap;
    uint32_t wcnt = 0;
    for (int i = 0; i < rounds; ++i) {
        const int f = tid + i * kBlock;
        const uint64_t kv = (f < n) ? list[f] : 0ull;
        const bool c = kv != 0ull && kv >= t64;
        const uint64_t m = __ballot(c);
        if (m) {
            const uint32_t pos = wcnt + (uint32_t)__popcll(m & below);
            if (c && pos < (uint32_t)kCap) wc[pos] = kv;
            wcnt += (uint32_t)__popcll(m);
        }
    }
    if (lane == 0) sm.wave_cnt[wave] = wcnt;
    __syncthreads();

    if (!any_overflow(sm)) {
        rank_candidates(sm, k, sm.sel);
        __syncthreads();
        return;
    }
    uint64_t prev = ~0ull;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
        for (int i = 0; i < rounds; ++i) {
            const int f = tid + i * kBlock;
            if (f < n) {
                const uint64_t kv = list[f];
                best = (kv < prev && kv > best) ? kv : best;
            }
        }
        best = block_max_u64(sm, best);
        if (tid == 0) sm.sel[r] = best;
        prev = best;
    }
    __syncthreads();
}

}  // namespace rts
