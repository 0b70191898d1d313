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

// Chunk selection over register-resident values.  v[e] holds the value of
// element idx = base + (e/4)*1024 + tid*4 + e%4; ids >= V hold NaN.  Values
// may be raw: NaN stands for -inf and +inf for the largest float, and both
// are mapped when a key is formed.  Writes the chunk's top-k keys in order to
// out[0..k).
template <int EPT>
__device__ __forceinline__ uint32_t elem_index(int base, int e)
{
    return (uint32_t)(base + (e >> 2) * 1024 + (int)threadIdx.x * 4 + (e & 3));
}

template <int EPT>
__device__ __forceinline__ void chunk_topk(SelectSmem &sm, float (&v)[EPT], int base, int V, int k,
                                           uint64_t *out_keys)
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const ToWorkspace out{out_keys};
    constexpr float kFltMax = 3.40282346638528859812e+38f;

    // fmaxf skips NaN, so the lane maximum is over the non-NaN values.
    float lmax = __builtin_nanf("");
#pragma unroll
    for (int e = 0; e < EPT; ++e) lmax = fmaxf(lmax, v[e]);
    lmax = (lmax == lmax) ? fminf(lmax, kFltMax) : lmax;  // fminf would turn NaN into FLT_MAX

    if (k == 1) {
        // Argmax: the lane's first element equal to its maximum (elements are
        // in increasing index order), then a block maximum of the keys.
        // Lanes whose maximum is -inf or empty offer nothing here; if every
        // lane is like that the general path below handles the chunk.
        uint64_t key = 0;
        if (lmax == lmax && lmax > -INFINITY) {
            int first = 0;
#pragma unroll
            for (int e = EPT - 1; e >= 0; --e)
                first = (v[e] == v[e] && fminf(v[e], kFltMax) == lmax) ? e : first;
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (e == first) key = cand_key(lmax, elem_index<EPT>(base, e));
        }
        key = block_max_u64(sm, key);  // every thread of the block takes part
        if (key != 0ull) {
            if (tid == 0) out.put(0, key);
            return;
        }
    }

    sm.lane_keys[tid] = (lmax != lmax) ? 0u : value_key(lmax);
    __syncthreads();

    const uint32_t lk[4] = {sm.lane_keys[lane], sm.lane_keys[lane + 64],
                            sm.lane_keys[lane + 128], sm.lane_keys[lane + 192]};
    const float tf = key_threshold(kth_largest_key_256<16>(lk, k));
    if (tf == -INFINITY) {
        // Degenerate chunk (fewer than k values above -inf): every id below V
        // is a candidate, NaN counting as -inf.
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            v[e] = ((int)elem_index<EPT>(base, e) < V) ? sanitize(v[e]) : __builtin_nanf("");
    }

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
                wc[pos] = cand_key(fminf(v[e], kFltMax), elem_index<EPT>(base, e));
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
            const uint32_t idx = elem_index<EPT>(base, e);
            if ((int)idx < V) {
                const uint64_t key = cand_key(sanitize(v[e]), idx);
                best = (key < prev && key > best) ? key : best;
            }
        }
        best = block_max_u64(sm, best);
        if (tid == 0) out.put(r, best);
        prev = best;
    }
}

// Row merge: top-k of the chunk lists, written in order to sm.sel[0..k).
// Chunk c published its top-k keys in descending order at list[c*k ..
// c*k + k), zero-padded.  The lists are read as sorted streams: with C <= 256
// chunks, lane (c, g) owns chunk c's ranks g, g + G, g + 2G, ... where
// G = 256 / C, so the lane's maximum is its first key and the 256 lane maxima
// are the top ranks of every chunk; the k-th largest of them is then close to
// the row's k-th key.  With more chunks each lane owns whole chunks t, t + 256,
// ...  A lane stops reading a stream at its first key below the threshold.
// Loads are device-coherent and issued eight at a time.  Ends after a barrier.
constexpr int kBatch = 8;

struct MergeStreams {
    int G;        // rank stride inside a stream
    int g;        // first rank
    int c0;       // first chunk of the lane
    int cstride;  // chunk stride between the lane's streams
    int nstreams; // streams of this lane
    int max_streams;
};

__device__ __forceinline__ MergeStreams merge_streams(int C, int k)
{
    const int t = threadIdx.x;
    MergeStreams m;
    if (C <= kBlock) {
        m.G = kBlock / C;
        m.g = t / C;
        m.c0 = t % C;
        m.cstride = 0;
        m.nstreams = (t < m.G * C && m.g < k) ? 1 : 0;
        m.max_streams = 1;
    } else {
        m.G = 1;
        m.g = 0;
        m.c0 = t;
        m.cstride = kBlock;
        m.nstreams = (C - t + kBlock - 1) / kBlock;
        m.max_streams = (C + kBlock - 1) / kBlock;
    }
    return m;
}

__device__ __forceinline__ void load_stream_batch(const uint64_t *list, int k, const MergeStreams &m,
                                                  int c, bool has, int j0, uint64_t (&kv)[kBatch])
{
    const int L = (k - m.g + m.G - 1) / m.G;  // keys in the stream
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const int j = j0 + u;
        kv[u] = (has && j < L) ? read_published_u64(list + (int64_t)c * k + m.g + m.G * j) : 0ull;
    }
}

__device__ __forceinline__ void list_topk(SelectSmem &sm, const uint64_t *list, int C, int k)
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const MergeStreams ms = merge_streams(C, k);

    // pass 1: the first batch of the first stream (kept), heads of the others
    uint64_t first[kBatch];
    load_stream_batch(list, k, ms, ms.c0, ms.nstreams > 0, 0, first);
    uint64_t lm = first[0];
    for (int si = 1; si < ms.max_streams; ++si) {
        const int c = ms.c0 + si * ms.cstride;
        if (si < ms.nstreams) {
            const uint64_t h = read_published_u64(list + (int64_t)c * k);
            lm = h > lm ? h : lm;
        }
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

    // pass 2: walk every stream while its keys reach the threshold
    const uint64_t below = lanes_below_mask();
    uint64_t *wc = sm.cand + wave * kCap;
    uint32_t wcnt = 0;
    for (int si = 0; si < ms.max_streams; ++si) {
        const int c = ms.c0 + si * ms.cstride;
        bool live = si < ms.nstreams;
        for (int j0 = 0; __ballot(live) != 0ull; j0 += kBatch) {
            uint64_t kv[kBatch];
            if (si == 0 && j0 == 0) {
#pragma unroll
                for (int u = 0; u < kBatch; ++u) kv[u] = first[u];
            } else {
                load_stream_batch(list, k, ms, c, live, j0, kv);
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const bool cnd = live && kv[u] != 0ull && kv[u] >= t64;
                const uint64_t m = __ballot(cnd);
                if (m) {
                    const uint32_t pos = wcnt + (uint32_t)__popcll(m & below);
                    if (cnd && pos < (uint32_t)kCap) wc[pos] = kv[u];
                    wcnt += (uint32_t)__popcll(m);
                }
            }
            // descending stream: it ends at its first key below the threshold
            live = live && kv[kBatch - 1] != 0ull && kv[kBatch - 1] >= t64;
        }
    }
    if (lane == 0) sm.wave_cnt[wave] = wcnt;
    pad_region(sm, wave, wcnt);
    __syncthreads();

    if (!any_overflow(sm)) {
        rank_candidates(sm, k, ToLds{sm.sel});
        __syncthreads();
        return;
    }
    // Fallback (massive ties): k argmax rounds over the whole list.
    const int n = C * k;
    uint64_t prev = ~0ull;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
        for (int f0 = 0; f0 < n; f0 += kBatch * kBlock) {
            uint64_t t[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int f = f0 + u * kBlock + tid;
                t[u] = (f < n) ? read_published_u64(list + f) : 0ull;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) best = (t[u] < prev && t[u] > best) ? t[u] : best;
        }
        best = block_max_u64(sm, best);
        if (tid == 0) sm.sel[r] = best;
        prev = best;
    }
    __syncthreads();
}

}  // namespace rts
