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

constexpr int kCap = 128;          // LDS candidate slots per wave
constexpr int kRegion = kCap + 8;  // region stride; the extra slots absorb overflowing writes

struct SelectSmem {
    uint32_t lane_keys[kBlock];
    uint32_t wave_cnt[4];
    uint32_t flag;
    uint32_t thr;  // a chunk selection's threshold key, broadcast by wave 0
    uint64_t red[4];
    uint64_t cand[4 * kRegion];
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

// A set of compacted candidates: four per-wave regions of up to kCap keys and
// their counts.  The selection's own set lives in SelectSmem; a kernel that
// keeps a second selection open at the same time brings another.
struct Cands {
    uint64_t *keys;  // [4 * kRegion], region w at w * kRegion
    uint32_t *cnt;   // [4]
};

__device__ __forceinline__ Cands own_cands(SelectSmem &sm) { return Cands{sm.cand, sm.wave_cnt}; }

// Regions are padded with zero keys (zero never outranks a real key) to a
// multiple of kPad, so the rank loop reads kPad keys per step.
constexpr uint32_t kPad = 8;

__device__ __forceinline__ uint32_t padded(uint32_t cnt) { return (cnt + kPad - 1u) & ~(kPad - 1u); }

__device__ __forceinline__ void pad_region(Cands cd, int wave, uint32_t cnt)
{
    const int lane = lane_id();
    if (cnt <= (uint32_t)kCap && cnt + (uint32_t)lane < padded(cnt))
        cd.keys[wave * kRegion + cnt + lane] = 0ull;
}

// Key at flat position f of the compacted candidates (regions in wave order).
__device__ __forceinline__ uint64_t cand_at(const uint64_t *keys, const uint32_t (&cnt)[4], uint32_t f)
{
    uint32_t w = 0;
    if (f >= cnt[0]) {
        f -= cnt[0]; w = 1;
        if (f >= cnt[1]) {
            f -= cnt[1]; w = 2;
            if (f >= cnt[2]) { f -= cnt[2]; w = 3; }
        }
    }
    return keys[w * kRegion + f];
}

// Rank of every compacted candidate; writes the ones ranked below k to
// out[rank] and zero-fills out[n..k) when fewer survived.  Each wave counts,
// for every candidate, the larger keys in its own region only (kPad LDS
// reads per step, shared by two candidates per lane); a barrier later the
// four partial counts (sm.part) are summed.  Requires every wave count <= kCap and padded regions.  Ends
// without a barrier.
template <typename Out>
__device__ __forceinline__ void rank_candidates(SelectSmem &sm, Cands cd, int k, Out out)
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const uint32_t cnt[4] = {cd.cnt[0], cd.cnt[1], cd.cnt[2], cd.cnt[3]};
    const uint32_t n = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    const uint64_t *cw = cd.keys + wave * kRegion;
    const uint32_t end = padded(cnt[wave]);
    // two candidates per lane and pass, so up to 128 take one pass over the region
    for (uint32_t f = lane; f < n; f += 128) {
        const bool two = f + 64 < n;
        const uint64_t key0 = cand_at(cd.keys, cnt, f);
        const uint64_t key1 = two ? cand_at(cd.keys, cnt, f + 64) : ~0ull;
        uint32_t r0 = 0, r1 = 0;
        for (uint32_t j = 0; j < end; j += kPad) {
            uint64_t c[kPad];
#pragma unroll
            for (uint32_t u = 0; u < kPad; ++u) c[u] = cw[j + u];
#pragma unroll
            for (uint32_t u = 0; u < kPad; ++u) {
                r0 += (c[u] > key0) ? 1u : 0u;
                r1 += (c[u] > key1) ? 1u : 0u;
            }
        }
        sm.part[wave][f] = (uint16_t)r0;
        if (two) sm.part[wave][f + 64] = (uint16_t)r1;
    }
    __syncthreads();
    for (uint32_t f = tid; f < n; f += kBlock) {
        const uint32_t rank = (uint32_t)sm.part[0][f] + sm.part[1][f] + sm.part[2][f] + sm.part[3][f];
        if (rank < (uint32_t)k) out.put((int)rank, cand_at(cd.keys, cnt, f));
    }
    for (int r = (int)n + tid; r < k; r += kBlock) out.put(r, 0ull);
}

// n <= 128 compacted candidates, sorted by the calling wave alone: lane l
// returns the key of rank l (zero past n).
__device__ __forceinline__ uint64_t wave_sorted_candidates(const uint64_t *keys,
                                                          const uint32_t (&cnt)[4])
{
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t n = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    uint64_t x0 = lane < n ? cand_at(keys, cnt, lane) : 0ull;
    uint64_t x1 = lane + 64u < n ? cand_at(keys, cnt, lane + 64u) : 0ull;
    if (n > 64u) wave_sort_desc<true>(x0, x1);
    else wave_sort_desc<false>(x0, x1);
    return x0;
}

__device__ __forceinline__ bool any_overflow(Cands cd)
{
    return (cd.cnt[0] > (uint32_t)kCap) | (cd.cnt[1] > (uint32_t)kCap) |
           (cd.cnt[2] > (uint32_t)kCap) | (cd.cnt[3] > (uint32_t)kCap);
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

// Id of register element e of the calling thread in the chunk at `base`:
// the chunk is read as EPT/4 coalesced passes of 1,024 ids, four per lane.
template <int EPT>
__device__ __forceinline__ uint32_t elem_index(int base, int e)
{
    return (uint32_t)(base + (e >> 2) * 1024 + (int)threadIdx.x * 4 + (e & 3));
}

// First half of a chunk selection: the threshold (the k-th largest of the
// 256 lane maxima) and the ballot compaction of every value at or above it
// into cd, whose regions are padded; ends after a barrier.  For k = 1 the
// argmax is written to out[0] directly and true is returned (nothing left to
// do); otherwise returns false.  In the degenerate case (fewer than k values
// above -inf) every id below V is a candidate and v is sanitised in place;
// with nan_absent, a NaN marks an id outside the row's candidate set (the
// caller has sanitised the others) and stays excluded.
template <int EPT, typename Out, bool COARSE = true>
__device__ __forceinline__ bool chunk_compact(SelectSmem &sm, float (&v)[EPT], int base, int V,
                                              int k, Cands cd, Out out, bool nan_absent = false)
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
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
            return true;
        }
    }

    sm.lane_keys[tid] = (lmax != lmax) ? 0u : value_key(lmax);
    __syncthreads();
    // One wave finds the threshold; the others would only repeat its work.
    if (wave == 0) {
        const uint32_t lk[4] = {sm.lane_keys[lane], sm.lane_keys[lane + 64],
                                sm.lane_keys[lane + 128], sm.lane_keys[lane + 192]};
        // COARSE = false (the fused-logprob variant, at its register limit):
        // the two-key search alone, without the rerun that would spill; a
        // sparse chunk it misjudges takes the degenerate path, still exact.
        const uint32_t t = COARSE ? selection_threshold(lk, k) : kth_largest_group_max<16, 2>(lk, k);
        if (lane == 0) sm.thr = t;
    }
    __syncthreads();
    const float tf = key_threshold(sm.thr);
    if (tf == -INFINITY) {
        // Degenerate chunk (fewer than k values above -inf): every id below V
        // is a candidate, NaN counting as -inf (unless it marks an absent id).
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            v[e] = ((int)elem_index<EPT>(base, e) < V && (!nan_absent || v[e] == v[e]))
                       ? sanitize(v[e]) : __builtin_nanf("");
    }

    // Ballot compaction of the raw entries (float bits, id): the slot is the
    // wave's running count plus the lanes below that also pass; slots past
    // kCap land in the region's spare slots (the region has then overflowed
    // and its contents are not used).
    uint64_t *wc = cd.keys + wave * kRegion;
    const uint32_t ibase = (uint32_t)(base + tid * 4);
    uint32_t wcnt = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const bool c = v[e] >= tf;
        const uint64_t m = __ballot(c);
        if (m) {
            uint32_t pos = wcnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            pos = pos < (uint32_t)kCap ? pos : (uint32_t)kCap;
            const uint32_t idx = ibase + (uint32_t)((e >> 2) * 1024 + (e & 3));
            if (c) wc[pos] = ((uint64_t)__float_as_uint(v[e]) << 32) | idx;
            wcnt += (uint32_t)__popcll(m);
        }
    }
    if (lane == 0) cd.cnt[wave] = wcnt;
    // The wave turns its own entries into keys and pads the region with zero
    // keys to a multiple of kPad; one wave's LDS accesses stay in order, so
    // this needs no workgroup barrier.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t nk = wcnt < (uint32_t)kCap ? wcnt : (uint32_t)kCap;
    const uint32_t end = padded(nk);
    for (uint32_t j = (uint32_t)lane; j < end; j += 64) {
        uint64_t key = 0ull;
        if (j < nk) {
            const uint64_t r = wc[j];
            key = cand_key(fminf(__uint_as_float((uint32_t)(r >> 32)), kFltMax), (uint32_t)r);
        }
        wc[j] = key;
    }
    __syncthreads();
    return false;
}

// Second half: rank the compacted candidates, or, when a wave region
// overflowed (massive ties), k argmax rounds over the register values, each
// taking the best key strictly below the previous pick.  Uses sm.part, so a
// barrier must separate it from the tail of an earlier rank.
template <int EPT, typename Out>
__device__ __forceinline__ void chunk_finish(SelectSmem &sm, const float (&v)[EPT], int base, int V,
                                             int k, Cands cd, Out out, bool nan_absent = false)
{
    const int tid = threadIdx.x;
    if (!any_overflow(cd)) {
        const uint32_t cnt[4] = {cd.cnt[0], cd.cnt[1], cd.cnt[2], cd.cnt[3]};
        if (cnt[0] + cnt[1] + cnt[2] + cnt[3] <= 128u) {
            // few candidates: wave 0 sorts them alone and writes the top k
            if ((tid >> 6) == 0) {
                const uint64_t key = wave_sorted_candidates(cd.keys, cnt);
                if (lane_id() < k) out.put(lane_id(), key);
            }
            return;
        }
        rank_candidates(sm, cd, k, out);
        return;
    }
    uint64_t prev = ~0ull;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const uint32_t idx = elem_index<EPT>(base, e);
            if ((int)idx < V && (!nan_absent || v[e] == v[e])) {
                const uint64_t key = cand_key(sanitize(v[e]), idx);
                best = (key < prev && key > best) ? key : best;
            }
        }
        best = block_max_u64(sm, best);
        if (tid == 0) out.put(r, best);
        prev = best;
    }
}

// Chunk selection over register-resident values.  v[e] holds the value of
// element idx = base + (e/4)*1024 + tid*4 + e%4; ids >= V hold NaN.  Values
// may be raw: NaN stands for -inf and +inf for the largest float, and both
// are mapped when a key is formed.  Writes the chunk's top-k keys in order to
// out_keys[0..k) with device-coherent stores.  Ends without a barrier.
template <int EPT, bool COARSE = true>
__device__ __forceinline__ void chunk_topk(SelectSmem &sm, float (&v)[EPT], int base, int V, int k,
                                           uint64_t *out_keys, bool nan_absent = false)
{
    const ToWorkspace out{out_keys};
    if (chunk_compact<EPT, ToWorkspace, COARSE>(sm, v, base, V, k, own_cands(sm), out, nan_absent)) return;
    chunk_finish<EPT>(sm, v, base, V, k, own_cands(sm), out, nan_absent);
}

// Row merge: top-k of the chunk lists, written in order to sm.sel[0..k).
// Chunk c published its top-k keys in descending order at list[c*k ..
// c*k + k), zero-padded.  The lists are read as sorted streams: with C <= 256
// chunks, lane (c, g) owns chunk c's ranks g, g + G, g + 2G, ... where
// G = 256 / C, so the lane's maximum is its first key and the 256 lane maxima
// are the top ranks of every chunk; the k-th largest of them is then close to
// the row's k-th key.  With more chunks each lane owns whole chunks t, t + 256,
// ...  A lane stops reading a stream at its first key below the threshold.
// Loads are device-coherent and issued kBatch (two) at a time.  Past the
// threshold a stream rarely keeps more than its head (a 20-key list over 31
// chunks has 3 keys per stream, ~23 of the 620 survive), so short batches
// leave few empty compaction steps; a stream that does continue costs one
// more round trip per batch (measured on MI355X: batches of 2 against 4,
// 1-row step -1 %, 5-row window -3.5 %; 4 against 8, -2.5 % and -2 %).
// The threshold is a
// lower bound from selection_threshold, so a few more keys than k survive.
// On return sm.sel is valid in wave 0 (in every wave only when the call
// ended with a barrier, which callers must not rely on).
constexpr int kBatch = 2;

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

struct NoWork {
    __device__ void operator()() const {}
};

// `overlap` runs once the first loads are in flight, so independent work of
// the caller hides behind their latency.
template <typename Overlap = NoWork>
__device__ __forceinline__ void list_topk(SelectSmem &sm, const uint64_t *list, int C, int k,
                                          Overlap overlap = NoWork{})
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const MergeStreams ms = merge_streams(C, k);

    // pass 1: the first batch of the first stream (kept), heads of the others
    uint64_t first[kBatch];
    load_stream_batch(list, k, ms, ms.c0, ms.nstreams > 0, 0, first);
    overlap();
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
    const uint64_t t64 = (uint64_t)selection_threshold(lk, k) << 32;

    // pass 2: walk every stream while its keys reach the threshold
    const uint64_t below = lanes_below_mask();
    uint64_t *wc = sm.cand + wave * kRegion;
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
    pad_region(own_cands(sm), wave, wcnt);
    __syncthreads();

    if (!any_overflow(own_cands(sm))) {
        const uint32_t cnt[4] = {sm.wave_cnt[0], sm.wave_cnt[1], sm.wave_cnt[2], sm.wave_cnt[3]};
        if (cnt[0] + cnt[1] + cnt[2] + cnt[3] <= 128u) {
            // Few candidates: wave 0 sorts them on its own, with no further
            // barrier; the other waves are done.
            if (wave == 0) {
                const uint64_t key = wave_sorted_candidates(sm.cand, cnt);
                if (lane < k) sm.sel[lane] = key;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
            return;
        }
        rank_candidates(sm, own_cands(sm), k, ToLds{sm.sel});
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

// ---------------------------------------------------------------------------
// Raw-logit log-softmax partials: per chunk (max, sum of exp(x - max)).
// ---------------------------------------------------------------------------

// Per-lane (max, sum) -> block (max, sum).  A lane whose values are all -inf
// carries its element count as the sum (the uniform reading for an all -inf
// domain); an empty lane carries (-inf, 0).  Ends after a barrier.
__device__ __forceinline__ float2 block_max_sum(SelectSmem &sm, float m, float s)
{
    float *red = reinterpret_cast<float *>(sm.red);  // 8 floats
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const float wm = wave_max_f32(m);
    if (lane == 0) red[wave] = wm;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float c;
    if (M == -INFINITY) c = s;
    else c = (m == -INFINITY) ? 0.0f : s * __expf(m - M);
    c = wave_sum_f32(c);
    if (lane == 0) red[4 + wave] = c;
    __syncthreads();
    const float S = (red[4] + red[5]) + (red[6] + red[7]);
    __syncthreads();
    return make_float2(M, S);
}

__device__ __forceinline__ void publish_partial(uint64_t *p, float2 ms)
{
    publish_u64(p, ((uint64_t)__float_as_uint(ms.y) << 32) | __float_as_uint(ms.x));
}

// Lane (max, sum) over EPT register values; NaN entries are skipped (ids past
// V and NaN logits, which count as -inf); +inf counts as the largest float.
// valid_count(): number of ids below V held by the lane, for the all -inf case.
template <int EPT, typename ValidCount>
__device__ __forceinline__ float2 lane_max_sum(const float (&v)[EPT], ValidCount valid_count)
{
    constexpr float kFltMax = 3.40282346638528859812e+38f;
    // fmaxf skips NaN, so one operation per element; +inf is clamped once
    // (m starts at -inf, so it is never NaN).
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < EPT; ++e) m = fmaxf(m, v[e]);
    m = fminf(m, kFltMax);
    float s = 0.0f;
    if (m == -INFINITY) {
        s = (float)valid_count();
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            s += (v[e] == v[e]) ? __expf(fminf(v[e], kFltMax) - m) : 0.0f;
    }
    return make_float2(m, s);
}

// Wave 0 of the merging workgroup: combine the row's chunk partials in fp64
// in a fixed order.  L = M + log(S); an all -inf row is uniform (L = log n).
__device__ __forceinline__ void combine_partials(const uint64_t *P, int nchunks, double *L,
                                                 bool *uniform)
{
    const int lane = lane_id();
    float mf = -INFINITY;
    for (int c = lane; c < nchunks; c += 64)
        mf = fmaxf(mf, __uint_as_float((uint32_t)read_published_u64(P + c)));
    const double M = (double)wave_max_f32(mf);
    double S = 0.0;
    for (int c = lane; c < nchunks; c += 64) {
        const uint64_t w = read_published_u64(P + c);
        const float px = __uint_as_float((uint32_t)w), py = __uint_as_float((uint32_t)(w >> 32));
        if (M == -INFINITY) S += (double)py;
        else if (px != -INFINITY) S += (double)py * exp((double)px - M);
    }
    S = wave_sum_f64(S);
    *uniform = (M == -INFINITY);
    *L = *uniform ? log(S) : M + log(S);
}

}  // namespace rts
