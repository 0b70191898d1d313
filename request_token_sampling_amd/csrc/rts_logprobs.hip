// rts_logprobs.hip -- raw-logit logprobs on gfx950.
//
// Page "#3200 [Engine] OpenAI logprobs / top_logprobs / allowed_token_ids for
// the CUDA/HIP engine" ("Problem and result", "Approach", "Limits") and page
// "#1916 OpenAI logprobs on /v1/chat/completions for the CUDA/HIP engine"
// ("What changed"): the reported value is the model's own distribution, a
// log-softmax of the head logits taken before penalties, temperature and the
// draw, with up to 20 top alternatives; allowed_token_ids renormalises it
// over exactly the ids named.
//
// Unrestricted rows: grid = rows x chunks.  Each workgroup reads its chunk
// once, keeps (max, sum of exp(x - max)) per lane in fp32 and its raw top-K
// keys (rts_select.h), and publishes one (max, sum) pair and K keys.  The
// last workgroup of the row combines the pairs in fp64 in chunk order and
// merges the keys.
// Restricted rows: one workgroup per row.  Where an LDS bitmap of the
// vocabulary fits (V <= 2^19) it drops repeats and foreign ids: lists of up to
// kAllowedFast ids are gathered at once into registers, the thread that sets
// an id's bit owning it; longer ones are marked first and the set bits walked,
// so each member is gathered exactly once.  Larger vocabularies take a hash
// set in LDS instead (rts_renorm.h), for lists of up to kRenormMax ids.
#include "rts_renorm.h"

namespace rts {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int EPT, bool VEC>
__global__ __launch_bounds__(kBlock, kMinWavesPerSimd) void logprob_kernel(const LogprobArgs a)
{
    constexpr int CH = EPT * kBlock;
    constexpr int NQ = EPT / 4;
    __shared__ SelectSmem sm;

    const int tid = threadIdx.x;
    const int lb = logical_block(a.early_xcds);
    if (lb < 0 || lb >= a.rows * a.nchunks) return;  // padding workgroup
    const int slot = lb / a.nchunks;
    const int chunk = lb - slot * a.nchunks;
    const int row = a.row[slot].row;
    const int V = a.V;
    const int K = a.top_n;
    const int base = chunk * CH;
    const float *x = a.logits + (int64_t)row * a.ld;

    float v[EPT];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int i0 = base + q * 1024 + tid * 4;
        if (VEC && i0 + 4 <= V) {
            // streamed once: the nontemporal hint, as in the sampler
            const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(x + i0));
            v[4 * q + 0] = t.x;
            v[4 * q + 1] = t.y;
            v[4 * q + 2] = t.z;
            v[4 * q + 3] = t.w;
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) v[4 * q + s] = (i0 + s < V) ? x[i0 + s] : 0.0f;
        }
    }
    float lmax = -INFINITY;
    int nvalid = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int i0 = base + q * 1024 + tid * 4;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bool in = i0 + s < V;
            const float t = in ? sanitize(v[4 * q + s]) : __builtin_nanf("");
            v[4 * q + s] = t;
            lmax = in ? fmaxf(lmax, t) : lmax;
            nvalid += in ? 1 : 0;
        }
    }
    float lsum = 0.0f;
    if (lmax == -INFINITY) {
        lsum = (float)nvalid;
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) lsum += (v[e] == v[e]) ? __expf(v[e] - lmax) : 0.0f;
    }
    const float2 ms = block_max_sum(sm, lmax, lsum);
    if (tid == 0)
        publish_partial(reinterpret_cast<uint64_t *>(a.partials) + (int64_t)slot * a.partial_stride +
                            chunk, ms);

    uint64_t *list = a.keys + (int64_t)slot * a.keys_stride;
    if (K > 0) chunk_topk<EPT>(sm, v, base, V, K, list + (int64_t)chunk * K);

    if (!take_last_ticket(&a.tickets[slot * kTicketStride], (uint32_t)a.nchunks, &sm.flag)) return;

    // ---- the last workgroup of the row.
    if (K > 0) list_topk(sm, list, a.nchunks, K);

    if ((tid >> 6) != 0) return;
    const int lane = lane_id();
    double L;
    bool uniform;
    combine_partials(reinterpret_cast<const uint64_t *>(a.partials) +
                         (int64_t)slot * a.partial_stride,
                     a.nchunks, &L, &uniform);

    if (lane == 0) {
        const int32_t t = a.tokens[row];
        float lp = -INFINITY;
        if (t >= 0 && t < V) lp = uniform ? (float)(-L) : (float)((double)sanitize(x[t]) - L);
        a.token_lp[row] = lp;
        a.tickets[slot * kTicketStride] = 0u;
    }
    if (lane < K) {
        const uint64_t key = sm.sel[lane];
        const bool valid = key != 0ull;
        a.top_ids[(int64_t)row * K + lane] = valid ? (int32_t)key_index(key) : -1;
        a.top_lp[(int64_t)row * K + lane] =
            valid ? (uniform ? (float)(-L) : (float)((double)key_logit(key) - L)) : -INFINITY;
    }
}

static_assert(sizeof(SelectSmem) + 4 <= kAllowedStaticLds, "static LDS bound");

// One workgroup per restricted row whose list is longer than kAllowedFast:
// the members are walked in the bitmap for each pass.  Dynamic LDS: the
// vocabulary bitmap.
__global__ __launch_bounds__(kBlock) void logprob_allowed_wide_kernel(const LogprobArgs a)
{
    extern __shared__ uint32_t bm[];
    __shared__ SelectSmem sm;
    __shared__ uint32_t s_cnt;

    const int tid = threadIdx.x, lane = lane_id();
    const LogprobRow R = a.row[blockIdx.x];
    const int row = R.row;
    const int V = a.V;
    const int K = a.top_n;
    const int nw = (V + 31) >> 5;
    const float *x = a.logits + (int64_t)row * a.ld;

    for (int w = tid; w < nw; w += kBlock) bm[w] = 0u;
    if (tid == 0) s_cnt = 0u;
    __syncthreads();
    const int32_t *ids = a.allowed + R.allowed_off;
    for (int64_t j = tid; j < R.allowed_cnt; j += kBlock) {
        const int32_t id = ids[j];
        if (id >= 0 && id < V) atomicOr(&bm[id >> 5], 1u << (id & 31));
    }
    __syncthreads();

    // pass 1: lane maximum and member count over the thread's bitmap words
    float lmax = -INFINITY;
    int nmem = 0;
    for (int w = tid; w < nw; w += kBlock) {
        uint32_t bits = bm[w];
        while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1u;
            lmax = fmaxf(lmax, sanitize(x[(w << 5) + b]));
            ++nmem;
        }
    }
    float *red = reinterpret_cast<float *>(sm.red);
    {
        const float wm = wave_max_f32(lmax);
        if (lane == 0) red[tid >> 6] = wm;
    }
    __syncthreads();
    const float Mf = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const double M = (double)Mf;
    // pass 2: fp64 sum of exp(x - M) (or the member count for an all -inf domain)
    double s = 0.0;
    for (int w = tid; w < nw; w += kBlock) {
        uint32_t bits = bm[w];
        while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1u;
            s += (Mf == -INFINITY) ? 1.0 : exp((double)sanitize(x[(w << 5) + b]) - M);
        }
    }
    s = wave_sum_f64(s);
    double *dred = reinterpret_cast<double *>(sm.cand);
    if (lane == 0) dred[tid >> 6] = s;
    const int nm = (int)wave_sum_f64((double)nmem);
    if (lane == 0) sm.wave_cnt[tid >> 6] = (uint32_t)nm;
    __syncthreads();
    const double S = (dred[0] + dred[1]) + (dred[2] + dred[3]);
    const uint32_t members = sm.wave_cnt[0] + sm.wave_cnt[1] + sm.wave_cnt[2] + sm.wave_cnt[3];
    __syncthreads();
    const bool empty = members == 0u;
    const bool uniform = !empty && Mf == -INFINITY;
    const double L = empty ? INFINITY : (uniform ? log(S) : M + log(S));

    if (K > 0) {
        // top-K members: lane maxima -> threshold -> LDS compaction -> rank
        sm.lane_keys[tid] = (nmem == 0) ? 0u : value_key(lmax);
        __syncthreads();
        const uint32_t lk[4] = {sm.lane_keys[lane], sm.lane_keys[lane + 64],
                                sm.lane_keys[lane + 128], sm.lane_keys[lane + 192]};
        const float tf = key_threshold(selection_threshold(lk, K));
        for (int w = tid; w < nw; w += kBlock) {
            uint32_t bits = bm[w];
            while (bits) {
                const int b = __ffs(bits) - 1;
                bits &= bits - 1u;
                const int id = (w << 5) + b;
                const float xv = sanitize(x[id]);
                if (xv >= tf) {
                    const uint32_t pos = atomicAdd(&s_cnt, 1u);
                    if (pos < (uint32_t)(4 * kCap)) sm.cand[pos] = cand_key(xv, (uint32_t)id);
                }
            }
        }
        __syncthreads();
        const uint32_t n = s_cnt;
        if (n <= (uint32_t)(4 * kCap)) {
            for (uint32_t f = tid; f < n; f += kBlock) {
                const uint64_t key = sm.cand[f];
                uint32_t rank = 0;
                for (uint32_t j = 0; j < n; ++j) rank += (sm.cand[j] > key) ? 1u : 0u;
                if (rank < (uint32_t)K) sm.sel[rank] = key;
            }
            for (int r = (int)n + tid; r < K; r += kBlock) sm.sel[r] = 0ull;
        } else {
            // massive ties at the threshold: K argmax rounds over the members
            uint64_t prev = ~0ull;
            for (int r = 0; r < K; ++r) {
                uint64_t best = 0;
                for (int w = tid; w < nw; w += kBlock) {
                    uint32_t bits = bm[w];
                    while (bits) {
                        const int b = __ffs(bits) - 1;
                        bits &= bits - 1u;
                        const int id = (w << 5) + b;
                        const uint64_t key = cand_key(sanitize(x[id]), (uint32_t)id);
                        best = (key < prev && key > best) ? key : best;
                    }
                }
                best = block_max_u64(sm, best);
                if (tid == 0) sm.sel[r] = best;
                prev = best;
            }
        }
        __syncthreads();
    }

    if (tid == 0) {
        const int32_t t = a.tokens[row];
        float lp = -INFINITY;
        if (t >= 0 && t < V && ((bm[t >> 5] >> (t & 31)) & 1u))
            lp = uniform ? (float)(-L) : (float)((double)sanitize(x[t]) - L);
        a.token_lp[row] = lp;
    }
    if (tid < K) {
        const uint64_t key = sm.sel[tid];
        const bool valid = key != 0ull;
        a.top_ids[(int64_t)row * K + tid] = valid ? (int32_t)key_index(key) : -1;
        a.top_lp[(int64_t)row * K + tid] =
            valid ? (uniform ? (float)(-L) : (float)((double)key_logit(key) - L)) : -INFINITY;
    }
}

// One workgroup per restricted row with at most kAllowedFast listed ids.
// Thread t reads listed ids t, t + 256, ... and gathers their logits at
// once; marking each id in an LDS bitmap of the vocabulary makes the thread
// that set its bit the id's owner, so duplicates count once and foreign ids
// are ignored.  Which thread owns a duplicate depends on timing, so the sum
// of exponentials is made order-free: each term is rounded to a multiple of
// 2^-40 and the multiples, below 2^53 in total, add exactly in fp64.  The
// max, the sum and the top-K all run from registers.  Dynamic LDS: the bitmap.
__global__ __launch_bounds__(kBlock) void logprob_allowed_kernel(const LogprobArgs a)
{
    extern __shared__ uint32_t bm[];
    __shared__ SelectSmem sm;

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const LogprobRow R = a.row[blockIdx.x];
    const int row = R.row;
    const int V = a.V;
    const int K = a.top_n;
    const int nw = (V + 31) >> 5;
    const float *x = a.logits + (int64_t)row * a.ld;
    // the token's logit, loaded now so its latency hides behind the rest
    const int32_t t = a.tokens[row];
    const float xt = (tid == 0 && t >= 0 && t < V) ? x[t] : 0.0f;

    // listed ids and their logits, all loads in flight together
    const int32_t *ids = a.allowed + R.allowed_off;
    const int cnt = (int)R.allowed_cnt;
    int32_t id[kAllowedPerThread];
    float v[kAllowedPerThread];
#pragma unroll
    for (int j = 0; j < kAllowedPerThread; ++j) {
        const int f = tid + j * kBlock;
        id[j] = (f < cnt) ? ids[f] : -1;
    }
#pragma unroll
    for (int j = 0; j < kAllowedPerThread; ++j)
        v[j] = (id[j] >= 0 && id[j] < V) ? x[id[j]] : __builtin_nanf("");

    for (int w = tid; w < nw; w += kBlock) bm[w] = 0u;
    __syncthreads();
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < kAllowedPerThread; ++j) {
        bool owner = false;
        if (id[j] >= 0 && id[j] < V) {
            const uint32_t bit = 1u << (id[j] & 31);
            owner = (atomicOr(&bm[id[j] >> 5], bit) & bit) == 0u;
        }
        v[j] = owner ? sanitize(v[j]) : __builtin_nanf("");  // NaN: not this thread's member
        mine += owner ? 1u : 0u;
    }

    float lmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kAllowedPerThread; ++j) lmax = (v[j] == v[j]) ? fmaxf(lmax, v[j]) : lmax;
    float *red = reinterpret_cast<float *>(sm.red);
    const float wm = wave_max_f32(lmax);
    const double wn = wave_sum_f64((double)mine);
    if (lane == 0) {
        red[wave] = wm;
        sm.wave_cnt[wave] = (uint32_t)wn;
    }
    __syncthreads();
    const float Mf = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const uint32_t members = sm.wave_cnt[0] + sm.wave_cnt[1] + sm.wave_cnt[2] + sm.wave_cnt[3];
    const double M = (double)Mf;
    constexpr double kUnit = 1099511627776.0;  // 2^40
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < kAllowedPerThread; ++j)
        if (v[j] == v[j]) s += (Mf == -INFINITY) ? 1.0 : rint((double)__expf(v[j] - Mf) * kUnit);
    s = wave_sum_f64(s);
    double *dred = reinterpret_cast<double *>(sm.cand);
    if (lane == 0) dred[wave] = s;
    __syncthreads();
    double S = (dred[0] + dred[1]) + (dred[2] + dred[3]);
    if (Mf != -INFINITY) S = S / kUnit;
    __syncthreads();
    const bool empty = members == 0u;
    const bool uniform = !empty && Mf == -INFINITY;
    const double L = empty ? INFINITY : (uniform ? log(S) : M + log(S));

    if (K > 0) {
        // top-K of the members: lane maxima -> threshold -> compaction -> rank
        sm.lane_keys[tid] = (lmax == -INFINITY && mine == 0u) ? 0u : value_key(lmax);
        __syncthreads();
        const uint32_t lk[4] = {sm.lane_keys[lane], sm.lane_keys[lane + 64],
                                sm.lane_keys[lane + 128], sm.lane_keys[lane + 192]};
        const float tf = key_threshold(selection_threshold(lk, K));
        const uint64_t below = lanes_below_mask();
        uint64_t *wc = sm.cand + wave * kRegion;
        uint32_t wcnt = 0;
#pragma unroll
        for (int j = 0; j < kAllowedPerThread; ++j) {
            const bool c = v[j] >= tf;               // NaN (no member) never passes
            const uint64_t m = __ballot(c);
            if (m) {
                const uint32_t p = wcnt + (uint32_t)__popcll(m & below);
                if (c && p < (uint32_t)kCap) wc[p] = cand_key(v[j], (uint32_t)id[j]);
                wcnt += (uint32_t)__popcll(m);
            }
        }
        if (lane == 0) sm.wave_cnt[wave] = wcnt;
        pad_region(own_cands(sm), wave, wcnt);
        __syncthreads();
        if (!any_overflow(own_cands(sm))) {
            rank_candidates(sm, own_cands(sm), K, ToLds{sm.sel});
        } else {
            // massive ties at the threshold: K argmax rounds over the members
            uint64_t prev = ~0ull;
            for (int r = 0; r < K; ++r) {
                uint64_t best = 0;
#pragma unroll
                for (int j = 0; j < kAllowedPerThread; ++j) {
                    if (v[j] == v[j]) {
                        const uint64_t key = cand_key(v[j], (uint32_t)id[j]);
                        best = (key < prev && key > best) ? key : best;
                    }
                }
                best = block_max_u64(sm, best);
                if (tid == 0) sm.sel[r] = best;
                prev = best;
            }
        }
        __syncthreads();
    }

    if (tid == 0) {
        float lp = -INFINITY;
        if (t >= 0 && t < V && ((bm[t >> 5] >> (t & 31)) & 1u))
            lp = uniform ? (float)(-L) : (float)((double)sanitize(xt) - L);
        a.token_lp[row] = lp;
    }
    if (tid < K) {
        const uint64_t key = sm.sel[tid];
        const bool valid = key != 0ull;
        a.top_ids[(int64_t)row * K + tid] = valid ? (int32_t)key_index(key) : -1;
        a.top_lp[(int64_t)row * K + tid] =
            valid ? (uniform ? (float)(-L) : (float)((double)key_logit(key) - L)) : -INFINITY;
    }
}

template <int EPT, bool VEC>
static int launch_full_t(const LogprobArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((logprob_kernel<EPT, VEC>), dim3(grid_for(a.rows * a.nchunks, a.early_xcds)),
                       dim3(kBlock), 0, s, a);
    return (int)hipGetLastError();
}

int launch_logprobs_full(const LogprobArgs &a, int ept, bool vec, hipStream_t s)
{
    switch (ept) {
    case 4: return vec ? launch_full_t<4, true>(a, s) : launch_full_t<4, false>(a, s);
    case 8: return vec ? launch_full_t<8, true>(a, s) : launch_full_t<8, false>(a, s);
    case 16: return vec ? launch_full_t<16, true>(a, s) : launch_full_t<16, false>(a, s);
    case 32: return vec ? launch_full_t<32, true>(a, s) : (int)hipErrorInvalidValue;  // see the host
    default: return (int)hipErrorInvalidValue;
    }
}

// One workgroup per restricted row with at most kRenormMax listed ids.
__global__ __launch_bounds__(kBlock) void logprob_allowed_hash_kernel(const LogprobArgs a)
{
    __shared__ SelectSmem sm;
    __shared__ uint32_t tab[kRenormSlots];
    __shared__ uint32_t s_member;

    const int tid = threadIdx.x;
    const LogprobRow R = a.row[blockIdx.x];
    const int row = R.row;
    const int V = a.V;
    const int K = a.top_n;
    const float *x = a.logits + (int64_t)row * a.ld;
    // the token and its logit, loaded now so their latency hides behind the rest
    const int32_t t = a.tokens[row];
    const bool tv = t >= 0 && t < V;
    const float xt = (tid == 0 && tv) ? x[t] : 0.0f;
    if (tid == 0) s_member = 0u;  // ordered before its use by the barriers below
    int32_t id[kRenormPerThread];
    double L;
    bool uniform;
    allowed_members(sm, tab, x, a.allowed + R.allowed_off, (int)R.allowed_cnt, V, K,
                    K > 0 ? a.top_ids + (int64_t)row * K : nullptr,
                    K > 0 ? a.top_lp + (int64_t)row * K : nullptr, id, L, uniform);
    bool hit = false;
#pragma unroll
    for (int j = 0; j < kRenormPerThread; ++j) hit = hit || (id[j] == t);
    if (tv && hit) s_member = 1u;
    __syncthreads();
    if (tid == 0) {
        float lp = -INFINITY;
        if (s_member != 0u) lp = uniform ? (float)(-L) : (float)((double)sanitize(xt) - L);
        a.token_lp[row] = lp;
    }
}

int launch_logprobs_allowed(const LogprobArgs &a, size_t lds_bytes, int kind, hipStream_t s)
{
    if (kind == kAllowedHash)
        hipLaunchKernelGGL(logprob_allowed_hash_kernel, dim3((unsigned)a.rows), dim3(kBlock), 0, s, a);
    else if (kind == kAllowedWide)
        hipLaunchKernelGGL(logprob_allowed_wide_kernel, dim3((unsigned)a.rows), dim3(kBlock),
                           (unsigned)lds_bytes, s, a);
    else
        hipLaunchKernelGGL(logprob_allowed_kernel, dim3((unsigned)a.rows), dim3(kBlock),
                           (unsigned)lds_bytes, s, a);
    return (int)hipGetLastError();
}

}  // namespace rts
