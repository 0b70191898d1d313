// rts_renorm.h -- logprobs renormalised over allowed_token_ids, computed by
// extra workgroups of the sampling launch (page "#3200 [Engine] OpenAI
// logprobs / top_logprobs / allowed_token_ids for the CUDA/HIP engine",
// "Problem and result" and "Approach": the reported distribution is the raw
// log-softmax, and an allowed list renormalises it over exactly the ids it
// names).
//
// One workgroup per restricted row gathers the row's list (at most
// kRenormMax ids) and its logits at once, drops repeated and out-of-range ids
// with a hash set in LDS, and computes L = log sum exp over the members and
// the top-K members.  These workgroups trail the grid: dispatched right after
// the sampling workgroups, they run while those stream the rows and finish
// long before the row's token is drawn (leading the grid instead delayed the
// start of every sampling workgroup: 4 % slower on 40 rows).  The token's logprob needs both halves: L, and the token
// with its raw logit.  Whichever half finishes second writes it, decided by
// one device-scope exchange on a per-row word:
//   - the renormalising workgroup exchanges in enc(L), an encoding that is
//     never 0 and never has an all-ones high word;
//   - the row's merging workgroup exchanges in kSamplerTag | token.
// The one that reads back the other's value finishes the row and returns the
// word to 0 for the next launch on the workspace.  Neither side waits.  The
// merging workgroup also reads the word while it draws: when enc(L) is
// already there, the renormalising workgroup has finished and left the row
// to it, and no exchange is needed.
#pragma once

#include "rts_select.h"

namespace rts {

constexpr uint64_t kSamplerTag = 0xFFFFFFFF00000000ull;  // | the sampled token
constexpr uint32_t kEmptySlot = 0xFFFFFFFFu;  // never an id below V <= 2^30

// enc(L) = bits + 1, where bits is L as an fp64 (never NaN: L is finite, or
// +inf for a list with no member) or, when every member's logit is -inf, a
// quiet NaN whose low word is the fp32 logprob -L every member then gets.
// bits + 1 is 0 only for the all-ones NaN, and has an all-ones high word
// only for a negative NaN: neither is produced.
__device__ __forceinline__ uint64_t renorm_encode(double L, bool uniform)
{
    const uint64_t bits = uniform
        ? (0x7FF8000000000000ull | (uint64_t)__float_as_uint((float)(-L)))
        : (uint64_t)__double_as_longlong(L);
    return bits + 1ull;
}

// The token's renormalised logprob from enc(L), whether the token is a
// member, and its raw logit.
__device__ __forceinline__ float renorm_token_lp(uint64_t enc, bool member, float xt)
{
    if (!member) return -INFINITY;
    const uint64_t bits = enc - 1ull;
    const bool uniform = (bits & 0x7FF0000000000000ull) == 0x7FF0000000000000ull &&
                         (bits & 0x000FFFFFFFFFFFFFull) != 0ull;
    if (uniform) return __uint_as_float((uint32_t)bits);
    return (float)((double)sanitize(xt) - __longlong_as_double((long long)bits));
}

__device__ __forceinline__ uint32_t renorm_hash(uint32_t id)
{
    return (id * 2654435761u) >> 20;  // Fibonacci hashing to 12 bits
}
static_assert(kRenormSlots == 1 << 12, "renorm_hash yields 12 bits");

// Logprobs over one allowed list, by one workgroup: the listed ids and their
// logits are gathered at once (kRenormPerThread per thread, cnt <= kRenormMax),
// repeats and ids outside [0, V) dropped with a hash set of kRenormSlots words
// in `tab` (LDS), then L = log sum exp over the members (log of the member
// count when every member is -inf; +inf when there is none) and the top-K
// members, written to top_ids / top_lp when K > 0.  Every member term of the
// sum is rounded to a multiple of 2^-40 before it is added, so the fp64 sum
// does not depend on which thread owns a repeated id.  Leaves each thread's
// listed ids in id[] (-1 past the list) and ends after a barrier.
__device__ __forceinline__ void allowed_members(SelectSmem &sm, uint32_t *tab, const float *x,
                                                const int32_t *ids, int cnt, int V, int K,
                                                int32_t *top_ids, float *top_lp,
                                                int32_t (&id)[kRenormPerThread], double &L_out,
                                                bool &uniform_out)
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    float v[kRenormPerThread];
#pragma unroll
    for (int j = 0; j < kRenormPerThread; ++j) {
        const int f = tid + j * kBlock;
        id[j] = (f < cnt) ? ids[f] : -1;
    }
#pragma unroll
    for (int j = 0; j < kRenormPerThread; ++j)
        v[j] = (id[j] >= 0 && id[j] < V) ? x[id[j]] : __builtin_nanf("");

    for (int w = tid; w < kRenormSlots; w += kBlock) tab[w] = kEmptySlot;
    __syncthreads();
    // The thread whose insert claims an id's slot owns the id; a repeat finds
    // it there.  The table is never full (at most kRenormMax ids in twice as
    // many slots), so every probe sequence ends.
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < kRenormPerThread; ++j) {
        bool owner = false;
        if (id[j] >= 0 && id[j] < V) {
            const uint32_t u = (uint32_t)id[j];
            uint32_t h = renorm_hash(u);
            for (int p = 0; p < kRenormSlots; ++p) {
                const uint32_t old = atomicCAS(&tab[h], kEmptySlot, u);
                if (old == kEmptySlot) { owner = true; break; }
                if (old == u) break;
                h = (h + 1u) & (uint32_t)(kRenormSlots - 1);
            }
        }
        v[j] = owner ? sanitize(v[j]) : __builtin_nanf("");  // NaN: not this thread's member
        mine += owner ? 1u : 0u;
    }

    float lmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kRenormPerThread; ++j) lmax = (v[j] == v[j]) ? fmaxf(lmax, v[j]) : lmax;
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
    for (int j = 0; j < kRenormPerThread; ++j)
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
    L_out = L;
    uniform_out = uniform;

    if (K > 0) {
        // top-K members: lane maxima -> threshold -> compaction -> rank
        sm.lane_keys[tid] = (lmax == -INFINITY && mine == 0u) ? 0u : value_key(lmax);
        __syncthreads();
        const uint32_t lk[4] = {sm.lane_keys[lane], sm.lane_keys[lane + 64],
                                sm.lane_keys[lane + 128], sm.lane_keys[lane + 192]};
        const float tf = key_threshold(selection_threshold(lk, K));
        const uint64_t below = lanes_below_mask();
        uint64_t *wc = sm.cand + wave * kRegion;
        uint32_t wcnt = 0;
#pragma unroll
        for (int j = 0; j < kRenormPerThread; ++j) {
            const bool c = v[j] >= tf;  // NaN (no member) never passes
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
                for (int j = 0; j < kRenormPerThread; ++j) {
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
        if (tid < K) {
            const uint64_t key = sm.sel[tid];
            const bool valid = key != 0ull;
            top_ids[tid] = valid ? (int32_t)key_index(key) : -1;
            top_lp[tid] =
                valid ? (uniform ? (float)(-L) : (float)((double)key_logit(key) - L)) : -INFINITY;
        }
    }
    __syncthreads();
}

// The renormalising workgroup of row `slot` in a sampling launch.  `tab` is
// kRenormSlots words of LDS besides `sm`.  Rows without kPackRenorm exit.
// Its results equal rts_token_logprobs' for the same list.
__device__ __forceinline__ void renorm_block(const SampleArgs &a, SelectSmem &sm, uint32_t *tab,
                                             int slot)
{
    const int tid = threadIdx.x;
    if (slot >= a.rows) return;
    const SampleRow R = a.row[slot];
    if ((R.pack & kPackRenorm) == 0u) return;
    const int V = a.V;
    const int K = a.lp_topn;
    const float *x = a.logits + (int64_t)slot * a.ld;
    int32_t id[kRenormPerThread];
    double L;
    bool uniform;
    allowed_members(sm, tab, x, a.allowed + R.allowed_off, R.allowed_cnt, V, K,
                    K > 0 ? a.lpa_ids + (int64_t)slot * K : nullptr,
                    K > 0 ? a.lpa_top + (int64_t)slot * K : nullptr, id, L, uniform);

    // the rendezvous with the row's merging workgroup
    uint64_t *w = a.lpa_w + (int64_t)slot * (kTicketStride / 2);
    const uint64_t enc = renorm_encode(L, uniform);
    if (tid == 0) {
        const uint64_t old = __hip_atomic_exchange(w, enc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool second = (old & kSamplerTag) == kSamplerTag;
        sm.flag = second ? 1u : 0u;
        sm.thr = (uint32_t)old;  // the token the merging workgroup left
        sm.wave_cnt[0] = 0u;     // set below by any thread holding the token's id
    }
    __syncthreads();
    if (sm.flag == 0u) return;  // the merging workgroup writes the token's logprob
    const int32_t t = (int32_t)sm.thr;
    const bool tv = t >= 0 && t < V;
    bool hit = false;
#pragma unroll
    for (int j = 0; j < kRenormPerThread; ++j) hit = hit || (id[j] == t);
    if (tv && hit) sm.wave_cnt[0] = 1u;
    __syncthreads();
    if (tid == 0) {
        a.lpa_token[slot] = renorm_token_lp(enc, sm.wave_cnt[0] != 0u, tv ? x[t] : 0.0f);
        publish_u64(w, 0ull);
    }
}

}  // namespace rts
