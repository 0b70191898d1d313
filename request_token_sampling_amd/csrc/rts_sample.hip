// rts_sample.hip -- the sampling chain on gfx950.
//
// One launch per group of up to 64 rows; grid = rows x chunks, 256 threads
// per workgroup.  A workgroup reads its chunk of the row from HBM once and
// (a) builds the chunk's slice of the penalty token bitmap and counts in LDS
// from the row's history window (page "#19 serve: per-request temperature/
// top_p/top_k/min_p/penalties sampling", "What changed", the min_p and
// penalties paragraph: only flagged candidates look up a count),
// (b) applies the repeat / frequency / presence penalties to flagged ids,
// (c) keeps its exact top-k keys (rts_select.h) in the workspace, and
// (d) takes the row's ticket.  The workgroup that finishes a row last merges
// the chunk lists into the kept sequence and one wavefront runs the cuts and
// the draw: min_p (head + logf(min_p), computed in fp32), top_p over the
// min_p survivors, temperature, and the Philox4x32-10 draw keyed by
// (seed, counter) ("A persistent per-request draw counter" paragraph).  The
// counter may live in device memory, where the call advances it, so a
// captured graph replaying the call keeps drawing fresh numbers ("Problem":
// a captured sampler would otherwise repeat its draws).
#include "rts_epilogue.h"
#include "rts_renorm.h"

namespace rts {

template <int EPT, bool LP>
struct SampleSmem {
    SelectSmem s;
    uint32_t pen_bits[EPT * kBlock / 32];  // one bit per id of the chunk
    // two 16-bit counts per word; a renormalising workgroup's hash table
    uint32_t pen_cnt[(LP && EPT * kBlock / 2 < kRenormSlots) ? kRenormSlots : EPT * kBlock / 2];
    uint64_t raw_keys[LP ? 4 * kRegion : 1];  // candidates of the raw top-K
    uint32_t raw_cnt[4];
    uint32_t lpa_member[4];  // the sampled token is in the row's allowed list (per wave)
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

// The chunk at `base` into registers, element e of the thread at
// elem_index(base, e); ids past V (only in the last chunk) read as NaN.
// A chunk wholly below V takes a path with no branch between its loads: a
// branch whose two sides fill the same registers makes the compiler wait
// for each 16-byte load before issuing the next (a full vmcnt(0) each).
// The 16-byte loads carry the nontemporal hint (the `nt` bit): the logits
// are streamed once, and on MI355X this measured 2-3 % faster on 40 rows and
// on one row read as two broadcast parameter rows (ld = 0), whose second
// reads still find the chunk in the XCD's L2.
template <int EPT, bool VEC>
__device__ __forceinline__ void load_chunk(const float *x, int base, int V, float (&v)[EPT])
{
    const int tid = threadIdx.x;
    if (VEC && base + (EPT / 4) * 1024 <= V) {
#pragma unroll
        for (int q = 0; q < EPT / 4; ++q) {
            const f32x4 t = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4 *>(x + base + q * 1024 + tid * 4));
            v[4 * q + 0] = t.x;
            v[4 * q + 1] = t.y;
            v[4 * q + 2] = t.z;
            v[4 * q + 3] = t.w;
        }
        return;
    }
#pragma unroll
    for (int q = 0; q < EPT / 4; ++q) {
        const int i0 = base + q * 1024 + tid * 4;
        if (VEC && i0 + 4 <= V) {
            const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(x + i0));
            v[4 * q + 0] = t.x;
            v[4 * q + 1] = t.y;
            v[4 * q + 2] = t.z;
            v[4 * q + 3] = t.w;
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                v[4 * q + s] = (i0 + s < V) ? x[i0 + s] : __builtin_nanf("");
        }
    }
}

template <int EPT, bool VEC, bool LP>
__global__ __launch_bounds__(kBlock, kMinWavesPerSimd) void sample_kernel(const SampleArgs a)
{
    constexpr int CH = EPT * kBlock;
    constexpr int NQ = EPT / 4;
    __shared__ SampleSmem<EPT, LP> sm;

    // Every argument the chunk's address depends on is read first and held
    // by an empty asm statement, so the compiler issues these scalar loads
    // together before the first branch instead of sinking each below the
    // branch that needs it: the chunk's loads then go out one round trip
    // after the start instead of three (measured on MI355X: one row read as
    // two parameter rows 10.3 -> 9.8 us, 5 rows 12.9 -> 12.5 us).
    const int early = a.early_xcds, cmaj = a.chunk_major, nch = a.nchunks, rows = a.rows;
    const int V = a.V;
    const float *const logits = a.logits;
    const int64_t ld = a.ld;
    asm volatile("" ::"s"(early), "s"(cmaj), "s"(nch), "s"(rows), "s"(V), "s"(logits), "s"(ld));
    if constexpr (LP) {
        // workgroups past the sampling grid renormalise over allowed lists
        const int nsamp = (int)grid_for(sample_work(rows, nch, early, cmaj), early);
        if ((int)blockIdx.x >= nsamp) {
            renorm_block(a, sm.s, sm.pen_cnt, (int)blockIdx.x - nsamp);
            return;
        }
    }
    const int tid = threadIdx.x;
    const int lb = logical_block(early);
    if (lb < 0 || lb >= sample_work(rows, nch, early, cmaj)) return;
    int slot, chunk;
    if (cmaj) {
        // Rows that share one logits row: the workgroups of one chunk for all
        // rows land on one XCD, so the chunk is fetched from HBM once and the
        // other rows read it from that XCD's L2.
        const int P = xcds_used(early), xx = lb % P, q = lb / P;
        slot = q % rows;
        chunk = (q / rows) * P + xx;
        if (chunk >= nch) return;  // padding workgroup
    } else {
        slot = lb / nch;
        chunk = lb - slot * nch;
    }
    const int base = chunk * CH;
    const float *x = logits + (int64_t)slot * ld;
    // The chunk's loads go out before the row's parameters are read.  Ids
    // past V read as NaN: never selected.
    float v[EPT];
    load_chunk<EPT, VEC>(x, base, V, v);
    const SampleRow R = a.row[slot];
    const int n_eff = (int)(R.pack & 0xFFFFu);
    const int k = (int)((R.pack >> 16) & 0x7Fu);
    const bool greedy = ((R.pack >> 24) & 1u) != 0u;
    // Each thread's first history id: loads return in order, so it arrives
    // with the chunk's last load and the bitmap build below waits for the
    // chunk.  Loading it first would need the row's parameters first, one
    // more scalar round trip before the chunk's loads, which measured slower
    // on every workload, penalised ones included.
    const int32_t *h = a.history + R.hist_off;
    const int32_t h0 = (!LP && n_eff > 0 && tid < n_eff) ? h[tid] : -1;

    // Raw-logit logprobs in the same pass (page "#3200 ...", "Approach": the
    // reported distribution is taken before penalties and temperature): the
    // chunk's (max, sum) of the raw values, and their top-K unless the kept
    // list will already be the raw top-K (no penalties and k_eff >= K).  The
    // raw selection's candidates are compacted now, from the raw values, and
    // ranked after the penalised selection, so only one set of values is
    // held in registers at a time.
    const int K = LP ? a.lp_topn : 0;
    // an allowed list restricts the candidates unless it only renormalises
    // the logprobs
    const bool masked = R.allowed_cnt > 0 && (R.pack & kPackRenorm) == 0u;
    const bool raw_sel = LP && K > 0 && !(n_eff == 0 && !masked && k >= K);
    const Cands rawc{sm.raw_keys, sm.raw_cnt};
    uint64_t *raw_out = LP ? a.raw_keys + (int64_t)slot * a.raw_stride + (int64_t)chunk * K : nullptr;
    bool raw_done = false;
    if (LP) {
        const float2 lms = lane_max_sum<EPT>(v, [&]() {
            // ids below V among the lane's groups of four
            int c = 0;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int left = V - (base + q * 1024 + tid * 4);
                c += left < 0 ? 0 : (left > 4 ? 4 : left);
            }
            return c;
        });
        const float2 ms = block_max_sum(sm.s, lms.x, lms.y);
        if (tid == 0)
            publish_partial(a.partials + (int64_t)slot * a.partial_stride + chunk, ms);
        if (raw_sel) raw_done = chunk_compact<EPT, ToWorkspace, false>(sm.s, v, base, V, K, rawc, ToWorkspace{raw_out});
    }

    // Ids read and ignored (outside [0, V)) are counted by each row's
    // chunk-0 workgroup, when the caller asks for the count.
    const bool count_ignored = a.ignored != nullptr && chunk == 0;
    if (n_eff > 0) {
        // Clear the chunk's bits and only the count words the window touches.
        for (int w = tid; w < CH / 32; w += kBlock) sm.pen_bits[w] = 0u;
        uint32_t bad = 0;
        for (int j = tid; j < n_eff; j += kBlock) {
            const int32_t id = (!LP && j == tid) ? h0 : h[j];
            const int rel = id - base;
            if (id >= 0 && id < V && rel >= 0 && rel < CH) sm.pen_cnt[rel >> 1] = 0u;
            bad += (id < 0 || id >= V) ? 1u : 0u;
        }
        if (count_ignored && bad) atomicAdd(a.ignored, bad);
        __syncthreads();
        for (int j = tid; j < n_eff; j += kBlock) {
            const int32_t id = (!LP && j == tid) ? h0 : h[j];
            const int rel = id - base;
            if (id >= 0 && id < V && rel >= 0 && rel < CH) {
                atomicOr(&sm.pen_bits[rel >> 5], 1u << (rel & 31));
                atomicAdd(&sm.pen_cnt[rel >> 1], 1u << ((rel & 1) * 16));
            }
        }
        __syncthreads();
        // Only flagged ids look up a count; they leave sanitised.
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int rel = q * 1024 + tid * 4;
            const uint32_t nib = (sm.pen_bits[rel >> 5] >> (rel & 31)) & 0xFu;
            if (nib) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if ((nib >> s) & 1u) {
                        const int r = rel + s;
                        const uint32_t c = (sm.pen_cnt[r >> 1] >> ((r & 1) * 16)) & 0xFFFFu;
                        v[4 * q + s] = penalize(sanitize(v[4 * q + s]), c, R.rep, R.freq, R.present);
                    }
                }
            }
        }
    }

    // A row with an allowed list samples among those ids only: the chunk's
    // members are marked in LDS (in the penalty bitmap's space, free by now)
    // and every other id reads as absent (NaN); members are sanitised, so a
    // NaN member still counts as -inf.
    if (masked) {
        __syncthreads();  // penalty lookups may still read the bitmap
        for (int w = tid; w < CH / 32; w += kBlock) sm.pen_bits[w] = 0u;
        __syncthreads();
        const int32_t *al = a.allowed + R.allowed_off;
        uint32_t bad = 0;
        for (int j = tid; j < R.allowed_cnt; j += kBlock) {
            const int32_t id = al[j];
            const int rel = id - base;
            if (id >= 0 && id < V && rel >= 0 && rel < CH)
                atomicOr(&sm.pen_bits[rel >> 5], 1u << (rel & 31));
            bad += (id < 0 || id >= V) ? 1u : 0u;
        }
        if (count_ignored && bad) atomicAdd(a.ignored, bad);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int rel = q * 1024 + tid * 4;
            const uint32_t nib = (sm.pen_bits[rel >> 5] >> (rel & 31)) & 0xFu;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                v[4 * q + s] = ((nib >> s) & 1u) ? sanitize(v[4 * q + s]) : __builtin_nanf("");
        }
    }

    uint64_t *list = a.keys + (int64_t)slot * a.keys_stride;
    // (the fused variant takes the two-key threshold search without the
    // full-search rerun: with the rerun its register peak passes 96)
    chunk_topk<EPT, !LP>(sm.s, v, base, V, k, list + (int64_t)chunk * k, masked);

    if (raw_sel && !raw_done) {
        __syncthreads();  // the penalised selection's rank may still read sm.part
        if (any_overflow(rawc)) load_chunk<EPT, VEC>(x, base, V, v);  // raw values again
        chunk_finish<EPT>(sm.s, v, base, V, K, rawc, ToWorkspace{raw_out});
    }

    if (!take_last_ticket(&a.tickets[slot * kTicketStride], (uint32_t)a.nchunks, &sm.s.flag)) return;

    // ---- the last workgroup of the row: merge, then the cuts and the draw.
    // The row's Philox counter (device-resident when given, else the
    // caller's value) and the draw's word x0 depend on neither, so they are
    // computed while the merge's first loads are in flight.
    const uint64_t ctr = a.counters ? a.counters[slot] : R.counter;
    uint32_t x0 = 0u;
    // A row renormalised over an allowed list: its ids load once the merge's
    // first loads are issued, so the merge hides their latency; the tail
    // looks the drawn token up in them.
    const bool renorm = LP && (R.pack & kPackRenorm) != 0u;
    int32_t al[kRenormPerThread];
    RowOut ro;
    list_topk(sm.s, list, a.nchunks, k, [&]() {
        ro = row_out(a);
        if (renorm) {
            const int32_t *ids = a.allowed + R.allowed_off;
#pragma unroll
            for (int j = 0; j < kRenormPerThread; ++j) {
                const int f = tid + j * kBlock;
                al[j] = f < R.allowed_cnt ? ids[f] : -1;
            }
        }
        if (!greedy) x0 = philox4x32_10_x0(ctr, R.seed);
    });

    const int wave = tid >> 6, lane = lane_id();
    if (!LP) {
        if (wave == 0) epilogue(ro, R, sm.s, slot, k, greedy, ctr, x0);
        return;
    }

    // ---- with raw logprobs: wave 0 loads the raw logit of every kept id
    // (the token is one of them) and runs the cuts and the draw while wave 1
    // combines the chunk partials; neither waits for the other's loads.  On a
    // row renormalised over an allowed list, every wave then looks the token
    // up in the list ids it loaded during the merge, and wave 0 meets the
    // row's renormalising workgroup (see rts_renorm.h).
    uint64_t *const lpa_w = a.lpa_w + (int64_t)slot * (kTicketStride / 2);
    float xt = 0.0f;      // wave 0: the sampled token's raw logit
    uint64_t enc = 0ull;  // wave 0, lane 0: the renormalising workgroup's enc(L), 0 if not done
    if (wave == 0) {
        const uint64_t kept = lane < k ? sm.s.sel[lane] : 0ull;
        const float xr = kept ? x[key_index(kept)] : 0.0f;
        if (renorm && lane == 0) enc = read_published_u64(lpa_w);  // done already?
        epilogue(ro, R, sm.s, slot, k, greedy, ctr, x0);
        const int32_t t = (int32_t)sm.s.flag;  // the sampled token, left by the epilogue
        if (renorm && lane == 0 && enc == 0ull)
            enc = __hip_atomic_exchange(lpa_w, kSamplerTag | (uint32_t)t, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t at = __ballot(kept != 0ull && (int32_t)key_index(kept) == t);
        xt = at ? lane_f32(xr, __ffsll((unsigned long long)at) - 1) : 0.0f;
    } else if (wave == 1) {
        double L1;
        bool u1;
        combine_partials(a.partials + (int64_t)slot * a.partial_stride, a.nchunks, &L1, &u1);
        if (lane == 0) {
            sm.s.red[0] = (uint64_t)__double_as_longlong(L1);
            sm.s.red[1] = u1 ? 1ull : 0ull;
        }
    }
    __syncthreads();
    const double L = __longlong_as_double((long long)sm.s.red[0]);
    const bool uniform = sm.s.red[1] != 0ull;
    if (renorm) {
        const int32_t t = (int32_t)sm.s.flag;
        bool hit = false;
#pragma unroll
        for (int j = 0; j < kRenormPerThread; ++j) hit = hit || (al[j] == t);
        const uint64_t b = __ballot(hit && t >= 0 && t < V);
        if (lane == 0) sm.lpa_member[wave] = b ? 1u : 0u;
    }
    __syncthreads();  // the raw merge below may reuse sm.red
    if (raw_sel) list_topk(sm.s, a.raw_keys + (int64_t)slot * a.raw_stride, a.nchunks, K);
    if (wave != 0) return;
    const bool lpa_copy = a.lpa_token != nullptr && !renorm;  // unrestricted: the same values
    if (lane == 0) {
        const int32_t t = (int32_t)sm.s.flag;
        float lp = -INFINITY;
        if (t >= 0 && t < V) lp = uniform ? (float)(-L) : (float)((double)sanitize(xt) - L);
        a.lp_token[slot] = lp;
        if (lpa_copy) a.lpa_token[slot] = lp;
        if (renorm && enc != 0ull) {
            // the renormalising workgroup finished first: this one writes
            const bool member =
                (sm.lpa_member[0] | sm.lpa_member[1] | sm.lpa_member[2] | sm.lpa_member[3]) != 0u;
            a.lpa_token[slot] = renorm_token_lp(enc, member, xt);
            publish_u64(lpa_w, 0ull);
        }
    }
    if (lane < K) {
        const uint64_t key = sm.s.sel[lane];
        const bool valid = key != 0ull;
        const int32_t tid_out = valid ? (int32_t)key_index(key) : -1;
        const float lp_out =
            valid ? (uniform ? (float)(-L) : (float)((double)key_logit(key) - L)) : -INFINITY;
        a.lp_ids[(int64_t)slot * K + lane] = tid_out;
        a.lp_top[(int64_t)slot * K + lane] = lp_out;
        if (lpa_copy) {
            a.lpa_ids[(int64_t)slot * K + lane] = tid_out;
            a.lpa_top[(int64_t)slot * K + lane] = lp_out;
        }
    }
}

template <int EPT, bool VEC, bool LP>
static int launch_t(const SampleArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((sample_kernel<EPT, VEC, LP>),
                       dim3(grid_for(sample_work(a.rows, a.nchunks, a.early_xcds, a.chunk_major),
                                     a.early_xcds) +
                            a.lpa_blocks),
                       dim3(kBlock), 0, s, a);
    return (int)hipGetLastError();
}

// Rows read element by element (unaligned, or ld % 4 != 0) use at most
// 4,096-element chunks: the 8,192-element form of that variant spills.
template <int EPT>
static int launch_e(const SampleArgs &a, bool vec, hipStream_t s)
{
    if constexpr (EPT == 32) {
        if (!vec) return (int)hipErrorInvalidValue;
        return a.lp_on ? launch_t<32, true, true>(a, s) : launch_t<32, true, false>(a, s);
    } else {
        if (a.lp_on) return vec ? launch_t<EPT, true, true>(a, s) : launch_t<EPT, false, true>(a, s);
        return vec ? launch_t<EPT, true, false>(a, s) : launch_t<EPT, false, false>(a, s);
    }
}

int launch_sample(const SampleArgs &a, int ept, bool vec, hipStream_t s)
{
    switch (ept) {
    case 4: return launch_e<4>(a, vec, s);
    case 8: return launch_e<8>(a, vec, s);
    case 16: return launch_e<16>(a, vec, s);
    case 32: return launch_e<32>(a, vec, s);
    default: return (int)hipErrorInvalidValue;
    }
}

// The streaming-read measuring stick: the sampler's grid, chunking and loads,
// with only a chunk maximum computed.
template <int EPT, bool VEC>
__global__ __launch_bounds__(kBlock) void read_rows_kernel(const float *x0, int rows, int V, int64_t ld,
                                                          int nchunks, int out_stride, float *out,
                                                          int early)
{
    const int lb = logical_block(early);
    if (lb < 0 || lb >= rows * nchunks) return;
    const int row = lb / nchunks, chunk = lb - row * nchunks;
    float v[EPT];
    load_chunk<EPT, VEC>(x0 + (int64_t)row * ld, chunk * EPT * kBlock, V, v);
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < EPT; ++e) m = fmaxf(m, v[e]);
    m = wave_max_f32(m);
    __shared__ float red[4];
    if (lane_id() == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
        out[(int64_t)row * out_stride + chunk] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <int EPT>
static void launch_read_t(const float *x, int rows, int V, int64_t ld, int nchunks, int out_stride,
                          float *out, bool vec, bool early, hipStream_t s)
{
    const dim3 g(grid_for(rows * nchunks, early ? 1 : 0));
    if (vec)
        hipLaunchKernelGGL((read_rows_kernel<EPT, true>), g, dim3(kBlock), 0, s, x, rows, V, ld,
                           nchunks, out_stride, out, early ? 1 : 0);
    else
        hipLaunchKernelGGL((read_rows_kernel<EPT, false>), g, dim3(kBlock), 0, s, x, rows, V, ld,
                           nchunks, out_stride, out, early ? 1 : 0);
}

int launch_read_rows(const float *x, int rows, int V, int64_t ld, int nchunks, int out_stride,
                     float *out, int ept, bool vec, bool early, hipStream_t s)
{
    switch (ept) {
    case 4: launch_read_t<4>(x, rows, V, ld, nchunks, out_stride, out, vec, early, s); break;
    case 8: launch_read_t<8>(x, rows, V, ld, nchunks, out_stride, out, vec, early, s); break;
    case 16: launch_read_t<16>(x, rows, V, ld, nchunks, out_stride, out, vec, early, s); break;
    case 32: launch_read_t<32>(x, rows, V, ld, nchunks, out_stride, out, vec, early, s); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

__global__ void zero_u32_kernel(uint32_t *p, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

int launch_zero_u32(uint32_t *p, size_t n, hipStream_t s)
{
    if (n == 0) return 0;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return (int)hipGetLastError();
}

}  // namespace rts
