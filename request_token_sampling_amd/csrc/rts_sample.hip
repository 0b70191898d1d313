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
#include "rts_select.h"

namespace rts {

template <int EPT>
struct SampleSmem {
    SelectSmem s;
    uint32_t pen_bits[EPT * kBlock / 32];  // one bit per id of the chunk
    uint32_t pen_cnt[EPT * kBlock / 2];    // two 16-bit counts per word
};

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

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int EPT, bool VEC>
__global__ __launch_bounds__(kBlock, kMinWavesPerSimd) void sample_kernel(const SampleArgs a)
{
    constexpr int CH = EPT * kBlock;
    constexpr int NQ = EPT / 4;
    __shared__ SampleSmem<EPT> sm;

    const int tid = threadIdx.x;
    const int slot = blockIdx.x / a.nchunks;
    const int chunk = blockIdx.x - slot * a.nchunks;
    const SampleRow R = a.row[slot];
    const int V = a.V;
    const int n_eff = (int)(R.pack & 0xFFFFu);
    const int k = (int)((R.pack >> 16) & 0x7Fu);
    const bool greedy = ((R.pack >> 24) & 1u) != 0u;
    const int base = chunk * CH;
    const float *x = a.logits + (int64_t)slot * a.ld;

    // Issue every load of the chunk first; the bitmap build below overlaps
    // them.  Ids past V (only in the last chunk) read as NaN: never selected.
    float v[EPT];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int i0 = base + q * 1024 + tid * 4;
        if (VEC && i0 + 4 <= V) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(x + i0);
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

    if (n_eff > 0) {
        for (int w = tid; w < CH / 32; w += kBlock) sm.pen_bits[w] = 0u;
        for (int w = tid; w < CH / 2; w += kBlock) sm.pen_cnt[w] = 0u;
        __syncthreads();
        const int32_t *h = a.history + R.hist_off;
        for (int j = tid; j < n_eff; j += kBlock) {
            const int32_t id = h[j];
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

    uint64_t *list = a.keys + (int64_t)slot * a.keys_stride;
    chunk_topk<EPT>(sm.s, v, base, V, k, list + (int64_t)chunk * k);

    if (!take_last_ticket(&a.tickets[slot], (uint32_t)a.nchunks, &sm.s.flag)) return;

    // ---- the last workgroup of the row: merge, then the cuts and the draw.
    list_topk(sm.s, list, a.nchunks, k);

    if ((tid >> 6) != 0) return;
    const int lane = lane_id();
    const uint64_t key = (lane < k) ? sm.s.sel[lane] : 0ull;
    const bool valid = key != 0ull;
    const int32_t id = valid ? (int32_t)key_index(key) : -1;
    const float y = valid ? key_logit(key) : -INFINITY;
    if (a.kept_ids) a.kept_ids[(int64_t)slot * kMaxK + lane] = id;
    if (a.kept_logits) a.kept_logits[(int64_t)slot * kMaxK + lane] = y;

    const float y0 = lane_f32(y, 0);
    // the row's Philox counter: device-resident when given (read here, then
    // advanced below), else the caller's value from the argument block
    const uint64_t ctr = a.counters ? a.counters[slot] : R.counter;
    int m = 1, n = 1, pick = 0;
    uint32_t x0 = 0u;
    if (!greedy) {
        // Everything that does not depend on the cuts first, so the fp64
        // exponentials and the Philox rounds overlap: top_p weights
        // exp(y - y0), tempered weights exp((y - y0) / T), and x0.
        const double dy = (double)y - (double)y0;
        const bool head_masked = (y0 == -INFINITY);
        const double d = (lane < k && !head_masked) ? exp(dy) : 0.0;
        const double w = (lane < k && !head_masked) ? exp(dy / (double)R.temperature) : 0.0;
        x0 = philox4x32_10_x0(ctr, R.seed);
        // min_p: keep the prefix with logit >= head + logf(min_p), in fp32.
        const float thr = y0 + R.lnp;
        m = __popcll(__ballot(lane < k && y >= thr));
        m = m < 1 ? 1 : m;
        // top_p: shortest prefix of the min_p survivors whose fp64 softmax
        // mass reaches top_p; a masked head (-inf) keeps one candidate.
        n = m;
        if (head_masked) {
            n = 1;
        } else if (!(R.top_p >= 1.0f)) {
            const double S = wave_scan_f64(lane < m ? d : 0.0);
            const double Z = lane_f64(S, m - 1);
            const uint64_t b = __ballot(lane < m && S / Z >= (double)R.top_p);
            n = b ? __ffsll((unsigned long long)b) : m;
        }
        // temperature, then the draw: u = x0 / 2^32 against the tempered CDF.
        const double u = (double)x0 * (1.0 / 4294967296.0);
        pick = n - 1;
        if (n > 1) {
            const double S = wave_scan_f64(lane < n ? w : 0.0);
            const double Z = lane_f64(S, n - 1);
            const uint64_t b = __ballot(lane < n - 1 && S / Z > u);
            if (b) pick = __ffsll((unsigned long long)b) - 1;
        }
    }
    const int32_t tok = lane_i32(id, pick);
    if (lane == 0) {
        a.token[slot] = tok;
        if (a.counts) {
            a.counts[3 * (int64_t)slot + 0] = k;
            a.counts[3 * (int64_t)slot + 1] = m;
            a.counts[3 * (int64_t)slot + 2] = n;
        }
        if (a.philox_x0) a.philox_x0[slot] = x0;
        if (a.counters) a.counters[slot] = ctr + (uint64_t)a.counter_stride;
        a.tickets[slot] = 0u;  // ready for the next launch on this workspace
    }
}

template <int EPT, bool VEC>
static int launch_t(const SampleArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((sample_kernel<EPT, VEC>), dim3((unsigned)(a.rows * a.nchunks)),
                       dim3(kBlock), 0, s, a);
    return (int)hipGetLastError();
}

int launch_sample(const SampleArgs &a, int ept, bool vec, hipStream_t s)
{
    switch (ept) {
    case 4: return vec ? launch_t<4, true>(a, s) : launch_t<4, false>(a, s);
    case 8: return vec ? launch_t<8, true>(a, s) : launch_t<8, false>(a, s);
    case 16: return vec ? launch_t<16, true>(a, s) : launch_t<16, false>(a, s);
    case 32: return vec ? launch_t<32, true>(a, s) : launch_t<32, false>(a, s);
    default: return (int)hipErrorInvalidValue;
    }
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
