// rts_prior.hip -- the pages' earlier sampler designs, kept as measured
// ablations of the single-pass chunked kernel (page "#19 serve:
// per-request temperature/top_p/top_k/min_p/penalties sampling", "What
// changed": the sampled chain first ran in one thread per token, top_k as
// k sequential full-vocabulary scans; it then became one block per token,
// the k argmax rounds back to back inside it, each a two-level reduction;
// penalty counts come from a per-block token bitmap built in one atomicOr
// pass, a candidate scanning the window only when its bit is set, where
// the earlier recount scanned the window for every candidate).
//
// One workgroup per row.  Every round rereads the row (from L2 after the
// first) and keeps, per thread, the best key strictly below the previous
// round's pick; the kept sequence then goes through the same cuts and draw
// as the single-pass kernel, so the outputs are identical.
#include "rts_epilogue.h"

namespace rts {

template <int DESIGN>
__global__ __launch_bounds__(kBlock) void prior_kernel(const SampleArgs a)
{
    extern __shared__ uint32_t bm[];  // the row's penalty bitmap, one bit per id
    __shared__ SelectSmem sm;

    const int tid = threadIdx.x;
    const int slot = blockIdx.x;
    const SampleRow R = a.row[slot];
    const int V = a.V;
    const int n_eff = (int)(R.pack & 0xFFFFu);
    const int k = (int)((R.pack >> 16) & 0x7Fu);
    const bool greedy = ((R.pack >> 24) & 1u) != 0u;
    const float *x = a.logits + (int64_t)slot * a.ld;
    const int32_t *h = a.history + R.hist_off;
    // PRIOR_THREAD: all of the row's work in thread 0; the others only take
    // part in the barriers.
    const int nth = (DESIGN == PRIOR_THREAD) ? 1 : kBlock;
    const bool worker = tid < nth;

    if (DESIGN != PRIOR_RECOUNT && n_eff > 0) {
        if (worker)
            for (int w = tid; w < (V + 31) / 32; w += nth) bm[w] = 0u;
        __syncthreads();
        if (worker)
            for (int j = tid; j < n_eff; j += nth) {
                const int32_t id = h[j];
                if (id >= 0 && id < V) atomicOr(&bm[id >> 5], 1u << (id & 31));
            }
        __syncthreads();
    }

    uint64_t prev = ~0ull;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0ull;
        if (worker) {
            for (int i = tid; i < V; i += nth) {
                float y = sanitize(x[i]);
                const bool scan = n_eff > 0 &&
                                  (DESIGN == PRIOR_RECOUNT || ((bm[i >> 5] >> (i & 31)) & 1u));
                if (scan) {
                    uint32_t c = 0u;
                    for (int j = 0; j < n_eff; ++j) c += (h[j] == i) ? 1u : 0u;
                    if (c > 0u) y = penalize(y, c, R.rep, R.freq, R.present);
                }
                const uint64_t key = cand_key(y, (uint32_t)i);
                best = (key < prev && key > best) ? key : best;
            }
        }
        best = block_max_u64(sm, best);
        if (tid == 0) sm.sel[r] = best;
        prev = best;
    }
    __syncthreads();
    if ((tid >> 6) == 0) {
        const uint64_t ctr = a.counters ? a.counters[slot] : R.counter;
        const uint32_t x0 = greedy ? 0u : philox4x32_10_x0(ctr, R.seed);
        epilogue(a, R, sm, slot, k, greedy, ctr, x0);
    }
}

int launch_prior(const SampleArgs &a, int design, size_t lds_bytes, hipStream_t s)
{
    switch (design) {
    case PRIOR_THREAD:
        hipLaunchKernelGGL(prior_kernel<PRIOR_THREAD>, dim3(a.rows), dim3(kBlock), lds_bytes, s, a);
        break;
    case PRIOR_BLOCK:
        hipLaunchKernelGGL(prior_kernel<PRIOR_BLOCK>, dim3(a.rows), dim3(kBlock), lds_bytes, s, a);
        break;
    case PRIOR_RECOUNT:
        hipLaunchKernelGGL(prior_kernel<PRIOR_RECOUNT>, dim3(a.rows), dim3(kBlock), 0, s, a);
        break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

}  // namespace rts
