// rts_device.h -- device helpers shared by the sampler and logprob kernels:
// orderable keys, 64-lane wavefront primitives and the Philox4x32-10 block.
//
// Written for gfx950 (CDNA4): 64-lane wavefronts, 256-thread workgroups of
// four waves.  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rts_internal.h"

namespace rts {

// ---------------------------------------------------------------------------
// Orderable keys.  A candidate is (value, index) under the order of page
// "#19 serve: per-request temperature/top_p/top_k/min_p/penalties sampling",
// "What changed", the one-block-per-token paragraph: larger value first,
// equal values by lower index.  The 32-bit value key is monotone in the
// float (with -0 folded onto +0 so equal values compare equal); the 64-bit
// key appends the complemented index, so a larger key is always the better
// candidate and every key of a real element is non-zero (0 marks "none").
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t value_key(float v)
{
    uint32_t b = __float_as_uint(v);
    b = (v == 0.0f) ? 0u : b;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_to_value(uint32_t k)
{
    const uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(b);
}

__device__ __forceinline__ uint64_t cand_key(float v, uint32_t idx)
{
    return ((uint64_t)value_key(v) << 32) | (uint64_t)(~idx);
}

__device__ __forceinline__ uint32_t key_index(uint64_t k) { return ~(uint32_t)k; }
__device__ __forceinline__ float key_logit(uint64_t k) { return key_to_value((uint32_t)(k >> 32)); }

// Threshold key -> float threshold.  Keys at or below that of -inf (including
// 0, "no lane") admit every non-NaN value.
__device__ __forceinline__ float key_threshold(uint32_t t)
{
    return (t <= 0x007FFFFFu) ? -INFINITY : key_to_value(t);
}

// NaN counts as -inf and +inf as the largest finite float.
__device__ __forceinline__ float sanitize(float v)
{
    return (v != v) ? -INFINITY : fminf(v, 3.40282346638528859812e+38f);
}

// ---------------------------------------------------------------------------
// 64-lane wavefront primitives.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

__device__ __forceinline__ uint64_t lanes_below_mask()
{
    return (1ull << lane_id()) - 1ull;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m)
{
    const int lo = __shfl_xor((int)(uint32_t)v, m, 64);
    const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m, 64);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t o = shfl_xor_u64(v, m);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Inclusive prefix sum over the 64 lanes (Hillis-Steele).
__device__ __forceinline__ double wave_scan_f64(double v)
{
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const double o = __shfl_up(v, (unsigned)d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

// Largest t (to `bits` leading bits) with #{keys >= t} >= k, over the four
// keys a[0..3] held by each lane of the wave (256 keys).  Every wave that runs
// this on the same keys gets the same t, so no broadcast is needed.
template <int BITS>
__device__ __forceinline__ uint32_t kth_largest_key_256(const uint32_t a[4], int k)
{
    uint32_t t = 0;
#pragma unroll
    for (int b = 31; b >= 32 - BITS; --b) {
        const uint32_t c = t | (1u << b);
        const int cnt = __popcll(__ballot(a[0] >= c)) + __popcll(__ballot(a[1] >= c)) +
                        __popcll(__ballot(a[2] >= c)) + __popcll(__ballot(a[3] >= c));
        if (cnt >= k) t = c;
    }
    return t;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11): ten rounds of the 4x32 S-box with multipliers
// 0xD2511F53 / 0xCD9E8D57 and a Weyl key schedule 0x9E3779B9 / 0xBB67AE85.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t philox4x32_10_x0(uint64_t counter, uint64_t seed)
{
    uint32_t c0 = (uint32_t)counter, c1 = (uint32_t)(counter >> 32), c2 = 0u, c3 = 0u;
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c0;
}

// Row-completion ticket: every workgroup of a row publishes its results,
// then takes a ticket; the one drawing the last ticket merges the row.
// Release/acquire at agent scope so stores from other XCDs are visible.
__device__ __forceinline__ bool take_last_ticket(uint32_t *ticket, uint32_t n, uint32_t *s_flag)
{
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = atomicAdd(ticket, 1u);
        *s_flag = (old == n - 1u) ? 1u : 0u;
    }
    __syncthreads();
    const bool last = *s_flag != 0u;
    if (last) __threadfence();
    return last;
}

}  // namespace rts
