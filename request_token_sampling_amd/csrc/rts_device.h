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

// ---------------------------------------------------------------------------
// DPP (data-parallel primitives) cross-lane steps.  Row ops move data inside
// 16-lane rows; row_bcast15/31 carry a row's last lane into the next rows.
// Lanes whose source is out of range or masked off read 0, the identity of
// the sums and unsigned maxima below.  These stay in the VALU, unlike
// LDS-routed shuffles (ds_bpermute / ds_swizzle).
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, BANK_MASK, true);
}

template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double x)
{
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = dpp_u32<CTRL, ROW_MASK, BANK_MASK>((uint32_t)b);
    const uint32_t hi = dpp_u32<CTRL, ROW_MASK, BANK_MASK>((uint32_t)(b >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x)
{
    const uint32_t lo = dpp_u32<CTRL, ROW_MASK, BANK_MASK>((uint32_t)x);
    const uint32_t hi = dpp_u32<CTRL, ROW_MASK, BANK_MASK>((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr3 = 0x113, kRowShr4 = 0x114,
              kRowShr8 = 0x118, kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes: within rows by shifts of 1..3, 4
// and 8, then across rows by the two broadcasts.
__device__ __forceinline__ double wave_scan_f64(double x)
{
    double s = x + dpp_f64<kRowShr1>(x);
    s = s + dpp_f64<kRowShr2>(x);
    s = s + dpp_f64<kRowShr3>(x);
    s = s + dpp_f64<kRowShr4, 0xF, 0xE>(s);
    s = s + dpp_f64<kRowShr8, 0xF, 0xC>(s);
    s = s + dpp_f64<kRowBcast15, 0xA, 0xF>(s);
    s = s + dpp_f64<kRowBcast31, 0xC, 0xF>(s);
    return s;
}

// Inclusive running maximum of unsigned 64-bit keys; lane 63 holds the
// maximum of the wave.
__device__ __forceinline__ uint64_t wave_scan_max_u64(uint64_t v)
{
    uint64_t o;
    o = dpp_u64<kRowShr1>(v); v = o > v ? o : v;
    o = dpp_u64<kRowShr2>(v); v = o > v ? o : v;
    o = dpp_u64<kRowShr4, 0xF, 0xE>(v); v = o > v ? o : v;
    o = dpp_u64<kRowShr8, 0xF, 0xC>(v); v = o > v ? o : v;
    o = dpp_u64<kRowBcast15, 0xA, 0xF>(v); v = o > v ? o : v;
    o = dpp_u64<kRowBcast31, 0xC, 0xF>(v); v = o > v ? o : v;
    return v;
}

// Values of one lane (uniform lane index) in every lane.
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int l)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
__device__ __forceinline__ int32_t lane_i32(int32_t v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_f32(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double lane_f64(double v, int l)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint64_t r = ((uint64_t)lane_u32((uint32_t)(b >> 32), l) << 32) | lane_u32((uint32_t)b, l);
    return __longlong_as_double((long long)r);
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l)
{
    return ((uint64_t)lane_u32((uint32_t)(v >> 32), l) << 32) | lane_u32((uint32_t)v, l);
}

// Wave reductions built on the DPP steps; every lane gets the result.
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ float dpp_max_f32(float v)
{
    // lanes without a source keep -inf, the identity of the maximum
    const float o = __int_as_float(__builtin_amdgcn_update_dpp(
        (int)0xFF800000, __float_as_int(v), CTRL, ROW_MASK, BANK_MASK, false));
    return fmaxf(v, o);
}

__device__ __forceinline__ float wave_max_f32(float v)
{
    v = dpp_max_f32<kRowShr1>(v);
    v = dpp_max_f32<kRowShr2>(v);
    v = dpp_max_f32<kRowShr4, 0xF, 0xE>(v);
    v = dpp_max_f32<kRowShr8, 0xF, 0xC>(v);
    v = dpp_max_f32<kRowBcast15, 0xA, 0xF>(v);
    v = dpp_max_f32<kRowBcast31, 0xC, 0xF>(v);
    return lane_f32(v, 63);
}

__device__ __forceinline__ double wave_sum_f64(double v) { return lane_f64(wave_scan_f64(v), 63); }

__device__ __forceinline__ float wave_sum_f32(float x)
{
    float s = x + __uint_as_float(dpp_u32<kRowShr1>(__float_as_uint(x)));
    s = s + __uint_as_float(dpp_u32<kRowShr2>(__float_as_uint(x)));
    s = s + __uint_as_float(dpp_u32<kRowShr3>(__float_as_uint(x)));
    s = s + __uint_as_float(dpp_u32<kRowShr4, 0xF, 0xE>(__float_as_uint(s)));
    s = s + __uint_as_float(dpp_u32<kRowShr8, 0xF, 0xC>(__float_as_uint(s)));
    s = s + __uint_as_float(dpp_u32<kRowBcast15, 0xA, 0xF>(__float_as_uint(s)));
    s = s + __uint_as_float(dpp_u32<kRowBcast31, 0xC, 0xF>(__float_as_uint(s)));
    return lane_f32(s, 63);
}

// The value held by lane (lane ^ J), J in {1, 2, 4, 8, 16, 32}: DPP quad
// permutes for 1 and 2, row shifts for 4, a row rotation for 8, and for 16
// and 32 gfx950's row-swap permutes (v_permlane16_swap / v_permlane32_swap
// of a register with itself leave the even and the odd 16-lane rows, or the
// two 32-lane halves, in every lane), all in the VALU.
template <int J>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t x)
{
    if constexpr (J == 1) {
        return dpp_u64<0xB1>(x);  // quad_perm [1, 0, 3, 2]
    } else if constexpr (J == 2) {
        return dpp_u64<0x4E>(x);  // quad_perm [2, 3, 0, 1]
    } else if constexpr (J == 4) {
        const uint64_t up = dpp_u64<0x104>(x), down = dpp_u64<0x114>(x);  // row_shl:4, row_shr:4
        return (lane_id() & 4) ? down : up;
    } else if constexpr (J == 8) {
        return dpp_u64<0x128>(x);  // row_ror:8
    } else if constexpr (J == 16) {
        // r[0]: rows 0, 0, 2, 2 of x; r[1]: rows 1, 1, 3, 3
        const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
        const bool odd = (lane_id() & 16) != 0;
        return ((uint64_t)(odd ? hi[0] : hi[1]) << 32) | (odd ? lo[0] : lo[1]);
    } else {
        static_assert(J == 32, "lane distance");
        // r[0]: lanes 0-31 of x in both halves; r[1]: lanes 32-63
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
        const bool upper = (lane_id() & 32) != 0;
        return ((uint64_t)(upper ? hi[0] : hi[1]) << 32) | (upper ? lo[0] : lo[1]);
    }
}

// Bitonic sort, descending, of one (ONE) or two (x1 = element lane + 64)
// u64 keys per lane across the wave (Batcher's network: sizes 2..N, each a
// merge of distance SIZE/2 .. 1).  Zero keys sink to the end.
__device__ __forceinline__ uint64_t keep(uint64_t x, uint64_t y, bool take_max)
{
    return ((x > y) == take_max) ? x : y;
}

template <int SIZE, int J, bool TWO>
__device__ __forceinline__ void bitonic_steps(uint64_t &x0, uint64_t &x1)
{
    const int lane = lane_id();
    const bool lower = (lane & J) == 0;
    const bool d0 = (lane & SIZE) == 0, d1 = ((lane + 64) & SIZE) == 0;
    const uint64_t y0 = xor_lane_u64<J>(x0);
    if constexpr (TWO) {
        const uint64_t y1 = xor_lane_u64<J>(x1);
        x1 = keep(x1, y1, d1 == lower);
    }
    x0 = keep(x0, y0, d0 == lower);
    if constexpr (J > 1) bitonic_steps<SIZE, J / 2, TWO>(x0, x1);
}

template <int SIZE, bool TWO>
__device__ __forceinline__ void bitonic_sizes(uint64_t &x0, uint64_t &x1)
{
    bitonic_steps<SIZE, SIZE / 2, TWO>(x0, x1);
    if constexpr (SIZE < 64) bitonic_sizes<SIZE * 2, TWO>(x0, x1);
}

template <bool TWO>
__device__ __forceinline__ void wave_sort_desc(uint64_t &x0, uint64_t &x1)
{
    bitonic_sizes<2, TWO>(x0, x1);
    if constexpr (TWO) {
        // size 128: x0 holds elements 0..63 (a descending run), x1 elements
        // 64..127 (ascending): one in-lane step, then distances 32 .. 1
        const uint64_t hi = x0 > x1 ? x0 : x1, lo = x0 > x1 ? x1 : x0;
        x0 = hi;
        x1 = lo;
        bitonic_steps<128, 32, true>(x0, x1);
    }
}

// Largest t (to BITS leading bits) with #{keys >= t} >= k, over the four
// keys a[0..3] held by each lane of the wave (256 keys), settled two bits per
// step: the three thresholds of a step are counted together.  Every wave that
// runs this on the same keys gets the same t, so no broadcast is needed.
template <int BITS>
__device__ __forceinline__ uint32_t kth_largest_key_256_q(const uint32_t a[4], int k)
{
    static_assert(BITS % 2 == 0, "two bits per step");
    uint32_t t = 0;
#pragma unroll
    for (int b = 30; b >= 32 - BITS; b -= 2) {
        const uint32_t c1 = t | (1u << b), c2 = t | (2u << b), c3 = t | (3u << b);
        const int n1 = __popcll(__ballot(a[0] >= c1)) + __popcll(__ballot(a[1] >= c1)) +
                       __popcll(__ballot(a[2] >= c1)) + __popcll(__ballot(a[3] >= c1));
        const int n2 = __popcll(__ballot(a[0] >= c2)) + __popcll(__ballot(a[1] >= c2)) +
                       __popcll(__ballot(a[2] >= c2)) + __popcll(__ballot(a[3] >= c2));
        const int n3 = __popcll(__ballot(a[0] >= c3)) + __popcll(__ballot(a[1] >= c3)) +
                       __popcll(__ballot(a[2] >= c3)) + __popcll(__ballot(a[3] >= c3));
        t = (n3 >= k) ? c3 : (n2 >= k) ? c2 : (n1 >= k) ? c1 : t;
    }
    return t;
}

// A lower bound of the k-th largest of the 256 keys a[0..3] of every lane,
// found over fewer keys: each lane keeps the largest of its four (G = 1) or
// the two largest (G = 2), so the search counts 64 * G keys instead of 256.
// At least k of the kept keys are >= t and each is a different lane key, so
// t is still at most the k-th largest of the 256; it admits a few more
// candidates, and a step costs G ballots per threshold, not four.
template <int BITS, int G>
__device__ __forceinline__ uint32_t kth_largest_group_max(const uint32_t a[4], int k)
{
    static_assert(BITS % 2 == 0 && (G == 1 || G == 2 || G == 4), "two bits per step");
    uint32_t g[G];
    if constexpr (G == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) g[i] = a[i];
    } else if constexpr (G == 2) {
        const uint32_t h01 = a[0] > a[1] ? a[0] : a[1], l01 = a[0] > a[1] ? a[1] : a[0];
        const uint32_t h23 = a[2] > a[3] ? a[2] : a[3], l23 = a[2] > a[3] ? a[3] : a[2];
        g[0] = h01 > h23 ? h01 : h23;
        const uint32_t m = h01 > h23 ? h23 : h01, l = l01 > l23 ? l01 : l23;
        g[1] = m > l ? m : l;
    } else {
        const uint32_t m0 = a[0] > a[1] ? a[0] : a[1], m1 = a[2] > a[3] ? a[2] : a[3];
        g[0] = m0 > m1 ? m0 : m1;
    }
    uint32_t t = 0;
#pragma unroll
    for (int b = 30; b >= 32 - BITS; b -= 2) {
        const uint32_t c1 = t | (1u << b), c2 = t | (2u << b), c3 = t | (3u << b);
        int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            n1 += __popcll(__ballot(g[i] >= c1));
            n2 += __popcll(__ballot(g[i] >= c2));
            n3 += __popcll(__ballot(g[i] >= c3));
        }
        t = (n3 >= k) ? c3 : (n2 >= k) ? c2 : (n1 >= k) ? c1 : t;
    }
    return t;
}

// Selection threshold over 256 lane keys (top 16 bits) from the kept keys
// above: one per lane for k <= 24, two for larger k (on N(0, 3) rows of
// 8,192-id chunks this admits 24 candidates at k = 20 and 79 at k = 64,
// against 21 and 74 for the full search).  When fewer than k kept keys lie
// above the key of -inf (sparse chunks, masked rows) the search runs again
// over all 256 keys, so the degenerate path is taken exactly when the full
// search would take it.
__device__ __forceinline__ uint32_t selection_threshold(const uint32_t a[4], int k)
{
    const uint32_t t = k <= 24 ? kth_largest_group_max<16, 1>(a, k) : kth_largest_group_max<16, 2>(a, k);
    return t > 0x007FFFFFu ? t : kth_largest_key_256_q<16>(a, k);
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

// ---------------------------------------------------------------------------
// XCD-aware placement for small launches.  Workgroups are dealt to the eight
// XCDs round-robin (blockIdx % 8), and on MI355X the dispatcher starts XCDs
// 0-1 about 1.5-2 us before XCDs 2-7 (measured with wall-clock stamps).  A
// launch whose work fits in the 64 CUs of XCDs 0-1 is padded to eight times
// its width and only workgroups with blockIdx % 8 < 2 take work; the others
// exit at once.  Returns the logical workgroup index, or -1.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int logical_block(int early_xcds_only)
{
    const int b = (int)blockIdx.x;
    if (!early_xcds_only) return b;
    const int x = b & 7;
    return (x < 2) ? ((b >> 3) * 2 + x) : -1;
}

// ---------------------------------------------------------------------------
// Row-completion protocol.  Every workgroup of a row publishes its results,
// then takes a ticket; the one drawing the last ticket merges the row.
//
// The published words are written with device-scope (agent) atomic stores and
// read back with device-scope atomic loads: on gfx950 these carry the device
// coherence bit, so they are written through to, and read from, the level
// shared by all XCDs, not an XCD's private L2.  Each thread waits for its
// stores to complete (vmcnt = 0) before the workgroup barrier, and only then
// does one thread take the ticket with a device-scope atomic add.  A release
// fence at agent scope would also order them, but it writes back the whole
// L2 of the XCD and its acquire invalidates it, once per workgroup; with
// ~1,000 workgroups per launch that maintenance dominated the kernel.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void publish_u64(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t read_published_u64(const uint64_t *p)
{
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// s_waitcnt with vmcnt = 0 and the other counters left free (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
__device__ __forceinline__ void wait_stores_complete() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ bool take_last_ticket(uint32_t *ticket, uint32_t n, uint32_t *s_flag)
{
    wait_stores_complete();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old =
            __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = (old == n - 1u) ? 1u : 0u;
    }
    __syncthreads();
    return *s_flag != 0u;
}

}  // namespace rts
