// rts_noalloc.hip -- rts_sample_tokens_noalloc: the sampling call for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).  The scratch memory
// that rts_sample_tokens keeps in the caller's workspace (row tickets, chunk
// key lists, logprob partials) is here one file-scope device array of
// kScratchBytes, which every GPU the library runs on holds until the process
// ends.  The call itself allocates nothing.
//
// In host code the array's name is a host-side stand-in, not a device
// address: its device address is looked up once per device, with that device
// current, by hipGetSymbolAddress, and only that address is passed to
// kernels.  Every call on one GPU shares that GPU's array: calls that can
// overlap on one GPU (two streams, two host threads) race on it.
#include <mutex>

#include "rts.h"
#include "rts_internal.h"

namespace {

// 16 MiB: a launch of 64 rows at V = 248,320 needs 10.6 MB; 64 rows fit up
// to V = 394,240, fewer rows fit larger vocabularies.
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices];  // the array's device address, per device

// The current device's copy of the array.  On first use its tickets are
// zeroed by a kernel on the call's stream (no memset node, so a call under
// stream capture records a plain kernel); the sampling kernels return them
// to zero at the end of every call after that.
int device_scratch(void **out, hipStream_t stream)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return rts::set_error(RTS_EDEVICE, "rts_sample_tokens_noalloc: no usable current device");
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return rts::set_error(RTS_EDEVICE,
                                  "rts_sample_tokens_noalloc: hipGetSymbolAddress of the scratch "
                                  "array on device %d: %s", dev, hipGetErrorString(e));
        const int z = rts::launch_zero_u32(static_cast<uint32_t *>(p), rts::kTicketBytes / 4u, stream);
        if (z != 0)
            return rts::set_error(RTS_EDEVICE, "rts_sample_tokens_noalloc: zero kernel: %s",
                                  hipGetErrorString((hipError_t)z));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return RTS_OK;
}

}  // namespace

extern "C" {

size_t rts_noalloc_scratch_bytes(void) { return kScratchBytes; }

int rts_sample_tokens_noalloc(const float *logits, int64_t B, int64_t V, int64_t ld,
                              const rts_row_params *params,
                              const int32_t *history, int64_t H, int64_t ldh,
                              const int32_t *history_len,
                              int32_t *token, int32_t *counts, int32_t *kept_ids,
                              float *kept_logits, uint32_t *philox_x0,
                              uint64_t *counters, int64_t counter_stride,
                              const rts_logprob_request *lp, const rts_sample_extras *ex,
                              hipStream_t stream)
{
    rts::clear_last_error();
    if (B > 0 && V > 0 && V <= RTS_MAX_V) {
        size_t need = 0;
        if (rts_workspace_bytes(B, V, &need) == RTS_OK && need > kScratchBytes)
            return rts::set_error(RTS_ENOSPC,
                                  "rts_sample_tokens_noalloc: %lld rows of V = %lld need %zu bytes "
                                  "of scratch; the library's static scratch holds %zu",
                                  (long long)B, (long long)V, need, kScratchBytes);
    }
    // every argument is checked before the scratch is looked up, so a refused
    // call touches no device
    return rts::sample_tokens_impl(logits, B, V, ld, params, history, H, ldh, history_len, token,
                                   counts, kept_ids, kept_logits, philox_x0, counters,
                                   counter_stride, lp, ex, nullptr, kScratchBytes, device_scratch,
                                   stream);
}

}  // extern "C"
