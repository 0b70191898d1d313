// c_abi_consumer.cpp -- a plain C++ user of the library through include/rts.h
// and the HIP runtime alone (no Python, no torch).  It reads B rows of V fp32
// logits from a file, samples them (even rows: top_k 8, top_p 0.9, min_p
// 0.05, temperature 0.8, seed 42, counter = row; odd rows: greedy), asks for
// the top-5 logprobs of the sampled tokens, and writes everything to a file:
//   in:  int32 B, int32 V, float logits[B][V]
//   out: int32 token[B], int32 counts[B][3], int32 kept_ids[B][64],
//        float token_lp[B], int32 top_ids[B][5], float top_lp[B][5]
// Exit status 0 on success; otherwise the failing call and rts_last_error()
// go to stderr.
#include <cstdint>
#include <cstdio>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "rts.h"

#define HIP_OK(x)                                                                   \
    do {                                                                            \
        const hipError_t e_ = (x);                                                  \
        if (e_ != hipSuccess) {                                                     \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));            \
            return 2;                                                               \
        }                                                                           \
    } while (0)

#define RTS_CALL(x)                                                                 \
    do {                                                                            \
        const int e_ = (x);                                                         \
        if (e_ != RTS_OK) {                                                         \
            std::fprintf(stderr, "%s: %s (%s)\n", #x, rts_strerror(e_), rts_last_error()); \
            return 3;                                                               \
        }                                                                           \
    } while (0)

int main(int argc, char **argv)
{
    if (argc != 3) {
        std::fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
        return 1;
    }
    FILE *in = std::fopen(argv[1], "rb");
    if (in == nullptr) return 1;
    int32_t dims[2];
    if (std::fread(dims, 4, 2, in) != 2 || dims[0] <= 0 || dims[1] <= 0) return 1;
    const int64_t B = dims[0], V = dims[1];
    std::vector<float> x((size_t)(B * V));
    if (std::fread(x.data(), 4, x.size(), in) != x.size()) return 1;
    std::fclose(in);

    constexpr int32_t kTopN = 5;
    float *d_x = nullptr, *d_lp = nullptr, *d_top_lp = nullptr;
    int32_t *d_tok = nullptr, *d_counts = nullptr, *d_kept = nullptr, *d_top_ids = nullptr;
    void *d_ws = nullptr;
    size_t ws_bytes = 0;
    RTS_CALL(rts_workspace_bytes(B, V, &ws_bytes));
    HIP_OK(hipMalloc((void **)&d_x, x.size() * 4));
    HIP_OK(hipMalloc((void **)&d_tok, (size_t)B * 4));
    HIP_OK(hipMalloc((void **)&d_counts, (size_t)B * 3 * 4));
    HIP_OK(hipMalloc((void **)&d_kept, (size_t)B * RTS_KEPT * 4));
    HIP_OK(hipMalloc((void **)&d_lp, (size_t)B * 4));
    HIP_OK(hipMalloc((void **)&d_top_ids, (size_t)B * kTopN * 4));
    HIP_OK(hipMalloc((void **)&d_top_lp, (size_t)B * kTopN * 4));
    HIP_OK(hipMalloc(&d_ws, ws_bytes));
    HIP_OK(hipMemcpy(d_x, x.data(), x.size() * 4, hipMemcpyHostToDevice));
    RTS_CALL(rts_workspace_init(d_ws, ws_bytes, nullptr));

    std::vector<rts_row_params> p((size_t)B);
    for (int64_t r = 0; r < B; ++r) {
        rts_row_params &q = p[(size_t)r];
        const bool sampled = r % 2 == 0;
        q.temperature = sampled ? 0.8f : 0.0f;
        q.top_k = sampled ? 8 : 0;
        q.top_p = sampled ? 0.9f : 1.0f;
        q.min_p = sampled ? 0.05f : 0.0f;
        q.penalty_repeat = 1.0f;
        q.penalty_freq = 0.0f;
        q.penalty_present = 0.0f;
        q.penalty_last_n = 0;
        q.history_row = -1;
        q.reserved = 0;
        q.seed = sampled ? 42u : 0u;
        q.counter = sampled ? (uint64_t)r : 0u;
    }
    RTS_CALL(rts_sample_tokens(d_x, B, V, V, p.data(), nullptr, 0, 0, nullptr, d_tok, d_counts,
                               d_kept, nullptr, nullptr, nullptr, 0, nullptr, nullptr, d_ws,
                               ws_bytes, nullptr));
    RTS_CALL(rts_token_logprobs(d_x, B, V, V, d_tok, kTopN, nullptr, nullptr, d_lp, d_top_ids,
                                d_top_lp, d_ws, ws_bytes, nullptr));
    HIP_OK(hipDeviceSynchronize());

    std::vector<int32_t> tok((size_t)B), counts((size_t)B * 3), kept((size_t)B * RTS_KEPT),
        top_ids((size_t)B * kTopN);
    std::vector<float> lp((size_t)B), top_lp((size_t)B * kTopN);
    HIP_OK(hipMemcpy(tok.data(), d_tok, tok.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(counts.data(), d_counts, counts.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(kept.data(), d_kept, kept.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lp.data(), d_lp, lp.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(top_ids.data(), d_top_ids, top_ids.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(top_lp.data(), d_top_lp, top_lp.size() * 4, hipMemcpyDeviceToHost));

    FILE *out = std::fopen(argv[2], "wb");
    if (out == nullptr) return 1;
    std::fwrite(tok.data(), 4, tok.size(), out);
    std::fwrite(counts.data(), 4, counts.size(), out);
    std::fwrite(kept.data(), 4, kept.size(), out);
    std::fwrite(lp.data(), 4, lp.size(), out);
    std::fwrite(top_ids.data(), 4, top_ids.size(), out);
    std::fwrite(top_lp.data(), 4, top_lp.size(), out);
    std::fclose(out);

    HIP_OK(hipFree(d_x));
    HIP_OK(hipFree(d_tok));
    HIP_OK(hipFree(d_counts));
    HIP_OK(hipFree(d_kept));
    HIP_OK(hipFree(d_lp));
    HIP_OK(hipFree(d_top_ids));
    HIP_OK(hipFree(d_top_lp));
    HIP_OK(hipFree(d_ws));
    return 0;
}
