// Reference Philox4x32-10 words from rocRAND's open-source host/device engine
// (rocrand_philox4x32_10.h).  Used only by the oracle's pin test: reads
// (seed, counter) pairs as uint64 from argv[1] and writes four uint32 words
// per pair to argv[2].  The engine is seeded with subsequence 0 and offset
// 4 * counter, which puts the counter's low and high words into the first two
// counter words of the block; its first four outputs are that block's words.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdint>
#include <cstdio>
#include <vector>

int main(int argc, char **argv)
{
    if (argc != 3) return 2;
    FILE *f = std::fopen(argv[1], "rb");
    if (!f) return 3;
    std::vector<unsigned long long> in;
    unsigned long long v;
    while (std::fread(&v, sizeof v, 1, f) == 1) in.push_back(v);
    std::fclose(f);
    std::vector<uint32_t> out;
    for (size_t i = 0; i + 1 < in.size(); i += 2) {
        const unsigned long long seed = in[i], counter = in[i + 1];
        rocrand_device::philox4x32_10_engine e(seed, 0ULL, 0ULL);
        // advance by whole blocks in pieces so 4 * counter never overflows
        unsigned long long c = counter;
        const unsigned long long step = 1ULL << 60;
        while (c >= step) { e.discard(4ULL * step); c -= step; }
        e.discard(4ULL * c);
        for (int w = 0; w < 4; ++w) out.push_back(e());
    }
    FILE *g = std::fopen(argv[2], "wb");
    if (!g) return 4;
    std::fwrite(out.data(), sizeof(uint32_t), out.size(), g);
    std::fclose(g);
    return 0;
}
