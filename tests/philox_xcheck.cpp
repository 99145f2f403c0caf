// Test-only cross-check: prints Philox4x32-10 words from rocRAND's source
// engine (rocrand/rocrand_philox4x32_10.h, compiled for the host) so the
// oracle's independent NumPy implementation can be compared with it.
// Usage: philox_xcheck SEED SUBSEQUENCE OFFSET N  -> N lines, word at OFFSET+i.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
    if (argc != 5) {
        std::fprintf(stderr, "usage: %s seed subsequence offset n\n", argv[0]);
        return 2;
    }
    const unsigned long long seed = std::strtoull(argv[1], nullptr, 0);
    const unsigned long long sub = std::strtoull(argv[2], nullptr, 0);
    const unsigned long long off = std::strtoull(argv[3], nullptr, 0);
    const long n = std::strtol(argv[4], nullptr, 0);
    for (long i = 0; i < n; ++i) {
        rocrand_device::philox4x32_10_engine eng(seed, sub, off + static_cast<unsigned long long>(i));
        std::printf("%u\n", eng.next());
    }
    return 0;
}
