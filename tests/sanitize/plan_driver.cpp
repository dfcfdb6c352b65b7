// Host-side plan and argument checks of the KDA library, driven over a grid of shapes (valid,
// invalid and at the limits) and call arguments, for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer.  Prints one line per counted outcome; exits non-zero if a check
// that must fail passes.
#include <cstdint>
#include <cstdio>
#include <limits>
#include <vector>

#include "kda_plan.h"

namespace {

int fails = 0;

void expect(bool ok, const char* what) {
    if (!ok) {
        std::printf("FAIL %s\n", what);
        ++fails;
    }
}

// Fake device addresses: every region of a call in its own 2^59-byte window, so none overlap
// (shapes whose tensors could exceed a window skip the checks that need disjoint regions).
const void* addr(int region) { return reinterpret_cast<const void*>(uintptr_t(region + 1) << 59); }
static_assert(sizeof(uintptr_t) == 8, "12 windows of 2^59 bytes need 64-bit addresses");

}  // namespace

int main() {
    const int layouts[] = {-1, 0, 1, 2, 3};
    const int batches[] = {0, 1, 2, 5, 300, std::numeric_limits<int>::max()};
    const int lens[] = {0, 1, 63, 64, 65, 4100, 131072, std::numeric_limits<int>::max() - 10,
                        std::numeric_limits<int>::max()};
    const int heads[][2] = {{1, 1}, {3, 3}, {4, 16}, {2, 3}, {0, 1}, {1, 0}, {32, 32},
                            {1, 1 << 17}, {1 << 20, 1 << 20}};
    const int dims[][2] = {{128, 128}, {64, 64}, {64, 128}, {32, 32}, {256, 256}, {0, 0}};
    const float scales[] = {0.088f, std::numeric_limits<float>::quiet_NaN(),
                            std::numeric_limits<float>::infinity()};
    const uint32_t flag_sets[] = {0u, 1u, 3u, 7u, 8u, 11u, 12u, 16u, 0x80000000u};
    long n_ok = 0, n_bad = 0, n_calls = 0;
    for (int lay : layouts)
        for (int b : batches)
            for (int s : lens)
                for (const auto& h : heads)
                    for (const auto& d : dims)
                        for (float sc : scales)
                            for (uint32_t fl : flag_sets) {
                                kda_shape sh{lay, b, s, h[0], h[1], d[0], d[1], sc, fl};
                                kda::Plan p;
                                const kda_status st = kda::make_plan(&sh, &p);
                                if (st != KDA_OK) {
                                    ++n_bad;
                                    continue;
                                }
                                ++n_ok;
                                expect(p.total > 0, "workspace size");
                                expect(p.intra_blocks > 0 && p.intra_blocks < (int64_t(1) << 31),
                                       "intra grid");
                                // a valid call, then each pointer taken away in turn
                                const void* ptr[10];
                                for (int i = 0; i < 10; ++i) ptr[i] = addr(i);
                                const int32_t* cu = static_cast<const int32_t*>(ptr[6]);
                                const kda_raw_gate gate{static_cast<const float*>(addr(10)),
                                                        static_cast<const float*>(addr(11)), -5.f};
                                auto call = [&](const void* const* x, size_t ws_bytes) {
                                    ++n_calls;
                                    return kda::check_call(
                                        &sh, p, x[0], x[1], x[2], x[3],
                                        (fl & KDA_RAW_GATE) ? &gate : nullptr,
                                        x[4], static_cast<const float*>(x[5]),
                                        static_cast<const int32_t*>(x[6]), x[7],
                                        static_cast<const float*>(x[8]), x[9], ws_bytes);
                                };
                                (void)cu;
                                const double tokens = lay == 2 ? double(s) : double(b) * s;
                                if (tokens * h[1] * d[0] * 4.0 >= 0x1p58 || double(p.total) >= 0x1p58)
                                    continue;
                                expect(call(ptr, p.total) == KDA_OK, "valid call");
                                expect(call(ptr, p.total - 1) == KDA_ERR_WORKSPACE, "short ws");
                                for (int i : {0, 1, 2, 3, 4, 7, 9}) {
                                    const void* x[10];
                                    for (int j = 0; j < 10; ++j) x[j] = ptr[j];
                                    x[i] = nullptr;
                                    expect(call(x, p.total) != KDA_OK, "null pointer");
                                }
                                {   // out over v
                                    const void* x[10];
                                    for (int j = 0; j < 10; ++j) x[j] = ptr[j];
                                    x[7] = x[2];
                                    expect(call(x, p.total) == KDA_ERR_INVALID_ARG, "alias");
                                }
                            }
    std::printf("shapes ok %ld, rejected %ld, calls %ld, failures %d\n", n_ok, n_bad, n_calls,
                fails);
    return fails == 0 ? 0 : 1;
}
