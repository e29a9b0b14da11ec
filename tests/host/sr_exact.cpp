// Host-side check of the stochastic-rounding cast's rounding step: the
// kernels' helper fp8q::sr_round, compiled as host code from their own header,
// against the oracle's orc_encode_sr.  The helper's result is monotone in the
// random word r, so for each v a bisection finds the smallest word t that
// rounds up; the oracle must give the same code at t - 1 and at t, and at the
// extreme words 0 and 2^32 - 1.  (Where no word rounds up -- v on the grid,
// or capped at the maximum -- only the extremes are compared.)  Codes are
// compared: the helper's value is encoded by the oracle's round-to-nearest
// encoder, which leaves an exact grid value unchanged.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "device_common.h"

extern "C" uint8_t orc_encode(float v, int fmt, int saturate);
extern "C" uint8_t orc_encode_sr(float v, uint32_t r, int fmt, int saturate);

static inline float f_of(uint32_t b) { float f; std::memcpy(&f, &b, 4); return f; }
static inline uint32_t b_of(float f) { uint32_t b; std::memcpy(&b, &f, 4); return b; }

template <int FMT>
static long check(float v) {
    auto code = [&](uint32_t r) { return orc_encode(fp8q::sr_round<FMT>(v, r), FMT, 0); };
    auto same = [&](uint32_t r) { return code(r) == orc_encode_sr(v, r, FMT, 0) ? 0 : 1; };
    long bad = same(0u) + same(0xffffffffu);
    const uint32_t down = b_of(fp8q::sr_round<FMT>(v, 0u));
    if (b_of(fp8q::sr_round<FMT>(v, 0xffffffffu)) != down) {
        uint32_t lo = 0u, hi = 0xffffffffu;   // sr_round(v, lo) rounds down, sr_round(v, hi) up
        while (hi - lo > 1u) {
            const uint32_t mid = lo + (hi - lo) / 2u;
            if (b_of(fp8q::sr_round<FMT>(v, mid)) == down) lo = mid; else hi = mid;
        }
        bad += same(lo) + same(hi);
    }
    return bad;
}

int main(int argc, char** argv) {
    const uint32_t stride = argc > 1 ? (uint32_t)std::atoi(argv[1]) : 31u;
    long bad[2] = {0, 0};
    // every bf16 pattern
    for (uint32_t b = 0; b < 65536u; ++b) {
        bad[0] += check<FP8Q_E4M3>(f_of(b << 16));
        bad[1] += check<FP8Q_E5M2>(f_of(b << 16));
    }
    std::printf("bf16 patterns: E4M3 %ld, E5M2 %ld mismatches\n", bad[0], bad[1]);
    // every stride-th fp32 pattern
    long bad4 = 0, bad5 = 0;
    const long long count = (1LL << 32) / stride;
#pragma omp parallel for reduction(+ : bad4, bad5) schedule(static)
    for (long long k = 0; k < count; ++k) {
        const float v = f_of((uint32_t)(k * stride));
        bad4 += check<FP8Q_E4M3>(v);
        bad5 += check<FP8Q_E5M2>(v);
    }
    std::printf("fp32 patterns (every %u-th): E4M3 %ld, E5M2 %ld mismatches\n", stride, bad4, bad5);
    return (bad[0] || bad[1] || bad4 || bad5) ? 1 : 0;
}
