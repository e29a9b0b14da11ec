// Host-side check of the quantizers' division: fp8q::div_by_scale(x, s, 1/s)
// must equal the correctly rounded fp32 quotient RN32(x / s) wherever the
// quotient can influence an 8-bit code (2^-18 <= |x/s| < 2^17); outside that
// range every candidate encodes to the same code (zero, or overflow).  And
// fp8q::div_by_own_scale must give div_by_scale's bits wherever x / s's
// estimate x (1/s) is finite.
// Compiled as host code from the kernels' own header.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "device_common.h"

static inline float f_of(uint32_t b) { float f; std::memcpy(&f, &b, 4); return f; }
static inline uint32_t bits_of(float f) { uint32_t b; std::memcpy(&b, &f, 4); return b; }
static inline uint32_t b_of(float f) { uint32_t b; std::memcpy(&b, &f, 4); return b; }

// 1 if the pair differs in a way that could change a code
static inline int relevant_mismatch(float x, float s, float r) {
    const float e = (float)((double)x / (double)s);
    const float g = fp8q::div_by_scale(x, s, r);
    if (b_of(e) == b_of(g)) return 0;
    if (std::isnan(e) && std::isnan(g)) return 0;
    const float ae = std::fabs(e);
    if (ae >= 131072.0f && std::fabs(g) >= 131072.0f) return 0;                 // both overflow every format
    if (ae < 0x1p-18f && std::fabs(g) < 0x1p-18f && std::signbit(e) == std::signbit(g)) return 0;  // both zero codes
    return 1;
}

// div_by_own_scale drops div_by_scale's check for a non-finite estimate x r,
// which its callers rule out: the same bits wherever x r is finite
static inline int own_mismatch(float x, float s, float r) {
    if (!(std::fabs(x * r) <= 3.402823466e38f)) return 0;
    return b_of(fp8q::div_by_own_scale(x, s, r)) == b_of(fp8q::div_by_scale(x, s, r)) ? 0 : 1;
}

int main(int argc, char** argv) {
    const int nscales = argc > 1 ? std::atoi(argv[1]) : 20000;
    std::vector<float> scales = {1e-12f, 1.0f, 448.0f / 448.0f, 1.0f / 448.0f, 1.0f / 57344.0f, 1.0f / 3.0f,
                                 f_of(0x3f7fffffu), f_of(0x3fffffffu), f_of(0x00800000u) * 1e30f, 0.0137f, 2.5e-3f};
    std::mt19937 rng(12345);
    while ((int)scales.size() < nscales) {
        // normal scales in [1e-12, ~1e30]: biased exponents 87..226, random mantissa
        const uint32_t e = 87 + rng() % 140, m = rng() & 0x7fffffu;
        scales.push_back(f_of((e << 23) | m));
    }
    long bad = 0;
    // every bf16 input against every scale
#pragma omp parallel for reduction(+ : bad) schedule(dynamic, 64)
    for (int si = 0; si < (int)scales.size(); ++si) {
        const float s = scales[si], r = 1.0f / s;
        for (uint32_t b = 0; b < 65536; ++b) bad += relevant_mismatch(f_of(b << 16), s, r) + own_mismatch(f_of(b << 16), s, r);
    }
    std::printf("bf16 x %zu scales: %ld relevant mismatches\n", scales.size(), bad);
    // every fp32 input against a few scales
    const float full[] = {1.0f / 3.0f, 0.0137f, f_of(0x3f7fffffu) * 0.01f};
    const int nfull = argc > 2 ? std::atoi(argv[2]) : 3;
    long bad2 = 0;
    for (int fi = 0; fi < nfull && fi < 3; ++fi) {
        const float s = full[fi];
        const float r = 1.0f / s;
#pragma omp parallel for reduction(+ : bad2) schedule(static)
        for (long long i = 0; i < (1LL << 32); ++i)
            bad2 += relevant_mismatch(f_of((uint32_t)i), s, r) + own_mismatch(f_of((uint32_t)i), s, r);
    }
    std::printf("all fp32 x %d scales: %ld relevant mismatches\n", nfull, bad2);
    // an infinite scale (an infinite amax): x / Inf exactly, sign of zero included
    long bad3 = 0;
    const float inf = f_of(0x7f800000u);
    for (uint32_t b = 0; b < 65536; ++b) {
        const float x = f_of(b << 16), want = x / inf, got = fp8q::div_by_scale(x, inf, 1.0f / inf);
        const bool same = (want != want) ? (got != got) : (bits_of(got) == bits_of(want));
        bad3 += same ? 0 : 1;
    }
    std::printf("bf16 x infinite scale: %ld mismatches\n", bad3);
    return (bad == 0 && bad2 == 0 && bad3 == 0) ? 0 : 1;
}
