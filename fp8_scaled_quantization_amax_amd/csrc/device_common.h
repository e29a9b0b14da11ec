// Device-side helpers shared by the fp8q HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q.h"
#include "launch.h"

namespace fp8q {

constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;
constexpr float kScaleFloor = 1e-12f;  // lower bound on a scale (lab page, scaled_roundtrip)

template <int FMT>
__host__ __device__ __forceinline__ constexpr float fmt_max() { return FMT == FP8Q_E4M3 ? kE4M3Max : kE5M2Max; }

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// s = max(RN32(amax / fmax), RN32(1e-12)), NaN-propagating.  The quotient uses
// the compiler's IEEE (correctly rounded) fp32 division.
template <int FMT>
__device__ __forceinline__ float scale_from_amax(float amax) {
    const float s = amax / fmt_max<FMT>();
    if (s != s) return s;
    return s < kScaleFloor ? kScaleFloor : s;
}

// Correctly rounded fp32 quotient x / s for a positive scale s, given
// r = RN32(1 / s).  q0 = x*r is within about 2 ulp; one FMA residual step
// makes it faithful; a second gives the correctly rounded quotient
// (Markstein's theorem: a faithful quotient corrected by the exact FMA
// residual times a correctly rounded reciprocal rounds correctly; see Muller
// et al., Handbook of Floating-Point Arithmetic, chapter on division with an
// FMA).  Non-finite q0 (x non-finite, or |x/s| beyond fp32) is returned as is:
// every such quotient encodes to the overflow / NaN code either way.  The
// sign is restored at the end because the residual steps turn -0 into +0.
// An infinite scale (an infinite amax) takes x * 0 = x / Inf instead: +-0 for
// finite x, NaN for infinite x, where the residual steps would form 0 * Inf.
__host__ __device__ __forceinline__ float div_by_scale(float x, float s, float r) {
    if (__builtin_isinf(s)) return x * r;
    const float q0 = x * r;
    if (!(__builtin_fabsf(q0) <= 3.402823466e38f)) return q0;
    float e = __builtin_fmaf(-q0, s, x);
    const float q1 = __builtin_fmaf(e, r, q0);
    e = __builtin_fmaf(-q1, s, x);
    const float q2 = __builtin_fmaf(e, r, q1);
    return __builtin_copysignf(q2, x);
}

// Stochastic rounding of a finite v to the format's grid with the word r (the
// result is exactly a grid value, or the step past the largest one, which the
// converter then overflows like any other value); NaN and Inf pass unchanged.
// With D the grid spacing at |v| (2^(max(e, emin) - mantissa bits) for
// |v| in [2^e, 2^(e + 1))), |v| = (n + f) D and the magnitude becomes
// (n + 1) D when r + floor(f 2^32) >= 2^32, else n D.  Two ways, by range:
//  * |v| >= 2^emin: D is the fp32 ulp of |v| times 2^(23 - mantissa bits), so
//    f 2^32 is the fraction field's low 23 - mb bits shifted up by 9 + mb,
//    whose low bits are zero; r then carries into bit 23 - mb of the
//    magnitude's bits exactly when its own top 23 - mb bits do, so adding
//    those to the bits and clearing the low ones rounds (a carry out of the
//    fraction field moves to the next binade, which is the next grid value).
//  * |v| < 2^emin: D = 2^(emin - mb) is fixed; y = |v| / D is exact (a power
//    of two), n = floor(y), and (y - n) 2^32 is an exact float below 2^32
//    whose conversion truncates to floor(f 2^32).  (A branch: a wave runs it
//    only when one of its lanes needs it.)
// Where the round-to-nearest cast of v is finite (|v| <= 464 for E4M3, the
// tie above 448 rounding down to it; |v| < 61440 for E5M2) the result is
// capped at fmax: current scaling leaves the amax element an ulp or two above
// fmax, and rounding it up to the next step would overflow.
template <int FMT>
__host__ __device__ __forceinline__ float sr_round(float v, uint32_t r) {
    constexpr int MB = FMT == FP8Q_E4M3 ? 3 : 2;
    constexpr int EMIN = FMT == FP8Q_E4M3 ? -6 : -14;
    constexpr uint32_t kLow = (1u << (23 - MB)) - 1u;
    constexpr uint32_t kMinNormal = (uint32_t)(EMIN + 127) << 23;                  // 2^emin
    constexpr float kToGrid = (float)(1u << (MB - EMIN));                           // 1 / D below 2^emin
    constexpr float kFromGrid = 1.0f / kToGrid;
    constexpr uint32_t kRneFiniteBits = FMT == FP8Q_E4M3 ? 0x43e80000u : 0x476fffffu;  // 464, below 61440
    const uint32_t ab = __builtin_bit_cast(uint32_t, v) & 0x7fffffffu;
    uint32_t mag = (ab + (r >> (9 + MB))) & ~kLow;
    if (ab < kMinNormal) {
        const float y = __builtin_bit_cast(float, ab) * kToGrid;
        const float n = __builtin_floorf(y);
        const uint32_t frac32 = (uint32_t)((y - n) * 4294967296.0f);
        mag = __builtin_bit_cast(uint32_t, (r > ~frac32 ? n + 1.0f : n) * kFromGrid);
    }
    // the cap compares bit patterns: for non-negative floats their order as
    // unsigned integers is the order of the values
    const uint32_t cap = ab <= kRneFiniteBits ? __builtin_bit_cast(uint32_t, fmt_max<FMT>()) : 0xffffffffu;
    const uint32_t capped = mag < cap ? mag : cap;
    return ab >= 0x7f800000u ? v : __builtin_bit_cast(float, capped | (__builtin_bit_cast(uint32_t, v) & 0x80000000u));
}

// div_by_scale for a finite scale s = max(amax / fmax, 1e-12) formed from
// the amax of the very tensor x belongs to: then |x| <= amax, so |x / s| stays
// within an ulp of fmax, the quotient estimate x r is finite and the check for
// a non-finite one is dead; the two residual steps are the same.  (A
// non-finite s comes from an infinite or NaN amax; div_by_scale returns x r
// for it, which callers take on a separate, uniform path.)
__host__ __device__ __forceinline__ float div_by_own_scale(float x, float s, float r) {
    const float q0 = x * r;
    float e = __builtin_fmaf(-q0, s, x);
    const float q1 = __builtin_fmaf(e, r, q0);
    e = __builtin_fmaf(-q1, s, x);
    return __builtin_copysignf(__builtin_fmaf(e, r, q1), x);
}

// Optional saturation: |v| > fmax -> +-fmax (NaN unchanged).
template <int FMT, bool SAT>
__device__ __forceinline__ float saturate(float v) {
    if constexpr (SAT) {
        return __builtin_fabsf(v) > fmt_max<FMT>() ? __builtin_copysignf(fmt_max<FMT>(), v) : v;
    } else {
        return v;
    }
}

// Four fp32 values -> four 8-bit codes packed little-endian in a dword.  The
// gfx950 conversions round to nearest even and, without clamping, overflow
// E4M3 to NaN and E5M2 to Inf (checked exhaustively against the definition
// on every fp32 input).
template <int FMT>
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
    int w = 0;
    if constexpr (FMT == FP8Q_E4M3) {
        w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    } else {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, w, false);
        w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    }
    return (uint32_t)w;
}

// Two fp32 values -> two 8-bit codes in the low half of a dword (pack2_lo),
// or into the high half of w (pack2_hi); the same conversions as pack4.
template <int FMT>
__device__ __forceinline__ uint32_t pack2_lo(float a, float b) {
    if constexpr (FMT == FP8Q_E4M3) return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    else return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
}
template <int FMT>
__device__ __forceinline__ uint32_t pack2_hi(float a, float b, uint32_t w) {
    if constexpr (FMT == FP8Q_E4M3) return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)w, true);
    else return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)w, true);
}

// |x| as an ordered integer key: NaN patterns sort above +Inf, so an integer
// max over keys is a NaN-propagating amax.
__device__ __forceinline__ uint32_t abs_key(float v) { return __float_as_uint(v) & 0x7fffffffu; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

// Max over lanes whose index differs only in the bits of `mask` (a power-of-two run).
template <int LO, int HI>
__device__ __forceinline__ uint32_t lanes_max_u32(uint32_t v) {
#pragma unroll
    for (int off = LO; off <= HI; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

// Max over each aligned group of 4 lanes, delivered to all 4 (DPP quad
// permutations: lane ^ 1, then lane ^ 2).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v = v > o ? v : o;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);            // quad_perm [2,3,0,1]
    return v > o ? v : o;
}

// Max over each aligned group of 16 lanes (a DPP row), delivered to all 16:
// quad maxima, then lane i <-> 7 - i within each half row, then i <-> 15 - i.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = quad_max_u32(v);
    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    v = v > o ? v : o;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);           // row_mirror
    return v > o ? v : o;
}

// Lane n (a compile-time constant after unrolling, 0..15) of each 16-lane
// DPP row broadcast to the whole row (row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast_n(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + N, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_lane_bcast(float v, int n) {
    switch (n) {
        case 0: return row_bcast_n<0>(v);
        case 1: return row_bcast_n<1>(v);
        case 2: return row_bcast_n<2>(v);
        case 3: return row_bcast_n<3>(v);
        case 4: return row_bcast_n<4>(v);
        case 5: return row_bcast_n<5>(v);
        case 6: return row_bcast_n<6>(v);
        default: return row_bcast_n<7>(v);
    }
}

// Block-wide max of a per-thread key (blockDim.x == 256).  Uses 4 words of LDS.
__device__ __forceinline__ uint32_t block_max_u32_256(uint32_t v, uint32_t* lds4) {
    v = wave_max_u32(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) lds4[wave] = v;
    __syncthreads();
    uint32_t r = lds4[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) r = r > lds4[i] ? r : lds4[i];
    __syncthreads();
    return r;
}

// Reduce the partial maxima written by the amax grid (one float per block).
// nparts <= 256 * 8; the eight loads of a thread are issued together.
__device__ __forceinline__ float reduce_partials_256(const float* partials, int nparts, uint32_t* lds4) {
    float p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = threadIdx.x + 256 * u;
        p[u] = i < nparts ? partials[i] : 0.0f;
    }
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const uint32_t k = abs_key(p[u]);
        m = m > k ? m : k;
    }
    return __uint_as_float(block_max_u32_256(m, lds4));
}

// E8M0 exponent for an MX block: e = ceil(log2 s) read from the bits of the
// (positive, normal) scale s; returns 255 for a non-finite s.
__device__ __forceinline__ int e8m0_from_scale(float s) {
    if (!(s <= 3.402823466e38f)) return 255;
    const uint32_t b = __float_as_uint(s);
    const int be = (int)(b >> 23);
    return ((b & 0x7fffffu) == 0 ? be - 127 : be - 126) + 127;
}

// 2^(127 - code) as fp32 (the exact reciprocal of an E8M0 scale), NaN for 255.
__device__ __forceinline__ float e8m0_recip(int code) {
    if (code == 255) return __uint_as_float(0x7fc00000u);
    return __uint_as_float((uint32_t)(254 - code) << 23);
}

// 16-byte load with the non-temporal hint, for inputs a pass reads once:
// keeping them in the caches would only evict other data (measured: the amax
// pass over 130 MB of bf16 went from 26.7 to 22.9 us with it).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    const u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC 2011): ten rounds of (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
// with (hi0, lo0) = 0xD2511F53 * c0 and (hi1, lo1) = 0xCD9E8D57 * c2 as full
// 64-bit products (one multiply-add instruction each); the key gains
// 0x9E3779B9 and 0xBB67AE85 before each round after the first.  Each
// three-way XOR is one gfx950 three-input bitwise instruction (truth table
// 0x96).
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96),
                       n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
    }
    return make_uint4(c0, c1, c2, c3);
}

// bf16 round to nearest even of an fp32 value (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    const uint32_t b = __float_as_uint(f);
    if ((b & 0x7fffffffu) > 0x7f800000u) return (b >> 16) | 0x40u;
    return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

}  // namespace fp8q
