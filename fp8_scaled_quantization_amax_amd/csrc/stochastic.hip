// Stochastically rounded FP8 cast with per-tensor current scaling, for gfx950.
//
// The low-precision training recipe of "How to Optimize Transformer-Based
// Models for Low-Precision Training" rounds its gradients stochastically;
// this applies that to the 8-bit formats.  The scale is the one of the
// "fp8_parity.py" lab page's scaled_roundtrip (amax / fmax, floored at 1e-12),
// and the quotient v = RN32(x / s) is then rounded to one of its two
// neighbouring grid values: with D the grid spacing at |v| and f the position
// of |v| between n D and (n + 1) D, it goes up when r + floor(f 2^32) >= 2^32
// for the element's random word r.  The words come from the counter-based
// generator Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC 2011), so a (seed, offset) pair fixes
// every decision: element i takes word i mod 4 of the block for counter
// (i / 4, offset) and key seed.
//
// Design: the amax pass is the shared partial-maximum grid; this kernel
// folds the partials into the scale (every block), then each thread takes
// groups of 4 elements, one generator call per group.  The generator's ten
// rounds of 32 x 32 -> 64-bit multiplies cost more VALU time than the HBM
// traffic of the group, so the kernel is ALU-bound.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace fp8q {

template <int HP>
__device__ __forceinline__ float load_one_sr(const void* __restrict__ x, int64_t i) {
    if constexpr (HP == FP8Q_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[i]);
    else return reinterpret_cast<const float*>(x)[i];
}

// VEC: x aligned to 4 elements and q to 4 bytes.  The grid strides over the
// n / 4 whole groups without per-element checks; the last thread of block 0
// casts the partial group at the end, if any.
template <int HP, int FMT, bool SAT, bool VEC>
__global__ __launch_bounds__(256) void quantize_sr_kernel(const void* __restrict__ x, int64_t n,
                                                          const float* __restrict__ partials, int nparts,
                                                          uint32_t k0, uint32_t k1, uint32_t o0, uint32_t o1,
                                                          uint8_t* __restrict__ q, float* scale_out,
                                                          float* amax_out) {
    __shared__ uint32_t red[4];
    const float amax = reduce_partials_256(partials, nparts, red);
    const float s = scale_from_amax<FMT>(amax);
    const float rc = 1.0f / s;
    // A finite s comes from this tensor's own amax, so the division needs no
    // check for a non-finite quotient; an infinite or NaN s (an infinite or
    // NaN amax) gives x / s = x * (1 / s) for every element.  The two cases
    // run as separate copies of the loop.
    auto run = [&](auto finite_c) {
    constexpr bool FIN = decltype(finite_c)::value;
    auto cast4 = [&](int64_t g, const float (&v)[4]) {
        const uint4 rw = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), o0, o1, k0, k1);
        auto div = [&](float xv) { return FIN ? div_by_own_scale(xv, s, rc) : xv * rc; };
        return pack4<FMT>(saturate<FMT, SAT>(sr_round<FMT>(div(v[0]), rw.x)),
                          saturate<FMT, SAT>(sr_round<FMT>(div(v[1]), rw.y)),
                          saturate<FMT, SAT>(sr_round<FMT>(div(v[2]), rw.z)),
                          saturate<FMT, SAT>(sr_round<FMT>(div(v[3]), rw.w)));
    };
    const int64_t nfull = n / 4;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < nfull; g += (int64_t)gridDim.x * 256) {
        const int64_t i0 = 4 * g;
        float v[4];
        if constexpr (VEC && HP == FP8Q_BF16) {
            const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + i0);
            v[0] = __uint_as_float(w.x << 16);
            v[1] = __uint_as_float(w.x & 0xffff0000u);
            v[2] = __uint_as_float(w.y << 16);
            v[3] = __uint_as_float(w.y & 0xffff0000u);
        } else if constexpr (VEC) {
            const uint4 w = load_stream16(reinterpret_cast<const float*>(x) + i0);
            v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
            v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = load_one_sr<HP>(x, i0 + e);
        }
        const uint32_t w = cast4(g, v);
        if constexpr (VEC) {
            *reinterpret_cast<uint32_t*>(q + i0) = w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) q[i0 + e] = (uint8_t)((w >> (8 * e)) & 0xffu);
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 255 && (n & 3)) {
        const int64_t i0 = 4 * nfull;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = i0 + e < n ? load_one_sr<HP>(x, i0 + e) : 0.0f;
        const uint32_t w = cast4(nfull, v);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (i0 + e < n) q[i0 + e] = (uint8_t)((w >> (8 * e)) & 0xffu);
    }
    };
    if (__builtin_isfinite(s)) run(std::true_type{});
    else run(std::false_type{});
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *scale_out = s;
        if (amax_out) *amax_out = amax;
    }
}

template <int HP, int FMT, bool SAT>
static void launch_sr_t(const void* x, int64_t n, const float* partials, int nparts, uint64_t seed, uint64_t offset,
                        uint8_t* q, float* scale_out, float* amax_out, bool vec, hipStream_t s) {
    const int64_t ngroups = (n + 3) / 4;
    const int64_t want = (ngroups + 255) / 256;
    const int grid = (int)(want < 4096 ? (want < 1 ? 1 : want) : 4096);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32), o0 = (uint32_t)offset,
                   o1 = (uint32_t)(offset >> 32);
    if (vec)
        hipLaunchKernelGGL((quantize_sr_kernel<HP, FMT, SAT, true>), dim3(grid), dim3(256), 0, s, x, n, partials,
                           nparts, k0, k1, o0, o1, q, scale_out, amax_out);
    else
        hipLaunchKernelGGL((quantize_sr_kernel<HP, FMT, SAT, false>), dim3(grid), dim3(256), 0, s, x, n, partials,
                           nparts, k0, k1, o0, o1, q, scale_out, amax_out);
}

hipError_t launch_quantize_sr(const void* x, int hp, int64_t n, int fmt, bool sat, uint64_t seed, uint64_t offset,
                              const float* partials, int nparts, uint8_t* q, float* scale_out, float* amax_out,
                              hipStream_t s) {
    const bool vec = (uintptr_t)x % (hp == FP8Q_BF16 ? 8 : 16) == 0 && (uintptr_t)q % 4 == 0;
    if (hp == FP8Q_BF16) {
        if (fmt == FP8Q_E4M3) {
            if (sat) launch_sr_t<FP8Q_BF16, FP8Q_E4M3, true>(x, n, partials, nparts, seed, offset, q, scale_out, amax_out, vec, s);
            else launch_sr_t<FP8Q_BF16, FP8Q_E4M3, false>(x, n, partials, nparts, seed, offset, q, scale_out, amax_out, vec, s);
        } else {
            if (sat) launch_sr_t<FP8Q_BF16, FP8Q_E5M2, true>(x, n, partials, nparts, seed, offset, q, scale_out, amax_out, vec, s);
            else launch_sr_t<FP8Q_BF16, FP8Q_E5M2, false>(x, n, partials, nparts, seed, offset, q, scale_out, amax_out, vec, s);
        }
    } else {
        if (fmt == FP8Q_E4M3) {
            if (sat) launch_sr_t<FP8Q_F32, FP8Q_E4M3, true>(x, n, partials, nparts, seed, offset, q, scale_out, amax_out, vec, s);
            else launch_sr_t<FP8Q_F32, FP8Q_E4M3, false>(x, n, partials, nparts, seed, offset, q, scale_out, amax_out, vec, s);
        } else {
            if (sat) launch_sr_t<FP8Q_F32, FP8Q_E5M2, true>(x, n, partials, nparts, seed, offset, q, scale_out, amax_out, vec, s);
            else launch_sr_t<FP8Q_F32, FP8Q_E5M2, false>(x, n, partials, nparts, seed, offset, q, scale_out, amax_out, vec, s);
        }
    }
    return hipGetLastError();
}

}  // namespace fp8q
