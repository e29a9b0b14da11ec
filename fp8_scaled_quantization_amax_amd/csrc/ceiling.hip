// Measurement aid, outside the FP8 path: the rate of the FP8 matrix cores when
// nothing else limits them.  Every wave runs `iters` rounds of 8 independent
// 16x16x128 E4M3 MFMAs on operands held in registers (no memory traffic, no
// LDS), so the result is the chip's sustained FP8 MFMA rate at the clock it
// holds under that load: the measured ceiling beside the nominal 5.0 PFLOP/s.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace fp8q {

typedef int v8i_c __attribute__((ext_vector_type(8)));
typedef float v4f_c __attribute__((ext_vector_type(4)));

// The operands are E4M3 ones (byte 0x38, passed in so that nothing folds):
// every MFMA adds 128 to each of its 4 values per lane, so each thread's
// output is exactly 8 * 4 * 128 * iters (exact in fp32 up to iters = 2^12),
// which also shows that every MFMA ran.
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* __restrict__ out, int iters, int ones) {
    v8i_c a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = b[i] = ones;
    v4f_c acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = v4f_c{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], 0, 0, 0, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;   // keeps the loop live
}

// Four E4M3 codes from a counter: random sign, exponent field 1..14 (normal
// values, never NaN) and mantissa, from a 32-bit integer hash of the counter
// (xor-shift-multiply finalizer).
__device__ __forceinline__ int random_codes4(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t c = (x >> (8 * b)) & 0xffu;
        const uint32_t e = 1u + ((c >> 3) & 0xfu) % 14u;
        w |= ((c & 0x80u) | (e << 3) | (c & 7u)) << (8 * b);
    }
    return (int)w;
}

// The same loop on operands that look like real data to the matrix cores:
// every lane holds 8 A and 8 B operand sets of pseudo-random E4M3 codes, and
// each MFMA takes a different (A, B) pair, so the multiplier inputs change
// every instruction as they do in a GEMM.  The MFMA energy depends on the
// data (all-ones operands barely toggle), so this is the ceiling the chip
// holds for such data under its power limit.  iters % 8 == 0.
__global__ __launch_bounds__(256) void mfma_loop_random_kernel(float* __restrict__ out, int iters) {
    const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
    v8i_c a[8], b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[s][i] = random_codes4(tid * 1024u + s * 64u + i);
            b[s][i] = random_codes4(tid * 1024u + s * 64u + 32u + i);
        }
    v4f_c acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = v4f_c{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; it += 8) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[j], b[(j + r) & 7], acc[j], 0, 0, 0, 0, 0,
                                                                         0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_mfma_loop(int blocks, int iters, int data, float* out, hipStream_t s) {
    if (data == 0)
        hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, s, out, iters, 0x38383838);
    else
        hipLaunchKernelGGL(mfma_loop_random_kernel, dim3(blocks), dim3(256), 0, s, out, iters);
    return hipGetLastError();
}

}  // namespace fp8q
