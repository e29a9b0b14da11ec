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

hipError_t launch_mfma_loop(int blocks, int iters, float* out, hipStream_t s) {
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, s, out, iters, 0x38383838);
    return hipGetLastError();
}

}  // namespace fp8q
