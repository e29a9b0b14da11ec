// Random Hadamard transform of a wgrad operand along its token axis, fused
// with per-tensor current FP8 quantization, for gfx950.
//
// "How to Optimize Transformer-Based Models for Low-Precision Training" lists
// random Hadamard transforms on the wgrad inputs among its recipe's extra
// operations.  wgrad contracts over tokens, dW = G^T X, so both operands may be
// multiplied along the tokens by the same orthogonal R, since
// (R G)^T (R X) = G^T R^T R X = G^T X; a block-diagonal R spreads an outlier
// token over its block before quantization.  Here R has 16 x 16 blocks
// (1/4) H16 diag(d): H16 the Sylvester Hadamard matrix, d a random sign per
// token, the top bit of the token's Philox4x32-10 word (counter (t / 4, 0),
// key seed; word t mod 4), so two operands with the same seed share R.
//
// Arithmetic: y = (1/4) H16 (d x) by the fast Walsh-Hadamard transform in
// fp32 -- signs applied (exact), four butterfly stages (a + b, a - b) with
// partners 1, 2, 4, 8 apart, then the exact factor 1/4 -- in this fixed order,
// which the codes depend on.  Then y is quantized as the per-tensor current
// cast quantizes x: amax over y, s = max(amax / fmax, 1e-12), q = fp8(RN32(y / s)).
//
// Design: the amax of y needs all of y first, so the transform runs twice
// from x instead of writing y out and reading it back (2 x 4 bytes per element
// more HBM traffic): pass 1 takes each block's max |y| as a partial maximum,
// pass 2 folds the partials into the scale and casts.  With the butterflies,
// the divisions and the sign draws done twice, the pair is ALU-heavy, and
// since a thread takes its unit from load to store with nothing else in
// flight, load latency shows as well.  A thread owns one 16-row block of 8
// columns: 16 loads of 16 bytes (bf16) from consecutive rows, 8 transforms of
// 16 values in registers, 16 stores of 8 codes; neighbouring threads take
// neighbouring column groups, so every load and store is coalesced.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace fp8q {

// Sign bits of the 16 tokens of block b (bit i set: token 16 b + i negated).
__device__ __forceinline__ uint32_t rht_signs(int64_t b, uint32_t k0, uint32_t k1) {
    uint32_t bits = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint64_t g = (uint64_t)b * 4 + q;   // tokens 16 b + 4 q .. + 3
        const uint4 w = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), 0u, 0u, k0, k1);
        bits |= ((w.x >> 31) << (4 * q)) | ((w.y >> 31) << (4 * q + 1)) | ((w.z >> 31) << (4 * q + 2)) |
                ((w.w >> 31) << (4 * q + 3));
    }
    return bits;
}

// y[0..16) for each of the thread's 8 columns: load, signs, butterflies, 1/4.
template <int HP>
__device__ __forceinline__ void rht_block(const void* __restrict__ x, int64_t cols, int64_t b, int64_t c0,
                                          uint32_t signs, float y[16][8]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t off = (b * 16 + i) * cols + c0;
        if constexpr (HP == FP8Q_BF16) {
            const uint4 w = load_stream16(reinterpret_cast<const uint16_t*>(x) + off);
            const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                y[i][2 * j] = __uint_as_float(d[j] << 16);
                y[i][2 * j + 1] = __uint_as_float(d[j] & 0xffff0000u);
            }
        } else {
            const float* p = reinterpret_cast<const float*>(x) + off;
            const uint4 a = load_stream16(p), c = load_stream16(p + 4);
            y[i][0] = __uint_as_float(a.x); y[i][1] = __uint_as_float(a.y);
            y[i][2] = __uint_as_float(a.z); y[i][3] = __uint_as_float(a.w);
            y[i][4] = __uint_as_float(c.x); y[i][5] = __uint_as_float(c.y);
            y[i][6] = __uint_as_float(c.z); y[i][7] = __uint_as_float(c.w);
        }
        if ((signs >> i) & 1u) {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[i][e] = -y[i][e];
        }
    }
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if ((i & h) == 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float a = y[i][e], c = y[i + h][e];
                    y[i][e] = a + c;
                    y[i + h][e] = a - c;
                }
            }
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) y[i][e] *= 0.25f;
}

// Pass 1: one partial max |y| per block (grid-stride over 16 x 8 units).
template <int HP>
__global__ __launch_bounds__(256) void rht_amax_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                       uint32_t k0, uint32_t k1, float* __restrict__ partials) {
    __shared__ uint32_t red[4];
    const int64_t ncg = cols / 8, nunits = rows / 16 * ncg;
    uint32_t key = 0;
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < nunits; u += (int64_t)gridDim.x * 256) {
        const int64_t b = u / ncg, c0 = (u % ncg) * 8;
        float y[16][8];
        rht_block<HP>(x, cols, b, c0, rht_signs(b, k0, k1), y);
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t k = abs_key(y[i][e]);
                key = key > k ? key : k;
            }
    }
    key = block_max_u32_256(key, red);
    if (threadIdx.x == 0) partials[blockIdx.x] = __uint_as_float(key);
}

// Pass 2: scale from the partials, then cast y.
template <int HP, int FMT, bool SAT>
__global__ __launch_bounds__(256) void rht_cast_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                       uint32_t k0, uint32_t k1, const float* __restrict__ partials,
                                                       int nparts, uint8_t* __restrict__ q, float* scale_out,
                                                       float* amax_out) {
    __shared__ uint32_t red[4];
    const float amax = reduce_partials_256(partials, nparts, red);
    const float s = scale_from_amax<FMT>(amax);
    const float rc = 1.0f / s;
    const int64_t ncg = cols / 8, nunits = rows / 16 * ncg;
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < nunits; u += (int64_t)gridDim.x * 256) {
        const int64_t b = u / ncg, c0 = (u % ncg) * 8;
        float y[16][8];
        rht_block<HP>(x, cols, b, c0, rht_signs(b, k0, k1), y);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float c[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) c[e] = saturate<FMT, SAT>(div_by_scale(y[i][e], s, rc));
            *reinterpret_cast<uint2*>(q + (b * 16 + i) * cols + c0) =
                make_uint2(pack4<FMT>(c[0], c[1], c[2], c[3]), pack4<FMT>(c[4], c[5], c[6], c[7]));
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *scale_out = s;
        if (amax_out) *amax_out = amax;
    }
}

template <int HP, int FMT, bool SAT>
static void launch_rht_t(const void* x, int64_t rows, int64_t cols, uint32_t k0, uint32_t k1, float* partials,
                         int nparts, uint8_t* q, float* scale_out, float* amax_out, hipStream_t s) {
    hipLaunchKernelGGL((rht_amax_kernel<HP>), dim3(nparts), dim3(256), 0, s, x, rows, cols, k0, k1, partials);
    const int64_t nunits = rows / 16 * (cols / 8);
    const int64_t want = (nunits + 255) / 256;
    const int grid = (int)(want < 2048 ? (want < 1 ? 1 : want) : 2048);
    hipLaunchKernelGGL((rht_cast_kernel<HP, FMT, SAT>), dim3(grid), dim3(256), 0, s, x, rows, cols, k0, k1, partials,
                       nparts, q, scale_out, amax_out);
}

int rht_partials_grid(int64_t rows, int64_t cols) {
    const int64_t want = (rows / 16 * (cols / 8) + 255) / 256;
    return (int)(want < kReduceParts ? (want < 1 ? 1 : want) : kReduceParts);
}

hipError_t launch_quantize_rht(const void* x, int hp, int64_t rows, int64_t cols, int fmt, bool sat, uint64_t seed,
                               float* partials, uint8_t* q, uint8_t* qT, float* scale_out, float* amax_out,
                               hipStream_t s) {
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const int nparts = rht_partials_grid(rows, cols);
    if (hp == FP8Q_BF16) {
        if (fmt == FP8Q_E4M3) {
            if (sat) launch_rht_t<FP8Q_BF16, FP8Q_E4M3, true>(x, rows, cols, k0, k1, partials, nparts, q, scale_out, amax_out, s);
            else launch_rht_t<FP8Q_BF16, FP8Q_E4M3, false>(x, rows, cols, k0, k1, partials, nparts, q, scale_out, amax_out, s);
        } else {
            if (sat) launch_rht_t<FP8Q_BF16, FP8Q_E5M2, true>(x, rows, cols, k0, k1, partials, nparts, q, scale_out, amax_out, s);
            else launch_rht_t<FP8Q_BF16, FP8Q_E5M2, false>(x, rows, cols, k0, k1, partials, nparts, q, scale_out, amax_out, s);
        }
    } else {
        if (fmt == FP8Q_E4M3) {
            if (sat) launch_rht_t<FP8Q_F32, FP8Q_E4M3, true>(x, rows, cols, k0, k1, partials, nparts, q, scale_out, amax_out, s);
            else launch_rht_t<FP8Q_F32, FP8Q_E4M3, false>(x, rows, cols, k0, k1, partials, nparts, q, scale_out, amax_out, s);
        } else {
            if (sat) launch_rht_t<FP8Q_F32, FP8Q_E5M2, true>(x, rows, cols, k0, k1, partials, nparts, q, scale_out, amax_out, s);
            else launch_rht_t<FP8Q_F32, FP8Q_E5M2, false>(x, rows, cols, k0, k1, partials, nparts, q, scale_out, amax_out, s);
        }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || qT == nullptr) return e;
    return launch_transpose_u8(q, rows, cols, qT, s);
}

}  // namespace fp8q
