// Rowwise FP8 quantization for gfx950: one fp32 scale per row (axis 0) or per
// column (axis 1) of a row-major [rows, cols] matrix.  This is the "rowwise"
// recipe of the "fp8_parity.py" lab page (torchao's rowwise Float8 training),
// where each GEMM input is scaled per row along its contraction; the
// arithmetic per group is that page's scaled_roundtrip: amax over the row or
// column, s = max(amax / fmax, 1e-12) in fp32, q = fp8(RN32(x / s)).
//
// Design (all HBM-bound):
//  * axis 0: one 256-thread block per row.  A first pass over the row takes
//    the abs-max key (16-byte loads when the row allows), a block reduction
//    gives the scale, and a second pass over the same row, which is still in
//    L2, divides and converts.  HBM traffic: the row read once, codes written
//    once (3 B per bf16 element).
//  * axis 1: the column maxima need the whole column, so they come first:
//    keys zeroed, then blocks of a 256-column stripe x a chunk of rows take
//    per-column maxima (8 columns per thread, 8 row lanes folded through LDS)
//    and merge them with an integer atomic max, which is order-free and hence
//    deterministic.  The keys, kept in the caller's scale array, then become
//    scales in place, and a cast pass with the same stripe layout converts
//    (each thread's 8 columns fixed, so their reciprocals are computed once).
//    The K-major copy comes from the byte transpose of the codes.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace fp8q {

template <int HP>
__device__ __forceinline__ float load_one(const void* __restrict__ x, int64_t i) {
    if constexpr (HP == FP8Q_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[i]);
    else return reinterpret_cast<const float*>(x)[i];
}

// Elements [i, i + 8) with 16-byte loads (i a multiple of 8, x 16-byte aligned).
template <int HP>
__device__ __forceinline__ void load_eight(const void* __restrict__ x, int64_t i, float v[8]) {
    if constexpr (HP == FP8Q_BF16) {
        const uint4 w = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + i)[0];
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(d[j] << 16);
            v[2 * j + 1] = __uint_as_float(d[j] & 0xffff0000u);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + i);
        const float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

template <int FMT, bool SAT>
__device__ __forceinline__ uint8_t code_of(float x, float s, float r) {
    return (uint8_t)(pack4<FMT>(saturate<FMT, SAT>(div_by_scale(x, s, r)), 0.0f, 0.0f, 0.0f) & 0xffu);
}

template <int FMT, bool SAT>
__device__ __forceinline__ uint2 codes_of8(const float v[8], const float s[8], const float r[8]) {
    float c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = saturate<FMT, SAT>(div_by_scale(v[e], s[e], r[e]));
    return make_uint2(pack4<FMT>(c[0], c[1], c[2], c[3]), pack4<FMT>(c[4], c[5], c[6], c[7]));
}

// ------------------------------------------------------------------ axis 0: per row

// VEC: cols % 8 == 0, x 16-byte aligned, q 8-byte aligned.
template <int HP, int FMT, bool SAT, bool VEC>
__global__ __launch_bounds__(256) void rowwise_rows_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                           uint8_t* __restrict__ q, float* __restrict__ scales) {
    __shared__ uint32_t red[4];
    const int t = threadIdx.x;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const int64_t base = r * cols;
        uint32_t key = 0;
        if constexpr (VEC) {
            for (int64_t c = 8 * t; c < cols; c += 8 * 256) {
                float v[8];
                load_eight<HP>(x, base + c, v);
#pragma unroll
                for (int e = 0; e < 8; ++e) { const uint32_t k = abs_key(v[e]); key = key > k ? key : k; }
            }
        } else {
            for (int64_t c = t; c < cols; c += 256) {
                const uint32_t k = abs_key(load_one<HP>(x, base + c));
                key = key > k ? key : k;
            }
        }
        key = block_max_u32_256(key, red);
        const float s = scale_from_amax<FMT>(__uint_as_float(key));
        const float rc = 1.0f / s;
        if (t == 0) scales[r] = s;
        if constexpr (VEC) {
            float sv[8], rv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) { sv[e] = s; rv[e] = rc; }
            for (int64_t c = 8 * t; c < cols; c += 8 * 256) {
                float v[8];
                load_eight<HP>(x, base + c, v);
                *reinterpret_cast<uint2*>(q + base + c) = codes_of8<FMT, SAT>(v, sv, rv);
            }
        } else {
            for (int64_t c = t; c < cols; c += 256) q[base + c] = code_of<FMT, SAT>(load_one<HP>(x, base + c), s, rc);
        }
    }
}

// ------------------------------------------------------------------ axis 1: per column

constexpr int kStripe = 256;   // columns per block (32 groups of 8)

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

// Thread t of a block: column group t % 32 (8 columns from c0), row lane
// t / 32 (rows r0 + lane, r0 + lane + 8, ... below r1).
// VEC: cols % 8 == 0 and x 16-byte aligned.
template <int HP, bool VEC>
__global__ __launch_bounds__(256) void colmax_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                     int64_t rchunk, uint32_t* __restrict__ keys) {
    __shared__ uint32_t part[8][kStripe];
    const int t = threadIdx.x, cg = t & 31, rl = t >> 5;
    const int64_t c0 = (int64_t)blockIdx.x * kStripe + cg * 8;
    const int64_t r0 = (int64_t)blockIdx.y * rchunk;
    const int64_t r1 = r0 + rchunk < rows ? r0 + rchunk : rows;
    uint32_t k[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (c0 < cols) {
        for (int64_t r = r0 + rl; r < r1; r += 8) {
            float v[8];
            if constexpr (VEC) {
                load_eight<HP>(x, r * cols + c0, v);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = c0 + e < cols ? load_one<HP>(x, r * cols + c0 + e) : 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) { const uint32_t a = abs_key(v[e]); k[e] = k[e] > a ? k[e] : a; }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rl][cg * 8 + e] = k[e];
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = m > part[i][t] ? m : part[i][t];
    const int64_t c = (int64_t)blockIdx.x * kStripe + t;
    if (c < cols && m != 0u) atomicMax(&keys[c], m);
}

// keys (abs-max bit patterns) -> scales, in place.
template <int FMT>
__global__ __launch_bounds__(256) void keys_to_scales_kernel(float* __restrict__ scales, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const uint32_t k = reinterpret_cast<const uint32_t*>(scales)[i];
        scales[i] = scale_from_amax<FMT>(__uint_as_float(k));
    }
}

// Same thread layout as colmax_kernel.  VEC: cols % 8 == 0, x 16-byte and q
// 8-byte aligned.
template <int HP, int FMT, bool SAT, bool VEC>
__global__ __launch_bounds__(256) void cast_cols_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                        int64_t rchunk, const float* __restrict__ scales,
                                                        uint8_t* __restrict__ q) {
    const int t = threadIdx.x, cg = t & 31, rl = t >> 5;
    const int64_t c0 = (int64_t)blockIdx.x * kStripe + cg * 8;
    if (c0 >= cols) return;
    const int64_t r0 = (int64_t)blockIdx.y * rchunk;
    const int64_t r1 = r0 + rchunk < rows ? r0 + rchunk : rows;
    float s[8], rc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s[e] = c0 + e < cols ? scales[c0 + e] : 1.0f;
        rc[e] = 1.0f / s[e];
    }
    for (int64_t r = r0 + rl; r < r1; r += 8) {
        if constexpr (VEC) {
            float v[8];
            load_eight<HP>(x, r * cols + c0, v);
            *reinterpret_cast<uint2*>(q + r * cols + c0) = codes_of8<FMT, SAT>(v, s, rc);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (c0 + e < cols) q[r * cols + c0 + e] = code_of<FMT, SAT>(load_one<HP>(x, r * cols + c0 + e), s[e], rc[e]);
        }
    }
}

// ------------------------------------------------------------------ launcher

template <int HP, int FMT, bool SAT>
static void launch_rowwise_t(const void* x, int64_t rows, int64_t cols, int axis, uint8_t* q, float* scales,
                             bool vec, hipStream_t s) {
    if (axis == 0) {
        const int grid = (int)(rows < 65536 ? rows : 65536);
        if (vec)
            hipLaunchKernelGGL((rowwise_rows_kernel<HP, FMT, SAT, true>), dim3(grid), dim3(256), 0, s, x, rows, cols, q,
                               scales);
        else
            hipLaunchKernelGGL((rowwise_rows_kernel<HP, FMT, SAT, false>), dim3(grid), dim3(256), 0, s, x, rows, cols, q,
                               scales);
        return;
    }
    const int64_t stripes = (cols + kStripe - 1) / kStripe;
    int64_t chunks = 2048 / stripes;
    const int64_t max_chunks = (rows + 7) / 8;
    if (chunks > max_chunks) chunks = max_chunks;
    if (chunks < 1) chunks = 1;
    if (chunks > 65535) chunks = 65535;
    const int64_t rchunk = (rows + chunks - 1) / chunks;
    chunks = (rows + rchunk - 1) / rchunk;
    const dim3 grid((unsigned)stripes, (unsigned)chunks);
    uint32_t* keys = reinterpret_cast<uint32_t*>(scales);
    const int fill = (int)((cols + 255) / 256 < 1024 ? (cols + 255) / 256 : 1024);
    hipLaunchKernelGGL(zero_u32_kernel, dim3(fill), dim3(256), 0, s, keys, cols);
    if (vec) hipLaunchKernelGGL((colmax_kernel<HP, true>), grid, dim3(256), 0, s, x, rows, cols, rchunk, keys);
    else hipLaunchKernelGGL((colmax_kernel<HP, false>), grid, dim3(256), 0, s, x, rows, cols, rchunk, keys);
    hipLaunchKernelGGL((keys_to_scales_kernel<FMT>), dim3(fill), dim3(256), 0, s, scales, cols);
    if (vec)
        hipLaunchKernelGGL((cast_cols_kernel<HP, FMT, SAT, true>), grid, dim3(256), 0, s, x, rows, cols, rchunk, scales,
                           q);
    else
        hipLaunchKernelGGL((cast_cols_kernel<HP, FMT, SAT, false>), grid, dim3(256), 0, s, x, rows, cols, rchunk,
                           scales, q);
}

hipError_t launch_quantize_rowwise(const void* x, int hp, int64_t rows, int64_t cols, int axis, int fmt, bool sat,
                                   uint8_t* q, uint8_t* qT, float* scales, hipStream_t s) {
    const bool vec = cols % 8 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)q % 8 == 0;
    if (hp == FP8Q_BF16) {
        if (fmt == FP8Q_E4M3) {
            if (sat) launch_rowwise_t<FP8Q_BF16, FP8Q_E4M3, true>(x, rows, cols, axis, q, scales, vec, s);
            else launch_rowwise_t<FP8Q_BF16, FP8Q_E4M3, false>(x, rows, cols, axis, q, scales, vec, s);
        } else {
            if (sat) launch_rowwise_t<FP8Q_BF16, FP8Q_E5M2, true>(x, rows, cols, axis, q, scales, vec, s);
            else launch_rowwise_t<FP8Q_BF16, FP8Q_E5M2, false>(x, rows, cols, axis, q, scales, vec, s);
        }
    } else {
        if (fmt == FP8Q_E4M3) {
            if (sat) launch_rowwise_t<FP8Q_F32, FP8Q_E4M3, true>(x, rows, cols, axis, q, scales, vec, s);
            else launch_rowwise_t<FP8Q_F32, FP8Q_E4M3, false>(x, rows, cols, axis, q, scales, vec, s);
        } else {
            if (sat) launch_rowwise_t<FP8Q_F32, FP8Q_E5M2, true>(x, rows, cols, axis, q, scales, vec, s);
            else launch_rowwise_t<FP8Q_F32, FP8Q_E5M2, false>(x, rows, cols, axis, q, scales, vec, s);
        }
    }
    if (qT != nullptr) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_transpose_u8(q, rows, cols, qT, s);
    }
    return hipGetLastError();
}

}  // namespace fp8q
