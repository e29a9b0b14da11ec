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
// pass 2 folds the partials into the scale and casts.
//  * A thread owns one unit, a 16-row block of 8 columns, at a time: 16 loads
//    of 16 bytes (bf16) from consecutive rows, the transforms of its 8
//    columns two at a time, 16 stores of 8 codes; neighbouring threads take
//    neighbouring column groups, so every load and store is coalesced.
//  * Both passes are persistent (two workgroups per CU, the most the
//    registers allow) and, for bf16, stage the thread's next unit in LDS with
//    direct-to-LDS loads while the current one is transformed, so each wave
//    keeps loads in flight without spending registers on them.  With one unit
//    per thread and nothing in flight during the transforms the pair was bound
//    by load latency, not by the ALU (123 us against 77 us for a bf16
//    [15872, 4096] operand, together with the two changes below).
//  * The factor 1/4 is not applied to y: pass 1 keeps max |H16 (d x)| and
//    scales that one value by 1/4 (exact, and rounding is monotone, so it is
//    the max of the rounded quarters), and pass 2 divides H16 (d x) by 4 s
//    instead of y by s.  Where (1/4) H16 (d x) is exact the two quotients are
//    the same real number; where it is not (|H16 (d x)| below 2^-124) both
//    quotients lie far below the smallest 8-bit subnormal and encode to a zero
//    of the same sign.  RN(1/(4 s)) = RN(1/s) / 4 for the reciprocal.
//  * When a wave's units all lie in one 16-row block (always, when the column
//    count is a multiple of 512), lanes 0-3 draw the block's 16 signs with one
//    generator call each and the wave shares them; otherwise every lane draws
//    its own block's signs.

#include <hip/hip_runtime.h>

#include <type_traits>

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

// The same bits when every active lane of the wave is in block b and lanes
// 0-3 are active: lane q draws the words of tokens 16 b + 4 q .. + 3.
__device__ __forceinline__ uint32_t rht_signs_wave(int64_t b, uint32_t k0, uint32_t k1) {
    const uint64_t g = (uint64_t)b * 4 + (threadIdx.x & 3);
    const uint4 w = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), 0u, 0u, k0, k1);
    const uint32_t nib = (w.x >> 31) | ((w.y >> 31) << 1) | ((w.z >> 31) << 2) | ((w.w >> 31) << 3);
    return (uint32_t)__builtin_amdgcn_readlane((int)nib, 0) | ((uint32_t)__builtin_amdgcn_readlane((int)nib, 1) << 4) |
           ((uint32_t)__builtin_amdgcn_readlane((int)nib, 2) << 8) | ((uint32_t)__builtin_amdgcn_readlane((int)nib, 3) << 12);
}

__device__ __forceinline__ uint32_t unit_signs(int64_t b, uint32_t k0, uint32_t k1) {
    const uint32_t blo = (uint32_t)b, bhi = (uint32_t)((uint64_t)b >> 32);
    const uint32_t flo = (uint32_t)__builtin_amdgcn_readfirstlane((int)blo),
                   fhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)bhi);
    const bool shared = __builtin_amdgcn_ballot_w64(blo != flo || bhi != fhi) == 0 &&
                        (__builtin_amdgcn_ballot_w64(true) & 0xfull) == 0xfull;
    return shared ? rht_signs_wave(b, k0, k1) : rht_signs(b, k0, k1);
}

// The raw rows of a unit: one 16-byte load per row (bf16, 8 columns), two
// (fp32).
template <int HP>
struct UnitRows {
    uint4 r[HP == FP8Q_BF16 ? 16 : 32];
};

template <int HP>
__device__ __forceinline__ void load_unit(const void* __restrict__ x, int64_t cols, int64_t b, int64_t c0,
                                          UnitRows<HP>& u) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t off = (b * 16 + i) * cols + c0;
        if constexpr (HP == FP8Q_BF16) {
            u.r[i] = load_stream16(reinterpret_cast<const uint16_t*>(x) + off);
        } else {
            u.r[2 * i] = load_stream16(reinterpret_cast<const float*>(x) + off);
            u.r[2 * i + 1] = load_stream16(reinterpret_cast<const float*>(x) + off + 4);
        }
    }
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int j) {
    return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// z = H16 (d x) (without the 1/4) of columns 2 j and 2 j + 1 of a unit: signs
// applied to the raw bits (exact), then the four butterfly stages in order.
template <int HP>
__device__ __forceinline__ void unit_pair(const UnitRows<HP>& u, int j, uint32_t signs, float za[16], float zb[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t neg = (uint32_t)(-(int32_t)((signs >> i) & 1u));   // all ones when row i is negated
        if constexpr (HP == FP8Q_BF16) {
            const uint32_t w = word_of(u.r[i], j) ^ (neg & 0x80008000u);
            za[i] = __uint_as_float(w << 16);
            zb[i] = __uint_as_float(w & 0xffff0000u);
        } else {
            const uint4& v = u.r[2 * i + (j >> 1)];
            za[i] = __uint_as_float(word_of(v, 2 * (j & 1)) ^ (neg & 0x80000000u));
            zb[i] = __uint_as_float(word_of(v, 2 * (j & 1) + 1) ^ (neg & 0x80000000u));
        }
    }
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if ((i & h) == 0) {
                const float a = za[i], c = za[i + h];
                za[i] = a + c;
                za[i + h] = a - c;
                const float e = zb[i], f = zb[i + h];
                zb[i] = e + f;
                zb[i + h] = e - f;
            }
}

// LDS staging of the next unit's rows (bf16): wave w's row i at
// stage + (16 w + i) * 1024, lane l's 16 bytes at + 16 l, written by
// direct-to-LDS loads, so prefetching takes no registers.
constexpr int kStageRowBytes = 64 * 16;
template <int HP>
constexpr int stage_bytes() { return HP == FP8Q_BF16 ? 4 * 16 * kStageRowBytes : 16; }

// The thread's units u = first, first + stride, ...: bf16 stages the next
// unit's rows in LDS while the current one is processed from registers; fp32
// loads each unit when it starts.
template <int HP, typename F>
__device__ __forceinline__ void run_units(const void* __restrict__ x, int64_t cols, int64_t ncg, int64_t nunits,
                                          int64_t stride, uint8_t* stage, F&& unit) {
    int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if constexpr (HP == FP8Q_BF16) {
        const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        uint8_t* my = stage + wave * 16 * kStageRowBytes;
        auto stage_unit = [&](int64_t v) {
            const uint16_t* src = reinterpret_cast<const uint16_t*>(x) + (v / ncg) * 16 * cols + (v % ncg) * 8;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + i * cols),
                                                 (__attribute__((address_space(3))) void*)(my + i * kStageRowBytes),
                                                 16, 0, 0);
        };
        if (u < nunits) stage_unit(u);
        for (; u < nunits; u += stride) {
            UnitRows<HP> cur;
#pragma unroll
            for (int i = 0; i < 16; ++i)   // (the compiler waits for the staging loads first)
                cur.r[i] = *reinterpret_cast<const uint4*>(my + i * kStageRowBytes + lane * 16);
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the rows are read before the next unit overwrites them
            if (u + stride < nunits) stage_unit(u + stride);
            unit(cur, u);
        }
    } else {
        for (; u < nunits; u += stride) {
            UnitRows<HP> cur;
            load_unit<HP>(x, cols, u / ncg, (u % ncg) * 8, cur);
            unit(cur, u);
        }
    }
}

// Grid of both passes: persistent, two workgroups per CU, at most one thread
// per unit.
static int rht_grid(int64_t rows, int64_t cols) {
    const int64_t want = (rows / 16 * (cols / 8) + 255) / 256;
    const int cap = 2 * persistent_grid();
    return (int)(want < cap ? (want < 1 ? 1 : want) : cap);
}

// Pass 1: one partial max |y| per block.
template <int HP>
__global__ __launch_bounds__(256, 2) void rht_amax_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                          uint32_t k0, uint32_t k1, float* __restrict__ partials) {
    __shared__ uint32_t red[4];
    __shared__ __attribute__((aligned(1024))) uint8_t stage[stage_bytes<HP>()];
    const int64_t ncg = cols / 8, nunits = rows / 16 * ncg, stride = (int64_t)gridDim.x * 256;
    uint32_t key = 0;
    auto unit = [&](const UnitRows<HP>& cur, int64_t u) {
        const int64_t b = u / ncg;
        const uint32_t signs = unit_signs(b, k0, k1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float za[16], zb[16];
            unit_pair<HP>(cur, j, signs, za, zb);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t ka = abs_key(za[i]), kb = abs_key(zb[i]);
                key = key > ka ? key : ka;
                key = key > kb ? key : kb;
            }
        }
    };
    run_units<HP>(x, cols, ncg, nunits, stride, stage, unit);
    key = block_max_u32_256(key, red);
    // max |y| = RN(max |z| / 4): the quarter is exact and rounding is monotone
    if (threadIdx.x == 0) partials[blockIdx.x] = __uint_as_float(key) * 0.25f;
}

// Pass 2: scale from the partials, then cast y = z / 4 as z / (4 s).
template <int HP, int FMT, bool SAT>
__global__ __launch_bounds__(256, 2) void rht_cast_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                          uint32_t k0, uint32_t k1, const float* __restrict__ partials,
                                                          int nparts, uint8_t* __restrict__ q, float* scale_out,
                                                          float* amax_out) {
    __shared__ uint32_t red[4];
    __shared__ __attribute__((aligned(1024))) uint8_t stage[stage_bytes<HP>()];
    const float amax = reduce_partials_256(partials, nparts, red);
    const float s = scale_from_amax<FMT>(amax);
    const float s4 = 4.0f * s, rc4 = 0.25f * (1.0f / s);   // 4 s and RN(1 / (4 s)), both exact scalings
    const int64_t ncg = cols / 8, nunits = rows / 16 * ncg, stride = (int64_t)gridDim.x * 256;
    // a finite s comes from this tensor's own amax, so the division needs no
    // check for a non-finite quotient; an infinite or NaN s gives z * (1 / 4s)
    // for every element (separate copies of the loop)
    auto run = [&](auto finite_c) {
    constexpr bool FIN = decltype(finite_c)::value;
    auto unit = [&](const UnitRows<HP>& cur, int64_t u) {
        const int64_t b = u / ncg, c0 = (u % ncg) * 8;
        const uint32_t signs = unit_signs(b, k0, k1);
        auto div = [&](float z) { return FIN ? div_by_own_scale(z, s4, rc4) : z * rc4; };
        // bf16: the 8 codes of a row in one store (two 4-byte halves stored
        // apart cost 1.5x the write traffic: partial lines).  fp32, whose rows
        // take twice the registers, stores the halves apart.
        constexpr int kParts = HP == FP8Q_BF16 ? 1 : 2, kPairs = 4 / kParts;
#pragma unroll
        for (int h = 0; h < kParts; ++h) {
            uint32_t w[16][2];
#pragma unroll
            for (int jj = 0; jj < kPairs; ++jj) {
                float za[16], zb[16];
                unit_pair<HP>(cur, h * kPairs + jj, signs, za, zb);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float ca = saturate<FMT, SAT>(div(za[i]));
                    const float cb = saturate<FMT, SAT>(div(zb[i]));
                    w[i][jj >> 1] = (jj & 1) ? pack2_hi<FMT>(ca, cb, w[i][jj >> 1]) : pack2_lo<FMT>(ca, cb);
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint8_t* dst = q + (b * 16 + i) * cols + c0;
                if constexpr (kParts == 1) *reinterpret_cast<uint2*>(dst) = make_uint2(w[i][0], w[i][1]);
                else *reinterpret_cast<uint32_t*>(dst + 4 * h) = w[i][0];
            }
        }
    };
    run_units<HP>(x, cols, ncg, nunits, stride, stage, unit);
    };
    if (__builtin_isfinite(s)) run(std::true_type{});
    else run(std::false_type{});
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *scale_out = s;
        if (amax_out) *amax_out = amax;
    }
}

template <int HP, int FMT, bool SAT>
static void launch_rht_t(const void* x, int64_t rows, int64_t cols, uint32_t k0, uint32_t k1, float* partials,
                         int nparts, uint8_t* q, float* scale_out, float* amax_out, hipStream_t s) {
    hipLaunchKernelGGL((rht_amax_kernel<HP>), dim3(nparts), dim3(256), 0, s, x, rows, cols, k0, k1, partials);
    hipLaunchKernelGGL((rht_cast_kernel<HP, FMT, SAT>), dim3(rht_grid(rows, cols)), dim3(256), 0, s, x, rows, cols, k0,
                       k1, partials, nparts, q, scale_out, amax_out);
}

int rht_partials_grid(int64_t rows, int64_t cols) {
    const int g = rht_grid(rows, cols);
    return g < kReduceParts ? g : kReduceParts;
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
