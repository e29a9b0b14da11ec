// amax reduction and FP8 quantization kernels for gfx950.
//
// What is computed follows the "fp8_parity.py" lab page, scaled_roundtrip:
// amax = max|x|, s = max(amax / fmax, 1e-12) in fp32, q = fp8(RN32(x / s)),
// and its smoke checks [3] (delayed scaling from an amax history) and [4]
// (1x128 tiles); 128x128 blocks and MX32 follow the recipe names "block" and
// "mxfp8" of SpikingJelly's "Training and Inference Precision" page.
//
// Design: everything is HBM-bound (2-4 B read and 1 B written per element), so
// the kernels stream 16-byte vector loads, keep one 128 x 128 tile per block
// in registers (64 values per thread), reduce tile maxima with wavefront
// shuffles and a little LDS, and stage codes in LDS only when a transposed
// copy is written.  Per-tensor current scaling is two-pass by dependency: an
// amax grid writes one partial maximum per block, and every block of the cast
// grid folds those partials (<= 1024 floats) into the scale itself, so no
// separate finalize launch sits between the passes.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace fp8q {

// ------------------------------------------------------------------ grid completion

// Called by thread 0 of every block once its key is final.  The key goes to
// keys[block] with an atomic exchange; the block then takes a ticket in a
// two-level tree (a counter per group of kTicketGroup blocks, each on its own
// 256-byte line, then a top counter), so no address sees more than
// kTicketGroup atomics.  Each ticket's increment is made to depend on the
// return of the atomic before it, so it is taken only after that atomic has
// been performed; the block that takes the last top ticket therefore sees
// every key.  Returns true in that one block.  Counters start at zero and are
// left at zero.
__device__ __forceinline__ bool grid_done(uint32_t* keys, uint32_t* ctrs, uint32_t key) {
    const uint32_t b = blockIdx.x, nb = gridDim.x;
    const uint32_t prev = atomicExch(&keys[b], key);
    uint32_t one;
    __asm__ volatile("v_mov_b32 %0, 1" : "=v"(one) : "v"(prev));
    const uint32_t g = b / kTicketGroup;
    const uint32_t gsize = nb - g * kTicketGroup < (uint32_t)kTicketGroup ? nb - g * kTicketGroup : kTicketGroup;
    uint32_t* gc = &ctrs[kTicketLine * (1 + g)];
    const uint32_t t = atomicAdd(gc, one);
    if (t != gsize - 1) return false;
    atomicExch(gc, 0u);
    __asm__ volatile("v_mov_b32 %0, 1" : "=v"(one) : "v"(t));
    const uint32_t ngroups = (nb + kTicketGroup - 1) / kTicketGroup;
    const uint32_t t2 = atomicAdd(&ctrs[0], one);
    if (t2 != ngroups - 1) return false;
    atomicExch(&ctrs[0], 0u);
    return true;
}

// Max of keys[0..n), n <= kReduceParts, read with device-coherent atomic
// loads (all 256 threads; a thread's loads are issued together).
__device__ __forceinline__ uint32_t fold_keys_256(const uint32_t* keys, int n, uint32_t* lds4) {
    static_assert(kReduceParts <= 256 * 8, "eight keys per thread");
    uint32_t k[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = threadIdx.x + 256 * u;
        k[u] = i < n ? __hip_atomic_load(&keys[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    }
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) m = m > k[u] ? m : k[u];
    return block_max_u32_256(m, lds4);
}

// ------------------------------------------------------------------ amax

// One partial maximum per block over a grid-stride range of x.  The abs key
// (bits with the sign cleared) is maximised as an integer: NaN propagates.
// bf16 keys are maximised two at a time as packed 16-bit integers.
// With `keys` set, the blocks fold their maxima with grid_done and the last
// block to finish writes the result to *amax_out: a standalone amax is one
// launch.
template <int HP>
__global__ __launch_bounds__(256) void amax_partials_kernel(const void* __restrict__ x, int64_t n,
                                                            float* __restrict__ partials,
                                                            fp8q_delayed_state* __restrict__ gate,
                                                            int vec, uint32_t* keys, uint32_t* ctrs,
                                                            float* amax_out) {
    __shared__ uint32_t red[4];
    __shared__ uint32_t last;
    if (gate != nullptr) {
        // the delayed cast launched next counts its overflows into the state
        if (blockIdx.x == 0 && threadIdx.x == 0) gate->overflows = 0u;
        uint32_t h = 0;
#pragma unroll
        for (int i = 0; i < FP8Q_HISTORY_LEN; ++i) h |= __float_as_uint(gate->amax_history[i]);
        if ((h & 0x7fffffffu) != 0) return;   // warm history: the delayed cast needs no amax pass
    }
    constexpr int EPV = HP == FP8Q_BF16 ? 8 : 4;   // elements per 16-byte vector
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nthr = (int64_t)gridDim.x * 256;
    uint32_t key = 0;
    int64_t done = 0;   // elements covered by the vector loop
    if (vec) {
        // one contiguous run of 16-byte vectors per block (a multiple of 256
        // vectors), 8 loads in flight per thread, masked at the run's end
        const uint4* __restrict__ xv = reinterpret_cast<const uint4*>(x);
        const int64_t nv = n / EPV;
        done = nv * EPV;
        const int64_t per = ((nv + gridDim.x - 1) / gridDim.x + 255) / 256 * 256;
        const int64_t b0 = (int64_t)blockIdx.x * per;
        const int64_t b1 = b0 + per < nv ? b0 + per : nv;
        if constexpr (HP == FP8Q_BF16) {
            typedef unsigned short us2 __attribute__((ext_vector_type(2)));
            us2 m2 = {0, 0};
            for (int64_t i = b0 + threadIdx.x; i < b1; i += 256 * 8) {
                uint4 w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) w[u] = i + u * 256 < b1 ? load_stream16(xv + i + u * 256) : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t d[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(us2, d[j] & 0x7fff7fffu));
                }
            }
            const uint32_t a = m2.x, b = m2.y;
            key = (a > b ? a : b) << 16;
        } else {
            for (int64_t i = b0 + threadIdx.x; i < b1; i += 256 * 8) {
                uint4 w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) w[u] = i + u * 256 < b1 ? load_stream16(xv + i + u * 256) : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t d[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t k = d[j] & 0x7fffffffu;
                        key = key > k ? key : k;
                    }
                }
            }
        }
    }
    for (int64_t i = done + tid; i < n; i += nthr) {   // tail, or everything when unaligned
        uint32_t k;
        if constexpr (HP == FP8Q_BF16) k = ((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16) & 0x7fffffffu;
        else k = reinterpret_cast<const uint32_t*>(x)[i] & 0x7fffffffu;
        key = key > k ? key : k;
    }
    key = block_max_u32_256(key, red);
    if (keys == nullptr) {
        if (threadIdx.x == 0) partials[blockIdx.x] = __uint_as_float(key);
        return;
    }
    if (threadIdx.x == 0) last = grid_done(keys, ctrs, key);
    __syncthreads();
    if (!last) return;
    const uint32_t all = fold_keys_256(keys, gridDim.x, red);
    if (threadIdx.x == 0) *amax_out = __uint_as_float(all);
}

// At most 512 blocks (two per CU): every block of the cast that follows folds
// these partials again, and 512 of them instead of 2048 made the transposing
// per-tensor cast 5% and the SR cast 4% faster on bf16 [15872, 4096] (the
// flat cast 1% slower, the autocast layer 0.4% faster; A/B in one call).
int amax_partials_grid(int64_t n) {
    const int64_t per_block = 256 * 8 * 8;   // 8 vectors of up to 8 elements per thread
    int64_t g = (n + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 512) g = 512;
    return (int)g;
}

hipError_t launch_amax_partials(const void* x, int hp, int64_t n, float* partials, int nparts,
                                fp8q_delayed_state* gate, hipStream_t s, uint32_t* keys,
                                uint32_t* ctrs, float* amax_out) {
    const int vec = ((uintptr_t)x % 16) == 0;
    if (hp == FP8Q_BF16)
        hipLaunchKernelGGL(amax_partials_kernel<FP8Q_BF16>, dim3(nparts), dim3(256), 0, s, x, n, partials, gate, vec,
                           keys, ctrs, amax_out);
    else
        hipLaunchKernelGGL(amax_partials_kernel<FP8Q_F32>, dim3(nparts), dim3(256), 0, s, x, n, partials, gate, vec,
                           keys, ctrs, amax_out);
    return hipGetLastError();
}


// ------------------------------------------------------------------ LDS tile transposes

constexpr int kTile = 128;          // tile edge (rows and columns)
constexpr int kLdsStride = 132;     // bytes per LDS row of a code tile (padded against bank conflicts)

// 4 x 4 byte transpose: d_i holds 4 consecutive bytes of row i; e_j returns
// column j (byte i from d_i).  v_perm_b32 picks bytes 0-3 from its second
// source and 4-7 from its first.
__device__ __forceinline__ void transpose4x4(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3,
                                             uint32_t& e0, uint32_t& e1, uint32_t& e2, uint32_t& e3) {
    const uint32_t t0 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);   // d0b0 d1b0 d0b1 d1b1
    const uint32_t t1 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);   // d0b2 d1b2 d0b3 d1b3
    const uint32_t t2 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);   // d2b0 d3b0 d2b1 d3b1
    const uint32_t t3 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);   // d2b2 d3b2 d2b3 d3b3
    e0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    e1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    e2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    e3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Write the transpose of a 128 x 128 code tile held in LDS (rows of kLdsStride
// bytes) to out[col * ld + row] for tile origin (r0, c0) of a rows x cols
// matrix (out is [cols, rows], ld = rows).  Thread t writes columns
// 4*(t/8)..+3, rows 16*(t%8)..+15: eight neighbouring threads cover 128
// contiguous output bytes.
__device__ __forceinline__ void store_tile_transposed(const uint8_t* lds, uint8_t* __restrict__ out,
                                                      int64_t rows, int64_t cols, int64_t r0, int64_t c0,
                                                      bool vec) {
    const int t = threadIdx.x;
    const int cg = t >> 3, rs = t & 7;
    uint32_t d[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        d[i] = *reinterpret_cast<const uint32_t*>(lds + (rs * 16 + i) * kLdsStride + cg * 4);
    uint32_t col[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        transpose4x4(d[4 * b], d[4 * b + 1], d[4 * b + 2], d[4 * b + 3], col[0][b], col[1][b], col[2][b], col[3][b]);
    const int64_t rbase = r0 + rs * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t c = c0 + cg * 4 + j;
        if (c >= cols || rbase >= rows) continue;
        uint8_t* dst = out + c * rows + rbase;
        if (vec && rbase + 16 <= rows) {
            *reinterpret_cast<uint4*>(dst) = make_uint4(col[j][0], col[j][1], col[j][2], col[j][3]);
        } else {
            for (int i = 0; i < 16 && rbase + i < rows; ++i) dst[i] = (uint8_t)(col[j][i >> 2] >> (8 * (i & 3)));
        }
    }
}

// ------------------------------------------------------------------ overflow count

// 1 if the cast of a finite x, with quotient v = RN32(x / s), overflows the
// format: the non-saturating conversion gives NaN (E4M3: |v| > 464; 464
// itself is the tie that rounds to the even-mantissa 448) or +-Inf (E5M2:
// |v| >= 61440, the tie above 57344 that rounds to even 2^16).
template <int FMT>
__device__ __forceinline__ uint32_t overflowed(float x, float v) {
    const bool finite = (__float_as_uint(x) & 0x7fffffffu) < 0x7f800000u;
    const float av = __builtin_fabsf(v);
    return finite && (FMT == FP8Q_E4M3 ? av > 464.0f : av >= 61440.0f) ? 1u : 0u;
}

// Adds the block's overflow count to the delayed state (integer atomics:
// the total does not depend on their order).
__device__ __forceinline__ void add_overflows(fp8q_delayed_state* st, uint32_t n, uint32_t* lds_sum) {
    if (threadIdx.x == 0) *lds_sum = 0u;
    __syncthreads();
    if (n != 0u) atomicAdd(lds_sum, n);
    __syncthreads();
    if (threadIdx.x == 0 && *lds_sum != 0u) atomicAdd(&st->overflows, *lds_sum);
}

// ------------------------------------------------------------------ tiled quantize

template <int HP>
__device__ __forceinline__ void load8(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t row,
                                      int64_t col, bool vec, float v[8]) {
    if (row < rows && vec && col + 8 <= cols) {
        if constexpr (HP == FP8Q_BF16) {
            const uint4 w = load_stream16(reinterpret_cast<const uint16_t*>(x) + row * cols + col);
            const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[2 * j] = __uint_as_float(d[j] << 16);
                v[2 * j + 1] = __uint_as_float(d[j] & 0xffff0000u);
            }
        } else {
            const float* p = reinterpret_cast<const float*>(x) + row * cols + col;
            const uint4 a = load_stream16(p), b = load_stream16(p + 4);
            v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
            v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
            v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
            v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float f = 0.0f;
            if (row < rows && col + e < cols) {
                if constexpr (HP == FP8Q_BF16) f = bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[row * cols + col + e]);
                else f = reinterpret_cast<const float*>(x)[row * cols + col + e];
            }
            v[e] = f;
        }
    }
}

// One block quantizes 128 x 128 tiles of x (grid-stride over tiles).  Thread t
// owns rows rg + 16p (p = 0..7, rg = t/16) and columns 8cc..8cc+7 (cc = t%16)
// of the tile: 64 values.
template <int HP, int FMT, int SCHEME, bool SAT>
__global__ __launch_bounds__(256) void quantize_tiled_kernel(QuantArgs a, int64_t ntr, int64_t ntc,
                                                             int vec_in, int vec_q, int vec_qt) {
    __shared__ uint32_t red[4];
    __shared__ __attribute__((aligned(16))) uint8_t lds_codes[kTile * kLdsStride];
    // cross-wave column maxima (axis-1 schemes only; the others keep their LDS
    // small so that more blocks fit on a CU)
    constexpr bool kColumnTiles = SCHEME == kTileAxis1 || SCHEME == kMxAxis1;
    __shared__ uint32_t lds_col[kColumnTiles ? 4 * 4 * kTile : 1];

    const int t = threadIdx.x;
    const int cc = t & 15, rg = t >> 4, wave = t >> 6;
    const int64_t rows = a.rows, cols = a.cols;
    constexpr bool kPerTensor = SCHEME == kPerTensorCurrent || SCHEME == kPerTensorDelayed;

    // per-tensor scale, identical in every block
    float s_pt = 0.0f, r_pt = 0.0f, amax_pt = 0.0f;
    bool cold = false;
    if constexpr (SCHEME == kPerTensorCurrent) {
        amax_pt = reduce_partials_256(a.partials, a.nparts, red);
        s_pt = scale_from_amax<FMT>(amax_pt);
    } else if constexpr (SCHEME == kPerTensorDelayed) {
        uint32_t h = 0, any = 0;
#pragma unroll
        for (int i = 0; i < FP8Q_HISTORY_LEN; ++i) {
            const uint32_t b = __float_as_uint(a.state->amax_history[i]);
            any |= b;
            const uint32_t k = b & 0x7fffffffu;
            h = h > k ? h : k;
        }
        cold = (any & 0x7fffffffu) == 0;
        const float hmax = cold ? reduce_partials_256(a.partials, a.nparts, red) : __uint_as_float(h);
        s_pt = scale_from_amax<FMT>(hmax);
    }
    if constexpr (kPerTensor) r_pt = 1.0f / s_pt;

    uint32_t key_all = 0;   // running amax key (delayed scaling)
    uint32_t nov = 0;       // overflowing elements (delayed scaling, COUNT_OVERFLOW)
    const int64_t ntiles = ntr * ntc;
    // A whole tile inside the matrix with aligned rows is loaded a tile ahead:
    // its raw 16-byte pieces are in flight while the block works on the
    // previous tile (edge tiles take the element-checked path on the spot).
    constexpr int RAWN = HP == FP8Q_BF16 ? 1 : 2;   // 16-byte pieces per 8 elements
    auto whole = [&](int64_t tl) {
        return vec_in && (tl / ntc + 1) * kTile <= rows && (tl % ntc + 1) * kTile <= cols;
    };
    uint4 raw[8][RAWN];
    auto raw_load = [&](int64_t tl) {
        const int64_t rr = (tl / ntc) * kTile + rg, cl = (tl % ntc) * kTile + cc * 8;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const char* base = reinterpret_cast<const char*>(a.x) + ((rr + 16 * p) * cols + cl) * (HP == FP8Q_F32 ? 4 : 2);
#pragma unroll
            for (int q = 0; q < RAWN; ++q) raw[p][q] = load_stream16(base + 16 * q);
        }
    };
    bool ahead = (int64_t)blockIdx.x < ntiles && whole(blockIdx.x);
    if (ahead) raw_load(blockIdx.x);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t tr = tile / ntc, tc = tile % ntc;
        const int64_t r0 = tr * kTile, c0 = tc * kTile;
        const int64_t col = c0 + cc * 8;

        float v[8][8];
        if (ahead) {
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                if constexpr (HP == FP8Q_BF16) {
                    const uint32_t d[4] = {raw[p][0].x, raw[p][0].y, raw[p][0].z, raw[p][0].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        v[p][2 * j] = __uint_as_float(d[j] << 16);
                        v[p][2 * j + 1] = __uint_as_float(d[j] & 0xffff0000u);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < RAWN; ++q) {
                        v[p][4 * q] = __uint_as_float(raw[p][q].x);
                        v[p][4 * q + 1] = __uint_as_float(raw[p][q].y);
                        v[p][4 * q + 2] = __uint_as_float(raw[p][q].z);
                        v[p][4 * q + 3] = __uint_as_float(raw[p][q].w);
                    }
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < 8; ++p) load8<HP>(a.x, rows, cols, r0 + rg + 16 * p, col, vec_in, v[p]);
        }
        {
            const int64_t nt = tile + gridDim.x;
            ahead = nt < ntiles && whole(nt);
            if (ahead) raw_load(nt);
        }

        uint32_t kp[8];   // per-row keys over this thread's 8 values
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            uint32_t k = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) { const uint32_t z = abs_key(v[p][e]); k = k > z ? k : z; }
            kp[p] = k;
        }

        uint32_t codes[8][2];
        if constexpr (kPerTensor) {
            if constexpr (SCHEME == kPerTensorDelayed) {
#pragma unroll
                for (int p = 0; p < 8; ++p) key_all = key_all > kp[p] ? key_all : kp[p];
            }
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                float d[8], q[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    d[e] = div_by_scale(v[p][e], s_pt, r_pt);
                    q[e] = saturate<FMT, SAT>(d[e]);
                }
                // elements outside the matrix were loaded as zeros: never counted
                if (SCHEME == kPerTensorDelayed && a.count_overflow) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) nov += overflowed<FMT>(v[p][e], d[e]);
                }
                codes[p][0] = pack4<FMT>(q[0], q[1], q[2], q[3]);
                codes[p][1] = pack4<FMT>(q[4], q[5], q[6], q[7]);
            }
        } else if constexpr (SCHEME == kTileAxis0 || SCHEME == kMxAxis0) {
            const int64_t nst = SCHEME == kTileAxis0 ? (cols + 127) / 128 : (cols + 31) / 32;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int64_t row = r0 + rg + 16 * p;
                float q[8];
                if constexpr (SCHEME == kTileAxis0) {
                    const uint32_t k = row16_max_u32(kp[p]);
                    const float s = scale_from_amax<FMT>(__uint_as_float(k));
                    const float r = 1.0f / s;
#pragma unroll
                    for (int e = 0; e < 8; ++e) q[e] = saturate<FMT, SAT>(div_by_scale(v[p][e], s, r));
                    if (cc == 0 && row < rows) a.scales[row * nst + tc] = s;
                } else {
                    const uint32_t k = quad_max_u32(kp[p]);
                    const int code = e8m0_from_scale(scale_from_amax<FMT>(__uint_as_float(k)));
                    const float inv = e8m0_recip(code);
#pragma unroll
                    for (int e = 0; e < 8; ++e) q[e] = saturate<FMT, SAT>(v[p][e] * inv);
                    if ((cc & 3) == 0 && row < rows && col < cols) a.e8m0[row * nst + (col >> 5)] = (uint8_t)code;
                }
                codes[p][0] = pack4<FMT>(q[0], q[1], q[2], q[3]);
                codes[p][1] = pack4<FMT>(q[4], q[5], q[6], q[7]);
            }
        } else if constexpr (SCHEME == kBlock) {
            uint32_t k = 0;
#pragma unroll
            for (int p = 0; p < 8; ++p) k = k > kp[p] ? k : kp[p];
            k = block_max_u32_256(k, red);
            const float s = scale_from_amax<FMT>(__uint_as_float(k));
            const float r = 1.0f / s;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                float q[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) q[e] = saturate<FMT, SAT>(div_by_scale(v[p][e], s, r));
                codes[p][0] = pack4<FMT>(q[0], q[1], q[2], q[3]);
                codes[p][1] = pack4<FMT>(q[4], q[5], q[6], q[7]);
            }
            if (t == 0) a.scales[tr * ntc + tc] = s;
        } else {   // kTileAxis1 / kMxAxis1: maxima down each column of the tile
            constexpr int NSEG = SCHEME == kTileAxis1 ? 1 : 4;   // 128-row or 32-row segments
            uint32_t kc[NSEG][8];
#pragma unroll
            for (int sgm = 0; sgm < NSEG; ++sgm)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint32_t k = 0;
#pragma unroll
                    for (int p = sgm * (8 / NSEG); p < (sgm + 1) * (8 / NSEG); ++p) {
                        const uint32_t z = abs_key(v[p][e]);
                        k = k > z ? k : z;
                    }
                    kc[sgm][e] = lanes_max_u32<16, 32>(k);
                }
            if ((t & 63) < 16) {
#pragma unroll
                for (int sgm = 0; sgm < NSEG; ++sgm)
#pragma unroll
                    for (int e = 0; e < 8; ++e) lds_col[(wave * 4 + sgm) * kTile + cc * 8 + e] = kc[sgm][e];
            }
            __syncthreads();
#pragma unroll
            for (int sgm = 0; sgm < NSEG; ++sgm)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint32_t k = 0;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint32_t z = lds_col[(w * 4 + sgm) * kTile + cc * 8 + e];
                        k = k > z ? k : z;
                    }
                    kc[sgm][e] = k;
                }
            float sc[NSEG][8], rc[NSEG][8];
#pragma unroll
            for (int sgm = 0; sgm < NSEG; ++sgm)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float s = scale_from_amax<FMT>(__uint_as_float(kc[sgm][e]));
                    if constexpr (SCHEME == kTileAxis1) {
                        sc[sgm][e] = s;
                        rc[sgm][e] = 1.0f / s;
                    } else {
                        const int code = e8m0_from_scale(s);
                        sc[sgm][e] = (float)code;
                        rc[sgm][e] = e8m0_recip(code);
                    }
                }
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int sgm = p / (8 / NSEG);
                float q[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if constexpr (SCHEME == kTileAxis1) q[e] = saturate<FMT, SAT>(div_by_scale(v[p][e], sc[sgm][e], rc[sgm][e]));
                    else q[e] = saturate<FMT, SAT>(v[p][e] * rc[sgm][e]);
                }
                codes[p][0] = pack4<FMT>(q[0], q[1], q[2], q[3]);
                codes[p][1] = pack4<FMT>(q[4], q[5], q[6], q[7]);
            }
            if (rg == 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int64_t c = col + e;
                    if (c >= cols) continue;
                    if constexpr (SCHEME == kTileAxis1) {
                        a.scales[c * ((rows + 127) / 128) + tr] = sc[0][e];
                    } else {
                        const int64_t nseg = (rows + 31) / 32;
#pragma unroll
                        for (int sgm = 0; sgm < NSEG; ++sgm)
                            if (r0 + 32 * sgm < rows) a.e8m0[c * nseg + r0 / 32 + sgm] = (uint8_t)sc[sgm][e];
                    }
                }
            }
        }

        // codes, row-major
        if (a.q != nullptr) {
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int64_t row = r0 + rg + 16 * p;
                if (row >= rows || col >= cols) continue;
                uint8_t* dst = a.q + row * cols + col;
                if (vec_q && col + 8 <= cols) {
                    *reinterpret_cast<uint2*>(dst) = make_uint2(codes[p][0], codes[p][1]);
                } else {
                    for (int e = 0; e < 8 && col + e < cols; ++e) dst[e] = (uint8_t)(codes[p][e >> 2] >> (8 * (e & 3)));
                }
            }
        }
        // codes, transposed (through LDS)
        if (a.qT != nullptr) {
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                uint32_t* dst = reinterpret_cast<uint32_t*>(lds_codes + (rg + 16 * p) * kLdsStride + cc * 8);
                dst[0] = codes[p][0];
                dst[1] = codes[p][1];
            }
            __syncthreads();
            store_tile_transposed(lds_codes, a.qT, rows, cols, r0, c0, vec_qt);
        }
        __syncthreads();   // LDS reuse by the next tile
    }

    if constexpr (SCHEME == kPerTensorCurrent) {
        if (blockIdx.x == 0 && t == 0) {
            *a.scale_out = s_pt;
            if (a.amax_out) *a.amax_out = amax_pt;
        }
    } else if constexpr (SCHEME == kPerTensorDelayed) {
        // The grid's amax goes into the history after every block has cast with
        // the old scale: the last block to finish folds the per-block maxima
        // and records it.
        __shared__ uint32_t last, ov_sum;
        if (a.count_overflow) add_overflows(a.state, nov, &ov_sum);
        const uint32_t k = block_max_u32_256(key_all, red);
        if (t == 0) last = grid_done(a.keys, a.ctrs, k);
        __syncthreads();
        if (last) {
            const float amax = __uint_as_float(fold_keys_256(a.keys, gridDim.x, red));
            if (t == 0) {
                fp8q_delayed_state* st = a.state;
                const int pos = st->pos;
                st->amax_history[pos] = amax;
                st->pos = (pos + 1) % FP8Q_HISTORY_LEN;
                st->last_scale = s_pt;
                *a.scale_out = s_pt;
                if (a.amax_out) *a.amax_out = amax;
            }
        }
    }
}

// Plain transpose of a code matrix through LDS (128 x 128 tiles).
__global__ __launch_bounds__(256) void transpose_u8_kernel(const uint8_t* __restrict__ in, int64_t rows, int64_t cols,
                                                           uint8_t* __restrict__ out, int64_t ntr, int64_t ntc,
                                                           int vec_in, int vec_out) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kTile * kLdsStride];
    const int t = threadIdx.x;
    const int ch = t & 7, rr = t >> 3;
    const int64_t ntiles = ntr * ntc;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t r0 = (tile / ntc) * kTile, c0 = (tile % ntc) * kTile;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lr = rr + 32 * i;
            const int64_t row = r0 + lr, col = c0 + ch * 16;
            uint4 w = make_uint4(0, 0, 0, 0);
            if (row < rows && col < cols) {
                if (vec_in && col + 16 <= cols) {
                    w = load_stream16(in + row * cols + col);
                } else {
                    uint32_t d[4] = {0, 0, 0, 0};
                    for (int e = 0; e < 16 && col + e < cols; ++e) d[e >> 2] |= (uint32_t)in[row * cols + col + e] << (8 * (e & 3));
                    w = make_uint4(d[0], d[1], d[2], d[3]);
                }
            }
            uint32_t* dst = reinterpret_cast<uint32_t*>(lds + lr * kLdsStride + ch * 16);
            dst[0] = w.x; dst[1] = w.y; dst[2] = w.z; dst[3] = w.w;
        }
        __syncthreads();
        store_tile_transposed(lds, out, rows, cols, r0, c0, vec_out);
        __syncthreads();
    }
}

// ------------------------------------------------------------------ flat quantize
//
// Row-major quantizers whose scale groups run along the rows (per tensor, 1x128
// tiles, MX32 blocks along the columns) and with no transposed copy: the
// tensor is streamed as a flat array of 8-element units (16 bytes of bf16, 32
// of fp32).  Each block takes one contiguous run of units (a multiple of 256,
// so a 1x128 tile - 16 units - or an MX block - 4 units - never straddles
// blocks or lane groups), each thread keeps UNR units in flight, tile and MX
// maxima are reduced across 16 or 4 neighbouring lanes, and every lane stores
// its 8 codes as one 8-byte word.  The flat unit index also gives the scale
// index directly: unit u belongs to 1x128 tile u / 16 and MX block u / 4.
// One loaded 8-element unit, kept as the raw 16 (bf16) or 32 (fp32) bytes
// until it is cast, so that a thread's UNR units in flight cost 4 (8) VGPRs
// each rather than 8 unpacked floats.
template <int HP>
struct Unit {
    uint4 w[HP == FP8Q_BF16 ? 1 : 2];

    __device__ __forceinline__ void load(const void* __restrict__ x, int64_t u) {
        if constexpr (HP == FP8Q_BF16) {
            w[0] = load_stream16(reinterpret_cast<const uint4*>(x) + u);
        } else {
            w[0] = load_stream16(reinterpret_cast<const uint4*>(x) + 2 * u);
            w[1] = load_stream16(reinterpret_cast<const uint4*>(x) + 2 * u + 1);
        }
    }
    // max |x| over the unit as an abs key (NaN sorts above Inf); bf16 keys
    // are maximised two at a time as packed 16-bit integers
    __device__ __forceinline__ uint32_t key() const {
        if constexpr (HP == FP8Q_BF16) {
            typedef unsigned short us2 __attribute__((ext_vector_type(2)));
            const uint32_t d[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
            us2 m = {0, 0};
#pragma unroll
            for (int j = 0; j < 4; ++j) m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, d[j] & 0x7fff7fffu));
            const uint32_t a = m.x, b = m.y;
            return (a > b ? a : b) << 16;
        } else {
            const uint32_t d[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
            uint32_t k = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) { const uint32_t z = d[e] & 0x7fffffffu; k = k > z ? k : z; }
            return k;
        }
    }
    __device__ __forceinline__ void unpack(float v[8]) const {
        if constexpr (HP == FP8Q_BF16) {
            const uint32_t d[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[2 * j] = __uint_as_float(d[j] << 16);
                v[2 * j + 1] = __uint_as_float(d[j] & 0xffff0000u);
            }
        } else {
            const uint32_t d[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(d[e]);
        }
    }
};

template <int HP, int FMT, int SCHEME, bool SAT>
__global__ __launch_bounds__(256) void quantize_flat_kernel(QuantArgs a, int64_t nunits) {
    constexpr int UNR = HP == FP8Q_BF16 ? 8 : 4;
    constexpr bool kPerTensor = SCHEME == kPerTensorCurrent || SCHEME == kPerTensorDelayed;
    __shared__ uint32_t red[4];
    const int t = threadIdx.x;

    float s_pt = 0.0f, r_pt = 0.0f, amax_pt = 0.0f;
    if constexpr (SCHEME == kPerTensorCurrent) {
        amax_pt = reduce_partials_256(a.partials, a.nparts, red);
        s_pt = scale_from_amax<FMT>(amax_pt);
    } else if constexpr (SCHEME == kPerTensorDelayed) {
        uint32_t h = 0, any = 0;
#pragma unroll
        for (int i = 0; i < FP8Q_HISTORY_LEN; ++i) {
            const uint32_t b = __float_as_uint(a.state->amax_history[i]);
            any |= b;
            const uint32_t k = b & 0x7fffffffu;
            h = h > k ? h : k;
        }
        const bool cold = (any & 0x7fffffffu) == 0;
        const float hmax = cold ? reduce_partials_256(a.partials, a.nparts, red) : __uint_as_float(h);
        s_pt = scale_from_amax<FMT>(hmax);
    }
    if constexpr (kPerTensor) r_pt = 1.0f / s_pt;

    const int64_t per = ((nunits + gridDim.x - 1) / gridDim.x + 255) / 256 * 256;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < nunits ? b0 + per : nunits;
    uint32_t key_all = 0;
    uint32_t nov = 0;   // overflowing elements (delayed scaling, COUNT_OVERFLOW)
    for (int64_t base = b0; base < b1; base += 256 * UNR) {
        Unit<HP> raw[UNR];
        // units past the run's end re-read its last unit (loads stay
        // unconditional); nothing of theirs is stored or counted
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            const int64_t u = base + k * 256 + t;
            raw[k].load(a.x, u < b1 ? u : b1 - 1);
        }
        // 1x128 tiles: the 16 lanes of a DPP row share a tile, so after the row
        // reduction every lane of row g holds the maxima of the row's UNR tiles
        // of this pass.  Rather than every lane working out the scale and
        // reciprocal of its tile for every unit (two IEEE divisions per 8
        // elements), lane k of each row works them out for unit k's tile, and
        // a DPP row broadcast hands them to the rest of the row: one pair of
        // divisions per lane per pass.
        float tsc[UNR], trc[UNR];
        if constexpr (SCHEME == kTileAxis0) {
            const int c = t & 15;
            uint32_t mine = 0;
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const uint32_t key = row16_max_u32(raw[k].key());
                if (k == c) mine = key;
            }
            const float sm = scale_from_amax<FMT>(__uint_as_float(mine));
            const float rm = 1.0f / sm;
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                tsc[k] = row_lane_bcast(sm, k);
                trc[k] = row_lane_bcast(rm, k);
            }
        }
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            const int64_t u = base + k * 256 + t;
            const bool valid = u < b1;
            float v[8];
            raw[k].unpack(v);
            float q[8];
            if constexpr (kPerTensor) {
                if constexpr (SCHEME == kPerTensorDelayed) {
                    const uint32_t key = raw[k].key();
                    key_all = valid && key > key_all ? key : key_all;
                }
                float d[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    d[e] = div_by_scale(v[e], s_pt, r_pt);
                    q[e] = saturate<FMT, SAT>(d[e]);
                }
                if (SCHEME == kPerTensorDelayed && a.count_overflow && valid) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) nov += overflowed<FMT>(v[e], d[e]);
                }
            } else if constexpr (SCHEME == kTileAxis0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) q[e] = saturate<FMT, SAT>(div_by_scale(v[e], tsc[k], trc[k]));
                if (valid && (t & 15) == 0) a.scales[u >> 4] = tsc[k];
            } else {   // kMxAxis0
                const uint32_t key = quad_max_u32(raw[k].key());
                const int code = e8m0_from_scale(scale_from_amax<FMT>(__uint_as_float(key)));
                const float inv = e8m0_recip(code);
#pragma unroll
                for (int e = 0; e < 8; ++e) q[e] = saturate<FMT, SAT>(v[e] * inv);
                if (valid && (t & 3) == 0) a.e8m0[u >> 2] = (uint8_t)code;
            }
            if (valid)
                reinterpret_cast<uint2*>(a.q)[u] = make_uint2(pack4<FMT>(q[0], q[1], q[2], q[3]),
                                                              pack4<FMT>(q[4], q[5], q[6], q[7]));
        }
    }

    if constexpr (SCHEME == kPerTensorCurrent) {
        if (blockIdx.x == 0 && t == 0) {
            *a.scale_out = s_pt;
            if (a.amax_out) *a.amax_out = amax_pt;
        }
    } else if constexpr (SCHEME == kPerTensorDelayed) {
        // as in the tiled kernel: the last block to finish folds the per-block
        // maxima and records the grid's amax in the history
        __shared__ uint32_t last, ov_sum;
        if (a.count_overflow) add_overflows(a.state, nov, &ov_sum);
        const uint32_t k = block_max_u32_256(key_all, red);
        if (t == 0) last = grid_done(a.keys, a.ctrs, k);
        __syncthreads();
        if (last) {
            const float amax = __uint_as_float(fold_keys_256(a.keys, gridDim.x, red));
            if (t == 0) {
                fp8q_delayed_state* st = a.state;
                const int pos = st->pos;
                st->amax_history[pos] = amax;
                st->pos = (pos + 1) % FP8Q_HISTORY_LEN;
                st->last_scale = s_pt;
                *a.scale_out = s_pt;
                if (a.amax_out) *a.amax_out = amax;
            }
        }
    }
}

// ------------------------------------------------------------------ launchers

static int tile_grid(int64_t ntiles) {
    const int64_t cap = 2048;
    return (int)(ntiles < cap ? ntiles : cap);
}

template <int HP, int FMT, int SCHEME>
static void launch_q3(const QuantArgs& a, int grid, int64_t ntr, int64_t ntc, int vin, int vq, int vqt, hipStream_t s) {
    if (a.saturate)
        hipLaunchKernelGGL((quantize_tiled_kernel<HP, FMT, SCHEME, true>), dim3(grid), dim3(256), 0, s, a, ntr, ntc, vin, vq, vqt);
    else
        hipLaunchKernelGGL((quantize_tiled_kernel<HP, FMT, SCHEME, false>), dim3(grid), dim3(256), 0, s, a, ntr, ntc, vin, vq, vqt);
}

template <int HP, int FMT>
static void launch_q2(const QuantArgs& a, int grid, int64_t ntr, int64_t ntc, int vin, int vq, int vqt, hipStream_t s) {
    switch (a.scheme) {
        case kPerTensorCurrent: launch_q3<HP, FMT, kPerTensorCurrent>(a, grid, ntr, ntc, vin, vq, vqt, s); break;
        case kPerTensorDelayed: launch_q3<HP, FMT, kPerTensorDelayed>(a, grid, ntr, ntc, vin, vq, vqt, s); break;
        case kTileAxis0: launch_q3<HP, FMT, kTileAxis0>(a, grid, ntr, ntc, vin, vq, vqt, s); break;
        case kTileAxis1: launch_q3<HP, FMT, kTileAxis1>(a, grid, ntr, ntc, vin, vq, vqt, s); break;
        case kBlock: launch_q3<HP, FMT, kBlock>(a, grid, ntr, ntc, vin, vq, vqt, s); break;
        case kMxAxis0: launch_q3<HP, FMT, kMxAxis0>(a, grid, ntr, ntc, vin, vq, vqt, s); break;
        default: launch_q3<HP, FMT, kMxAxis1>(a, grid, ntr, ntc, vin, vq, vqt, s); break;
    }
}

template <int HP, int FMT, int SCHEME>
static void launch_flat3(const QuantArgs& a, int64_t nunits, hipStream_t s) {
    const int64_t g = (nunits + 2047) / 2048;   // >= 8 units per thread
    const int grid = (int)(g < 1 ? 1 : (g > 2048 ? 2048 : g));
    if (a.saturate)
        hipLaunchKernelGGL((quantize_flat_kernel<HP, FMT, SCHEME, true>), dim3(grid), dim3(256), 0, s, a, nunits);
    else
        hipLaunchKernelGGL((quantize_flat_kernel<HP, FMT, SCHEME, false>), dim3(grid), dim3(256), 0, s, a, nunits);
}

template <int HP, int FMT>
static void launch_flat2(const QuantArgs& a, int64_t nunits, hipStream_t s) {
    switch (a.scheme) {
        case kPerTensorCurrent: launch_flat3<HP, FMT, kPerTensorCurrent>(a, nunits, s); break;
        case kPerTensorDelayed: launch_flat3<HP, FMT, kPerTensorDelayed>(a, nunits, s); break;
        case kTileAxis0: launch_flat3<HP, FMT, kTileAxis0>(a, nunits, s); break;
        default: launch_flat3<HP, FMT, kMxAxis0>(a, nunits, s); break;
    }
}

// The flat kernel serves row-direction schemes without a transposed copy when
// 8-element units are 16-byte aligned and never straddle a row, and rows hold
// whole 1x128 tiles (cols % 128 == 0) or MX blocks (cols % 32 == 0).
static bool flat_ok(const QuantArgs& a) {
    bool scheme = false;
    if (a.scheme == kPerTensorCurrent || a.scheme == kPerTensorDelayed) scheme = a.cols % 8 == 0;
    else if (a.scheme == kTileAxis0) scheme = a.cols % 128 == 0;
    else if (a.scheme == kMxAxis0) scheme = a.cols % 32 == 0;
    return scheme && a.qT == nullptr && a.q != nullptr && (uintptr_t)a.x % 16 == 0 && (uintptr_t)a.q % 8 == 0;
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
    if (flat_ok(a)) {
        const int64_t nunits = a.rows * a.cols / 8;
        if (a.hp == FP8Q_BF16) {
            if (a.fmt == FP8Q_E4M3) launch_flat2<FP8Q_BF16, FP8Q_E4M3>(a, nunits, s);
            else launch_flat2<FP8Q_BF16, FP8Q_E5M2>(a, nunits, s);
        } else {
            if (a.fmt == FP8Q_E4M3) launch_flat2<FP8Q_F32, FP8Q_E4M3>(a, nunits, s);
            else launch_flat2<FP8Q_F32, FP8Q_E5M2>(a, nunits, s);
        }
        return hipGetLastError();
    }
    const int64_t ntr = (a.rows + kTile - 1) / kTile, ntc = (a.cols + kTile - 1) / kTile;
    const int grid = tile_grid(ntr * ntc);
    const int esz = a.hp == FP8Q_BF16 ? 2 : 4;
    const int vin = ((uintptr_t)a.x % 16 == 0) && ((a.cols * esz) % 16 == 0);
    const int vq = a.q == nullptr || (((uintptr_t)a.q % 8 == 0) && (a.cols % 8 == 0));
    const int vqt = a.qT == nullptr || (((uintptr_t)a.qT % 16 == 0) && (a.rows % 16 == 0));
    if (a.hp == FP8Q_BF16) {
        if (a.fmt == FP8Q_E4M3) launch_q2<FP8Q_BF16, FP8Q_E4M3>(a, grid, ntr, ntc, vin, vq, vqt, s);
        else launch_q2<FP8Q_BF16, FP8Q_E5M2>(a, grid, ntr, ntc, vin, vq, vqt, s);
    } else {
        if (a.fmt == FP8Q_E4M3) launch_q2<FP8Q_F32, FP8Q_E4M3>(a, grid, ntr, ntc, vin, vq, vqt, s);
        else launch_q2<FP8Q_F32, FP8Q_E5M2>(a, grid, ntr, ntc, vin, vq, vqt, s);
    }
    return hipGetLastError();
}

// Zero n 32-bit words with plain vector stores: a kernel, not a memset, so
// that it can sit inside a captured graph.
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t s) {
    const int64_t g = (n + 255) / 256;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)(g < 1 ? 1 : g)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_transpose_u8(const uint8_t* in, int64_t rows, int64_t cols, uint8_t* out, hipStream_t s) {
    const int64_t ntr = (rows + kTile - 1) / kTile, ntc = (cols + kTile - 1) / kTile;
    const int vin = ((uintptr_t)in % 16 == 0) && (cols % 16 == 0);
    const int vout = ((uintptr_t)out % 16 == 0) && (rows % 16 == 0);
    hipLaunchKernelGGL(transpose_u8_kernel, dim3(tile_grid(ntr * ntc)), dim3(256), 0, s, in, rows, cols, out, ntr, ntc, vin, vout);
    return hipGetLastError();
}

}  // namespace fp8q
