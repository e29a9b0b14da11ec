// Scaled FP8 GEMM for gfx950: C[M,N] = sum_k A[m,k] B[n,k] with per-tensor,
// per-128-K-block (1x128 tiles / 128x128 blocks) or MX32 (E8M0 per 32 K)
// scales, fp32 accumulation on the CDNA4 FP8 matrix cores, fp32 or bf16 out.
//
// Follows the "fp8_parity.py" lab page, class FP8Matmul (the product of the
// two quantized operands, both scales applied to the fp32 result) and the blog post
// "How to Optimize Transformer-Based Models for Low-Precision Training"
// (fprop / dgrad / wgrad GEMMs of a layer; MXFP8 and 2D-block recipes).
//
// Design:
//  * Both operands arrive K-contiguous (codes [rows, K]); the dgrad / wgrad
//    layouts are brought to this form by the quantizer's transposed output
//    (or a transpose into the workspace) before the GEMM.
//  * Block tile 256 x 256, K step 128 (one 16x16x128 MFMA per 16x16 output
//    per K step).  4 waves in a 2 x 2 grid, each computing 128 x 128 with
//    8 x 8 MFMAs; 256 fp32 accumulators per lane (one wave per SIMD).
//  * The MFMA is issued with the B fragment as its first operand and the A
//    fragment as its second, so each lane ends up holding 4 consecutive
//    columns of one output row (8- or 16-byte stores in the epilogue).
//  * Operand tiles go global -> registers -> LDS (128 B rows, 16-byte chunks
//    XOR-swizzled by row so that fragment reads are bank-conflict free),
//    double-buffered: the next K step's global loads are in flight while the
//    current step's MFMAs run.
//  * Tile order is XCD-aware: workgroups are dealt round-robin to the 8 XCDs,
//    so consecutive logical tiles are remapped onto one XCD, and ordered in
//    groups of 8 M-tiles so that concurrently running tiles share A and B
//    panels in that XCD's L2.
//  * Block scaling: each 16x16x128 MFMA is one 128-K block, so its result is
//    scaled by sA(m,kb) * sB(n,kb) and accumulated with FMAs; the scales of
//    the tile's rows for the K block are staged in LDS with the operands.
//  * MX32: the E8M0 scales go straight into v_mfma_scale; lane l supplies the
//    scale of row l%16 for the 32-K block l/16 of the 128-K step.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BK = 128;
constexpr int kThreads = 256;
constexpr int kTileBytes = BM * BK;     // the A tile of one stage (B takes BN * BK)

enum ScaleMode : int { kSmPerTensor = 0, kSmBlock = 1, kSmMx = 2 };

// Logical tile of this workgroup: XCD-contiguous, then grouped by 8 M-tiles.
__device__ __forceinline__ void tile_of_block(int ntm, int ntn, int& tm, int& tn) {
    const int nb = gridDim.x, bid = blockIdx.x;
    const int full = (nb / 8) * 8;
    const int logical = bid < full ? (bid % 8) * (nb / 8) + bid / 8 : bid;
    constexpr int GM = 8;
    const int per_group = GM * ntn;
    const int group = logical / per_group;
    const int first_m = group * GM;
    const int gsize = ntm - first_m < GM ? ntm - first_m : GM;
    const int in_group = logical % per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// LDS byte offset of 16-byte chunk c (0..7) of tile row r.
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ (r & 7)) << 4); }

// Load this thread's NC chunks of an (NC * 32) x 128 operand tile (rows row0.., K from k0).
template <int NC>
__device__ __forceinline__ void gload_tile(const uint8_t* __restrict__ P, int64_t nrows, int64_t K,
                                           int64_t row0, int64_t k0, u32x4 st[NC]) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int id = threadIdx.x + kThreads * i;
        const int r = id >> 3, c = id & 7;
        const int64_t row = row0 + r, k = k0 + c * 16;
        if (row < nrows && k < K) st[i] = *reinterpret_cast<const u32x4*>(P + row * K + k);
        else st[i] = u32x4{0u, 0u, 0u, 0u};
    }
}

template <int NC>
__device__ __forceinline__ void swrite_tile(uint8_t* lds, const u32x4 st[NC]) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int id = threadIdx.x + kThreads * i;
        const int r = id >> 3, c = id & 7;
        *reinterpret_cast<u32x4*>(lds + swz(r, c)) = st[i];
    }
}

// MFMA fragment of 16 tile rows starting at r0: lane l takes row r0 + l%16 and
// K bytes [16g, 16g+16) and [64+16g, 64+16g+16), g = l/16 (the 8-bit operand
// layout of the 16x16x128 MFMA).
__device__ __forceinline__ v8i frag(const uint8_t* lds, int r0) {
    const int l = threadIdx.x & 63;
    const int r = r0 + (l & 15), g = l >> 4;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(lds + swz(r, g));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(lds + swz(r, g + 4));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Scale of operand row `row` for 128-K block kb (fp32 scale modes).
__device__ __forceinline__ float row_scale(const GemmScale& s, int64_t row, int64_t kb) {
    const float* p = reinterpret_cast<const float*>(s.s);
    if (s.gran == FP8Q_PER_TENSOR) return p[0];
    return p[(row >> s.rshift) * s.ld + kb * s.kstride];
}

// BN is 256 (waves of 128 x 128) or 128 (waves of 128 x 64, used by the
// block-scaled mode whose accumulators must live in VGPRs for the FMAs).
template <int FA, int FB, int OUT, int SM, int BN>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmArgs g, int ntm, int ntn) {
    constexpr int NJ = BN / 32;                 // 16-column MFMA tiles per wave
    constexpr int NCB = BN / 32;                // B chunks per thread per stage
    __shared__ __attribute__((aligned(16))) uint8_t lds_ab[2][kTileBytes + BN * BK];
    __shared__ float lds_sc[2][BM + BN];        // block-scale mode: row scales of the K block
    __shared__ uint32_t lds_mx[2][BM + BN];     // MX mode: 4 E8M0 bytes (the 128-K step) per row

    int tm, tn;
    tile_of_block(ntm, ntn, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t M = g.M, N = g.N, K = g.K;
    const int t = threadIdx.x, l = t & 63, w = t >> 6;
    const int wm = (w >> 1) * 128, wn = (w & 1) * (BN / 2);
    constexpr int kFmtA = FA == FP8Q_E4M3 ? 0 : 1;
    constexpr int kFmtB = FB == FP8Q_E4M3 ? 0 : 1;

    v4f acc[8][NJ];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nk = (int)((K + BK - 1) / BK);
    u32x4 sta[8], stb[NCB];
    float sca = 0.f;
    uint32_t mxa = 0;   // staged scale of row t of A (t < 256) / of B (same thread)
    float scb = 0.f;
    uint32_t mxb = 0;

    auto load_scales = [&](int kt) {
        if constexpr (SM == kSmBlock) {
            const int64_t ra = m0 + t, rb = n0 + t;
            sca = ra < M ? row_scale(g.sa, ra, kt) : 0.f;
            scb = (t < BN && rb < N) ? row_scale(g.sb, rb, kt) : 0.f;
        } else if constexpr (SM == kSmMx) {
            // 4 E8M0 bytes of the 32-K blocks 4kt..4kt+3; blocks past K get 127 (2^0)
            const int64_t ra = m0 + t, rb = n0 + t;
            const int64_t nkb = K / 32;
            uint32_t va = 0x7f7f7f7fu, vb = 0x7f7f7f7fu;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int64_t kb = (int64_t)kt * 4 + b;
                if (kb < nkb) {
                    const uint32_t ea = ra < M ? reinterpret_cast<const uint8_t*>(g.sa.s)[ra * g.sa.ld + kb] : 127u;
                    const uint32_t eb = (t < BN && rb < N) ? reinterpret_cast<const uint8_t*>(g.sb.s)[rb * g.sb.ld + kb] : 127u;
                    va = (va & ~(0xffu << (8 * b))) | (ea << (8 * b));
                    vb = (vb & ~(0xffu << (8 * b))) | (eb << (8 * b));
                }
            }
            mxa = va;
            mxb = vb;
        }
    };
    auto store_scales = [&](int buf) {
        if constexpr (SM == kSmBlock) {
            lds_sc[buf][t] = sca;
            if (t < BN) lds_sc[buf][BM + t] = scb;
        } else if constexpr (SM == kSmMx) {
            lds_mx[buf][t] = mxa;
            if (t < BN) lds_mx[buf][BM + t] = mxb;
        }
    };

    // prologue: K step 0 into buffer 0
    gload_tile<8>(g.A, M, K, m0, 0, sta);
    gload_tile<NCB>(g.B, N, K, n0, 0, stb);
    load_scales(0);
    swrite_tile<8>(lds_ab[0], sta);
    swrite_tile<NCB>(lds_ab[0] + kTileBytes, stb);
    store_scales(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            gload_tile<8>(g.A, M, K, m0, (int64_t)(kt + 1) * BK, sta);
            gload_tile<NCB>(g.B, N, K, n0, (int64_t)(kt + 1) * BK, stb);
            load_scales(kt + 1);
        }
        const uint8_t* la = lds_ab[cur];
        const uint8_t* lb = lds_ab[cur] + kTileBytes;
        v8i bf[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) bf[j] = frag(lb, wn + 16 * j);

        if constexpr (SM == kSmPerTensor) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const v8i af = frag(la, wm + 16 * i);
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], kFmtB, kFmtA,
                                                                                 0, 0, 0, 0);
            }
        } else if constexpr (SM == kSmBlock) {
            // scales of this lane's 4 columns for each j, and of its row for each i
            float sbv[NJ][4];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float4 v = *reinterpret_cast<const float4*>(&lds_sc[cur][BM + wn + 16 * j + 4 * (l >> 4)]);
                sbv[j][0] = v.x; sbv[j][1] = v.y; sbv[j][2] = v.z; sbv[j][3] = v.w;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const v8i af = frag(la, wm + 16 * i);
                const float sai = lds_sc[cur][wm + 16 * i + (l & 15)];
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, v4f{0.f, 0.f, 0.f, 0.f},
                                                                                  kFmtB, kFmtA, 0, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], sai * sbv[j][r], acc[i][j][r]);
                }
            }
        } else {   // kSmMx
            const int kb = l >> 4;   // 32-K block of the step this lane's scale describes
            int sbs[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) sbs[j] = (int)((lds_mx[cur][BM + wn + 16 * j + (l & 15)] >> (8 * kb)) & 0xffu);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const v8i af = frag(la, wm + 16 * i);
                const int sas = (int)((lds_mx[cur][wm + 16 * i + (l & 15)] >> (8 * kb)) & 0xffu);
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], kFmtB, kFmtA,
                                                                                 0, sbs[j], 0, sas);
            }
        }

        if (more) {
            swrite_tile<8>(lds_ab[cur ^ 1], sta);
            swrite_tile<NCB>(lds_ab[cur ^ 1] + kTileBytes, stb);
            store_scales(cur ^ 1);
        }
        __syncthreads();
    }

    // epilogue: per-tensor scales, then store
    float S = 1.0f;
    if constexpr (SM == kSmPerTensor)
        S = reinterpret_cast<const float*>(g.sa.s)[0] * reinterpret_cast<const float*>(g.sb.s)[0];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t m = m0 + wm + 16 * i + (l & 15);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t n = n0 + wn + 16 * j + 4 * (l >> 4);
            if (n >= N) continue;
            const v4f v = acc[i][j] * S;
            if constexpr (OUT == FP8Q_BF16) {
                const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
                const uint32_t hi = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(g.C) + m * N + n) = make_uint2(lo, hi);
            } else {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(g.C) + m * N + n) = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

// ------------------------------------------------------------------ per-tensor fast path
//
// Per-tensor scales, K a multiple of 128 and every operand offset below 2^32:
// the same 256 x 256 x 128 tiling, but operand tiles go straight from global
// memory into LDS (global_load_lds, no register staging), and the LDS reads
// and waits are ordered by hand so that every wait covers reads issued at
// least one MFMA group earlier.

// Swizzle of the 16-byte chunks of a 128-byte LDS row: chunk c of row r sits
// at c ^ ((r / 2) % 8).  A fragment read serves 16 consecutive rows at one
// logical chunk per phase; the XOR spreads them over 8 chunk positions x 2
// row parities, i.e. over all 64 banks.
__device__ __forceinline__ int swz2(int r, int c) { return r * BK + ((c ^ ((r >> 1) & 7)) << 4); }

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at their maxima): every LDS
// read issued so far has landed.
__device__ __forceinline__ void lds_wait_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier for the staged pipeline.  Each wave has already waited
// for its own loads of the stage about to be read (vm_wait) and for its own
// LDS reads of the stage about to be overwritten (lds_wait_all), so only the
// execution barrier is needed; __syncthreads() would add a full vmcnt(0)
// wait.  The empty asm keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void stage_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) with lgkmcnt and expcnt at their maxima (vmcnt is six
// bits: [3:0] and [15:14] of the immediate); N < 64.
template <int N>
__device__ __forceinline__ void vm_wait() { __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14)); }

__device__ __forceinline__ v8i frag2(const uint8_t* lds, int r0) {
    const int l = threadIdx.x & 63;
    const int r = r0 + (l & 15), g = l >> 4;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(lds + swz2(r, g));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(lds + swz2(r, g + 4));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Direct global -> LDS loads of one 256 x 128 operand tile: wave w brings rows
// [64w, 64w+64) in 8 instructions of 8 rows.  The hardware writes lane l's 16
// bytes at the instruction's LDS base + 16 l, i.e. row l/8, physical chunk
// l%8 of the 8-row group; the lane therefore fetches the logical chunk that
// the swizzle places there.  Rows past the matrix edge re-read the last row
// (their products only reach outputs that are never stored).  The per-lane
// offsets are computed once per tile; a step moves the base pointer by its K
// offset, and the LDS destination (M0) is scalar arithmetic on the wave index.
struct Dma2 {
    uint32_t off[8];
};

__device__ __forceinline__ Dma2 dma2_plan(int64_t nrows, int64_t K, int64_t row0, int wave) {
    const int l = threadIdx.x & 63;
    Dma2 d;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int r = wave * 64 + u * 8 + (l >> 3);
        const int c = (l & 7) ^ ((r >> 1) & 7);
        int64_t row = row0 + r;
        row = row < nrows ? row : nrows - 1;
        d.off[u] = (uint32_t)(row * K + c * 16);
    }
    return d;
}

__device__ __forceinline__ void dload_tile(const uint8_t* __restrict__ base, const Dma2& d, uint8_t* lds, int wave) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
        __builtin_amdgcn_global_load_lds(base + d.off[u],
                                         (__attribute__((address_space(3))) void*)(lds + (wave * 64 + u * 8) * BK),
                                         16, 0, 0);
}

template <int FA, int FB, int OUT>
__global__ __launch_bounds__(kThreads, 1) void gemm_pt_kernel(GemmArgs g, int ntm, int ntn) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_ab[2][2 * kTileBytes];
    int tm, tn;
    tile_of_block(ntm, ntn, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * 256;
    const int64_t M = g.M, N = g.N, K = g.K;
    const int t = threadIdx.x, l = t & 63, w = t >> 6;
    const int wm = (w >> 1) * 128, wn = (w & 1) * 128;
    constexpr int kFmtA = FA == FP8Q_E4M3 ? 0 : 1;
    constexpr int kFmtB = FB == FP8Q_E4M3 ? 0 : 1;

    v4f acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nk = (int)(K / BK);
    const int wave = __builtin_amdgcn_readfirstlane(w);
    const Dma2 da = dma2_plan(M, K, m0, wave), db = dma2_plan(N, K, n0, wave);
    dload_tile(g.A, da, lds_ab[0], wave);
    dload_tile(g.B, db, lds_ab[0] + kTileBytes, wave);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            dload_tile(g.A + (int64_t)(kt + 1) * BK, da, lds_ab[cur ^ 1], wave);
            dload_tile(g.B + (int64_t)(kt + 1) * BK, db, lds_ab[cur ^ 1] + kTileBytes, wave);
        }
        const uint8_t* la = lds_ab[cur];
        const uint8_t* lb = lds_ab[cur] + kTileBytes;
        // The first 2 x 8 MFMA row pair runs in 2 x 2 blocks while the B
        // fragments stream in; each later row pair's A fragments are fetched
        // one row pair ahead.  sched_barrier pins this program order.
        v8i bf[8];
        v8i af[2][2];
        af[0][0] = frag2(la, wm);
        af[0][1] = frag2(la, wm + 16);
        bf[0] = frag2(lb, wn);
        bf[1] = frag2(lb, wn + 16);
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            lds_wait_all();
            if (jb < 3) {
                bf[2 * jb + 2] = frag2(lb, wn + 16 * (2 * jb + 2));
                bf[2 * jb + 3] = frag2(lb, wn + 16 * (2 * jb + 3));
            } else {
                af[1][0] = frag2(la, wm + 32);
                af[1][1] = frag2(la, wm + 48);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int j = 2 * jb + jj;
                    acc[ii][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[0][ii], acc[ii][j], kFmtB,
                                                                                  kFmtA, 0, 0, 0, 0);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int p = 1; p < 4; ++p) {
            lds_wait_all();
            if (p < 3) {
                af[(p + 1) & 1][0] = frag2(la, wm + 32 * (p + 1));
                af[(p + 1) & 1][1] = frag2(la, wm + 32 * (p + 1) + 16);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[2 * p + ii][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        bf[j], af[p & 1][ii], acc[2 * p + ii][j], kFmtB, kFmtA, 0, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // this wave has read all of the current stage and its loads of the
        // next stage have landed; after the barrier the same holds for all
        lds_wait_all();
        vm_wait<0>();
        stage_barrier();
    }

    const float S = reinterpret_cast<const float*>(g.sa.s)[0] * reinterpret_cast<const float*>(g.sb.s)[0];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t m = m0 + wm + 16 * i + (l & 15);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t n = n0 + wn + 16 * j + 4 * (l >> 4);
            if (n >= N) continue;
            const v4f v = acc[i][j] * S;
            if constexpr (OUT == FP8Q_BF16) {
                const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
                const uint32_t hi = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(g.C) + m * N + n) = make_uint2(lo, hi);
            } else {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(g.C) + m * N + n) = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

template <int FA, int FB, int OUT>
static void launch_sm(const GemmArgs& g, int sm, hipStream_t s) {
    const int ntm = (int)((g.M + BM - 1) / BM);
    if (sm == kSmBlock) {
        const int ntn = (int)((g.N + 127) / 128);
        hipLaunchKernelGGL((gemm_kernel<FA, FB, OUT, kSmBlock, 128>), dim3(ntm * ntn), dim3(kThreads), 0, s, g, ntm, ntn);
        return;
    }
    const int ntn = (int)((g.N + 255) / 256);
    const bool offsets32 = g.M * g.K <= (int64_t(1) << 32) && g.N * g.K <= (int64_t(1) << 32);
    if (sm == kSmPerTensor && g.K % BK == 0 && offsets32)
        hipLaunchKernelGGL((gemm_pt_kernel<FA, FB, OUT>), dim3(ntm * ntn), dim3(kThreads), 0, s, g, ntm, ntn);
    else if (sm == kSmPerTensor)
        hipLaunchKernelGGL((gemm_kernel<FA, FB, OUT, kSmPerTensor, 256>), dim3(ntm * ntn), dim3(kThreads), 0, s, g, ntm, ntn);
    else
        hipLaunchKernelGGL((gemm_kernel<FA, FB, OUT, kSmMx, 256>), dim3(ntm * ntn), dim3(kThreads), 0, s, g, ntm, ntn);
}

template <int FA, int FB>
static void launch_out(const GemmArgs& g, int sm, hipStream_t s) {
    if (g.c_dtype == FP8Q_BF16) launch_sm<FA, FB, FP8Q_BF16>(g, sm, s);
    else launch_sm<FA, FB, FP8Q_F32>(g, sm, s);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
    int sm = kSmPerTensor;
    if (g.sa.gran == FP8Q_MX32) sm = kSmMx;
    else if (g.sa.gran != FP8Q_PER_TENSOR || g.sb.gran != FP8Q_PER_TENSOR) sm = kSmBlock;
    if (g.fa == FP8Q_E4M3) {
        if (g.fb == FP8Q_E4M3) launch_out<FP8Q_E4M3, FP8Q_E4M3>(g, sm, s);
        else launch_out<FP8Q_E4M3, FP8Q_E5M2>(g, sm, s);
    } else {
        if (g.fb == FP8Q_E4M3) launch_out<FP8Q_E5M2, FP8Q_E4M3>(g, sm, s);
        else launch_out<FP8Q_E5M2, FP8Q_E5M2>(g, sm, s);
    }
    return hipGetLastError();
}

}  // namespace fp8q
