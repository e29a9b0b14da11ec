// Block-scaled FP8 GEMM (1x128 activation / gradient tiles with 128x128
// weight blocks, or 1x128 tiles on both wgrad operands): persistent kernel.
// Every 128-K block gets its own partial product, which is scaled by
// sA(m, kb) * sB(n, kb) and added to fp32 accumulators.
//
// This file is compiled with MFMA results placed in VGPRs, where the FMAs
// that add each K block's partial can read them directly (the other GEMM
// kernels keep their accumulators in AGPRs).
//
// 1x128 row scales on A, and on B either 128x128 block scales (fprop / dgrad
// weights) or 1x128 row scales (wgrad operands); K a multiple of 512.  Each
// 16x16x128 MFMA covers exactly one 128-K block, so it runs with a zero
// accumulator and its result is added into the fp32 accumulators with one
// FMA per value: acc += (sA(m, kb) * sB(n, kb)) * partial.  Those FMAs need
// the accumulators in VGPRs, so a wave owns 128 x 64 outputs (128 VGPRs).
//  * Two waves per SIMD: eight waves over a 256 x 256 workgroup tile, two
//    64 KB stages loaded one K step ahead by direct-to-LDS loads, the last
//    step loading the next tile's first stage.  While one wave of a SIMD
//    waits for a partial or issues its FMAs, the other's MFMAs keep the
//    matrix core busy.  The first form, four waves of 128 x 64 (one per
//    SIMD) over 256 x 128 tiles with three 48 KB stages, kept the MFMA pipes
//    busy only 0.44 of the cycles, with about as many cycles per MFMA in
//    which neither the MFMA nor the VALU pipe was busy as cycles of MFMA;
//    this form ran 16% faster in the same call (wgrad 20%).
//  * Each tile is a buffer descriptor from its first row on (scalar
//    registers), so a lane's load offsets are fixed for the kernel and rows
//    past the matrix read as zeros; that keeps the waves within the 256
//    registers two waves per SIMD leave each.
//  * Row scales travel like the MX exponents: 16 bytes per row (four K
//    blocks) per direct-to-LDS load, one group of four K steps ahead, double
//    buffered.  With block-scaled B the 64 columns of a wave share one scale
//    per K block (one uniform load per step, a step ahead), so the FMA
//    factor is one product per fragment row and step.
//  * The FMAs of fragment row i run under the MFMAs of row i + 1.  The last
//    row's MFMAs (and the FMAs of the last two rows) run after the next
//    barrier, from registers, while the next step's fragments are read.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "gemm_common.h"
#include "launch.h"

namespace fp8q {

// bytes spanned by a fp32 scale array (rows >> rshift, ld, kstride) over nkb K blocks
__device__ __forceinline__ int64_t scale_bytes(const GemmScale& s, int64_t rows, int64_t nkb) {
    return ((((rows - 1) >> s.rshift) * s.ld + (nkb - 1) * s.kstride) + 1) * 4;
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, voff, 0, 0));
}

// Fragment reads with immediate offsets.  For fragment rows starting at a
// multiple of 16 the LDS chunk swizzle ((r / 2) % 8) depends on the lane's
// row l % 16 only, so fragment row r0 + 16 i of a stage sits at a per-lane
// offset fixed for the kernel (FragLane, for r0 = the wave's first row) plus
// 16 i rows: one address register per stage and operand half, and every
// read takes its row as the instruction's offset instead of an address add.
struct FragLane {
    uint32_t lo, hi;   // chunks g and g + 4 of row r0 + l % 16 (g = l / 16)
};
__device__ __forceinline__ FragLane frag_lane(int r0) {
    const int l = threadIdx.x & 63, r = r0 + (l & 15), g = l >> 4;
    return FragLane{(uint32_t)swz2(r, g), (uint32_t)swz2(r, g + 4)};
}
__device__ __forceinline__ v8i frag_at(const uint8_t* lo, const uint8_t* hi, int row16) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(lo + row16 * 16 * BK);
    const u32x4 b = *reinterpret_cast<const u32x4*>(hi + row16 * 16 * BK);
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

template <int FA, int FB, int OUT, bool BROW>
__global__ __launch_bounds__(512, 1) void gemm_bs_kernel(GemmArgs g, int ntm, int ntn) {
    constexpr int BNb = 256;
    constexpr int kStage = kTileBytes + BNb * BK;   // A 256 x 128 + B 256 x 128 bytes
    constexpr int kScA = BM * 16, kScGroup = kScA + (BROW ? BNb * 16 : 0);
    __shared__ __attribute__((aligned(1024))) uint8_t lds_all[2 * kStage + 2 * kScGroup];
    uint8_t* const lds_sc = lds_all + 2 * kStage;
    const int64_t M = g.M, N = g.N, K = g.K;
    const int t = threadIdx.x, l = t & 63, w = t >> 6;
    const int wm = (w >> 2) * 128, wn = (w & 3) * 64;
    const FragLane fa = frag_lane(wm), fb = frag_lane(wn);
    constexpr int kFmtA = FA == FP8Q_E4M3 ? 0 : 1;
    constexpr int kFmtB = FB == FP8Q_E4M3 ? 0 : 1;
    const int nt = ntm * ntn;
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8, per = gridDim.x / 8;
    const int lo = (int)((int64_t)nt * xcd / 8), hi = (int)((int64_t)nt * (xcd + 1) / 8);
    int logical = lo + slot;
    if (logical >= hi) return;
    const int nk = (int)(K / BK);
    const int ngroups = nk / 4;
    const int wave = __builtin_amdgcn_readfirstlane(w);
    const uint32_t K32 = (uint32_t)K;
    const __amdgpu_buffer_rsrc_t rsb = buffer_rsrc(g.sb.s, scale_bytes(g.sb, N, nk));
    const uint32_t lda4 = (uint32_t)(g.sa.ld * 4), ldb4 = (uint32_t)(g.sb.ld * 4);
    const uint32_t ksb4 = (uint32_t)(g.sb.kstride * 4);
    // the scale rows a wave stages: waves 0-3 A rows 64 (wave % 4) + lane;
    // waves 4-7 the same rows of B (row-scaled B) or of A again (the same
    // bytes to the same place), so every wave issues one load per group
    const bool gb = BROW && wave >= 4;
    const int sc_dst = (gb ? kScA : 0) + (wave & 3) * 64 * 16;
    // Offsets relative to the tile's first row, fixed for the kernel: a
    // wave loads rows 32 wave + l / 8 (+ 8 u) of both operand tiles, and its
    // scale row; the tile itself is a buffer descriptor over its first row
    // onwards (scalar registers), whose end turns rows past the matrix into zeros.
    const DmaB dl = dmab_rows(K, 32 * wave);
    const uint32_t sg_lane = (uint32_t)(64 * (wave & 3) + l) * (gb ? ldb4 : lda4);

    struct TileState {
        __amdgpu_buffer_rsrc_t ra, rb, rs;   // the tile's rows of A, of B, of the staged scales
        uint32_t sb_blk;                     // block-scaled B: the wave's B block scale for K block 0
    };
    auto tile_state = [&](int lg) {
        int tm, tn;
        tile_coords(lg, ntm, ntn, tm, tn);
        const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BNb;
        TileState s;
        s.ra = buffer_rsrc(g.A + m0 * K, (M - m0) * K);
        s.rb = buffer_rsrc(g.B + n0 * K, (N - n0) * K);
        s.rs = gb ? buffer_rsrc(reinterpret_cast<const float*>(g.sb.s) + n0 * g.sb.ld, scale_bytes(g.sb, N - n0, nk))
                  : buffer_rsrc(reinterpret_cast<const float*>(g.sa.s) + m0 * g.sa.ld, scale_bytes(g.sa, M - m0, nk));
        s.sb_blk = 0;
        if constexpr (!BROW) {
            const int64_t nb = (n0 + wn) >> 7, nb_last = (N - 1) >> 7;
            s.sb_blk = (uint32_t)(nb < nb_last ? nb : nb_last) * ldb4;
        }
        return s;
    };
    // load instruction u (0..7) of a stage: 4 of A rows, then 4 of B rows
    auto stage_load = [&](const TileState& s, uint32_t ko, uint8_t* dst, int u) {
        const uint32_t off = (((u & 1) ? dl.o : dl.e) + (uint32_t)((u & 3) * 8) * K32) + ko;
        if (u < 4) dma_one(s.ra, off, 0u, dst + (wave * 32 + u * 8) * BK);
        else dma_one(s.rb, off, 0u, dst + kTileBytes + (wave * 32 + (u - 4) * 8) * BK);
    };
    auto group_load = [&](const TileState& s, int buf, int gi) {
        dma_one(s.rs, sg_lane + (uint32_t)gi * 16, 0u, lds_sc + buf * kScGroup + sc_dst);
    };
    float sbn = 0.f;

    TileState cur = tile_state(logical);
#pragma unroll
    for (int u = 0; u < 8; ++u) stage_load(cur, 0u, lds_all, u);
    group_load(cur, 0, 0);
    if constexpr (!BROW) sbn = load_f32(rsb, cur.sb_blk);

    constexpr int NSB = BROW ? 16 : 1;
    v4f acc[8][4];
    v4f p[2][4];
    v8i b[4], a[2];
    float sf[8], sbr[NSB], sraw[8];
    int par = 0, gpar = 0;   // buffers (of 2) holding the tile's stage 0 / first scale group
    while (true) {
        const int next = logical + per;
        const bool has_next = next < hi;
        const TileState nxt = tile_state(has_next ? next : logical);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        auto mfma_one = [&](int i, int j) {
            p[i & 1][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                b[j], a[i & 1], v4f{0.f, 0.f, 0.f, 0.f}, kFmtB, kFmtA, 0, 0, 0, 0);
        };
        auto fma_one = [&](int i, int j) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[i][j][r] = __builtin_fmaf(p[i & 1][j][r], BROW ? sf[i] * sbr[4 * j + r] : sf[i], acc[i][j][r]);
        };
        // One K step: stage kt sits in buffer (par + kt) % 2; the step loads
        // stage kt + 1 (or the next tile's stage 0) into the other buffer,
        // which every wave finished reading before the barrier (a tile's
        // first step, with no rows of the previous step to run, issues the
        // loads at once).  With DEF the previous step's fragment row 7 is
        // still open: its MFMAs run first, straight after the barrier and
        // from registers only, while this step's fragments are read; its
        // FMAs follow under row 0's MFMAs.  Row i's FMAs run under row
        // i + 1's MFMAs, whose partial they do not touch; row i + 1's A
        // fragment is read into the registers row i - 1 used.  The
        // scheduling barriers keep this order (left free, the compiler put
        // each FMA group right behind the MFMA producing it).
        auto step = [&](auto def_c, int kt) {
            constexpr bool DEF = decltype(def_c)::value;
            // this stage, its scale group and the B block scale landed;
            // every wave is done with the buffer the loads below overwrite
            vm_wait<0>();
            stage_barrier();
            const bool last = kt + 1 == nk;
            const int gi = kt >> 2;
            if (last) group_load(nxt, (ngroups + gpar) & 1, 0);
            else if ((kt & 3) == 0 && gi + 1 < ngroups) group_load(cur, (gi + 1 + gpar) & 1, gi + 1);
            float sbc = 0.f;
            if constexpr (!BROW) {
                sbc = sbn;
                sbn = load_f32(rsb, last ? nxt.sb_blk : cur.sb_blk + (uint32_t)(kt + 1) * ksb4);
            }
            TileState ld;   // field by field: a selected reference would live in scratch memory
            ld.ra = last ? nxt.ra : cur.ra;
            ld.rb = last ? nxt.rb : cur.rb;
            const uint32_t ko = (uint32_t)(last ? 0 : kt + 1) * BK;
            const uint8_t* la = lds_all + ((par + kt) & 1) * kStage;
            const uint8_t* lb = la + kTileBytes;
            uint8_t* dst = lds_all + ((par + kt + 1) & 1) * kStage;
            const uint8_t* gs = lds_sc + ((gi + gpar) & 1) * kScGroup + 4 * (kt & 3);
            const uint8_t* alo = la + fa.lo;
            const uint8_t* ahi = la + fa.hi;
            const uint8_t* blo = lb + fb.lo;
            const uint8_t* bhi = lb + fb.hi;
            const uint8_t* gsa = gs + (wm + (l & 15)) * 16;
            const uint8_t* gsb = gs + kScA + (wn + 4 * (l >> 4)) * 16;

            // the next stage's eight loads, two under each of the first four
            // fragment rows the step runs (the previous step's row 7 - row
            // -1 here - then rows 0-2): issued later they landed too late for
            // the next step, all under row 7 they queued behind each other
            auto spread_load = [&](int i, int j) {
                if (DEF && i <= 2 && (j & 1)) stage_load(ld, ko, dst, 2 * (i + 1) + (j >> 1));
            };
            __builtin_amdgcn_sched_barrier(0);
            a[0] = frag_at(alo, ahi, 0);
            if constexpr (DEF) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    mfma_one(7, j);
                    b[j] = frag_at(blo, bhi, j);
                    spread_load(-1, j);
                    fma_one(6, j);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j] = frag_at(blo, bhi, j);
#pragma unroll
                for (int u = 0; u < 8; ++u) stage_load(ld, ko, dst, u);
            }
            a[1] = frag_at(alo, ahi, 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                mfma_one(0, j);
                spread_load(0, j);
                if constexpr (DEF) fma_one(7, j);
                __builtin_amdgcn_sched_barrier(0);
            }
            // row scales: rows 0 and 1 here, row i + 1 under row i's MFMAs
            // (a few live registers rather than all eight)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                sraw[i] = __uint_as_float(*reinterpret_cast<const uint32_t*>(gsa + 16 * i * 16));
            if constexpr (BROW) {
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    sbr[q] = __uint_as_float(*reinterpret_cast<const uint32_t*>(gsb + (16 * (q >> 2) + (q & 3)) * 16));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 1; i < 7; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    mfma_one(i, j);
                    if (j == 0) {
                        a[(i + 1) & 1] = frag_at(alo, ahi, i + 1);
                        sraw[i + 1] = __uint_as_float(*reinterpret_cast<const uint32_t*>(gsa + 16 * (i + 1) * 16));
                        sf[i - 1] = BROW ? sraw[i - 1] : sraw[i - 1] * sbc;
                    }
                    spread_load(i, j);
                    fma_one(i - 1, j);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int i = 6; i < 8; ++i) sf[i] = BROW ? sraw[i] : sraw[i] * sbc;
            lds_wait_all();
        };
        using T = std::true_type;
        using F = std::false_type;
        step(F{}, 0);
        for (int kt = 1; kt < nk; ++kt) step(T{}, kt);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            mfma_one(7, j);
            fma_one(6, j);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) fma_one(7, j);
        // every wave is done reading the last stage before it is reused
        stage_barrier();
        int tm, tn;
        tile_coords(logical, ntm, ntn, tm, tn);
        const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BNb;
        uint8_t* ep0 = lds_all + ((par + nk - 1) & 1) * kStage;
        if constexpr (OUT == FP8Q_BF16) {
            typedef float v2f_t __attribute__((ext_vector_type(2)));
            typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
            constexpr int kPitch = 144;   // 64 bf16 + 16 bytes
            uint8_t* ep = ep0 + w * (32 * kPitch);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
                for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const v4f v = acc[2 * qq + ii][j];
                        const v2bf_t p0 = __builtin_convertvector(v2f_t{v[0], v[1]}, v2bf_t);
                        const v2bf_t p1 = __builtin_convertvector(v2f_t{v[2], v[3]}, v2bf_t);
                        const int row = 16 * ii + (l & 15);
                        *reinterpret_cast<uint2*>(ep + row * kPitch + (16 * j + 4 * (l >> 4)) * 2) =
                            make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
                    }
                lds_wait_all();
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int row = 8 * u + (l >> 3), ch = l & 7;
                    const u32x4 d = *reinterpret_cast<const u32x4*>(ep + row * kPitch + ch * 16);
                    const int64_t m = m0 + wm + 32 * qq + row;
                    const int64_t n = n0 + wn + ch * 8;
                    if (m < M && n < N) __builtin_nontemporal_store(d, reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(g.C) + m * N + n));
                }
            }
        } else {
            constexpr int kPitch = 272;   // 64 fp32 + 16 bytes
            uint8_t* ep = ep0 + w * (16 * kPitch);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<v4f*>(ep + (l & 15) * kPitch + (16 * j + 4 * (l >> 4)) * 4) = acc[i][j];
                lds_wait_all();
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int row = 4 * u + (l >> 4), ch = l & 15;
                    const u32x4 d = *reinterpret_cast<const u32x4*>(ep + row * kPitch + ch * 16);
                    const int64_t m = m0 + wm + 16 * i + row;
                    const int64_t n = n0 + wn + ch * 4;
                    if (m < M && n < N) __builtin_nontemporal_store(d, reinterpret_cast<u32x4*>(reinterpret_cast<float*>(g.C) + m * N + n));
                }
            }
        }
        if (!has_next) break;
        logical = next;
        par = (par + nk) & 1;
        gpar = (ngroups + gpar) & 1;
        cur = nxt;
    }
    // the last step's extra loads land before the workgroup's LDS is released
    vm_wait<0>();
}

template <int FA, int FB, int OUT>
static void launch_out(const GemmArgs& g, hipStream_t s) {
    const int ntm = (int)((g.M + BM - 1) / BM), ntn = (int)((g.N + 255) / 256);
    if (g.sb.rshift == 0)
        hipLaunchKernelGGL((gemm_bs_kernel<FA, FB, OUT, true>), dim3(persistent_grid()), dim3(512), 0, s, g, ntm,
                           ntn);
    else
        hipLaunchKernelGGL((gemm_bs_kernel<FA, FB, OUT, false>), dim3(persistent_grid()), dim3(512), 0, s, g,
                           ntm, ntn);
}

template <int FA, int FB>
static void launch_fb(const GemmArgs& g, hipStream_t s) {
    if (g.c_dtype == FP8Q_BF16) launch_out<FA, FB, FP8Q_BF16>(g, s);
    else launch_out<FA, FB, FP8Q_F32>(g, s);
}

bool launch_gemm_block_persistent(const GemmArgs& g, hipStream_t s) {
    // direct-to-LDS operand loads: K a multiple of the 128-K step, at least
    // two steps, every lane offset below 2^32; row scales staged in groups of
    // four K blocks (16 bytes per row): K % 512 == 0, K-contiguous, 16-byte
    // aligned rows; B either row scales or 128x128 blocks
    auto rows16 = [](const GemmScale& sc) {
        return sc.rshift == 0 && sc.kstride == 1 && sc.ld % 4 == 0 && (uintptr_t)sc.s % 16 == 0;
    };
    const bool offsets32 = g.M * g.K < (int64_t(1) << 32) && g.N * g.K < (int64_t(1) << 32);
    const bool scales32 = g.M * (g.K / BK) < (int64_t(1) << 29) && g.N * (g.K / BK) < (int64_t(1) << 29);
    if (!(g.K % 512 == 0 && g.K >= 2 * BK && offsets32 && scales32 && rows16(g.sa))) return false;
    if (!(rows16(g.sb) || g.sb.rshift == 7)) return false;
    if (g.fa == FP8Q_E4M3) {
        if (g.fb == FP8Q_E4M3) launch_fb<FP8Q_E4M3, FP8Q_E4M3>(g, s);
        else launch_fb<FP8Q_E4M3, FP8Q_E5M2>(g, s);
    } else {
        if (g.fb == FP8Q_E4M3) launch_fb<FP8Q_E5M2, FP8Q_E4M3>(g, s);
        else launch_fb<FP8Q_E5M2, FP8Q_E5M2>(g, s);
    }
    return true;
}

}  // namespace fp8q
