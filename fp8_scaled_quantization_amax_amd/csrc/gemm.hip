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

#include <type_traits>

#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace fp8q {


// kSmRow: one scale per operand row (rowwise recipe; a per-tensor operand
// broadcasts its scale), applied in the epilogue as acc * (sA[m] * sB[n]).
enum ScaleMode : int { kSmPerTensor = 0, kSmBlock = 1, kSmMx = 2, kSmRow = 3 };

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

        if constexpr (SM == kSmPerTensor || SM == kSmRow) {
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
            v4f v = acc[i][j] * S;
            if constexpr (SM == kSmRow) {
                const float sam = row_scale(g.sa, m, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = acc[i][j][r] * (sam * row_scale(g.sb, n + r, 0));
            }
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
// Per-tensor scales, K a multiple of 128 and at least 256, every operand
// offset below 2^32: a persistent kernel with the same 256 x 256 x 128 tile.
//  * One workgroup per CU slot.  Workgroups are dealt round-robin to the 8
//    XCDs; each XCD takes a contiguous range of logical tiles (grouped by 8
//    M-tiles), and its workgroups walk that range together, so the tiles that
//    run at the same time on one XCD share A and B panels in its L2.
//  * Operand tiles go straight from global memory into LDS
//    (global_load_lds_dwordx4, no register staging), two stages.  The 16 loads
//    of a wave for the next stage are spread one per two MFMAs over the first
//    half of each K step; the last K step of a tile loads the first stage of
//    the workgroup's next tile, so the epilogue overlaps those loads.
//  * Each K step starts right after the barrier with the previous step's
//    last row pair (registers only), column by column, and reads each B
//    fragment of the new step into the registers its predecessor just left;
//    the new step's first row pair then waits only for the fragment it needs
//    (partial lgkmcnt waits: LDS reads of one wave complete in order).
//  * Epilogue: results are scaled (bf16: rounded by the hardware convert,
//    round to nearest even, NaN stays NaN), staged through the LDS stage
//    buffer the last step read, and stored as 16-byte row-contiguous pieces,
//    so each store instruction writes whole cache lines.  The stores carry
//    the non-temporal hint: the output is not read again here, and keeping it
//    out of the way leaves L2 to the operand panels (+2.7% measured; the same
//    hint on the operand loads cost 16%, since those panels are shared by the
//    tiles running on an XCD).

// s_waitcnt lgkmcnt(n) (vmcnt, expcnt at their maxima) for an n that is a
// compile-time constant after unrolling; n above 15 waits for 15, which is
// at least as strong since LDS reads complete in order.
__device__ __forceinline__ void lgkm_wait(int n) {
    switch (n < 15 ? n : 15) {
        case 0: __builtin_amdgcn_s_waitcnt(0xC07F); break;
        case 1: __builtin_amdgcn_s_waitcnt(0xC17F); break;
        case 2: __builtin_amdgcn_s_waitcnt(0xC27F); break;
        case 3: __builtin_amdgcn_s_waitcnt(0xC37F); break;
        case 4: __builtin_amdgcn_s_waitcnt(0xC47F); break;
        case 5: __builtin_amdgcn_s_waitcnt(0xC57F); break;
        case 6: __builtin_amdgcn_s_waitcnt(0xC67F); break;
        case 7: __builtin_amdgcn_s_waitcnt(0xC77F); break;
        case 8: __builtin_amdgcn_s_waitcnt(0xC87F); break;
        case 9: __builtin_amdgcn_s_waitcnt(0xC97F); break;
        case 10: __builtin_amdgcn_s_waitcnt(0xCA7F); break;
        case 11: __builtin_amdgcn_s_waitcnt(0xCB7F); break;
        case 12: __builtin_amdgcn_s_waitcnt(0xCC7F); break;
        case 13: __builtin_amdgcn_s_waitcnt(0xCD7F); break;
        case 14: __builtin_amdgcn_s_waitcnt(0xCE7F); break;
        default: __builtin_amdgcn_s_waitcnt(0xCF7F); break;
    }
}

constexpr int kEpPitch = 272;     // bytes per staged bf16 row of 128 values (+16: conflict-free)
constexpr int kEpPitch32 = 528;   // bytes per staged fp32 row of 128 values (+16)

// MX (SM == kSmMx, K % 512 == 0): the E8M0 scales travel to LDS in groups of
// four K steps: for each tile row, 16 bytes = its four 32-K blocks of four
// consecutive K steps, one 16-byte direct-to-LDS load per lane (64 rows per
// instruction), double-buffered by group and loaded one group ahead.  Under
// the MFMAs of a step's rows 4, 5 every lane reads the byte of its fragment
// rows and 32-K block for all 16 fragments of the next step (a tile's first
// step reads its own at its start), and the MFMAs take them as their scale
// operands.  The scales of the row pair that runs after the barrier are kept
// from the previous step; the bytes change registers just before the
// barrier.
template <int FA, int FB, int OUT, int SM>
__global__ __launch_bounds__(kThreads, 1) void gemm_pt_kernel(GemmArgs g, int ntm, int ntn) {
    constexpr bool MX = SM == kSmMx;
    // One LDS allocation with the operand stages at offset 0 and the MX scale
    // groups after them (with the compiler free to place a separate scale
    // array first, the same kernel ran about 3x slower).
    constexpr int kScaleGroupBytes = 2 * 256 * 16;
    __shared__ __attribute__((aligned(1024))) uint8_t lds_all[2 * 2 * kTileBytes + (MX ? 2 * kScaleGroupBytes : 0)];
    uint8_t(*lds_ab)[2 * kTileBytes] = reinterpret_cast<uint8_t(*)[2 * kTileBytes]>(lds_all);
    uint8_t(*lds_sc)[kScaleGroupBytes] = reinterpret_cast<uint8_t(*)[kScaleGroupBytes]>(lds_all + 2 * 2 * kTileBytes);
    const int64_t M = g.M, N = g.N, K = g.K;
    const int t = threadIdx.x, l = t & 63, w = t >> 6;
    const int wm = (w >> 1) * 128, wn = (w & 1) * 128;
    constexpr int kFmtA = FA == FP8Q_E4M3 ? 0 : 1;
    constexpr int kFmtB = FB == FP8Q_E4M3 ? 0 : 1;
    const int nt = ntm * ntn;
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8, per = gridDim.x / 8;
    const int lo = (int)((int64_t)nt * xcd / 8), hi = (int)((int64_t)nt * (xcd + 1) / 8);
    int logical = lo + slot;
    if (logical >= hi) return;
    const int nk = (int)(K / BK);
    const int wave = __builtin_amdgcn_readfirstlane(w);
    int tm, tn;
    tile_coords(logical, ntm, ntn, tm, tn);
    const uint32_t K32 = (uint32_t)K;
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(g.A, M * K), rb = buffer_rsrc(g.B, N * K);
    DmaB da = dmab_plan(K, (int64_t)tm * BM, wave), db = dmab_plan(K, (int64_t)tn * 256, wave);
    // instruction u of a tile's loads at K offset ko (both in the lane offset,
    // so the bounds check covers them)
    auto tile_load = [&](const __amdgpu_buffer_rsrc_t& rs, const DmaB& p, uint32_t ko, uint8_t* dst, int u) {
        dma_one(rs, ((u & 1) ? p.o : p.e) + (uint32_t)(u * 8) * K32 + ko, 0u, dst + (wave * 64 + u * 8) * BK);
    };
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        tile_load(ra, da, 0u, lds_ab[0], u);
        tile_load(rb, db, 0u, lds_ab[0] + kTileBytes, u);
    }
    // MX scale rows of this wave's loads: rows 64 * wave + lane of the A and B
    // tiles (rows past the edge read as zeros, like the operands)
    const uint32_t sld = (uint32_t)(K / 32);   // bytes per scale row
    auto srow = [&](int64_t row0) { return (uint32_t)((row0 + wave * 64 + l) * sld); };
    uint32_t sa_off = 0, sb_off = 0, nsa_off = 0, nsb_off = 0;
    // (per-tensor mode: descriptors over the scalar scales, never used)
    const __amdgpu_buffer_rsrc_t rsa = buffer_rsrc(g.sa.s, MX ? M * (K / 32) : 4);
    const __amdgpu_buffer_rsrc_t rsb = buffer_rsrc(g.sb.s, MX ? N * (K / 32) : 4);
    const int ngroups = (nk + 3) / 4;   // MX scale groups of four K steps
    int gpar = 0;                       // group gi of the current tile lives in scale buffer (gi + gpar) % 2
    // 16-byte loads of scale group gi of this wave's A and B rows into buffer `buf`
    auto load_group = [&](int buf, uint32_t aoff, uint32_t boff, int gi) {
        uint8_t* st = lds_sc[buf];
        dma_one(rsa, aoff + (uint32_t)gi * 16, 0u, st + wave * 64 * 16);
        dma_one(rsb, boff + (uint32_t)gi * 16, 0u, st + 4096 + wave * 64 * 16);
    };
    if constexpr (MX) {
        sa_off = srow((int64_t)tm * BM);
        sb_off = srow((int64_t)tn * 256);
        load_group(0, sa_off, sb_off, 0);
    }
    const float S = MX ? 1.0f : reinterpret_cast<const float*>(g.sa.s)[0] * reinterpret_cast<const float*>(g.sb.s)[0];
    // kSmRow: this lane's scales of its 8 output rows (16 i + l % 16 of the
    // wave's rows) and 32 output columns (16 j + 4 (l / 16) + r), loaded at
    // the start of each tile so that they have landed by its epilogue
    constexpr bool ROW = SM == kSmRow;
    constexpr int kRowRegs = ROW ? 8 : 1;
    float rwa[kRowRegs];
    float rwb[kRowRegs][4];
    auto load_row_scales = [&](int tm_, int tn_) {
        if constexpr (ROW) {
            const float* pa = reinterpret_cast<const float*>(g.sa.s);
            const float* pb = reinterpret_cast<const float*>(g.sb.s);
            const bool ta = g.sa.gran == FP8Q_PER_TENSOR, tb = g.sb.gran == FP8Q_PER_TENSOR;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t m = (int64_t)tm_ * BM + wm + 16 * i + (l & 15);
                rwa[i] = pa[ta ? 0 : (m < M ? m : M - 1)];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t n = (int64_t)tn_ * 256 + wn + 16 * j + 4 * (l >> 4) + r;
                    rwb[j][r] = pb[tb ? 0 : (n < N ? n : N - 1)];
                }
        }
    };
    // acc[i][j] with its scales applied
    auto scaled = [&](const v4f& a, int i, int j) -> v4f {
        if constexpr (ROW) {
            return v4f{a[0] * (rwa[i] * rwb[j][0]), a[1] * (rwa[i] * rwb[j][1]), a[2] * (rwa[i] * rwb[j][2]),
                       a[3] * (rwa[i] * rwb[j][3])};
        } else {
            return a * S;
        }
    };

    v4f acc[8][8];
    v8i b[8];
    v8i ax[2], ay[2];
    DmaB na{0u, 0u}, nb{0u, 0u};
    int sa[8], sb[8];         // MX: this step's E8M0 bytes for A rows 16i.. and B rows 16j..
    int sa_o[2], sb_o[8];     // MX: the previous step's, for its rows 6, 7
    int sa_n[8], sb_n[8];     // MX: the next step's, read during this one
#pragma unroll
    for (int i = 0; i < 8; ++i) sa[i] = sb[i] = sb_o[i] = sa_n[i] = sb_n[i] = 127;
    sa_o[0] = sa_o[1] = 127;

    // MFMA of A fragment row i, B fragment column j; sbv / sav are the E8M0
    // scale bytes (MX) of the B and A rows of this lane
    auto mfma_s = [&](int i, const v8i& bb, const v8i& a, int j, int sbv, int sav) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bb, a, acc[i][j], kFmtB, kFmtA, 0, sbv, 0, sav);
    };
    auto mfma = [&](int i, const v8i& bb, const v8i& a, int j) {
        if constexpr (MX) mfma_s(i, bb, a, j, sb[j], sa[i]);
        else mfma_s(i, bb, a, j, 0, 0);
    };
    // Stage kt of the current tile lives in buffer (kt + par) % 2.  Load slot
    // u (0..15) of a wave: MODE 1 = stage kt+1 of this tile, MODE 2 = stage 0
    // of the next tile; both go to the buffer the current step does not read.
    int par = 0;
    // K direction of the current tile (non-MX modes): consecutive tiles of a
    // workgroup walk K forward and backward in turn.  The tiles an XCD runs
    // at the same time move on together to tiles over the same A panels, so
    // a tile that starts where the previous ones ended finds those K blocks
    // of the panels still in L2.  (MX keeps the forward walk: its scale
    // groups follow K.)
    int rev = 0;
    auto kblock = [&](int r, int kt) { return (uint32_t)(r ? nk - 1 - kt : kt) * BK; };
    auto dma = [&](auto mode_c, int kt, int u) {
        constexpr int MODE = decltype(mode_c)::value;
        const uint32_t ko = MODE == 1 ? kblock(rev, kt + 1) : kblock(MX ? 0 : rev ^ 1, 0);
        uint8_t* dst = lds_ab[(kt + 1 + par) & 1];
        if (u < 8) {
            tile_load(ra, MODE == 1 ? da : na, ko, dst, u);
        } else if (u < 16) {
            tile_load(rb, MODE == 1 ? db : nb, ko, dst + kTileBytes, u - 8);
        } else if constexpr (MX) {   // u = 16: the next scale group of this tile, or the next tile's first
            if (MODE == 1) {
                if (kt % 4 == 0 && kt / 4 + 1 < ngroups) load_group((kt / 4 + 1 + gpar) & 1, sa_off, sb_off, kt / 4 + 1);
            } else {
                load_group(((nk - 1) / 4 + 1 + gpar) & 1, nsa_off, nsb_off, 0);
            }
        }
    };

    // MX: this lane's E8M0 bytes of K step kt (its 32-K block l/16) for the
    // 8 A and 8 B fragment rows; one base per operand, row i 256 bytes on
    auto read_scales = [&](int kt, int (&ra_)[8], int (&rb_)[8]) {
        const uint8_t* grp = lds_sc[(kt / 4 + gpar) & 1] + 4 * (kt % 4) + (l >> 4);
        const uint8_t* spa = grp + (wm + (l & 15)) * 16;
        const uint8_t* spb = grp + 4096 + (wn + (l & 15)) * 16;
#pragma unroll
        for (int i = 0; i < 8; ++i) ra_[i] = spa[256 * i];
#pragma unroll
        for (int j = 0; j < 8; ++j) rb_[j] = spb[256 * j];
    };
    // Half-fragment read: h = 0 brings K bytes [16g, 16g+16) of the lane's
    // row, h = 1 bytes [64+16g, 64+16g+16) (g = lane / 16).
    auto rdh = [&](v8i& f, const uint8_t* p, int r0, int h) {
        const int r = r0 + (l & 15), gq = (l >> 4) + 4 * h;
        const u32x4 v = *reinterpret_cast<const u32x4*>(p + swz2(r, gq));
        if (h == 0) {
            f[0] = (int)v.x; f[1] = (int)v.y; f[2] = (int)v.z; f[3] = (int)v.w;
        } else {
            f[4] = (int)v.x; f[5] = (int)v.y; f[6] = (int)v.z; f[7] = (int)v.w;
        }
    };
    // One K step: 64 MFMAs with the step's 32 LDS reads (16 bytes per lane
    // each) issued one after each of the first MFMAs, in this order: 0-3 ax
    // (rows 0, 1), 4-15 b[0..5], 16-19 b[6..7], 20-23 ay (rows 2, 3), 24-27
    // ax (rows 4, 5), 28-31 ay (rows 6, 7).  Before an MFMA, lgkm_wait leaves
    // outstanding only reads issued after the last one it needs.
    auto step = [&](auto mode_c, auto deferred_c, int kt) {
        constexpr int MODE = decltype(mode_c)::value;
        constexpr bool DEFERRED = decltype(deferred_c)::value;
        const uint8_t* la = lds_ab[(kt + par) & 1];
        const uint8_t* lb = la + kTileBytes;
        if constexpr (MX) {
            // a tile's first step reads its own scale bytes, before every
            // fragment read so that the waits below cover them too (later
            // steps' were read, and moved into place, by the previous step)
            if constexpr (!DEFERRED) read_scales(kt, sa, sb);
            __builtin_amdgcn_sched_barrier(0);
        }
        // previous step's rows 6, 7 (column-major, registers only) while
        // reads 0-15 go out; b[j] is re-read only after its last old use
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            if constexpr (DEFERRED) {
                if constexpr (MX) mfma_s(6 + (q & 1), b[q >> 1], ay[q & 1], q >> 1, sb_o[q >> 1], sa_o[q & 1]);
                else mfma(6 + (q & 1), b[q >> 1], ay[q & 1], q >> 1);
            }
            if (q < 4) rdh(ax[q >> 1], la, wm + 16 * (q >> 1), q & 1);
            else rdh(b[(q - 4) >> 1], lb, wn + 16 * ((q - 4) >> 1), q & 1);
            if (MODE && (q & 1)) dma(mode_c, kt, q >> 1);
            if (MX && MODE && q == 0) dma(mode_c, kt, 16);
            __builtin_amdgcn_sched_barrier(0);
        }
        // rows 0, 1 (column-major); reads 16-23
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int j = m >> 1, i = m & 1;
            const int issued = 16 + (m < 8 ? m : 8);
            const int need = j < 6 ? 5 + 2 * j : (j == 6 ? 17 : 19);
            lgkm_wait(issued - need - 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma(i, b[j], ax[i], j);
            if (m < 4) rdh(b[6 + (m >> 1)], lb, wn + 16 * (6 + (m >> 1)), m & 1);
            else if (m < 8) rdh(ay[(m - 4) >> 1], la, wm + 32 + 16 * ((m - 4) >> 1), m & 1);
            if (MODE && (m & 1)) dma(mode_c, kt, 8 + (m >> 1));
            __builtin_amdgcn_sched_barrier(0);
        }
        // rows 2, 3; reads 24-27
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int j = m & 7, i = m >> 3;
            const int issued = 24 + (m < 4 ? m : 4);
            lgkm_wait(issued - (i == 0 ? 21 : 23) - 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma(2 + i, b[j], ay[i], j);
            if (m < 4) rdh(ax[m >> 1], la, wm + 64 + 16 * (m >> 1), m & 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        // rows 4, 5; reads 28-31 (MX: then the next step's 16 scale bytes,
        // which only the end-of-step wait covers)
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int j = m & 7, i = m >> 3;
            const int issued = 28 + (m < 4 ? m : 4) + (MX && MODE == 1 && m > 8 ? 16 : 0);
            lgkm_wait(issued - (i == 0 ? 25 : 27) - 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma(4 + i, b[j], ax[i], j);
            if (m < 4) rdh(ay[m >> 1], la, wm + 96 + 16 * (m >> 1), m & 1);
            if (MX && MODE == 1 && m == 8) read_scales(kt + 1, sa_n, sb_n);
            __builtin_amdgcn_sched_barrier(0);
        }
        // MX: the scale bytes move into place for the next step here, where
        // the waits below stall anyway (moved at the next step's start, they
        // delayed its first MFMAs after the barrier): this step's rows 6, 7
        // keep theirs, the next step takes the ones just read
        if constexpr (MX && MODE == 1) {
            // (explicit moves: as plain assignments the compiler put them
            // back after the barrier, on the loop's back edge)
            auto mv = [](int& dst, int src) { __asm__ volatile("v_mov_b32 %0, %1" : "=v"(dst) : "v"(src)); };
#pragma unroll
            for (int i = 0; i < 2; ++i) mv(sa_o[i], sa[6 + i]);
#pragma unroll
            for (int j = 0; j < 8; ++j) mv(sb_o[j], sb[j]);
#pragma unroll
            for (int i = 0; i < 8; ++i) mv(sa[i], sa_n[i]);
#pragma unroll
            for (int j = 0; j < 8; ++j) mv(sb[j], sb_n[j]);
        }
        // this stage fully read; the next stage of this tile landed (the next
        // tile's first stage is waited for at the top of the tile loop)
        lds_wait_all();
        if (MODE == 1) vm_wait<0>();
        stage_barrier();
    };
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using T = std::true_type;
    using F = std::false_type;

    while (true) {
        const int next = logical + per;
        const bool has_next = next < hi;
        // without a next tile the last step re-loads this tile's first stage
        // into the free buffer: harmless, and it keeps the step branch-free
        int ntm_, ntn_;
        tile_coords(has_next ? next : logical, ntm, ntn, ntm_, ntn_);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        load_row_scales(tm, tn);
        // this tile's first stage (and the previous tile's stores) complete
        vm_wait<0>();
        stage_barrier();
        step(C1{}, F{}, 0);
        for (int kt = 1; kt + 1 < nk; ++kt) step(C1{}, T{}, kt);
        na = dmab_plan(K, (int64_t)ntm_ * BM, wave);
        nb = dmab_plan(K, (int64_t)ntn_ * 256, wave);
        if constexpr (MX) {
            nsa_off = srow((int64_t)ntm_ * BM);
            nsb_off = srow((int64_t)ntn_ * 256);
        }
        step(C2{}, T{}, nk - 1);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            mfma(6, b[j], ay[0], j);
            mfma(7, b[j], ay[1], j);
        }
        if constexpr (MX) {
            // keep the last MFMAs here: left free, the compiler sinks them
            // into the epilogue's store branches and spills the fragments
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(acc[i][j]));
        }

        const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * 256;
        if constexpr (OUT == FP8Q_BF16) {
            typedef float v2f_t __attribute__((ext_vector_type(2)));
            typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
            // this wave's 32-row staging area in the stage buffer the last step read
            uint8_t* ep = lds_ab[(nk - 1 + par) & 1] + w * (32 * kEpPitch);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
                for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const v4f v = scaled(acc[2 * qq + ii][j], 2 * qq + ii, j);
                        const v2bf_t p0 = __builtin_convertvector(v2f_t{v[0], v[1]}, v2bf_t);
                        const v2bf_t p1 = __builtin_convertvector(v2f_t{v[2], v[3]}, v2bf_t);
                        const int row = 16 * ii + (l & 15);
                        *reinterpret_cast<uint2*>(ep + row * kEpPitch + (16 * j + 4 * (l >> 4)) * 2) =
                            make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
                    }
                lds_wait_all();
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int row = 4 * u + (l >> 4), ch = l & 15;
                    const u32x4 d = *reinterpret_cast<const u32x4*>(ep + row * kEpPitch + ch * 16);
                    const int64_t m = m0 + wm + 32 * qq + row;
                    const int64_t n = n0 + wn + ch * 8;
                    if (m < M && n < N) __builtin_nontemporal_store(d, reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(g.C) + m * N + n));
                }
            }
        } else {
            // fp32: 16 rows x 128 values per round, pitch 528 B
            uint8_t* ep = lds_ab[(nk - 1 + par) & 1] + w * (16 * kEpPitch32);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    *reinterpret_cast<v4f*>(ep + (l & 15) * kEpPitch32 + (16 * j + 4 * (l >> 4)) * 4) = scaled(acc[i][j], i, j);
                lds_wait_all();
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int row = 2 * u + (l >> 5), ch = l & 31;
                    const u32x4 d = *reinterpret_cast<const u32x4*>(ep + row * kEpPitch32 + ch * 16);
                    const int64_t m = m0 + wm + 16 * i + row;
                    const int64_t n = n0 + wn + ch * 4;
                    if (m < M && n < N) __builtin_nontemporal_store(d, reinterpret_cast<u32x4*>(reinterpret_cast<float*>(g.C) + m * N + n));
                }
            }
        }
        if (!has_next) break;
        logical = next;
        par = (nk + par) & 1;
        if constexpr (!MX) rev ^= 1;
        gpar = (ngroups + gpar) & 1;
        tm = ntm_;
        tn = ntn_;
        da = na;
        db = nb;
        sa_off = nsa_off;
        sb_off = nsb_off;
    }
    // the last step's extra loads land before the workgroup's LDS is released
    vm_wait<0>();
}

template <int FA, int FB, int OUT>
static void launch_sm(const GemmArgs& g, int sm, hipStream_t s) {
    const int ntm = (int)((g.M + BM - 1) / BM);
    // lane offsets, K offset included, stay below 2^32 (rows past the edge may
    // wrap; the buffer load's bounds check then returns zeros or in-range bytes)
    const bool offsets32 = g.M * g.K < (int64_t(1) << 32) && g.N * g.K < (int64_t(1) << 32);
    const bool fast = g.K % BK == 0 && g.K >= 2 * BK && offsets32;
    if (sm == kSmBlock) {
        if (launch_gemm_block_persistent(g, s)) return;
        const int ntn = (int)((g.N + 127) / 128);
        hipLaunchKernelGGL((gemm_kernel<FA, FB, OUT, kSmBlock, 128>), dim3(ntm * ntn), dim3(kThreads), 0, s, g, ntm,
                           ntn);
        return;
    }
    const int ntn = (int)((g.N + 255) / 256);
    if (sm == kSmPerTensor && fast)
        hipLaunchKernelGGL((gemm_pt_kernel<FA, FB, OUT, kSmPerTensor>), dim3(persistent_grid()), dim3(kThreads), 0, s,
                           g, ntm, ntn);
    else if (sm == kSmRow && fast)
        hipLaunchKernelGGL((gemm_pt_kernel<FA, FB, OUT, kSmRow>), dim3(persistent_grid()), dim3(kThreads), 0, s, g,
                           ntm, ntn);
    else if (sm == kSmMx && fast && g.K % 512 == 0 && (uintptr_t)g.sa.s % 16 == 0 && (uintptr_t)g.sb.s % 16 == 0)
        hipLaunchKernelGGL((gemm_pt_kernel<FA, FB, OUT, kSmMx>), dim3(persistent_grid()), dim3(kThreads), 0, s, g,
                           ntm, ntn);
    else if (sm == kSmPerTensor)
        hipLaunchKernelGGL((gemm_kernel<FA, FB, OUT, kSmPerTensor, 256>), dim3(ntm * ntn), dim3(kThreads), 0, s, g, ntm, ntn);
    else if (sm == kSmRow)
        hipLaunchKernelGGL((gemm_kernel<FA, FB, OUT, kSmRow, 256>), dim3(ntm * ntn), dim3(kThreads), 0, s, g, ntm, ntn);
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
    else if (g.sa.gran == FP8Q_ROWWISE || g.sb.gran == FP8Q_ROWWISE) sm = kSmRow;
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
