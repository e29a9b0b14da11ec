// Host-side launchers of the fp8q HIP kernels (internal; the C ABI is in fp8q.h).
// Launchers assume validated arguments and return the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fp8q.h"

namespace fp8q {

// Largest number of blocks a reduction grid uses; the reduce workspace holds
// one fp32 partial maximum per block.
constexpr int kReduceParts = 2048;
// Reduce workspace layout: kReduceParts partial maxima (read by the next
// kernel), kReduceParts per-block keys (folded by the last block of the same
// kernel), then completion counters for a two-level ticket tree: a top counter
// and one counter per group of kTicketGroup blocks, each on its own 256-byte
// line.  The counters are zero between calls.
constexpr int kTicketGroup = 32;
constexpr int kTicketLine = 64;   // uint32 words per counter line
constexpr size_t kReduceKeysOffset = kReduceParts * sizeof(float);
constexpr size_t kReduceCtrOffset = kReduceKeysOffset + kReduceParts * sizeof(uint32_t);
constexpr size_t kReduceCtrBytes = (1 + kReduceParts / kTicketGroup) * kTicketLine * sizeof(uint32_t);
constexpr size_t kReduceWsBytes = kReduceCtrOffset + kReduceCtrBytes;
static_assert(kReduceParts <= 256 * 8, "reduce_partials_256 folds at most 8 partials per thread");

// Workgroups of a persistent kernel with one workgroup per CU: the CU count,
// rounded down to a multiple of the 8 XCDs (the GEMMs split their tiles into
// 8 per-XCD ranges).
// (Cached per device; threads that race to fill an entry store the same value.)
inline int persistent_grid() {
    static std::atomic<int> cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int g = cached[dev].load(std::memory_order_relaxed);
    if (g == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) cus = 256;
        g = cus / 8 * 8;
        cached[dev].store(g, std::memory_order_relaxed);
    }
    return g;
}

// Quantization schemes of the tiled quantize kernel.
enum Scheme : int {
    kPerTensorCurrent = 0,  // s from the amax partials of a preceding amax grid
    kPerTensorDelayed = 1,  // s from the amax history (cold start: partials)
    kTileAxis0 = 2,         // 1 x 128 along columns
    kTileAxis1 = 3,         // 128 x 1 along rows
    kBlock = 4,             // 128 x 128
    kMxAxis0 = 5,           // 1 x 32 along columns, E8M0
    kMxAxis1 = 6            // 32 x 1 along rows, E8M0
};

struct QuantArgs {
    const void* x;
    int hp;
    int64_t rows, cols;
    int fmt;
    int scheme;
    bool saturate;
    uint8_t* q;            // [rows, cols] or NULL
    uint8_t* qT;           // [cols, rows] or NULL
    float* scales;         // tile / block scales
    uint8_t* e8m0;         // MX scales
    const float* partials; // amax partials (per-tensor current; delayed cold start)
    int nparts;
    uint32_t* keys;        // per-block keys and ticket counters of the reduce
    uint32_t* ctrs;        // workspace (delayed scaling's grid-wide amax)
    fp8q_delayed_state* state;
    float* scale_out;
    float* amax_out;
    bool count_overflow;   // delayed scaling: add overflowing elements to state->overflows
};

// amax partial maxima over n elements: one float per block into partials[0..nparts).
// If gate != NULL the grid does nothing unless gate's history is all zero; in
// either case it first clears gate->overflows (the delayed cast that follows
// counts into it).
// If keys != NULL the blocks instead fold their maxima among themselves (keys and
// ticket counters of the reduce workspace) and the last block writes *amax_out.
int amax_partials_grid(int64_t n);
hipError_t launch_amax_partials(const void* x, int hp, int64_t n, float* partials, int nparts,
                                fp8q_delayed_state* gate, hipStream_t s, uint32_t* keys = nullptr,
                                uint32_t* ctrs = nullptr, float* amax_out = nullptr);

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);

// n 32-bit words at p set to zero by a kernel (capturable in a graph)
hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t s);

// codes [rows, cols] -> [cols, rows]
hipError_t launch_transpose_u8(const uint8_t* in, int64_t rows, int64_t cols, uint8_t* out, hipStream_t s);

// Per-tensor current scaling with a stochastically rounded cast: the scale
// from the amax partials (as the current-scaling cast), element i rounded with
// word i mod 4 of Philox4x32-10(counter (i / 4, offset), key seed).
hipError_t launch_quantize_sr(const void* x, int hp, int64_t n, int fmt, bool sat, uint64_t seed, uint64_t offset,
                              const float* partials, int nparts, uint8_t* q, float* scale_out, float* amax_out,
                              hipStream_t s);

// Random Hadamard transform along rows (16-row blocks, signs from Philox with
// key seed) fused with per-tensor current quantization of the result;
// rows % 16 == 0, cols % 8 == 0, x 16-byte and q 8-byte aligned.  partials:
// the reduce workspace's partial maxima (kReduceParts floats).
hipError_t launch_quantize_rht(const void* x, int hp, int64_t rows, int64_t cols, int fmt, bool sat, uint64_t seed,
                               float* partials, uint8_t* q, uint8_t* qT, float* scale_out, float* amax_out,
                               hipStream_t s);

// Measurement aid: `blocks` workgroups of 256 threads, each wave running
// `iters` rounds of 8 register-only FP8 MFMAs on all-ones operands (data 0)
// or on pseudo-random codes that change every MFMA (data 1, iters % 8 == 0);
// out holds blocks * 256 floats.
hipError_t launch_mfma_loop(int blocks, int iters, int data, float* out, hipStream_t s);

// Rowwise quantization: one fp32 scale per row (axis 0) or per column (axis
// 1) into scales, codes into q [rows, cols], and (if qT != NULL) their
// transpose into qT [cols, rows].  Axis 1 keeps integer maxima in `scales`
// until its cast pass has converted them.
hipError_t launch_quantize_rowwise(const void* x, int hp, int64_t rows, int64_t cols, int axis, int fmt, bool sat,
                                   uint8_t* q, uint8_t* qT, float* scales, hipStream_t s);

// Scaled GEMM on K-contiguous codes: C[M,N] = sum_k A[m,k] B[n,k] with scales.
struct GemmScale {
    const void* s;     // float* or uint8_t* (E8M0)
    int gran;          // fp8q_gran
    int64_t ld;        // row stride of the scale array (elements)
    int64_t kstride;   // stride between K blocks (elements)
    int rshift;        // operand row -> scale row: row >> rshift (0: per row, 7: 128-row blocks)
};

struct GemmArgs {
    const uint8_t* A;  // [M, K]
    const uint8_t* B;  // [N, K]
    void* C;           // [M, N]
    int64_t M, N, K;
    int fa, fb;        // fp8q_format
    int c_dtype;       // fp8q_hp
    GemmScale sa, sb;
};

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s);
// Block-scaled GEMM on the persistent kernel when its conditions hold (K %
// 512 == 0, K-contiguous 16-byte-aligned row scales, ...); false: not launched.
bool launch_gemm_block_persistent(const GemmArgs& g, hipStream_t s);

}  // namespace fp8q
