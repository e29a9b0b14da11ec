/*
 * fp8q: dynamic FP8 scaling and the scaled FP8 GEMM on AMD MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a DEVICE pointer unless stated otherwise,
 * and every call enqueues its work on `stream` (a hipStream_t; NULL is the
 * null stream) and returns without synchronising.  Arguments are validated on
 * the host before any HIP call: a call that returns an error has enqueued
 * nothing and changed nothing.  The library allocates no device memory and
 * keeps no state between calls except a per-device cache of the device
 * architecture; buffers (including workspaces and delayed-scaling state) are
 * owned by the caller.  Outputs must not alias inputs.  No call ever falls
 * back to another precision or another algorithm: an unsupported request is
 * an error (FP8Q_EUNSUPPORTED).
 *
 * What the operations compute (page citations name the source page and its
 * section):
 *   amax      max |x_i|, NaN-propagating.  "fp8_parity.py" lab page,
 *             scaled_roundtrip.
 *   scale     s = max(amax / fmax, 1e-12) in fp32, fmax = 448 (E4M3) or
 *             57344 (E5M2).  Same function; constants E4M3_MAX / E5M2_MAX.
 *   cast      q_i = RNE_fp8(RN_fp32(x_i / s)), OCP float8_e4m3fn / float8_e5m2,
 *             non-saturating (E4M3 overflow -> NaN, E5M2 -> Inf) unless
 *             FP8Q_SATURATE.  Same function (divide, then convert); smoke
 *             check [2] fixes the overflow rule.
 *   delayed   s from the maximum of an amax history of earlier steps (16
 *             entries); the current amax is recorded afterwards.  Smoke
 *             check [3]; SpikingJelly "Training and Inference Precision",
 *             recipe "delayed".
 *   rowwise   one scale per row of each GEMM input along its contraction,
 *             applied to the product as an outer product sA[m] * sB[n].  Lab
 *             page, --recipe rowwise (torchao's rowwise Float8 recipe).
 *   granular  one scale per 1x128 tile (smoke check [4]), per 128x128 block
 *             (SpikingJelly recipe "block"; "How to Optimize
 *             Transformer-Based Models for Low-Precision Training", 2D block
 *             scaling of weights) or one power-of-two E8M0 scale per 32
 *             elements (recipe "mxfp8").
 *   GEMM      y = (Aq . Bq) * sA * sB with fp32 accumulation; fprop (NT),
 *             dgrad (NN), wgrad (TN).  Lab page, class FP8Matmul (forward
 *             and backward products of the quantized operands); the blog post's
 *             fprop / dgrad / wgrad shapes and its autocast vs pre-quantize
 *             modes.
 *
 * Layouts: all matrices are row-major and dense (row stride = columns).
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Version 4: the GEMM workspace starts with its reduce region (so one
 * zero-filled workspace serves calls of any shape), and the entry points
 * fp8_quantize_per_tensor_noalloc and fp8q_mfma_loop_data were added. */
#define FP8Q_ABI_VERSION 4

/* Status codes returned by every entry point. */
typedef enum fp8q_status {
    FP8Q_OK = 0,
    FP8Q_EINVAL = 1,       /* null pointer, negative or zero size, unknown enum or flag */
    FP8Q_EALIGN = 2,       /* a dimension is not a multiple of what the operation needs */
    FP8Q_EUNSUPPORTED = 3, /* a valid combination this library does not implement */
    FP8Q_EDEVICE = 4,      /* no HIP device, or the current device is not gfx950 */
    FP8Q_ELAUNCH = 5,      /* a HIP launch failed (message in fp8q_last_error) */
    FP8Q_EWORKSPACE = 6    /* workspace missing or smaller than required */
} fp8q_status;

/* 8-bit formats: OCP float8_e4m3fn (max 448) and float8_e5m2 (max 57344). */
typedef enum fp8q_format { FP8Q_E4M3 = 0, FP8Q_E5M2 = 1 } fp8q_format;

/* High-precision element types: IEEE fp32 and bfloat16. */
typedef enum fp8q_hp { FP8Q_F32 = 0, FP8Q_BF16 = 1 } fp8q_hp;

/* Scale granularity. */
typedef enum fp8q_gran {
    FP8Q_PER_TENSOR = 0,    /* one fp32 scale */
    FP8Q_TILE_1x128 = 1,    /* one fp32 scale per 128 consecutive elements along K */
    FP8Q_BLOCK_128x128 = 2, /* one fp32 scale per 128 x 128 block */
    FP8Q_MX32 = 3,          /* one E8M0 scale (2^(code-127)) per 32 elements along K */
    FP8Q_ROWWISE = 4        /* one fp32 scale per operand row, over all of K */
} fp8q_gran;

/* Per-tensor scaling mode. */
typedef enum fp8q_scaling { FP8Q_CURRENT = 0, FP8Q_DELAYED = 1 } fp8q_scaling;

/* Flags. */
#define FP8Q_SATURATE 1u   /* clamp finite and infinite overflow to +-fmax instead of NaN / Inf */
/* Count, into state->overflows, the elements of a delayed-scaling cast that
 * overflow the format: finite x whose quotient v = RN32(x / s) the
 * non-saturating cast would turn into NaN (E4M3: |v| > 464, the midpoint
 * above 448 rounding to the odd-mantissa value past the maximum) or +-Inf
 * (E5M2: |v| >= 61440, the tie above 57344 rounding to even 2^16); counted
 * the same way under FP8Q_SATURATE, where such elements are clamped.  This
 * is how a caller detects the overflow that delayed scaling risks when the
 * amax grows past its history (the lab page's smoke check [3]).  Only with
 * DELAYED per-tensor scaling (the count lives in its state); elsewhere
 * FP8Q_EINVAL. */
#define FP8Q_COUNT_OVERFLOW 2u

#define FP8Q_HISTORY_LEN 16

/*
 * Delayed-scaling state, in DEVICE memory, owned by the caller.  Create it
 * zero-filled (an all-zero history is a cold start, which uses the current
 * amax).  The grid-wide amax of a call is folded in the call's reduce
 * workspace; arrive is reserved (keep it zero).  overflows: after every
 * delayed call, the number of elements that overflowed the format when the
 * call had FP8Q_COUNT_OVERFLOW, else 0.  One state
 * must not be used by two calls that may run concurrently.  Saving
 * amax_history and pos checkpoints the recipe.
 */
typedef struct fp8q_delayed_state {
    float amax_history[FP8Q_HISTORY_LEN]; /* amaxes of earlier steps (ring) */
    int32_t pos;                          /* next ring slot to write */
    uint32_t overflows;                   /* overflowing elements of the last call (FP8Q_COUNT_OVERFLOW) */
    uint32_t arrive;                      /* reserved, zero */
    float last_scale;                     /* scale used by the most recent call */
} fp8q_delayed_state;

/* ---------------------------------------------------------------- misc */

/* FP8Q_ABI_VERSION of the loaded library. */
int fp8q_abi_version(void);

/* Static description of a status code (never NULL). */
const char* fp8q_status_string(int status);

/* Detail of the most recent failed call on this host thread ("" if none).
 * The string stays valid until the next call on this thread. */
const char* fp8q_last_error(void);

/* Bytes of device workspace the reductions need: amax partial maxima,
 * per-block keys and completion counters.  The counters must be zero before
 * the workspace's first use (zero-fill a new workspace once); every call
 * leaves them at zero.  Calls that may overlap on the device must not share a
 * workspace. */
size_t fp8q_reduce_workspace_bytes(void);

/* ---------------------------------------------------------------- amax */

/*
 * amax_out[0] = max_i |x_i| over n elements of type hp (NaN if any x_i is
 * NaN).  x: n elements, any alignment of the element type.  ws: at least
 * fp8q_reduce_workspace_bytes() bytes (zero-filled before its first use;
 * see fp8q_reduce_workspace_bytes).  One launch: the last block to finish
 * folds the per-block maxima.  Lab page, scaled_roundtrip.
 */
int fp8_amax(const void* x, int hp, int64_t n, float* amax_out,
             void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- quantize */

/*
 * Per-tensor quantization of x [rows, cols] (type hp) to codes q [rows, cols]
 * in format fmt.
 *   scaling = FP8Q_CURRENT: s = max(amax(x)/fmax, 1e-12) (two passes over x).
 *   scaling = FP8Q_DELAYED: s = max(max(history)/fmax, 1e-12) from `state`
 *     (cold start: current amax); one pass casts and measures amax(x), which
 *     is then written to history[pos] and pos advances modulo 16.
 * qT: optional (may be NULL) second copy of the codes transposed, [cols, rows]
 *   (the K-major operand of a dgrad or wgrad GEMM).
 * scale_out: required, receives s.  amax_out: optional, receives amax(x).
 * flags: FP8Q_SATURATE and, with DELAYED, FP8Q_COUNT_OVERFLOW.
 * ws: fp8q_reduce_workspace_bytes() bytes, zero-filled before its first use
 * (see fp8q_reduce_workspace_bytes).
 * state: required for DELAYED, ignored for CURRENT.
 * Lab page: scaled_roundtrip; smoke check [3] (delayed vs current).
 */
int fp8_quantize_per_tensor(const void* x, int hp, int64_t rows, int64_t cols,
                            int fmt, int scaling, fp8q_delayed_state* state,
                            uint8_t* q, uint8_t* qT, float* scale_out, float* amax_out,
                            unsigned flags, void* ws, size_t ws_bytes, void* stream);

/*
 * fp8_quantize_per_tensor without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments (minus ws,
 * ws_bytes), same results, same errors.  Its reduce region lives in a 64 KiB
 * array of device memory inside the library: each device holds one copy from
 * its first call until the process ends, and the call allocates nothing (no
 * hipMalloc, no allocating library routine).  The region's size does not
 * depend on the input, so every size the workspace form takes fits; a build
 * whose region outgrew the array would return FP8Q_EWORKSPACE.  All calls on
 * one device share that array: calls that may overlap on a device (other
 * streams, other host threads) race and must not be issued.  With DELAYED
 * scaling each call first clears its completion counters with a kernel (no
 * memset), so the call can be captured into a graph and replayed.
 */
int fp8_quantize_per_tensor_noalloc(const void* x, int hp, int64_t rows, int64_t cols,
                                    int fmt, int scaling, fp8q_delayed_state* state,
                                    uint8_t* q, uint8_t* qT, float* scale_out, float* amax_out,
                                    unsigned flags, void* stream);

/*
 * Per-tensor current scaling with a stochastically rounded cast (the
 * gradient rounding of "How to Optimize Transformer-Based Models for
 * Low-Precision Training", applied to the 8-bit formats).
 * s = max(amax / fmax, 1e-12) as fp8_quantize_per_tensor; v = RN32(x / s);
 * v lies between the grid values n D and (n + 1) D (D the grid spacing at
 * |v|, f = |v| / D - n) and becomes (n + 1) D, with the sign of v, when
 * r + floor(f * 2^32) >= 2^32, else n D; the result is encoded as a cast is
 * (overflow rule and FP8Q_SATURATE as above; NaN stays NaN).
 * r for element i (row-major) is word i mod 4 of Philox4x32-10 (Salmon,
 * Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC
 * 2011) with counter (low, high 32 bits of i / 4, low, high 32 bits of
 * offset) and key (low, high 32 bits of seed): equal (seed, offset) give
 * equal codes; callers advance offset (or seed) between steps.
 * q [rows, cols] is required; qT [cols, rows] optional; ws, ws_bytes: the
 * reduce workspace as for fp8_quantize_per_tensor.  Errors as
 * fp8_quantize_per_tensor.
 */
int fp8_quantize_per_tensor_sr(const void* x, int hp, int64_t rows, int64_t cols, int fmt,
                               uint64_t seed, uint64_t offset,
                               uint8_t* q, uint8_t* qT, float* scale_out, float* amax_out,
                               unsigned flags, void* ws, size_t ws_bytes, void* stream);

/*
 * Random Hadamard transform along the rows (the token axis of a wgrad operand;
 * "How to Optimize Transformer-Based Models for Low-Precision Training" lists
 * random Hadamard transforms on the wgrad inputs in its recipe) fused with
 * per-tensor current quantization of the result.
 * y = R x with R block-diagonal over 16-row blocks, each block
 * (1/4) H16 diag(d): H16 the Sylvester Hadamard matrix, H16[i][j] =
 * (-1)^popcount(i & j); d_t = -1 when the top bit of word t mod 4 of
 * Philox4x32-10(counter (low, high 32 bits of t / 4, 0, 0), key (low, high
 * 32 bits of seed)) is set, else +1.  R is orthogonal, so two wgrad operands
 * transformed with the same seed give the same product: (R G)^T (R X) = G^T X.
 * y is computed in fp32 in this order: signs, then the butterflies
 * (a + b, a - b) with partners 1, 2, 4, 8 rows apart, then times 1/4.
 * y is then quantized like fp8_quantize_per_tensor with current scaling:
 * s = max(amax(y) / fmax, 1e-12), q = RNE_fp8(RN_fp32(y / s)).  y itself is
 * not stored.
 * Needs rows % 16 == 0 and cols % 8 == 0, x 16-byte and q 8-byte aligned
 * (else FP8Q_EALIGN).  q [rows, cols] is required; qT [cols, rows] is
 * optional (the K-major copy for fp8_gemm_scaled_TN).  ws: the reduce
 * workspace.  Other errors as fp8_quantize_per_tensor.
 */
int fp8_quantize_per_tensor_rht(const void* x, int hp, int64_t rows, int64_t cols, int fmt,
                                uint64_t seed, uint8_t* q, uint8_t* qT, float* scale_out,
                                float* amax_out, unsigned flags, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * 1x128 tile quantization with fp32 scales (lab page smoke check [4]).
 *   axis = 0: tiles of 128 consecutive columns of a row;
 *             scales [rows, ceil(cols/128)].
 *   axis = 1: tiles of 128 consecutive rows of a column (the 128x1 tiles a
 *             wgrad operand needs, whose contraction runs over rows);
 *             scales [cols, ceil(rows/128)].
 * A tile at the end of a row or column may be shorter.  q [rows, cols];
 * qT optional [cols, rows].  Each tile: s = max(amax(tile)/fmax, 1e-12).
 */
int fp8_quantize_tile1x128(const void* x, int hp, int64_t rows, int64_t cols, int axis,
                           int fmt, uint8_t* q, uint8_t* qT, float* scales,
                           unsigned flags, void* stream);

/*
 * 128x128 block quantization with fp32 scales [ceil(rows/128), ceil(cols/128)]
 * (weights; SpikingJelly recipe "block", blog: 2D block scaling for weights).
 * q [rows, cols]; qT optional [cols, rows].
 */
int fp8_quantize_block128x128(const void* x, int hp, int64_t rows, int64_t cols,
                              int fmt, uint8_t* q, uint8_t* qT, float* scales,
                              unsigned flags, void* stream);

/*
 * MX32 quantization: one E8M0 byte per 32 elements (SpikingJelly recipe
 * "mxfp8").  Scale 2^e with e = ceil(log2(max(amax/fmax, 1e-12))) so that no
 * scaled element exceeds fmax; E8M0 code = e + 127 (255 if the block holds a
 * NaN or Inf).  axis and layouts as fp8_quantize_tile1x128 with 32 in place
 * of 128: e8m0 [rows, ceil(cols/32)] (axis 0) or [cols, ceil(rows/32)] (axis 1).
 */
int fp8_quantize_mx32(const void* x, int hp, int64_t rows, int64_t cols, int axis,
                      int fmt, uint8_t* q, uint8_t* qT, uint8_t* e8m0,
                      unsigned flags, void* stream);

/*
 * Rowwise quantization with fp32 scales: the lab page's "rowwise" recipe,
 * which scales each GEMM input per row along the contraction.
 *   axis = 0: one scale per row, s_r = max(amax(row r) / fmax, 1e-12);
 *             scales [rows].  q [rows, cols] is required; qT must be NULL.
 *             This is the form of an operand whose contraction runs along
 *             its stored columns (fprop x and w, dgrad's gradient).
 *   axis = 1: one scale per column, s_c = max(amax(column c) / fmax, 1e-12);
 *             scales [cols].  q [rows, cols] is required; qT [cols, rows] is
 *             optional and holds the same codes K-major.  This is the form of
 *             an operand whose contraction runs along its stored rows
 *             (dgrad's weight, both wgrad operands).
 * Every code: q = RNE_fp8(RN_fp32(x / s)) with its row's or column's s.
 * Returns FP8Q_EINVAL for null x, q or scales, non-positive sizes, unknown
 * enums or flags, and FP8Q_EUNSUPPORTED for a qT with axis 0.  With axis 1,
 * `scales` holds integer maxima while the call runs.
 */
int fp8_quantize_rowwise(const void* x, int hp, int64_t rows, int64_t cols, int axis,
                         int fmt, uint8_t* q, uint8_t* qT, float* scales,
                         unsigned flags, void* stream);

/* ---------------------------------------------------------------- GEMM */

/*
 * One GEMM operand.
 *
 * Pre-quantized (quantized = 1): `data` holds uint8 codes in the operand's
 * stored layout for the operation (see the GEMM entry points) and `scale`
 * holds its scales:
 *   PER_TENSOR     float[1]
 *   TILE_1x128     float [R, K/128], R = M for A and N for B, indexed by
 *                  (operand row, K block) -- what fp8_quantize_tile1x128
 *                  produces with its tiles running along K (axis 0 when K is
 *                  the stored column axis, axis 1 when K is the stored row axis)
 *   BLOCK_128x128  float [ceil(stored rows/128), ceil(stored cols/128)] in the
 *                  operand's STORED layout (one weight array serves fprop and dgrad)
 *   MX32           uint8 E8M0 [R, K/32], indexed like TILE_1x128
 *   ROWWISE        float [R], one per operand row (what fp8_quantize_rowwise
 *                  produces with axis 0 when K is the stored column axis,
 *                  axis 1 when K is the stored row axis); pre-quantized only
 *   `data_kmajor` optionally holds the same codes already laid out [R, K]
 *   (K contiguous); if NULL and the stored layout is not K-contiguous, the
 *   library transposes the codes into the workspace.
 * Autocast (quantized = 0): `data` holds fp32 or bf16 values (`hp`) in the
 *   stored layout; the GEMM quantizes them itself with `granularity`
 *   (PER_TENSOR with `scaling` CURRENT or DELAYED + `state`, or TILE_1x128 /
 *   BLOCK_128x128 / MX32 with current scaling) into the workspace, inside the
 *   same enqueued work, and writes the per-tensor scale / amax to
 *   scale_out / amax_out when they are not NULL.
 */
typedef struct fp8q_operand {
    const void* data;
    const void* data_kmajor;
    const void* scale;
    int32_t quantized;
    int32_t format;       /* fp8q_format */
    int32_t granularity;  /* fp8q_gran */
    int32_t hp;           /* fp8q_hp (autocast) */
    int32_t scaling;      /* fp8q_scaling (autocast, per-tensor) */
    uint32_t flags;       /* FP8Q_SATURATE; FP8Q_COUNT_OVERFLOW with DELAYED (autocast) */
    fp8q_delayed_state* state;
    float* scale_out;
    float* amax_out;
} fp8q_operand;

/*
 * Workspace bytes a GEMM call with these arguments needs (0 if none).
 * op: 0 = NT, 1 = NN, 2 = TN.  Returns (size_t)-1 for invalid arguments.
 */
size_t fp8_gemm_workspace_bytes(int op, int64_t M, int64_t N, int64_t K,
                                const fp8q_operand* A, const fp8q_operand* B);

/*
 * C [M, N] = sum_k A(m,k) * B(n,k), with each product's operands' scales
 * applied per the granularity (per-tensor: the sum times sA * sB; 1x128 /
 * 128x128: per 128-element K block; MX32: per 32-element K block), fp32
 * accumulation, C written as c_dtype (FP8Q_F32 or FP8Q_BF16, round to
 * nearest even).
 *
 *   fp8_gemm_scaled_NT (fprop, y = x w^T):  A stored [M, K], B stored [N, K]
 *   fp8_gemm_scaled_NN (dgrad, dx = g w):   A stored [M, K], B stored [K, N]
 *   fp8_gemm_scaled_TN (wgrad, dw = g^T x): A stored [K, M], B stored [K, N]
 *
 * Alignment: M, N, K multiples of 16 (SpikingJelly alignment rule, lab page
 * module_filter_fn); K a multiple of 128 with TILE_1x128 / BLOCK_128x128
 * operands and of 32 with MX32.  Granularities: A and B each PER_TENSOR,
 * TILE_1x128 or BLOCK_128x128 in any combination, or both MX32, or ROWWISE
 * with ROWWISE or PER_TENSOR (C = sum * sA[m] * sB[n], per-tensor scales
 * broadcast).  ROWWISE operands must be pre-quantized (autocast with ROWWISE
 * returns FP8Q_EUNSUPPORTED).
 * ws: fp8_gemm_workspace_bytes(...) bytes (may be NULL when that is 0),
 * 256-byte aligned, zero-filled before its first use: autocast operands
 * reduce in it, and its completion counters must start at zero (every call
 * leaves them at zero).  A non-empty workspace always begins with the
 * reduction region (fp8q_reduce_workspace_bytes() bytes, counters included),
 * and staged codes and scales follow it, so one zero-filled workspace as
 * large as each call needs may serve GEMMs of different shapes and
 * granularities in turn.  Calls that may overlap on the device must not
 * share a workspace.
 */
int fp8_gemm_scaled_NT(int64_t M, int64_t N, int64_t K, const fp8q_operand* A,
                       const fp8q_operand* B, void* C, int c_dtype,
                       void* ws, size_t ws_bytes, void* stream);
int fp8_gemm_scaled_NN(int64_t M, int64_t N, int64_t K, const fp8q_operand* A,
                       const fp8q_operand* B, void* C, int c_dtype,
                       void* ws, size_t ws_bytes, void* stream);
int fp8_gemm_scaled_TN(int64_t M, int64_t N, int64_t K, const fp8q_operand* A,
                       const fp8q_operand* B, void* C, int c_dtype,
                       void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ measurement aid
 * fp8q_mfma_loop: not part of the FP8 path.  Launches `blocks` workgroups of
 * 256 threads; every wave runs `iters` rounds of 8 independent 16x16x128
 * E4M3 MFMAs on operands held in registers (all codes 1.0) and writes one
 * float per thread to out (device, blocks * 256 floats, caller-owned): exactly
 * 4096 * iters, exact for iters <= 4096.  Each round of a wave is 8 * 2 * 16 * 16 * 128
 * FLOP, so timing the call gives the sustained FP8 MFMA rate with no memory
 * traffic: the measured ceiling beside the nominal dense peak.
 * EINVAL for blocks <= 0, iters <= 0 or out == NULL; enqueued on `stream`.
 */
int fp8q_mfma_loop(int blocks, int iters, float* out, void* stream);

/* fp8q_mfma_loop with a choice of operand data: data = 0 is fp8q_mfma_loop
 * (all codes 1.0, exact output); data = 1 gives every lane 8 A and 8 B
 * operand sets of pseudo-random E4M3 codes (random sign, normal exponent,
 * any mantissa; never NaN) and feeds each MFMA a different pair, so the
 * matrix cores see data that changes every instruction, as in a GEMM.  The
 * cores' energy depends on their data, so under the chip's power limit this
 * is the sustained rate for such data; its output is finite but not
 * checkable exactly.  data = 1 needs iters % 8 == 0.  EINVAL otherwise, as
 * fp8q_mfma_loop. */
int fp8q_mfma_loop_data(int blocks, int iters, int data, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
