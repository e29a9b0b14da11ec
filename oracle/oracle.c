/*
 * CPU oracle for dynamic FP8 scaling and the scaled FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the GPU library computes.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or constant generator with the HIP library, and the HIP
 * library never calls it.
 *
 * Sources (web pages; cited by title and section):
 *   [LAB]  "fp8_parity.py" course lab page (FP8 numerics on CPU ...):
 *          constants E4M3_MAX / E5M2_MAX, function scaled_roundtrip,
 *          class FP8Matmul, smoke() checks [1]-[5].
 *   [SJ]   SpikingJelly "Training and Inference Precision": recipe names
 *          delayed / current / block / mxfp8, alignment rule.
 *   [BLOG] "How to Optimize Transformer-Based Models for Low-Precision
 *          Training" (machine-reworded copy): autocast vs pre-quantize,
 *          fprop / dgrad / wgrad GEMM shapes, MXFP8 and 2D block scaling.
 *
 * Precision: the pages fix the arithmetic of the quantizer (fp32 tensors
 * divided by an fp32 scale, then cast to an 8-bit float), so scales and
 * quotients are fp32, each correctly rounded.  A binary32 quotient is
 * obtained as (float)((double)a / (double)b); the double rounding is
 * innocuous because 53 >= 2*24 + 2 (Figueroa, "When is double rounding
 * innocuous?", 1995).  GEMM dot products of 8-bit codes are summed exactly
 * in integers and scaled in fp64.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   overflow of a cast is non-saturating by default (E4M3 -> NaN, E5M2 ->
 *   +-Inf), which is the only rule under which [LAB] smoke check [2] holds;
 *   a SATURATE option clamps to +-max instead.  MX32 scales are
 *   2^ceil(log2(amax/fmax)) (parity unpinned: a convention).  Delayed
 *   scaling with an all-zero history (cold start) uses the current amax
 *   (parity unpinned: a convention).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_E4M3 0
#define ORC_E5M2 1
#define ORC_F32 0
#define ORC_BF16 1

/* ------------------------------------------------------------------ */
/* Formats.  OCP 8-bit floats as named by [LAB] (torch.float8_e4m3fn,    */
/* torch.float8_e5m2), maxima 448 and 57344 ([LAB] constants, check [1]) */
/* ------------------------------------------------------------------ */

static int fmt_mbits(int fmt) { return fmt == ORC_E4M3 ? 3 : 2; }
static int fmt_bias(int fmt) { return fmt == ORC_E4M3 ? 7 : 15; }

double orc_fmax(int fmt) { return fmt == ORC_E4M3 ? 448.0 : 57344.0; }

/* Smallest normal magnitude: 2^-6 (E4M3), 2^-14 (E5M2) ([LAB] check [1]). */
double orc_smallest_normal(int fmt) { return ldexp(1.0, 1 - fmt_bias(fmt)); }

/* Value of an 8-bit code.  E4M3 (fn variant): no infinities, S.1111.111 is
 * NaN.  E5M2: IEEE-like, exponent field 31 is Inf (mantissa 0) or NaN. */
double orc_decode(uint8_t code, int fmt)
{
    const int mb = fmt_mbits(fmt), bias = fmt_bias(fmt);
    const int ebits = 7 - mb;
    const int sign = code >> 7;
    const int e = (code >> mb) & ((1 << ebits) - 1);
    const int m = code & ((1 << mb) - 1);
    double v;
    if (fmt == ORC_E4M3 && e == 15 && m == 7)
        return NAN;
    if (fmt == ORC_E5M2 && e == 31)
        return m == 0 ? (sign ? -INFINITY : INFINITY) : NAN;
    if (e == 0)
        v = ldexp((double)m, 1 - bias - mb);                  /* subnormal */
    else
        v = ldexp((double)((1 << mb) + m), e - bias - mb);    /* normal */
    return sign ? -v : v;
}

/* Encode an fp32 value: round to nearest on the format's grid (subnormals
 * included), ties to the even code; sign kept (so -0 and tiny negatives give
 * 0x80); NaN gives the NaN code with the sign kept.  A rounded magnitude
 * above the format maximum overflows: NaN for E4M3, Inf for E5M2, or, with
 * saturate, the largest finite code.  Inf input overflows the same way. */
uint8_t orc_encode(float v, int fmt, int saturate)
{
    const int mb = fmt_mbits(fmt), bias = fmt_bias(fmt);
    const double fmax = orc_fmax(fmt);
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const uint8_t maxcode = fmt == ORC_E4M3 ? 0x7E : 0x7B;
    const uint8_t ovfcode = fmt == ORC_E4M3 ? 0x7F : 0x7C;
    double a, quantum, n, r;
    int e, E;

    if (isnan(v))
        return sign | 0x7F;
    a = fabs((double)v);
    if (isinf(a))
        return sign | (saturate ? maxcode : ovfcode);
    if (a == 0.0)
        return sign;
    /* grid spacing at |v|: 2^(max(floor(log2|v|), emin) - mbits) */
    frexp(a, &e);
    E = e - 1;
    if (E < 1 - bias)
        E = 1 - bias;
    quantum = ldexp(1.0, E - mb);
    n = nearbyint(a / quantum);          /* exact quotient; RNE (default mode) */
    r = n * quantum;
    if (r > fmax)
        return sign | (saturate ? maxcode : ovfcode);
    if (r == 0.0)
        return sign;
    frexp(r, &e);
    E = e - 1;                           /* exponent after rounding (may carry) */
    if (E < 1 - bias)
        return sign | (uint8_t)n;        /* subnormal code: mantissa = n */
    {
        const int mant = (int)ldexp(r, mb - E) - (1 << mb);
        return sign | (uint8_t)(((E + bias) << mb) | mant);
    }
}

/* ------------------------------------------------------------------ */
/* Element access                                                      */
/* ------------------------------------------------------------------ */

/* bf16 widens to fp32 exactly: its bits are the top half of an fp32. */
static float load_hp(const void* x, int hp, int64_t i)
{
    if (hp == ORC_BF16) {
        uint32_t b = (uint32_t)((const uint16_t*)x)[i] << 16;
        float f;
        memcpy(&f, &b, 4);
        return f;
    }
    return ((const float*)x)[i];
}

/* Correctly rounded binary32 quotient (see header). */
static float div_rn32(float a, float b) { return (float)((double)a / (double)b); }

/* ------------------------------------------------------------------ */
/* amax, scale, cast: [LAB] scaled_roundtrip                            */
/* ------------------------------------------------------------------ */

/* amax = max |x_i|, NaN-propagating (torch's max), -0 counted as 0. */
float orc_amax_strided(const void* x, int hp, int64_t n, int64_t stride)
{
    float m = 0.0f;
    int64_t i;
    for (i = 0; i < n; ++i) {
        const float a = fabsf(load_hp(x, hp, i * stride));
        if (isnan(a))
            return NAN;
        if (a > m)
            m = a;
    }
    return m;
}

float orc_amax(const void* x, int hp, int64_t n) { return orc_amax_strided(x, hp, n, 1); }

/* s = max(amax / fmax, 1e-12), in fp32 ([LAB] scaled_roundtrip: the largest
 * magnitude over the format maximum, bounded below by 1e-12; a NaN amax
 * gives a NaN scale). */
float orc_scale_from_amax(float amax, int fmt)
{
    const float floor_s = (float)1e-12;
    const float s = div_rn32(amax, (float)orc_fmax(fmt));
    if (isnan(s))
        return s;
    return s < floor_s ? floor_s : s;
}

/* q_i = encode(RN32(x_i / s)): [LAB] scaled_roundtrip divides by the scale
 * in fp32, then converts to the 8-bit type. */
uint8_t orc_cast1(float x, float s, int fmt, int saturate)
{
    return orc_encode(div_rn32(x, s), fmt, saturate);
}

void orc_cast(const void* x, int hp, int64_t n, float s, int fmt, int saturate, uint8_t* q)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        q[i] = orc_cast1(load_hp(x, hp, i), s, fmt, saturate);
}

/* Per-tensor current scaling: amax, scale, cast ([LAB] scaled_roundtrip with
 * scale=None; [SJ] recipe "current"). */
void orc_quantize_per_tensor(const void* x, int hp, int64_t n, int fmt, int saturate,
                             uint8_t* q, float* scale_out, float* amax_out)
{
    const float amax = orc_amax(x, hp, n);
    const float s = orc_scale_from_amax(amax, fmt);
    orc_cast(x, hp, n, s, fmt, saturate, q);
    if (scale_out) *scale_out = s;
    if (amax_out) *amax_out = amax;
}

/* Delayed scaling ([LAB] smoke check [3]; [SJ] recipe "delayed"): the scale
 * comes from the maximum of the amax history of earlier steps; the current
 * amax is then recorded in the ring of 16 entries.  Cold start (every entry
 * zero) uses the current amax. */
void orc_quantize_delayed(const void* x, int hp, int64_t n, int fmt, int saturate,
                          float* hist, int32_t* pos, int hist_len,
                          uint8_t* q, float* scale_out, float* amax_out)
{
    const float amax = orc_amax(x, hp, n);
    float hmax = 0.0f, s;
    int i;
    for (i = 0; i < hist_len; ++i) {
        if (isnan(hist[i])) { hmax = NAN; break; }
        if (hist[i] > hmax) hmax = hist[i];
    }
    s = orc_scale_from_amax(hmax == 0.0f ? amax : hmax, fmt);
    orc_cast(x, hp, n, s, fmt, saturate, q);
    hist[*pos] = amax;
    *pos = (*pos + 1) % hist_len;
    if (scale_out) *scale_out = s;
    if (amax_out) *amax_out = amax;
}

/* Overflow count of a cast with scale s: the finite x_i whose non-saturating
 * code encode(RN32(x_i / s)) is the format's overflow code (E4M3: NaN, as
 * the format has no infinities; E5M2: +-Inf).  This is what delayed scaling
 * risks when the amax outgrows its history ([LAB] smoke check [3]); a
 * saturating cast clamps the same elements. */
int64_t orc_overflow_count(const void* x, int hp, int64_t n, float s, int fmt)
{
    int64_t i, count = 0;
#pragma omp parallel for reduction(+ : count) schedule(static)
    for (i = 0; i < n; ++i) {
        const float xi = load_hp(x, hp, i);
        uint8_t c;
        if (!isfinite(xi)) continue;
        c = orc_cast1(xi, s, fmt, 0);
        if (fmt == ORC_E4M3 ? (c & 0x7F) == 0x7F : (c & 0x7F) == 0x7C) ++count;
    }
    return count;
}

/* ------------------------------------------------------------------ */
/* Stochastic rounding of a cast ([BLOG]: the low-precision recipe rounds */
/* its gradients stochastically; applied here to the 8-bit formats).      */
/* ------------------------------------------------------------------ */

/* Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): ten rounds; a
 * round multiplies counter words 0 and 2 by 0xD2511F53 and 0xCD9E8D57 (32 x
 * 32 -> 64 bits) and forms (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key
 * grows by the Weyl increments 0x9E3779B9, 0xBB67AE85 before every round
 * after the first. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
    int r;
    for (r = 0; r < 10; ++r) {
        uint64_t p0, p1;
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        p0 = (uint64_t)0xD2511F53u * c0;
        p1 = (uint64_t)0xCD9E8D57u * c2;
        c0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        c1 = (uint32_t)p1;
        c2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c3 = (uint32_t)p0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Random word of element i (reading, in the design notes): word i mod 4 of
 * Philox4x32-10 with counter (low, high half of i / 4, low, high half of
 * offset) and key (low, high half of seed). */
uint32_t orc_sr_word(uint64_t seed, uint64_t offset, uint64_t i)
{
    const uint64_t g = i >> 2;
    const uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return out[i & 3];
}

/* Stochastic rounding of v with the random word r (reading, in the design
 * notes).  |v| lies in [n D, (n + 1) D) for the grid spacing D at |v|
 * (2^(max(floor(log2|v|), 1 - bias) - mantissa bits)); with
 * f = |v| / D - n, the magnitude becomes (n + 1) D when
 * r + floor(f * 2^32) >= 2^32 -- probability floor(f * 2^32) / 2^32 for a
 * uniform r -- and n D otherwise.  Where the round-to-nearest cast of v is
 * finite, the magnitude is capped at the format maximum: a v just above the
 * maximum (current scaling puts the amax element within an ulp or two of
 * it) must not round up to a step past it and overflow.  Where that cast
 * overflows, the stochastic result is encoded as it stands (a step past the
 * maximum then overflows like a cast).  The sign is kept.  NaN and +-Inf
 * are encoded unchanged. */
uint8_t orc_encode_sr(float v, uint32_t r, int fmt, int saturate)
{
    double a, D, n, f, mag;
    uint64_t frac32;
    int e;
    if (isnan(v) || isinf(v)) return orc_encode(v, fmt, saturate);
    a = fabs((double)v);
    e = 1 - fmt_bias(fmt);
    if (a != 0.0) {
        int ea;
        frexp(a, &ea);          /* a = m 2^ea, m in [0.5, 1): floor(log2 a) = ea - 1 */
        if (ea - 1 > e) e = ea - 1;
    }
    D = ldexp(1.0, e - fmt_mbits(fmt));
    n = floor(a / D);           /* a / D exact: D is a power of two */
    f = a / D - n;
    frac32 = (uint64_t)floor(ldexp(f, 32));
    if ((uint64_t)r + frac32 >= ((uint64_t)1 << 32)) n += 1.0;
    mag = n * D;
    if (mag > orc_fmax(fmt)) {
        const uint8_t rne = orc_encode(v, fmt, 0);
        const int rne_finite = fmt == ORC_E4M3 ? (rne & 0x7F) != 0x7F : (rne & 0x7F) < 0x7C;
        if (rne_finite) mag = orc_fmax(fmt);
    }
    return orc_encode((float)copysign(mag, (double)v), fmt, saturate);
}

/* Per-tensor current scaling with a stochastically rounded cast: amax and
 * scale as orc_quantize_per_tensor, then q_i = encode_sr(RN32(x_i / s),
 * word(seed, offset, i)). */
void orc_quantize_per_tensor_sr(const void* x, int hp, int64_t n, int fmt, int saturate, uint64_t seed,
                                uint64_t offset, uint8_t* q, float* scale_out, float* amax_out)
{
    const float amax = orc_amax(x, hp, n);
    const float s = orc_scale_from_amax(amax, fmt);
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        q[i] = orc_encode_sr(div_rn32(load_hp(x, hp, i), s), orc_sr_word(seed, offset, (uint64_t)i), fmt, saturate);
    if (scale_out) *scale_out = s;
    if (amax_out) *amax_out = amax;
}

/* ------------------------------------------------------------------ */
/* Random Hadamard transform of a wgrad operand ([BLOG] lists random      */
/* Hadamard transforms on the wgrad inputs among its recipe's extra       */
/* operations; the form below is a reading, listed in the design notes). */
/* ------------------------------------------------------------------ */

/* Sign of token t: -1 when the top bit of its Philox word (offset 0) is set. */
int orc_rht_sign(uint64_t seed, int64_t t)
{
    return (orc_sr_word(seed, 0, (uint64_t)t) >> 31) ? -1 : 1;
}

/* y = R x along rows, R = blockdiag over 16-row blocks of (1/4) H16 diag(d):
 * in fp32, signs first, then the Walsh-Hadamard butterflies (a + b, a - b)
 * with partners 1, 2, 4, 8 rows apart (which multiply by the Sylvester H16,
 * H16[i][j] = (-1)^popcount(i & j)), then the factor 1/4.  rows % 16 == 0. */
void orc_rht(const void* x, int hp, int64_t rows, int64_t cols, uint64_t seed, float* y)
{
    const int64_t nb = rows / 16;
    int64_t b;
#pragma omp parallel for schedule(static)
    for (b = 0; b < nb; ++b) {
        int sg[16], i, h;
        int64_t c;
        for (i = 0; i < 16; ++i) sg[i] = orc_rht_sign(seed, b * 16 + i);
        for (c = 0; c < cols; ++c) {
            float v[16];
            for (i = 0; i < 16; ++i) {
                v[i] = load_hp(x, hp, (b * 16 + i) * cols + c);
                if (sg[i] < 0) v[i] = -v[i];
            }
            for (h = 1; h < 16; h <<= 1)
                for (i = 0; i < 16; ++i)
                    if ((i & h) == 0) {
                        const float a = v[i], d = v[i + h];
                        v[i] = a + d;
                        v[i + h] = a - d;
                    }
            for (i = 0; i < 16; ++i) y[(b * 16 + i) * cols + c] = v[i] * 0.25f;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Granular scaling: 1 x T tiles ([LAB] check [4]: scaled_roundtrip per   */
/* 128-wide row), T x 1 tiles, Br x Bc blocks ([SJ] "block"; [BLOG] 2D    */
/* block scaling for weights), MX blocks of 32 with an E8M0 power-of-two  */
/* scale ([SJ] "mxfp8").  x is row-major [rows, cols].  Tiles at the end  */
/* of a row or column may be shorter (ragged).                            */
/* ------------------------------------------------------------------ */

/* Quantize one rectangular block of x (rows r0..r1, cols c0..c1) with its own
 * scale; returns the scale used (for MX, the power of two 2^e) and, for MX,
 * writes the E8M0 code. */
static float quantize_rect(const void* x, int hp, int64_t cols, int64_t r0, int64_t r1,
                           int64_t c0, int64_t c1, int fmt, int saturate, uint8_t* q,
                           int mx, uint8_t* e8m0_out)
{
    float amax = 0.0f, s;
    int64_t r, c;
    for (r = r0; r < r1 && !isnan(amax); ++r)
        for (c = c0; c < c1; ++c) {
            const float a = fabsf(load_hp(x, hp, r * cols + c));
            if (isnan(a)) { amax = NAN; break; }
            if (a > amax) amax = a;
        }
    s = orc_scale_from_amax(amax, fmt);
    if (mx) {
        /* E8M0: 2^e with e = ceil(log2 s), read from the bits of s. */
        uint8_t code;
        if (!isfinite(s)) {
            code = 0xFF;
            s = NAN;
        } else {
            uint32_t b;
            int be, e;
            memcpy(&b, &s, 4);
            be = (int)(b >> 23);
            e = (b & 0x7FFFFF) == 0 ? be - 127 : be - 126;
            code = (uint8_t)(e + 127);
            s = ldexpf(1.0f, e);
        }
        *e8m0_out = code;
    }
    for (r = r0; r < r1; ++r)
        for (c = c0; c < c1; ++c)
            q[r * cols + c] = orc_cast1(load_hp(x, hp, r * cols + c), s, fmt, saturate);
    return s;
}

/* axis 0: 1 x T tiles along each row, scales [rows, ceil(cols/T)].
 * axis 1: T x 1 tiles along each column, scales [cols, ceil(rows/T)].
 * mx != 0: scales are E8M0 bytes (e8m0 output), else fp32 (scales output). */
void orc_quantize_tiles(const void* x, int hp, int64_t rows, int64_t cols, int axis,
                        int64_t T, int fmt, int saturate, int mx,
                        uint8_t* q, float* scales, uint8_t* e8m0)
{
    int64_t r, c;
    if (axis == 0) {
        const int64_t nt = (cols + T - 1) / T;
#pragma omp parallel for private(c) schedule(static)
        for (r = 0; r < rows; ++r)
            for (c = 0; c < nt; ++c) {
                const int64_t c0 = c * T, c1 = c0 + T < cols ? c0 + T : cols;
                uint8_t e = 0;
                const float s = quantize_rect(x, hp, cols, r, r + 1, c0, c1, fmt, saturate, q, mx, &e);
                if (mx) e8m0[r * nt + c] = e; else scales[r * nt + c] = s;
            }
    } else {
        const int64_t nt = (rows + T - 1) / T;
#pragma omp parallel for private(r) schedule(static)
        for (c = 0; c < cols; ++c)
            for (r = 0; r < nt; ++r) {
                const int64_t r0 = r * T, r1 = r0 + T < rows ? r0 + T : rows;
                uint8_t e = 0;
                const float s = quantize_rect(x, hp, cols, r0, r1, c, c + 1, fmt, saturate, q, mx, &e);
                if (mx) e8m0[c * nt + r] = e; else scales[c * nt + r] = s;
            }
    }
}

/* Br x Bc blocks, scales [ceil(rows/Br), ceil(cols/Bc)] row-major. */
void orc_quantize_blocks(const void* x, int hp, int64_t rows, int64_t cols, int64_t Br,
                         int64_t Bc, int fmt, int saturate, uint8_t* q, float* scales)
{
    const int64_t nbr = (rows + Br - 1) / Br, nbc = (cols + Bc - 1) / Bc;
    int64_t i, j;
#pragma omp parallel for private(j) schedule(static)
    for (i = 0; i < nbr; ++i)
        for (j = 0; j < nbc; ++j) {
            const int64_t r0 = i * Br, r1 = r0 + Br < rows ? r0 + Br : rows;
            const int64_t c0 = j * Bc, c1 = c0 + Bc < cols ? c0 + Bc : cols;
            scales[i * nbc + j] = quantize_rect(x, hp, cols, r0, r1, c0, c1, fmt, saturate, q, 0, NULL);
        }
}

/* ------------------------------------------------------------------ */
/* Scaled GEMM ([LAB] FP8Matmul: forward = input times transposed weight, */
/* backward = gradient times weight and transposed gradient times input; */
/* [BLOG] fprop / dgrad / wgrad):                                        */
/*   y[m,n] = sum over K-blocks kb of sA(m,kb) * sB(n,kb) *               */
/*            sum_{k in kb} qA[m,k] * qB[n,k]                             */
/* The inner sums are exact: an E4M3 value is an integer multiple of 2^-9 */
/* and an E5M2 value one of 2^-16, so code products are integers times    */
/* 2^-(fa+fb) and are summed in __int128.  Each block sum is converted to */
/* fp64 (one rounding, relative 2^-53), scaled in fp64 and accumulated in */
/* fp64.  Operands are addressed by strides so that one routine covers    */
/* every storage layout:  A(m,k) = A[m*a_sm + k*a_sk], B(n,k) likewise.   */
/* Scales: s(row,k) = S[(row / rblk) * s_rs + (k / kblk) * s_ks], fp32 or */
/* E8M0 (2^(code-127)).  Per-tensor scaling is rblk = rows, kblk = K,     */
/* strides 0.  Non-finite codes propagate with IEEE rules.                */
/* ------------------------------------------------------------------ */

typedef struct orc_scale_desc {
    const void* s;     /* float* or uint8_t* (E8M0) */
    int32_t e8m0;      /* 1: E8M0 bytes */
    int32_t pad;
    int64_t rblk, kblk, s_rs, s_ks;
} orc_scale_desc;

/* code -> integer multiple of 2^-frac, or flags non-finite */
static int code_to_int(uint8_t c, int fmt, int64_t* out)
{
    const double v = orc_decode(c, fmt);
    if (!isfinite(v))
        return 0;
    *out = (int64_t)ldexp(v, fmt == ORC_E4M3 ? 9 : 16);   /* exact */
    return 1;
}

static double scale_at(const orc_scale_desc* d, int64_t row, int64_t k)
{
    const int64_t idx = (row / d->rblk) * d->s_rs + (k / d->kblk) * d->s_ks;
    if (d->e8m0) {
        const uint8_t c = ((const uint8_t*)d->s)[idx];
        return c == 0xFF ? NAN : ldexp(1.0, (int)c - 127);
    }
    return (double)((const float*)d->s)[idx];
}

void orc_gemm(int64_t M, int64_t N, int64_t K,
              const uint8_t* A, int64_t a_sm, int64_t a_sk, int fa, const orc_scale_desc* sa,
              const uint8_t* B, int64_t b_sn, int64_t b_sk, int fb, const orc_scale_desc* sb,
              const int64_t* rows, int64_t nrows, double* C)
{
    const int frac = (fa == ORC_E4M3 ? 9 : 16) + (fb == ORC_E4M3 ? 9 : 16);
    const int64_t kblk = sa->kblk < sb->kblk ? sa->kblk : sb->kblk;
    int64_t ia_tab[256], ib_tab[256];
    int fa_tab[256], fb_tab[256];
    int64_t ri;
    int c;
    (void)M;
    for (c = 0; c < 256; ++c) {          /* integer value of every code, once per call */
        fa_tab[c] = code_to_int((uint8_t)c, fa, &ia_tab[c]);
        fb_tab[c] = code_to_int((uint8_t)c, fb, &ib_tab[c]);
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (ri = 0; ri < nrows; ++ri) {
        const int64_t m = rows ? rows[ri] : ri;
        int64_t n;
        for (n = 0; n < N; ++n) {
            double acc = 0.0;
            int nan = 0, pinf = 0, ninf = 0;
            int64_t k0;
            for (k0 = 0; k0 < K; k0 += kblk) {
                const int64_t k1 = k0 + kblk < K ? k0 + kblk : K;
                __int128 sum = 0;
                int64_t k;
                for (k = k0; k < k1; ++k) {
                    const uint8_t ca = A[m * a_sm + k * a_sk], cb = B[n * b_sn + k * b_sk];
                    if (fa_tab[ca] && fb_tab[cb]) {
                        sum += (__int128)ia_tab[ca] * (__int128)ib_tab[cb];
                    } else {
                        const double p = orc_decode(ca, fa) * orc_decode(cb, fb);
                        if (isnan(p)) nan = 1;
                        else if (p > 0) pinf = 1;
                        else ninf = 1;
                    }
                }
                acc += ldexp((double)sum, -frac) * (scale_at(sa, m, k0) * scale_at(sb, n, k0));
            }
            if (nan || (pinf && ninf)) acc = NAN;
            else if (pinf) acc = isnan(acc) ? NAN : INFINITY;
            else if (ninf) acc = isnan(acc) ? NAN : -INFINITY;
            C[ri * N + n] = acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Bulk helpers for tests                                              */
/* ------------------------------------------------------------------ */

void orc_encode_array(const float* v, int64_t n, int fmt, int saturate, uint8_t* out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = orc_encode(v[i], fmt, saturate);
}

/* Encode every fp32 bit pattern in [lo, hi) and count the patterns whose
 * code differs from ref[] (indexed from lo); NaN codes compare equal to any
 * NaN code of the same format.  Returns the count and the first mismatch. */
int64_t orc_encode_compare_range(uint64_t lo, uint64_t hi, int fmt, const uint8_t* ref,
                                 uint64_t* first_bad)
{
    int64_t bad = 0;
    uint64_t first = UINT64_MAX;
    int64_t i;
    const int64_t n = (int64_t)(hi - lo);
#pragma omp parallel for reduction(+ : bad) reduction(min : first) schedule(static)
    for (i = 0; i < n; ++i) {
        const uint32_t b = (uint32_t)(lo + (uint64_t)i);
        float f;
        uint8_t c, r;
        memcpy(&f, &b, 4);
        c = orc_encode(f, fmt, 0);
        r = ref[i];
        if (c != r) {
            const int cn = isnan(orc_decode(c, fmt)), rn = isnan(orc_decode(r, fmt));
            if (!(cn && rn)) {
                if (lo + (uint64_t)i < first) first = lo + (uint64_t)i;
                ++bad;
            }
        }
    }
    if (first_bad) *first_bad = first;
    return bad;
}

/* Thread count of the parallel loops, for timing the oracle on one core or on
 * all of them.  Results do not depend on it: the maxima are order-free and
 * the GEMM sums integers exactly. */
void orc_set_threads(int n) {
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
