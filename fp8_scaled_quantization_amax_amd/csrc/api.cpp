// C ABI of the fp8q library: argument validation, workspace planning and
// launch sequencing.  Every check happens before the first HIP call, so a
// rejected call has enqueued nothing.  See include/fp8q.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "fp8q.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return FP8Q_OK;
}

// Per-device cache of "is this a gfx950".
int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(FP8Q_EDEVICE, "no HIP device available");
    }
    static std::mutex mu;
    static std::vector<int> cache;   // -1 unknown, 0 no, 1 yes
    {
        std::lock_guard<std::mutex> lk(mu);
        if ((int)cache.size() > dev && cache[dev] >= 0) {
            if (cache[dev] == 1) return FP8Q_OK;
            return fail(FP8Q_EDEVICE, "device %d is not gfx950", dev);
        }
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(FP8Q_EDEVICE, "cannot query device %d", dev);
    }
    const int yes = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    {
        std::lock_guard<std::mutex> lk(mu);
        if ((int)cache.size() <= dev) cache.resize(dev + 1, -1);
        cache[dev] = yes;
    }
    if (!yes) return fail(FP8Q_EDEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
    return FP8Q_OK;
}

int launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FP8Q_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
    return FP8Q_OK;
}

// Scratch of fp8_quantize_per_tensor_noalloc, for callers that cannot
// allocate: the reduce region (partial maxima, per-block keys, completion
// counters) in device memory the library owns.  Every device the library
// runs on holds its own copy, at its own address, until the process ends.
// In host code `scratch` names a host-side stand-in, never the device
// memory: kernels and copies take the address from scratch_address().
constexpr size_t kScratchBytes = 64 * 1024;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of this device's scratch (the current device must be
// valid), looked up once per device with that device current.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(FP8Q_EDEVICE, "no HIP device available");
    }
    static std::mutex mu;
    static std::vector<void*> addr;
    std::lock_guard<std::mutex> lk(mu);
    if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return fail(FP8Q_ELAUNCH, "scratch address on device %d: %s", dev,
                        e != hipSuccess ? hipGetErrorString(e) : "null address");
        }
        addr[dev] = p;
    }
    *out = addr[dev];
    return FP8Q_OK;
}

bool valid_hp(int hp) { return hp == FP8Q_F32 || hp == FP8Q_BF16; }
bool valid_fmt(int f) { return f == FP8Q_E4M3 || f == FP8Q_E5M2; }
bool valid_flags(unsigned f) { return (f & ~(FP8Q_SATURATE | FP8Q_COUNT_OVERFLOW)) == 0; }
size_t hp_size(int hp) { return hp == FP8Q_BF16 ? 2 : 4; }

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ------------------------------------------------------------------ GEMM planning

enum Op { kNT = 0, kNN = 1, kTN = 2 };

// How one operand reaches the GEMM kernel as K-contiguous codes [R, K].
struct OperandPlan {
    bool kcontig_stored;   // stored layout already [R, K]
    bool autocast;
    bool transpose;        // pre-quantized, codes need a transpose into the workspace
    size_t codes_off, codes_bytes;
    size_t scale_off, scale_bytes;
};

struct GemmPlan {
    OperandPlan a, b;
    size_t partials_off;
    size_t total;
};

int validate_operand(const fp8q_operand* o, const char* name, int64_t K) {
    if (o == nullptr) return fail(FP8Q_EINVAL, "operand %s is NULL", name);
    if (o->data == nullptr) return fail(FP8Q_EINVAL, "operand %s has no data", name);
    if (!valid_fmt(o->format)) return fail(FP8Q_EINVAL, "operand %s: unknown format %d", name, o->format);
    const int gr = o->granularity;
    if (gr < FP8Q_PER_TENSOR || gr > FP8Q_ROWWISE)
        return fail(FP8Q_EINVAL, "operand %s: unknown granularity %d", name, gr);
    if (gr == FP8Q_ROWWISE && !o->quantized)
        return fail(FP8Q_EUNSUPPORTED, "operand %s: rowwise scaling needs pre-quantized codes (no autocast)", name);
    if ((gr == FP8Q_TILE_1x128 || gr == FP8Q_BLOCK_128x128) && K % 128 != 0)
        return fail(FP8Q_EALIGN, "operand %s: K=%lld must be a multiple of 128 for 1x128 / 128x128 scaling", name,
                    (long long)K);
    if (gr == FP8Q_MX32 && K % 32 != 0)
        return fail(FP8Q_EALIGN, "operand %s: K=%lld must be a multiple of 32 for MX32 scaling", name, (long long)K);
    if (o->quantized) {
        if (o->scale == nullptr) return fail(FP8Q_EINVAL, "operand %s has no scale", name);
        if ((uintptr_t)o->data % 16 != 0 || (o->data_kmajor && (uintptr_t)o->data_kmajor % 16 != 0))
            return fail(FP8Q_EALIGN, "operand %s: code pointers must be 16-byte aligned", name);
    } else {
        if (!valid_hp(o->hp)) return fail(FP8Q_EINVAL, "operand %s: unknown element type %d", name, o->hp);
        if (!valid_flags(o->flags)) return fail(FP8Q_EINVAL, "operand %s: unknown flags %#x", name, o->flags);
        if (o->scaling != FP8Q_CURRENT && o->scaling != FP8Q_DELAYED)
            return fail(FP8Q_EINVAL, "operand %s: unknown scaling %d", name, o->scaling);
        if (o->scaling == FP8Q_DELAYED) {
            if (gr != FP8Q_PER_TENSOR)
                return fail(FP8Q_EUNSUPPORTED, "operand %s: delayed scaling is per-tensor only", name);
            if (o->state == nullptr) return fail(FP8Q_EINVAL, "operand %s: delayed scaling needs a state", name);
        }
        if ((o->flags & FP8Q_COUNT_OVERFLOW) && !(o->scaling == FP8Q_DELAYED && gr == FP8Q_PER_TENSOR))
            return fail(FP8Q_EINVAL, "operand %s: FP8Q_COUNT_OVERFLOW needs delayed per-tensor scaling", name);
    }
    return FP8Q_OK;
}

size_t scale_bytes_for(int gran, int64_t R, int64_t K) {
    switch (gran) {
        case FP8Q_PER_TENSOR: return sizeof(float);
        case FP8Q_TILE_1x128: return (size_t)R * (size_t)(K / 128) * sizeof(float);
        case FP8Q_BLOCK_128x128: return (size_t)((R + 127) / 128) * (size_t)(K / 128) * sizeof(float);
        case FP8Q_ROWWISE: return (size_t)R * sizeof(float);
        default: return (size_t)R * (size_t)(K / 32);
    }
}

int plan_gemm(int op, int64_t M, int64_t N, int64_t K, const fp8q_operand* A, const fp8q_operand* B, GemmPlan& p) {
    if (M <= 0 || N <= 0 || K <= 0) return fail(FP8Q_EINVAL, "M, N, K must be positive");
    if (M % 16 || N % 16 || K % 16)
        return fail(FP8Q_EALIGN, "M=%lld N=%lld K=%lld must be multiples of 16", (long long)M, (long long)N,
                    (long long)K);
    int r;
    if ((r = validate_operand(A, "A", K)) != FP8Q_OK) return r;
    if ((r = validate_operand(B, "B", K)) != FP8Q_OK) return r;
    const bool amx = A->granularity == FP8Q_MX32, bmx = B->granularity == FP8Q_MX32;
    if (amx != bmx) return fail(FP8Q_EUNSUPPORTED, "MX32 scaling must be used on both operands");
    const bool arow = A->granularity == FP8Q_ROWWISE, brow = B->granularity == FP8Q_ROWWISE;
    if ((arow || brow) && !((arow || A->granularity == FP8Q_PER_TENSOR) && (brow || B->granularity == FP8Q_PER_TENSOR)))
        return fail(FP8Q_EUNSUPPORTED, "rowwise scaling combines only with rowwise or per-tensor scaling");
    // A non-empty workspace starts with the reduce region (partial maxima,
    // per-block keys, completion counters), whatever the shapes and
    // granularities: its counters then sit at the same place in every call,
    // so one zero-filled workspace can serve GEMMs of different plans in turn
    // without a later call's counters landing on codes an earlier one wrote.
    auto needs_ws = [&](const fp8q_operand* o, bool kcontig) {
        return !o->quantized || (!kcontig && o->data_kmajor == nullptr);
    };
    size_t off = 0;
    p.partials_off = 0;
    if (needs_ws(A, op != kTN) || needs_ws(B, op == kNT)) off = align_up(fp8q::kReduceWsBytes);
    auto plan_one = [&](const fp8q_operand* o, bool kcontig, int64_t R, OperandPlan& q) {
        q = OperandPlan{};
        q.kcontig_stored = kcontig;
        q.autocast = !o->quantized;
        q.transpose = o->quantized && !kcontig && o->data_kmajor == nullptr;
        if (q.autocast || q.transpose) {
            q.codes_off = off;
            q.codes_bytes = (size_t)R * (size_t)K;
            off = align_up(off + q.codes_bytes);
        }
        if (q.autocast) {
            q.scale_off = off;
            q.scale_bytes = scale_bytes_for(o->granularity, R, K);
            off = align_up(off + q.scale_bytes);
        }
    };
    plan_one(A, op != kTN, M, p.a);
    plan_one(B, op == kNT, N, p.b);
    p.total = off;
    return FP8Q_OK;
}

// Scale descriptor for the kernel, given where the scales live and the
// operand's stored orientation (blocks are indexed in the stored layout).
fp8q::GemmScale make_scale(int gran, const void* s, bool kcontig_stored, int64_t R, int64_t K) {
    fp8q::GemmScale g{};
    g.s = s;
    g.gran = gran;
    switch (gran) {
        case FP8Q_PER_TENSOR: break;
        case FP8Q_TILE_1x128: g.ld = K / 128; g.kstride = 1; g.rshift = 0; break;
        case FP8Q_ROWWISE: g.ld = 1; g.kstride = 0; g.rshift = 0; break;
        case FP8Q_BLOCK_128x128:
            g.rshift = 7;
            if (kcontig_stored) { g.ld = K / 128; g.kstride = 1; }
            else { g.ld = 1; g.kstride = (R + 127) / 128; }
            break;
        default: g.ld = K / 32; g.kstride = 1; g.rshift = 0; break;
    }
    return g;
}

// Quantize an autocast operand into the workspace as K-contiguous codes.  A
// per-tensor scale is written to the caller's scale_out when given (and read
// from there by the GEMM), else to the workspace; *scale_used reports which.
int autocast_operand(const fp8q_operand* o, bool kcontig, int64_t R, int64_t K, uint8_t* ws_codes, void* ws_scale,
                     float* partials, hipStream_t s, const void** scale_used) {
    *scale_used = ws_scale;
    fp8q::QuantArgs a{};
    a.x = o->data;
    a.hp = o->hp;
    // stored layout: [R, K] when K-contiguous, else [K, R]
    a.rows = kcontig ? R : K;
    a.cols = kcontig ? K : R;
    a.fmt = o->format;
    a.saturate = (o->flags & FP8Q_SATURATE) != 0;
    a.q = kcontig ? ws_codes : nullptr;
    a.qT = kcontig ? nullptr : ws_codes;
    a.partials = partials;
    a.nparts = fp8q::amax_partials_grid(a.rows * a.cols);
    a.keys = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(partials) + fp8q::kReduceKeysOffset);
    a.ctrs = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(partials) + fp8q::kReduceCtrOffset);
    int r;
    switch (o->granularity) {
        case FP8Q_PER_TENSOR: {
            const bool delayed = o->scaling == FP8Q_DELAYED;
            a.scheme = delayed ? fp8q::kPerTensorDelayed : fp8q::kPerTensorCurrent;
            a.state = o->state;
            a.count_overflow = delayed && (o->flags & FP8Q_COUNT_OVERFLOW) != 0;
            a.scale_out = o->scale_out != nullptr ? o->scale_out : reinterpret_cast<float*>(ws_scale);
            *scale_used = a.scale_out;
            a.amax_out = o->amax_out;
            if ((r = launched(fp8q::launch_amax_partials(a.x, a.hp, a.rows * a.cols, partials, a.nparts,
                                                         delayed ? o->state : nullptr, s),
                              "amax")) != FP8Q_OK)
                return r;
            break;
        }
        case FP8Q_TILE_1x128:
            a.scheme = kcontig ? fp8q::kTileAxis0 : fp8q::kTileAxis1;
            a.scales = reinterpret_cast<float*>(ws_scale);
            break;
        case FP8Q_BLOCK_128x128:
            a.scheme = fp8q::kBlock;
            a.scales = reinterpret_cast<float*>(ws_scale);
            break;
        default:
            a.scheme = kcontig ? fp8q::kMxAxis0 : fp8q::kMxAxis1;
            a.e8m0 = reinterpret_cast<uint8_t*>(ws_scale);
            break;
    }
    if ((r = launched(fp8q::launch_quantize(a, s), "quantize")) != FP8Q_OK) return r;
    return FP8Q_OK;
}

int gemm_entry(int op, int64_t M, int64_t N, int64_t K, const fp8q_operand* A, const fp8q_operand* B, void* C,
               int c_dtype, void* ws, size_t ws_bytes, void* stream) {
    GemmPlan p;
    int r;
    if ((r = plan_gemm(op, M, N, K, A, B, p)) != FP8Q_OK) return r;
    if (C == nullptr) return fail(FP8Q_EINVAL, "C is NULL");
    if (!valid_hp(c_dtype)) return fail(FP8Q_EINVAL, "unknown output type %d", c_dtype);
    if ((uintptr_t)C % (c_dtype == FP8Q_F32 ? 16 : 8) != 0) return fail(FP8Q_EALIGN, "C is not aligned");
    if (p.total > 0 && (ws == nullptr || ws_bytes < p.total))
        return fail(FP8Q_EWORKSPACE, "workspace of %zu bytes needed, %zu given", p.total, ws == nullptr ? 0 : ws_bytes);
    if (p.total > 0 && (uintptr_t)ws % kAlign != 0) return fail(FP8Q_EALIGN, "workspace must be 256-byte aligned");
    if ((r = check_device()) != FP8Q_OK) return r;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
    float* partials = p.total > 0 ? reinterpret_cast<float*>(wsb + p.partials_off) : nullptr;

    auto prepare = [&](const fp8q_operand* o, const OperandPlan& q, int64_t R, const uint8_t*& codes,
                       fp8q::GemmScale& sc) -> int {
        if (q.autocast) {
            const void* scale_used = nullptr;
            int rr = autocast_operand(o, q.kcontig_stored, R, K, wsb + q.codes_off, wsb + q.scale_off, partials, s,
                                      &scale_used);
            if (rr != FP8Q_OK) return rr;
            codes = wsb + q.codes_off;
            // autocast block scales are produced in the stored layout
            sc = make_scale(o->granularity, scale_used, q.kcontig_stored, R, K);
            return FP8Q_OK;
        }
        if (q.transpose) {
            int rr = launched(fp8q::launch_transpose_u8(reinterpret_cast<const uint8_t*>(o->data), K, R,
                                                        wsb + q.codes_off, s),
                              "transpose");
            if (rr != FP8Q_OK) return rr;
            codes = wsb + q.codes_off;
        } else {
            codes = reinterpret_cast<const uint8_t*>(q.kcontig_stored ? o->data
                                                                      : (o->data_kmajor ? o->data_kmajor : o->data));
        }
        sc = make_scale(o->granularity, o->scale, q.kcontig_stored, R, K);
        return FP8Q_OK;
    };

    fp8q::GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.fa = A->format; g.fb = B->format;
    g.c_dtype = c_dtype;
    g.C = C;
    if ((r = prepare(A, p.a, M, g.A, g.sa)) != FP8Q_OK) return r;
    if ((r = prepare(B, p.b, N, g.B, g.sb)) != FP8Q_OK) return r;
    if ((r = launched(fp8q::launch_gemm(g, s), "gemm")) != FP8Q_OK) return r;
    return ok();
}

}  // namespace

extern "C" {

int fp8q_abi_version(void) { return FP8Q_ABI_VERSION; }

const char* fp8q_status_string(int status) {
    switch (status) {
        case FP8Q_OK: return "ok";
        case FP8Q_EINVAL: return "invalid argument";
        case FP8Q_EALIGN: return "misaligned dimension or pointer";
        case FP8Q_EUNSUPPORTED: return "unsupported combination";
        case FP8Q_EDEVICE: return "no gfx950 device";
        case FP8Q_ELAUNCH: return "kernel launch failed";
        case FP8Q_EWORKSPACE: return "workspace too small";
        default: return "unknown status";
    }
}

const char* fp8q_last_error(void) { return g_last_error.c_str(); }

size_t fp8q_reduce_workspace_bytes(void) { return fp8q::kReduceWsBytes; }

int fp8_amax(const void* x, int hp, int64_t n, float* amax_out, void* ws, size_t ws_bytes, void* stream) {
    if (x == nullptr || amax_out == nullptr) return fail(FP8Q_EINVAL, "x and amax_out are required");
    if (n <= 0) return fail(FP8Q_EINVAL, "n must be positive");
    if (!valid_hp(hp)) return fail(FP8Q_EINVAL, "unknown element type %d", hp);
    if ((uintptr_t)x % hp_size(hp) != 0) return fail(FP8Q_EALIGN, "x is not aligned to its element type");
    if (ws == nullptr || ws_bytes < fp8q::kReduceWsBytes)
        return fail(FP8Q_EWORKSPACE, "reduce workspace of %zu bytes needed", fp8q::kReduceWsBytes);
    int r;
    if ((r = check_device()) != FP8Q_OK) return r;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    float* partials = reinterpret_cast<float*>(ws);
    // the folded form's completion chain grows with the block count: the
    // grid's 512 blocks (two per CU) keep the stream at full rate and the
    // tail short (bf16 [15872, 4096]: 22.5-23.0 us against 23.1-23.6 with
    // 1024 and 24.6-25.8 with 256 or 2048)
    const int np = fp8q::amax_partials_grid(n);
    uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
    uint32_t* keys = reinterpret_cast<uint32_t*>(wsb + fp8q::kReduceKeysOffset);
    uint32_t* ctrs = reinterpret_cast<uint32_t*>(wsb + fp8q::kReduceCtrOffset);
    if ((r = launched(fp8q::launch_amax_partials(x, hp, n, partials, np, nullptr, s, keys, ctrs, amax_out),
                      "amax")) != FP8Q_OK)
        return r;
    return ok();
}

// allowed: the flags this entry point takes (FP8Q_COUNT_OVERFLOW only where
// delayed scaling keeps the count)
static int check_quant_common(const void* x, int hp, int64_t rows, int64_t cols, int fmt, const uint8_t* q,
                              unsigned flags, unsigned allowed = FP8Q_SATURATE) {
    if (x == nullptr || q == nullptr) return fail(FP8Q_EINVAL, "x and q are required");
    if (rows <= 0 || cols <= 0) return fail(FP8Q_EINVAL, "rows and cols must be positive");
    if (!valid_hp(hp)) return fail(FP8Q_EINVAL, "unknown element type %d", hp);
    if (!valid_fmt(fmt)) return fail(FP8Q_EINVAL, "unknown format %d", fmt);
    if (!valid_flags(flags)) return fail(FP8Q_EINVAL, "unknown flags %#x", flags);
    if (flags & ~allowed) return fail(FP8Q_EINVAL, "flags %#x not taken by this call", flags & ~allowed);
    if ((uintptr_t)x % hp_size(hp) != 0) return fail(FP8Q_EALIGN, "x is not aligned to its element type");
    return FP8Q_OK;
}

// Argument checks of the per-tensor quantizer (its workspace aside).
static int check_per_tensor(const void* x, int hp, int64_t rows, int64_t cols, int fmt, int scaling,
                            const fp8q_delayed_state* state, const uint8_t* q, const float* scale_out,
                            unsigned flags) {
    int r;
    if ((r = check_quant_common(x, hp, rows, cols, fmt, q, flags, FP8Q_SATURATE | FP8Q_COUNT_OVERFLOW)) != FP8Q_OK)
        return r;
    if (scale_out == nullptr) return fail(FP8Q_EINVAL, "scale_out is required");
    if (scaling != FP8Q_CURRENT && scaling != FP8Q_DELAYED) return fail(FP8Q_EINVAL, "unknown scaling %d", scaling);
    if (scaling == FP8Q_DELAYED && state == nullptr) return fail(FP8Q_EINVAL, "delayed scaling needs a state");
    if ((flags & FP8Q_COUNT_OVERFLOW) && scaling != FP8Q_DELAYED)
        return fail(FP8Q_EINVAL, "FP8Q_COUNT_OVERFLOW needs delayed scaling (the count lives in its state)");
    return FP8Q_OK;
}

// Enqueue the per-tensor quantizer with its reduce region at ws
// (kReduceWsBytes, completion counters zero): the amax grid, then the cast.
static int enqueue_per_tensor(const void* x, int hp, int64_t rows, int64_t cols, int fmt, int scaling,
                              fp8q_delayed_state* state, uint8_t* q, uint8_t* qT, float* scale_out, float* amax_out,
                              unsigned flags, void* ws, hipStream_t s) {
    int r;
    fp8q::QuantArgs a{};
    a.x = x; a.hp = hp; a.rows = rows; a.cols = cols; a.fmt = fmt;
    a.saturate = (flags & FP8Q_SATURATE) != 0;
    a.q = q; a.qT = qT;
    float* partials = reinterpret_cast<float*>(ws);
    a.partials = partials;
    a.nparts = fp8q::amax_partials_grid(rows * cols);
    a.keys = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ws) + fp8q::kReduceKeysOffset);
    a.ctrs = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ws) + fp8q::kReduceCtrOffset);
    a.state = state;
    a.scale_out = scale_out;
    a.amax_out = amax_out;
    a.scheme = scaling == FP8Q_DELAYED ? fp8q::kPerTensorDelayed : fp8q::kPerTensorCurrent;
    a.count_overflow = (flags & FP8Q_COUNT_OVERFLOW) != 0;
    if ((r = launched(fp8q::launch_amax_partials(x, hp, rows * cols, partials, a.nparts,
                                                 scaling == FP8Q_DELAYED ? state : nullptr, s),
                      "amax")) != FP8Q_OK)
        return r;
    if ((r = launched(fp8q::launch_quantize(a, s), "quantize")) != FP8Q_OK) return r;
    return FP8Q_OK;
}

int fp8_quantize_per_tensor(const void* x, int hp, int64_t rows, int64_t cols, int fmt, int scaling,
                            fp8q_delayed_state* state, uint8_t* q, uint8_t* qT, float* scale_out, float* amax_out,
                            unsigned flags, void* ws, size_t ws_bytes, void* stream) {
    int r;
    if ((r = check_per_tensor(x, hp, rows, cols, fmt, scaling, state, q, scale_out, flags)) != FP8Q_OK) return r;
    if (ws == nullptr || ws_bytes < fp8q::kReduceWsBytes)
        return fail(FP8Q_EWORKSPACE, "reduce workspace of %zu bytes needed", fp8q::kReduceWsBytes);
    if ((r = check_device()) != FP8Q_OK) return r;
    if ((r = enqueue_per_tensor(x, hp, rows, cols, fmt, scaling, state, q, qT, scale_out, amax_out, flags, ws,
                                reinterpret_cast<hipStream_t>(stream))) != FP8Q_OK)
        return r;
    return ok();
}

int fp8_quantize_per_tensor_noalloc(const void* x, int hp, int64_t rows, int64_t cols, int fmt, int scaling,
                                    fp8q_delayed_state* state, uint8_t* q, uint8_t* qT, float* scale_out,
                                    float* amax_out, unsigned flags, void* stream) {
    int r;
    if ((r = check_per_tensor(x, hp, rows, cols, fmt, scaling, state, q, scale_out, flags)) != FP8Q_OK) return r;
    // the reduce region's size does not depend on the input (the amax grid is
    // capped at kReduceParts blocks), so every input size fits
    if (fp8q::kReduceWsBytes > kScratchBytes)
        return fail(FP8Q_EWORKSPACE, "the reduce region (%zu bytes) exceeds the library's %zu-byte scratch",
                    fp8q::kReduceWsBytes, kScratchBytes);
    if ((r = check_device()) != FP8Q_OK) return r;
    void* ws = nullptr;
    if ((r = scratch_address(&ws)) != FP8Q_OK) return r;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // The scratch keeps whatever the last call on this device left there.  Only
    // delayed scaling's completion counters must start at zero (every call
    // leaves them at zero, but a call that never ran to its end would not):
    // clear them with a kernel, which a captured graph replays.
    if (scaling == FP8Q_DELAYED &&
        (r = launched(fp8q::launch_zero_words(reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ws) +
                                                                          fp8q::kReduceCtrOffset),
                                              (int64_t)(fp8q::kReduceCtrBytes / sizeof(uint32_t)), s),
                      "clear")) != FP8Q_OK)
        return r;
    if ((r = enqueue_per_tensor(x, hp, rows, cols, fmt, scaling, state, q, qT, scale_out, amax_out, flags, ws, s)) !=
        FP8Q_OK)
        return r;
    return ok();
}

int fp8_quantize_per_tensor_sr(const void* x, int hp, int64_t rows, int64_t cols, int fmt, uint64_t seed,
                               uint64_t offset, uint8_t* q, uint8_t* qT, float* scale_out, float* amax_out,
                               unsigned flags, void* ws, size_t ws_bytes, void* stream) {
    int r;
    if ((r = check_quant_common(x, hp, rows, cols, fmt, q, flags)) != FP8Q_OK) return r;
    if (scale_out == nullptr) return fail(FP8Q_EINVAL, "scale_out is required");
    if (ws == nullptr || ws_bytes < fp8q::kReduceWsBytes)
        return fail(FP8Q_EWORKSPACE, "reduce workspace of %zu bytes needed", fp8q::kReduceWsBytes);
    if ((r = check_device()) != FP8Q_OK) return r;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    float* partials = reinterpret_cast<float*>(ws);
    const int nparts = fp8q::amax_partials_grid(rows * cols);
    if ((r = launched(fp8q::launch_amax_partials(x, hp, rows * cols, partials, nparts, nullptr, s), "amax")) !=
        FP8Q_OK)
        return r;
    if ((r = launched(fp8q::launch_quantize_sr(x, hp, rows * cols, fmt, (flags & FP8Q_SATURATE) != 0, seed, offset,
                                               partials, nparts, q, scale_out, amax_out, s),
                      "quantize")) != FP8Q_OK)
        return r;
    if (qT != nullptr && (r = launched(fp8q::launch_transpose_u8(q, rows, cols, qT, s), "transpose")) != FP8Q_OK)
        return r;
    return ok();
}

int fp8_quantize_per_tensor_rht(const void* x, int hp, int64_t rows, int64_t cols, int fmt, uint64_t seed,
                                uint8_t* q, uint8_t* qT, float* scale_out, float* amax_out, unsigned flags, void* ws,
                                size_t ws_bytes, void* stream) {
    int r;
    if ((r = check_quant_common(x, hp, rows, cols, fmt, q, flags)) != FP8Q_OK) return r;
    if (scale_out == nullptr) return fail(FP8Q_EINVAL, "scale_out is required");
    if (rows % 16 != 0 || cols % 8 != 0)
        return fail(FP8Q_EALIGN, "rows=%lld must be a multiple of 16 and cols=%lld of 8", (long long)rows,
                    (long long)cols);
    if ((uintptr_t)x % 16 != 0 || (uintptr_t)q % 8 != 0)
        return fail(FP8Q_EALIGN, "x must be 16-byte and q 8-byte aligned");
    if (ws == nullptr || ws_bytes < fp8q::kReduceWsBytes)
        return fail(FP8Q_EWORKSPACE, "reduce workspace of %zu bytes needed", fp8q::kReduceWsBytes);
    if ((r = check_device()) != FP8Q_OK) return r;
    if ((r = launched(fp8q::launch_quantize_rht(x, hp, rows, cols, fmt, (flags & FP8Q_SATURATE) != 0, seed,
                                                reinterpret_cast<float*>(ws), q, qT, scale_out, amax_out,
                                                reinterpret_cast<hipStream_t>(stream)),
                      "quantize")) != FP8Q_OK)
        return r;
    return ok();
}

int fp8q_mfma_loop_data(int blocks, int iters, int data, float* out, void* stream) {
    if (blocks <= 0 || iters <= 0 || out == nullptr)
        return fail(FP8Q_EINVAL, "blocks and iters must be positive and out non-NULL");
    if (data != 0 && data != 1) return fail(FP8Q_EINVAL, "data must be 0 (ones) or 1 (random codes)");
    if (data == 1 && iters % 8 != 0) return fail(FP8Q_EINVAL, "random-operand loop needs iters %% 8 == 0");
    int r;
    if ((r = check_device()) != FP8Q_OK) return r;
    if ((r = launched(fp8q::launch_mfma_loop(blocks, iters, data, out, reinterpret_cast<hipStream_t>(stream)),
                      "mfma loop")) != FP8Q_OK)
        return r;
    return ok();
}

int fp8q_mfma_loop(int blocks, int iters, float* out, void* stream) {
    return fp8q_mfma_loop_data(blocks, iters, 0, out, stream);
}

int fp8_quantize_tile1x128(const void* x, int hp, int64_t rows, int64_t cols, int axis, int fmt, uint8_t* q,
                           uint8_t* qT, float* scales, unsigned flags, void* stream) {
    int r;
    if ((r = check_quant_common(x, hp, rows, cols, fmt, q, flags)) != FP8Q_OK) return r;
    if (scales == nullptr) return fail(FP8Q_EINVAL, "scales is required");
    if (axis != 0 && axis != 1) return fail(FP8Q_EINVAL, "axis must be 0 or 1");
    if ((r = check_device()) != FP8Q_OK) return r;
    fp8q::QuantArgs a{};
    a.x = x; a.hp = hp; a.rows = rows; a.cols = cols; a.fmt = fmt;
    a.saturate = (flags & FP8Q_SATURATE) != 0;
    a.q = q; a.qT = qT; a.scales = scales;
    a.scheme = axis == 0 ? fp8q::kTileAxis0 : fp8q::kTileAxis1;
    if ((r = launched(fp8q::launch_quantize(a, reinterpret_cast<hipStream_t>(stream)), "quantize")) != FP8Q_OK)
        return r;
    return ok();
}

int fp8_quantize_rowwise(const void* x, int hp, int64_t rows, int64_t cols, int axis, int fmt, uint8_t* q,
                         uint8_t* qT, float* scales, unsigned flags, void* stream) {
    int r;
    if ((r = check_quant_common(x, hp, rows, cols, fmt, q, flags)) != FP8Q_OK) return r;
    if (scales == nullptr) return fail(FP8Q_EINVAL, "scales is required");
    if (axis != 0 && axis != 1) return fail(FP8Q_EINVAL, "axis must be 0 or 1");
    if (axis == 0 && qT != nullptr)
        return fail(FP8Q_EUNSUPPORTED, "rowwise axis 0 writes no transposed copy (qT must be NULL)");
    if ((uintptr_t)scales % sizeof(float) != 0) return fail(FP8Q_EALIGN, "scales is not 4-byte aligned");
    if ((r = check_device()) != FP8Q_OK) return r;
    if ((r = launched(fp8q::launch_quantize_rowwise(x, hp, rows, cols, axis, fmt, (flags & FP8Q_SATURATE) != 0, q, qT,
                                                    scales, reinterpret_cast<hipStream_t>(stream)),
                      "quantize")) != FP8Q_OK)
        return r;
    return ok();
}

int fp8_quantize_block128x128(const void* x, int hp, int64_t rows, int64_t cols, int fmt, uint8_t* q, uint8_t* qT,
                              float* scales, unsigned flags, void* stream) {
    int r;
    if ((r = check_quant_common(x, hp, rows, cols, fmt, q, flags)) != FP8Q_OK) return r;
    if (scales == nullptr) return fail(FP8Q_EINVAL, "scales is required");
    if ((r = check_device()) != FP8Q_OK) return r;
    fp8q::QuantArgs a{};
    a.x = x; a.hp = hp; a.rows = rows; a.cols = cols; a.fmt = fmt;
    a.saturate = (flags & FP8Q_SATURATE) != 0;
    a.q = q; a.qT = qT; a.scales = scales;
    a.scheme = fp8q::kBlock;
    if ((r = launched(fp8q::launch_quantize(a, reinterpret_cast<hipStream_t>(stream)), "quantize")) != FP8Q_OK)
        return r;
    return ok();
}

int fp8_quantize_mx32(const void* x, int hp, int64_t rows, int64_t cols, int axis, int fmt, uint8_t* q, uint8_t* qT,
                      uint8_t* e8m0, unsigned flags, void* stream) {
    int r;
    if ((r = check_quant_common(x, hp, rows, cols, fmt, q, flags)) != FP8Q_OK) return r;
    if (e8m0 == nullptr) return fail(FP8Q_EINVAL, "e8m0 is required");
    if (axis != 0 && axis != 1) return fail(FP8Q_EINVAL, "axis must be 0 or 1");
    if ((r = check_device()) != FP8Q_OK) return r;
    fp8q::QuantArgs a{};
    a.x = x; a.hp = hp; a.rows = rows; a.cols = cols; a.fmt = fmt;
    a.saturate = (flags & FP8Q_SATURATE) != 0;
    a.q = q; a.qT = qT; a.e8m0 = e8m0;
    a.scheme = axis == 0 ? fp8q::kMxAxis0 : fp8q::kMxAxis1;
    if ((r = launched(fp8q::launch_quantize(a, reinterpret_cast<hipStream_t>(stream)), "quantize")) != FP8Q_OK)
        return r;
    return ok();
}

size_t fp8_gemm_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, const fp8q_operand* A,
                                const fp8q_operand* B) {
    if (op < kNT || op > kTN) return (size_t)-1;
    GemmPlan p;
    if (plan_gemm(op, M, N, K, A, B, p) != FP8Q_OK) return (size_t)-1;
    return p.total;
}

int fp8_gemm_scaled_NT(int64_t M, int64_t N, int64_t K, const fp8q_operand* A, const fp8q_operand* B, void* C,
                       int c_dtype, void* ws, size_t ws_bytes, void* stream) {
    return gemm_entry(kNT, M, N, K, A, B, C, c_dtype, ws, ws_bytes, stream);
}

int fp8_gemm_scaled_NN(int64_t M, int64_t N, int64_t K, const fp8q_operand* A, const fp8q_operand* B, void* C,
                       int c_dtype, void* ws, size_t ws_bytes, void* stream) {
    return gemm_entry(kNN, M, N, K, A, B, C, c_dtype, ws, ws_bytes, stream);
}

int fp8_gemm_scaled_TN(int64_t M, int64_t N, int64_t K, const fp8q_operand* A, const fp8q_operand* B, void* C,
                       int c_dtype, void* ws, size_t ws_bytes, void* stream) {
    return gemm_entry(kTN, M, N, K, A, B, C, c_dtype, ws, ws_bytes, stream);
}

}  // extern "C"
