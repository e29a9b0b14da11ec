// Pieces shared by the persistent GEMM kernels (per-tensor / MX and
// block-scaled): operand tile geometry, the LDS swizzle and fragment read,
// direct-to-LDS load plans, waits and barriers, the tile walk.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BK = 128;
constexpr int kThreads = 256;
constexpr int kTileBytes = BM * BK;     // the A tile of one stage (B takes BN * BK)

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

// The same loads in compact form for the buffer (bounds-checked) load: the
// chunk swizzle of instruction u depends on u only through its parity, so a
// lane keeps two offsets - row base (row0 + 64 wave + l/8) * K plus the
// swizzled chunk for even and for odd u - and instruction u adds u * 8 * K.
// Nothing is clamped: rows past the matrix edge give offsets past the
// buffer's end, which the buffer load returns as zeros.
struct DmaB {
    uint32_t e, o;
};

__device__ __forceinline__ DmaB dmab_plan(int64_t K, int64_t row0, int wave) {
    const int l = threadIdx.x & 63;
    const int64_t rb = (row0 + wave * 64 + (l >> 3)) * K;
    const int ce = (l & 7) ^ (l >> 4), co = (l & 7) ^ (4 + (l >> 4));
    return DmaB{(uint32_t)(rb + ce * 16), (uint32_t)(rb + co * 16)};
}

// The same plan for rows rowbase + l/8 (+ 8 u for instruction u).
__device__ __forceinline__ DmaB dmab_rows(int64_t K, int64_t rowbase) {
    const int l = threadIdx.x & 63;
    const int64_t rb = (rowbase + (l >> 3)) * K;
    const int ce = (l & 7) ^ (l >> 4), co = (l & 7) ^ (4 + (l >> 4));
    return DmaB{(uint32_t)(rb + ce * 16), (uint32_t)(rb + co * 16)};
}

// Logical tile lg -> (tm, tn): groups of 8 M-tiles, N-tiles walked inside a group.
__device__ __forceinline__ void tile_coords(int lg, int ntm, int ntn, int& tm, int& tn) {
    constexpr int GM = 8;
    const int per_group = GM * ntn;
    const int group = lg / per_group;
    const int first_m = group * GM;
    const int gsize = ntm - first_m < GM ? ntm - first_m : GM;
    const int in_group = lg % per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// Raw buffer descriptor over [p, p + bytes) (bytes clamped to 2^32 - 1) for
// the buffer form of the direct-to-LDS load: per-lane 32-bit offset in a
// VGPR, per-step K offset in an SGPR, so no 64-bit address arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int64_t bytes) {
    const int64_t n = bytes < 0xFFFFFFFFll ? bytes : 0xFFFFFFFFll;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)(uint32_t)n, 0x00020000);
}

__device__ __forceinline__ void dma_one(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint8_t* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

}  // namespace fp8q
