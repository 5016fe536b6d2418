// Shared helpers of the HIP kernels: element types, 16-byte vector access,
// host-side validation and launch-status plumbing.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moe.h"

namespace moe {

// ----------------------------------------------------------------- types

typedef uint16_t bf16_t;                       // raw bf16 bits in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Round to nearest even (the gfx950 packed convert, NaN stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return (bf16_t)(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// Element load/store in fp32 for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float ld(const float* p) { return *p; }
    static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
    static constexpr int kVec = 4;             // elements per 16 bytes
};
template <> struct Elem<bf16_t> {
    static __device__ __forceinline__ float ld(const bf16_t* p) {
        return bf16_to_f32(*p);
    }
    static __device__ __forceinline__ void st(bf16_t* p, float v) {
        *p = f32_to_bf16(v);
    }
    static constexpr int kVec = 8;
};

// 16-byte vector <-> fp32 registers.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void ld(const float* p, float* o) {
        float4 v = *reinterpret_cast<const float4*>(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    static __device__ __forceinline__ void st(float* p, const float* o) {
        *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
    }
};
template <> struct Vec16<bf16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void ld(const bf16_t* p, float* o) {
        uint4 v = *reinterpret_cast<const uint4*>(p);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void st(bf16_t* p, const float* o) {
        uint4 v;
        v.x = pack_bf16x2(o[0], o[1]);
        v.y = pack_bf16x2(o[2], o[3]);
        v.z = pack_bf16x2(o[4], o[5]);
        v.w = pack_bf16x2(o[6], o[7]);
        *reinterpret_cast<uint4*>(p) = v;
    }
};

// A 16-byte vector of a row as raw bits, loaded or stored plainly or
// nontemporally (NT: the line is not kept in the caches; streaming row
// kernels whose rows exceed the 256 MB MALL use it, since the rows are touched
// once and keeping them only evicts other data).  unpack16 / pack16 convert
// between the bits and the vector's V floats.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ u32x4_t ld16(const void* p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    else
        return *reinterpret_cast<const u32x4_t*>(p);
}
template <bool NT>
__device__ __forceinline__ void st16(void* p, u32x4_t w) {
    if constexpr (NT)
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
    else
        *reinterpret_cast<u32x4_t*>(p) = w;
}
template <typename T>
__device__ __forceinline__ void unpack16(u32x4_t w, float* o) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(w[i]);
    }
}
template <typename T>
__device__ __forceinline__ u32x4_t pack16(const float* o) {
    u32x4_t w;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(o[i]);
    }
    return w;
}
constexpr long kMallBytes = 256l << 20;

// ------------------------------------------------------- wave/block scans

// Inclusive prefix sum of v over the 64 lanes of a wave, with DPP moves (no
// LDS): lanes i-1, i-2, i-4, i-8 of the same 16-lane row are added in turn
// (a source lane outside the row reads 0), which scans each row; then lane
// 15 of rows 0 and 2 is added to rows 1 and 3 (row_bcast:15), and lane 31
// (the sum of rows 0-1) to rows 2 and 3 (row_bcast:31).  Every lane of the
// wave must be active.  Integer sums, so the result does not depend on the
// order of the additions.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Exclusive prefix sum of v over the NT threads of a block (NT a multiple of
// 64, at most 1024), and the block's total in *total.  sh holds NT/64 ints
// of LDS.  Every thread of the block must call it (it has block barriers).
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
    static_assert(NT % 64 == 0 && NT <= 1024, "whole waves");
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int inc = wave_incl_scan(v);
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int t = sh[i];
        base += i < w ? t : 0;
        tot += t;
    }
    __syncthreads();                         // sh may be reused after this
    *total = tot;
    return base + inc - v;
}

// ------------------------------------------------------- debug bounds

// Debug build (-DMOE_DEBUG_BOUNDS): device-side checks of indexes that come
// from data -- caller-supplied segment offsets, routing, the tile plan --
// before the accesses they guard.  A failed check ends the kernel with a
// trap, so that a fault is reported where the bad index arises instead of
// as a stray access later.  Empty in the normal build (the library's code
// is the same with or without the checks' source lines).  For finding the
// cause of a fault; never for timing.
#ifdef MOE_DEBUG_BOUNDS
#define MOE_DASSERT(cond)                  \
    do {                                   \
        if (!(cond)) __builtin_trap();     \
    } while (0)
#else
#define MOE_DASSERT(cond) \
    do {                  \
    } while (0)
#endif

// ------------------------------------------------------------ host side

// Checks (once per device) that the current device is gfx950 and returns
// its compute-unit count, or a negative moe_status.
int device_cus();

inline bool aligned16(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// Per-device side stream for launches that overlap the caller's stream
// (kernels with no data dependence on each other).  A SideStream object
// locks the device's side stream for the duration of one call, makes it wait
// for all work queued on the caller's stream so far (fork), and makes the
// caller's stream wait for everything queued on it (join) when finished, so
// the whole call stays ordered on the caller's stream.
class SideStream {
   public:
    // allow = false: the call stays on the caller's stream (as with
    // moe_set_overlap(0)); the callers decide this from the product's shape
    explicit SideStream(hipStream_t main, bool allow = true);
    ~SideStream();
    bool ok() const { return ok_; }
    hipStream_t get() const { return side_; }
    // record mark i (0..2) on the side stream / make the caller's stream wait for it
    bool mark(int i);
    bool wait(int i);
    // the side stream waits for all work queued on the caller's stream so far
    bool follow();
    bool join();

   private:
    hipStream_t main_, side_ = nullptr;
    hipEvent_t* ev_ = nullptr;
    int dev_ = -1;
    bool ok_ = false, joined_ = false;
};

// Kernel timing hooks (see moe_profile_enable).  prof_mark(name, s, 0)
// before a launch, prof_mark(name, s, 1) after it; no-ops when disabled.
extern bool g_prof_on;
void prof_mark(const char* name, hipStream_t s, int end);

// Resolves the device address of the no-alloc FFN scratch array on the
// current device (called by moe_init).
moe_status ffn_scratch_init();

inline moe_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe

// Launch a kernel, bracketed by timing events when profiling is enabled.
#define MOE_LAUNCH(NAME, STREAM, ...)                                  \
    do {                                                              \
        if (moe::g_prof_on) moe::prof_mark(NAME, STREAM, 0);          \
        __VA_ARGS__;                                                  \
        if (moe::g_prof_on) moe::prof_mark(NAME, STREAM, 1);          \
    } while (0)

#define MOE_CHECK_ARG(cond) \
    do { if (!(cond)) return MOE_ERR_INVALID_ARG; } while (0)

#define MOE_CHECK_DEVICE()                              \
    do {                                                \
        int cus_ = moe::device_cus();                   \
        if (cus_ < 0) return (moe_status)cus_;          \
    } while (0)
