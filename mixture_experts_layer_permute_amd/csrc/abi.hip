// Library-wide entry points: status text, version, device check.
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>

#include "common.h"

namespace moe {

namespace {
constexpr int kMaxDevices = 64;
// 0 = not checked yet, >0 = CU count of a gfx950 device, <0 = moe_status.
int g_dev_state[kMaxDevices];
}  // namespace

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    int s = __atomic_load_n(&g_dev_state[dev], __ATOMIC_ACQUIRE);
    if (s != 0) return s;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        s = MOE_ERR_UNSUPPORTED;
    } else {
        s = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
    }
    __atomic_store_n(&g_dev_state[dev], s, __ATOMIC_RELEASE);
    return s;
}

// ------------------------------------------------------- side streams
namespace {
struct SideState {
    std::mutex mu;
    hipStream_t s = nullptr;
    hipEvent_t ev[4] = {};   // 0 fork, 1..2 marks, 3 join
    bool made = false;
};
SideState g_side[kMaxDevices];
}  // namespace

std::atomic<int> g_overlap{1};

SideStream::SideStream(hipStream_t main, bool allow) : main_(main) {
    if (!allow || !g_overlap.load(std::memory_order_relaxed) || g_prof_on)
        return;                                                // caller's stream only
    int d = -1;
    if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDevices) return;
    SideState& st = g_side[d];
    std::unique_lock<std::mutex> lk(st.mu);
    if (!st.made) {
        // (a failure leaves what was made for the next attempt to complete)
        if (!st.s && hipStreamCreateWithFlags(&st.s, hipStreamNonBlocking) != hipSuccess) {
            st.s = nullptr;
            return;
        }
        for (int i = 0; i < 4; ++i)
            if (!st.ev[i] &&
                hipEventCreateWithFlags(&st.ev[i], hipEventDisableTiming) != hipSuccess) {
                st.ev[i] = nullptr;
                return;
            }
        st.made = true;
    }
    if (hipEventRecord(st.ev[0], main_) != hipSuccess ||
        hipStreamWaitEvent(st.s, st.ev[0], 0) != hipSuccess)
        return;
    side_ = st.s;
    ev_ = st.ev;
    ok_ = true;
    dev_ = d;
    lk.release();                 // held until the destructor
}

bool SideStream::mark(int i) {
    return ok_ && i >= 1 && i <= 2 && hipEventRecord(ev_[i], side_) == hipSuccess;
}

bool SideStream::wait(int i) {
    return ok_ && i >= 1 && i <= 2 && hipStreamWaitEvent(main_, ev_[i], 0) == hipSuccess;
}

bool SideStream::follow() {
    return ok_ && hipEventRecord(ev_[0], main_) == hipSuccess &&
           hipStreamWaitEvent(side_, ev_[0], 0) == hipSuccess;
}

bool SideStream::join() {
    if (!ok_ || joined_) return ok_;
    joined_ = true;
    return hipEventRecord(ev_[3], side_) == hipSuccess &&
           hipStreamWaitEvent(main_, ev_[3], 0) == hipSuccess;
}

SideStream::~SideStream() {
    if (dev_ < 0) return;
    if (ok_) join();
    g_side[dev_].mu.unlock();
}

// ------------------------------------------------------------ timing
bool g_prof_on = false;

namespace {
struct ProfRec {
    const char* name;
    hipEvent_t a, b;
};
ProfRec* g_prof = nullptr;
int g_prof_cap = 0, g_prof_n = 0;
bool g_prof_open = false;
}  // namespace

void prof_mark(const char* name, hipStream_t s, int end) {
    if (!end) {
        if (g_prof_n >= g_prof_cap) return;
        g_prof[g_prof_n].name = name;
        (void)hipEventRecord(g_prof[g_prof_n].a, s);
        g_prof_open = true;
    } else {
        if (!g_prof_open) return;
        (void)hipEventRecord(g_prof[g_prof_n].b, s);
        g_prof_open = false;
        ++g_prof_n;
    }
}

// ------------------------------------------------- attainable MFMA rate
// Every wave issues iters rounds of four independent bf16 32x32x16 matrix
// instructions on register operands (no memory traffic), so the kernel's
// rate is what the matrix cores sustain at the clock they run at.  Lane 0
// of each wave stores one sum so that nothing is optimised away.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        a[q] = (__bf16)(0.001f * (float)(lane + q));
        b[q] = (__bf16)(0.002f * (float)(lane - q));
    }
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[c][v];
    if (lane == 0) out[blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = s;
}
// The same loop on operands that change with every instruction: each wave
// holds eight A and eight B fragments of random bf16 values (a counter hash
// of block, wave, lane and slot, |v| < 1) and cycles through them, so the
// matrix cores see operand bits toggle as in a GEMM on random data.  On this
// part the matrix instructions' sustained rate depends on the data (power
// and clock): constant operands run faster than random ones.
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x7feb352du;
    h ^= h >> 15;
    h *= 0x846ca68bu;
    h ^= h >> 16;
    return h;
}
__global__ __launch_bounds__(256) void mfma_loop_random_kernel(int rounds, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const uint32_t seed = ((uint32_t)blockIdx.x * 256u + threadIdx.x) * 256u;
    bf16x8 a[8], b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            // a float in (-1, 1): random mantissa bits, exponents of 2^-1 .. 2^-8
            const uint32_t ha = mix32(seed + (uint32_t)(s * 16 + q));
            const uint32_t hb = mix32(seed + (uint32_t)(s * 16 + 8 + q) + 0x9e3779b9u);
            a[s][q] = (__bf16)__uint_as_float((ha & 0x807fffffu) | ((126u - (ha >> 28 & 7u)) << 23));
            b[s][q] = (__bf16)__uint_as_float((hb & 0x807fffffu) | ((126u - (hb >> 28 & 7u)) << 23));
        }
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
    for (int i = 0; i < rounds; ++i) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(u + c) & 7], b[(u + 3 * c + 1) & 7],
                                                                acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[c][v];
    if (lane == 0) out[blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = s;
}

}  // namespace moe

extern "C" {

moe_status moe_mfma_loop(int blocks, int iters, float* out, size_t out_floats,
                         hipStream_t stream) {
    using namespace moe;
    MOE_CHECK_ARG(blocks >= 1 && iters >= 1 && out);
    MOE_CHECK_ARG(out_floats >= (size_t)blocks * 4);
    MOE_CHECK_DEVICE();
    MOE_LAUNCH("mfma_loop", stream,
               mfma_loop_kernel<<<blocks, 256, 0, stream>>>(iters, out));
    return launch_status();
}

moe_status moe_mfma_loop_random(int blocks, int iters, float* out, size_t out_floats,
                                hipStream_t stream) {
    using namespace moe;
    MOE_CHECK_ARG(blocks >= 1 && iters >= 8 && iters % 8 == 0 && out);
    MOE_CHECK_ARG(out_floats >= (size_t)blocks * 4);
    MOE_CHECK_DEVICE();
    MOE_LAUNCH("mfma_loop_random", stream,
               mfma_loop_random_kernel<<<blocks, 256, 0, stream>>>(iters / 8, out));
    return launch_status();
}

void moe_profile_disable(void) {
    using namespace moe;
    g_prof_on = false;
    for (int i = 0; i < g_prof_cap; ++i) {
        (void)hipEventDestroy(g_prof[i].a);
        (void)hipEventDestroy(g_prof[i].b);
    }
    delete[] g_prof;
    g_prof = nullptr;
    g_prof_cap = g_prof_n = 0;
    g_prof_open = false;
}

moe_status moe_profile_enable(int capacity) {
    using namespace moe;
    if (capacity < 1) return MOE_ERR_INVALID_ARG;
    moe_profile_disable();
    g_prof = new (std::nothrow) ProfRec[capacity];
    if (!g_prof) return MOE_ERR_INVALID_ARG;
    for (int i = 0; i < capacity; ++i) {
        if (hipEventCreate(&g_prof[i].a) != hipSuccess ||
            hipEventCreate(&g_prof[i].b) != hipSuccess) {
            g_prof_cap = i;
            moe_profile_disable();
            return MOE_ERR_HIP;
        }
    }
    g_prof_cap = capacity;
    g_prof_n = 0;
    g_prof_on = true;
    return MOE_OK;
}

void moe_profile_reset(void) {
    moe::g_prof_n = 0;
    moe::g_prof_open = false;
}

int moe_profile_count(void) { return moe::g_prof_n; }

moe_status moe_profile_get(int i, const char** name, float* ms) {
    using namespace moe;
    if (i < 0 || i >= g_prof_n || !name || !ms) return MOE_ERR_INVALID_ARG;
    if (hipEventSynchronize(g_prof[i].b) != hipSuccess) return MOE_ERR_HIP;
    if (hipEventElapsedTime(ms, g_prof[i].a, g_prof[i].b) != hipSuccess) return MOE_ERR_HIP;
    *name = g_prof[i].name;
    return MOE_OK;
}


const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported device or mode (gfx950 only)";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int moe_abi_version(void) { return 7; }

moe_status moe_set_overlap(int enable) {
    moe::g_overlap.store(enable != 0 ? 1 : 0, std::memory_order_relaxed);
    return MOE_OK;
}

moe_status moe_init(int device) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_HIP;
    if (device != cur && hipSetDevice(device) != hipSuccess) return MOE_ERR_HIP;
    int r = moe::device_cus();
    // the no-alloc entry point's scratch address on this device
    if (r >= 0) r = moe::ffn_scratch_init();
    if (device != cur) (void)hipSetDevice(cur);
    return r < 0 ? (moe_status)r : MOE_OK;
}

}  // extern "C"
