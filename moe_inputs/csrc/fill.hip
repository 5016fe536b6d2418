// Device twin of moe_inputs/rng.py: the counter-based deviate generator.
// Element c of stream `key` is a pure function of (key, c), computed with the
// same integer steps and the same two correctly rounded fp32 multiplies as
// the NumPy version, so host and device produce identical bits.
//
// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014): state = key + (c+1)*gamma,
// output = finaliser(state).  Element c takes the outputs at counters 3c,
// 3c+1, 3c+2, each cut into four 16-bit integers; D = sum of the twelve + 6 -
// 393216 is exact, z = fl32(D) * 2^-16 (exact: twelve uniforms minus 6),
// value = fl32(z * scale).
//
// Test infrastructure (input generation); holds none of the MoE layer's
// arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t splitmix64_at(uint64_t key, uint64_t c) {
    uint64_t z = key + (c + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ float deviate(uint64_t key, uint64_t c, float scale) {
    int s = 0;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const uint64_t h = splitmix64_at(key, 3 * c + q);
        s += (int)(h & 0xFFFFu) + (int)((h >> 16) & 0xFFFFu) +
             (int)((h >> 32) & 0xFFFFu) + (int)(h >> 48);
    }
    const int dd = s + 6 - 393216;
    const float z = (float)dd * (1.0f / 65536.0f);
    return z * scale;
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__global__ void fill_kernel(void* out, int bf16, uint64_t key, uint64_t start,
                            uint64_t count, float scale) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += stride) {
        const float v = deviate(key, start + i, scale);
        if (bf16)
            static_cast<uint16_t*>(out)[i] = to_bf16(v);
        else
            static_cast<float*>(out)[i] = v;
    }
}

}  // namespace

extern "C" int moe_inputs_fill_normal(void* out, int bf16, uint64_t key,
                                      uint64_t start, uint64_t count, float scale,
                                      hipStream_t stream) {
    if (count == 0) return 0;
    if (!out) return -1;
    uint64_t blocks = (count + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    fill_kernel<<<(unsigned)blocks, 256, 0, stream>>>(out, bf16, key, start, count,
                                                     scale);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
