// Combine (gate-weighted gather back to token order), its backward, and the
// permutation's backward (the sum of each token's k gradient rows).
//
// Source: FastMoE review, 제안 방법 -- the scatter/gather layout; the gather
// side returns each expert's outputs to the tokens that sent them.  Every
// kernel here is a gather keyed by dest[t,j] (one wave per token, 16-byte
// lanes), so no two lanes ever write the same element and nothing depends on
// the order of atomics: results are bit-identical run to run.
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

constexpr int U = 2;   // 16-byte vectors per lane in flight per slot

// y[t] = sum_j w[t,j] * out_perm[dest[t,j]], fp32 in slot order.  NT: the
// rows bypass the caches (out_perm larger than the MALL).
template <typename T, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(
    const T* __restrict__ out_perm, const int32_t* __restrict__ dest,
    const float* __restrict__ w, int Tn, int k, int d, T* __restrict__ y) {
    constexpr int V = Vec16<T>::N;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long t = (long)blockIdx.x * 4 + wv;
    if (t >= Tn) return;
    const int nvec = d / V;
    for (int v0 = 0; v0 < nvec; v0 += 64 * U) {
        float acc[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < V; ++q) acc[u][q] = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int r = dest[t * k + j];
            if ((unsigned)r >= (unsigned)(Tn * k)) continue;
            const float wj = w[t * k + j];
            const T* row = out_perm + (long)r * d;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * 64 + lane;
                if (v < nvec) {
                    float o[V];
                    Vec16s<T, NT>::ld(row + (long)v * V, o);
#pragma unroll
                    for (int q = 0; q < V; ++q) acc[u][q] = fmaf(wj, o[q], acc[u][q]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * 64 + lane;
            if (v < nvec) Vec16s<T, NT>::st(y + t * d + (long)v * V, acc[u]);
        }
    }
}

// d_out_perm[dest[t,j]] = w[t,j] dy[t];  dw[t,j] = <dy[t], out_perm[dest[t,j]]>.
// Slots are taken 8 at a time so dy is read once for k <= 8.
constexpr int KG = 8;

template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const T* __restrict__ dy, const T* __restrict__ out_perm,
    const int32_t* __restrict__ dest, const float* __restrict__ w, int Tn,
    int k, int d, T* __restrict__ d_out, float* __restrict__ dw) {
    constexpr int V = Vec16<T>::N;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long t = (long)blockIdx.x * 4 + wv;
    if (t >= Tn) return;
    const int nvec = d / V;
    for (int jg = 0; jg < k; jg += KG) {
        const int nj = min(KG, k - jg);
        float dot[KG];
#pragma unroll
        for (int jj = 0; jj < KG; ++jj) dot[jj] = 0.0f;
        for (int v = lane; v < nvec; v += 64) {
            float g[V];
            Vec16<T>::ld(dy + t * d + (long)v * V, g);
#pragma unroll
            for (int jj = 0; jj < KG; ++jj) {
                if (jj < nj) {
                    const int j = jg + jj;
                    const int r = dest[t * k + j];
                    if ((unsigned)r >= (unsigned)(Tn * k)) continue;
                    const float wj = w[t * k + j];
                    float o[V], s[V];
                    Vec16<T>::ld(out_perm + (long)r * d + (long)v * V, o);
#pragma unroll
                    for (int q = 0; q < V; ++q) {
                        dot[jj] = fmaf(g[q], o[q], dot[jj]);
                        s[q] = wj * g[q];
                    }
                    Vec16<T>::st(d_out + (long)r * d + (long)v * V, s);
                }
            }
        }
#pragma unroll
        for (int jj = 0; jj < KG; ++jj) {
            float v = dot[jj];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
            if (jj < nj && lane == 0) dw[t * k + jg + jj] = v;
        }
    }
}

// dx[t] (+)= sum_j dx_perm[dest[t,j]], fp32 in slot order.  NT: the rows
// bypass the caches (dx_perm larger than the MALL).
template <typename T, bool NT>
__global__ __launch_bounds__(256) void unpermute_grad_kernel(
    const T* __restrict__ dxp, const int32_t* __restrict__ dest, int Tn, int k,
    int d, int accumulate, T* __restrict__ dx) {
    constexpr int V = Vec16<T>::N;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long t = (long)blockIdx.x * 4 + wv;
    if (t >= Tn) return;
    const int nvec = d / V;
    for (int v0 = 0; v0 < nvec; v0 += 64 * U) {
        float acc[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * 64 + lane;
            if (accumulate && v < nvec) {
                Vec16<T>::ld(dx + t * d + (long)v * V, acc[u]);
            } else {
#pragma unroll
                for (int q = 0; q < V; ++q) acc[u][q] = 0.0f;
            }
        }
        float sum[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < V; ++q) sum[u][q] = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int r = dest[t * k + j];
            if ((unsigned)r >= (unsigned)(Tn * k)) continue;
            const T* row = dxp + (long)r * d;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * 64 + lane;
                if (v < nvec) {
                    float o[V];
                    Vec16s<T, NT>::ld(row + (long)v * V, o);
#pragma unroll
                    for (int q = 0; q < V; ++q) sum[u][q] += o[q];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * 64 + lane;
            if (v < nvec) {
#pragma unroll
                for (int q = 0; q < V; ++q) acc[u][q] += sum[u][q];
                Vec16s<T, NT>::st(dx + t * d + (long)v * V, acc[u]);
            }
        }
    }
}

bool rows_ok(moe_dtype dt, int d) {
    return (dt == MOE_F32 || dt == MOE_BF16) && d % 64 == 0;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_combine(const void* out_perm, const int32_t* dest,
                       const float* topk_w, int T, int k, int d, moe_dtype dt,
                       void* y, hipStream_t stream) {
    MOE_CHECK_ARG(T >= 0 && k >= 1 && d >= 64 && rows_ok(dt, d));
    MOE_CHECK_ARG((long long)T * k < (1ll << 31));
    if (T == 0) return MOE_OK;
    MOE_CHECK_ARG(out_perm && dest && topk_w && y);
    MOE_CHECK_ARG(aligned16(out_perm) && aligned16(y));
    MOE_CHECK_DEVICE();
    const bool nt = (long)T * k * d * (dt == MOE_BF16 ? 2 : 4) > kMallBytes;
    auto go = [&](auto tag, auto ntc) {
        using E = decltype(tag);
        MOE_LAUNCH("combine", stream,
            (combine_kernel<E, decltype(ntc)::value><<<cdiv(T, 4), 256, 0, stream>>>(
                static_cast<const E*>(out_perm), dest, topk_w, T, k, d, static_cast<E*>(y))));
    };
    if (dt == MOE_BF16) {
        if (nt) go(bf16_t{}, std::true_type{}); else go(bf16_t{}, std::false_type{});
    } else {
        if (nt) go(float{}, std::true_type{}); else go(float{}, std::false_type{});
    }
    return launch_status();
}

moe_status moe_combine_bwd(const void* dy, const void* out_perm,
                           const int32_t* dest, const float* topk_w, int T,
                           int k, int d, moe_dtype dt, void* d_out_perm,
                           float* d_topk_w, hipStream_t stream) {
    MOE_CHECK_ARG(T >= 0 && k >= 1 && d >= 64 && rows_ok(dt, d));
    MOE_CHECK_ARG((long long)T * k < (1ll << 31));
    if (T == 0) return MOE_OK;
    MOE_CHECK_ARG(dy && out_perm && dest && topk_w && d_out_perm && d_topk_w);
    MOE_CHECK_ARG(aligned16(dy) && aligned16(out_perm) && aligned16(d_out_perm));
    MOE_CHECK_DEVICE();
    if (dt == MOE_BF16)
        MOE_LAUNCH("combine_bwd", stream,
            combine_bwd_kernel<bf16_t><<<cdiv(T, 4), 256, 0, stream>>>(
                static_cast<const bf16_t*>(dy), static_cast<const bf16_t*>(out_perm),
                dest, topk_w, T, k, d, static_cast<bf16_t*>(d_out_perm), d_topk_w));
    else
        MOE_LAUNCH("combine_bwd", stream,
            combine_bwd_kernel<float><<<cdiv(T, 4), 256, 0, stream>>>(
                static_cast<const float*>(dy), static_cast<const float*>(out_perm),
                dest, topk_w, T, k, d, static_cast<float*>(d_out_perm), d_topk_w));
    return launch_status();
}

moe_status moe_unpermute_grad(const void* dx_perm, const int32_t* dest, int T,
                              int k, int d, moe_dtype dt, void* dx,
                              int accumulate, hipStream_t stream) {
    MOE_CHECK_ARG(T >= 0 && k >= 1 && d >= 64 && rows_ok(dt, d));
    MOE_CHECK_ARG((long long)T * k < (1ll << 31));
    if (T == 0) return MOE_OK;
    MOE_CHECK_ARG(dx_perm && dest && dx);
    MOE_CHECK_ARG(aligned16(dx_perm) && aligned16(dx));
    MOE_CHECK_DEVICE();
    const bool nt = (long)T * k * d * (dt == MOE_BF16 ? 2 : 4) > kMallBytes;
    auto go = [&](auto tag, auto ntc) {
        using E = decltype(tag);
        MOE_LAUNCH("unpermute_grad", stream,
            (unpermute_grad_kernel<E, decltype(ntc)::value><<<cdiv(T, 4), 256, 0, stream>>>(
                static_cast<const E*>(dx_perm), dest, T, k, d, accumulate,
                static_cast<E*>(dx))));
    };
    if (dt == MOE_BF16) {
        if (nt) go(bf16_t{}, std::true_type{}); else go(bf16_t{}, std::false_type{});
    } else {
        if (nt) go(float{}, std::true_type{}); else go(float{}, std::false_type{});
    }
    return launch_status();
}

}  // extern "C"
