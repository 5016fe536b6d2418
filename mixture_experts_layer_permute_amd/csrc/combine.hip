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

constexpr int U = 2;   // 16-byte vectors per lane per slot in one batch of loads

// The k slots of a token are taken KG at a time (KG = 1, 2, 4 or 8, the
// launcher's smallest >= min(k, 8)): a lane issues the loads of all rows of a
// group before it uses any of them, so that KG * U loads are in flight per
// lane.  A slot past k or with an invalid row loads row 0 and is skipped.
template <int KG>
struct Slots {
    long off[KG];        // element offset of the slot's row
    float w[KG];         // the slot's gate weight (0 for a skipped slot; no weights: 0)
    bool ok[KG];
    __device__ __forceinline__ Slots(const int32_t* __restrict__ dest,
                                     const float* __restrict__ wt, long t, int k, int jg,
                                     int d, unsigned R) {
#pragma unroll
        for (int jj = 0; jj < KG; ++jj) {
            const int j = jg + jj;
            const long jc = t * k + min(j, k - 1);
            const int r = dest[jc];
            ok[jj] = j < k && (unsigned)r < R;
            off[jj] = ok[jj] ? (long)r * d : 0;
            w[jj] = wt && ok[jj] ? wt[jc] : 0.0f;
        }
    }
};

// y[t] = sum_j w[t,j] * out_perm[dest[t,j]], fp32 in slot order.  NT: the
// rows bypass the caches (out_perm larger than the MALL).
template <typename T, bool NT, int KG>
__global__ __launch_bounds__(256) void combine_kernel(
    const T* __restrict__ out_perm, const int32_t* __restrict__ dest,
    const float* __restrict__ w, int Tn, int k, int d, T* __restrict__ y) {
    constexpr int V = Vec16<T>::N;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long t = (long)blockIdx.x * 4 + wv;
    if (t >= Tn) return;
    const int nvec = d / V;
    const Slots<KG> s0(dest, w, t, k, 0, d, (unsigned)(Tn * k));   // the first group
    for (int v0 = 0; v0 < nvec; v0 += 64 * U) {
        float acc[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < V; ++q) acc[u][q] = 0.0f;
        for (int jg = 0; jg < k; jg += KG) {
            const Slots<KG> sl = jg == 0 ? s0 : Slots<KG>(dest, w, t, k, jg, d, (unsigned)(Tn * k));
            u32x4_t raw[KG][U];
#pragma unroll
            for (int jj = 0; jj < KG; ++jj)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    // out-of-row lanes load the row's last vector (never stored)
                    const int v = min(v0 + u * 64 + lane, nvec - 1);
                    raw[jj][u] = ld16<NT>(out_perm + sl.off[jj] + (long)v * V);
                }
#pragma unroll
            for (int jj = 0; jj < KG; ++jj) {
                if (!sl.ok[jj]) continue;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float o[V];
                    unpack16<T>(raw[jj][u], o);
#pragma unroll
                    for (int q = 0; q < V; ++q) acc[u][q] = fmaf(sl.w[jj], o[q], acc[u][q]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * 64 + lane;
            if (v < nvec) st16<NT>(y + t * d + (long)v * V, pack16<T>(acc[u]));
        }
    }
}

// d_out_perm[dest[t,j]] = w[t,j] dy[t];  dw[t,j] = <dy[t], out_perm[dest[t,j]]>.
// dy is read once per group of KG slots (once for k <= 8); each lane takes
// two of its vectors per batch of loads, in order, so each dot is the same
// fp32 sequence over the lane's vectors as one at a time.
template <typename T, int KG>
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
        const Slots<KG> sl(dest, w, t, k, jg, d, (unsigned)(Tn * k));
        float dot[KG];
#pragma unroll
        for (int jj = 0; jj < KG; ++jj) dot[jj] = 0.0f;
        for (int v0 = lane; v0 < nvec; v0 += 64 * U) {
            u32x4_t graw[U], raw[KG][U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = min(v0 + u * 64, nvec - 1);
                graw[u] = ld16<false>(dy + t * d + (long)v * V);
#pragma unroll
                for (int jj = 0; jj < KG; ++jj)
                    raw[jj][u] = ld16<false>(out_perm + sl.off[jj] + (long)v * V);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * 64;
                if (v >= nvec) break;
                float g[V];
                unpack16<T>(graw[u], g);
#pragma unroll
                for (int jj = 0; jj < KG; ++jj) {
                    if (!sl.ok[jj]) continue;
                    float o[V], s[V];
                    unpack16<T>(raw[jj][u], o);
#pragma unroll
                    for (int q = 0; q < V; ++q) {
                        dot[jj] = fmaf(g[q], o[q], dot[jj]);
                        s[q] = sl.w[jj] * g[q];
                    }
                    st16<false>(d_out + sl.off[jj] + (long)v * V, pack16<T>(s));
                }
            }
        }
#pragma unroll
        for (int jj = 0; jj < KG; ++jj) {
            float v = dot[jj];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
            if (jg + jj < k && lane == 0) dw[t * k + jg + jj] = v;
        }
    }
}

// dx[t] (+)= sum_j dx_perm[dest[t,j]], fp32 in slot order.  NT: the rows
// bypass the caches (dx_perm larger than the MALL).
template <typename T, bool NT, int KG>
__global__ __launch_bounds__(256) void unpermute_grad_kernel(
    const T* __restrict__ dxp, const int32_t* __restrict__ dest, int Tn, int k,
    int d, int accumulate, T* __restrict__ dx) {
    constexpr int V = Vec16<T>::N;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long t = (long)blockIdx.x * 4 + wv;
    if (t >= Tn) return;
    const int nvec = d / V;
    const Slots<KG> s0(dest, nullptr, t, k, 0, d, (unsigned)(Tn * k));   // the first group
    for (int v0 = 0; v0 < nvec; v0 += 64 * U) {
        u32x4_t old[U];
        if (accumulate) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = min(v0 + u * 64 + lane, nvec - 1);
                old[u] = ld16<false>(dx + t * d + (long)v * V);
            }
        }
        float sum[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < V; ++q) sum[u][q] = 0.0f;
        for (int jg = 0; jg < k; jg += KG) {
            const Slots<KG> sl = jg == 0 ? s0 : Slots<KG>(dest, nullptr, t, k, jg, d, (unsigned)(Tn * k));
            u32x4_t raw[KG][U];
#pragma unroll
            for (int jj = 0; jj < KG; ++jj)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int v = min(v0 + u * 64 + lane, nvec - 1);
                    raw[jj][u] = ld16<NT>(dxp + sl.off[jj] + (long)v * V);
                }
#pragma unroll
            for (int jj = 0; jj < KG; ++jj) {
                if (!sl.ok[jj]) continue;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float o[V];
                    unpack16<T>(raw[jj][u], o);
#pragma unroll
                    for (int q = 0; q < V; ++q) sum[u][q] += o[q];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * 64 + lane;
            if (v < nvec) {
                float acc[V];
                if (accumulate) {
                    unpack16<T>(old[u], acc);
                } else {
#pragma unroll
                    for (int q = 0; q < V; ++q) acc[q] = 0.0f;
                }
#pragma unroll
                for (int q = 0; q < V; ++q) acc[q] += sum[u][q];
                st16<NT>(dx + t * d + (long)v * V, pack16<T>(acc));
            }
        }
    }
}

// Calls f(std::integral_constant<int, KG>) for the slot group of k.
template <class F>
void with_kg(int k, F&& f) {
    if (k <= 1) f(std::integral_constant<int, 1>{});
    else if (k <= 2) f(std::integral_constant<int, 2>{});
    else if (k <= 4) f(std::integral_constant<int, 4>{});
    else f(std::integral_constant<int, 8>{});
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
        with_kg(k, [&](auto kg) {
            MOE_LAUNCH("combine", stream,
                (combine_kernel<E, decltype(ntc)::value, decltype(kg)::value>
                 <<<cdiv(T, 4), 256, 0, stream>>>(static_cast<const E*>(out_perm), dest, topk_w,
                                                  T, k, d, static_cast<E*>(y))));
        });
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
    auto go = [&](auto tag) {
        using E = decltype(tag);
        with_kg(k, [&](auto kg) {
            MOE_LAUNCH("combine_bwd", stream,
                (combine_bwd_kernel<E, decltype(kg)::value><<<cdiv(T, 4), 256, 0, stream>>>(
                    static_cast<const E*>(dy), static_cast<const E*>(out_perm), dest, topk_w, T,
                    k, d, static_cast<E*>(d_out_perm), d_topk_w)));
        });
    };
    if (dt == MOE_BF16) go(bf16_t{}); else go(float{});
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
        with_kg(k, [&](auto kg) {
            MOE_LAUNCH("unpermute_grad", stream,
                (unpermute_grad_kernel<E, decltype(ntc)::value, decltype(kg)::value>
                 <<<cdiv(T, 4), 256, 0, stream>>>(static_cast<const E*>(dx_perm), dest, T, k, d,
                                                  accumulate, static_cast<E*>(dx))));
        });
    };
    if (dt == MOE_BF16) {
        if (nt) go(bf16_t{}, std::true_type{}); else go(bf16_t{}, std::false_type{});
    } else {
        if (nt) go(float{}, std::true_type{}); else go(float{}, std::false_type{});
    }
    return launch_status();
}

}  // extern "C"
