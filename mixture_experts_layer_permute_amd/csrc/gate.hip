// Gate: logits, top-k choice and gate weights (forward); gradient through
// the gate weights into the logits, the gate matrix and the tokens (backward).
//
// Source: ES-MoE review (xllm-io), 三 技术架构 / 专家级卸载与处理 -- the
// expert choice comes out of the gating network before any expert runs.
// The page prints no gate formula; the reading here is a linear gate with a
// softmax over the k selected logits (or over all E when renorm = 0).
//
// The logits decide integer routing, so they are summed in one fixed fp32
// order: increasing feature index i, each product and each sum rounded.
// This file is compiled with -ffp-contract=off so no multiply-add is fused
// for fp32 inputs; for bf16 inputs the fp32 product of two 8-bit
// significands is exact (while it stays in fp32's normal range: at or above
// 2^-126 and below overflow) and an explicit fused multiply-add gives the
// same bits.
#include <float.h>

#include <type_traits>
#include <utility>

#include "common.h"

namespace moe {
namespace {

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>): an
// unrolled loop whose index is a compile-time constant in the body.
template <class F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// Top-k order: larger logit first, the lower expert index on a tie.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// ------------------------------------------------------------ logits
// Block: 256 threads.  TE experts per block column, EPT of them per thread
// (experts tx, tx + TX, ...: rows a TX apart keep the LDS reads spread);
// the other thread dimension spans tokens (MT per thread), so every thread
// carries MT x EPT independent fp32 chains, each summed in increasing
// feature order.  Features come in chunks of GKC: the token rows are copied
// to LDS as raw 16-byte vectors (padded rows), the gate columns as fp32
// transposed to [expert][feature] so that one 16-byte read yields four
// consecutive features of one expert; the next NPF chunks are fetched into
// registers while the current one is consumed.  With few experts a thread
// has a single chain, so the chunk is long (256 features).
//
// FUSE (E <= TE, one block column): the block holds every expert of its
// tokens, so it also takes each token's top-k and gate weights (below).
template <typename T, int TE, int EPT, int MT, int GKC, int NPF, bool FUSE>
__global__ __launch_bounds__(256) void gate_logits_kernel(
    const T* __restrict__ x, const T* __restrict__ Wg,
    const float* __restrict__ bias, int Tn, int d, int E,
    float* __restrict__ logits, int k, int renorm, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
#pragma clang fp contract(off)
    constexpr int GWP = GKC + 4;               // padded LDS row of a gate column
    constexpr int TX = TE / EPT;               // threads across experts
    constexpr int TY = 256 / TX;               // threads across tokens
    constexpr int TT = MT * TY;                // tokens per block
    constexpr int V = 16 / sizeof(T);          // elements per 16-byte vector
    constexpr int VPR = GKC / V;               // vectors per token per chunk
    constexpr int XV = (TT * VPR + 255) / 256; // x vectors per thread per chunk
    constexpr int XROW = GKC * sizeof(T) + 16; // padded LDS row (bytes)
    constexpr int WV = (GKC * TE + 255) / 256; // gate elements per thread per chunk
    static_assert(TE % EPT == 0 && 256 % TX == 0, "thread layout");
    __shared__ __attribute__((aligned(16))) uint8_t xs[TT * XROW];
    __shared__ __attribute__((aligned(16))) float ws[TE * GWP];

    const int tid = threadIdx.x;
    const int tx = tid % TX, ty = tid / TX;
    const long t0 = (long)blockIdx.x * TT;
    const int e0 = blockIdx.y * TE;

    // NPF chunks in flight: chunk c lives in register slot c % NPF from its
    // fetch until it is copied to LDS
    uint4 xr_all[NPF][XV];
    float wr_all[NPF][WV];
    auto fetch = [&](int k0, uint4 (&xr)[XV], float (&wr)[WV]) {
        // Every load is issued (out-of-range ones read element 0) and the
        // value selected afterwards: a load under a branch is followed by a
        // full wait for it, which would serialise the fetch.
#pragma unroll
        for (int q = 0; q < XV; ++q) {
            const int idx = tid + 256 * q;
            const int tok = idx / VPR, c = idx % VPR;
            const long t = t0 + tok;
            const int k = k0 + c * V;
            const bool ok = idx < TT * VPR && t < Tn && k < d;
            const uint4 v = *reinterpret_cast<const uint4*>(x + (ok ? t * d + k : 0));
            xr[q] = ok ? v : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < WV; ++q) {
            const int idx = tid + 256 * q;
            const int kk = idx / TE, ee = idx % TE;
            const bool ok = idx < GKC * TE && k0 + kk < d && e0 + ee < E;
            const float v = Elem<T>::ld(Wg + (ok ? (long)(k0 + kk) * E + e0 + ee : 0));
            wr[q] = ok ? v : 0.0f;
        }
    };
    auto stash = [&](const uint4 (&xr)[XV], const float (&wr)[WV]) {
#pragma unroll
        for (int q = 0; q < XV; ++q) {
            const int idx = tid + 256 * q;
            if (idx < TT * VPR)
                *reinterpret_cast<uint4*>(xs + (idx / VPR) * XROW + (idx % VPR) * 16) = xr[q];
        }
#pragma unroll
        for (int q = 0; q < WV; ++q) {
            const int idx = tid + 256 * q;
            if (idx < GKC * TE) ws[(idx % TE) * GWP + idx / TE] = wr[q];
        }
    };

    float acc[MT][EPT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int b = 0; b < EPT; ++b) acc[m][b] = 0.0f;

    // one chunk: copy it to LDS, refill its register slot with the chunk
    // NPF further on, then run every chain over its features
    auto chunk = [&](int k0, auto slot) {
        constexpr int c = decltype(slot)::value;
        __syncthreads();
        stash(xr_all[c], wr_all[c]);
        __syncthreads();
        if (k0 + NPF * GKC < d) fetch(k0 + NPF * GKC, xr_all[c], wr_all[c]);
        const int kmax = min(GKC, d - k0);          // a multiple of V
        for (int kv = 0; kv < kmax / V; ++kv) {
            float xv[MT][V];
#pragma unroll
            for (int m = 0; m < MT; ++m)
                Vec16<T>::ld(reinterpret_cast<const T*>(xs + (ty * MT + m) * XROW + kv * 16),
                             xv[m]);
#pragma unroll
            for (int q4 = 0; q4 < V / 4; ++q4) {
                float wv[EPT][4];
#pragma unroll
                for (int b = 0; b < EPT; ++b) {
                    const float4 w4 = *reinterpret_cast<const float4*>(
                        &ws[(tx + TX * b) * GWP + kv * V + q4 * 4]);
                    wv[b][0] = w4.x; wv[b][1] = w4.y; wv[b][2] = w4.z; wv[b][3] = w4.w;
                }
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                    for (int m = 0; m < MT; ++m)
#pragma unroll
                        for (int b = 0; b < EPT; ++b) {
                            const float xq = xv[m][q4 * 4 + qq];
                            if constexpr (sizeof(T) == 2) {
                                // exact product: one rounding either way
                                acc[m][b] = __builtin_fmaf(xq, wv[b][qq], acc[m][b]);
                            } else {
                                const float pr = xq * wv[b][qq];
                                acc[m][b] = acc[m][b] + pr;
                            }
                        }
            }
        }
    };
    if constexpr (NPF == 1) {
        fetch(0, xr_all[0], wr_all[0]);
        for (int k0 = 0; k0 < d; k0 += GKC) chunk(k0, std::integral_constant<int, 0>{});
    } else {
#pragma unroll
        for (int c = 0; c < NPF; ++c) fetch(c * GKC, xr_all[c], wr_all[c]);   // zeros past d
        for (int kb = 0; kb < d; kb += NPF * GKC)
            static_for<NPF>([&](auto c) {
                if (kb + c * GKC < d) chunk(kb + c * GKC, c);
            });
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const long t = t0 + ty * MT + m;
        if (t >= Tn) continue;
#pragma unroll
        for (int b = 0; b < EPT; ++b) {
            const int e = e0 + tx + TX * b;
            if (e >= E) continue;
            float v = acc[m][b];
            if (bias) v = v + bias[e];
            logits[t * E + e] = v;
        }
    }
    if constexpr (FUSE) {
        // A token's experts sit in the TX consecutive lanes of its row (lane
        // tx holds experts tx, tx + TX, ...; e0 = 0).  k rounds of a
        // segmented wave arg-max on (value desc, index asc) pick the experts
        // in order, the winner taken out of its lane, as in topk_kernel; the
        // weights are the softmax of the k picked logits (renorm = 1) or of
        // all E, then picked (renorm = 0).  Every lane takes part (the
        // shuffles); tokens past Tn are not stored.
        static_assert(64 % TX == 0 && EPT <= 32, "token rows within a wave");
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const long t = t0 + ty * MT + m;
            const bool store = tx == 0 && t < Tn;
            float v[EPT];
            uint32_t live = 0;
#pragma unroll
            for (int b = 0; b < EPT; ++b) {
                const int e = tx + TX * b;
                float lv = acc[m][b];
                if (bias && e < E) lv = lv + bias[e];
                v[b] = lv;
                if (e < E) live |= 1u << b;
            }
            float best0 = 0.0f, den = 0.0f;
            for (int j = 0; j < k; ++j) {
                float bv = -FLT_MAX;
                int bi = 0x7fffffff;
#pragma unroll
                for (int b = 0; b < EPT; ++b) {
                    const int e = tx + TX * b;
                    if (((live >> b) & 1u) && (bi == 0x7fffffff || better(v[b], e, bv, bi))) {
                        bv = v[b];
                        bi = e;
                    }
                }
#pragma unroll
                for (int off = TX / 2; off > 0; off >>= 1) {
                    const float ov = __shfl_xor(bv, off);
                    const int oi = __shfl_xor(bi, off);
                    if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) {
                        bv = ov;
                        bi = oi;
                    }
                }
                if (bi % TX == tx) live &= ~(1u << (bi / TX));
                if (j == 0) best0 = bv;
                const float ex = expf(bv - best0);
                if (renorm) den = den + ex;
                if (store) {
                    topk_idx[t * k + j] = bi;
                    topk_w[t * k + j] = ex;        // scaled below
                }
            }
            if (!renorm) {
                float sum = 0.0f;
#pragma unroll
                for (int b = 0; b < EPT; ++b)
                    if (tx + TX * b < E) sum = sum + expf(v[b] - best0);
#pragma unroll
                for (int off = TX / 2; off > 0; off >>= 1) sum = sum + __shfl_xor(sum, off);
                den = sum;
            }
            const float inv = 1.0f / den;
            if (store)
                for (int j = 0; j < k; ++j) topk_w[t * k + j] = topk_w[t * k + j] * inv;
        }
    }
}

// ------------------------------------------------------------- top-k
// One wave per token.  Lane l holds experts l, l+64, ...  Each of the k
// rounds is a wave arg-max on (value desc, index asc); the winner is taken
// out of its lane.  Selected logits wait in LDS for the weight pass.

template <int NV>
__global__ __launch_bounds__(256) void topk_kernel(
    const float* __restrict__ logits, int Tn, int E, int k, int renorm,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    extern __shared__ float sel_val[];       // [4][k]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const long t = (long)blockIdx.x * 4 + wv;
    if (t >= Tn) return;                      // whole wave leaves together
    float* sv = sel_val + wv * k;
    float v[NV];
    uint32_t live = 0;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        const int e = lane + 64 * q;
        v[q] = e < E ? logits[t * E + e] : -FLT_MAX;
        if (e < E) live |= 1u << q;
    }
    float best0 = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = -FLT_MAX;
        int bi = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int e = lane + 64 * q;
            if ((live >> q) & 1u) {
                if (bi == 0x7fffffff || better(v[q], e, bv, bi)) {
                    bv = v[q];
                    bi = e;
                }
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) live &= ~(1u << (bi >> 6));
        if (j == 0) best0 = bv;
        if (lane == 0) {
            topk_idx[t * k + j] = bi;
            sv[j] = bv;
        }
    }
    // normaliser
    float den = 0.0f;
    if (renorm) {
        for (int j = lane; j < k; j += 64) den += expf(sv[j] - best0);
    } else {
#pragma unroll
        for (int q = 0; q < NV; ++q)
            if (lane + 64 * q < E) den += expf(v[q] - best0);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
    const float inv = 1.0f / den;
    for (int j = lane; j < k; j += 64)
        topk_w[t * k + j] = expf(sv[j] - best0) * inv;
}

// s = sum_j w_j dw_j of one token, in slot order.  The gate's dl and the
// dx kernel both take their coefficients w_j (dw_j - s) from this sum.
__device__ __forceinline__ float coef_sum(const float* __restrict__ w,
                                          const float* __restrict__ dw, int k) {
    float s = 0.0f;
    for (int j = 0; j < k; ++j) s = fmaf(w[j], dw[j], s);
    return s;
}

// dl[t,:] (the logits' gradient), one token per thread:
//   renorm=1: dl[t,idx_j] = w_j (dw_j - s), 0 elsewhere;
//   renorm=0: dl[t,e] = p_e (g_e - s), p = softmax(logits[t,:]), g_e = dw_j
//             where e = idx_j else 0.
// Blocks past the tokens' write WgT[e][i] = Wg[i][e] (a gate column
// contiguous, in the gate's own type, for the dx kernel).
template <typename T>
__global__ __launch_bounds__(256) void gate_prep_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const float* __restrict__ dw, int Tn, int E,
    int k, int renorm, float* __restrict__ dl, const T* __restrict__ Wg, int d,
    T* __restrict__ WgT, int tblocks) {
    if ((int)blockIdx.x >= tblocks) {
        const long q = (long)(blockIdx.x - tblocks) * 256 + threadIdx.x;
        if (q < (long)d * E) WgT[(q % E) * d + q / E] = Wg[q];
        return;
    }
    const long t = (long)blockIdx.x * 256 + threadIdx.x;
    if (t >= Tn) return;
    const int32_t* it = topk_idx + t * k;
    const float* wt = topk_w + t * k;
    const float* dwt = dw + t * k;
    const float s = coef_sum(wt, dwt, k);
    float* out = dl + t * E;
    if (renorm) {
        for (int e = 0; e < E; ++e) out[e] = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int e = it[j];
            if (e >= 0 && e < E) out[e] = wt[j] * (dwt[j] - s);
        }
        return;
    }
    const float* lt = logits + t * E;
    float m = -FLT_MAX;
    for (int e = 0; e < E; ++e) m = fmaxf(m, lt[e]);
    float z = 0.0f;
    for (int e = 0; e < E; ++e) z += expf(lt[e] - m);
    const float inv = 1.0f / z;
    for (int e = 0; e < E; ++e) out[e] = expf(lt[e] - m) * inv * (0.0f - s);
    for (int j = 0; j < k; ++j) {
        const int e = it[j];
        if (e >= 0 && e < E) out[e] = expf(lt[e] - m) * inv * (dwt[j] - s);
    }
}

// partial[c][i][e] = sum over the tokens of chunk c of x[t,i] * dl[t,e], on
// the fp32 matrix cores (v_mfma_f32_32x32x2_f32: features are the rows,
// experts the columns, tokens the reduction).  One wave owns 128 features
// and 32 experts of one chunk.  Lane l reads 4 consecutive features of token
// 2p + l/32 in one load and feeds feature 4*(l%32) + j to feature tile j,
// so row m of tile j is feature 4m + j.  The next DW_TS tokens are loaded
// while the current ones are multiplied.
constexpr int DW_FT = 4;        // feature tiles per wave (4 consecutive features per lane)
constexpr int DW_TS = 32;       // tokens per register batch (16 MFMA steps)

template <typename T> struct Quad;
template <> struct Quad<float> {
    typedef float4 raw;
    static __device__ __forceinline__ raw ld(const float* p) { return *reinterpret_cast<const float4*>(p); }
    static __device__ __forceinline__ float get(const raw& r, int j) {
        return j == 0 ? r.x : j == 1 ? r.y : j == 2 ? r.z : r.w;
    }
};
template <> struct Quad<bf16_t> {
    typedef uint2 raw;
    static __device__ __forceinline__ raw ld(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
    static __device__ __forceinline__ float get(const raw& r, int j) {
        const uint32_t w = j < 2 ? r.x : r.y;
        return __uint_as_float(j & 1 ? w & 0xFFFF0000u : w << 16);
    }
};

template <typename T>
__global__ __launch_bounds__(256) void gate_dwg_partial_kernel(
    const T* __restrict__ x, const float* __restrict__ dl, int Tn, int d,
    int E, int tc, int nft, float* __restrict__ partial) {
    typedef typename Quad<T>::raw raw;
    const int lane = threadIdx.x & 63;
    const int ft = blockIdx.x * 4 + (threadIdx.x >> 6);   // feature group of this wave
    if (ft >= nft) return;                                 // whole wave leaves
    const int e0 = blockIdx.y * 32;
    const long c = blockIdx.z;
    const long tbeg = c * tc;
    const long tend = min((long)Tn, tbeg + tc);
    const int col = lane & 31, half = lane >> 5;
    const int fbase = ft * 32 * DW_FT;
    const int i = fbase + 4 * col;                          // d % 4 == 0: all 4 or none
    const int e = e0 + col;

    f32x16 acc[DW_FT];
#pragma unroll
    for (int j = 0; j < DW_FT; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;

    constexpr int NP = DW_TS / 2;
    raw xa[NP];
    float da[NP];
    auto load = [&](long t0) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const long t = t0 + 2 * p + half;
            const bool tok = t < tend;
            da[p] = tok && e < E ? dl[t * E + e] : 0.0f;
            xa[p] = raw{};
            if (tok && i < d) xa[p] = Quad<T>::ld(x + t * d + i);
        }
    };
    load(tbeg);
    for (long t0 = tbeg; t0 < tend; t0 += DW_TS) {
        raw xc[NP];
        float dc[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) xc[p] = xa[p], dc[p] = da[p];
        if (t0 + DW_TS < tend) load(t0 + DW_TS);
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int j = 0; j < DW_FT; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(Quad<T>::get(xc[p], j), dc[p],
                                                             acc[j], 0, 0, 0);
    }
    // acc[j][v]: row m = (v/4)*8 + half*4 + v%4 of tile j = feature fbase + 4m + j
    if (e >= E) return;
    float* out = partial + c * (long)d * E;
#pragma unroll
    for (int j = 0; j < DW_FT; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int fi = fbase + 4 * ((v >> 2) * 8 + half * 4 + (v & 3)) + j;
            if (fi < d) out[(long)fi * E + e] = acc[j][v];
        }
}

// dWg[q] = sum over chunks c in increasing order of partial[c][q], regrouped:
// thread (g, column) sums chunks g, g+16, ... of 4 consecutive outputs, then
// the 16 group sums are added in order g = 0..15.  Same order every run.
constexpr int DW_RG = 16;

template <typename T>
__global__ __launch_bounds__(256) void gate_dwg_reduce_kernel(const float* __restrict__ partial,
                                                              int nchunk, long n,
                                                              T* __restrict__ dWg) {
    __shared__ f32x4 part[DW_RG][256 / DW_RG];
    const int g = threadIdx.x / (256 / DW_RG), cl = threadIdx.x % (256 / DW_RG);
    const long q = ((long)blockIdx.x * (256 / DW_RG) + cl) * 4;    // n % 4 == 0
    f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
    if (q < n) {
#pragma unroll 4
        for (int c = g; c < nchunk; c += DW_RG)
            s += *reinterpret_cast<const f32x4*>(partial + (long)c * n + q);
    }
    part[g][cl] = s;
    __syncthreads();
    if (g != 0 || q >= n) return;
    f32x4 tot = part[0][cl];
#pragma unroll
    for (int h = 1; h < DW_RG; ++h) tot += part[h][cl];
#pragma unroll
    for (int v = 0; v < 4; ++v) Elem<T>::st(dWg + q + v, tot[v]);
}

// dx[t,:] (+)= sum_e dl[t,e] WgT[e,:], one thread per V consecutive features
// of a token.  renorm=1 takes the k nonzero entries (coefficients
// w_j (dw_j - s) recomputed from w and dw, as gate_prep does); renorm=0 reads
// dl.  Without accumulate the old dx is not read: the sum is added to +0,
// which gives the bits that adding it to a zeroed dx gives.
template <typename T>
__global__ __launch_bounds__(256) void gate_dx_kernel(
    const T* __restrict__ WgT, const float* __restrict__ dl,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
    const float* __restrict__ dw, int Tn, int d, int E, int k, int renorm, int accumulate,
    T* __restrict__ dx) {
    constexpr int V = Vec16<T>::N;
    const int nq = d / V;
    const long q = (long)blockIdx.x * 256 + threadIdx.x;
    if (q >= (long)Tn * nq) return;
    const long t = q / nq;
    const int i0 = (int)(q - t * nq) * V;
    float acc[V];
#pragma unroll
    for (int u = 0; u < V; ++u) acc[u] = 0.0f;
    if (renorm) {
        const int32_t* it = topk_idx + t * k;
        const float* wt = topk_w + t * k;
        const float* dwt = dw + t * k;
        const float s = coef_sum(wt, dwt, k);
        for (int j = 0; j < k; ++j) {
            const int e = it[j];
            if (e < 0 || e >= E) continue;
            const float cf = wt[j] * (dwt[j] - s);
            float wg[V];
            Vec16<T>::ld(WgT + (long)e * d + i0, wg);
#pragma unroll
            for (int u = 0; u < V; ++u) acc[u] = fmaf(cf, wg[u], acc[u]);
        }
    } else {
        for (int e = 0; e < E; ++e) {
            const float cf = dl[t * E + e];
            float wg[V];
            Vec16<T>::ld(WgT + (long)e * d + i0, wg);
#pragma unroll
            for (int u = 0; u < V; ++u) acc[u] = fmaf(cf, wg[u], acc[u]);
        }
    }
    float cur[V];
    if (accumulate) {
        Vec16<T>::ld(dx + t * d + i0, cur);
    } else {
#pragma unroll
        for (int u = 0; u < V; ++u) cur[u] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < V; ++u) cur[u] = cur[u] + acc[u];
    Vec16<T>::st(dx + t * d + i0, cur);
}

// Chunks in flight per thread: when the grid is at most a couple of blocks
// per compute unit, a thread's chain is the only work its SIMD has, so the
// loads of several chunks are put in flight at once; a larger grid hides
// the fetch with other blocks and keeps its registers for occupancy.
constexpr int kNpfFew = 4, kNpfMany = 1;

// The top-k arguments of a FUSE launch; unused otherwise.
struct TopkOut {
    int k, renorm;
    int32_t* idx;
    float* w;
};

template <typename T, int TE, int EPT, int MT, int GKC, bool FUSE>
void logits_go(dim3 g, const T* xp, const T* wp, const float* bias, int Tn, int d, int E,
               float* logits, const TopkOut& o, hipStream_t s) {
    if ((long)g.x * g.y <= 2L * max(device_cus(), 1))
        MOE_LAUNCH("gate_logits", s,
            gate_logits_kernel<T, TE, EPT, MT, GKC, kNpfFew, FUSE><<<g, 256, 0, s>>>(
                xp, wp, bias, Tn, d, E, logits, o.k, o.renorm, o.idx, o.w));
    else
        MOE_LAUNCH("gate_logits", s,
            gate_logits_kernel<T, TE, EPT, MT, GKC, kNpfMany, FUSE><<<g, 256, 0, s>>>(
                xp, wp, bias, Tn, d, E, logits, o.k, o.renorm, o.idx, o.w));
}

// The logits, and with E <= 64 (every expert of a token in one block) the
// top-k and gate weights in the same launch; with more experts those come
// from topk_kernel.
template <typename T>
moe_status launch_logits(const void* x, const void* Wg, const float* bias,
                         int Tn, int d, int E, float* logits, const TopkOut& o,
                         hipStream_t s) {
    const T* xp = static_cast<const T*>(x);
    const T* wp = static_cast<const T*>(Wg);
    // tokens per block = MT * 256 / (TE / EPT); one expert per thread for
    // small E keeps the grid at Tn/32 or more blocks
    if (E <= 8)
        logits_go<T, 8, 1, 1, 256, true>(dim3(cdiv(Tn, 32), cdiv(E, 8)), xp, wp, bias, Tn, d,
                                         E, logits, o, s);
    else if (E <= 16) {
        // bf16: 2 experts per thread, 5 LDS bytes per multiply-add instead of
        // 6 (16 experts, 16384 tokens, d 2048, x in the MALL: 51 -> 43 us;
        // with x read from HBM, as in a layer step, about the same), while
        // the grid still gives every compute unit two blocks.  (fp32 rows
        // would take more registers than there are.)
        if constexpr (sizeof(T) == 2) {
            if ((long)cdiv(Tn, 32) * cdiv(E, 16) >= 2L * max(device_cus(), 1)) {
                logits_go<T, 16, 2, 1, 256, true>(dim3(cdiv(Tn, 32), cdiv(E, 16)), xp, wp, bias,
                                                  Tn, d, E, logits, o, s);
                return launch_status();
            }
        }
        logits_go<T, 16, 1, 1, 256, true>(dim3(cdiv(Tn, 16), cdiv(E, 16)), xp, wp, bias, Tn, d,
                                          E, logits, o, s);
    }
    else if (E <= 32)
        logits_go<T, 32, 2, 1, 128, true>(dim3(cdiv(Tn, 16), cdiv(E, 32)), xp, wp, bias, Tn, d,
                                          E, logits, o, s);
    else if ((long)cdiv(Tn, 64) * cdiv(E, 64) >= 2L * max(device_cus(), 1)) {
        // 2 tokens x 8 experts per thread: per 16-byte slice of features a
        // thread reads 2 token vectors and 8 gate vectors for 16 chains,
        // 2.25 LDS bytes per multiply-add instead of 4.5 with 1 x 4 (the
        // kernel was bound by those reads: 64 experts 142 -> 94 us, 128
        // experts at d 4096 1.85 -> 1.15 ms), while the grid still gives
        // every compute unit two blocks
        if (E <= 64) {
            logits_go<T, 64, 8, 2, 64, true>(dim3(cdiv(Tn, 64), 1), xp, wp, bias, Tn, d, E,
                                             logits, o, s);
        } else {
            logits_go<T, 64, 8, 2, 64, false>(dim3(cdiv(Tn, 64), cdiv(E, 64)), xp, wp, bias, Tn,
                                              d, E, logits, o, s);
        }
    } else if (E <= 64) {
        logits_go<T, 64, 4, 1, 64, true>(dim3(cdiv(Tn, 16), 1), xp, wp, bias, Tn, d, E, logits,
                                         o, s);
    } else {
        logits_go<T, 64, 4, 1, 64, false>(dim3(cdiv(Tn, 16), cdiv(E, 64)), xp, wp, bias, Tn, d,
                                          E, logits, o, s);
    }
    return launch_status();
}

moe_status launch_topk(const float* logits, int Tn, int E, int k, int renorm,
                       int32_t* idx, float* w, hipStream_t s) {
    const int blocks = cdiv(Tn, 4);
    const size_t lds = sizeof(float) * 4 * (size_t)k;
    const int nv = cdiv(E, 64);
    if (nv <= 1)
        MOE_LAUNCH("topk", s,
            topk_kernel<1><<<blocks, 256, lds, s>>>(logits, Tn, E, k, renorm, idx, w));
    else if (nv <= 2)
        MOE_LAUNCH("topk", s,
            topk_kernel<2><<<blocks, 256, lds, s>>>(logits, Tn, E, k, renorm, idx, w));
    else if (nv <= 4)
        MOE_LAUNCH("topk", s,
            topk_kernel<4><<<blocks, 256, lds, s>>>(logits, Tn, E, k, renorm, idx, w));
    else if (nv <= 8)
        MOE_LAUNCH("topk", s,
            topk_kernel<8><<<blocks, 256, lds, s>>>(logits, Tn, E, k, renorm, idx, w));
    else
        MOE_LAUNCH("topk", s,
            topk_kernel<16><<<blocks, 256, lds, s>>>(logits, Tn, E, k, renorm, idx, w));
    return launch_status();
}

// dWg work split: feature groups of 32*DW_FT, expert tiles of 32, and token
// chunks (multiples of DW_TS) so that the grid holds about 1024 waves.
struct DwgSplit {
    int nft, net, tc, nchunk;
};
DwgSplit dwg_split(int Tn, int d, int E) {
    DwgSplit z;
    z.nft = cdiv(d, 32 * DW_FT);
    z.net = cdiv(E, 32);
    const int want = max(1, 1024 / (z.nft * z.net));
    z.tc = max(DW_TS, cdiv(cdiv(max(Tn, 1), want), DW_TS) * DW_TS);
    z.nchunk = max(1, cdiv(Tn, z.tc));
    return z;
}

struct GateBwdWs {
    size_t dl, wgt, partial, total;
};

GateBwdWs gate_bwd_layout(int Tn, int d, int E) {
    GateBwdWs w;
    const size_t nchunk = (size_t)dwg_split(Tn, d, E).nchunk;
    w.dl = 0;
    w.wgt = align_up(w.dl + sizeof(float) * (size_t)Tn * E, 256);
    w.partial = align_up(w.wgt + sizeof(float) * (size_t)E * d, 256);
    w.total = align_up(w.partial + sizeof(float) * nchunk * d * E, 256);
    return w;
}

template <typename T>
moe_status launch_gate_bwd(const void* x, const void* Wg, const float* logits,
                           const int32_t* idx, const float* w, const float* dw,
                           int Tn, int d, int E, int k, int renorm, void* dx,
                           int accumulate, void* dWg, void* ws, hipStream_t s) {
    const GateBwdWs L = gate_bwd_layout(Tn, d, E);
    char* base = static_cast<char*>(ws);
    float* dl = reinterpret_cast<float*>(base + L.dl);
    T* wgt = reinterpret_cast<T*>(base + L.wgt);
    float* partial = reinterpret_cast<float*>(base + L.partial);
    const T* xp = static_cast<const T*>(x);

    const int tblocks = cdiv(Tn, 256);
    MOE_LAUNCH("gate_prep", s,
        gate_prep_kernel<T><<<tblocks + cdiv((long)d * E, 256), 256, 0, s>>>(
            logits, idx, w, dw, Tn, E, k, renorm, dl, static_cast<const T*>(Wg), d, wgt,
            tblocks));
    // dWg = x^T dl, then dx (+)= dl Wg^T, in order on the caller's stream.
    // (Forked onto the library's side stream, dWg queued ahead of the FFN
    // backward's side work whenever the two calls run on different streams,
    // as a layer runs them: the MoE-S-like step was 2% slower that way.)
    const DwgSplit z = dwg_split(Tn, d, E);
    const dim3 g(cdiv(z.nft, 4), z.net, z.nchunk);
    MOE_LAUNCH("gate_dwg_partial", s,
        gate_dwg_partial_kernel<T><<<g, 256, 0, s>>>(xp, dl, Tn, d, E, z.tc, z.nft, partial));
    const long n = (long)d * E;
    MOE_LAUNCH("gate_dwg_reduce", s,
        gate_dwg_reduce_kernel<T><<<cdiv(n / 4, 256 / DW_RG), 256, 0, s>>>(
            partial, z.nchunk, n, static_cast<T*>(dWg)));
    if (Tn > 0)     // no tokens: dWg is zero (one empty chunk), dx is empty
        MOE_LAUNCH("gate_dx", s,
            gate_dx_kernel<T><<<cdiv((long)Tn * (d / Vec16<T>::N), 256), 256, 0, s>>>(
                wgt, dl, idx, w, dw, Tn, d, E, k, renorm, accumulate ? 1 : 0,
                static_cast<T*>(dx)));
    return launch_status();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_gate_topk(const void* x, const void* Wg, const float* logit_bias,
                         int T, int d, int E, int k, int renorm, moe_dtype dt,
                         float* logits, int32_t* topk_idx, float* topk_w,
                         hipStream_t stream) {
    MOE_CHECK_ARG(T >= 0 && d >= 1 && E >= 1 && E <= 1024 && k >= 1 && k <= E);
    MOE_CHECK_ARG((long long)T * k < (1ll << 31) && (long long)T * E < (1ll << 40));
    MOE_CHECK_ARG(dt == MOE_F32 || dt == MOE_BF16);
    MOE_CHECK_ARG(d % 8 == 0);
    if (T == 0) return MOE_OK;
    MOE_CHECK_ARG(x && Wg && logits && topk_idx && topk_w);
    MOE_CHECK_ARG(aligned16(x));
    MOE_CHECK_DEVICE();
    const TopkOut o{k, renorm, topk_idx, topk_w};
    moe_status st = dt == MOE_BF16
        ? launch_logits<bf16_t>(x, Wg, logit_bias, T, d, E, logits, o, stream)
        : launch_logits<float>(x, Wg, logit_bias, T, d, E, logits, o, stream);
    if (st != MOE_OK || E <= 64) return st;    // E <= 64: top-k in the logits launch
    return launch_topk(logits, T, E, k, renorm, topk_idx, topk_w, stream);
}

size_t moe_gate_bwd_workspace_bytes(int T, int d, int E) {
    if (T < 0 || d < 1 || E < 1) return 0;
    return gate_bwd_layout(T, d, E).total;
}

moe_status moe_gate_topk_bwd(const void* x, const void* Wg, const float* logits,
                             const int32_t* topk_idx, const float* topk_w,
                             const float* d_topk_w, int T, int d, int E, int k,
                             int renorm, moe_dtype dt, void* dx, int accumulate,
                             void* dWg, void* ws, size_t ws_bytes, hipStream_t stream) {
    MOE_CHECK_ARG(T >= 0 && d >= 1 && E >= 1 && E <= 1024 && k >= 1 && k <= E);
    MOE_CHECK_ARG((long long)T * k < (1ll << 31));
    MOE_CHECK_ARG(dt == MOE_F32 || dt == MOE_BF16);
    const int vec = dt == MOE_BF16 ? 8 : 4;
    MOE_CHECK_ARG(d % vec == 0);
    MOE_CHECK_ARG(Wg && dWg);
    // T = 0: nothing of the tokens is read (empty tensors may have null
    // pointers); dWg is still written (zeros)
    MOE_CHECK_ARG(T == 0 || (x && logits && topk_idx && topk_w && d_topk_w && dx));
    MOE_CHECK_ARG(aligned16(x));
    MOE_CHECK_ARG(dx == nullptr || aligned16(dx));
    if (ws_bytes < moe_gate_bwd_workspace_bytes(T, d, E) || !ws) return MOE_ERR_WORKSPACE;
    MOE_CHECK_DEVICE();
    return dt == MOE_BF16
        ? launch_gate_bwd<bf16_t>(x, Wg, logits, topk_idx, topk_w, d_topk_w, T, d,
                                  E, k, renorm, dx, accumulate, dWg, ws, stream)
        : launch_gate_bwd<float>(x, Wg, logits, topk_idx, topk_w, d_topk_w, T, d,
                                 E, k, renorm, dx, accumulate, dWg, ws, stream);
}

}  // extern "C"
