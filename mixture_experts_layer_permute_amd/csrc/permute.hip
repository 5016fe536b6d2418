// Permute: stable counting sort of the (token, slot) pairs by expert, then
// the row copy into contiguous, unpadded per-expert segments.
//
// Sources: ES-MoE review (xllm-io), 三 技术架构 / 专家级卸载与处理 and
// 四 核心创新 -- tokens are handed to their target experts in sequence
// instead of through a dense dispatch mask, which is where the memory saving
// comes from; FastMoE review, 제안 방법 -- a scatter/gather layout that
// batches each expert's inputs together.
//
// Four kernels:
//   hist    per block of tokens, count pairs per expert (LDS counters)
//   scan    per expert, exclusive scan of the block counts -> block bases
//           (with at most kFuseScanBlocks blocks the scatter sums them itself)
//   scatter per block, stable ranks inside the block from wave ballots
//           (ranks never depend on the order atomics land in), dest and src
//   copy    x_perm[dest[t,j]] = x[t]: each token row is read once and
//           written k times, 16 bytes per lane
// Counts use LDS atomics (order-independent sums); every position is a pure
// function of topk_idx, so the result is identical run to run.
#include "common.h"

namespace moe {
namespace {

constexpr int PERM_ENT = 1024;    // target (token, slot) pairs per block
constexpr int kFuseScanBlocks = 64;

inline int tokens_per_block(int k) { return k >= PERM_ENT ? 1 : PERM_ENT / k; }

__global__ __launch_bounds__(256) void perm_hist_kernel(
    const int32_t* __restrict__ idx, int Tn, int E, int k, int tpb, int nblk,
    int32_t* __restrict__ block_counts) {
    extern __shared__ int hist[];
    const int b = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
    __syncthreads();
    const long beg = (long)b * tpb * k;
    const long end = min((long)Tn, (long)(b + 1) * tpb) * k;
    for (long i = beg + threadIdx.x; i < end; i += 256) {
        const int e = idx[i];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256)
        block_counts[(long)e * nblk + b] = hist[e];
}

// Exclusive scan of one expert's block counts (one workgroup per expert).
__global__ __launch_bounds__(256) void perm_scan_kernel(
    const int32_t* __restrict__ block_counts, int nblk,
    int32_t* __restrict__ block_base, int32_t* __restrict__ counts) {
    __shared__ int sh[4];
    const int e = blockIdx.x;
    const int32_t* in = block_counts + (long)e * nblk;
    int32_t* out = block_base + (long)e * nblk;
    const int per = (nblk + 255) / 256;
    const int lo = threadIdx.x * per, hi = min(nblk, lo + per);
    int s = 0;
    for (int i = lo; i < hi; ++i) s += in[i];
    int total;
    int run = block_excl_scan<256>(s, sh, &total);   // DPP wave scans, then the 4 wave sums
    if (threadIdx.x == 0) counts[e] = total;
    for (int i = lo; i < hi; ++i) {
        const int v = in[i];
        out[i] = run;
        run += v;
    }
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// Lanes holding the same expert id as this lane (valid lanes only).
__device__ __forceinline__ uint64_t match_peers(int e, bool valid, int nbits) {
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    return peers;
}

// FUSED (at most kFuseScanBlocks blocks): no perm_scan launch; each block
// sums the block counts itself, all of them for counts[e] (block 0 stores
// those) and those of the blocks before it for its own bases.  Integer sums,
// so the result is the same as through perm_scan.
template <bool FUSED>
__global__ __launch_bounds__(256) void perm_scatter_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ counts,
    const int32_t* __restrict__ block_counts, const int32_t* __restrict__ block_base,
    int Tn, int E, int k, int tpb, int nblk, int nbits, int32_t* __restrict__ offsets,
    int32_t* __restrict__ dest, int32_t* __restrict__ src) {
    extern __shared__ int sm[];
    int* offs = sm;                  // [E+1]
    int* wcnt = sm + E + 1;          // [4][E]
    int* cnt_l = sm + 5 * E + 1;     // FUSED: [E] counts, [E] this block's bases
    int* base_l = cnt_l + E;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int b = blockIdx.x;

    if constexpr (FUSED) {
        for (int e = tid; e < E; e += 256) {
            const int32_t* bc = block_counts + (long)e * nblk;
            int before = 0, all = 0;
            for (int q = 0; q < nblk; ++q) {
                const int v = bc[q];
                before += q < b ? v : 0;
                all += v;
            }
            cnt_l[e] = all;
            base_l[e] = before;
            if (b == 0) counts[e] = all;
        }
        __syncthreads();
    }
    const int32_t* cnt = FUSED ? cnt_l : counts;
    // expert offsets: exclusive scan of counts (E <= 1024: up to 4
    // consecutive experts per thread, then a block scan of the threads' sums)
    {
        __shared__ int sh[4];
        const int per = (E + 255) / 256;
        const int lo = min(E, tid * per), hi = min(E, lo + per);
        int s = 0;
        for (int e = lo; e < hi; ++e) s += cnt[e];
        int total;
        int run = block_excl_scan<256>(s, sh, &total);
        for (int e = lo; e < hi; ++e) {
            offs[e] = run;
            run += cnt[e];
        }
        if (tid == 0) offs[E] = total;
    }
    for (int q = tid; q < 4 * E; q += 256) wcnt[q] = 0;
    __syncthreads();
    if (b == 0)
        for (int e = tid; e <= E; e += 256) offsets[e] = offs[e];

    const long beg = (long)b * tpb * k;
    const long end = min((long)Tn, (long)(b + 1) * tpb) * k;
    const int nchunk = (int)((end - beg + 63) / 64);
    const int cpw = (nchunk + 3) / 4;
    const int c0 = w * cpw, c1 = min(nchunk, c0 + cpw);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // pass 1: per-wave counts
    for (int c = c0; c < c1; ++c) {
        const long i = beg + (long)c * 64 + lane;
        int e = -1;
        if (i < end) e = idx[i];
        const bool valid = e >= 0 && e < E;
        const uint64_t peers = match_peers(valid ? e : 0, valid, nbits);
        if (valid && (peers & lt) == 0) wcnt[w * E + e] += popc64(peers);
    }
    __syncthreads();
    // per-wave bases: exclusive scan over the 4 waves
    for (int e = tid; e < E; e += 256) {
        int run = 0;
        for (int q = 0; q < 4; ++q) {
            const int v = wcnt[q * E + e];
            wcnt[q * E + e] = run;
            run += v;
        }
    }
    __syncthreads();
    // pass 2: ranks
    for (int c = c0; c < c1; ++c) {
        const long i = beg + (long)c * 64 + lane;
        int e = -1;
        if (i < end) e = idx[i];
        const bool valid = e >= 0 && e < E;
        const uint64_t peers = match_peers(valid ? e : 0, valid, nbits);
        if (valid) {
            const int pos = offs[e] + (FUSED ? base_l[e] : block_base[(long)e * nblk + b]) +
                            wcnt[w * E + e] + popc64(peers & lt);
            MOE_DASSERT((unsigned)pos < (unsigned)(Tn * k));
            dest[i] = pos;
            src[pos] = (int)(i / k);
        } else if (i < end) {
            dest[i] = -1;            // an expert id outside [0,E): no row
        }
        __builtin_amdgcn_wave_barrier();
        if (valid && (peers & lt) == 0) wcnt[w * E + e] += popc64(peers);
        __builtin_amdgcn_wave_barrier();
    }
}

// x_perm[dest[t,j], :] = x[t, :].  One wave per token; 16-byte lanes; the
// row is loaded once and stored k times.  The four vectors a lane carries
// are named values, not an array: an array read back inside the runtime-k
// loop is placed in LDS by the compiler, with a full wait after every load.
template <typename T>
__global__ __launch_bounds__(256) void perm_copy_kernel(
    const T* __restrict__ x, const int32_t* __restrict__ dest, int Tn, int d,
    int k, T* __restrict__ x_perm) {
    constexpr int V = 16 / sizeof(T);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long t = (long)blockIdx.x * 4 + w;
    if (t >= Tn) return;
    const int nvec = d / V;
    const uint4* xr = reinterpret_cast<const uint4*>(x + t * d);
    for (int v0 = 0; v0 < nvec; v0 += 64 * 4) {
        const int va = v0 + lane, vb = va + 64, vc = va + 128, vd = va + 192;
        // out-of-row lanes load the row's last vector (never stored)
        const uint4 b0 = xr[min(va, nvec - 1)];
        const uint4 b1 = xr[min(vb, nvec - 1)];
        const uint4 b2 = xr[min(vc, nvec - 1)];
        const uint4 b3 = xr[min(vd, nvec - 1)];
        for (int j = 0; j < k; ++j) {
            const int r = dest[t * k + j];
            if ((unsigned)r >= (unsigned)(Tn * k)) continue;
            uint4* outr = reinterpret_cast<uint4*>(x_perm + (long)r * d);
            if (va < nvec) outr[va] = b0;
            if (vb < nvec) outr[vb] = b1;
            if (vc < nvec) outr[vc] = b2;
            if (vd < nvec) outr[vd] = b3;
        }
    }
}

struct PermWs {
    size_t counts, base, total;
};

PermWs perm_layout(int Tn, int E, int k) {
    const int tpb = tokens_per_block(k);
    const size_t nblk = (size_t)cdiv(Tn, tpb);
    PermWs w;
    w.counts = 0;
    w.base = align_up(sizeof(int32_t) * nblk * E, 256);
    w.total = align_up(w.base + sizeof(int32_t) * nblk * E, 256);
    return w;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_permute_workspace_bytes(int T, int E, int k) {
    if (T < 0 || E < 1 || k < 1) return 0;
    return perm_layout(T, E, k).total;
}

moe_status moe_permute(const int32_t* topk_idx, const void* x, int T, int d,
                       int E, int k, moe_dtype dt, int32_t* counts,
                       int32_t* offsets, int32_t* dest, int32_t* src,
                       void* x_perm, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    MOE_CHECK_ARG(T >= 0 && d >= 1 && E >= 1 && E <= 1024 && k >= 1 && k <= E);
    MOE_CHECK_ARG((long long)T * k < (1ll << 31));
    MOE_CHECK_ARG(dt == MOE_F32 || dt == MOE_BF16);
    const int vec = dt == MOE_BF16 ? 8 : 4;
    MOE_CHECK_ARG(d % vec == 0);
    MOE_CHECK_ARG(counts && offsets);
    // x_perm == NULL: routing only (the expert GEMMs gather rows of x by src)
    MOE_CHECK_ARG(T == 0 || (topk_idx && dest && src && (!x_perm || x)));
    MOE_CHECK_ARG(T == 0 || !x_perm || (aligned16(x) && aligned16(x_perm)));
    if (ws_bytes < moe_permute_workspace_bytes(T, E, k) || (!ws && T > 0))
        return MOE_ERR_WORKSPACE;
    MOE_CHECK_DEVICE();
    const PermWs L = perm_layout(T, E, k);
    const int tpb = tokens_per_block(k);
    const int nblk = cdiv(T, tpb);
    char* base = static_cast<char*>(ws);
    int32_t* bcounts = reinterpret_cast<int32_t*>(base + L.counts);
    int32_t* bbase = reinterpret_cast<int32_t*>(base + L.base);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;

    if (T == 0) {
        // empty input: counts = 0, offsets = 0, from one scatter block that
        // sums no block counts and ranks no pairs
        MOE_LAUNCH("perm_scatter", stream,
            perm_scatter_kernel<true><<<1, 256, sizeof(int) * (7 * (size_t)E + 1), stream>>>(
                topk_idx, counts, bcounts, bbase, 0, E, k, tpb, 0, nbits, offsets, dest, src));
        return launch_status();
    }
    MOE_LAUNCH("perm_hist", stream,
        perm_hist_kernel<<<nblk, 256, sizeof(int) * (size_t)E, stream>>>(
            topk_idx, T, E, k, tpb, nblk, bcounts));
    if (nblk <= kFuseScanBlocks) {
        MOE_LAUNCH("perm_scatter", stream,
            perm_scatter_kernel<true><<<nblk, 256, sizeof(int) * (7 * (size_t)E + 1), stream>>>(
                topk_idx, counts, bcounts, bbase, T, E, k, tpb, nblk, nbits, offsets, dest, src));
    } else {
        MOE_LAUNCH("perm_scan", stream,
            perm_scan_kernel<<<E, 256, 0, stream>>>(bcounts, nblk, bbase, counts));
        MOE_LAUNCH("perm_scatter", stream,
            perm_scatter_kernel<false><<<nblk, 256, sizeof(int) * (5 * (size_t)E + 1), stream>>>(
                topk_idx, counts, bcounts, bbase, T, E, k, tpb, nblk, nbits, offsets, dest, src));
    }
    if (!x_perm) return launch_status();
    if (dt == MOE_BF16)
        MOE_LAUNCH("perm_copy", stream,
            perm_copy_kernel<bf16_t><<<cdiv(T, 4), 256, 0, stream>>>(
                static_cast<const bf16_t*>(x), dest, T, d, k, static_cast<bf16_t*>(x_perm)));
    else
        MOE_LAUNCH("perm_copy", stream,
            perm_copy_kernel<float><<<cdiv(T, 4), 256, 0, stream>>>(
                static_cast<const float*>(x), dest, T, d, k, static_cast<float*>(x_perm)));
    return launch_status();
}

}  // extern "C"
