// Grouped GEMM over ragged expert segments: the expert FFN forward and
// backward.
//
// Sources: FastMoE review (nubint.ai), 제안 방법 -- a dedicated expert FFN
// whose linear module runs the experts' linear layers in parallel over a
// layout that batches each expert's inputs; ES-MoE review (xllm-io),
// 三 技术架构 / 专家级卸载与处理 and 自适应卸载 -- no dispatch mask and no
// padding to a capacity: each expert's segment is exactly as long as its
// token count.
//
// Two product shapes cover all six GEMMs of a layer:
//  RAGGED_M  C[rows of segment e, N] = A[rows, K] . B_e[K, N]   (x W1, a W2,
//            dO W2^T, dH W1^T).  Work unit = (expert, 256-row tile, N tile);
//            a device-side prefix of per-expert tile counts maps the flat
//            block index to its unit, so no row is padded and the host never
//            reads the routing.
//  RAGGED_K  C_e[M, N] = A[seg e, M]^T . B[seg e, N]   (dW1, dW2, dW3).  The
//            reduction runs over the expert's rows; units are dealt out
//            heaviest expert first (longest-processing-time order), the same
//            greedy idea the ES-MoE review applies to expert placement
//            (三 技术架构 / 动态专家放置), here applied across compute units.
//            An expert with no rows writes zeros.
//
// bf16 path: block tile 256x256, 8 waves of 64 (4x2, 64x128 each), gfx950
// MFMA v_mfma_f32_32x32x16_bf16 with fp32 accumulators.  Operands go from
// HBM straight into an LDS ring (two 64-deep stages for RAGGED_M, four
// 32-deep ones for RAGGED_K, or two 64-deep ones over long segments);
// K-contiguous operands are read as
// 16-byte fragments, M/N-contiguous ones with the transposing LDS read.
// Products that are a few rounds of workgroups run as a full-tile launch
// and a partial-tile launch; independent launches may run on a side stream.
// fp32 path (tiny fp32 workload): a plain LDS-tiled FMA kernel with the same
// tile scheduler and epilogues.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"

// Scratch of moe_expert_ffn_fwd_noalloc: the forward's tile plan (four int32
// arrays of E+1 entries, 256-byte aligned; 17 KiB at E = 1024) in a
// library-owned array, one copy per GPU, held until the process ends.  Host
// code never passes `scratch` itself to a kernel (in host code the name is a
// host-side stand-in): it uses the device address that hipGetSymbolAddress
// returned for the current device.
constexpr size_t kFfnScratchBytes = 32u << 10;
static __device__ __align__(256) unsigned char scratch[kFfnScratchBytes];

namespace moe {
namespace {

enum { RAGGED_M = 0, RAGGED_K = 1 };
enum { KMAJ = 0, MNMAJ = 1 };   // operand storage: row-of-K contiguous or M/N contiguous

template <typename T>
struct GemmArgs {
    const T* A;
    long lda;
    const T* B;
    long ldb;
    long bstride;        // elements between experts' B (RAGGED_M)
    const T* B2;         // DUAL: second weight; KSPLIT: weight for k >= Ksplit
    const int32_t* offsets;      // [E+1]
    const int32_t* tile_prefix;  // [E+1] per-expert prefix of M tiles (RAGGED_M)
    const int32_t* order;        // [E] experts heaviest first (RAGGED_K)
    const int32_t* full_prefix;  // [E+1] per-expert prefix of full M tiles
    const int32_t* part_list;    // experts with a partial last tile; count at [E]
    int E, M, N, K, Ksplit;
    int nM, nN;
    int part_mode;       // RAGGED_M: 0 all row tiles, 1 full tiles only,
                         // 2 partial tiles cut into BM-row slices
    int bm_plan;         // row tile of the plan (part_mode 2)
    int xcd_run;         // logical tiles per XCD run (block -> tile remap)
    // Row gather of the A operand (NULL: none).  RAGGED_M: row r of the
    // expert-ordered A is A[gather[r]]; RAGGED_K: reduction row r (the
    // segment's rows) is A[gather[r]].  A then has gather_rows rows.
    const int32_t* gather;
    long gather_rows;
    // RAGGED_K work items (NULL: one item per expert, in `order`): x expert,
    // y first row, z rows, w partial slot (-1: the item is the expert's
    // whole segment and its tile is finished in the epilogue; >= 0: one
    // chunk of a split segment, stored in fp32 at partial + w * partial_ld).
    const int4* items;
    const int32_t* item_count;
    int item_max;        // host bound on the work items (grid size)
    int k_grouped;       // RAGGED_K tile order inside an item: grouped (1) or
                         // column by column (0), chosen by the launcher
    int round16;         // RAGGED_M tile order in rounds of 16 x 16 tiles (1), or
                         // groups of GROUP_M row tiles (0), chosen by the launcher
    float* partial;
    long partial_ld;
};

// ------------------------------------------------------------ epilogues

// fp32 tensors: the library erff / expf and an IEEE division.
__device__ __forceinline__ float gelu_exact(float z) {
    return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_grad_exact(float z) {
    const float cdf = 0.5f * (1.0f + erff(z * 0.70710678118654752f));
    const float pdf = 0.3989422804014327f * expf(-0.5f * z * z);
    return cdf + z * pdf;
}
__device__ __forceinline__ float sigmoid_exact(float z) { return 1.0f / (1.0f + expf(-z)); }

// bf16 tensors (results rounded to 8 significant bits): the standard normal
// CDF from the rational approximation of erf in Abramowitz & Stegun,
// Handbook of Mathematical Functions, formula 7.1.26 (after Hastings):
// erfc(x) ~= t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),
// t = 1 / (1 + p x), x >= 0, absolute error at most 1.5e-7.  With
// x = |z| / sqrt(2) the factor exp(-x^2) = exp(-z^2/2) is also the unscaled
// normal density, so one hardware exp2 serves both Phi(z) and phi(z).
struct NormCP {
    float cdf, pdf;
};
__device__ __forceinline__ NormCP norm_fast(float z) {
    // p/sqrt(2) takes |z| straight to 1 + p x; the coefficients are halved
    // (exactly, a power of two) so that the sum is Q(|z|) = erfc(x) / 2.
    constexpr float PS = 0.3275911f * 0.70710678118654752f;
    constexpr float H1 = 0.5f * 0.254829592f, H2 = 0.5f * -0.284496736f,
                    H3 = 0.5f * 1.421413741f, H4 = 0.5f * -1.453152027f,
                    H5 = 0.5f * 1.061405429f;
    const float t = __builtin_amdgcn_rcpf(fmaf(fabsf(z), PS, 1.0f));
    const float q = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, H5, H4), H3), H2), H1);
    const float g = __builtin_amdgcn_exp2f(z * z * -0.72134752044448170f);  // e^(-z^2/2)
    const float tail = q * g;                                                 // Q(|z|)
    return {z >= 0.0f ? 1.0f - tail : tail, 0.3989422804014327f * g};
}
__device__ __forceinline__ float sigmoid_fast(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

template <typename T>
__device__ __forceinline__ float sigmoid_f(float z) {
    if constexpr (sizeof(T) == 2) return sigmoid_fast(z);
    else return sigmoid_exact(z);
}

// GeLU(z) and GeLU'(z) from one evaluation of the normal CDF and density.
template <typename T>
__device__ __forceinline__ void gelu_and_grad(float z, float& a, float& g) {
    if constexpr (sizeof(T) == 2) {
        const NormCP n = norm_fast(z);
        a = z * n.cdf;
        g = fmaf(z, n.pdf, n.cdf);
    } else {
        a = gelu_exact(z);
        g = gelu_grad_exact(z);
    }
}
// The SwiGLU factors the backward needs: s1 = H3 * SiLU'(H1), s3 = SiLU(H1).
template <typename T>
__device__ __forceinline__ void swiglu_saved(float h1, float h3, float& s1, float& s3) {
    const float sg = sigmoid_f<T>(h1);
    s3 = h1 * sg;
    s1 = h3 * sg * (1.0f + h1 * (1.0f - sg));
}

// Epilogue functors.  vec8(e, row, col, v) finishes 8 consecutive outputs.
// Functors that read memory split that into pre8() (issue the loads, return
// the raw data) and vec8p(..., pre), so the bf16 kernel can put all loads of
// a slab in flight before it consumes the first; kPre says which do.
struct NoPre {};

template <typename T>
struct EpiStore {            // C[e*cstride + row*ldc + col] = v
    static constexpr bool kPre = false;
    typedef NoPre Pre;
    __device__ __forceinline__ Pre pre8(int, long, int) const { return {}; }
    T* C;
    long ldc, cstride;
    __device__ __forceinline__ void operator()(int e, long row, int col, float v) const {
        Elem<T>::st(C + e * cstride + row * ldc + col, v);
    }
    __device__ __forceinline__ void vec8(int e, long row, int col, const float* v) const {
        Vec16<T>::st(C + e * cstride + row * ldc + col, v);
    }
    __device__ __forceinline__ void vec8p(int e, long row, int col, const float* v,
                                          const Pre&) const {
        vec8(e, row, col, v);
    }
};

// The forward saves what the backward's activation derivative needs, not
// the pre-activation: GeLU'(H) for GeLU, [H3 SiLU'(H1) | SiLU(H1)] for
// SwiGLU, each computed from the fp32 accumulator, so the backward epilogue
// is one (two) multiplications per element.
template <typename T>
struct EpiGeluFwd {          // S = GeLU'(v) (saved for the backward), A = GeLU(v)
    static constexpr bool kPre = false;
    typedef NoPre Pre;
    __device__ __forceinline__ Pre pre8(int, long, int) const { return {}; }
    T* S;
    T* A;
    long ld;
    __device__ __forceinline__ void operator()(int, long row, int col, float v) const {
        float a, g;
        gelu_and_grad<T>(v, a, g);
        Elem<T>::st(S + row * ld + col, g);
        Elem<T>::st(A + row * ld + col, a);
    }
    __device__ __forceinline__ void vec8(int, long row, int col, const float* v) const {
        float a[8], g[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) gelu_and_grad<T>(v[q], a[q], g[q]);
        Vec16<T>::st(S + row * ld + col, g);
        Vec16<T>::st(A + row * ld + col, a);
    }
    __device__ __forceinline__ void vec8p(int e, long row, int col, const float* v,
                                          const Pre&) const {
        vec8(e, row, col, v);
    }
};

template <typename T>
struct EpiSwigluFwd {        // S = [H3 SiLU'(H1) | SiLU(H1)] per row, A = SiLU(H1) H3
    static constexpr bool kPre = false;
    typedef NoPre Pre;
    __device__ __forceinline__ Pre pre8(int, long, int) const { return {}; }
    T* S;
    T* A;
    long f;
    __device__ __forceinline__ void operator()(int, long row, int col, float v1,
                                               float v3) const {
        float s1, s3;
        swiglu_saved<T>(v1, v3, s1, s3);
        Elem<T>::st(S + row * 2 * f + col, s1);
        Elem<T>::st(S + row * 2 * f + f + col, s3);
        Elem<T>::st(A + row * f + col, s3 * v3);
    }
    __device__ __forceinline__ void vec8(int, long row, int col, const float* v1,
                                         const float* v3) const {
        float s1[8], s3[8], a[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            swiglu_saved<T>(v1[q], v3[q], s1[q], s3[q]);
            a[q] = s3[q] * v3[q];
        }
        Vec16<T>::st(S + row * 2 * f + col, s1);
        Vec16<T>::st(S + row * 2 * f + f + col, s3);
        Vec16<T>::st(A + row * f + col, a);
    }
};

__device__ __forceinline__ void unpack_bf16x8(const uint4& r, float* o) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        o[2 * q] = __uint_as_float(w[q] << 16);
        o[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
}

template <typename T>
struct EpiAcc {              // C[e*cstride + row*ldc + col] += v: one fp32 sum, one rounding
    static constexpr bool kPre = sizeof(T) == 2;
    struct Pre {
        uint4 c;                    // 8 bf16 of C, raw (bf16 kernels only)
    };
    __device__ __forceinline__ Pre pre8(int e, long row, int col) const {
        static_assert(sizeof(T) == 2, "prefetching epilogue is for bf16 tensors");
        return {*reinterpret_cast<const uint4*>(C + e * cstride + row * ldc + col)};
    }
    T* C;
    long ldc, cstride;
    __device__ __forceinline__ void operator()(int e, long row, int col, float v) const {
        T* q = C + e * cstride + row * ldc + col;
        Elem<T>::st(q, Elem<T>::ld(q) + v);
    }
    __device__ __forceinline__ void vec8(int e, long row, int col, const float* v) const {
        float c[8];
        T* q = C + e * cstride + row * ldc + col;
        Vec16<T>::ld(q, c);
#pragma unroll
        for (int i = 0; i < Vec16<T>::N; ++i) c[i] += v[i];
        Vec16<T>::st(q, c);
    }
    __device__ __forceinline__ void vec8p(int e, long row, int col, const float* v,
                                          const Pre& pr) const {
        float c[8];
        unpack_bf16x8(pr.c, c);
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] += v[i];
        Vec16<T>::st(C + e * cstride + row * ldc + col, c);
    }
};

template <typename T>
struct EpiGeluBwd {          // dH = dA * S, S = GeLU'(H) saved by the forward
    static constexpr bool kPre = true;
    struct Pre {
        uint4 s;                    // 8 bf16 of S, raw (bf16 kernels only)
    };
    __device__ __forceinline__ Pre pre8(int, long row, int col) const {
        static_assert(sizeof(T) == 2, "prefetching epilogue is for bf16 tensors");
        return {*reinterpret_cast<const uint4*>(S + row * ld + col)};
    }
    const T* S;
    T* dH;
    long ld;
    __device__ __forceinline__ void operator()(int, long row, int col, float v) const {
        Elem<T>::st(dH + row * ld + col, v * Elem<T>::ld(S + row * ld + col));
    }
    __device__ __forceinline__ void vec8(int, long row, int col, const float* v) const {
        float g[8], o[8];
        Vec16<T>::ld(S + row * ld + col, g);
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = v[q] * g[q];
        Vec16<T>::st(dH + row * ld + col, o);
    }
    __device__ __forceinline__ void vec8p(int, long row, int col, const float* v,
                                          const Pre& pr) const {
        float g[8], o[8];
        unpack_bf16x8(pr.s, g);
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = v[q] * g[q];
        Vec16<T>::st(dH + row * ld + col, o);
    }
};

template <typename T>
struct EpiSwigluBwd {        // dH1 = dA * S1, dH3 = dA * S3 (S saved by the forward)
    static constexpr bool kPre = true;
    struct Pre {
        uint4 s1, s3;               // 8 bf16 each of S1 and S3, raw (bf16 kernels only)
    };
    __device__ __forceinline__ Pre pre8(int, long row, int col) const {
        static_assert(sizeof(T) == 2, "prefetching epilogue is for bf16 tensors");
        return {*reinterpret_cast<const uint4*>(S + row * 2 * f + col),
                *reinterpret_cast<const uint4*>(S + row * 2 * f + f + col)};
    }
    const T* S;
    T* dH;
    long f;
    __device__ __forceinline__ void operator()(int, long row, int col, float v) const {
        Elem<T>::st(dH + row * 2 * f + col, v * Elem<T>::ld(S + row * 2 * f + col));
        Elem<T>::st(dH + row * 2 * f + f + col, v * Elem<T>::ld(S + row * 2 * f + f + col));
    }
    __device__ __forceinline__ void vec8(int, long row, int col, const float* v) const {
        float s1[8], s3[8], o1[8], o3[8];
        Vec16<T>::ld(S + row * 2 * f + col, s1);
        Vec16<T>::ld(S + row * 2 * f + f + col, s3);
#pragma unroll
        for (int q = 0; q < 8; ++q) o1[q] = v[q] * s1[q], o3[q] = v[q] * s3[q];
        Vec16<T>::st(dH + row * 2 * f + col, o1);
        Vec16<T>::st(dH + row * 2 * f + f + col, o3);
    }
    __device__ __forceinline__ void vec8p(int, long row, int col, const float* v,
                                          const Pre& pr) const {
        float s1[8], s3[8], o1[8], o3[8];
        unpack_bf16x8(pr.s1, s1);
        unpack_bf16x8(pr.s3, s3);
#pragma unroll
        for (int q = 0; q < 8; ++q) o1[q] = v[q] * s1[q], o3[q] = v[q] * s3[q];
        Vec16<T>::st(dH + row * 2 * f + col, o1);
        Vec16<T>::st(dH + row * 2 * f + f + col, o3);
    }
};

// ------------------------------------------------------ tile decoding

struct TileInfo {
    int e;          // expert
    long r0;        // RAGGED_M: first global row of the tile
    int rows;       // RAGGED_M: valid rows in the tile
    int m0, n0;     // RAGGED_K: tile origin in C_e; n0 also used by RAGGED_M
    long kbeg;      // RAGGED_K: first row of the segment
    int klen;       // reduction length
    int pslot;      // RAGGED_K: partial slot of a split segment's chunk, or -1
    bool live;
};

// Block -> tile.  Workgroups are dealt to the 8 XCDs round-robin (block b
// runs on XCD b % 8), and each XCD has its own L2.  The flat block index is
// therefore re-mapped so that each XCD receives runs of XCD_RUN consecutive
// logical tiles, and logical tiles are ordered so that a run shares
// operands: RAGGED_M in groups of GROUP_M row tiles (all N tiles of the
// group before the next group), RAGGED_K expert by expert, row tiles
// fastest.  Grids are padded to a multiple of 8 * XCD_RUN.  A RAGGED_M
// launch covers all row tiles, only the full ones, or only the partial last
// tiles of the experts, cut into BM-row slices (part_mode 0, 1, 2).
constexpr int NXCD = 8;
constexpr int GROUP_M = 8;

__device__ __forceinline__ int xcd_logical(int b, int run) {
    const int x = b % NXCD, j = b / NXCD;
    return ((j / run) * NXCD + x) * run + (j % run);
}

template <int MODE, int BM, int BN, typename T>
__device__ __forceinline__ TileInfo decode_tile(const GemmArgs<T>& p) {
    TileInfo ti;
    const int L = xcd_logical(blockIdx.x, p.xcd_run);
    if (MODE == RAGGED_M) {
        const int sub = p.part_mode == 2 ? p.bm_plan / BM : 1;   // slices per partial tile
        const int total = p.part_mode == 0 ? p.tile_prefix[p.E]
                        : p.part_mode == 1 ? p.full_prefix[p.E]
                                           : p.part_list[p.E] * sub;
        int mt, nt;
        if (p.round16) {
            // rounds of 256 tiles, 16 row tiles x 16 column tiles, row tiles
            // outer: XCD x takes rows (x / 4) * 8 .. + 8 and columns
            // (x % 4) * 4 .. + 4 of its round (runs of 32), so a round reads
            // 16 weight panels once and the next round reuses its 16 row panels
            const int round = L >> 8, within = L & 255;
            const int x = within >> 5, j = within & 31;
            const int ncb = (p.nN + 15) >> 4;
            const int rb = round / ncb;
            mt = rb * 16 + (x >> 2) * 8 + (j & 7);
            nt = (round - rb * ncb) * 16 + (x & 3) * 4 + (j >> 3);
            ti.live = mt < total && nt < p.nN;
        } else {
            ti.live = L < total * p.nN;
            const int per_group = GROUP_M * p.nN;
            const int first = (L / per_group) * GROUP_M;
            const int gm = min(GROUP_M, total - first);
            const int w = L % per_group;
            mt = first + w % gm;
            nt = w / gm;
        }
        if (!ti.live) return ti;
        if (p.part_mode == 2) {
            const int e = p.part_list[mt / sub];
            const int seg0 = p.offsets[e], seg1 = p.offsets[e + 1];
            const int nfull = (seg1 - seg0) / p.bm_plan;
            const int lo = nfull * p.bm_plan + (mt % sub) * BM;   // slice start in segment
            ti.e = e;
            ti.r0 = (long)seg0 + lo;
            ti.rows = min(BM, seg1 - seg0 - lo);
            if (ti.rows <= 0) {
                ti.live = false;
                return ti;
            }
        } else {
            const int32_t* pre = p.part_mode == 0 ? p.tile_prefix : p.full_prefix;
            int lo = 0, hi = p.E;                 // largest e with pre[e] <= mt
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (pre[mid] <= mt) lo = mid; else hi = mid;
            }
            ti.e = lo;
            const int seg0 = p.offsets[lo], seg1 = p.offsets[lo + 1];
            ti.r0 = (long)seg0 + (long)(mt - pre[lo]) * BM;
            ti.rows = (int)min((long)BM, (long)seg1 - ti.r0);
            MOE_DASSERT(seg0 >= 0 && seg0 <= seg1 && ti.rows > 0);
        }
        ti.n0 = nt * BN;
        ti.m0 = 0;
        ti.kbeg = 0;
        ti.klen = p.K;
        ti.pslot = -1;
    } else {
        const int per = p.nM * p.nN;
        const int es = L / per, rem = L % per;
        if (p.k_grouped) {
            // groups of GROUP_M row tiles, every column tile of a group, row
            // tiles fastest: a run of 32 on one XCD is 8 row x 4 column tiles
            const int first = (rem / (GROUP_M * p.nN)) * GROUP_M;
            const int gm = min(GROUP_M, p.nM - first);
            const int w = rem - first * p.nN;
            ti.m0 = (first + w % gm) * BM;
            ti.n0 = (w / gm) * BN;
        } else {
            ti.m0 = (rem % p.nM) * BM;
            ti.n0 = (rem / p.nM) * BN;
        }
        ti.r0 = 0;
        ti.rows = BM;
        if (p.items) {
            ti.live = es < *p.item_count;
            if (!ti.live) return ti;
            const int4 it = p.items[es];
            MOE_DASSERT(it.x >= 0 && it.x < p.E && it.y >= 0 && it.z >= 0);
            ti.e = it.x;
            ti.kbeg = it.y;
            ti.klen = it.z;
            ti.pslot = it.w;
        } else {
            ti.live = es < p.E;
            if (!ti.live) return ti;
            ti.e = p.order ? p.order[es] : es;
            ti.kbeg = p.offsets[ti.e];
            ti.klen = p.offsets[ti.e + 1] - p.offsets[ti.e];
            ti.pslot = -1;
        }
    }
    return ti;
}

// =====================================================================
// bf16 MFMA kernel
// =====================================================================
// Operand tiles go from HBM straight into LDS with buffer_load_dwordx4 ...
// lds (each wave instruction fills 1 KB: lane l's 16 bytes land at base +
// 16*l), through a ring of NSTG stages of BK reduction steps, with no
// register staging.  The descriptor's byte range covers exactly the valid
// part of the tile, so lanes past a ragged segment end, the end of the
// reduction, a partial tile or the allocation read zeros, with no branch.
constexpr uint32_t OOB = 0x80000000u;    // an offset past any descriptor range
// Rows of the reduction-row gather map held in LDS at a time (RAGGED_K); a
// power of two.
constexpr int KG_CHUNK = 4096;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;


// K-major stage tile: rows of BK bf16 (CH = BK/8 chunks of 16 B), chunk c of
// row r stored at chunk c ^ ((r ^ r/CH) mod CH), so that the rows one
// fragment read touches spread over distinct banks.
template <int CH>
__device__ __forceinline__ int swzk(int r, int c) {
    constexpr int L = CH == 4 ? 2 : 3;
    static_assert(CH == 4 || CH == 8, "32 or 64 reduction steps per stage");
    return r * (CH * 16) + ((c ^ ((r ^ (r >> L)) & (CH - 1))) << 4);
}
// M/N-major stage tile: BK rows of ROWS elements; chunk c of row k is
// stored at chunk c ^ 4*(k mod 4), which spreads the four rows a transposing
// read touches over distinct banks.
template <int ROWS>
__device__ __forceinline__ int mnoff(int k, int c) {
    return k * ROWS * 2 + ((c ^ ((k & 3) << 2)) << 4);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// The four words of a raw buffer resource: base address, stride 0,
// num_records = nbytes (clamped at 0), and word 3 = 0x00020000 (data format
// 32 bits, no swizzle), the usual raw-access setting on gfx9 parts.  Reads at
// offsets >= nbytes return zero.
__device__ __forceinline__ i32x4_t rsrc_words(const bf16_t* base, long nbytes) {
    const uint64_t a = (uint64_t)base;
    const uint32_t n = nbytes <= 0 ? 0u : (uint32_t)nbytes;
    // the words are wave-uniform; readfirstlane states it where the
    // compiler cannot see it (operand fields set on two paths)
    return i32x4_t{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                   __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu)),
                   __builtin_amdgcn_readfirstlane((int)n), 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}
// One wave-wide 16-byte-per-lane load from a buffer straight into LDS: lane
// l's bytes at voff land at lds + 16*l.  Issued from inline assembly so that
// the compiler does not tie every later LDS read to its completion; callers
// wait on vmcnt themselves (stage_barrier) before reading the stage.
__device__ __forceinline__ void lds_dma16(i32x4_t rs, uint32_t voff, uint32_t lds) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rs)
        : "memory", "m0");
}

template <int ROWS, int LAY, int NT, int BK>
struct DmaOperand {
    static constexpr int NW = NT / 64;
    static constexpr int CH = BK / 8;                     // K-major: chunks per row
    static constexpr int TILE = ROWS * BK * 2;            // bytes per stage
    static constexpr int NLOAD = TILE / 1024 / NW;        // 1 KB loads per wave
    static_assert(TILE % (1024 * NW) == 0, "tile/wave mismatch");
    static_assert(LAY == KMAJ || ROWS >= 128, "M/N-major swizzle needs 16 chunks per row");
    static_assert(TILE >= 1024 * NW, "every wave loads at least 1 KB per stage");
    const bf16_t* P;
    long ld;
    int row_lim;
    long k_lim;
    long span;               // K-major: bytes from P that hold valid rows
    uint32_t off[NLOAD];

    __device__ __forceinline__ void init(const bf16_t* P_, long ld_, int row_lim_,
                                         long k_lim_) {
        P = P_;
        ld = ld_;
        row_lim = row_lim_;
        k_lim = k_lim_;
        span = (long)row_lim_ * ld_ * 2;
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            const int blk = w + NW * i;                    // 1 KB block of the stage
            if (LAY == KMAJ) {
                constexpr int L = CH == 4 ? 2 : 3;
                const int row = blk * (64 / CH) + lane / CH;
                const int c = (lane % CH) ^ ((row ^ (row >> L)) & (CH - 1));
                off[i] = (uint32_t)(row * ld * 2 + c * 16);
            } else {
                constexpr int NC = ROWS / 8;               // chunks per row
                constexpr int RB = 1024 / (ROWS * 2);      // rows per block
                const int k = blk * RB + lane / NC;
                const int c = (lane % NC) ^ ((k & 3) << 2);
                off[i] = c * 8 < row_lim ? (uint32_t)(k * ld * 2 + c * 16) : OOB;
            }
        }
    }

    // K-major operand whose tile row r (< row_lim) is source row map[r] of a
    // source of src_rows rows at P; the byte range then covers the whole
    // source (under 2^31 bytes, checked on the host) and rows past row_lim
    // get an offset past it.
    __device__ __forceinline__ void init_gather(const bf16_t* P_, long ld_, int row_lim_,
                                                const int32_t* map, long src_rows) {
        static_assert(LAY == KMAJ, "row gather of a K-major operand");
        P = P_;
        ld = ld_;
        row_lim = row_lim_;
        k_lim = 0;
        span = src_rows * ld_ * 2;
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        constexpr int L = CH == 4 ? 2 : 3;
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            const int row = (w + NW * i) * (64 / CH) + lane / CH;
            const int c = (lane % CH) ^ ((row ^ (row >> L)) & (CH - 1));
            off[i] = row < row_lim ? (uint32_t)((long)map[row] * ld * 2 + c * 16) : OOB;
        }
    }

    // M/N-major operand whose reduction row k (< k_lim) is a gathered row of
    // a source with src_rows rows; P points at the tile's first column (of
    // row_lim valid ones).  off[] holds each load's chunk offset in a row.
    __device__ __forceinline__ void init_kgather(const bf16_t* P_, long ld_, int row_lim_,
                                                 long k_lim_, long src_rows, int m0) {
        static_assert(LAY != KMAJ, "reduction-row gather of an M/N-major operand");
        P = P_;
        ld = ld_;
        row_lim = row_lim_;
        k_lim = k_lim_;
        span = src_rows * ld_ * 2 - (long)m0 * 2;
        constexpr int NC = ROWS / 8;
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            const int k = (w + NW * i) * (1024 / (ROWS * 2)) + lane / NC;
            const int c = (lane % NC) ^ ((k & 3) << 2);
            off[i] = c * 8 < row_lim ? (uint32_t)(c * 16) : OOB;
        }
    }
    // Source rows of the loads of the stage of reduction rows k0 .. k0+BK-1:
    // row k is source row lmap[k - kmap] (lmap in LDS; k - kmap lies inside
    // the map chunk for a stage of it, so the read is unconditional and the
    // value is only looked at when the stage is issued: the LDS wait of
    // this read-ahead stays off the issue path).
    __device__ __forceinline__ void rows_of(long k0, const int32_t* lmap, long kmap,
                                            int32_t* rows) const {
        constexpr int NC = ROWS / 8;
        constexpr int RB = 1024 / (ROWS * 2);
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
        for (int i = 0; i < NLOAD; ++i)
            rows[i] = lmap[(k0 + (w + NW * i) * RB + lane / NC - kmap) & (KG_CHUNK - 1)];
    }
    // Issue the stage at k0, given rows_of's result; loads past the segment
    // or the tile's columns get an offset past the source.
    __device__ __forceinline__ void dma_rows(long k0, uint8_t* stage, const int32_t* rows) const {
        constexpr int NC = ROWS / 8;
        constexpr int RB = 1024 / (ROWS * 2);
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        const i32x4_t rs = rsrc_words(P, span);
        const uint32_t lds0 = lds_addr(stage) + (uint32_t)(w * 1024);
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            // branch-free: a source row offset is below 2^31 (host check),
            // so setting bit 31 (a column past the tile: off[i] = OOB, or a
            // row past the segment) sends the load past the descriptor range
            const long k = k0 + (w + NW * i) * RB + lane / NC;
            const uint32_t o = ((uint32_t)rows[i] * (uint32_t)(ld * 2) + off[i]) |
                               ((uint32_t)(k >= k_lim) << 31);
            lds_dma16(rs, o, lds0 + NW * i * 1024);
        }
    }

    __device__ __forceinline__ void dma(long k0, uint8_t* stage) const {
        const bf16_t* base;
        long nbytes;
        if (LAY == KMAJ) {
            base = P + k0;
            nbytes = span - k0 * 2;
        } else {
            base = P + k0 * ld;
            nbytes = min((long)BK, k_lim - k0) * ld * 2;
        }
        const i32x4_t rs = rsrc_words(base, nbytes);
        const uint32_t lds0 = lds_addr(stage) + (uint32_t)((threadIdx.x >> 6) * 1024);
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) lds_dma16(rs, off[i], lds0 + NW * i * 1024);
    }
};

template <int ROWS, int LAY, int BK>
__device__ __forceinline__ bf16x8 dma_frag(const uint8_t* lds, int row0, int ks, int lane) {
    if constexpr (LAY == KMAJ) {
        const uint4 v = *reinterpret_cast<const uint4*>(
            lds + swzk<BK / 8>(row0 + (lane & 31), ks * 2 + (lane >> 5)));
        return __builtin_bit_cast(bf16x8, v);
    } else {
        const int k = ks * 16 + (lane >> 5) * 8 + ((lane & 15) >> 2);
        const int col = row0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const uint8_t* p0 = lds + mnoff<ROWS>(k, col >> 3) + (col & 7) * 2;
        const uint8_t* p1 = lds + mnoff<ROWS>(k + 4, col >> 3) + (col & 7) * 2;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)p0);
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)p1);
        typedef short v8i16_t __attribute__((ext_vector_type(8)));
        const v8i16_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, v);
    }
}

// Order a wave's LDS writes before its later LDS reads (and reads before
// later writes) of data other lanes of the same wave touch: one wave's LDS
// instructions execute in order, so only the compiler must not move them.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// Wait until at most N direct-to-LDS loads of this wave are in flight and
// its LDS reads have returned, then meet the other waves of the block.  The
// compiler does not read the wait inside the asm; the lgkmcnt(0) after it
// (which then costs nothing) tells it that no LDS read is outstanding, so
// its own waits for the next fragments count only the reads issued after
// the barrier instead of draining them all (dW products 2-3% faster).
template <int N>
__device__ __forceinline__ void stage_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);                // lgkmcnt(0), no vmcnt wait
}
// stage_barrier with `ahead` (0..MAXA, wave-uniform) later stages of NL loads
// each allowed to stay in flight
template <int NL, int MAXA>
__device__ __forceinline__ void stage_barrier_ahead(int ahead) {
    if constexpr (MAXA <= 0) {
        stage_barrier<0>();
    } else {
        if (ahead >= MAXA) stage_barrier<NL * MAXA>();
        else stage_barrier_ahead<NL, MAXA - 1>(ahead);
    }
}

// Epilogue of the bf16 kernels, through LDS: each wave stages its own 16-row
// slabs of the accumulators in the ring (which every wave is done with), so
// the waves only order their own LDS writes and reads: no block barriers.
template <int BM, int BN, int WM, int WN, int NSTG, int STAGE, int MODE, bool DUAL, class Epi,
          int FM, int FN, int FMD, int FND>
__device__ __forceinline__ void bf16_epilogue(uint8_t* ringbuf, const TileInfo& ti,
                                              const GemmArgs<bf16_t>& p, const Epi& epi,
                                              const f32x16 (&acc)[FM][FN],
                                              const f32x16 (&acc2)[FMD][FND]) {
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int NBT = DUAL ? 2 : 1;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = wv / WN, wn = wv % WN;
    constexpr int LDW = WTN + 4;
    constexpr int SLAB = 16 * LDW;                   // floats per wave half-slab
    constexpr int WPS = STAGE / (SLAB * NBT * 4);    // wave slabs per stage array
    static_assert(WPS * NSTG >= NT / 64, "epilogue slabs do not fit");
    uint8_t* home = ringbuf + (wv / WPS) * STAGE;
    float* slab = reinterpret_cast<float*>(home) + (wv % WPS) * SLAB * NBT;
    constexpr int LPR = WTN / 8;
    constexpr int RPP = 64 / LPR;
    constexpr int NPS = 16 / RPP;                         // sub-passes of a slab
    const int c0 = (lane % LPR) * 8;
    const int col = ti.n0 + wn * WTN + c0;
    // slab q = 2i + h holds rows i*32 + h*16 .. +15 of the wave's tile
    auto row_of = [&](int q, int ps) {
        return wm * WTM + (q >> 1) * 32 + (q & 1) * 16 + ps * RPP + lane / LPR;
    };
    auto ok_of = [&](int rl) {
        return col < p.N && (MODE == RAGGED_M ? rl < ti.rows : ti.m0 + rl < p.M);
    };
    auto grow = [&](int rl) { return MODE == RAGGED_M ? ti.r0 + rl : (long)ti.m0 + rl; };
    // a chunk of a split dW segment: its fp32 partial product, summed
    // with the segment's other chunks (in order) by the reduce kernel
    const bool split = MODE == RAGGED_K && ti.pslot >= 0;
    auto to_partial = [&](int rl, const float* v) {
        float* q = p.partial + (long)ti.pslot * p.partial_ld + ((long)ti.m0 + rl) * p.N + col;
        *reinterpret_cast<float4*>(q) = *reinterpret_cast<const float4*>(v);
        *reinterpret_cast<float4*>(q + 4) = *reinterpret_cast<const float4*>(v + 4);
    };
    // Epilogues that read memory: the reads of slab q + 1 are issued before
    // slab q is consumed and stored, so each slab waits for its reads at most
    // as long as the previous slab takes (the reads of slab 0 go out before
    // its accumulators are staged); stores count in the same in-order
    // counter, so a read issued after a slab's stores would also wait for them.
    constexpr bool PRE = Epi::kPre && !DUAL;
    typedef typename Epi::Pre Pre;
    // The reads are not predicated: a lane whose row or column is outside
    // the product reads the tile's first row at column 0 instead (always in
    // bounds) and drops the data, so no branch hides a read from the
    // compiler's count of reads in flight (a branch around them makes it
    // wait for all of them).  A chunk of a split dW segment reads no C.
    auto issue = [&](int q, Pre (&pre)[NPS]) {
        if (split) return;
#pragma unroll
        for (int ps = 0; ps < NPS; ++ps) {
            const int rl = row_of(q, ps);
            const bool in = ok_of(rl);
            pre[ps] = epi.pre8(ti.e, grow(in ? rl : 0), in ? col : 0);
        }
    };
    Pre pre[2 * FM][NPS];                                 // one set per slab: no copies
    if constexpr (PRE) issue(0, pre[0]);
#pragma unroll
    for (int q = 0; q < 2 * FM; ++q) {
        const int i = q >> 1, h = q & 1;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int vv = 0; vv < 8; ++vv) {
                const int v = h * 8 + vv;
                const int r = (vv >> 2) * 8 + (lane >> 5) * 4 + (vv & 3);
                slab[r * LDW + j * 32 + (lane & 31)] = acc[i][j][v];
                if constexpr (DUAL)
                    slab[SLAB + r * LDW + j * 32 + (lane & 31)] = acc2[i][j][v];
            }
        wave_lds_sync();
        if constexpr (PRE) {
            if (q + 1 < 2 * FM) issue(q + 1, pre[q + 1]);
#pragma unroll
            for (int ps = 0; ps < NPS; ++ps) {
                const int rl = row_of(q, ps);
                const float* src = &slab[(ps * RPP + lane / LPR) * LDW + c0];
                float v[8];
                *reinterpret_cast<float4*>(v) = *reinterpret_cast<const float4*>(src);
                *reinterpret_cast<float4*>(v + 4) = *reinterpret_cast<const float4*>(src + 4);
                if (ok_of(rl)) {
                    if (split) to_partial(rl, v);
                    else epi.vec8p(ti.e, grow(rl), col, v, pre[q][ps]);
                }
            }
        } else {
#pragma unroll 1
            for (int ps = 0; ps < NPS; ++ps) {
                const int rl = row_of(q, ps);
                const float* src = &slab[(ps * RPP + lane / LPR) * LDW + c0];
                float v[8];
                *reinterpret_cast<float4*>(v) = *reinterpret_cast<const float4*>(src);
                *reinterpret_cast<float4*>(v + 4) = *reinterpret_cast<const float4*>(src + 4);
                if (ok_of(rl)) {
                    if constexpr (DUAL) {
                        float v3[8];
                        *reinterpret_cast<float4*>(v3) = *reinterpret_cast<const float4*>(src + SLAB);
                        *reinterpret_cast<float4*>(v3 + 4) =
                            *reinterpret_cast<const float4*>(src + SLAB + 4);
                        epi.vec8(ti.e, ti.r0 + rl, col, v, v3);
                    } else if (MODE == RAGGED_M) {
                        epi.vec8(ti.e, ti.r0 + rl, col, v);
                    } else if (split) {
                        to_partial(rl, v);
                    } else {
                        epi.vec8(ti.e, (long)ti.m0 + rl, col, v);
                    }
                }
            }
        }
        wave_lds_sync();
    }
}

template <int BM, int BN, int WM, int WN, int NSTG, int BK, int MODE, int ALAY, int BLAY,
          bool DUAL, bool KSPLIT, bool GATHER, class Epi>
__global__ __launch_bounds__(64 * WM * WN, 2) void ggemm_bf16_dma_kernel(GemmArgs<bf16_t> p,
                                                                         Epi epi) {
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int NBT = DUAL ? 2 : 1;
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    constexpr int STAGE = A_BYTES + NBT * B_BYTES;
    constexpr bool KGATHER = GATHER && MODE == RAGGED_K;
    static_assert(!GATHER || (ALAY == KMAJ) == (MODE == RAGGED_M), "gather form");
    static_assert(KG_CHUNK % BK == 0, "map chunks hold whole stages");
    constexpr int KGM = KGATHER ? KG_CHUNK : 1;
    static_assert(NSTG >= 2 && STAGE % 1024 == 0 && NSTG * STAGE + KGM * 4 <= 160 * 1024,
                  "ring size");
    __shared__ __attribute__((aligned(1024))) uint8_t ringbuf[NSTG * STAGE];
    __shared__ int32_t kmap[KGM];        // source rows of reduction rows kmap0 ..

    const TileInfo ti = decode_tile<MODE, BM, BN>(p);
    if (!ti.live) return;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv / WN, wn = wv % WN;

    DmaOperand<BM, ALAY, NT, BK> opA;
    DmaOperand<BN, BLAY, NT, BK> opB;
    DmaOperand<BN, BLAY, NT, BK> opB2;
    const bf16_t* bsplit[2];
    if constexpr (MODE == RAGGED_M) {
        if constexpr (GATHER)
            opA.init_gather(p.A, p.lda, ti.rows, p.gather + ti.r0, p.gather_rows);
        else
            opA.init(p.A + ti.r0 * p.lda, p.lda, ti.rows, p.K);
        const long eoff = (long)ti.e * p.bstride;
        const long nofs = BLAY == KMAJ ? (long)ti.n0 * p.ldb : (long)ti.n0;
        opB.init(p.B + eoff + nofs, p.ldb, p.N - ti.n0, p.K);
        if (DUAL) opB2.init(p.B2 + eoff + nofs, p.ldb, p.N - ti.n0, p.K);
        if (KSPLIT) bsplit[0] = opB.P, bsplit[1] = p.B2 + eoff + nofs;
    } else {
        if constexpr (KGATHER)
            opA.init_kgather(p.A + ti.m0, p.lda, p.M - ti.m0, ti.klen, p.gather_rows, ti.m0);
        else
            opA.init(p.A + ti.kbeg * p.lda + ti.m0, p.lda, p.M - ti.m0, ti.klen);
        opB.init(p.B + ti.kbeg * p.ldb + ti.n0, p.ldb, p.N - ti.n0, ti.klen);
    }
    // KGATHER: the source rows of reduction rows kmap0 .. kmap0+KG_CHUNK-1
    // of the segment, reloaded between stages when the issue crosses a
    // chunk (the barriers make every wave finish with the old chunk first)
    auto load_kmap = [&](long kmap0) {
        if constexpr (KGATHER) {
            static_assert(KG_CHUNK % NT == 0, "map chunk per thread");
            constexpr int PER = KG_CHUNK / NT;
            __syncthreads();
            if (kmap0 < ti.klen) {
                // every load in flight before the first store (clamped
                // addresses, so no load is conditional)
                int32_t v[PER];
                const long last = ti.klen - 1;
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    const long q = kmap0 + threadIdx.x + u * NT;
                    v[u] = p.gather[ti.kbeg + (q < last ? q : last)];
                }
#pragma unroll
                for (int u = 0; u < PER; ++u) kmap[threadIdx.x + u * NT] = v[u];
            }
            __syncthreads();
        }
    };
    constexpr int NL = DmaOperand<BM, ALAY, NT, BK>::NLOAD + NBT * DmaOperand<BN, BLAY, NT, BK>::NLOAD;
    static_assert(NL * (NSTG - 1) <= 63, "vmcnt counts at most 63 loads");

    f32x16 acc[FM][FN];
    f32x16 acc2[DUAL ? FM : 1][DUAL ? FN : 1];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    if constexpr (DUAL) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc2[i][j][v] = 0.0f;
    }

    // KGATHER: source rows of the next stage to issue, read from the map one
    // stage ahead so that the issue does not wait on LDS
    int32_t krow[KGATHER ? DmaOperand<BM, ALAY, NT, BK>::NLOAD : 1];
    auto issue = [&](uint8_t* stg, int j) {
        const long k0 = (long)j * BK;
        if constexpr (KGATHER) {
            const long c0 = k0 / KG_CHUNK * KG_CHUNK;
            if (k0 == c0 && k0 > 0) {            // next map chunk
                load_kmap(c0);
                opA.rows_of(k0, kmap, c0, krow);
            }
            opA.dma_rows(k0, stg, krow);
            // the next stage's rows (read modulo the chunk: at a chunk switch
            // they are read again after the reload)
            opA.rows_of(k0 + BK, kmap, c0, krow);
        } else {
            opA.dma(k0, stg);
        }
        if constexpr (KSPLIT) {
            const bool hi = k0 >= p.Ksplit;
            opB.P = bsplit[hi];
            opB.dma(hi ? k0 - p.Ksplit : k0, stg + A_BYTES);
        } else {
            opB.dma(k0, stg + A_BYTES);
        }
        if constexpr (DUAL) opB2.dma(k0, stg + A_BYTES + B_BYTES);
    };
    // Fragments are double-buffered across k-steps and across stages: the
    // first fragments of stage j+1 are read while the last MFMAs of stage j
    // run, so the matrix pipe never waits for a stage boundary.
    constexpr int KS = BK / 16;                       // MFMA k-steps per stage
    static_assert(KS % 2 == 0, "fragment buffer parity assumes an even count");
    bf16x8 af[2][FM], bfr[2][FN], bf2[2][DUAL ? FN : 1];
    auto read_frags = [&](const uint8_t* stg, int ks, int buf) {
        const uint8_t* sA = stg;
        const uint8_t* sB = stg + A_BYTES;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            af[buf][i] = dma_frag<BM, ALAY, BK>(sA, wm * WTM + i * 32, ks, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bfr[buf][j] = dma_frag<BN, BLAY, BK>(sB, wn * WTN + j * 32, ks, lane);
        if constexpr (DUAL) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf2[buf][j] = dma_frag<BN, BLAY, BK>(sB + B_BYTES, wn * WTN + j * 32, ks, lane);
        }
    };
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfr[buf][j],
                                                                   acc[i][j], 0, 0, 0);
        if constexpr (DUAL) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        af[buf][i], bf2[buf][j], acc2[i][j], 0, 0, 0);
        }
    };
    auto ring = [&](int q) -> uint8_t* { return ringbuf + q * STAGE; };
    // Ring of NSTG stages.  Every read of stage j-1 has returned once the
    // waves meet at the barrier of stage j-1 (fragments go to registers),
    // so stage j+NSTG-1 is issued into that slot at the top of stage j,
    // away from the barrier and behind the MFMAs still in the pipe: while
    // stage j is multiplied, j+1 .. j+NSTG-1 are landing.
    const int nj = (ti.klen + BK - 1) / BK;
    load_kmap(0);
    if constexpr (KGATHER) opA.rows_of(0, kmap, 0, krow);
    // Prologue: the first NP stages.  With both operands K-contiguous the
    // slot of stage NSTG-1 is filled here too (one stage more in flight
    // from the start: dA, dX 2-3% faster); with a transposed operand that
    // was slower (long-context down and dW 2-2.5%, the MoE-S-like products
    // 2-6%), although reads and loads do not slow each other in LDS itself.
    constexpr int NP = ALAY == KMAJ && BLAY == KMAJ ? NSTG : NSTG - 1;
#pragma unroll
    for (int q = 0; q < NP; ++q)
        if (q < nj) issue(ring(q), q);
    stage_barrier_ahead<NL, NP - 1>(min(nj - 1, NP - 1));   // stage 0 landed
    if (nj > 0) read_frags(ring(0), 0, 0);
    // all stages but the last; the last one is peeled off so that the loop
    // body has one path and the compiler's LDS waits before its final MFMAs
    // do not cover the reads of the next stage
    int qc = 0;                                        // ring slot of stage j
#pragma unroll 1
    for (int j = 0; j + 1 < nj; ++j) {
        const uint8_t* cur = ring(qc);
        const int qn = qc + 1 == NSTG ? 0 : qc + 1;    // slot of stage j+1
        const int qf = qc == 0 ? NSTG - 1 : qc - 1;    // slot of stage j-1 = j+NSTG-1
        const bool more = (NP < NSTG || j > 0) && j + NSTG - 1 < nj;
        // a gathered issue (row indices read from LDS a stage ahead) goes
        // behind the first k-step's MFMAs: at the top of the stage it was 2%
        // slower on the long-context dW shapes (60.5 against 59.2-59.5 ms)
        if (!KGATHER && more) issue(ring(qf), j + NSTG - 1);
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
            read_frags(cur, ks + 1, (ks + 1) & 1);
            mfmas(ks & 1);
            if (KGATHER && ks == 0 && more) issue(ring(qf), j + NSTG - 1);
            if constexpr (DUAL) {
                // the two-weight product: one fragment read after each
                // MFMA, so the reads of the next k-step (two transposed
                // reads per fragment of each weight) do not bunch up
                // ahead of the MFMAs (5% faster on the long-context shapes;
                // the single-weight products were 1-3% slower with it)
                constexpr int NMF = FM * FN * 2;
                constexpr int NRD = FM * (ALAY == KMAJ ? 1 : 2) + 2 * FN * (BLAY == KMAJ ? 1 : 2);
                constexpr int PER = NMF / NRD > 0 ? NMF / NRD : 1;
#pragma unroll
                for (int r = 0; r < NRD; ++r) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // LDS read
                    if (r * PER < NMF) __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // MFMA
                }
                if (NRD * PER < NMF) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NRD * PER, 0);
            }
        }
        stage_barrier_ahead<NL, NSTG - 2>(min(nj - 2 - j, NSTG - 2));  // stage j+1 landed
        read_frags(ring(qn), 0, 0);
        mfmas((KS - 1) & 1);
        qc = qn;
    }
    if (nj > 0) {
        const uint8_t* cur = ring(qc);
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
            read_frags(cur, ks + 1, (ks + 1) & 1);
            mfmas(ks & 1);
        }
        mfmas((KS - 1) & 1);
    }
    __syncthreads();
    bf16_epilogue<BM, BN, WM, WN, NSTG, STAGE, MODE, DUAL>(ringbuf, ti, p, epi, acc, acc2);
}

// =====================================================================
// fp32 SIMT kernel (correctness path for fp32 layers)
// =====================================================================

constexpr int FB = 64, FK = 16;

template <int MODE, int ALAY, int BLAY, bool DUAL, bool KSPLIT, class Epi>
__global__ __launch_bounds__(256) void ggemm_f32_kernel(GemmArgs<float> p, Epi epi) {
    __shared__ float sA[FK][FB + 4];
    __shared__ float sB[FK][FB + 4];
    __shared__ float sB2[DUAL ? FK : 1][FB + 4];
    const TileInfo ti = decode_tile<MODE, FB, FB>(p);
    if (!ti.live) return;
    const int tid = threadIdx.x, tm = tid / 16, tn = tid % 16;
    float acc[4][4], acc2[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = acc2[a][b] = 0.0f;
    const long eoff = MODE == RAGGED_M ? (long)ti.e * p.bstride : 0;
    for (int k0 = 0; k0 < ti.klen; k0 += FK) {
        for (int q = tid; q < FB * FK; q += 256) {
            int m, kk;
            float v = 0.0f;
            if (ALAY == KMAJ) { m = q / FK; kk = q % FK; } else { m = q % FB; kk = q / FB; }
            const long k = k0 + kk;
            if (MODE == RAGGED_M) {
                if (m < ti.rows) {
                    const long r = ti.r0 + m;
                    v = p.A[(p.gather ? (long)p.gather[r] : r) * p.lda + k];
                }
            } else {
                if (k < ti.klen && ti.m0 + m < p.M) {
                    const long r = ti.kbeg + k;
                    v = p.A[(p.gather ? (long)p.gather[r] : r) * p.lda + ti.m0 + m];
                }
            }
            sA[kk][m] = v;
        }
        for (int q = tid; q < FB * FK; q += 256) {
            int n, kk;
            if (BLAY == KMAJ) { n = q / FK; kk = q % FK; } else { n = q % FB; kk = q / FB; }
            const long k = k0 + kk;
            const int gn = ti.n0 + n;
            float v = 0.0f, v2 = 0.0f;
            if (gn < p.N) {
                if (MODE == RAGGED_M) {
                    if (BLAY == KMAJ) {
                        if (KSPLIT && k >= p.Ksplit)
                            v = p.B2[eoff + (long)gn * p.ldb + (k - p.Ksplit)];
                        else
                            v = p.B[eoff + (long)gn * p.ldb + k];
                    } else {
                        v = p.B[eoff + k * p.ldb + gn];
                        if (DUAL) v2 = p.B2[eoff + k * p.ldb + gn];
                    }
                } else if (k < ti.klen) {
                    v = p.B[(ti.kbeg + k) * p.ldb + gn];
                }
            }
            sB[kk][n] = v;
            if (DUAL) sB2[kk][n] = v2;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < FK; ++kk) {
            float av[4], bv[4], bv2[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) av[a] = sA[kk][tm * 4 + a];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                bv[b] = sB[kk][tn * 4 + b];
                if (DUAL) bv2[b] = sB2[kk][tn * 4 + b];
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    acc[a][b] = fmaf(av[a], bv[b], acc[a][b]);
                    if (DUAL) acc2[a][b] = fmaf(av[a], bv2[b], acc2[a][b]);
                }
        }
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int rl = tm * 4 + a;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int col = ti.n0 + tn * 4 + b;
            if (col >= p.N) continue;
            if (MODE == RAGGED_M) {
                if (rl >= ti.rows) continue;
                if constexpr (DUAL) epi(ti.e, ti.r0 + rl, col, acc[a][b], acc2[a][b]);
                else epi(ti.e, ti.r0 + rl, col, acc[a][b]);
            } else {
                if (ti.m0 + rl >= p.M) continue;
                if constexpr (!DUAL) epi(ti.e, (long)ti.m0 + rl, col, acc[a][b]);
            }
        }
    }
}

// =====================================================================
// planner: per-expert M-tile prefix and heaviest-first expert order
// =====================================================================

// Split of a weight-gradient segment (RAGGED_K) over its rows.  An expert
// whose dW tiles are fewer than the compute units cannot fill the GPU, and
// with a long segment its tiles set the whole product's critical path (one
// expert with 39% of the rows, 64 tiles on 256 compute units).  Such a
// segment (more than 2 * kSplitRows rows, fewer than kSplitTiles tiles) is
// cut into chunks of kc = max(kSplitRows, rows / kSplitChunks rounded up to
// 256) rows; each chunk's tiles store fp32 partial products and the reduce
// kernel sums them in chunk order, so the split depends only on the
// segment's length and the matrix shape and the sum order is fixed.
constexpr int kSplitRows = 4096;
constexpr int kSplitChunks = 64;
constexpr int kSplitTiles = 256;

__host__ __device__ inline int split_chunk_rows(int n) {
    const int per = (n + kSplitChunks - 1) / kSplitChunks;
    const int kc = (per + 255) / 256 * 256;
    return kc > kSplitRows ? kc : kSplitRows;
}

// Bounds on the split plan of a product with R rows over E experts and
// dw_tiles tiles per expert: partial slots (chunks of split segments) and
// split segments.  A split segment has n > 2 kSplitRows rows and
// ceil(n / kc) <= n / kSplitRows + 1 < 1.5 n / kSplitRows chunks.
struct SplitBound {
    long slots, splits;
};
inline SplitBound split_bound(long R, int E, int dw_tiles) {
    if (dw_tiles >= kSplitTiles) return {0, 0};
    const long splits = std::min<long>(E, R / (2L * kSplitRows + 1));
    const long slots = std::min<long>((long)kSplitChunks * splits, 3 * R / (2L * kSplitRows) + 1);
    return {splits > 0 ? slots : 0, splits};
}

// The tile plan of a call, from the segment offsets (one workgroup):
//  tile_prefix[e] RAGGED_M row tiles of the experts before e (plus the total)
//  full_prefix[e] the same for full 256-row tiles; part_list the experts with
//                 a partial last tile (count at [E])
//  order          experts by row count, heaviest first (ties: lower index)
//  items          (dw_tiles > 0) the RAGGED_K work items in dealing order:
//                 the chunks of split segments (heaviest expert first), then
//                 the whole segments of the other experts in `order`;
//                 counts[0] = items, counts[1] = split segments, whose
//                 (expert, first slot, chunks) are listed in splits
__global__ __launch_bounds__(1024) void ffn_plan_kernel(const int32_t* __restrict__ offsets,
                                                        int E, int bm, int dw_tiles,
                                                        int32_t* __restrict__ tile_prefix,
                                                        int32_t* __restrict__ order,
                                                        int32_t* __restrict__ full_prefix,
                                                        int32_t* __restrict__ part_list,
                                                        int4* __restrict__ items,
                                                        int4* __restrict__ splits,
                                                        int32_t* __restrict__ counts) {
    __shared__ int cnt[1024];
    __shared__ int ord[1024];
    __shared__ int sh[16];
    const int e = threadIdx.x;
    const int c_e = e < E ? offsets[e + 1] - offsets[e] : 0;
    MOE_DASSERT(c_e >= 0 && (e > 0 || offsets[0] >= 0));   // nondecreasing, from row >= 0
    if (e < E) cnt[e] = c_e;
    // per-expert prefixes of the row tiles, of the full row tiles and of the
    // experts with a partial last tile (block scans; experts in index order)
    int tot_tiles, tot_full, tot_part;
    const int p_tiles = block_excl_scan<1024>((c_e + bm - 1) / bm, sh, &tot_tiles);
    const int p_full = block_excl_scan<1024>(c_e / bm, sh, &tot_full);
    const int has_part = e < E && c_e % bm != 0;
    const int p_part = block_excl_scan<1024>(has_part, sh, &tot_part);
    if (e < E) {
        tile_prefix[e] = p_tiles;
        full_prefix[e] = p_full;
        if (has_part) part_list[p_part] = e;
    }
    if (e == 0) {
        tile_prefix[E] = tot_tiles;
        full_prefix[E] = tot_full;
        part_list[E] = tot_part;
    }
    if (e < E) {
        const int c = cnt[e];
        int rank = 0;
        for (int q = 0; q < E; ++q) {
            const int cq = cnt[q];
            rank += (cq > c) || (cq == c && q < e);
        }
        order[rank] = e;
        ord[rank] = e;
    }
    __syncthreads();
    if (!items) return;
    // dW work items: the chunks of the split segments (heaviest first), then
    // the whole segments in rank order.  Only the heaviest experts can split,
    // so the first loop is short; its counts reach the other threads in LDS.
    __shared__ int nsplit[2];
    if (e == 0) {
        int ni = 0, ns = 0, slot = 0;
        const bool may_split = dw_tiles < kSplitTiles;
        for (int r = 0; r < E; ++r) {
            const int q = ord[r], n = cnt[q];
            if (!may_split || n <= 2 * kSplitRows) break;   // the rest are shorter
            const int kc = split_chunk_rows(n);
            const int nc = (n + kc - 1) / kc;
            for (int c = 0; c < nc; ++c)
                items[ni++] = make_int4(q, offsets[q] + c * kc, min(kc, n - c * kc), slot + c);
            splits[ns++] = make_int4(q, slot, nc, 0);
            slot += nc;
        }
        nsplit[0] = ni;
        nsplit[1] = ns;
        counts[0] = ni + (E - ns);
        counts[1] = ns;
    }
    __syncthreads();
    const int ni = nsplit[0], ns = nsplit[1];
    if (e >= ns && e < E) {                         // whole segments
        const int q = ord[e];
        items[ni + (e - ns)] = make_int4(q, offsets[q], cnt[q], -1);
    }
}

// C_e (+)= the sum of a split segment's fp32 chunk products, in chunk order
// (after the old value when accumulating), rounded once.  Block row j is the
// j-th split segment; each thread finishes 8 consecutive elements of C_e.
template <typename T>
__global__ __launch_bounds__(256) void dw_split_reduce_kernel(
    const int4* __restrict__ splits, const int32_t* __restrict__ counts,
    const float* __restrict__ partial, long mn, T* __restrict__ C, long cstride,
    int accumulate) {
    const int j = blockIdx.y;
    if (j >= counts[1]) return;
    const long i0 = ((long)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i0 >= mn) return;
    const int4 sp = splits[j];                      // expert, first slot, chunks
    T* c = C + (long)sp.x * cstride + i0;
    float acc[8];
    if (accumulate) {
        if constexpr (sizeof(T) == 2) {
            Vec16<T>::ld(c, acc);
        } else {
            Vec16<T>::ld(c, acc);
            Vec16<T>::ld(c + 4, acc + 4);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    }
    for (int k = 0; k < sp.z; ++k) {
        const float4* q = reinterpret_cast<const float4*>(partial + (long)(sp.y + k) * mn + i0);
        const float4 a = q[0], b = q[1];
        acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
        acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    if constexpr (sizeof(T) == 2) {
        Vec16<T>::st(c, acc);
    } else {
        Vec16<T>::st(c, acc);
        Vec16<T>::st(c + 4, acc + 4);
    }
}

// ------------------------------------------------------------- launches

constexpr int BM_BF16 = 256;

// Workspace of an FFN call: the tile plan (forward and backward), then, for
// the backward, dH and (bf16) the split plan of the dW products: work items,
// split segments, their counts, and two fp32 partial regions (dW2 may run on
// the side stream while dW1 / dW3 run on the caller's stream).
struct FfnWs {
    size_t prefix, order, full, part, dh, items, splits, counts, part0, part1, total;
    long item_max, split_max, slot_max;
};

inline int dw_tiles_of(int d, int f) { return cdiv(d, 256) * cdiv(f, 256); }

FfnWs ffn_layout(int R, int E, int d, int f, moe_act act, moe_dtype dt, int backward) {
    FfnWs w;
    w.prefix = 0;
    w.order = align_up(sizeof(int32_t) * (E + 1), 256);
    w.full = align_up(w.order + sizeof(int32_t) * E, 256);
    w.part = align_up(w.full + sizeof(int32_t) * (E + 1), 256);
    w.dh = align_up(w.part + sizeof(int32_t) * (E + 1), 256);
    size_t dh = 0;
    w.item_max = w.split_max = w.slot_max = 0;
    if (backward) {
        const size_t es = dt == MOE_BF16 ? 2 : 4;
        dh = es * (size_t)R * f * (act == MOE_ACT_SWIGLU ? 2 : 1);
    }
    w.items = align_up(w.dh + dh, 256);
    if (backward && dt == MOE_BF16) {
        const SplitBound sb = split_bound(R, E, dw_tiles_of(d, f));
        w.slot_max = sb.slots;
        w.split_max = sb.splits;
        w.item_max = E + sb.slots;
    }
    w.splits = align_up(w.items + sizeof(int4) * w.item_max, 256);
    w.counts = align_up(w.splits + sizeof(int4) * w.split_max, 256);
    const size_t region = sizeof(float) * (size_t)w.slot_max * d * f;
    w.part0 = align_up(w.counts + (w.item_max ? 2 * sizeof(int32_t) : 0), 256);
    w.part1 = align_up(w.part0 + region, 256);
    w.total = align_up(w.part1 + region, 256);
    return w;
}

// G: the product may gather its A rows (p.gather != NULL selects that kernel)
template <int BM, int BN, int WM, int WN, int NSTG, int BK, int MODE, int ALAY, int BLAY,
          bool DUAL, bool KSPLIT, bool G, class Epi>
void launch_bf16(GemmArgs<bf16_t> p, Epi epi, int R, hipStream_t s, const char* name) {
    p.nN = (p.N + BN - 1) / BN;
    int blocks;
    if (MODE == RAGGED_M) {
        // row tiles at most: all < ceil(R/BM) + E, full <= R/BM, partial <= min(E, R)
        const int rt = p.part_mode == 0 ? (R + BM - 1) / BM + p.E
                     : p.part_mode == 1 ? R / BM
                                        : min(p.E, R) * (p.bm_plan / BM);
        blocks = rt * p.nN;
        // The dual-weight (SwiGLU up) product in rounds of 16 x 16 tiles: 1.5%
        // faster on the long-context shapes; the single-weight products were
        // 1-11% slower that way (their panels are read from L2 in the grouped
        // order already), so they keep it
        p.round16 = DUAL && p.part_mode == 0 && p.xcd_run <= 0;
        if (p.round16) {
            p.xcd_run = 32;
            blocks = ((rt + 15) / 16) * ((p.nN + 15) / 16) * 256;
        }
    } else {
        p.nM = (p.M + BM - 1) / BM;
        blocks = (p.items ? p.item_max : p.E) * p.nM * p.nN;
        // Each XCD holds four runs of 8 consecutive tiles at once (32 compute
        // units), runs 8 apart in the dealing order.  Column by column, those
        // four runs share their row tiles (A panels) only when the row-tile
        // count divides 64; otherwise (f = 14336: 56 row tiles of dW2) the
        // tiles go in groups of 8 row tiles, runs of 32 (dW2 on the
        // long-context shapes -11%; with a power-of-two row-tile count the
        // column order was 1-4% faster)
        p.k_grouped = 64 % p.nM != 0;
        if (p.xcd_run <= 0) p.xcd_run = p.k_grouped ? 32 : 8;
    }
    if (blocks <= 0) return;
    if (p.xcd_run <= 0) p.xcd_run = 32;
    const int pad = NXCD * p.xcd_run;                      // whole XCD runs
    blocks = (blocks + pad - 1) / pad * pad;
    if constexpr (G) {
        if (p.gather) {
            MOE_LAUNCH(name, s,
                       ggemm_bf16_dma_kernel<BM, BN, WM, WN, NSTG, BK, MODE, ALAY, BLAY, DUAL,
                                             KSPLIT, true, Epi>
                       <<<blocks, 64 * WM * WN, 0, s>>>(p, epi));
            return;
        }
    }
    MOE_LAUNCH(name, s,
               ggemm_bf16_dma_kernel<BM, BN, WM, WN, NSTG, BK, MODE, ALAY, BLAY, DUAL, KSPLIT,
                                     false, Epi>
               <<<blocks, 64 * WM * WN, 0, s>>>(p, epi));
}

template <int MODE, int ALAY, int BLAY, bool DUAL, bool KSPLIT, class Epi>
void launch_f32(GemmArgs<float> p, Epi epi, int R, hipStream_t s, const char* name) {
    p.nN = (p.N + FB - 1) / FB;
    p.xcd_run = 1;
    int blocks;
    if (MODE == RAGGED_M) {
        blocks = ((R + FB - 1) / FB + p.E) * p.nN;
    } else {
        p.nM = (p.M + FB - 1) / FB;
        blocks = p.E * p.nM * p.nN;
    }
    if (blocks <= 0) return;
    MOE_LAUNCH(name, s, ggemm_f32_kernel<MODE, ALAY, BLAY, DUAL, KSPLIT, Epi><<<blocks, 256, 0, s>>>(p, epi));
}

struct Plan {
    const int32_t *prefix, *order, *full, *part;
};

template <typename T>
GemmArgs<T> base_args(const int32_t* offsets, const Plan& pl, int E) {
    GemmArgs<T> p = {};
    p.offsets = offsets;
    p.tile_prefix = pl.prefix;
    p.order = pl.order;
    p.full_prefix = pl.full;
    p.part_list = pl.part;
    p.E = E;
    p.part_mode = 0;
    p.bm_plan = 0;
    p.xcd_run = 0;
    p.gather = nullptr;
    p.gather_rows = 0;
    p.items = nullptr;
    p.item_count = nullptr;
    p.item_max = 0;
    p.k_grouped = 0;
    p.round16 = 0;
    p.partial = nullptr;
    p.partial_ld = 0;
    return p;
}

// Tile configuration of the bf16 path: block tile and wave grid for the
// single-product GEMMs, for the dual-weight (SwiGLU up) product, and for the
// tail launch of a split RAGGED_M product (BMT = 0: never split), in a wide
// (BNT) and a narrow (BNN) column variant.
// Ring<NS, BK>: an LDS ring of NS stages of BK reduction steps.
template <int NS_, int BK_>
struct Ring {
    static constexpr int NS = NS_, BK = BK_;
};
// RM, RT, RN are the rings of the main, wide-tail and narrow-tail kernels
// of RAGGED_M products, RK the ring of RAGGED_K (dW) products.
template <int BM_, int BN_, int WM_, int WN_, int BND_, int WMD_, int WND_, int BMT_ = 0,
          int BNT_ = 0, int WMT_ = 0, int WNT_ = 0, int BNN_ = 0, int WNN_ = 0,
          class RM_ = Ring<4, 32>, class RT_ = Ring<4, 32>, class RN_ = Ring<4, 32>,
          class RK_ = RM_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int BND = BND_, WMD = WMD_, WND = WND_;
    static constexpr int BMT = BMT_, BNT = BNT_, WMT = WMT_, WNT = WNT_;
    static constexpr int BNN = BNN_, WNN = WNN_;
    typedef RM_ RM;
    typedef RT_ RT;
    typedef RN_ RN;
    typedef RK_ RK;
};
// RAGGED_M main and wide-tail tiles: two 64-deep stages (half the barriers
// of 32-deep ones; the next stage is issued at the top of the current one).  dW
// products, whose reduction is a segment that may be short, keep four
// 32-deep stages, unless the segments are long (LongKCfg).  The narrow tail
// (64x128 slices, few MFMAs per stage) takes 64-deep stages in a 5-stage
// ring, three in flight.
using DefaultCfg = TileCfg<256, 256, 4, 2, 128, 4, 2, 64, 256, 1, 4, 128, 4, Ring<2, 64>,
                           Ring<2, 64>, Ring<5, 64>, Ring<4, 32>>;
// dW products over segments of kLongSegmentRows rows or more on average
// (R >= kLongSegmentRows * E): two 64-deep stages, half the barriers of four
// 32-deep ones (the long-context step 1.9% faster; with 2048-row segments,
// MoE-S-like, they were 0.4% slower, so shorter segments keep the 32-deep
// ring).  Same summation order: the outputs do not change.
template <class C>
using LongKCfg = TileCfg<C::BM, C::BN, C::WM, C::WN, C::BND, C::WMD, C::WND, C::BMT, C::BNT,
                         C::WMT, C::WNT, C::BNN, C::WNN, typename C::RM, typename C::RT,
                         typename C::RN, Ring<2, 64>>;
constexpr long kLongSegmentRows = 4096;

// Wave quantisation.  A RAGGED_M product has between ceil(R/BM) and
// ceil(R/BM) + E - 1 row tiles, since each expert's last tile is usually
// partial; with nN column tiles per row tile the last round of workgroups
// is often nearly empty (e.g. 72 x 4 tiles on 256 compute units: two rounds
// for 1.125 rounds of work), and the partial tiles cost as much as full
// ones.  Split (when the product is under kSplitRounds rounds of
// workgroups): one launch multiplies the full row tiles of all experts,
// a second one only the partial last tiles, cut into BMT-row slices (empty
// slices exit at once) with BNT-wide columns, or BNN-wide ones when the
// wide tail would leave most compute units idle, spread over all XCDs.
// Every output element is still one fixed-order sum over k: identical
// results.
constexpr int kSplitRounds = 8;

inline int xcd_run_for(long tiles) {
    int run = 1;
    while (run < 32 && (long)run * 2 * NXCD <= tiles) run *= 2;
    return run;
}

template <typename T, class Cfg>
struct Launch;

template <class Cfg>
struct Launch<bf16_t, Cfg> {
    // Whether go() splits a product of this shape (given a tail name).
    template <int MODE, bool DUAL>
    static bool splits(int R, int E, int N) {
        if constexpr (MODE == RAGGED_M && !DUAL && Cfg::BMT > 0) {
            // Split only when the product is a few rounds of workgroups:
            // with many rounds the one partially filled last round is a
            // small share, and the narrow slices cost more than they save.
            // (Also with many small experts: on the 64-expert workload, where
            // a fifth of the row tiles are an expert's mostly empty last
            // tile, splitting the up and dA products made them 9% slower --
            // a 64-row slice with one wave per SIMD runs its reduction at
            // the same per-stage latency as a full tile.)
            const long tiles = (long)(cdiv(R, Cfg::BM) + E / 2) * cdiv(N, Cfg::BN);
            return tiles < (long)kSplitRounds * device_cus();
        }
        return false;
    }
    // Returns true when the product was split: full row tiles on s, the
    // partial last tiles on ts.  Otherwise everything ran on s.
    template <int MODE, int ALAY, int BLAY, bool DUAL, bool KSPLIT, bool G = false, class Epi>
    static bool go(GemmArgs<bf16_t> p, Epi epi, int R, hipStream_t s, const char* name,
                   const char* tail_name = nullptr, hipStream_t ts = nullptr) {
        using RR = std::conditional_t<MODE == RAGGED_K, typename Cfg::RK, typename Cfg::RM>;
        if (!ts) ts = s;           // stream of the tail launch
        if constexpr (DUAL) {
            launch_bf16<Cfg::BM, Cfg::BND, Cfg::WMD, Cfg::WND, RR::NS, RR::BK, MODE, ALAY, BLAY, DUAL,
                        KSPLIT, G>(p, epi, R, s, name);
            return false;
        } else {
            if constexpr (MODE == RAGGED_M && Cfg::BMT > 0) {
                if (tail_name && splits<MODE, DUAL>(R, p.E, p.N)) {
                    GemmArgs<bf16_t> q = p;
                    q.part_mode = 1;
                    q.bm_plan = Cfg::BM;
                    launch_bf16<Cfg::BM, Cfg::BN, Cfg::WM, Cfg::WN, RR::NS, RR::BK, MODE, ALAY, BLAY,
                                DUAL, KSPLIT, G>(q, epi, R, s, name);
                    q.part_mode = 2;
                    // expected live slices: about half of the slots of the partial tiles
                    const long slices = (long)min(p.E, R) * (Cfg::BM / Cfg::BMT) / 2;
                    if (Cfg::BNN > 0 && slices * cdiv(p.N, Cfg::BNT) < device_cus()) {
                        q.xcd_run = xcd_run_for(slices * cdiv(p.N, Cfg::BNN));
                        launch_bf16<Cfg::BMT, Cfg::BNN, Cfg::WMT, Cfg::WNN, Cfg::RN::NS, Cfg::RN::BK, MODE,
                                    ALAY, BLAY, DUAL, KSPLIT, G>(q, epi, R, ts, tail_name);
                    } else {
                        q.xcd_run = xcd_run_for(slices * cdiv(p.N, Cfg::BNT));
                        launch_bf16<Cfg::BMT, Cfg::BNT, Cfg::WMT, Cfg::WNT, Cfg::RT::NS, Cfg::RT::BK, MODE,
                                    ALAY, BLAY, DUAL, KSPLIT, G>(q, epi, R, ts, tail_name);
                    }
                    return true;
                }
            }
            launch_bf16<Cfg::BM, Cfg::BN, Cfg::WM, Cfg::WN, RR::NS, RR::BK, MODE, ALAY, BLAY, DUAL,
                        KSPLIT, G>(p, epi, R, s, name);
            return false;
        }
    }
    static constexpr int BM = Cfg::BM;
};

template <class Cfg>
struct Launch<float, Cfg> {
    template <int MODE, bool DUAL>
    static bool splits(int, int, int) { return false; }
    template <int MODE, int ALAY, int BLAY, bool DUAL, bool KSPLIT, bool G = false, class Epi>
    static bool go(GemmArgs<float> p, Epi epi, int R, hipStream_t s, const char* name,
                   const char* = nullptr, hipStream_t = nullptr) {
        launch_f32<MODE, ALAY, BLAY, DUAL, KSPLIT>(p, epi, R, s, name);
        return false;
    }
    static constexpr int BM = FB;
};

// Whether the FFN backward runs its partial-tile launches and dW2 on the side
// stream beside the main launches (the forward keeps everything on the
// caller's stream).  With per-expert weights up to 8 Mi
// elements (16 MB in bf16; the MoE-S-like and 64-expert shapes) the side
// work fills the last, partly idle rounds: 1-2% faster steps.  With larger
// ones (d 2048 x f 8192, d 4096 x f 14336) two products in flight at once
// lost more to each other than they gained: the skewed and long-context
// steps were 3% and 1% faster with everything on the caller's stream.
inline bool side_stream_pays(int d, int f) { return (long)d * f <= (8L << 20); }

// One dW product (RAGGED_K), with the ring that suits the segment length.
template <typename T, class Cfg, bool G, class Epi>
void dw_go(bool long_k, const GemmArgs<T>& p, Epi epi, int R, hipStream_t s, const char* name) {
    if constexpr (sizeof(T) == 2) {
        if (long_k) {
            Launch<T, LongKCfg<Cfg>>::template go<RAGGED_K, MNMAJ, MNMAJ, false, false, G>(
                p, epi, R, s, name);
            return;
        }
    }
    Launch<T, Cfg>::template go<RAGGED_K, MNMAJ, MNMAJ, false, false, G>(p, epi, R, s, name);
}

template <typename T, class Cfg = DefaultCfg>
moe_status ffn_fwd(const void* x_perm, const int32_t* offsets, int R, int E,
                   int d, int f, moe_act act, const void* W1, const void* W3,
                   const void* W2, void* h_save, void* a_save, void* out_perm,
                   void* ws, hipStream_t s, const int32_t* gather = nullptr, long T_src = 0) {
    // gather != NULL: x_perm is the token-order input [T_src,d] and permuted row
    // r is its row gather[r] (the permute's row copy fused into GEMM1)
    const FfnWs L = ffn_layout(R, E, d, f, act, sizeof(T) == 2 ? MOE_BF16 : MOE_F32, 0);
    char* base = static_cast<char*>(ws);
    int32_t* prefix = reinterpret_cast<int32_t*>(base + L.prefix);
    int32_t* order = reinterpret_cast<int32_t*>(base + L.order);
    int32_t* full = reinterpret_cast<int32_t*>(base + L.full);
    int32_t* part = reinterpret_cast<int32_t*>(base + L.part);
    const Plan pl{prefix, order, full, part};
    MOE_LAUNCH("ffn_plan", s,
               ffn_plan_kernel<<<1, 1024, 0, s>>>(offsets, E, Launch<T, Cfg>::BM, 0, prefix,
                                                  order, full, part, nullptr, nullptr,
                                                  nullptr));

    const T* xp = static_cast<const T*>(x_perm);
    T* H = static_cast<T*>(h_save);
    T* A = static_cast<T*>(a_save);
    // GEMM1 (+ activation): [R,d] x W1[e] [d,f]
    GemmArgs<T> p = base_args<T>(offsets, pl, E);
    p.A = xp; p.lda = d;
    p.gather = gather; p.gather_rows = T_src;
    p.B = static_cast<const T*>(W1); p.ldb = f; p.bstride = (long)d * f;
    p.N = f; p.K = d;
    // GEMM2: A [R,f] x W2[e] [f,d]
    GemmArgs<T> q = base_args<T>(offsets, pl, E);
    q.A = A; q.lda = f;
    q.B = static_cast<const T*>(W2); q.ldb = d; q.bstride = (long)f * d;
    q.N = d; q.K = f;
    if (act == MOE_ACT_SWIGLU) {       // one launch over all rows, before the fork
        p.B2 = static_cast<const T*>(W3);
        Launch<T, Cfg>::template go<RAGGED_M, KMAJ, MNMAJ, true, false, true>(
            p, EpiSwigluFwd<T>{H, A, f}, R, s, "gemm_up_swiglu");
    }
    // The experts' full tiles (main launches) and their partial last tiles
    // (tail launches) run one after the other on the caller's stream.  On
    // the side stream the tails only stretched the up GEMM's main launch
    // (kernel trace of the MoE-S-like step: 177 -> 277 us), and the steps were
    // 0.2-0.6% slower than with the forward on one stream.
    if (act == MOE_ACT_GELU)
        Launch<T, Cfg>::template go<RAGGED_M, KMAJ, MNMAJ, false, false, true>(
            p, EpiGeluFwd<T>{H, A, f}, R, s, "gemm_up_gelu", "gemm_up_gelu_tail", s);
    if (!out_perm)                     // GEMM1 only (recomputation of the saved state)
        return launch_status();
    Launch<T, Cfg>::template go<RAGGED_M, KMAJ, MNMAJ, false, false>(
        q, EpiStore<T>{static_cast<T*>(out_perm), d, 0}, R, s, "gemm_down", "gemm_down_tail",
        s);
    return launch_status();
}

template <typename T, class Cfg = DefaultCfg>
moe_status ffn_bwd(const void* d_out, const void* x_perm, const void* h_save,
                   const void* a_save, const int32_t* offsets, int R, int E,
                   int d, int f, moe_act act, const void* W1, const void* W3,
                   const void* W2, void* dx_perm, void* dW1, void* dW3,
                   void* dW2, void* ws, hipStream_t s, const int32_t* gather = nullptr,
                   long T_src = 0, bool accumulate = false) {
    // accumulate: dW1/dW2/dW3 += the products (fp32 sum, one rounding)
    // gather != NULL: x_perm is the token-order input [T_src,d]; dW1/dW3 read
    // permuted row r as its row gather[r]
    const FfnWs L = ffn_layout(R, E, d, f, act, sizeof(T) == 2 ? MOE_BF16 : MOE_F32, 1);
    const bool long_k = (long)R >= kLongSegmentRows * E;     // ring of the dW products
    char* base = static_cast<char*>(ws);
    int32_t* prefix = reinterpret_cast<int32_t*>(base + L.prefix);
    int32_t* order = reinterpret_cast<int32_t*>(base + L.order);
    int32_t* full = reinterpret_cast<int32_t*>(base + L.full);
    int32_t* part = reinterpret_cast<int32_t*>(base + L.part);
    const Plan pl{prefix, order, full, part};
    T* dH = reinterpret_cast<T*>(base + L.dh);
    const bool sw = act == MOE_ACT_SWIGLU;
    const long ldh = sw ? 2L * f : (long)f;
    // dW work items (bf16): whole segments and the chunks of split ones
    int4* items = L.item_max ? reinterpret_cast<int4*>(base + L.items) : nullptr;
    int4* splits = reinterpret_cast<int4*>(base + L.splits);
    int32_t* counts = reinterpret_cast<int32_t*>(base + L.counts);
    MOE_LAUNCH("ffn_plan", s,
               ffn_plan_kernel<<<1, 1024, 0, s>>>(offsets, E, Launch<T, Cfg>::BM,
                                                  dw_tiles_of(d, f), prefix, order, full,
                                                  part, items, splits, counts));
    // a dW product over the work items; part: its fp32 partial region
    auto with_items = [&](GemmArgs<T>& p, size_t part_off) {
        if (!items) return;
        p.items = items;
        p.item_count = counts;
        p.item_max = (int)L.item_max;
        p.partial = reinterpret_cast<float*>(base + part_off);
        p.partial_ld = (long)d * f;
    };
    // the split segments' dW: their chunks summed in order, into C (+=)
    auto reduce_splits = [&](void* C, size_t part_off, hipStream_t st, const char* name) {
        if (!items || L.split_max == 0) return;
        const long mn = (long)d * f;
        const dim3 grid((unsigned)cdiv(mn, 256 * 8), (unsigned)L.split_max);
        MOE_LAUNCH(name, st,
                   dw_split_reduce_kernel<T><<<grid, 256, 0, st>>>(
                       splits, counts, reinterpret_cast<const float*>(base + part_off), mn,
                       static_cast<T*>(C), mn, accumulate ? 1 : 0));
    };

    const T* dO = static_cast<const T*>(d_out);
    // Caller's stream: dA (full tiles) -> dX (full tiles) -> dW1, dW3.
    // Side stream:     dA (partial tiles) -> dW2 -> dX (partial tiles).
    // dW2 depends on neither dA nor dX; dW1/dW3 need every row of dH.  A
    // product that is not split runs whole on the caller's stream, and the
    // stream that consumes its rows waits for it.
    SideStream side(s, side_stream_pays(d, f));
    hipStream_t ts = side.ok() ? side.get() : s;
    bool dA_split = false;
    // dA = dO W2[e]^T with the activation derivative in the epilogue -> dH
    {
        GemmArgs<T> p = base_args<T>(offsets, pl, E);
        p.A = dO; p.lda = d;
        p.B = static_cast<const T*>(W2); p.ldb = d; p.bstride = (long)f * d;
        p.N = f; p.K = d;
        if (!sw)
            dA_split = Launch<T, Cfg>::template go<RAGGED_M, KMAJ, KMAJ, false, false>(
                p, EpiGeluBwd<T>{static_cast<const T*>(h_save), dH, f}, R, s, "gemm_dA_gelu",
                "gemm_dA_gelu_tail", ts);
        else
            dA_split = Launch<T, Cfg>::template go<RAGGED_M, KMAJ, KMAJ, false, false>(
                p, EpiSwigluBwd<T>{static_cast<const T*>(h_save), dH, f}, R, s,
                "gemm_dA_swiglu", "gemm_dA_swiglu_tail", ts);
        if (side.ok() && dA_split && !side.mark(1)) return MOE_ERR_HIP;  // dH, partial tiles
    }
    // dW2[e] = A_e^T dO_e   [f, d]
    {
        GemmArgs<T> p = base_args<T>(offsets, pl, E);
        p.A = static_cast<const T*>(a_save); p.lda = f; p.M = f;
        p.B = dO; p.ldb = d; p.N = d;
        with_items(p, L.part0);
        if (accumulate)
            dw_go<T, Cfg, false>(long_k, p, EpiAcc<T>{static_cast<T*>(dW2), d, (long)f * d}, R,
                                 ts, "gemm_dW2");
        else
            dw_go<T, Cfg, false>(long_k, p, EpiStore<T>{static_cast<T*>(dW2), d, (long)f * d},
                                 R, ts, "gemm_dW2");
        reduce_splits(dW2, L.part0, ts, "dw_split_reduce");
    }
    // dX = dH1 W1[e]^T (+ dH3 W3[e]^T)   [R, d]
    const bool dX_split = Launch<T, Cfg>::template splits<RAGGED_M, false>(R, E, d);
    if (side.ok() && dA_split != dX_split) {
        // dA split, dX whole: dX (caller's stream) needs the side's rows of dH;
        // dA whole, dX split: dX's tail (side stream) needs dH made on s
        const bool ok = dA_split ? side.wait(1) : side.follow();
        if (!ok) return MOE_ERR_HIP;
    }
    {
        GemmArgs<T> p = base_args<T>(offsets, pl, E);
        p.A = dH; p.lda = ldh;
        p.B = static_cast<const T*>(W1); p.ldb = f; p.bstride = (long)d * f;
        p.N = d;
        EpiStore<T> st{static_cast<T*>(dx_perm), d, 0};
        if (!sw) {
            p.K = f;
            Launch<T, Cfg>::template go<RAGGED_M, KMAJ, KMAJ, false, false>(p, st, R, s, "gemm_dX",
                                                                            "gemm_dX_tail", ts);
        } else {
            p.K = 2 * f;
            p.Ksplit = f;
            p.B2 = static_cast<const T*>(W3);
            Launch<T, Cfg>::template go<RAGGED_M, KMAJ, KMAJ, false, true>(p, st, R, s, "gemm_dX",
                                                                           "gemm_dX_tail", ts);
        }
    }
    // dW1[e] = X_e^T dH1_e  [d, f]   (dW3 with dH3): needs every row of dH
    if (side.ok() && dA_split && !side.wait(1)) return MOE_ERR_HIP;
    {
        GemmArgs<T> p = base_args<T>(offsets, pl, E);
        p.A = static_cast<const T*>(x_perm); p.lda = d; p.M = d;
        p.gather = gather; p.gather_rows = T_src;
        p.B = dH; p.ldb = ldh; p.N = f;
        with_items(p, L.part1);
        auto dw = [&](void* C, const char* name) {
            if (accumulate)
                dw_go<T, Cfg, true>(long_k, p, EpiAcc<T>{static_cast<T*>(C), f, (long)d * f}, R,
                                    s, name);
            else
                dw_go<T, Cfg, true>(long_k, p, EpiStore<T>{static_cast<T*>(C), f, (long)d * f},
                                    R, s, name);
            reduce_splits(C, L.part1, s, "dw_split_reduce");
        };
        dw(dW1, "gemm_dW1");
        if (sw) {
            p.B = dH + f;
            dw(dW3, "gemm_dW3");
        }
    }
    if (side.ok() && !side.join()) return MOE_ERR_HIP;
    return launch_status();
}

// Device address of `scratch` per device, resolved once per device with that
// device current (moe_init, or the first no-alloc call on the device).
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];

moe_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kScratchDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return MOE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// ------------------------------------------------------------ LDS probe
// The rates of the LDS paths of the main loop, alone and side by side
// (moe_lds_probe).  Bits of MODE: 1 plain 16-byte fragment reads
// (ds_read_b128), 2 transposing 8-byte reads of M/N-contiguous operands
// (ds_read_b64_tr_b16), 4 direct-to-LDS buffer loads of the ring
// (buffer_load_dwordx4 ... lds, lds_dma16) from a source window of
// win_mask + 1 bytes; 8: the reads three times per round, the ratio of
// fragment reads to ring loads of a 256 x 256 tile.  Each wave reads its own
// 8 KB and loads into another 8 KB; lanes take consecutive 16- (8-) byte
// slots, so a read touches every bank once per phase.  Every kind moves 8 KB
// per wave and round (the reads 24 KB with bit 8).
constexpr int PROBE_WAVE_LDS = 8192;

template <int MODE>
__global__ __launch_bounds__(256) void lds_probe_kernel(const bf16_t* src, uint32_t win_mask,
                                                        int iters, float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint8_t rd[4 * PROBE_WAVE_LDS];
    __shared__ __attribute__((aligned(16))) uint8_t dm[4 * PROBE_WAVE_LDS];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint8_t* my = rd + w * PROBE_WAVE_LDS;
    for (int i = lane; i < PROBE_WAVE_LDS / 16; i += 64)
        reinterpret_cast<uint4*>(my)[i] = make_uint4(i, lane, w, blockIdx.x);
    wave_lds_sync();
    uint32_t acc = 0;
    const uint32_t gw = blockIdx.x * 4 + w;
    const uint32_t ldm = lds_addr(dm + w * PROBE_WAVE_LDS);
    for (int it = 0; it < iters; ++it) {
        asm volatile("" ::: "memory");       // the reads are issued again every round
        if constexpr ((MODE & 4) != 0) {
            const i32x4_t rs = rsrc_words(src, (long)win_mask + 1);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t o = ((gw * 8 + j + (uint32_t)it * 8) * 1024 + lane * 16) & win_mask;
                lds_dma16(rs, o, ldm + j * 1024);
            }
        }
        constexpr int NR = (MODE & 8) != 0 ? 3 : 1;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            if (r > 0) asm volatile("" ::: "memory");   // read again, not reuse
            if constexpr ((MODE & 1) != 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint4 v = *reinterpret_cast<const uint4*>(my + j * 1024 + lane * 16);
                    acc ^= v.x ^ v.y ^ v.z ^ v.w;
                }
            }
            if constexpr ((MODE & 2) != 0) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_v4i16_t*)(my + j * 512 + lane * 8));
                    acc ^= (uint32_t)(uint16_t)v[0] ^ ((uint32_t)(uint16_t)v[1] << 16) ^
                           (uint32_t)(uint16_t)v[2] ^ ((uint32_t)(uint16_t)v[3] << 16);
                }
            }
        }
        if constexpr ((MODE & 4) != 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if (lane == 0) out[gw] = (float)acc;
}

moe_status ffn_check(int R, int E, int d, int f, moe_act act, moe_dtype dt) {
    if (R < 0 || E < 1 || E > 1024 || d < 64 || f < 64) return MOE_ERR_INVALID_ARG;
    if (d % 64 != 0 || f % 64 != 0) return MOE_ERR_INVALID_ARG;
    if (act != MOE_ACT_GELU && act != MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARG;
    if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

}  // namespace

// moe_init's set-up of this file: the scratch address of the current device.
moe_status ffn_scratch_init() {
    void* p = nullptr;
    return scratch_address(&p);
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_ffn_workspace_bytes(int R, int E, int d, int f, moe_act act,
                               moe_dtype dt, int backward) {
    if (ffn_check(R, E, d, f, act, dt) != MOE_OK) return 0;
    return ffn_layout(R, E, d, f, act, dt, backward).total;
}

moe_status moe_expert_ffn_fwd(const void* x_perm, const int32_t* offsets,
                              int R, int E, int d, int f, moe_act act,
                              moe_dtype dt, const void* W1, const void* W3,
                              const void* W2, void* h_save, void* a_save,
                              void* out_perm, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
    moe_status st = ffn_check(R, E, d, f, act, dt);
    if (st != MOE_OK) return st;
    if (R == 0) return MOE_OK;
    // out_perm == NULL: GEMM1 only (h_save and a_save), W2 unused
    MOE_CHECK_ARG(x_perm && offsets && W1 && h_save && a_save && (W2 || !out_perm));
    MOE_CHECK_ARG(act != MOE_ACT_SWIGLU || W3);
    MOE_CHECK_ARG(aligned16(x_perm) && aligned16(W1) && (!W2 || aligned16(W2)) &&
                  aligned16(h_save) && aligned16(a_save) && (!out_perm || aligned16(out_perm)) &&
                  (W3 == nullptr || aligned16(W3)));
    if (!ws || ws_bytes < moe_ffn_workspace_bytes(R, E, d, f, act, dt, 0))
        return MOE_ERR_WORKSPACE;
    MOE_CHECK_DEVICE();
    if (dt == MOE_BF16)
        return ffn_fwd<bf16_t>(x_perm, offsets, R, E, d, f, act, W1, W3, W2, h_save,
                               a_save, out_perm, ws, stream);
    return ffn_fwd<float>(x_perm, offsets, R, E, d, f, act, W1, W3, W2, h_save, a_save,
                          out_perm, ws, stream);
}

moe_status moe_expert_ffn_bwd(const void* d_out_perm, const void* x_perm,
                              const void* h_save, const void* a_save,
                              const int32_t* offsets, int R, int E, int d,
                              int f, moe_act act, moe_dtype dt, const void* W1,
                              const void* W3, const void* W2, void* dx_perm,
                              void* dW1, void* dW3, void* dW2, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
    moe_status st = ffn_check(R, E, d, f, act, dt);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(offsets && W1 && W2 && dW1 && dW2);
    MOE_CHECK_ARG(act != MOE_ACT_SWIGLU || (W3 && dW3));
    MOE_CHECK_ARG(R == 0 || (d_out_perm && x_perm && h_save && a_save && dx_perm));
    if (!ws || ws_bytes < moe_ffn_workspace_bytes(R, E, d, f, act, dt, 1))
        return MOE_ERR_WORKSPACE;
    MOE_CHECK_DEVICE();
    // R == 0 still writes dW = 0 (every expert is empty)
    if (dt == MOE_BF16)
        return ffn_bwd<bf16_t>(d_out_perm, x_perm, h_save, a_save, offsets, R, E, d, f,
                               act, W1, W3, W2, dx_perm, dW1, dW3, dW2, ws, stream);
    return ffn_bwd<float>(d_out_perm, x_perm, h_save, a_save, offsets, R, E, d, f, act,
                          W1, W3, W2, dx_perm, dW1, dW3, dW2, ws, stream);
}

// moe_expert_ffn_bwd with dW1/dW2/dW3 += instead of =: the gradient of one
// chunk of tokens added to the chunks before it.
moe_status moe_expert_ffn_bwd_accumulate(const void* d_out_perm, const void* x_perm,
                                         const void* h_save, const void* a_save,
                                         const int32_t* offsets, int R, int E, int d, int f,
                                         moe_act act, moe_dtype dt, const void* W1,
                                         const void* W3, const void* W2, void* dx_perm,
                                         void* dW1, void* dW3, void* dW2, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
    moe_status st = ffn_check(R, E, d, f, act, dt);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(offsets && W1 && W2 && dW1 && dW2);
    MOE_CHECK_ARG(act != MOE_ACT_SWIGLU || (W3 && dW3));
    MOE_CHECK_ARG(R == 0 || (d_out_perm && x_perm && h_save && a_save && dx_perm));
    if (!ws || ws_bytes < moe_ffn_workspace_bytes(R, E, d, f, act, dt, 1))
        return MOE_ERR_WORKSPACE;
    MOE_CHECK_DEVICE();
    if (R == 0) return MOE_OK;         // nothing to add
    if (dt == MOE_BF16)
        return ffn_bwd<bf16_t>(d_out_perm, x_perm, h_save, a_save, offsets, R, E, d, f, act,
                               W1, W3, W2, dx_perm, dW1, dW3, dW2, ws, stream, nullptr, 0,
                               true);
    return ffn_bwd<float>(d_out_perm, x_perm, h_save, a_save, offsets, R, E, d, f, act, W1,
                          W3, W2, dx_perm, dW1, dW3, dW2, ws, stream, nullptr, 0, true);
}

// moe_expert_ffn_fwd with its workspace (the tile plan) in the library's
// static scratch array of the current device: no allocation, no workspace
// argument.  Calls that overlap in time on one GPU share that array and race.
moe_status moe_expert_ffn_fwd_noalloc(const void* x_perm, const int32_t* offsets, int R,
                                      int E, int d, int f, moe_act act, moe_dtype dt,
                                      const void* W1, const void* W3, const void* W2,
                                      void* h_save, void* a_save, void* out_perm,
                                      hipStream_t stream) {
    moe_status st = ffn_check(R, E, d, f, act, dt);
    if (st != MOE_OK) return st;
    if (moe_ffn_workspace_bytes(R, E, d, f, act, dt, 0) > kFfnScratchBytes)
        return MOE_ERR_WORKSPACE;
    MOE_CHECK_DEVICE();
    void* ws = nullptr;
    if ((st = scratch_address(&ws)) != MOE_OK) return st;
    return moe_expert_ffn_fwd(x_perm, offsets, R, E, d, f, act, dt, W1, W3, W2, h_save,
                              a_save, out_perm, ws, kFfnScratchBytes, stream);
}

// The permute's row copy fused into the expert GEMMs: x is read in token
// order through src.  The 32-bit buffer offsets of the bf16 path bound the
// source at 2^31 bytes.
static moe_status gather_check(const void* x, const int32_t* src, int T, int R, int d,
                               moe_dtype dt) {
    MOE_CHECK_ARG(T >= 0 && (R == 0 || (T > 0 && x && src && aligned16(x))));
    if (dt == MOE_BF16 && (long long)T * d * 2 >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status moe_expert_ffn_fwd_gather(const void* x, const int32_t* src,
                                     const int32_t* offsets, int T, int R, int E, int d,
                                     int f, moe_act act, moe_dtype dt, const void* W1,
                                     const void* W3, const void* W2, void* h_save,
                                     void* a_save, void* out_perm, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
    moe_status st = ffn_check(R, E, d, f, act, dt);
    if (st != MOE_OK) return st;
    if ((st = gather_check(x, src, T, R, d, dt)) != MOE_OK) return st;
    if (R == 0) return MOE_OK;
    MOE_CHECK_ARG(offsets && W1 && h_save && a_save && (W2 || !out_perm));
    MOE_CHECK_ARG(act != MOE_ACT_SWIGLU || W3);
    MOE_CHECK_ARG(aligned16(W1) && (!W2 || aligned16(W2)) && aligned16(h_save) &&
                  aligned16(a_save) && (!out_perm || aligned16(out_perm)) &&
                  (W3 == nullptr || aligned16(W3)));
    if (!ws || ws_bytes < moe_ffn_workspace_bytes(R, E, d, f, act, dt, 0))
        return MOE_ERR_WORKSPACE;
    MOE_CHECK_DEVICE();
    if (dt == MOE_BF16)
        return ffn_fwd<bf16_t>(x, offsets, R, E, d, f, act, W1, W3, W2, h_save, a_save,
                               out_perm, ws, stream, src, T);
    return ffn_fwd<float>(x, offsets, R, E, d, f, act, W1, W3, W2, h_save, a_save, out_perm,
                          ws, stream, src, T);
}

moe_status moe_expert_ffn_bwd_gather(const void* d_out_perm, const void* x,
                                     const int32_t* src, const void* h_save,
                                     const void* a_save, const int32_t* offsets, int T,
                                     int R, int E, int d, int f, moe_act act, moe_dtype dt,
                                     const void* W1, const void* W3, const void* W2,
                                     void* dx_perm, void* dW1, void* dW3, void* dW2,
                                     void* ws, size_t ws_bytes, hipStream_t stream) {
    moe_status st = ffn_check(R, E, d, f, act, dt);
    if (st != MOE_OK) return st;
    if ((st = gather_check(x, src, T, R, d, dt)) != MOE_OK) return st;
    MOE_CHECK_ARG(offsets && W1 && W2 && dW1 && dW2);
    MOE_CHECK_ARG(act != MOE_ACT_SWIGLU || (W3 && dW3));
    MOE_CHECK_ARG(R == 0 || (d_out_perm && h_save && a_save && dx_perm));
    if (!ws || ws_bytes < moe_ffn_workspace_bytes(R, E, d, f, act, dt, 1))
        return MOE_ERR_WORKSPACE;
    MOE_CHECK_DEVICE();
    if (dt == MOE_BF16)
        return ffn_bwd<bf16_t>(d_out_perm, x, h_save, a_save, offsets, R, E, d, f, act, W1,
                               W3, W2, dx_perm, dW1, dW3, dW2, ws, stream, src, T);
    return ffn_bwd<float>(d_out_perm, x, h_save, a_save, offsets, R, E, d, f, act, W1, W3,
                          W2, dx_perm, dW1, dW3, dW2, ws, stream, src, T);
}


moe_status moe_lds_probe(int mode, int blocks, int iters, const void* src, size_t src_bytes,
                         float* out, size_t out_floats, hipStream_t stream) {
    MOE_CHECK_ARG(mode >= 1 && mode <= 15 && (mode & 7) != 0);
    MOE_CHECK_ARG(blocks >= 1 && iters >= 1 && out);
    MOE_CHECK_ARG(out_floats >= (size_t)blocks * 4);
    if (mode & 4) {
        MOE_CHECK_ARG(src && aligned16(src));
        MOE_CHECK_ARG(src_bytes >= 8192 && src_bytes <= (1u << 30) &&
                      (src_bytes & (src_bytes - 1)) == 0);
    }
    MOE_CHECK_DEVICE();
    const bf16_t* sp = static_cast<const bf16_t*>(src);
    const uint32_t wm = (mode & 4) ? (uint32_t)(src_bytes - 1) : 0u;
    switch (mode) {
#define PROBE_CASE(M)                                                                    \
    case M:                                                                              \
        MOE_LAUNCH("lds_probe", stream,                                                  \
                   lds_probe_kernel<M><<<blocks, 256, 0, stream>>>(sp, wm, iters, out)); \
        break;
        PROBE_CASE(1) PROBE_CASE(2) PROBE_CASE(3) PROBE_CASE(4) PROBE_CASE(5) PROBE_CASE(6)
        PROBE_CASE(7) PROBE_CASE(9) PROBE_CASE(10) PROBE_CASE(11) PROBE_CASE(12)
        PROBE_CASE(13) PROBE_CASE(14) PROBE_CASE(15)
#undef PROBE_CASE
    }
    return launch_status();
}

}  // extern "C"
