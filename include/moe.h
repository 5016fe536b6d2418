/*
 * libmoe -- MoE layer forward and backward on one AMD Instinct MI355X (gfx950).
 *
 * The layer: a gate scores each token against every expert, each token goes
 * to its k best experts, the (token, slot) pairs are counting-sorted into one
 * contiguous, unpadded segment per expert, every expert runs its FFN on its
 * segment as one grouped GEMM, and the outputs are gathered back to token
 * order weighted by the gate.  Backward runs the same steps in reverse.
 *
 * Sources (page title, section):
 *  - "ES-MoE: Scaling Beyond the GPU Memory Limit for Large Mixture-of-Experts
 *    Model Training" (xllm-io paper review), 三 技术架构 / 专家级卸载与处理 and
 *    四 核心创新: expert placement follows the gate; tokens are assigned to
 *    their experts in sequence instead of a batched matmul over a dense
 *    dispatch mask; zero padding is removed (自适应卸载, GPU-only mode).
 *  - "FastMoE: A Fast Mixture-of-Expert Training System" (nubint.ai review),
 *    제안 방법: a scatter/gather layout batches each expert's inputs; the
 *    expert FFN runs the experts' linear layers in parallel.
 *  - "Flattening Every Memory Peak in Long-Context Mixture-of-Experts
 *    Training", abstract: the dispatch buffer grows with the routing matrix;
 *    reordering work leaves loss and gradients exact.
 *
 * Conventions shared by every entry point
 *  - All tensors are device pointers to dense row-major arrays.  Element type
 *    of x, weights, activations and their gradients is `dt` (MOE_F32 or
 *    MOE_BF16); logits, gate weights and their gradients are always float;
 *    indices are int32.
 *  - The caller owns every buffer, including workspaces; the library never
 *    allocates or frees device memory and never copies device -> host.
 *  - Every call is asynchronous on `stream`.  Arguments are validated on the
 *    host before anything is launched; on error nothing is launched and the
 *    status says why.  No C++ exception crosses this interface.
 *  - Outputs are overwritten unless an argument says "accumulated".
 *  - Bit-reproducible: no float atomics; every reduction has a fixed order.
 *  - Limits: 1 <= k <= E <= 1024; T*k < 2^31; d a multiple of 8 for the gate
 *    and the permute, of 64 for the FFN, combine and unpermute; f a multiple
 *    of 64; device pointers to rows 16-byte aligned.  T = 0 (R = 0) is
 *    accepted: nothing of the tokens is read and their pointers may be NULL;
 *    outputs with entries are still written: the permute's counts and
 *    offsets, the FFN backward's dW and the gate backward's dWg (all zeros;
 *    dW unchanged by the accumulating FFN backward).
 *  - Threads: entry points are reentrant; concurrent calls on different
 *    streams must not share output or workspace buffers.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,  /* bad size, null pointer, misaligned pointer */
    MOE_ERR_UNSUPPORTED = -2,  /* device is not gfx950, or dtype/act not built */
    MOE_ERR_WORKSPACE = -3,    /* workspace too small (see *_workspace_bytes) */
    MOE_ERR_HIP = -4           /* a HIP runtime call or launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum { MOE_ACT_GELU = 0, MOE_ACT_SWIGLU = 1 } moe_act;

/* Human-readable text of a status code (static storage). */
const char *moe_status_string(moe_status s);

/* Interface version; bumped on any signature change. */
int moe_abi_version(void);

/*
 * moe_init -- check that `device` is a gfx950 GPU and cache its properties.
 * Optional: every entry point checks the current device itself on first use.
 * Returns MOE_ERR_UNSUPPORTED for another architecture.
 */
moe_status moe_init(int device);

/*
 * moe_set_overlap -- whether moe_expert_ffn_bwd (and its _accumulate and
 * _gather forms) may run launches that do not depend on each other (the
 * experts' partial last tiles, dW2) on a library-owned side stream of the
 * current device, concurrently with the rest of the call on `stream`
 * (enable != 0, the default; used only when an expert's weight has at most
 * 8 Mi elements, where it pays), or run every kernel in order on `stream`
 * (enable = 0).  Either way a call is ordered on `stream` as a whole (the
 * side stream forks from it and joins back through events) and the results
 * are bit-identical.  Every other call runs in order on `stream`.
 * Process-wide setting.  While kernel timing is enabled (moe_profile_enable)
 * the library runs as with enable = 0 so that every timed kernel runs alone.
 */
moe_status moe_set_overlap(int enable);

/*
 * moe_gate_topk -- gate scores, top-k choice and gate weights.
 *   logits[t,e] = sum_{i=0..d-1} x[t,i]*Wg[i,e] (+ logit_bias[e]), fp32,
 *                 summed in increasing i with every product and sum rounded
 *                 (bf16 products are exact in fp32, so a fused chain gives the
 *                 same bits); this fixed order makes the routing reproducible.
 *   topk_idx[t,j] = index of the j-th largest logit (ties: lower index first).
 *   topk_w[t,j]   = renorm ? softmax over the k selected logits
 *                          : softmax over all E logits, at the selected expert.
 * Source: ES-MoE review, 三 技术架构 (placement known after the gating network);
 * the gate formula is not printed -- linear gate + softmax top-k is the reading.
 *   x [T,d] dt, Wg [d,E] dt, logit_bias [E] float or NULL (a workload input,
 *   not a trained parameter), logits [T,E] float, topk_idx [T,k] int32,
 *   topk_w [T,k] float.
 */
moe_status moe_gate_topk(const void *x, const void *Wg, const float *logit_bias,
                         int T, int d, int E, int k, int renorm, moe_dtype dt,
                         float *logits, int32_t *topk_idx, float *topk_w,
                         hipStream_t stream);

/*
 * moe_permute -- stable counting sort of the (token, slot) pairs by expert
 * and the row copy into expert-segment order.  No dispatch mask, no padding.
 *   counts[e]   = number of pairs routed to e
 *   offsets[e]  = sum_{e'<e} counts[e'], offsets[E] = T*k
 *   dest[t,j]   = offsets[e] + #{t' < t : e in topk_idx[t']}, e = topk_idx[t,j]
 *   src[r]      = token of permuted row r (src[dest[t,j]] = t)
 *   x_perm[r,:] = x[src[r],:]
 * Integer outputs are exact and independent of scheduling (no atomic-order
 * dependence).  Sources: ES-MoE review, 三 技术架构 / 专家级卸载与处理 (tokens
 * assigned to experts in sequence); FastMoE review, 제안 방법 (scatter/gather
 * layout by expert).
 *   topk_idx [T,k] int32 (each row: k distinct experts in [0,E)), x [T,d] dt,
 *   counts [E], offsets [E+1], dest [T,k], src [T*k] int32, x_perm [T*k,d] dt.
 *   x_perm == NULL skips the row copy (x may then be NULL too): routing only,
 *   for the *_gather FFN entry points, which read x through src.
 *   ws: device workspace of at least moe_permute_workspace_bytes(T,E,k).
 * Entries of topk_idx outside [0,E) are a caller error that the device
 * cannot report: such a pair is left out of counts and offsets (offsets[E]
 * is then the number of valid pairs), its dest entry is set to -1 (which
 * moe_combine, moe_combine_bwd and moe_unpermute_grad skip) and src holds
 * no entry for it (src[offsets[E]..T*k-1] are left as they were).
 */
size_t moe_permute_workspace_bytes(int T, int E, int k);
moe_status moe_permute(const int32_t *topk_idx, const void *x, int T, int d,
                       int E, int k, moe_dtype dt, int32_t *counts,
                       int32_t *offsets, int32_t *dest, int32_t *src,
                       void *x_perm, void *ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * moe_expert_ffn_fwd -- every expert's FFN on its segment, one grouped GEMM
 * per product over the ragged segments (rows offsets[e]..offsets[e+1]).
 *   GeLU:   H = X_e W1[e], A = GeLU(H) (erf form), O = A W2[e]
 *   SwiGLU: H1 = X_e W1[e], H3 = X_e W3[e], A = SiLU(H1)*H3, O = A W2[e]
 * For bf16 the normal CDF inside GeLU is evaluated with the rational
 * approximation of erf of Abramowitz & Stegun 7.1.26 (|error| <= 1.5e-7).
 * Source: FastMoE review, 제안 방법 (dedicated expert FFN, parallel expert
 * linear layers); ES-MoE review, 三 技术架构 (experts take their tokens in
 * sequence, no padding).
 *   x_perm [R,d] dt, offsets [E+1] int32 (device; absolute row indices,
 *     nondecreasing, offsets[E] <= R; rows outside offsets[0]..offsets[E] are
 *     neither read nor written, so experts e0..e0+E-1 of a larger routing are
 *     passed as offsets + e0 with E = their count and their own weights),
 *   W1 [E,d,f], W3 [E,d,f] (SwiGLU only, else NULL), W2 [E,f,d] dt,
 *   h_save: what the backward needs of the pre-activation, computed from the
 *     fp32 accumulator: GeLU: [R,f] = GeLU'(H); SwiGLU: [R,2f], row r =
 *     H3*SiLU'(H1) then SiLU(H1).  Only moe_expert_ffn_bwd reads it.
 *   a_save [R,f] (A), out_perm [R,d] dt.  Accumulation is fp32.
 *   out_perm == NULL: GEMM1 only (h_save and a_save; W2 may be NULL) -- the
 *   recomputation of the saved state for a chunk's backward.
 *   ws: at least moe_ffn_workspace_bytes(R,E,d,f,act,dt,0).
 */
size_t moe_ffn_workspace_bytes(int R, int E, int d, int f, moe_act act,
                               moe_dtype dt, int backward);
moe_status moe_expert_ffn_fwd(const void *x_perm, const int32_t *offsets,
                              int R, int E, int d, int f, moe_act act,
                              moe_dtype dt, const void *W1, const void *W3,
                              const void *W2, void *h_save, void *a_save,
                              void *out_perm, void *ws, size_t ws_bytes,
                              hipStream_t stream);

/*
 * moe_expert_ffn_fwd_noalloc -- moe_expert_ffn_fwd for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments and
 * results (bit-identical) without ws/ws_bytes: the tile plan the forward
 * needs (17 KiB at most, E <= 1024) lives in a library-owned static device
 * array of 32 KiB per GPU, held until the process ends; its address is
 * resolved by moe_init (or by the first call on a device).  The call
 * allocates nothing and calls no allocating routine.  Every call on one GPU
 * shares that array: calls that overlap in time on one GPU (other streams or
 * host threads) race on it and must be ordered by the caller; consecutive
 * calls on one stream are safe.  A plan larger than the array gives
 * MOE_ERR_WORKSPACE.
 */
moe_status moe_expert_ffn_fwd_noalloc(const void *x_perm,
                                      const int32_t *offsets, int R, int E,
                                      int d, int f, moe_act act, moe_dtype dt,
                                      const void *W1, const void *W3,
                                      const void *W2, void *h_save,
                                      void *a_save, void *out_perm,
                                      hipStream_t stream);

/*
 * moe_expert_ffn_bwd -- gradients of moe_expert_ffn_fwd.
 *   dA = dO W2[e]^T;  GeLU: dH = dA * GeLU'(H)
 *                     SwiGLU: dH1 = dA*H3*SiLU'(H1), dH3 = dA*SiLU(H1)
 *   dW2[e] = A_e^T dO_e;  dW1[e] = X_e^T dH(1)_e;  dW3[e] = X_e^T dH3_e
 *   dx_perm = dH W1[e]^T (+ dH3 W3[e]^T)
 * An expert with no rows gets dW = 0.  The dW products sum over the ragged
 * segment length; each output tile is summed by one workgroup in order.
 * Sources: "Flattening Every Memory Peak in Long-Context MoE Training",
 * English abstract (reordering the work leaves loss and gradients exact, so
 * the gradients of the permuted, unpadded layout are those of the dense
 * layer); FastMoE review, 제안 방법 (the experts' linear layers over the
 * scatter/gather layout -- their backward is the same grouped products,
 * transposed).
 *   d_out_perm [R,d], x_perm [R,d], h_save, a_save as written by the forward,
 *   dx_perm [R,d], dW1 [E,d,f], dW3 [E,d,f] (SwiGLU only), dW2 [E,f,d], dt.
 *   offsets as for moe_expert_ffn_fwd (a subset of experts: offsets + e0,
 *   their count, their weights and weight gradients; dx_perm rows of other
 *   experts are left as they are).
 *   ws: at least moe_ffn_workspace_bytes(R,E,d,f,act,dt,1) (holds dH).
 */
moe_status moe_expert_ffn_bwd(const void *d_out_perm, const void *x_perm,
                              const void *h_save, const void *a_save,
                              const int32_t *offsets, int R, int E, int d,
                              int f, moe_act act, moe_dtype dt, const void *W1,
                              const void *W3, const void *W2, void *dx_perm,
                              void *dW1, void *dW3, void *dW2, void *ws,
                              size_t ws_bytes, hipStream_t stream);

/*
 * moe_expert_ffn_bwd_accumulate -- moe_expert_ffn_bwd with the weight
 * gradients added to what dW1, dW2 (dW3) hold: dW += X_e^T dH_e etc., the
 * old value and the new product summed in fp32 and rounded once.  For a
 * batch processed in chunks of tokens: the first chunk calls
 * moe_expert_ffn_bwd, the later ones this entry point.  In exact arithmetic
 * the chunked sum equals the whole one; in bf16 storage each chunk adds one
 * rounding of the running sum.  Sources: MPipeMoE (icslab.whu.edu.cn),
 * 研究方法 (buffers reused across micro-batches, recomputation); "Flattening
 * Every Memory Peak in Long-Context MoE Training", English abstract (a cap on
 * the tokens of each dispatch chunk; only order and granularity change).
 *   Arguments as moe_expert_ffn_bwd; R == 0 leaves dW unchanged.
 */
moe_status moe_expert_ffn_bwd_accumulate(const void *d_out_perm,
                                         const void *x_perm, const void *h_save,
                                         const void *a_save,
                                         const int32_t *offsets, int R, int E,
                                         int d, int f, moe_act act, moe_dtype dt,
                                         const void *W1, const void *W3,
                                         const void *W2, void *dx_perm,
                                         void *dW1, void *dW3, void *dW2,
                                         void *ws, size_t ws_bytes,
                                         hipStream_t stream);

/*
 * moe_expert_ffn_fwd_gather / moe_expert_ffn_bwd_gather -- the products of
 * moe_expert_ffn_fwd / moe_expert_ffn_bwd with the permute's row copy fused
 * into the operand loads: permuted row r is read as x[src[r],:] straight from
 * the token-order input, so no x_perm buffer is written or read.  GEMM1 and
 * dW1 (dW3) gather their rows while loading tiles; every result is bit-
 * identical to moe_permute's copy followed by the plain entry points.
 * Sources: ES-MoE review, 三 技术架构 / 专家级卸载与处理 (token permutation
 * overlapped with the expert work; no dispatch buffer); FastMoE review,
 * 제안 방법 (scatter/gather layout to reduce data movement).
 *   x [T,d] dt (16-byte aligned), src [R] int32 from moe_permute, every entry
 *   in [0,T) (a precondition: not checked on the device).  Other arguments
 *   as in the plain entry points; same workspace sizes.
 *   bf16 needs T*d*2 < 2^31 bytes (32-bit buffer offsets): MOE_ERR_UNSUPPORTED
 *   otherwise.
 */
moe_status moe_expert_ffn_fwd_gather(const void *x, const int32_t *src,
                                     const int32_t *offsets, int T, int R, int E,
                                     int d, int f, moe_act act, moe_dtype dt,
                                     const void *W1, const void *W3,
                                     const void *W2, void *h_save, void *a_save,
                                     void *out_perm, void *ws, size_t ws_bytes,
                                     hipStream_t stream);
moe_status moe_expert_ffn_bwd_gather(const void *d_out_perm, const void *x,
                                     const int32_t *src, const void *h_save,
                                     const void *a_save, const int32_t *offsets,
                                     int T, int R, int E, int d, int f,
                                     moe_act act, moe_dtype dt, const void *W1,
                                     const void *W3, const void *W2,
                                     void *dx_perm, void *dW1, void *dW3,
                                     void *dW2, void *ws, size_t ws_bytes,
                                     hipStream_t stream);

/*
 * moe_combine -- y[t,:] = sum_{j=0..k-1} topk_w[t,j] * out_perm[dest[t,j],:],
 * fp32 sum in slot order, rounded once to dt.  The gather back to token
 * order (FastMoE review, 제안 방법).
 *   out_perm [T*k,d] dt, dest [T,k] int32, topk_w [T,k] float, y [T,d] dt.
 */
moe_status moe_combine(const void *out_perm, const int32_t *dest,
                       const float *topk_w, int T, int k, int d, moe_dtype dt,
                       void *y, hipStream_t stream);

/*
 * moe_combine_bwd -- derivative of moe_combine:
 *   d_out_perm[dest[t,j],:] = topk_w[t,j] * dy[t,:]
 *   d_topk_w[t,j]           = sum_i dy[t,i] * out_perm[dest[t,j],i]  (fp32)
 * The derivative of the gather-combine of the scatter/gather layout (FastMoE
 * review, 제안 방법), written as a gather over dest so that no two lanes write
 * one row; exact under the reordering ("Flattening Every Memory Peak in
 * Long-Context MoE Training", English abstract: loss and gradients exact).
 *   dy [T,d] dt, out_perm [T*k,d] dt, dest [T,k], topk_w [T,k] float,
 *   d_out_perm [T*k,d] dt, d_topk_w [T,k] float.
 */
moe_status moe_combine_bwd(const void *dy, const void *out_perm,
                           const int32_t *dest, const float *topk_w, int T,
                           int k, int d, moe_dtype dt, void *d_out_perm,
                           float *d_topk_w, hipStream_t stream);

/*
 * moe_unpermute_grad -- backward of moe_permute's row copy, the sum back to
 * token order: dx[t,:] (+)= sum_j dx_perm[dest[t,j],:], gathered per token in
 * slot order (deterministic, no atomics).  Sources: FastMoE review, 제안 방법
 * (the scatter of token rows into the per-expert layout; its derivative
 * returns each row's gradient to the token that sent it); "Flattening Every
 * Memory Peak in Long-Context MoE Training", English abstract (reordering
 * leaves the gradients exact).
 *   dx_perm [T*k,d] dt, dest [T,k] int32, dx [T,d] dt;
 *   accumulate != 0 adds to dx instead of overwriting it.
 */
moe_status moe_unpermute_grad(const void *dx_perm, const int32_t *dest, int T,
                              int k, int d, moe_dtype dt, void *dx,
                              int accumulate, hipStream_t stream);

/*
 * moe_gate_topk_bwd -- backward of moe_gate_topk through the gate weights
 * (the selection itself is piecewise constant).  Sources: ES-MoE review,
 * 三 技术架构 (the gating network's output decides each token's experts;
 * the gate is trained with the layer); "Flattening Every Memory Peak in
 * Long-Context MoE Training", English abstract (gradients stay exact under
 * the reordering, so the gate's gradient is the dense layer's).  The gate
 * formula is not printed: the derivative of softmax top-k is the reading.
 *   renorm=1: dl[t,idx_j] = w_j (dw_j - sum_j' w_j' dw_j'), 0 elsewhere
 *   renorm=0: dl[t,e] = p_e (g_e - sum_j w_j dw_j), p = softmax(logits[t,:]),
 *             g_e = dw_j where e = idx_j else 0
 *   dWg = x^T dl (overwritten; the sum over tokens runs in fixed chunks
 *         reduced in order); dx = dl Wg^T, or dx += dl Wg^T when
 *         accumulate != 0 (then dx must hold values, e.g. the output of
 *         moe_unpermute_grad).
 *   x [T,d] dt, Wg [d,E] dt, logits [T,E], topk_idx [T,k], topk_w [T,k],
 *   d_topk_w [T,k] float, dx [T,d] dt, dWg [d,E] dt.
 *   ws: at least moe_gate_bwd_workspace_bytes(T,d,E).
 */
size_t moe_gate_bwd_workspace_bytes(int T, int d, int E);
moe_status moe_gate_topk_bwd(const void *x, const void *Wg, const float *logits,
                             const int32_t *topk_idx, const float *topk_w,
                             const float *d_topk_w, int T, int d, int E, int k,
                             int renorm, moe_dtype dt, void *dx,
                             int accumulate, void *dWg, void *ws,
                             size_t ws_bytes, hipStream_t stream);

/*
 * Kernel timing (benchmark support, off by default).
 * moe_profile_enable(capacity) creates 2*capacity HIP events; from then on
 * every kernel the library launches is bracketed by two of them on its
 * stream, until `capacity` launches have been recorded (later launches run
 * untimed).  moe_profile_get(i, ...) waits for record i and returns the
 * kernel's name (static storage) and its duration in milliseconds.
 * moe_profile_reset() forgets the records and keeps the events;
 * moe_profile_disable() destroys the events.  Not thread-safe: enable,
 * launch and read from one host thread.
 */
moe_status moe_profile_enable(int capacity);
void moe_profile_disable(void);
void moe_profile_reset(void);
int moe_profile_count(void);
moe_status moe_profile_get(int i, const char **name, float *ms);

/*
 * moe_mfma_loop -- benchmark support: the attainable rate of the bf16 matrix
 * instructions.  `blocks` workgroups of 4 waves each run `iters` rounds of
 * four independent v_mfma_f32_32x32x16_bf16 on register operands (no memory
 * traffic): 4 * 4 * iters * 2*32*32*16 FLOP per workgroup.  Timed by the
 * caller on `stream`, it gives the matrix cores' rate at the clock they run
 * at under load, against which the grouped GEMMs are also rated.
 *   out: device buffer of at least blocks * 4 floats (one value per wave,
 *   meaningless; written so that the work is not optimised away).
 */
moe_status moe_mfma_loop(int blocks, int iters, float *out, size_t out_floats,
                         hipStream_t stream);

/*
 * moe_mfma_loop_random -- benchmark support: moe_mfma_loop on operands that
 * change with every instruction.  Each wave cycles through eight A and eight
 * B fragments of random bf16 values (|v| < 1, random mantissas), so the
 * matrix cores see operand bits toggle as in a GEMM on random data.  The
 * sustained rate of the matrix instructions depends on the data (power and
 * clock), and this is the ceiling that applies to GEMMs on such inputs.
 *   iters: a positive multiple of 8 (rounds of four instructions per wave).
 *   out: as for moe_mfma_loop.
 *   Errors: MOE_ERR_INVALID_ARG for blocks < 1, iters not a positive
 *   multiple of 8, out NULL or out_floats < blocks * 4.
 */
moe_status moe_mfma_loop_random(int blocks, int iters, float *out, size_t out_floats,
                                hipStream_t stream);

/*
 * moe_lds_probe -- benchmark support: the rates of the LDS paths the grouped
 * GEMM's main loop uses, alone and side by side.  `blocks` workgroups of 4
 * waves each run `iters` rounds; per round each wave does, for every set bit
 * of `mode`:
 *   1: eight 16-byte-per-lane LDS reads (ds_read_b128, 1 KB per wave each),
 *   2: sixteen 8-byte-per-lane transposing LDS reads (ds_read_b64_tr_b16,
 *      512 B per wave each), the read of M/N-contiguous operand fragments,
 *   4: eight direct-to-LDS buffer loads of 16 bytes per lane
 *      (buffer_load_dwordx4 ... lds, 1 KB per wave each) from `src`, cycling
 *      through its src_bytes bytes (size it under the L2 to time L2-to-LDS
 *      loads), then a wait for them,
 *   8: the reads of bits 1 and 2 three times (the ratio of fragment reads to
 *      ring loads of the GEMM's 256 x 256 tile),
 * so each kind moves 32 KB per workgroup and round (reads 96 KB with bit 8).  Each workgroup holds
 * 64 KB of LDS (two per compute unit).  Timed by the caller on `stream`.
 *   src: device buffer, 16-byte aligned, read only when bit 4 is set (may be
 *   NULL otherwise); src_bytes a power of two from 8 KB to 1 GB.
 *   out: device buffer of at least blocks * 4 floats (one value per wave,
 *   meaningless; written so that the work is not optimised away).
 *   Errors: MOE_ERR_INVALID_ARG for mode outside 1..15 or with none of
 *   bits 1, 2, 4 set, blocks < 1,
 *   iters < 1, out NULL or out_floats < blocks * 4, or, with bit 4 set, src
 *   NULL or unaligned or src_bytes not a power of two in [8 KB, 1 GB].
 */
moe_status moe_lds_probe(int mode, int blocks, int iters, const void *src, size_t src_bytes,
                         float *out, size_t out_floats, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
