/*
 * moe_ep.h -- C ABI of the MI355X (gfx950) MoE expert-parallel hot path,
 * one GPU's share:
 *
 *   moe_dispatch_layout -> moe_permute -> moe_grouped_gemm_w13
 *     -> (moe_silu_mul) -> moe_grouped_gemm_w2 -> moe_combine
 *
 * and its backward (the end of this file).
 *
 * Pages cited (by title):
 *   [EP]  "SGLang、NCCL 与 MoE EP：从职责边界到执行机制"
 *   [ECB] "SGLang Expert Compute Backend：从接收布局到 Triton 专家计算"
 *   [DEP] "DeepEP 架构与实现笔记"
 *   [XT]  "XTuner Domino EP"
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is DEVICE memory owned by the caller; the
 *     library never allocates, frees or keeps a pointer after returning.
 *   - Every call enqueues work on `stream` and returns without waiting for
 *     the GPU.  Launch shapes depend only on the size arguments, never on
 *     device-side counts, so the calls can be captured in a hipGraph and
 *     replayed with new routing (the device re-derives all counts).
 *   - Tensors are dense row-major, shapes as written below.  bf16 and
 *     OCP e4m3fn ("float8_e4m3fn", largest finite 448) are stored as raw
 *     16-/8-bit patterns.
 *   - Argument errors are detected on the host and returned before anything
 *     is enqueued (MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED).  A launch
 *     failure reported by the HIP runtime returns MOE_ERR_HIP.  Errors that
 *     depend on data (capacity overflow, bad expert id) are written to
 *     device memory by moe_dispatch_layout (see dev_status).
 *   - Expert-major buffers: local expert e owns rows
 *     [offsets[e], offsets[e] + counts[e]) -- a contiguous valid prefix of its
 *     block ([EP] §2.3.4).  Rows outside these ranges ("padding") are never
 *     read for a result and never written by any entry point.
 *   - rows_cap is the number of rows of every expert-major buffer:
 *     L*R with capacity R, or T*K with exact-fit offsets.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,   /* null pointer, negative size, bad enum    */
  MOE_ERR_UNSUPPORTED = -2,   /* valid but unsupported dtype/shape combo  */
  MOE_ERR_WORKSPACE = -3,     /* workspace smaller than required          */
  MOE_ERR_HIP = -5            /* the HIP runtime rejected a launch        */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8_E4M3 = 2            /* OCP e4m3fn codes with fp32 group scales  */
} moe_dtype;

/* Epilogue of the gate/up GEMM. */
typedef enum moe_w13_epilogue {
  MOE_EPI_STORE_G = 0,        /* out = G [rows_cap, 2I] fp32               */
  MOE_EPI_SILU_MUL = 1        /* out = Z = SiLU(G[:, :I]) * G[:, I:]       */
} moe_w13_epilogue;

/* Layout of the gate/up weights given to moe_grouped_gemm_w13. */
typedef enum moe_weight_layout {
  MOE_W_ROW_MAJOR = 0,        /* [L, 2I, H]: [expert, out, in]                     */
  MOE_W_PACKED = 1            /* as written by moe_pack_w13                        */
} moe_weight_layout;

/* Bits of dev_status[0] written by moe_dispatch_layout. */
#define MOE_FLAG_CAPACITY 1      /* a local expert received more than R routes */
#define MOE_FLAG_BAD_EXPERT_ID 2 /* an id was < -1 or >= E_global              */

/* Human-readable name of a moe_status value (static string). */
const char* moe_status_string(int status);

/* ABI version; bumped on any signature change or added entry point (2: moe_router_topk;
 * 3: GEMM workspace for the K-split last round; 4: moe_pack_w13 and the W13 layout;
 * 5: the backward entry points; 6: moe_grouped_gemm_wgrad; 7: moe_dispatch_layout_noalloc; 8: moe_grouped_gemm_w2_combine;
 * 9: moe_grouped_gemm_w13_silu_backward). */
int moe_abi_version(void);

/* Bytes of device workspace moe_dispatch_layout needs for (T, K, L). */
size_t moe_dispatch_layout_workspace_bytes(int T, int K, int L);

/*
 * moe_dispatch_layout -- counts, offsets, slots and the reverse map.
 *
 * Defined by [EP] §2.3.4 (per-expert row allocator: a route to local
 * expert e gets s = counter[e]++ and row q = offsets[e] + s, each expert's
 * rows a contiguous prefix), [EP] §2.3.6 (reverse map (t,k) -> q, -1 for
 * top-k entries not owned here) and [DEP] §9.4 (dispatch_convert: tokens,
 * then top-k positions, in order).  Rows of one expert are ordered by the
 * flattened route index i = t*K + k, so the result is unique and
 * deterministic (the pages' atomic order is one of many valid orders).
 *
 *   topk_ids   [T,K] int32  global expert ids; -1 = no route
 *   E_global   number of global experts; ids must lie in [-1, E_global)
 *   expert_begin, L   this GPU owns global experts [expert_begin, expert_begin+L)
 *   R          capacity rows per local expert (> 0), or 0 for exact-fit
 *              offsets (offsets = exclusive prefix sum of counts, [ECB] §4.1)
 *   BM         tile rows used for tile_offsets (> 0)
 * Outputs (all fully rewritten on every call; stale contents never count):
 *   counts       [L]    min(routes to e, R)            (exact-fit: routes to e)
 *   offsets      [L+1]  e*R, or prefix sums of counts; offsets[L] = rows used
 *   slot_of      [T,K]  row q of route (t,k), or -1 (no route, not local,
 *                       bad id, or beyond capacity)
 *   row_src      [rows_cap] t*K + k for valid rows, -1 for padding rows
 *   tile_offsets [L+1]  prefix sums of ceil(counts[e] / BM)
 *   dev_status   [2]    [0] = MOE_FLAG_* bits, [1] = routes dropped because
 *                       of capacity.  Routes beyond capacity are never written.
 *   workspace    >= moe_dispatch_layout_workspace_bytes(T, K, L) bytes
 * Limits: 1 <= L <= 1024, T*K <= 2^30.
 */
moe_status moe_dispatch_layout(const int32_t* topk_ids, int T, int K, int E_global,
                               int expert_begin, int L, int R, int BM,
                               int32_t* counts, int32_t* offsets, int32_t* slot_of,
                               int32_t* row_src, int32_t* tile_offsets, int32_t* dev_status,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_dispatch_layout_noalloc -- moe_dispatch_layout without a caller
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results and errors as moe_dispatch_layout; the count pass's
 * per-block histograms go to a scratch array of the library instead, one per
 * device, held until the process ends.  The call allocates nothing.
 *   Limit: moe_dispatch_layout_workspace_bytes(T, K, L) must not exceed
 *   moe_dispatch_layout_noalloc_max_bytes() (4 MiB: up to about 32 million
 *   routes T*K at L = 32, 4 million at L = 256); larger sizes return
 *   MOE_ERR_WORKSPACE before anything is enqueued.  MOE_ERR_HIP if the runtime cannot resolve the scratch address.
 *   Every call on a device shares that device's scratch: calls that overlap
 *   in time on one device (other streams, other host threads) race and must
 *   be ordered by the caller.  Each call rewrites every scratch entry it
 *   reads, so nothing of an earlier call carries over.
 */
moe_status moe_dispatch_layout_noalloc(const int32_t* topk_ids, int T, int K, int E_global,
                                       int expert_begin, int L, int R, int BM,
                                       int32_t* counts, int32_t* offsets, int32_t* slot_of,
                                       int32_t* row_src, int32_t* tile_offsets, int32_t* dev_status,
                                       hipStream_t stream);

/* Largest workspace (bytes) moe_dispatch_layout_noalloc can stand in for. */
size_t moe_dispatch_layout_noalloc_max_bytes(void);

/*
 * moe_permute -- fill the expert-major buffer from token rows.
 *
 * buf[slot_of[t,k], :] = x[t, :] for every (t,k) with slot_of >= 0
 * ([EP] §2.3.4 recv_tokens[e, s, :] = payload; [DEP] §9.4 recv_x_all[m] =
 * recv_x[token]).  With buf_dt == MOE_FP8_E4M3 each written row is quantised
 * per group of 128 columns ([EP] §2.3.5 FP8 [L,M,H] + fp32 [L,M,H/128];
 * recipe of [DEP] §11): amax = max|x| over the group clamped below at 1e-4,
 * code = e4m3fn(x * (448/amax)) rounded to nearest even, scale = amax/448,
 * every step a single fp32 operation.  Each token row is read once.
 *
 *   x          [T,H]  x_dt in {MOE_F32, MOE_BF16}
 *   slot_of    [T,K]  from moe_dispatch_layout (values >= rows_cap are skipped)
 *   buf        [rows_cap,H]  buf_dt: same as x_dt, or MOE_FP8_E4M3
 *   buf_scales [rows_cap,H/128] fp32 when buf_dt == MOE_FP8_E4M3, else unused
 * Limits: H % 128 == 0, K <= 64.  Padding rows of buf are left untouched.
 */
moe_status moe_permute(const void* x, moe_dtype x_dt, int T, int K, int H,
                       const int32_t* slot_of, int64_t rows_cap,
                       void* buf, moe_dtype buf_dt, float* buf_scales, hipStream_t stream);

/*
 * moe_pack_w13 -- the gate/up weights in the GEMM's staging order.
 *
 * Same bytes as w13 [L, 2I, H] (w_dt), rearranged so that each (128-column
 * block nb of Z, 128-byte K stage ks) of an expert is one contiguous 32 KB
 * run: [L][I/128][H*esz/128][256 rows][128 bytes], rows 0..127 the gate
 * rows nb*128 + r, rows 128..255 the up rows I + nb*128 + r.  Values are
 * copied, never converted; the FP8 block scales keep their layout.  The
 * gate/up GEMM stages that layout with 1 KB contiguous loads instead of
 * eight 128-byte row pieces.  Weights are static, so the caller packs once
 * and keeps the packed copy (same size as w13, caller-owned,
 * non-overlapping).  Limits: H % 128 == 0, I % 128 == 0.
 */
moe_status moe_pack_w13(const void* w13, moe_dtype w_dt, int L, int H, int I, void* w13_packed,
                        hipStream_t stream);

/*
 * moe_grouped_gemm_w13 -- gate/up projection of every local expert.
 *
 * For each expert e and valid row q of e: G[q, n] = sum_k A[q,k] W13[e,n,k]
 * ([ECB] §1.1: X_e [m_e,H] -> [m_e,2I]; §2.3: one grouped launch over all
 * experts' valid rows; weights stored [expert, out, in], §3.5).  With FP8
 * operands the block-wise scales apply per 128-wide K group ([ECB] §3.5):
 * G[q,n] = sum_g a_scales[q,g] * w13_scales[e, n/128, g] * sum_{k in g} a8*w8,
 * accumulated in fp32.  Only tiles that contain valid rows are computed (an
 * in-kernel scheduler walks ceil(counts[e]/BM) row tiles per expert, [ECB]
 * §2.5/§2.6); rows beyond counts[e] are never stored.
 *
 *   a          [rows_cap,H]  a_dt;  a_scales [rows_cap,H/128] fp32 for FP8
 *   w13        [L,2I,H]      w_dt == a_dt; rows [0,I) are gate, [I,2I) up
 *              (w13_layout MOE_W_ROW_MAJOR), or as packed by moe_pack_w13
 *              (MOE_W_PACKED)
 *   w13_scales [L,2I/128,H/128] fp32 for FP8, else unused
 *   counts, offsets  [L], [L+1] as produced by moe_dispatch_layout
 *   epi == MOE_EPI_STORE_G:  out = G [rows_cap,2I], out_dt = MOE_F32
 *   epi == MOE_EPI_SILU_MUL: out = Z [rows_cap,I] = SiLU(gate) * up computed
 *        from the fp32 accumulators ([ECB] §3.6 non-interleaved gate/up;
 *        §4.4 fusion of SiLU*up with the group quantisation); out_dt in
 *        {MOE_F32, MOE_BF16, MOE_FP8_E4M3}; for FP8, out_scales
 *        [rows_cap, I/128] fp32 get the same per-128 recipe as moe_permute.
 *   workspace  NULL, or >= moe_grouped_gemm_workspace_bytes() bytes of device
 *        memory, 16-byte aligned, owned by the caller and not shared with a
 *        concurrent GEMM call.  With a workspace, tiles of an incomplete last
 *        round of the persistent schedule are split along K. Their fp32
 *        partial sums meet in the workspace, and a second kernel on the same
 *        stream adds them in a fixed order. Without one, no tile is split.
 *        Results differ only in fp32 summation order.  A workspace that is
 *        given but too small returns MOE_ERR_WORKSPACE.
 * dtype pairs (a_dt = w_dt): F32, BF16, FP8_E4M3.  Limits: H % 128 == 0,
 * I % 128 == 0, L <= 1024.
 */
moe_status moe_grouped_gemm_w13(const void* a, moe_dtype a_dt, const float* a_scales,
                                const void* w13, moe_dtype w_dt, const float* w13_scales,
                                moe_weight_layout w13_layout,
                                const int32_t* counts, const int32_t* offsets, int L,
                                int64_t rows_cap, int H, int I, moe_w13_epilogue epi,
                                void* out, moe_dtype out_dt, float* out_scales,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Device workspace bytes that moe_grouped_gemm_w13 and moe_grouped_gemm_w2
 * use at most on the current device (one fp32 128 x 256 partial tile and a
 * 64-byte descriptor per compute unit).  Host-only; no device work. */
size_t moe_grouped_gemm_workspace_bytes(void);

/*
 * moe_silu_mul -- Z = SiLU(G[:, :I]) * G[:, I:] on valid rows only
 * ([ECB] §3.6: activation filtered to valid expert rows; Z re-quantised for
 * the down GEMM with its own scales).  SiLU(v) = v / (1 + exp(-v)) in fp32.
 *   g [rows_cap,2I] fp32;  z [rows_cap,I] z_dt in {F32, BF16, FP8_E4M3};
 *   z_scales [rows_cap,I/128] fp32 for FP8 (recipe of moe_permute).
 * Limits: I % 128 == 0.
 */
moe_status moe_silu_mul(const float* g, const int32_t* counts, const int32_t* offsets, int L,
                        int64_t rows_cap, int I, void* z, moe_dtype z_dt, float* z_scales,
                        hipStream_t stream);

/*
 * moe_grouped_gemm_w2 -- down projection of every local expert.
 *
 * out[q, n] = sum_k Z[q,k] W2[e,n,k] for valid rows q of expert e
 * ([ECB] §1.1: [m_e,I] -> [m_e,H]; §3.6: same grouping as the gate/up GEMM,
 * K = I), block-FP8 scaled as in moe_grouped_gemm_w13, fp32 accumulation,
 * stored as out_dt; results stay at row q ([ECB] §3.7).  The router weight
 * is NOT applied here ([EP] §1.1).
 *   z [rows_cap,I] z_dt;  z_scales [rows_cap,I/128] fp32 for FP8
 *   w2 [L,H,I] w_dt == z_dt;  w2_scales [L,H/128,I/128] fp32 for FP8
 *   out [rows_cap,H] out_dt in {MOE_F32, MOE_BF16}
 *   workspace, workspace_bytes  as for moe_grouped_gemm_w13
 * Limits: H % 128 == 0, I % 128 == 0, L <= 1024.
 */
moe_status moe_grouped_gemm_w2(const void* z, moe_dtype z_dt, const float* z_scales,
                               const void* w2, moe_dtype w_dt, const float* w2_scales,
                               const int32_t* counts, const int32_t* offsets, int L,
                               int64_t rows_cap, int H, int I,
                               void* out, moe_dtype out_dt,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_gemm_w2_combine -- the down GEMM with the combine folded into
 * its epilogue: y[t] = sum over the rows q of token t of topk_weights[t,k] *
 * (Z[q] W2[e]^T), with (t,k) = row_src[q] decoded as t*K + k.  The pages
 * describe the in-kernel weighted reduce on the combine path ("DeepEP
 * 架构与实现笔记" §9.6) and fusing the necessary conversions into the expert
 * computation ("SGLang Expert Compute Backend" §2.4, §4.4).  Three kernels on
 * `stream`: y_acc = 0; the down GEMM, whose epilogue adds w * out[q, n] into
 * y_acc[t, n] with fp32 atomic adds (the row outputs are not rounded to the
 * output format and the sum's order is the arrival order, so results are
 * not bit-reproducible; they stay within the layer's tolerance); y = y_acc
 * rounded to y_dt.  Tokens without a local route get 0.
 *   z, z_scales, w2, w2_scales, counts, offsets: as for moe_grouped_gemm_w2
 *   row_src [rows_cap] from moe_dispatch_layout; topk_weights [T,K] fp32
 *   y_acc [T,H] fp32 scratch (caller-owned, 16-byte aligned);
 *   y [T,H] y_dt in {MOE_F32, MOE_BF16} (16-byte aligned)
 * At the prefill shape (8117 rows, H = 7168) the fp32 atomic adds make it
 * about 3.5x slower than moe_grouped_gemm_w2 followed by moe_combine; at
 * decode (128 tokens, about 130 rows) the two are level.  Kept as a tested
 * alternative.
 * Every argument is checked before the first launch.
 * Limits as moe_grouped_gemm_w2.
 */
moe_status moe_grouped_gemm_w2_combine(const void* z, moe_dtype z_dt, const float* z_scales,
                                       const void* w2, moe_dtype w_dt, const float* w2_scales,
                                       const int32_t* counts, const int32_t* offsets, int L,
                                       int64_t rows_cap, int H, int I, const int32_t* row_src,
                                       const float* topk_weights, int T, int K, float* y_acc,
                                       void* y, moe_dtype y_dt, hipStream_t stream);

/*
 * moe_combine -- weighted gather-sum back to token order.
 *
 * y[t, :] = sum over k with slot_of[t,k] >= 0 of topk_weights[t,k] *
 * expert_out[slot_of[t,k], :], accumulated in fp32 in k order, stored as
 * y_dt; 0 for a token with no local route ([EP] §1.1: weights multiply
 * expert outputs; §2.3.6: follow the (t,k) -> q map back; [DEP] §9.4
 * combine_convert).
 *   expert_out [rows_cap,H] eo_dt in {F32, BF16};  slot_of [T,K];
 *   topk_weights [T,K] fp32;  y [T,H] y_dt in {F32, BF16}
 * Limits: H % 8 == 0, K <= 64.
 */
moe_status moe_combine(const void* expert_out, moe_dtype eo_dt, const int32_t* slot_of,
                       const float* topk_weights, int T, int K, int H, int64_t rows_cap,
                       void* y, moe_dtype y_dt, hipStream_t stream);

/*
 * moe_router_topk -- router logits -> the TopKOutput the path starts from.
 *
 * The router scores every expert and a selection policy returns K expert
 * ids and K weights per token ([EP] §1.1; §3.6 TopKOutput topk_ids [T,K],
 * topk_weights [T,K]).  The pages leave the arithmetic to the model; this
 * entry point implements the renormalised-softmax top-K:
 *   score[t,e]  = logits[t,e] + bias[e]  (one fp32 add; bias may be NULL)
 *   topk_ids[t,k]  = expert with the k-th largest score, k = 0 largest;
 *                    equal scores go to the lower expert id; a NaN score
 *                    ranks below every number
 *   topk_weights[t,k] = exp(v_k - max v) / sum_j exp(v_j - max v) over the
 *                    K selected experts (fp32), v = score, or the unbiased
 *                    logit when bias_in_weights == 0 (bias steers the
 *                    selection only); NaN if a selected value is NaN
 *   logits [T,E] fp32 row-major (device); bias [E] fp32 (device) or NULL;
 *   topk_ids [T,K] int32 and topk_weights [T,K] fp32 (device, written).
 * Limits: 1 <= K <= E, E <= 1024, K <= 64.  Returns MOE_ERR_INVALID_ARG
 * for K > E or missing pointers, MOE_ERR_UNSUPPORTED beyond the limits.
 */
moe_status moe_router_topk(const float* logits, const float* bias, int T, int E, int K,
                           int bias_in_weights, int32_t* topk_ids, float* topk_weights,
                           hipStream_t stream);

/* ---------------------------------------------------------------- backward
 *
 * The gradients of the path, consumed in the reverse order of the forward
 * ([XT] "XTuner Domino EP": the DeepEP part's complete run path consumes the
 * saved routing -- here slot_of, counts, offsets -- in reverse; the UltraEP
 * part's backward runs combine backward, the grouped GEMMs' gradients and the
 * inverse permutation).  Formulas: the derivatives of the forward ([EP] §1.1,
 * [ECB] §1.1, §3.6).  bf16 and fp32 data only.  Per GPU share, a route without
 * a local row contributes nothing: its d_w is 0 and it writes no row.
 *
 *   d_out = combine_backward(dy)            moe_combine_backward (also d_w)
 *   dZ    = d_out W2[e]                     moe_grouped_gemm_w2 on W2^T [L,I,H]
 *   G     = A W13[e]^T  (recomputed)        moe_grouped_gemm_w13, MOE_EPI_STORE_G
 *   dG    = silu_mul_backward(G, dZ)        moe_silu_mul_backward
 *   dA    = dG W13[e]                       moe_grouped_gemm_w2 on W13^T [L,H,2I]
 *   dx    = permute_backward(dA)            moe_permute_backward
 *   dW2   = d_out^T Z   per expert          moe_grouped_gemm_wgrad
 *   dW13  = dG^T A      per expert          moe_grouped_gemm_wgrad
 *
 * moe_grouped_gemm_w2 computes rows * W^T for any [L, N, K] weights (N = its
 * H argument, K = its I argument), so with the transposes written once by
 * moe_transpose_weights it is the data gradient of both GEMMs.
 */

/*
 * moe_combine_backward -- the gradient of moe_combine.
 *   d_out[q]   = topk_weights[t,k] * dy[t]   (one fp32 product, rounded to
 *                d_out_dt) for every local route q = slot_of[t,k]
 *   d_weights[t,k] = sum_h dy[t,h] * expert_out[q,h] (fp32 accumulation),
 *                0 for a route without a local row
 *   dy [T,H] (dy_dt), expert_out [rows_cap,H] (eo_dt, the forward's output),
 *   d_out [rows_cap,H] (padding rows untouched), d_weights [T,K] fp32.
 * dtypes: F32 or BF16.  Limits: H % 8 == 0, K <= 64.
 */
moe_status moe_combine_backward(const void* dy, moe_dtype dy_dt, const void* expert_out,
                                moe_dtype eo_dt, const int32_t* slot_of, const float* topk_weights,
                                int T, int K, int H, int64_t rows_cap, void* d_out,
                                moe_dtype d_out_dt, float* d_weights, hipStream_t stream);

/*
 * moe_silu_mul_backward -- the gradient of Z = SiLU(gate) * up on valid rows:
 *   d_gate = dZ * up * s * (1 + gate * (1 - s)),  d_up = dZ * SiLU(gate),
 *   s = sigmoid(gate), fp32 (hardware exp2 / reciprocal), rounded to dg_dt.
 *   g [rows_cap,2I] fp32 (the forward's G); dz [rows_cap,I] (dz_dt);
 *   dg [rows_cap,2I] (dg_dt: d_gate in columns [0,I), d_up in [I,2I)).
 * dtypes: F32 or BF16.  Limits: I % 4 == 0.
 */
moe_status moe_silu_mul_backward(const float* g, const void* dz, moe_dtype dz_dt,
                                 const int32_t* counts, const int32_t* offsets, int L,
                                 int64_t rows_cap, int I, void* dg, moe_dtype dg_dt,
                                 hipStream_t stream);

/*
 * moe_grouped_gemm_w13_silu_backward -- the gate/up GEMM recomputed for the
 * backward with the SiLU*up gradient in its epilogue: for each valid row q of
 * expert e, G[q] = A[q] W13[e]^T as in moe_grouped_gemm_w13 (fp32 sums, never
 * stored), then dG[q] from G[q] and dZ[q] exactly as moe_silu_mul_backward
 * computes it (same fp32 operations, so the same bits as G stored by
 * MOE_EPI_STORE_G followed by moe_silu_mul_backward).  The XTuner Domino EP
 * page's backward consumes the forward's saved routing in reverse order; the
 * gradient is the derivative of the pages' expert MLP ([ECB] §1.1, §3.6).
 * Saves writing fp32 G and reading it back when the forward did not keep G.
 *   a [rows_cap,H], w13 [L,2I,H] (or packed, w13_layout), a_dt = w_dt in
 *   {F32, BF16};  dz [rows_cap,I] (dz_dt F32 or BF16);  dg [rows_cap,2I]
 *   (dg_dt F32 or BF16: d_gate in columns [0,I), d_up in [I,2I)).
 *   counts, offsets, workspace as for moe_grouped_gemm_w13.
 * Limits: H % 128 == 0, I % 128 == 0, L <= 1024.  Padding rows of dg are left
 * untouched.
 */
moe_status moe_grouped_gemm_w13_silu_backward(const void* a, moe_dtype a_dt, const void* w13, moe_dtype w_dt,
                                              moe_weight_layout w13_layout, const int32_t* counts,
                                              const int32_t* offsets, int L, int64_t rows_cap, int H, int I,
                                              const void* dz, moe_dtype dz_dt, void* dg, moe_dtype dg_dt,
                                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_permute_backward -- the gradient of moe_permute (an unweighted combine):
 *   dx[t] = sum over local routes k, in increasing k, of d_buf[slot_of[t,k]]
 *   (fp32, rounded to dx_dt); 0 for a token without a local route.
 *   d_buf [rows_cap,H] (d_buf_dt), dx [T,H] (dx_dt).  dtypes: F32 or BF16.
 * Limits: H % 8 == 0, K <= 64.
 */
moe_status moe_permute_backward(const void* d_buf, moe_dtype d_buf_dt, const int32_t* slot_of,
                                int T, int K, int H, int64_t rows_cap, void* dx, moe_dtype dx_dt,
                                hipStream_t stream);

/*
 * moe_transpose_weights -- wt[e] = w[e]^T: w [L,N,K] -> wt [L,K,N] (same
 * dtype, F32 or BF16), caller-owned, non-overlapping; once per weight update.
 */
moe_status moe_transpose_weights(const void* w, moe_dtype w_dt, int L, int N, int K, void* wt,
                                 hipStream_t stream);

/*
 * moe_grouped_gemm_wgrad -- weight gradient of a grouped GEMM: for every local
 * expert e, C[e] = sum over its valid rows q of b[q]^T a[q] (an outer-product
 * sum, fp32 accumulation), i.e. dW2[e] = d_out^T Z (b = d_out, a = Z) and
 * dW13[e] = dG^T A (b = dG, a = the permuted buffer).  Rows are expert e's
 * [offsets[e], offsets[e] + counts[e]) (clamped to rows_cap); padding rows
 * are never read.  An expert without rows gets C[e] = 0.
 *   b [rows_cap,N], a [rows_cap,K] (dt, row-major, 16-byte aligned),
 *   c [L,N,K] fp32 (16-byte aligned), caller-owned, every element written.
 * dtypes: F32 or BF16 (FP8 buffers: MOE_ERR_UNSUPPORTED).
 * Limits: N % 128 == 0, K % 128 == 0, L <= 65535.
 */
moe_status moe_grouped_gemm_wgrad(const void* b, const void* a, moe_dtype dt, const int32_t* counts,
                                  const int32_t* offsets, int L, int64_t rows_cap, int N, int K,
                                  float* c, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_EP_H */
