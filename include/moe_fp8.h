/*
 * moe_fp8.h - C ABI of libmoe_fp8.so, the DeepSeekMoE layer forward on
 * MI355X (gfx950).
 *
 * The layer follows the DeepSeek-V3 pages:
 *   - sigmoid gating with a per-expert bias used only to choose experts
 *     (aliyun study note developer.aliyun.com/article/1776647, section 2.2;
 *     news.qq.com/rain/a/20241229A05OQF00, section 无额外损耗的负载均衡);
 *   - 1 shared + 256 routed experts, 8 routed per token, at most 4 nodes per
 *     token (news.qq.com article, sections DeepSeekMoE 架构 and 节点限制路由);
 *   - FP8 GEMMs with 1x128 activation tiles, 128x128 weight blocks and
 *     high-precision accumulation (news.qq.com article, section FP8 低精度训练,
 *     items 细粒度量化 and 提高累加精度).
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or keeps a pointer after the call.
 *   - Layouts are row-major and dense unless a leading dimension is given.
 *     "bf16" buffers hold raw bfloat16 bit patterns (uint16).  "e4m3" buffers
 *     hold OCP E4M3FN bytes.  Scales are fp32.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; the caller keeps every buffer
 *     alive until the stream has finished.  No call synchronises the host.
 *   - Arguments are validated on the host before anything is launched.  On
 *     error nothing is launched, the return value is negative and
 *     moe_last_error() describes it.  Faults inside kernels surface at the
 *     caller's next synchronisation, as for any HIP kernel.
 *   - Outputs are fully overwritten, never accumulated into.  Inputs and
 *     outputs must not alias (except where a call says "in place").
 *   - A zero-sized problem (T == 0, M_total == 0) is a successful no-op that
 *     still writes the outputs that do not depend on it (counts, offsets).
 *   - NaN or Inf inputs give unspecified results.
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MOE_OK               0
#define MOE_ERR_INVALID     -1  /* null pointer, bad shape or parameter      */
#define MOE_ERR_UNSUPPORTED -2  /* valid but outside what the kernels handle */
#define MOE_ERR_HIP         -3  /* a HIP launch or API call failed            */
#define MOE_ERR_WORKSPACE   -4  /* workspace too small                        */

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

/*
 * moe_route - router: sigmoid scores, selection bias, group-limited top-k.
 *
 * Follows the aliyun study note, section 2.2 (sigmoid gate per expert, a bias
 * per expert that shifts only the choice), and the news.qq.com article,
 * sections DeepSeekMoE 架构 (top-8 of 256) and 节点限制路由 (at most 4 nodes;
 * here: groups).  Gating stays in high precision (same article,
 * 选择性高精度): logits are computed with fp32 accumulation of exact
 * products (bf16 x times a three-piece bf16 split of the fp32 centroids).
 *
 * For each token t:
 *   l[e]  = sum_h x[t,h] * centroids[e,h]
 *   s[e]  = 1 / (1 + exp(-l[e]))               (fp32)
 *   s'[e] = s[e] + bias[e]                     (fp32, used to choose only)
 *   experts form n_group contiguous groups of E/n_group; a group's score is
 *   the sum of its two largest s'; the topk_group best groups are kept; the
 *   k largest s' among the kept experts are chosen; ties go to the lower
 *   index; ids are written in ascending order;
 *   w[j]  = s[e_j] / sum_j' s[e_j']            (unbiased scores, fp32)
 *   expert_counts[e] = number of tokens that chose e (overwritten).
 *
 * x_bf16          [T, H] bf16
 * centroids       [E, H] fp32
 * bias            [E] fp32
 * topk_idx  (out) [T, k] int32, ascending per row
 * topk_w    (out) [T, k] fp32, each row sums to 1
 * expert_counts (out) [E] int32
 * workspace       device scratch of at least moe_route_workspace_bytes(T, H, E)
 *                 bytes (partial logits); contents on entry are ignored.
 * topk_s    (out, optional: NULL skips it) [T, k] fp32, 4-byte aligned: the
 *                 unbiased scores s[e_j] of the chosen experts (w[j] times
 *                 their sum), which moe_router_backward can take instead of
 *                 computing the logits again.
 * Requirements: H % 128 == 0; 2 <= E <= 256; E % n_group == 0; the group
 * size E/n_group is 4 times a power of two (4 .. 256); 1 <= topk_group <=
 * n_group; 1 <= k <= 8; k <= topk_group * E / n_group.
 */
size_t moe_route_workspace_bytes(int64_t T, int64_t H, int32_t E);
int moe_route(const void* x_bf16, int64_t T, int64_t H,
              const float* centroids, const float* bias,
              int32_t E, int32_t n_group, int32_t topk_group, int32_t k,
              int32_t* topk_idx, float* topk_w, int32_t* expert_counts,
              void* workspace, size_t workspace_bytes, float* topk_s, void* stream);

/*
 * moe_route_scores - moe_route that also writes what the sequence-wise
 * balance statistic reads: scores [T, E] fp32, the unbiased sigmoid score of
 * every routed expert for every token (16-byte aligned), and score_sums [T]
 * fp32, their sum per token.  Same arguments, requirements, workspace and
 * results as moe_route otherwise.
 */
int moe_route_scores(const void* x_bf16, int64_t T, int64_t H,
                     const float* centroids, const float* bias,
                     int32_t E, int32_t n_group, int32_t topk_group, int32_t k,
                     int32_t* topk_idx, float* topk_w, int32_t* expert_counts,
                     void* workspace, size_t workspace_bytes, float* scores,
                     float* score_sums, float* topk_s, void* stream);

/*
 * moe_seq_balance - sequence-wise balance statistic (news.qq.com article,
 * section 无额外损耗的负载均衡: factor alpha = 0.0001; the V3 summary at
 * m.jxzklqfsx.com/aigc/3586.html, section （二）無輔助損失負載均衡策略革新: a
 * sequence-level term against imbalance inside one sequence).  The pages
 * give no formula; computed here, for each sequence b of L_b consecutive
 * tokens (runs of seq_len, the last may be shorter):
 *   P[b, e] = (1/L_b) sum_t scores[t, e] / score_sums[t]
 *   f[b, e] = E * (tokens of b that chose e) / (k * L_b)
 *   loss[b] = alpha * sum_e f[b, e] * P[b, e]
 * in fp32 with fixed summation order (f is exact up to one rounding).
 * scores, score_sums: moe_route_scores' outputs; topk_idx [T, k];
 * f_out, p_out (out) [B, E]; loss_out (out) [B], B = ceil(T / seq_len).
 * workspace: moe_seq_balance_workspace_bytes(T, E, seq_len) bytes.
 * Requirements: 1 <= E <= 256, 1 <= k <= E, 1 <= seq_len <= 65536.
 */
size_t moe_seq_balance_workspace_bytes(int64_t T, int32_t E, int64_t seq_len);
int moe_seq_balance(const float* scores, const float* score_sums, const int32_t* topk_idx,
                    int64_t T, int32_t E, int32_t k, int64_t seq_len, float alpha,
                    float* f_out, float* p_out, float* loss_out, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * moe_bias_update - aux-loss-free balancing step, in place.
 *
 * aliyun study note section 2.2 (overloaded experts' bias goes down,
 * underloaded goes up, no loss term) and news.qq.com article section
 * 无额外损耗的负载均衡 (update speed gamma = 0.001).  With total = sum_e
 * counts[e]: bias[e] -= gamma if counts[e]*E > total; bias[e] += gamma if
 * counts[e]*E < total; unchanged otherwise.  fp32 arithmetic; integer test.
 *
 * expert_counts [E] int32 (e.g. the output of moe_route for this batch)
 * bias          [E] fp32, updated in place
 * Requirements: 1 <= E <= 1024.
 */
int moe_bias_update(const int32_t* expert_counts, float* bias, int32_t E,
                    float gamma, void* stream);

/*
 * moe_permute - dispatch: expert-contiguous order of the token-expert
 * assignments (the all-to-all dispatch of the news.qq.com article, section
 * DualPipe 流水线并行, done inside one GPU).
 *
 * Rows of expert e are the assignments (t, j) with topk_idx[t,j] == e in
 * ascending (t, j) order; the n_shared shared expert(s) follow, one block of
 * T rows each in token order.  R = T*k + n_shared*T.
 *
 * topk_idx       [T, k] int32, values in [0, E)
 * expert_counts  [E] int32, the histogram of topk_idx (as moe_route writes)
 * offsets  (out) [E + n_shared + 1] int32: exclusive prefix sum of group sizes
 * perm_src (out) [R] int32: token of each row
 * inv_perm (out) [T*k] int32: row of assignment (t, j) at t*k + j
 * xq, xs         optional [T, H] e4m3 and [T, H/128] fp32; when a_out is not
 *                NULL, a_out[r] = xq[perm_src[r]] and a_scale_out[r] =
 *                xs[perm_src[r]] ([R, H] e4m3, [R, H/128] fp32).
 * workspace      at least moe_permute_workspace_bytes(T, k, E) bytes.
 * Requirements: 1 <= k <= 8; 1 <= E <= 4096; n_shared in {0, 1};
 * H % 128 == 0 when gathering.  topk_idx and expert_counts must be consistent.
 */
size_t moe_permute_workspace_bytes(int64_t T, int32_t k, int32_t E);
int moe_permute(const int32_t* topk_idx, const int32_t* expert_counts,
                int64_t T, int32_t k, int32_t E, int32_t n_shared,
                int32_t* offsets, int32_t* perm_src, int32_t* inv_perm,
                const uint8_t* xq, const float* xs, int64_t H,
                uint8_t* a_out, float* a_scale_out,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_permute_noalloc - moe_permute for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, outputs and errors as moe_permute minus
 * the workspace: the per-chunk histograms live in a static device array of
 * MOE_PERMUTE_SCRATCH_BYTES bytes that the library keeps on every GPU it
 * runs on until the process ends (its address is looked up once per device,
 * on the first call with that device current).  The call allocates nothing.
 * Its scratch need is moe_permute_workspace_bytes(T, k, E); a larger need
 * (ceil(T/64) * E > 262144, e.g. T > 65536 at E = 256) returns
 * MOE_ERR_WORKSPACE without launching.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (different streams, or host
 * threads without ordering) race; calls ordered on one stream do not.
 */
#define MOE_PERMUTE_SCRATCH_BYTES ((size_t)1 << 20)
int moe_permute_noalloc(const int32_t* topk_idx, const int32_t* expert_counts,
                        int64_t T, int32_t k, int32_t E, int32_t n_shared,
                        int32_t* offsets, int32_t* perm_src, int32_t* inv_perm,
                        const uint8_t* xq, const float* xs, int64_t H,
                        uint8_t* a_out, float* a_scale_out, void* stream);

/*
 * fp8_quant_1x128 - fine-grained activation quantisation (news.qq.com
 * article, section FP8 低精度训练 › 细粒度量化: 1x128 tiles for activations).
 *
 * For each row m and 128-column tile j of the output:
 *   v     = mode 0: in[m, j*128 + c]
 *           mode 1: silu(g) * u with g = in[m, j*128 + c], u = in[m, K + j*128 + c]
 *                   evaluated in fp32 as a = g / (1 + exp(-g)); v = a * u
 *   amax  = max_c |v|;  s = amax / 448 (fp32), or 1 if amax == 0
 *   out   = E4M3FN(v / s): correctly rounded fp32 division, round to nearest
 *           even, saturate to +-448, sign of zero kept
 *   scales[m, j] = s
 *
 * in_bf16  [M, ld_in] bf16; mode 0 needs ld_in >= K, mode 1 needs ld_in >= 2K
 * out_e4m3 [M, K] e4m3;  scales [M, K/128] fp32
 * Requirements: K % 128 == 0, ld_in % 8 == 0, mode in {0, 1}.
 */
int fp8_quant_1x128(const void* in_bf16, int64_t M, int64_t K, int64_t ld_in,
                    int32_t mode, uint8_t* out_e4m3, float* scales, void* stream);

/*
 * fp8_quant_128x128 - weight quantisation in 128x128 blocks (aliyun study
 * note section 4.1; news.qq.com article section 细粒度量化).  Same scale and
 * rounding rule as fp8_quant_1x128, with amax taken over each block.
 *
 * w_f32    [G, N, K] fp32;  out_e4m3 [G, N, K];  scales [G, N/128, K/128]
 * Requirements: N % 128 == 0, K % 128 == 0.
 */
int fp8_quant_128x128(const float* w_f32, int64_t G, int64_t N, int64_t K,
                      uint8_t* out_e4m3, float* scales, void* stream);

/*
 * fp8_transpose_128x128 - weights in 128x128 blocks, transposed block by block
 * (news.qq.com article, section FP8 低精度训练 › 细粒度量化: 128x128 weight
 * blocks; section 工程 › DualPipe 流水线并行: the pipeline's backward-for-input
 * chunks).  The expert GEMM C = A W^T has the input gradient dA = dY W, a
 * contraction over n: grouped_fp8_gemm computes it with dY quantised by
 * fp8_quant_1x128 and B = W^T from this call (N' = K, K' = N).
 *
 *   wt[g, k, n] = w[g, n, k];   wt_scale[g, kb, nb] = w_scale[g, nb, kb]
 *
 * Codes and scales move unchanged, so the output is exactly the 128x128
 * quantisation of W^T.
 * w_e4m3   [G, N, K] e4m3 (16-byte aligned);  w_scale [G, N/128, K/128] fp32
 * wt_e4m3  (out) [G, K, N] e4m3;  wt_scale (out) [G, K/128, N/128] fp32
 * Requirements: N % 128 == 0, K % 128 == 0, 0 <= G <= 65535, outputs not
 * aliasing inputs.  G == 0 is a no-op.
 */
int fp8_transpose_128x128(const uint8_t* w_e4m3, const float* w_scale, int64_t G,
                          int64_t N, int64_t K, uint8_t* wt_e4m3, float* wt_scale,
                          void* stream);

/*
 * fp8_quant_128x1_grouped - the weight-gradient operands: per-group FP8
 * quantisation in 128x1 tiles along the token axis (news.qq.com article,
 * section FP8 低精度训练 › 细粒度量化 gives 1x128 activation tiles; the
 * weight gradient contracts over tokens, so the tile is taken along them - a
 * reading, the pages give no backward orientation; section 工程 › DualPipe
 * 流水线并行 names the backward-for-weights chunks).
 *
 * Group g (rows group_offsets[g] .. group_offsets[g+1]) is cut into 128-row
 * chunks from its first row, the last one padded with zeros; chunk c of the
 * layout is the c-th in group order (group g's chunks start at the sum over
 * g' < g of ceil(rows_g' / 128)).  Stored chunk-major: for column j and
 * chunk c,
 *   s = amax over the chunk's rows of |in[r, j]| / 448 (1 if 0)
 *   out_c[c, j, i]  = E4M3(in[row i of chunk c, j] / s)  (0 for padding)
 *   scales_c[c, j]  = s
 * with the rounding of fp8_quant_1x128.  (out_c[c] transposed is the 128
 * tokens of chunk c as rows: a tile's chunk is one contiguous block.)
 *
 * in_bf16   [in_rows, ld_in] bf16 (C columns used; 16-byte aligned, ld_in % 8 == 0)
 * row_index [M_total] int32 or NULL: layout row r reads input row row_index[r]
 *           (an entry outside [0, in_rows) reads row in_rows - 1), else row r
 * in_rows   rows of in_bf16: >= M_total without a row index, >= 1 with one
 * group_offsets [G+1] int32 on the device, as in grouped_fp8_gemm
 * out_c     (out) [chunks_cap, C, 128] e4m3 (16-byte aligned)
 * scales_c  (out) [chunks_cap, C] fp32
 * chunks_cap >= ceil(M_total / 128) + G (chunks past the last are not written)
 * Requirements: 1 <= G <= 1024, C % 128 == 0, ld_in >= C.
 */
int fp8_quant_128x1_grouped(const void* in_bf16, int64_t ld_in, const int32_t* row_index,
                            int64_t in_rows, const int32_t* group_offsets, int32_t G,
                            int64_t M_total, int64_t C, uint8_t* out_c, float* scales_c,
                            int64_t chunks_cap, void* stream);

/*
 * grouped_fp8_wgrad - weight gradient of the expert GEMMs (news.qq.com article,
 * section 工程 › DualPipe 流水线并行: backward-for-weights chunks; section FP8
 * 低精度训练: FP8 products accumulated in FP32 at a fixed K interval).
 *
 * For the forward C_g = A_g W_g^T (W_g [N, K]) and the output gradient dY,
 *   dW[g, n, k] = sum_{c in group g's chunks}  dy_scale_c[c, n] * a_scale_c[c, k]
 *                 * sum_{i<128} dy_c[c, n, i] * a_c[c, k, i]
 * with dy_c / a_c from fp8_quant_128x1_grouped of dY [M_total, N] and
 * A [M_total, K] on the same group_offsets.  Each chunk's 128-term FP8
 * partial is an FP32 MFMA sum added to one FP32 accumulator kept in units of
 * the current chunk's scale product (rescaled by the ratio of consecutive
 * chunks' scales, multiplied by the last one at the end).  A group without
 * rows gets dW[g] = 0.
 *
 * dy_c [chunks_cap, N, 128], dy_scale_c [chunks_cap, N];
 * a_c  [chunks_cap, K, 128], a_scale_c  [chunks_cap, K]
 * dW   (out) [G, N, K] fp32 (overwritten)
 * Requirements: N % 128 == 0, K % 128 == 0, 1 <= G <= 65535,
 * chunks_cap >= ceil(M_total / 128) + G; operands and dW 16-byte, scales
 * 4-byte aligned.
 */
int grouped_fp8_wgrad(const uint8_t* dy_c, const float* dy_scale_c, const uint8_t* a_c,
                      const float* a_scale_c, int64_t chunks_cap, const int32_t* group_offsets,
                      int32_t G, int64_t M_total, int64_t N, int64_t K, float* dW,
                      void* stream);

/*
 * moe_combine_backward - backward of moe_combine (news.qq.com article, section
 * DeepSeekMoE 架构: gate-weighted routed experts plus the always-on shared
 * one; section 工程 › DualPipe 流水线并行: the backward-for-input chunks).
 *
 * For the forward y[t] = sum_j w[t,j] D[inv_perm[t*k+j]] + D[T*k + t]:
 *   dD[inv_perm[t*k+j], :] = bf16( w[t,j] * dy[t, :] )   (fp32 product)
 *   dD[T*k + t, :]         = dy[t, :]                      (n_shared == 1)
 *   dw[t*k + j]            = sum_h dy[t, h] * D[inv_perm[t*k+j], h]  (fp32,
 *                            summed in a fixed order)
 * dy_bf16 [T, H]; inv_perm [T*k] (a permutation of [0, T*k)); topk_w [T*k];
 * expert_out_bf16 D [T*k + n_shared*T, H]; d_expert_out_bf16 (out) like D;
 * d_topk_w (out) [T*k] fp32.
 * d_expert_out_e4m3, d_expert_out_scale (out, both or neither; NULL: not
 * written) [T*k + n_shared*T, H] e4m3 and [.., H/128] fp32: the 1x128
 * quantisation of dD as stored (bit for bit what fp8_quant_1x128 mode 0
 * writes for d_expert_out_bf16), formed in the same pass so the input-
 * gradient GEMM's operand needs no second read of dD (section FP8 低精度训练
 * › 细粒度量化); requires H % 128 == 0, codes 8-byte and scales 4-byte aligned.
 * Requirements: 1 <= k <= 8, H % 8 == 0, n_shared in {0, 1}; dy, D, dD
 * 16-byte aligned, dD not aliasing D.
 */
int moe_combine_backward(const void* dy_bf16, const int32_t* inv_perm, const float* topk_w,
                         const void* expert_out_bf16, int64_t T, int32_t k, int64_t H,
                         int32_t n_shared, void* d_expert_out_bf16, float* d_topk_w,
                         uint8_t* d_expert_out_e4m3, float* d_expert_out_scale, void* stream);

/*
 * swiglu_backward - backward of h = silu(g) * u (the experts' SwiGLU, see
 * grouped_fp8_gemm_swiglu) from the bf16 gate/up outputs, in fp32:
 *   s = 1 / (1 + exp(-g));  dg = dh * u * s * (1 + g * (1 - s));  du = dh * g * s;
 *   h = g * s * u
 * gu_bf16 [M, 2I] = [g | u]; dh_bf16 [M, I]; dgu_bf16 (out) [M, 2I] = [dg | du];
 * h_bf16 (out) [M, I] (the down projection's weight-gradient operand); all
 * stored as bf16 (round to nearest even), 16-byte aligned.  I % 8 == 0.
 * dgu_e4m3, dgu_scale (out, both or neither; NULL: not written) [M, 2I] e4m3
 * and [M, 2I/128] fp32: the 1x128 quantisation of dGU as stored (bit for
 * bit what fp8_quant_1x128 mode 0 writes for dgu_bf16), in the same pass;
 * requires I % 128 == 0, codes 8-byte and scales 4-byte aligned.
 */
int swiglu_backward(const void* gu_bf16, const void* dh_bf16, int64_t M, int64_t I,
                    void* dgu_bf16, void* h_bf16, uint8_t* dgu_e4m3, float* dgu_scale,
                    void* stream);

/*
 * swiglu_backward_grouped - swiglu_backward over the rows of G groups (the
 * experts' permuted rows) that also writes the FP8 operands the backward's
 * GEMMs read, from the stored bf16 values, in the same pass (news.qq.com
 * article, section FP8 低精度训练 › 细粒度量化; section 工程 › DualPipe
 * 流水线并行: backward-for-input and backward-for-weights chunks):
 *   dgu_bf16, h_bf16 (out, optional: both NULL to skip them): as
 *     swiglu_backward, bit for bit (the codes below do not depend on them);
 *   dgu_e4m3 [M_total, 2I], dgu_scale [M_total, 2I/128] (out): what
 *     fp8_quant_1x128 mode 0 writes for dgu_bf16;
 *   dgu_c, dgu_scale_c (out, C = 2I) and h_c, h_scale_c (out, C = I): what
 *     fp8_quant_128x1_grouped writes for dgu_bf16 and h_bf16 with the same
 *     group_offsets and chunks_cap (chunk-major, zero-padded chunks).
 * gu_bf16 [M_total, 2I] = [g | u]; dh_bf16 [M_total, I]; group_offsets [G+1]
 * int32 on the device (non-decreasing, [0] == 0, [G] == M_total).
 * Requirements: I % 128 == 0, 1 <= G <= 1024, chunks_cap >= ceil(M_total/128)
 * + G; tensors and codes 16-byte aligned, scales 4-byte aligned.  M_total ==
 * 0 is a no-op.
 */
int swiglu_backward_grouped(const void* gu_bf16, const void* dh_bf16,
                            const int32_t* group_offsets, int32_t G, int64_t M_total, int64_t I,
                            void* dgu_bf16, void* h_bf16, uint8_t* dgu_e4m3, float* dgu_scale,
                            int64_t chunks_cap, uint8_t* dgu_c, float* dgu_scale_c, uint8_t* h_c,
                            float* h_scale_c, void* stream);

/*
 * moe_router_backward - backward of the gate weights to the router's input and
 * the per-expert logits (news.qq.com article: section 无额外损耗的负载均衡 - the
 * bias only selects, so neither it nor the choice of experts has a gradient;
 * section FP8 低精度训练 - the gating stays in FP32).
 *
 * For token t with selected experts e_j = topk_idx[t, j] and the unbiased
 * scores s_j = sigmoid(x[t] . C[e_j]) - the forward's (topk_s as moe_route
 * wrote it), or recomputed here in fp32 when topk_s is NULL - (S = sum_j
 * s_j in slot order, w_j = s_j / S, the forward's gate weights):
 *   dlogit_j = (dw_j - sum_i dw_i w_i) / S * s_j * (1 - s_j)
 *   dx_out[t, :] = bf16( dx_in[t, :] + sum_j dlogit_j * C[e_j, :] )   (fp32 sums)
 *   dlogit_rows[inv_perm[t*k + j]] = dlogit_j   (expert-row order, for the
 *                                                centroid gradient)
 * x_bf16 [T, H]; centroids [E, H] fp32; topk_idx, d_topk_w, inv_perm [T*k];
 * dx_in_bf16 [T, H] or NULL (then 0); dx_out_bf16 (out) [T, H] (may equal
 * dx_in); dlogit_rows (out) [T*k] fp32.  Requirements: 1 <= k <= 8, k <= E,
 * H % 8 == 0; x, centroids, dx_in, dx_out 16-byte aligned.  Expert ids
 * outside [0, E) read centroid E - 1 and inv_perm rows outside [0, T*k) are
 * not written (neither occurs for moe_route / moe_permute outputs).
 */
int moe_router_backward(const void* x_bf16, const float* centroids, const int32_t* topk_idx,
                        const float* d_topk_w, const int32_t* inv_perm, const void* dx_in_bf16,
                        int64_t T, int64_t H, int32_t E, int32_t k, void* dx_out_bf16,
                        float* dlogit_rows, const float* topk_s, void* stream);

/*
 * moe_router_dcentroids - gradient of the router centroids (same sections):
 *   dC[e, :] = sum over rows r in [group_offsets[e], group_offsets[e+1]) of
 *              dlogit_rows[r] * x[perm_src[r], :]
 * summed in fp32 in row order (the rows of expert e are its tokens in
 * ascending order, as moe_permute lays them out).
 * x_bf16 [T, H]; perm_src, dlogit_rows: moe_permute's / moe_router_backward's;
 * group_offsets [E+1] (the routed part of moe_permute's offsets, on the device);
 * d_centroids (out) [E, H] fp32.  Requirements: H % 8 == 0, 1 <= E <= 65535;
 * x and d_centroids 16-byte aligned.  T = 0 writes d_centroids = 0 (the other
 * pointers may then be NULL).  perm_src entries outside [0, T) read token
 * T - 1; group_offsets must be moe_permute's.
 */
int moe_router_dcentroids(const void* x_bf16, const int32_t* perm_src,
                          const int32_t* group_offsets, const float* dlogit_rows, int64_t T,
                          int64_t H, int32_t E, float* d_centroids, void* stream);

/*
 * moe_router_backward_dense - the router's backward when the loss also holds
 * the sequence-wise balance term alpha * sum_b L_bal,b of moe_seq_balance
 * (news.qq.com article, section 无额外损耗的负载均衡: the bias only selects,
 * alpha = 0.0001; section FP8 低精度训练: gating in FP32; the V3 summary at
 * m.jxzklqfsx.com/aigc/3586.html, section （二）無輔助損失負載均衡策略革新).
 * With the selection (and so f) held fixed, for token t of sequence b
 * (L_b tokens), s = scores[t, :], S = score_sums[t]:
 *   dlogit[t, e] = alpha / L_b * (f[b, e] - sum_i f[b, i] s_i / S) / S
 *                  * s_e (1 - s_e)
 *                + on each chosen expert e_j: (dw_j - sum_i dw_i w_i) / S_sel
 *                  * s_j (1 - s_j), S_sel = sum_j s_{e_j}, w_j = s_{e_j} / S_sel
 *   dx_out[t, :]  = bf16(dx_in[t, :] + sum_e dlogit[t, e] C[e, :])  (fp32 sums)
 *   d_centroids[e, :] = sum_t dlogit[t, e] x[t, :]  (fp32, tokens in slices of
 *                       ~1024 summed in order, then the slices in order)
 * x_bf16 [T, H]; centroids [E, H] fp32; topk_idx, d_topk_w [T, k]; scores,
 * score_sums: moe_route_scores' outputs of the forward; seq_f [B, E]:
 * moe_seq_balance's f for the same seq_len; dx_in_bf16 [T, H] or NULL (0),
 * must not alias dx_out; dx_out_bf16 (out) [T, H]; d_centroids (out) [E, H];
 * dlogit (out) [T, E] fp32.  workspace:
 * moe_router_backward_dense_workspace_bytes(T, H, E) bytes (0: none needed).
 * Requirements: E % 16 == 0, 16 <= E <= 256, 1 <= k <= 8, H % 128 == 0,
 * 1 <= seq_len <= 65536; x, centroids, scores, seq_f, dx_in, dx_out,
 * d_centroids, dlogit 16-byte aligned.  T = 0 writes d_centroids = 0.
 * Expert ids outside [0, E) count as expert E - 1.
 */
size_t moe_router_backward_dense_workspace_bytes(int64_t T, int64_t H, int32_t E);
int moe_router_backward_dense(const void* x_bf16, const float* centroids,
                              const int32_t* topk_idx, const float* d_topk_w,
                              const float* scores, const float* score_sums, const float* seq_f,
                              int64_t T, int64_t H, int32_t E, int32_t k, int64_t seq_len,
                              float alpha, const void* dx_in_bf16, void* dx_out_bf16,
                              float* d_centroids, float* dlogit, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * grouped_fp8_gemm - block-scaled FP8 grouped GEMM with FP32 accumulation
 * (news.qq.com article, section FP8 低精度训练, items 细粒度量化 and
 * 提高累加精度).
 *
 * For group g, rows r in [group_offsets[g], group_offsets[g+1]):
 *   C[r, n] = bf16( sum_kb  sa[r, kb] * B_scale[g, n/128, kb]
 *                           * sum_{k in block kb} a[r, k] * B[g, n, k] )
 * where a[r, :] = A[src(r), :], sa[r, :] = A_scale[src(r), :], and
 * src(r) = a_row_index[r] if a_row_index is not NULL, else r.  Each 128-wide
 * K block is one FP8 MFMA partial in FP32 that is scaled and added to an FP32
 * total; the total is rounded to bf16 (nearest even) once.
 *
 * A        [A_rows, K] e4m3
 * A_scale  [A_rows, K/128] fp32
 * a_row_index  [M_total] int32 or NULL; entries should lie in [0, A_rows):
 *          an entry outside it reads row A_rows - 1 (never memory past A)
 * A_rows   rows of A and A_scale: >= M_total when a_row_index is NULL, >= 1
 *          otherwise
 * B        [G, N, K] e4m3 (each group's matrix stored N x K, K contiguous)
 * B_scale  [G, N/128, K/128] fp32
 * group_offsets [G+1] int32 on the device, non-decreasing, [0] == 0,
 *          [G] == M_total (read by the kernels, never by the host)
 * C  (out) [M_total, N] bf16
 * Requirements: N % 128 == 0, K % 128 == 0, G >= 1 (more than 1024 groups returns
 * MOE_ERR_UNSUPPORTED).
 */
int grouped_fp8_gemm(const uint8_t* A, const float* A_scale, const int32_t* a_row_index,
                     int64_t A_rows, const uint8_t* B, const float* B_scale,
                     const int32_t* group_offsets, int32_t G, int64_t M_total,
                     int64_t N, int64_t K, void* C_bf16, void* stream);

/*
 * grouped_fp8_gemm_dgrad - the input gradient of grouped_fp8_gemm, read
 * from the weights in their forward layout (news.qq.com article, section
 * FP8 低精度训练 › 细粒度量化: 1x128 activation tiles, 128x128 weight blocks;
 * section 工程 › DualPipe 流水线并行: the backward-for-input chunks).  For
 * the forward C = A W^T of group g (W [N, K]), the gradient is dA = dC W, a
 * contraction over n:
 *   dA[r, k] = bf16( sum_nb  sdc[r, nb] * W_scale[g, nb, k/128]
 *                            * sum_{n in block nb} dC[r, n] * W[g, n, k] )
 * with dC quantised by fp8_quant_1x128 along n.  Each 128-wide n block is one
 * FP8 MFMA partial in FP32, as in grouped_fp8_gemm, whose result this equals
 * bit for bit when given B = the fp8_transpose_128x128 of W; no transposed
 * copy is made (the kernel forms its operand with LDS transpose reads).
 *
 * dC       [M_total, N] e4m3;  dC_scale [M_total, N/128] fp32
 * W        [G, N, K] e4m3, W_scale [G, N/128, K/128] fp32: the forward B
 * group_offsets [G+1] int32 on the device, as in grouped_fp8_gemm
 * dA (out) [M_total, K] bf16
 * Requirements: N % 128 == 0, K % 128 == 0, G >= 1 (more than 1024 groups
 * returns MOE_ERR_UNSUPPORTED).
 */
int grouped_fp8_gemm_dgrad(const uint8_t* dC, const float* dC_scale, const uint8_t* W,
                           const float* W_scale, const int32_t* group_offsets, int32_t G,
                           int64_t M_total, int64_t N, int64_t K, void* dA_bf16, void* stream);

/*
 * grouped_fp8_gemm_swiglu - the gate+up GEMM of the experts with SwiGLU and
 * 1x128 requantisation fused into its epilogue (news.qq.com article, section
 * FP8 低精度训练: FP8 GEMM with fine-grained scales and FP32 accumulation,
 * activations kept in FP8; the SwiGLU form is this layer's expert FFN).
 *
 * B holds each group's fused weight [2I, K]: rows [0, I) gate, [I, 2I) up.
 * For row r of group g and column c < I, with the FP32 totals
 *   gt = sum_kb sa[r,kb] * B_scale[g, c/128, kb]     * sum_k a[r,k] B[g, c, k]
 *   ut = sum_kb sa[r,kb] * B_scale[g, (I+c)/128, kb] * sum_k a[r,k] B[g, I+c, k]
 * (accumulated as in grouped_fp8_gemm but never rounded to bf16 or stored):
 *   h = (gt / (1 + exp(-gt))) * ut  in fp32, then per 128 columns of h
 *   s = amax/448 (1 if 0), H_e4m3[r, c] = E4M3(h / s), H_scale[r, c/128] = s.
 *
 * A, A_scale, a_row_index, A_rows, B_scale, group_offsets: as grouped_fp8_gemm with
 * N = 2I.  H_e4m3 (out) [M_total, I] e4m3; H_scale (out) [M_total, I/128].
 * Requirements: I % 128 == 0, K % 128 == 0, 1 <= G <= 1024.
 */
int grouped_fp8_gemm_swiglu(const uint8_t* A, const float* A_scale,
                            const int32_t* a_row_index, int64_t A_rows, const uint8_t* B,
                            const float* B_scale, const int32_t* group_offsets,
                            int32_t G, int64_t M_total, int64_t I, int64_t K,
                            uint8_t* H_e4m3, float* H_scale, void* stream);

/*
 * grouped_fp8_gemm_swiglu_keep - grouped_fp8_gemm_swiglu that also writes
 * the gate/up totals as bf16 (round to nearest even): GU_bf16 [M_total, 2I]
 * = [gt | ut], the bits grouped_fp8_gemm would write for the same operands.
 * For training: the backward's SwiGLU step reads them instead of running the
 * gate+up GEMM again (the pages' FP8 training keeps the FP8 GEMMs; keeping
 * rather than recomputing these outputs is this library's choice, with the
 * HBM to hold them).  Same arguments, requirements and H outputs as
 * grouped_fp8_gemm_swiglu; GU_bf16 16-byte aligned.  Groups below the fused
 * 256-row kernel's size run the fused kernel and grouped_fp8_gemm in turn.
 */
int grouped_fp8_gemm_swiglu_keep(const uint8_t* A, const float* A_scale,
                                 const int32_t* a_row_index, int64_t A_rows, const uint8_t* B,
                                 const float* B_scale, const int32_t* group_offsets,
                                 int32_t G, int64_t M_total, int64_t I, int64_t K,
                                 uint8_t* H_e4m3, float* H_scale, void* GU_bf16, void* stream);

/*
 * moe_combine - weighted combine plus shared expert (news.qq.com article,
 * section DeepSeekMoE 架构: shared experts are always on, routed experts are
 * weighted by their gates).
 *
 *   y[t, :] = bf16( sum_{j<k} w[t, j] * D[inv_perm[t*k + j], :] + S[t, :] )
 * accumulated in fp32 in slot order j = 0..k-1, then S added.
 *
 * expert_out_bf16 D [R, H] bf16 (R >= T*k)
 * inv_perm        [T*k] int32
 * topk_w          [T, k] fp32
 * shared_out_bf16 S [T, H] bf16, or NULL for no shared expert
 * y_bf16    (out) [T, H] bf16
 * Requirements: 1 <= k <= 8, H % 8 == 0.
 */
int moe_combine(const void* expert_out_bf16, const int32_t* inv_perm,
                const float* topk_w, const void* shared_out_bf16,
                int64_t T, int32_t k, int64_t H, void* y_bf16, void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif /* MOE_FP8_H */
