// Launchers of the MoE kernels; the C ABI in moe_api.hip validates arguments
// and calls these.  All sizes here have been checked by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_common.h"

namespace moe {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

hipError_t launch_router_topk(const void* x, const void* Wg, int T, int d, int E, int K,
                              int dtype, int32_t* topk_idx, float* topk_w, float* logits,
                              hipStream_t stream);

// Glue between pre-norm blocks for small batches (one workgroup per token):
// [the previous block's combine into h with the residual add, when O is not
// null], RMSNorm of h into xn, and the router of the next block on xn.
// Bit-identical to launch_combine(accumulate) + launch_rmsnorm +
// launch_router_topk.  Needs stack_glue_supported().
constexpr int kStackGlueMaxD = 16384;
bool stack_glue_supported(int T, int d, int E, int dtype);
hipError_t launch_stack_glue(void* h, void* xn, const float* O, int o_splits, int64_t slice,
                             float* topk_w, const int32_t* pos, int32_t* topk_idx, const void* Wg,
                             int T, int d, int E, int K, float eps, hipStream_t stream);
// The glue without the router, for any batch: [the previous block's combine
// into h with the residual add, when O is not null] and RMSNorm of h into xn,
// one workgroup per token.  Bit-identical to launch_combine(accumulate) +
// launch_rmsnorm.  Needs stack_norm_supported().
bool stack_norm_supported(int d, int dtype);
hipError_t launch_stack_norm(void* h, void* xn, const float* O, int o_splits, int64_t slice,
                             const float* topk_w, const int32_t* pos, int T, int d, int K,
                             float eps, hipStream_t stream);

hipError_t launch_route_permute(const int32_t* topk_idx, int T, int E, int K, int32_t* offsets,
                                int32_t* sorted_token, int32_t* pos, hipStream_t stream);

// counts[e] = pairs routed to e; repeats[0] = #{t >= 1 : idx[t][0] == idx[t-1][0]}.
hipError_t launch_routing_stats(const int32_t* topk_idx, int T, int E, int K, int32_t* counts,
                                int32_t* repeats, hipStream_t stream);

// a6: H[r] = round(SiLU(A[r] W1[e]) * (A[r] W3[e])) over the expert-sorted
// rows r of expert e, A[r] = x[sorted_token[r]].
hipError_t launch_expert_swiglu_bf16(const void* x, const int32_t* sorted_token,
                                     const ExpertPtrs& W1, const ExpertPtrs& W3,
                                     const int32_t* offsets, int P, int d, int d_ff, int E,
                                     void* H, hipStream_t stream);
hipError_t launch_expert_swiglu_f32(const void* x, const int32_t* sorted_token,
                                    const ExpertPtrs& W1, const ExpertPtrs& W3,
                                    const int32_t* offsets, int P, int d, int d_ff, int E,
                                    void* H, hipStream_t stream);

// a7: O[r] = H[r] W2[e] over expert-sorted rows, fp32 O.
hipError_t launch_expert_down_bf16(const void* H, const ExpertPtrs& W2, const int32_t* offsets,
                                   int P, int d, int d_ff, int E, float* O, hipStream_t stream);
hipError_t launch_expert_down_f32(const void* H, const ExpertPtrs& W2, const int32_t* offsets,
                                  int P, int d, int d_ff, int E, float* O, hipStream_t stream);

// Weight-streaming variants for small batches (every expert segment of at
// most 16 rows per token tile), N in tiles of kStreamFeat features.
constexpr int kStreamFeat = 256;
// W1/W3 launch when about `tiles` token tiles hold rows: 0 = fused (H written
// by the product), s >= 1 = one matrix at a time over a persistent grid that
// divides the weight rows evenly between the compute units, leaving fp32
// partial sums in up to s slices per matrix (completed by
// launch_swiglu_finish_bf16, which reads the expert offsets to know how many
// each unit has); -1 if the shape cannot stream.
int stream_swiglu_splits(int d, int d_ff, double tiles);
// W2 K split (slices of O) for about `tiles` busy token tiles; 0 if the
// shape cannot stream.
int stream_down_splits(int d_ff, int d, double tiles);
// With topk_idx non-null the kernels build the dispatch tables themselves
// from the routing table and write offsets, sorted_token and pos (so no
// dispatch launch is needed); otherwise they read the caller's offsets and
// sorted_token.
hipError_t launch_stream_swiglu_bf16(const void* x, const int32_t* sorted_token,
                                     const ExpertPtrs& W1, const ExpertPtrs& W3,
                                     const int32_t* offsets, int P, int d, int d_ff, int E,
                                     int splits, float* part, void* H, const int32_t* topk_idx,
                                     int K, int32_t* pos, hipStream_t stream);
// H[r][f] = bf16(SiLU(sum_s part[s][0][r][f]) * sum_s part[s][1][r][f]), over
// the splits the W1/W3 launch took.
hipError_t launch_swiglu_finish_bf16(const float* part, const int32_t* offsets, int P, int d,
                                     int d_ff, int E, void* H, hipStream_t stream);
hipError_t launch_stream_down_bf16(const void* H, const ExpertPtrs& W2, const int32_t* offsets,
                                   int P, int d, int d_ff, int E, int splits, float* O,
                                   hipStream_t stream);

// CDNA4 tiled variants for large batches (direct-to-LDS loads, transposed
// LDS reads); need Kdim % 128 == 0 and N % 128 (W1/W3) or N % 256 (W2).
// a_rows: rows of the token operand (x or H); their byte offsets must fit
// 32 bits, else the grouped kernels of expert_gemm_bf16.hip take the product.
bool tiled_gemm_supported(int Kdim, int N, bool dual, int splits, int64_t a_rows);
int tiled_gemm_tiles(int P, int E, int N, bool dual);  // worst-case workgroups per split
// Whether the tiled W1/W3 launch chooses its tile shape per expert (128 x 512
// for experts of at most 128 rows, 256 x 256 otherwise).
bool tiled_swiglu_mixed(int P, int E, int d_ff);
// Whether the tiled products copy weights with the non-temporal cache policy
// (each expert's rows fill about one token tile, so each weight tile is read
// once).
bool weights_read_once(int64_t P, int E);
hipError_t launch_tiled_swiglu_bf16(const void* x, const int32_t* sorted_token,
                                    const ExpertPtrs& W1, const ExpertPtrs& W3,
                                    const int32_t* offsets, int P, int d, int d_ff, int E,
                                    void* H, hipStream_t stream);
// With `side` (tiled_down_side_bytes bytes, splits == 1) the W2 launch runs
// whole tiles for its complete rounds of compute units and cuts the tiles of
// its last, partial round into K pieces whose fp32 partial sums land in
// `side`; launch_tiled_down_fixup then writes their O rows.  O has one slice.
size_t tiled_down_side_bytes(int P, int d, int d_ff);
hipError_t launch_tiled_down_bf16(const void* H, const ExpertPtrs& W2, const int32_t* offsets,
                                  int P, int d, int d_ff, int E, int splits, float* O,
                                  float* side, size_t side_bytes, hipStream_t stream);
hipError_t launch_tiled_down_fixup(const float* side, size_t side_bytes, const int32_t* offsets,
                                   int P, int d, int d_ff, int E, float* O, hipStream_t stream);

// Lets `kernel` use `bytes` of dynamic LDS on the current device (once per
// device and kernel).
hipError_t allow_dynamic_lds(const void* kernel, int bytes);

// O holds o_splits slices of [P, d]; each token sums its K rows in rank order
// after summing the slices in slice order.
hipError_t launch_combine(const float* O, int o_splits, int64_t slice, const float* topk_w,
                          const int32_t* pos, int T, int d, int K, void* y, int y_dtype,
                          int accumulate, hipStream_t stream);

hipError_t launch_rmsnorm(const void* h, void* out, int T, int d, float eps, int dtype,
                          hipStream_t stream);

// Sliding-window grouped-query attention (swa_attention.hip).
int swa_head_dim();
int swa_plan_splits(int B, int T, int W, int H, int KVH, int* qtiles_out, int* qsub_out);
hipError_t launch_swa_attention(const void* q, const void* k_new, const void* v_new,
                                const void* k_cache, const void* v_cache, const int32_t* pos0,
                                int B, int T, int W, int H, int KVH, void* out, int out_f32,
                                float* part_o, float* part_ml, hipStream_t stream);
hipError_t launch_swa_append(const void* k_new, const void* v_new, const int32_t* pos0, int B,
                             int T, int W, int KVH, void* k_cache, void* v_cache,
                             hipStream_t stream);

}  // namespace moe
