/*
 * moe_mi355x.h -- C ABI of the Mixtral sparse mixture-of-experts layer
 * forward on one AMD Instinct MI355X (gfx950).
 *
 * The layer ("从Mistral 7B到MoE模型Mixtral 8x7B的全面解析：从原理分析到代码解读",
 * aiqianji.com, section 2.1.1; "Mixtral of Experts", xyznot.com, section
 * "Method with key equations"):
 *
 *     l      = x . W_g                              router logits, no bias
 *     G(x)   = Softmax(TopK(l))                     TopK masks all but K logits
 *     y      = sum_i G(x)_i * SwiGLU_i(x)           only experts with G_i > 0
 *     SwiGLU_i(x) = (SiLU(x W1_i) * (x W3_i)) W2_i  (section 3.2.4, code block D)
 *
 * Layout (row-major, the pages' "x . W" orientation):
 *     x, y      [T, d]
 *     W_g       [d, E]
 *     W1[e], W3[e]  [d, d_ff]
 *     W2[e]     [d_ff, d]
 * W1, W3, W2 are HOST arrays of E device pointers, read during the call only.
 * Every other pointer is device memory owned by the caller.  The library
 * allocates no device memory on these calls; moe_forward carves its
 * intermediates from the caller's workspace.
 *
 * Types: dtype MOE_F32 means float32 storage and float32 arithmetic;
 * MOE_BF16 means bfloat16 storage with float32 accumulation (bf16 x bf16 ->
 * fp32 matrix-core products).  Gate weights and logits are float32 in both.
 *
 * Errors: arguments are validated on the host before anything is enqueued;
 * a non-zero status means nothing was launched.  MOE_EHIP reports a launch
 * failure.  Execution is asynchronous on `stream` (a hipStream_t, NULL = the
 * default stream): faults surface at the caller's next synchronisation.
 * Results are bit-identical across runs for identical inputs (no atomics on
 * any floating-point result).  Inputs must be finite.  Calls on distinct
 * (stream, workspace) pairs may run concurrently.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5
#define MOE_MAX_EXPERTS 64

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* bad pointer, size, K/E, aliasing, alignment */
  MOE_EUNSUPPORTED = 2,  /* valid but not supported (e.g. bf16 d % 64 != 0) */
  MOE_EWORKSPACE = 3,    /* workspace missing or smaller than moe_workspace_size */
  MOE_EHIP = 4           /* a HIP launch reported an error */
} moe_status;

/*
 * How moe_forward runs a shape; the stage entry points follow the same plan,
 * so a caller of the stages runs exactly the kernels moe_forward runs.
 */
typedef struct moe_plan {
  int32_t swiglu_splits;        /* W1/W3 product: 0 = fused (writes H itself); s >= 1 =  */
                                /* fp32 partial sums over at most s K slices per matrix */
                                /* (the kernels take the count for the number of token  */
                                /* tiles that hold rows), which moe_swiglu_finish       */
                                /* completes                                            */
  int32_t down_splits;          /* K splits of the W2 product = slices of O             */
  size_t swiglu_scratch_bytes;  /* fp32 partial sums the W1/W3 product needs (0 if none) */
  int32_t streaming;            /* 1: weight-streaming (small batch) kernels, 0: tiled   */
  size_t down_scratch_bytes;    /* fp32 partial sums the W2 product needs (0 if none):  */
                                /* large batches run whole-K tiles for the complete     */
                                /* rounds of compute units and cut the tiles of the     */
                                /* last round into K pieces, summed into O by the same  */
                                /* call (down_splits is then 1)                         */
  int32_t swiglu_mixed;         /* 1: the tiled W1/W3 product picks its tile shape per  */
                                /* expert: 128 tokens x 512 columns for experts of at   */
                                /* most 128 rows, 256 x 256 for the others              */
  int32_t weights_nt;           /* 1: the tiled products read each weight tile once and */
                                /* copy it with the non-temporal cache policy (0: only  */
                                /* the copies of experts that fit one token tile are)   */
} moe_plan;

/* Index of each intermediate inside the workspace; see moe_workspace_layout. */
typedef enum {
  MOE_WS_TOPK_IDX = 0,     /* int32 [T, K]   expert of rank r of token t            */
  MOE_WS_TOPK_W = 1,       /* float [T, K]   gate weight of rank r                  */
  MOE_WS_OFFSETS = 2,      /* int32 [E + 1]  exclusive scan of pairs per expert     */
  MOE_WS_SORTED_TOKEN = 3, /* int32 [T*K]    token of each expert-sorted pair       */
  MOE_WS_POS = 4,          /* int32 [T, K]   sorted position of pair (t, r)         */
  MOE_WS_H = 5,            /* dtype [T*K, d_ff]  SwiGLU product, expert-sorted rows */
  MOE_WS_O = 6,            /* float [down_splits, T*K, d]  expert outputs (slices)  */
  MOE_WS_SCRATCH = 7,      /* max(swiglu_, down_scratch_bytes) of fp32 partial sums */
  MOE_WS_COUNT = 8
} moe_ws_item;

/* Human-readable name of a status. */
const char* moe_status_str(moe_status s);

/* Detail of the last error reported on the calling thread ("" if none). */
const char* moe_last_error(void);

/* MOE_ABI_VERSION of the loaded library. */
int32_t moe_abi_version(void);

/*
 * The plan moe_forward uses for this shape.  Errors: MOE_EINVAL for bad
 * sizes or a NULL `plan`, MOE_EUNSUPPORTED as moe_forward.
 */
moe_status moe_plan_for(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K, int32_t dtype,
                        moe_plan* plan);

/*
 * Bytes of workspace moe_forward needs for this shape (256-byte aligned
 * sub-buffers).  Errors: MOE_EINVAL for bad sizes or a NULL `bytes`.
 */
moe_status moe_workspace_size(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K,
                              int32_t dtype, size_t* bytes);

/*
 * Byte offset of every intermediate of moe_forward inside the workspace
 * (offsets[MOE_WS_COUNT]), so a caller can read the routing tables after a
 * call.  Same shape arguments and errors as moe_workspace_size.
 */
moe_status moe_workspace_layout(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K,
                                int32_t dtype, size_t* offsets);

/*
 * The whole layer: router + top-K + softmax, dispatch tables, W1/W3 SwiGLU
 * grouped GEMM (+ the split finish for small batches), W2 grouped GEMM,
 * gate-weighted combine -- five or six kernels, no host synchronisation.
 *   y_dtype     MOE_F32 or MOE_BF16: storage type of y.  A bf16 layer may
 *               write fp32 y (the pre-rounding sum); an fp32 layer writes fp32.
 *   accumulate  0: y = MoE(x).  1: y = round(y + MoE(x)) (residual add).
 *   workspace   device buffer of at least moe_workspace_size bytes,
 *               256-byte aligned.
 * x must not overlap y.  T == 0 returns MOE_OK and launches nothing.
 * Limits: 1 <= K <= E <= 64; T*K < 2^31; bf16 needs d % 64 == 0,
 * d_ff % 64 == 0 and 16-byte aligned x, W*, y (else MOE_EUNSUPPORTED).
 * Products whose sizes the streaming and tiled kernels cannot tile (they
 * take multiples of 128 or 256) run the general grouped matrix-core
 * kernels, which take multiples of 64.
 */
moe_status moe_forward(const void* x, const void* W_g, const void* const* W1,
                       const void* const* W3, const void* const* W2, int64_t T, int64_t d,
                       int64_t d_ff, int32_t E, int32_t K, int32_t dtype, void* y,
                       int32_t y_dtype, int32_t accumulate, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, serving
 * loops, harnesses that forbid hipMalloc): moe_forward with its workspace
 * taken from a static device array of MOE_NOALLOC_SCRATCH_BYTES (64 MiB)
 * inside the library instead of a caller's buffer.  Same arguments as
 * moe_forward minus the workspace; same results, bit for bit.
 *   - Each device the library runs on holds its own copy of the array until
 *     the process ends; its address is looked up on the first call made with
 *     that device current.  The call allocates nothing and calls no
 *     allocating routine.
 *   - A shape whose moe_workspace_size exceeds MOE_NOALLOC_SCRATCH_BYTES is
 *     refused with MOE_EWORKSPACE before anything is enqueued (at Mixtral
 *     shape, d = 4096, d_ff = 14336, E = 8, K = 2, that is above ~300 tokens).
 *   - Every call on one device uses that device's one array, and nothing in
 *     it needs clearing between calls (each kernel writes what a later one
 *     reads).  Calls that overlap in time on one device (other streams, other
 *     threads) race on it: order them, e.g. on one stream.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)

moe_status moe_forward_noalloc(const void* x, const void* W_g, const void* const* W1,
                               const void* const* W3, const void* const* W2, int64_t T,
                               int64_t d, int64_t d_ff, int32_t E, int32_t K, int32_t dtype,
                               void* y, int32_t y_dtype, int32_t accumulate, void* stream);

/* ---- the five steps, one kernel each, for callers that own the buffers ---- */

/*
 * Step 1+2 (section 2.1.4: bias-free linear router; section 2.1.1: TopK then
 * softmax): logits in fp32, the K largest by key (-logit, expert index) so
 * ties go to the lower index, gate weights = softmax over the K selected.
 *   topk_idx int32 [T, K], topk_w float [T, K] (rank order), logits float
 *   [T, E] or NULL.
 */
moe_status moe_router_topk(const void* x, const void* W_g, int64_t T, int64_t d, int32_t E,
                           int32_t K, int32_t dtype, int32_t* topk_idx, float* topk_w,
                           float* logits, void* stream);

/*
 * Steps 3-5 (section 3.1.2, code blocks B and C: for each expert the pairs it
 * processes): stable counting sort of the T*K pairs p = t*K + r by expert.
 *   offsets int32 [E+1]; sorted_token int32 [T*K] (token ascending inside a
 *   segment); pos int32 [T, K] = sorted position of pair (t, r).
 * Bit-exact and deterministic.  A pair whose expert index lies outside
 * [0, E) is dropped: it belongs to no segment (offsets[E] counts only the
 * kept pairs) and gets pos = -1, which moe_combine reads as "adds nothing".
 * moe_router_topk writes such an index (-1) only for a token whose logits
 * are not finite, which the finite-input contract excludes.
 */
moe_status moe_route_permute(const int32_t* topk_idx, int64_t T, int32_t E, int32_t K,
                             int32_t* offsets, int32_t* sorted_token, int32_t* pos,
                             void* stream);

/*
 * Routing statistics of one layer, from the router's table ("Mixtral of
 * Experts", xyznot.com, limitations: consecutive tokens share their
 * first-choice expert more often than random routing's 1/E; "杀疯了的开源专家
 * 模型 Mixtral 8x7B 论文公开啦！", redian.news, 实验: per layer, consecutive
 * tokens are often assigned the same expert):
 *   counts  int32 [E]: pairs (t, r) with topk_idx[t, r] = e (the load of e)
 *   repeats int32 [1]: tokens t in 1..T-1 whose first choice equals that of
 *           token t-1 (the first-choice repeat rate is repeats / (T - 1))
 * topk_idx int32 [T, K] in rank order, as moe_router_topk writes it; an index
 * outside [0, E) counts nowhere and never repeats.  Bit-exact integers.
 * T == 0 launches nothing and leaves the outputs as they are.
 */
moe_status moe_routing_stats(const int32_t* topk_idx, int64_t T, int32_t E, int32_t K,
                             int32_t* counts, int32_t* repeats, void* stream);

/*
 * Step 6 (code block D, first line): for every expert-sorted pair row r of
 * expert e, H[r] = round(SiLU(x[sorted_token[r]] W1[e]) * (x[...] W3[e])),
 * fp32 accumulation, one rounding to dtype.  H [T*K, d_ff] in dtype.
 * scratch: device buffer of plan.swiglu_scratch_bytes (may be NULL when that
 * is 0); MOE_EWORKSPACE if smaller.  With plan.swiglu_splits > 0 this call
 * leaves fp32 partial sums of both products over K slices in scratch and
 * moe_swiglu_finish writes H; with plan.swiglu_splits == 0 it writes H
 * itself.
 */
moe_status moe_expert_swiglu(const void* x, const void* const* W1, const void* const* W3,
                             int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K,
                             int32_t dtype, const int32_t* offsets, const int32_t* sorted_token,
                             void* H, void* scratch, size_t scratch_bytes, void* stream);

/*
 * Completes step 6 when plan.swiglu_splits > 0 (small batches): the fp32
 * partial sums that moe_expert_swiglu left in `scratch` are added in split
 * order and H = round(SiLU(a) * b) is written.  offsets: the same expert
 * offsets moe_expert_swiglu read (they fix how many K slices it wrote).
 * With plan.swiglu_splits == 0 H is already complete and this call does
 * nothing (MOE_OK).
 */
moe_status moe_swiglu_finish(const void* scratch, int64_t T, int64_t d, int64_t d_ff, int32_t E,
                             int32_t K, int32_t dtype, const int32_t* offsets, void* H,
                             void* stream);

/*
 * Step 7 (code block D, second line): O_s[r] = H[r, k-slice s] W2[e][k-slice s]
 * for every sorted row r of expert e and every split s < plan.down_splits,
 * fp32 accumulation.  O float [plan.down_splits, T*K, d]; the sum over s is
 * taken by moe_combine.  scratch: device buffer of plan.down_scratch_bytes
 * (may be NULL when that is 0; MOE_EWORKSPACE if smaller), which may be the
 * buffer given to moe_expert_swiglu: with down_scratch_bytes > 0 the call
 * keeps the K pieces of its last round of tiles there and adds them into O
 * (in piece order) before it returns.
 */
moe_status moe_expert_down(const void* H, const void* const* W2, int64_t T, int64_t d,
                           int64_t d_ff, int32_t E, int32_t K, int32_t dtype,
                           const int32_t* offsets, float* O, void* scratch, size_t scratch_bytes,
                           void* stream);

/*
 * Step 8 (section 2.1.1 sum; code block E, zero-initialised accumulator):
 * o_r = sum over s < o_splits of O[s][pos[t,r]] (in s order), then
 * s = w[t,0]*o_0 and s = fma(w[t,r], o_r, s) for r = 1..K-1, in fp32;
 * y[t] = round(s), or round(y[t] + s) when accumulate = 1.
 * pos[t,r] must be -1 or a row of O (< the rows of one slice); a pair with
 * pos = -1 (dropped by moe_route_permute) contributes o_r = 0.
 */
moe_status moe_combine(const float* O, int32_t o_splits, const float* topk_w, const int32_t* pos,
                       int64_t T, int64_t d, int32_t K, void* y, int32_t y_dtype,
                       int32_t accumulate, void* stream);

/*
 * Bytes of workspace moe_stack_forward needs: one layer's intermediates
 * (moe_workspace_layout) followed by the normalised block input [T, d].
 */
moe_status moe_stack_workspace_size(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K,
                                    int32_t dtype, size_t* bytes);

/*
 * A stack of L pre-norm blocks ("【DL輪読会】Mixtral of Experts" slides,
 * "Architecture – 全体": RMSNorm, then the mixture of experts, then the
 * residual add), in place on h [T, d]:
 *     for l = 0 .. L-1:   h = round(h + MoE_l(RMSNorm(h)))
 * with RMSNorm(h) = round(h / sqrt(mean(h^2) + eps)), unit gain.
 *   W_g   host array of L device pointers, block l's router [d, E]
 *   W1, W3, W2  host arrays of L*E device pointers; block l, expert e at
 *         index l*E + e (shapes as in moe_forward)
 *   stats NULL, or device int32 [L][E + 1]: block l's expert loads and then
 *         its first-choice repeats (what moe_routing_stats writes for it)
 *   workspace  moe_stack_workspace_size bytes, 256-byte aligned, not
 *         overlapping h
 * The result is that of moe_rmsnorm followed by moe_forward(accumulate = 1)
 * for each block in turn, bit for bit.  For small batches (the streaming
 * plan) one launch joins consecutive blocks: the previous block's combine
 * with the residual add, the RMSNorm and the next block's router.  Same
 * limits and errors as moe_forward; L = 0 or T = 0 is a no-op.
 */
moe_status moe_stack_forward(void* h, const void* const* W_g, const void* const* W1,
                             const void* const* W3, const void* const* W2, int32_t L, int64_t T,
                             int64_t d, int64_t d_ff, int32_t E, int32_t K, float eps,
                             int32_t dtype, int32_t* stats, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Pre-norm glue for a stack of blocks ("【DL輪読会】Mixtral of Experts"
 * slides, "Architecture – 全体": RMSNorm before the MoE block):
 * out[t] = round(h[t] / sqrt(mean(h[t]^2) + eps)), unit gain, fp32 math.
 * h and out are [T, d] in dtype and may not overlap.
 */
moe_status moe_rmsnorm(const void* h, void* out, int64_t T, int64_t d, float eps, int32_t dtype,
                       void* stream);

/* ------------------------------------------------------------------------
 * The attention sub-block in front of the MoE ("从Mistral 7B到MoE模型Mixtral
 * 8x7B的全面解析", aiqianji.com, sections 1.1 and 1.2.1-1.2.3):
 * grouped-query attention over a sliding window of W positions, with a
 * rolling-buffer key/value cache and chunked prefill.
 *
 *   position of query token t of sequence b:   p = pos0[b] + t
 *   keys it attends to:                         positions max(0, p-W+1) .. p
 *   key/value head of query head h:             h / (n_heads / n_kv_heads)
 *   weights:                                    softmax over those keys of
 *                                               q.k / sqrt(head_dim)
 *   output:                                     sum of weight * v
 *
 * Layout (row-major, bf16):
 *   q                  [B, T, n_heads, head_dim]
 *   k_new, v_new       [B, T, n_kv_heads, head_dim]   the chunk's keys/values
 *   k_cache, v_cache   [B, W, n_kv_heads, head_dim]   rolling buffer (section
 *                      1.2.2): position j lives in slot j mod W
 *   pos0               [B] int32, device: position of the chunk's first token
 *   out                [B, T, n_heads, head_dim], bf16 or fp32 (out_dtype)
 * Supported: head_dim = 128; n_heads / n_kv_heads in {1, 2, 4}; 1 <= T <= W
 * (the pages chunk prompts by the window size).  T = 0 or B = 0 is a no-op.
 *
 * Contract on the device data: a key at position j < pos0[b] is read from
 * the cache slot j mod W, so the cache must hold positions
 * max(0, pos0[b] - W + 1) .. pos0[b] - 1 (every earlier chunk appended with
 * swa_cache_append, in order); keys at positions >= pos0[b] come from
 * k_new / v_new.  Attention reads the cache as it stands; append the chunk
 * after the attention call (section 1.2.3).
 * ---------------------------------------------------------------------- */

/* Workspace bytes swa_attention needs for this shape (0 when the key range
 * is not split over workgroups). */
moe_status swa_workspace_size(int64_t B, int64_t T, int64_t W, int32_t n_heads,
                              int32_t n_kv_heads, int32_t head_dim, size_t* bytes);

/* One chunk of sliding-window grouped-query attention (sections 1.1, 1.2.1,
 * 1.2.3).  workspace: device buffer of swa_workspace_size bytes, 256-byte
 * aligned (may be NULL when that is 0).  All pointers 16-byte aligned; out
 * may not overlap q, k_new, v_new or the cache.  pos0[b] >= 0. */
moe_status swa_attention(const void* q, const void* k_new, const void* v_new,
                         const void* k_cache, const void* v_cache, const int32_t* pos0,
                         int64_t B, int64_t T, int64_t W, int32_t n_heads, int32_t n_kv_heads,
                         int32_t head_dim, void* out, int32_t out_dtype, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Rolling-buffer append (section 1.2.2): the keys and values of position
 * pos0[b] + t are written to slot (pos0[b] + t) mod W of sequence b's cache,
 * for the last min(T, W) tokens of the chunk (earlier ones would be
 * overwritten by later ones of the same chunk).  k_new, v_new
 * [B, T, n_kv_heads, head_dim]; k_cache, v_cache [B, W, n_kv_heads, head_dim];
 * bf16, 16-byte aligned; T >= 1 (any T; T = 0 is a no-op). */
moe_status swa_cache_append(const void* k_new, const void* v_new, const int32_t* pos0,
                            int64_t B, int64_t T, int64_t W, int32_t n_kv_heads, int32_t head_dim,
                            void* k_cache, void* v_cache, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
