// Router GEMV + top-K + softmax over the selected logits, one wavefront per
// token ("从Mistral 7B到MoE模型Mixtral 8x7B的全面解析" (aiqianji.com) section
// 2.1.4: the router is a bias-free linear layer to num_experts scores; section
// 2.1.1: G(x) = Softmax(TopK(x W_g)), TopK masks every logit outside the K
// largest to -inf).
//
// Each lane accumulates a strided slice of the dot products in fp32, a
// butterfly over the 64 lanes finishes them (fixed order: deterministic).
// Selection takes K rounds of a wave-wide arg-max with key (-logit, index),
// so equal logits go to the lower expert index.  The softmax over the K
// selected logits is exp(l_r - l_0) / sum_s exp(l_s - l_0).
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

template <typename T>
__device__ __forceinline__ float load_f(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_f<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f<bf16_t>(const bf16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// true if (va, ia) ranks before (vb, ib): larger value, then lower index.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return (ia >= 0) && (ib < 0 || va > vb || (va == vb && ia < ib));
}

template <typename T>
__global__ __launch_bounds__(256) void router_topk_kernel(const T* __restrict__ x,
                                                          const T* __restrict__ Wg, int T_,
                                                          int d, int E, int K,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w,
                                                          float* __restrict__ logits_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T_) return;
  const T* xr = x + static_cast<int64_t>(t) * d;

  float my_logit = 0.0f;  // lane e keeps logit e (e < E)
  for (int e0 = 0; e0 < E; e0 += 8) {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    for (int k = lane; k < d; k += 64) {
      const float xv = load_f(xr, k);
      const T* wrow = Wg + static_cast<int64_t>(k) * E + e0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (e0 + j < E) acc[j] = fmaf(xv, load_f(wrow, j), acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float s = wave_sum(acc[j]);
      if (lane == e0 + j) my_logit = s;
    }
  }
  if (logits_out && lane < E) logits_out[static_cast<int64_t>(t) * E + lane] = my_logit;

  // K rounds of wave arg-max; lane 0 writes rank r as soon as it is known
  // (the weight first unnormalised, divided by the total afterwards).
  bool taken = false;
  float first = 0.0f, denom = 0.0f;
  int32_t* out_idx = topk_idx + static_cast<int64_t>(t) * K;
  float* out_w = topk_w + static_cast<int64_t>(t) * K;
  for (int r = 0; r < K; ++r) {
    float v = my_logit;
    int i = (lane < E && !taken) ? lane : -1;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(v, m, 64);
      const int oi = __shfl_xor(i, m, 64);
      if (ranks_before(ov, oi, v, i)) {
        v = ov;
        i = oi;
      }
    }
    if (lane == i) taken = true;
    if (r == 0) first = v;
    const float ex = expf(v - first);
    denom += ex;
    if (lane == 0) {
      out_idx[r] = i;
      out_w[r] = ex;
    }
  }
  if (lane == 0)
    for (int r = 0; r < K; ++r) out_w[r] = out_w[r] / denom;
}

}  // namespace

hipError_t launch_router_topk(const void* x, const void* Wg, int T, int d, int E, int K,
                              int dtype, int32_t* topk_idx, float* topk_w, float* logits,
                              hipStream_t stream) {
  const int tokens_per_block = 4;
  dim3 grid((T + tokens_per_block - 1) / tokens_per_block);
  dim3 block(64 * tokens_per_block);
  if (dtype == kBF16)
    hipLaunchKernelGGL(router_topk_kernel<bf16_t>, grid, block, 0, stream,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(Wg), T, d, E, K,
                       topk_idx, topk_w, logits);
  else
    hipLaunchKernelGGL(router_topk_kernel<float>, grid, block, 0, stream,
                       static_cast<const float*>(x), static_cast<const float*>(Wg), T, d, E, K,
                       topk_idx, topk_w, logits);
  return hipGetLastError();
}

}  // namespace moe
