// Gate-weighted combine of the expert outputs, and the RMSNorm that joins
// stacked blocks.
//
// Combine: "从Mistral 7B到MoE模型Mixtral 8x7B的全面解析" (aiqianji.com) section
// 2.1.1 (y = sum_i G(x)_i E_i(x)) and section 3.2.5 code block E (the output
// starts from zero and each routed expert output is added).  Here each token
// gathers its K expert rows O[pos[t, r]] (each the sum of the K-split slices
// of the W2 product, added in slice order) and sums them in rank order in fp32
// with one fixed expression, s = w0*O0, then s = fma(w_r, O_r, s); y is rounded
// once (after adding the residual in accumulate mode).  A pair with pos < 0
// (dropped by the dispatch) adds nothing.  No atomics: bitwise reproducible.
//
// RMSNorm: "【DL輪読会】Mixtral of Experts" (docswell slides), slide
// "Architecture – 全体" (RMSNorm ahead of the mixture of experts); unit gain.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

template <typename YT>
__device__ __forceinline__ float load_y(const YT* y, int64_t i);
template <>
__device__ __forceinline__ float load_y<float>(const float* y, int64_t i) { return y[i]; }
template <>
__device__ __forceinline__ float load_y<bf16_t>(const bf16_t* y, int64_t i) {
  return bf16_to_f32(y[i]);
}
__device__ __forceinline__ void store_y(float* y, int64_t i, float v) { y[i] = v; }
__device__ __forceinline__ void store_y(bf16_t* y, int64_t i, float v) { y[i] = f32_to_bf16(v); }

// Sum of the o_splits slices of O at features c..c+3 of sorted row p, in
// slice order.  A pair the dispatch dropped (pos = -1: its expert index was
// outside [0, E)) has no row and contributes zeros.
__device__ __forceinline__ float4 load_o4(const float* O, int splits, int64_t slice, int32_t p,
                                          int d, int c) {
  if (p < 0) return make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  const int64_t i = (int64_t)p * d + c;
  float4 v = *reinterpret_cast<const float4*>(O + i);
  for (int s = 1; s < splits; ++s) {
    const float4 u = *reinterpret_cast<const float4*>(O + s * slice + i);
    v.x += u.x;
    v.y += u.y;
    v.z += u.z;
    v.w += u.w;
  }
  return v;
}

__device__ __forceinline__ float load_o1(const float* O, int splits, int64_t slice, int32_t p,
                                        int d, int c) {
  if (p < 0) return 0.0f;
  const int64_t i = (int64_t)p * d + c;
  float v = O[i];
  for (int s = 1; s < splits; ++s) v += O[s * slice + i];
  return v;
}

// One thread per 4 consecutive features of one token (d % 4 == 0).
template <typename YT, bool ACC>
__global__ __launch_bounds__(256) void combine_vec4_kernel(const float* __restrict__ O, int splits,
                                                           int64_t slice,
                                                           const float* __restrict__ topk_w,
                                                           const int32_t* __restrict__ pos, int T,
                                                           int d, int K, YT* __restrict__ y) {
  const int64_t groups = (int64_t)T * (d / 4);
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(g / (d / 4));
    const int c = (int)(g % (d / 4)) * 4;
    const float* wt = topk_w + (int64_t)t * K;
    const int32_t* pt = pos + (int64_t)t * K;
    const float4 o0 = load_o4(O, splits, slice, pt[0], d, c);
    const float w0 = wt[0];
    float s0 = w0 * o0.x, s1 = w0 * o0.y, s2 = w0 * o0.z, s3 = w0 * o0.w;
    for (int r = 1; r < K; ++r) {
      const float4 o = load_o4(O, splits, slice, pt[r], d, c);
      const float w = wt[r];
      s0 = fmaf(w, o.x, s0);
      s1 = fmaf(w, o.y, s1);
      s2 = fmaf(w, o.z, s2);
      s3 = fmaf(w, o.w, s3);
    }
    const int64_t base = (int64_t)t * d + c;
    if (ACC) {
      s0 = load_y(y, base + 0) + s0;
      s1 = load_y(y, base + 1) + s1;
      s2 = load_y(y, base + 2) + s2;
      s3 = load_y(y, base + 3) + s3;
    }
    if constexpr (sizeof(YT) == 4) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + base) = make_float4(s0, s1, s2, s3);
    } else {
      uint2 v;
      v.x = pack_bf16x2(s0, s1);
      v.y = pack_bf16x2(s2, s3);
      *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(y) + base) = v;
    }
  }
}

// Scalar fallback for any d.
template <typename YT, bool ACC>
__global__ __launch_bounds__(256) void combine_scalar_kernel(const float* __restrict__ O,
                                                             int splits, int64_t slice,
                                                             const float* __restrict__ topk_w,
                                                             const int32_t* __restrict__ pos,
                                                             int T, int d, int K,
                                                             YT* __restrict__ y) {
  const int64_t n = (int64_t)T * d;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(g / d);
    const int c = (int)(g % d);
    const float* wt = topk_w + (int64_t)t * K;
    const int32_t* pt = pos + (int64_t)t * K;
    float s = wt[0] * load_o1(O, splits, slice, pt[0], d, c);
    for (int r = 1; r < K; ++r) s = fmaf(wt[r], load_o1(O, splits, slice, pt[r], d, c), s);
    if (ACC) s = load_y(y, g) + s;
    store_y(y, g, s);
  }
}

template <typename YT, bool ACC>
hipError_t launch_combine_t(const float* O, int splits, int64_t slice, const float* w,
                            const int32_t* pos, int T, int d, int K, void* y, hipStream_t stream) {
  const int threads = 256;
  if (d % 4 == 0) {
    const int64_t groups = (int64_t)T * (d / 4);
    const int blocks = (int)std::min<int64_t>((groups + threads - 1) / threads, 4096);
    hipLaunchKernelGGL((combine_vec4_kernel<YT, ACC>), dim3(blocks), dim3(threads), 0, stream, O,
                       splits, slice, w, pos, T, d, K, static_cast<YT*>(y));
  } else {
    const int64_t n = (int64_t)T * d;
    const int blocks = (int)std::min<int64_t>((n + threads - 1) / threads, 4096);
    hipLaunchKernelGGL((combine_scalar_kernel<YT, ACC>), dim3(blocks), dim3(threads), 0, stream,
                       O, splits, slice, w, pos, T, d, K, static_cast<YT*>(y));
  }
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* __restrict__ h, T* __restrict__ out,
                                                      int d, float eps) {
  __shared__ float part[256];
  const int64_t row = blockIdx.x;
  const T* hr = h + row * d;
  float s = 0.0f;
  for (int c = threadIdx.x; c < d; c += 256) {
    const float v = load_y(hr, c);
    s = fmaf(v, v, s);
  }
  part[threadIdx.x] = s;
  __syncthreads();
  for (int m = 128; m >= 1; m >>= 1) {
    if (threadIdx.x < m) part[threadIdx.x] += part[threadIdx.x + m];
    __syncthreads();
  }
  const float inv = 1.0f / sqrtf(part[0] / (float)d + eps);
  T* orow = out + row * d;
  for (int c = threadIdx.x; c < d; c += 256) store_y(orow, c, load_y(hr, c) * inv);
}

}  // namespace

hipError_t launch_combine(const float* O, int o_splits, int64_t slice, const float* topk_w,
                          const int32_t* pos, int T, int d, int K, void* y, int y_dtype,
                          int accumulate, hipStream_t stream) {
  if (y_dtype == kBF16)
    return accumulate
               ? launch_combine_t<bf16_t, true>(O, o_splits, slice, topk_w, pos, T, d, K, y, stream)
               : launch_combine_t<bf16_t, false>(O, o_splits, slice, topk_w, pos, T, d, K, y,
                                                 stream);
  return accumulate
             ? launch_combine_t<float, true>(O, o_splits, slice, topk_w, pos, T, d, K, y, stream)
             : launch_combine_t<float, false>(O, o_splits, slice, topk_w, pos, T, d, K, y, stream);
}

hipError_t launch_rmsnorm(const void* h, void* out, int T, int d, float eps, int dtype,
                          hipStream_t stream) {
  if (dtype == kBF16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, dim3(T), dim3(256), 0, stream,
                       static_cast<const bf16_t*>(h), static_cast<bf16_t*>(out), d, eps);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(T), dim3(256), 0, stream,
                       static_cast<const float*>(h), static_cast<float*>(out), d, eps);
  return hipGetLastError();
}

}  // namespace moe
