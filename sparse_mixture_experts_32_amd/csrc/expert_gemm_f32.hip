// Grouped float32 GEMMs of the SwiGLU experts: the fp32 storage type, used by
// small layers.  Same semantics as the bf16 kernels ("从Mistral 7B到MoE模型
// Mixtral 8x7B的全面解析" (aiqianji.com) code block D), plain vector FMA with
// 16x16 LDS tiles; H stays float32 (no rounding).
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kTile = 16;

template <bool DUAL>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ offsets, ExpertPtrs Wa, ExpertPtrs Wb, float* __restrict__ out,
    int Kdim, int N, int E, int max_tiles) {
  __shared__ float sA[kTile][kTile + 1];
  __shared__ float sW[2][kTile][kTile + 1];

  const int ttile = blockIdx.x % max_tiles;
  const int ftile = blockIdx.x / max_tiles;
  int e, row_begin, row_end;
  if (!find_tile(offsets, E, kTile, ttile, e, row_begin, row_end)) return;
  const int tx = threadIdx.x % kTile;  // feature within tile / k when loading A
  const int ty = threadIdx.x / kTile;  // row within tile / k when loading W
  const int r = row_begin + ty;
  const int f = ftile * kTile + tx;
  const bool row_ok = r < row_end;
  const int64_t src_row = row_ok ? (gather ? gather[r] : r) : 0;
  const float* W0 = static_cast<const float*>(Wa.p[e]);
  const float* W1 = static_cast<const float*>(DUAL ? Wb.p[e] : Wa.p[e]);

  float a = 0.0f, b = 0.0f;
  for (int k0 = 0; k0 < Kdim; k0 += kTile) {
    const int ka = k0 + tx;
    sA[ty][tx] = (row_ok && ka < Kdim) ? A[src_row * Kdim + ka] : 0.0f;
    const int kw = k0 + ty;
    const bool w_ok = kw < Kdim && f < N;
    sW[0][ty][tx] = w_ok ? W0[(int64_t)kw * N + f] : 0.0f;
    if (DUAL) sW[1][ty][tx] = w_ok ? W1[(int64_t)kw * N + f] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kTile; ++k) {
      a = fmaf(sA[ty][k], sW[0][k][tx], a);
      if (DUAL) b = fmaf(sA[ty][k], sW[1][k][tx], b);
    }
    __syncthreads();
  }
  if (row_ok && f < N) out[(int64_t)r * N + f] = DUAL ? silu_f32(a) * b : a;
}

int max_tiles_for(int P, int E) { return (int)(((int64_t)P + (int64_t)E * (kTile - 1)) / kTile); }

}  // namespace

hipError_t launch_expert_swiglu_f32(const void* x, const int32_t* sorted_token,
                                    const ExpertPtrs& W1, const ExpertPtrs& W3,
                                    const int32_t* offsets, int P, int d, int d_ff, int E,
                                    void* H, hipStream_t stream) {
  const int mt = max_tiles_for(P, E);
  if (mt <= 0) return hipSuccess;
  const int tf = (d_ff + kTile - 1) / kTile;
  hipLaunchKernelGGL(grouped_gemm_f32_kernel<true>, dim3(mt * tf), dim3(256), 0, stream,
                     static_cast<const float*>(x), sorted_token, offsets, W1, W3,
                     static_cast<float*>(H), d, d_ff, E, mt);
  return hipGetLastError();
}

hipError_t launch_expert_down_f32(const void* H, const ExpertPtrs& W2, const int32_t* offsets,
                                  int P, int d, int d_ff, int E, float* O, hipStream_t stream) {
  const int mt = max_tiles_for(P, E);
  if (mt <= 0) return hipSuccess;
  const int tf = (d + kTile - 1) / kTile;
  hipLaunchKernelGGL(grouped_gemm_f32_kernel<false>, dim3(mt * tf), dim3(256), 0, stream,
                     static_cast<const float*>(H), nullptr, offsets, W2, W2, O, d_ff, d, E, mt);
  return hipGetLastError();
}

}  // namespace moe
