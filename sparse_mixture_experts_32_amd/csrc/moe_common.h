// Internal helpers shared by the HIP kernels of the MoE layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 64;

// bfloat16 is carried as its raw 16-bit pattern.
typedef uint16_t bf16_t;

// Matrix-core operand: 8 bf16 values in 4 VGPRs.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even.  Inputs are finite by
// contract; a NaN is kept a quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Pack two floats as bf16 (lo, hi) in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// SiLU(z) = z * sigmoid(z) = z / (1 + e^-z), in float32.
__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// Expert pointer tables travel by value in the kernel arguments.
struct ExpertPtrs {
  const void* p[kMaxExperts];
};

// Token tiles of bt rows that hold rows: sum over experts of ceil(count_e / bt).
__device__ __forceinline__ int busy_tiles(const int32_t* __restrict__ offsets, int E, int bt) {
  int n = 0;
  for (int e = 0; e < E; ++e) n += (offsets[e + 1] - offsets[e] + bt - 1) / bt;
  return n;
}

// The dispatch tables of a small batch (P <= 64 pairs, E <= 64 experts),
// built by the calling wavefront: the stable counting sort of the dispatch
// kernel (pair p = t K + r routed to expert e goes to offsets[e] + #{p' < p :
// idx[p'] = e}); a pair whose index lies outside [0, E) is dropped, pos = -1.
// off[E + 1], tok[P] (token of each sorted position) and pos[P] may be LDS
// or global memory.
__device__ __forceinline__ void small_route(const int32_t* __restrict__ topk_idx, int P, int K,
                                            int E, int32_t* off, int32_t* tok, int32_t* pos) {
  const int lane = threadIdx.x & 63;
  int e = lane < P ? topk_idx[lane] : -1;
  if (e >= E) e = -1;
  const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int dest = -1, total = 0;
  for (int x = 0; x < E; ++x) {
    const uint64_t m = __ballot(e == x);
    if (e == x) dest = total + __popcll(m & lower);
    if (lane == 0) off[x] = total;
    total += __popcll(m);
  }
  if (lane == 0) off[E] = total;
  if (dest >= 0) tok[dest] = lane / K;
  if (lane < P) pos[lane] = dest;
}

// Locate the token tile `tile` among the experts' segments: expert e owns
// ceil(count_e / bt) tiles, experts in index order.  Returns false when the
// tile index is past the last real tile.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int bt,
                                          int tile, int& expert, int& row_begin, int& row_end) {
  int acc = 0;
  for (int e = 0; e < E; ++e) {
    const int b = offsets[e];
    const int n = offsets[e + 1] - b;
    const int tiles = (n + bt - 1) / bt;
    if (tile < acc + tiles) {
      expert = e;
      row_begin = b + (tile - acc) * bt;
      row_end = offsets[e + 1];
      return true;
    }
    acc += tiles;
  }
  return false;
}

}  // namespace moe
