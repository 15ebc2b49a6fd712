// Expert histogram, exclusive scan and stable permutation of the (token, rank)
// pairs -- the device-side form of the pages' expert-major dispatch
// ("从Mistral 7B到MoE模型Mixtral 8x7B的全面解析" (aiqianji.com) section 3.1.2 and
// code blocks B, C: for every expert, the list of pairs routed to it).
//
// One workgroup of 1024 threads.  Pass 1 counts pairs per expert with LDS
// integer atomics (the counts do not depend on the order).  Thread 0 scans
// the E counts.  Pass 2 walks the pairs in rounds of 1024 in pair order
// p = t*K + r; inside a round a wavefront ranks its lanes per expert with one
// ballot per expert, waves are ordered by their index, and a per-expert
// running count carries across rounds.  So the destination of pair p is
//   offsets[e] + #{p' < p : idx[p'] = e},
// a stable counting sort: bit-exact and deterministic.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kPermuteThreads = 1024;
constexpr int kPermuteWaves = kPermuteThreads / 64;

__global__ __launch_bounds__(kPermuteThreads) void route_permute_kernel(
    const int32_t* __restrict__ topk_idx, int P, int E, int K, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ pos) {
  __shared__ int counts[kMaxExperts];
  __shared__ int offs[kMaxExperts + 1];
  __shared__ int running[kMaxExperts];
  __shared__ int wave_cnt[kPermuteWaves][kMaxExperts];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid < kMaxExperts) {
    counts[tid] = 0;
    running[tid] = 0;
  }
  __syncthreads();

  for (int p = tid; p < P; p += kPermuteThreads) {
    const int e = topk_idx[p];
    if (e >= 0 && e < E) atomicAdd(&counts[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    offs[0] = 0;
    for (int e = 0; e < E; ++e) offs[e + 1] = offs[e] + counts[e];
  }
  __syncthreads();
  if (tid <= E) offsets[tid] = offs[tid];

  const uint64_t lower_lanes = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < P; base += kPermuteThreads) {
    const int p = base + tid;
    int e = (p < P) ? topk_idx[p] : -1;
    if (e >= E) e = -1;
    int my_rank = 0;
    for (int x = 0; x < E; ++x) {
      const uint64_t m = __ballot(e == x);
      if (lane == 0) wave_cnt[wave][x] = __popcll(m);
      if (e == x) my_rank = __popcll(m & lower_lanes);
    }
    __syncthreads();
    if (e >= 0) {
      int before = running[e];
      for (int w = 0; w < wave; ++w) before += wave_cnt[w][e];
      const int dest = offs[e] + before + my_rank;
      sorted_token[dest] = p / K;
      pos[p] = dest;
    } else if (p < P) {
      pos[p] = -1;  // out-of-range expert index: the pair is dropped
    }
    __syncthreads();
    if (tid < E) {
      int s = 0;
      for (int w = 0; w < kPermuteWaves; ++w) s += wave_cnt[w][tid];
      running[tid] += s;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_route_permute(const int32_t* topk_idx, int T, int E, int K, int32_t* offsets,
                                int32_t* sorted_token, int32_t* pos, hipStream_t stream) {
  hipLaunchKernelGGL(route_permute_kernel, dim3(1), dim3(kPermuteThreads), 0, stream, topk_idx,
                     T * K, E, K, offsets, sorted_token, pos);
  return hipGetLastError();
}

}  // namespace moe
