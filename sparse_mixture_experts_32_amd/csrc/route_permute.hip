// Expert histogram, exclusive scan and stable permutation of the (token, rank)
// pairs -- the device-side form of the pages' expert-major dispatch
// ("从Mistral 7B到MoE模型Mixtral 8x7B的全面解析" (aiqianji.com) section 3.1.2 and
// code blocks B, C: for every expert, the list of pairs routed to it).
//
// One workgroup of 1024 threads computes, for pair p = t*K + r routed to
// expert e, the destination
//   offsets[e] + #{p' < p : idx[p'] = e},
// a stable counting sort: bit-exact and deterministic.  Two forms: from
// 2049 to 16384 pairs and up to 16 experts, the pairs are held in registers
// and counted per (round of 1024, wavefront) at once; otherwise they stream
// through in rounds (LDS atomics for the histogram, then one ranking pass
// per round).
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kPermuteThreads = 1024;
constexpr int kPermuteWaves = kPermuteThreads / 64;

// Streaming form (any P): rounds of 1024 pairs in pair order; inside a
// round a wavefront ranks its lanes per expert with one ballot per expert,
// waves are ordered by their index, and a per-expert running count carries
// across rounds.
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

// Held form (P <= R * 1024, E <= 16): every pair is loaded once into
// registers; the pairs of round j, wave w that go to expert x are counted
// with one ballot (cnt[x][j * 16 + w], in pair order along the second
// index); one wavefront per expert turns its row into an exclusive prefix
// (lane l sums R/4 consecutive entries, then a wave-wide scan); thread 0
// scans the expert totals.  Destination of a pair: offsets[x] + prefix of
// its (round, wave) + its rank among the lanes of its wave -- the same
// stable counting sort as the streaming form, with three barriers in all.
template <int R>
__global__ __launch_bounds__(kPermuteThreads) void route_permute_held_kernel(
    const int32_t* __restrict__ topk_idx, int P, int E, int K, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ pos) {
  constexpr int kMaxE = 16;
  constexpr int kCols = R * kPermuteWaves;          // (round, wave) slots per expert
  static_assert(kCols % 64 == 0 || kCols < 64, "whole lanes per slot group");
  __shared__ int cnt[kMaxE][kCols];
  __shared__ int total[kMaxE];
  __shared__ int offs[kMaxE + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint64_t lower_lanes = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  int held[R], rank[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int p = j * kPermuteThreads + tid;
    const int e = p < P ? topk_idx[p] : -1;
    held[j] = (e >= 0 && e < E) ? e : -1;
  }
#pragma unroll
  for (int j = 0; j < R; ++j) {
    rank[j] = 0;
    for (int x = 0; x < E; ++x) {
      const uint64_t m = __ballot(held[j] == x);
      if (lane == 0) cnt[x][j * kPermuteWaves + wave] = __popcll(m);
      if (held[j] == x) rank[j] = __popcll(m & lower_lanes);
    }
  }
  __syncthreads();
  // exclusive prefix of each expert's row, one wavefront per expert
  if (wave < E) {
    constexpr int kPer = kCols >= 64 ? kCols / 64 : 1;   // entries per lane
    int vals[kPer];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = lane * kPer + i;
      vals[i] = c < kCols ? cnt[wave][c] : 0;
      sum += vals[i];
    }
    int incl = sum;                                       // inclusive scan over lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = lane * kPer + i;
      if (c < kCols) cnt[wave][c] = run;
      run += vals[i];
    }
    if (lane == 63) total[wave] = incl;
  }
  __syncthreads();
  if (tid == 0) {
    offs[0] = 0;
    for (int e = 0; e < E; ++e) offs[e + 1] = offs[e] + total[e];
  }
  __syncthreads();
  if (tid <= E) offsets[tid] = offs[tid];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int p = j * kPermuteThreads + tid;
    const int e = held[j];
    if (e >= 0) {
      const int dest = offs[e] + cnt[e][j * kPermuteWaves + wave] + rank[j];
      sorted_token[dest] = p / K;
      pos[p] = dest;
    } else if (p < P) {
      pos[p] = -1;  // out-of-range expert index: the pair is dropped
    }
  }
}

// Routing statistics of one layer: pairs per expert and first-choice repeats
// between consecutive tokens ("Mixtral of Experts" (xyznot.com),
// limitations: consecutive tokens keep their first-choice expert more often
// than the 1/E of random routing).  One workgroup; LDS integer atomics and a
// wave sum of integers, so the counts do not depend on the order of updates.
__global__ __launch_bounds__(kPermuteThreads) void routing_stats_kernel(
    const int32_t* __restrict__ topk_idx, int T, int E, int K, int32_t* __restrict__ counts,
    int32_t* __restrict__ repeats) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int rep;
  const int tid = threadIdx.x;
  if (tid < kMaxExperts) cnt[tid] = 0;
  if (tid == 0) rep = 0;
  __syncthreads();
  const int64_t P = (int64_t)T * K;
  for (int64_t p = tid; p < P; p += kPermuteThreads) {
    const int e = topk_idx[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  int mine = 0;
  for (int64_t t = 1 + tid; t < T; t += kPermuteThreads) {
    const int a = topk_idx[(t - 1) * K], b = topk_idx[t * K];
    mine += (b == a && b >= 0 && b < E) ? 1 : 0;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mine += __shfl_xor(mine, m, 64);
  if ((tid & 63) == 0 && mine) atomicAdd(&rep, mine);
  __syncthreads();
  if (tid < E) counts[tid] = cnt[tid];
  if (tid == 0) repeats[0] = rep;
}

}  // namespace

hipError_t launch_routing_stats(const int32_t* topk_idx, int T, int E, int K, int32_t* counts,
                                int32_t* repeats, hipStream_t stream) {
  hipLaunchKernelGGL(routing_stats_kernel, dim3(1), dim3(kPermuteThreads), 0, stream, topk_idx, T,
                     E, K, counts, repeats);
  return hipGetLastError();
}

hipError_t launch_route_permute(const int32_t* topk_idx, int T, int E, int K, int32_t* offsets,
                                int32_t* sorted_token, int32_t* pos, hipStream_t stream) {
  const int P = T * K;
  const int rounds = (P + kPermuteThreads - 1) / kPermuteThreads;
#define MOE_PERMUTE_HELD(R)                                                                 \
  hipLaunchKernelGGL(route_permute_held_kernel<R>, dim3(1), dim3(kPermuteThreads), 0, stream, \
                     topk_idx, P, E, K, offsets, sorted_token, pos)
  // one or two rounds stream faster than the held form's fixed four
  const bool held = E <= 16 && rounds >= 3 && rounds <= 16;
  if (held && rounds <= 4) MOE_PERMUTE_HELD(4);
  else if (held && rounds <= 8) MOE_PERMUTE_HELD(8);
  else if (held) MOE_PERMUTE_HELD(16);
  else
    hipLaunchKernelGGL(route_permute_kernel, dim3(1), dim3(kPermuteThreads), 0, stream, topk_idx,
                       P, E, K, offsets, sorted_token, pos);
#undef MOE_PERMUTE_HELD
  return hipGetLastError();
}

}  // namespace moe
