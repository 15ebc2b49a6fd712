// Router GEMV + top-K + softmax over the selected logits
// ("从Mistral 7B到MoE模型Mixtral 8x7B的全面解析" (aiqianji.com) section 2.1.4:
// the router is a bias-free linear layer to num_experts scores; section 2.1.1:
// G(x) = Softmax(TopK(x W_g)), TopK masks every logit outside the K largest
// to -inf, so the softmax runs over the K selected logits only).
//
// TPT threads per token (64 or 256).  Each thread accumulates fp32 partial
// logits over a strided set of 8-wide k chunks; the 8 partials of a block
// of experts are combined by one transposed butterfly inside each wavefront
// and then across the token's wavefronts in wave order (fixed order:
// deterministic).  In the vector path (bf16,
// E % 8 == 0, d % 8 == 0) a chunk is one 16-byte load of x and eight 16-byte
// loads of the matching W_g rows.  Selection takes K rounds of a wave-wide
// arg-max with key (-logit, index), so equal logits go to the lower index.
// The gate weights are exp(l_r - l_0) / sum_s exp(l_s - l_0) over the K
// selected, in rank order.
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

// Sum 8 per-lane partials over the wavefront in 10 exchanges: at each of
// the strides 32, 16, 8 a lane keeps half of its values and adds its
// partner's copy of them, so afterwards lane l holds value
// e(l) = 4 bit5(l) + 2 bit4(l) + bit3(l) = l / 8 summed over its stride
// partners, and strides 4, 2, 1 finish the sum.  Every lane of a group of
// 8 ends with the same bits (each addition is commutative).
__device__ __forceinline__ float wave_sum8(const float (&a)[8], int lane) {
  const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
  float v4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    v4[j] = (b5 ? a[j + 4] : a[j]) + __shfl_xor(b5 ? a[j] : a[j + 4], 32, 64);
  float v2[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    v2[j] = (b4 ? v4[j + 2] : v4[j]) + __shfl_xor(b4 ? v4[j] : v4[j + 2], 16, 64);
  float v = (b3 ? v2[1] : v2[0]) + __shfl_xor(b3 ? v2[0] : v2[1], 8, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 1, 64);
  return v;
}

// true if (va, ia) ranks before (vb, ib): larger value, then lower index.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return (ia >= 0) && (ib < 0 || va > vb || (va == vb && ia < ib));
}

__device__ __forceinline__ void bf16x8_to_f32(const uint4& v, float f[8]) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16);
  f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16);
  f[7] = __uint_as_float(v.w & 0xffff0000u);
}

// Partial logits of experts e0 .. e0+7 of one token, vector path (bf16,
// E % 8 == 0, d % 8 == 0): the thread `sub` of the token's TPT threads takes
// the 8-wide chunks k0 = 8 sub, 8 sub + 8 TPT, ...; a chunk is one 16-byte
// load of x and eight 16-byte loads of the matching W_g rows.  xr may point
// to global memory or to LDS.
template <int TPT>
__device__ __forceinline__ void vec_partials(const bf16_t* xr, const bf16_t* __restrict__ Wg,
                                             int d, int E, int e0, int sub, float (&acc)[8]) {
#pragma unroll 4
  for (int k0 = sub * 8; k0 < d; k0 += TPT * 8) {
    float xv[8];
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(xr + k0), xv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float wv[8];
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(Wg + (int64_t)(k0 + i) * E + e0), wv);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(xv[i], wv[j], acc[j]);
    }
  }
}

// Top-K of one token whose logit e sits in lane e of the calling wavefront
// (lanes >= E hold nothing): K rounds of a wave arg-max with key
// (-logit, index); lane 0 writes rank r as soon as it is known (the weight
// first unnormalised, divided by the total afterwards).
__device__ __forceinline__ void select_topk(float my_logit, int lane, int E, int K,
                                            int32_t* out_idx, float* out_w) {
  bool taken = false;
  float first = 0.0f, denom = 0.0f;
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

template <typename T, int TPT, bool VEC>
__global__ __launch_bounds__(256) void router_topk_kernel(const T* __restrict__ x,
                                                          const T* __restrict__ Wg, int T_,
                                                          int d, int E, int K,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w,
                                                          float* __restrict__ logits_out) {
  constexpr int kWavesPerTok = TPT / 64;
  __shared__ float wave_part[256 / 64][kMaxExperts];
  __shared__ float logit_sh[256 / TPT][kMaxExperts];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tok_local = threadIdx.x / TPT;
  const int sub = threadIdx.x % TPT;          // thread index inside the token's group
  const int wave_in_tok = sub >> 6;
  const int t = blockIdx.x * (256 / TPT) + tok_local;
  const bool live = t < T_;
  const T* xr = x + static_cast<int64_t>(live ? t : 0) * d;

  for (int e0 = 0; e0 < E; e0 += 8) {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    if (live) {
      if constexpr (VEC) {
        vec_partials<TPT>(reinterpret_cast<const bf16_t*>(xr), reinterpret_cast<const bf16_t*>(Wg),
                          d, E, e0, sub, acc);
      } else {
        for (int k = sub; k < d; k += TPT) {
          const float xv = load_f(xr, k);
          const T* wrow = Wg + static_cast<int64_t>(k) * E + e0;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (e0 + j < E) acc[j] = fmaf(xv, load_f(wrow, j), acc[j]);
        }
      }
    }
    const float s = wave_sum8(acc, lane);              // value lane / 8
    if ((lane & 7) == 0 && e0 + (lane >> 3) < E) wave_part[wave][e0 + (lane >> 3)] = s;
  }
  __syncthreads();
  // Combine the token's waves in order; lane e of the token's first wave keeps logit e.
  if (wave_in_tok == 0 && lane < E) {
    float v = 0.0f;
    for (int w = 0; w < kWavesPerTok; ++w) v += wave_part[wave + w][lane];
    logit_sh[tok_local][lane] = v;
  }
  __syncthreads();
  if (!live || wave_in_tok != 0) return;
  const float my_logit = lane < E ? logit_sh[tok_local][lane] : 0.0f;
  if (logits_out && lane < E) logits_out[static_cast<int64_t>(t) * E + lane] = my_logit;

  select_topk(my_logit, lane, E, K, topk_idx + static_cast<int64_t>(t) * K,
              topk_w + static_cast<int64_t>(t) * K);
}

// Many tokens, 8 experts, bf16: a workgroup takes 4 tokens, so every
// 16-byte piece of W_g it loads serves 4 tokens (a token per wavefront would
// read all of W_g once per token), and its 4 wavefronts split the features:
// lane l of wave w accumulates the 8-wide chunks 64 w + l, 64 w + l + 256,
// ... of each token.  (One wavefront per 4 tokens left one wave per SIMD
// at T = 4096 and ran 1.4x longer: its load round trips were exposed.)  After
// the transposed butterfly lane l holds expert l / 8 of the wave's partial;
// the 4 partials are added in wave order through LDS.  Top-K then runs for
// the 4 tokens at once in wave 0: lane 16 n + e (e < 8) holds expert e of
// token n, and K rounds of an arg-max over each 16-lane group pick the
// experts with key (-logit, index), as in the general kernel.
constexpr int kRouterTokPerGroup = 4;

__global__ __launch_bounds__(256) void router_e8_kernel(const bf16_t* __restrict__ x,
                                                        const bf16_t* __restrict__ Wg, int T_,
                                                        int d, int K,
                                                        int32_t* __restrict__ topk_idx,
                                                        float* __restrict__ topk_w,
                                                        float* __restrict__ logits_out) {
  constexpr int NT = kRouterTokPerGroup;
  __shared__ float part[4][NT][8];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * NT;                       // first token of this workgroup
  if (t0 >= T_) return;                                 // workgroup-uniform
  const bf16_t* xr[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) xr[n] = x + (int64_t)min(t0 + n, T_ - 1) * d;
  float acc[NT][8];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[n][j] = 0.0f;
#pragma unroll 2
  for (int k0 = (wave * 64 + lane) * 8; k0 < d; k0 += 256 * 8) {
    float wv[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(Wg + (int64_t)(k0 + i) * 8), wv[i]);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float xv[8];
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(xr[n] + k0), xv);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[n][j] = fmaf(xv[i], wv[i][j], acc[n][j]);
    }
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const float s = wave_sum8(acc[n], lane);              // expert lane / 8
    if ((lane & 7) == 0) part[wave][n][lane >> 3] = s;
  }
  __syncthreads();
  if (wave != 0) return;
  float lg[NT];                                         // lane l: expert l / 8 of token n
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int e = lane >> 3;
    lg[n] = ((part[0][n][e] + part[1][n][e]) + part[2][n][e]) + part[3][n][e];
  }
  if (logits_out && (lane & 7) == 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
      if (t0 + n < T_) logits_out[(int64_t)(t0 + n) * 8 + (lane >> 3)] = lg[n];
  }
  // lane 16 n + e: expert e of token n (e < 8; lanes with e >= 8 hold nothing)
  const int n = lane >> 4;
  const int e = lane & 15;
  float v = 0.0f;
#pragma unroll
  for (int m = 0; m < NT; ++m) {
    const float g = __shfl(lg[m], 8 * (e & 7), 64);
    if (m == n) v = g;
  }
  const bool live = t0 + n < T_;
  bool taken = false;
  float first = 0.0f, denom = 0.0f;
  const int64_t t = t0 + n;
  for (int r = 0; r < K; ++r) {
    float bv = v;
    int bi = (e < 8 && !taken) ? e : -1;
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oi = __shfl_xor(bi, m, 64);
      if (ranks_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (e == bi) taken = true;
    if (r == 0) first = bv;
    const float ex = expf(bv - first);
    denom += ex;
    if (e == 0 && live) {
      topk_idx[t * K + r] = bi;
      topk_w[t * K + r] = ex;
    }
  }
  if (e == 0 && live)
    for (int r = 0; r < K; ++r) topk_w[t * K + r] = topk_w[t * K + r] / denom;
}

// Glue between two pre-norm blocks of a stack, for small batches (one
// workgroup of 512 threads per token), bf16, E % 8 == 0, d % 8 == 0.  In one
// launch, for token t:
//   1. (COMBINE) the previous block's combine with the residual add, one
//      thread per 4 features: s = w0 O[pos0] + ... in rank order (O summed
//      over its slices in slice order), h[t] = round(h[t] + s) -- the
//      arithmetic of the combine kernel;
//   2. RMSNorm ("【DL輪読会】Mixtral of Experts" slides, "Architecture –
//      全体"): thread i < 256 sums the squares of features i, i + 256, ... in
//      order (read back from LDS), then a fixed tree over those 256 sums,
//      xn = round(h / sqrt(mean + eps)) -- the arithmetic of the RMSNorm
//      kernel;
//   3. (ROUTE) the next block's router on xn, held in LDS, by the first four
//      wavefronts -- the arithmetic of the router kernel with four
//      wavefronts per token.  Their first W_g rows are loaded at the start of
//      the kernel, so those loads overlap steps 1 and 2.  Without ROUTE
//      (large batches, whose router is the many-token kernel, launched
//      after this one) the kernel ends after step 2.
// The results are those of the separate kernels, bit for bit.  Token
// t's previous gate weights and positions are read in step 1, before the
// barriers after which wave 0 overwrites them with the new ones, and by the
// workgroup of token t only.
constexpr int kGlueThreads = 512;
constexpr int kGluePrefetch = 2;     // 8-row W_g chunks held per router thread
constexpr int kGlueRanks = 2;        // the combine's loads are all issued at once for
constexpr int kGlueSlices = 4;       // K <= kGlueRanks and splits <= kGlueSlices

template <bool COMBINE, bool ROUTE>
__global__ __launch_bounds__(kGlueThreads) void stack_glue_kernel(
    bf16_t* __restrict__ h, bf16_t* __restrict__ xn, const float* __restrict__ O, int splits,
    int64_t slice, float* __restrict__ topk_w, const int32_t* __restrict__ pos,
    int32_t* __restrict__ topk_idx, const bf16_t* __restrict__ Wg, int d, int E, int K,
    float eps) {
  extern __shared__ __align__(16) bf16_t xs[];   // [d]: the new h, then xn
  __shared__ float part[256];
  __shared__ float wave_part[4][kMaxExperts];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t t = blockIdx.x;
  const bool router = tid < 256;

  // W_g rows of the router threads' first chunks (experts 0..7)
  uint4 wpre[kGluePrefetch][8];
#pragma unroll
  for (int q = 0; q < kGluePrefetch; ++q) {
    const int k0 = tid * 8 + q * 256 * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      wpre[q][i] = (ROUTE && router && k0 < d) ? *reinterpret_cast<const uint4*>(Wg + (int64_t)(k0 + i) * E)
                                      : make_uint4(0, 0, 0, 0);
  }

  bf16_t* hr = h + t * d;
  if constexpr (COMBINE) {
    const float* wt = topk_w + t * K;
    const int32_t* pt = pos + t * K;
    // h[c..c+3] = round(h + s) from the rank sums o_r (slices added in slice
    // order): s = w0 o_0, then s = fma(w_r, o_r, s) in rank order
    auto store = [&](int c, uint2 hv, float s0, float s1, float s2, float s3) {
      uint2 out;
      out.x = pack_bf16x2(__uint_as_float(hv.x << 16) + s0, __uint_as_float(hv.x & 0xffff0000u) + s1);
      out.y = pack_bf16x2(__uint_as_float(hv.y << 16) + s2, __uint_as_float(hv.y & 0xffff0000u) + s3);
      *reinterpret_cast<uint2*>(hr + c) = out;
      *reinterpret_cast<uint2*>(xs + c) = out;
    };
    auto o_row = [&](int r, int sl, int c) {
      const int p = pt[r];
      if (p < 0) return make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      return *reinterpret_cast<const float4*>(O + sl * slice + (int64_t)p * d + c);
    };
    if (K <= kGlueRanks && splits <= kGlueSlices) {
      // every load of the thread's two groups issued before any is used
      for (int c0 = tid * 4; c0 < d; c0 += 2 * kGlueThreads * 4) {
        float4 buf[2][kGlueRanks][kGlueSlices];
        uint2 hv[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int c = c0 + g * kGlueThreads * 4;
          const bool live = c < d;
          hv[g] = live ? *reinterpret_cast<const uint2*>(hr + c) : make_uint2(0, 0);
#pragma unroll
          for (int r = 0; r < kGlueRanks; ++r)
#pragma unroll
            for (int sl = 0; sl < kGlueSlices; ++sl)
              buf[g][r][sl] = (live && r < K && sl < splits) ? o_row(r, sl, c)
                                                             : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int c = c0 + g * kGlueThreads * 4;
          if (c >= d) continue;
          float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
          for (int r = 0; r < kGlueRanks; ++r) {
            if (r >= K) break;
            float4 o = buf[g][r][0];
#pragma unroll
            for (int sl = 1; sl < kGlueSlices; ++sl) {
              if (sl >= splits) break;
              o.x += buf[g][r][sl].x;
              o.y += buf[g][r][sl].y;
              o.z += buf[g][r][sl].z;
              o.w += buf[g][r][sl].w;
            }
            const float wr = wt[r];
            if (r == 0) {
              s0 = wr * o.x, s1 = wr * o.y, s2 = wr * o.z, s3 = wr * o.w;
            } else {
              s0 = fmaf(wr, o.x, s0);
              s1 = fmaf(wr, o.y, s1);
              s2 = fmaf(wr, o.z, s2);
              s3 = fmaf(wr, o.w, s3);
            }
          }
          store(c, hv[g], s0, s1, s2, s3);
        }
      }
    } else {
      for (int c = tid * 4; c < d; c += kGlueThreads * 4) {
        const uint2 hv = *reinterpret_cast<const uint2*>(hr + c);
        float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
        for (int r = 0; r < K; ++r) {
          float4 o = o_row(r, 0, c);
          for (int sl = 1; sl < splits; ++sl) {
            const float4 u = o_row(r, sl, c);
            o.x += u.x;
            o.y += u.y;
            o.z += u.z;
            o.w += u.w;
          }
          const float wr = wt[r];
          if (r == 0) {
            s0 = wr * o.x, s1 = wr * o.y, s2 = wr * o.z, s3 = wr * o.w;
          } else {
            s0 = fmaf(wr, o.x, s0);
            s1 = fmaf(wr, o.y, s1);
            s2 = fmaf(wr, o.z, s2);
            s3 = fmaf(wr, o.w, s3);
          }
        }
        store(c, hv, s0, s1, s2, s3);
      }
    }
  } else {
    for (int c = tid * 4; c < d; c += kGlueThreads * 4)
      *reinterpret_cast<uint2*>(xs + c) = *reinterpret_cast<const uint2*>(hr + c);
  }
  __syncthreads();
  if (router) {
    float sq = 0.0f;
    for (int c = tid; c < d; c += 256) {
      const float v = bf16_to_f32(xs[c]);
      sq = fmaf(v, v, sq);
    }
    part[tid] = sq;
  }
  __syncthreads();
  for (int m = 128; m >= 1; m >>= 1) {
    if (tid < m) part[tid] += part[tid + m];
    __syncthreads();
  }
  const float inv = 1.0f / sqrtf(part[0] / (float)d + eps);
  bf16_t* xr = xn + t * d;
  for (int c = tid * 4; c < d; c += kGlueThreads * 4) {
    const uint2 hv = *reinterpret_cast<const uint2*>(xs + c);
    uint2 xb;
    xb.x = pack_bf16x2(__uint_as_float(hv.x << 16) * inv, __uint_as_float(hv.x & 0xffff0000u) * inv);
    xb.y = pack_bf16x2(__uint_as_float(hv.y << 16) * inv, __uint_as_float(hv.y & 0xffff0000u) * inv);
    *reinterpret_cast<uint2*>(xs + c) = xb;
    *reinterpret_cast<uint2*>(xr + c) = xb;
  }
  if constexpr (!ROUTE) return;   // the next block's router runs as its own launch
  __syncthreads();

  // the router kernel's vector path with TPT = 256 (see vec_partials): the
  // same chunks in the same order, the first kGluePrefetch from registers
  for (int e0 = 0; router && e0 < E; e0 += 8) {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    int q = 0;
    for (int k0 = tid * 8; k0 < d; k0 += 256 * 8, ++q) {
      float xv[8];
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(xs + k0), xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float wv[8];
        if (e0 == 0 && q < kGluePrefetch) {
          uint4 pre = wpre[0][i];
#pragma unroll
          for (int qq = 1; qq < kGluePrefetch; ++qq)
            if (q == qq) pre = wpre[qq][i];
          bf16x8_to_f32(pre, wv);
        } else {
          bf16x8_to_f32(*reinterpret_cast<const uint4*>(Wg + (int64_t)(k0 + i) * E + e0), wv);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(xv[i], wv[j], acc[j]);
      }
    }
    const float sum = wave_sum8(acc, lane);             // value lane / 8
    if ((lane & 7) == 0 && e0 + (lane >> 3) < E) wave_part[wave][e0 + (lane >> 3)] = sum;
  }
  __syncthreads();
  if (wave != 0) return;
  float logit = 0.0f;
  if (lane < E) {
    for (int v = 0; v < 4; ++v) logit += wave_part[v][lane];
  }
  select_topk(logit, lane, E, K, topk_idx + t * K, topk_w + t * K);
}

template <typename T, int TPT, bool VEC>
void launch_t(const void* x, const void* Wg, int T_, int d, int E, int K, int32_t* idx,
              float* w, float* logits, hipStream_t stream) {
  const int per_block = 256 / TPT;
  hipLaunchKernelGGL((router_topk_kernel<T, TPT, VEC>), dim3((T_ + per_block - 1) / per_block),
                     dim3(256), 0, stream, static_cast<const T*>(x), static_cast<const T*>(Wg), T_,
                     d, E, K, idx, w, logits);
}

}  // namespace

bool stack_glue_supported(int T, int d, int E, int dtype) {
  return dtype == kBF16 && T < 1024 && E % 8 == 0 && d % 8 == 0 && d <= kStackGlueMaxD;
}

hipError_t launch_stack_glue(void* h, void* xn, const float* O, int o_splits, int64_t slice,
                             float* topk_w, const int32_t* pos, int32_t* topk_idx, const void* Wg,
                             int T, int d, int E, int K, float eps, hipStream_t stream) {
  const int lds = d * (int)sizeof(bf16_t);
  if (O) {
    hipError_t e =
        allow_dynamic_lds(reinterpret_cast<const void*>(&stack_glue_kernel<true, true>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((stack_glue_kernel<true, true>), dim3(T), dim3(kGlueThreads), lds, stream,
                       static_cast<bf16_t*>(h), static_cast<bf16_t*>(xn), O, o_splits, slice,
                       topk_w, pos, topk_idx, static_cast<const bf16_t*>(Wg), d, E, K, eps);
  } else {
    hipError_t e =
        allow_dynamic_lds(reinterpret_cast<const void*>(&stack_glue_kernel<false, true>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((stack_glue_kernel<false, true>), dim3(T), dim3(kGlueThreads), lds, stream,
                       static_cast<bf16_t*>(h), static_cast<bf16_t*>(xn), nullptr, 1, 0, topk_w,
                       nullptr, topk_idx, static_cast<const bf16_t*>(Wg), d, E, K, eps);
  }
  return hipGetLastError();
}

bool stack_norm_supported(int d, int dtype) {
  return dtype == kBF16 && d % 8 == 0 && d <= kStackGlueMaxD;
}

hipError_t launch_stack_norm(void* h, void* xn, const float* O, int o_splits, int64_t slice,
                             const float* topk_w, const int32_t* pos, int T, int d, int K,
                             float eps, hipStream_t stream) {
  const int lds = d * (int)sizeof(bf16_t);
  if (O) {
    hipError_t e =
        allow_dynamic_lds(reinterpret_cast<const void*>(&stack_glue_kernel<true, false>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((stack_glue_kernel<true, false>), dim3(T), dim3(kGlueThreads), lds, stream,
                       static_cast<bf16_t*>(h), static_cast<bf16_t*>(xn), O, o_splits, slice,
                       const_cast<float*>(topk_w), pos, nullptr, nullptr, d, 0, K, eps);
  } else {
    hipError_t e =
        allow_dynamic_lds(reinterpret_cast<const void*>(&stack_glue_kernel<false, false>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((stack_glue_kernel<false, false>), dim3(T), dim3(kGlueThreads), lds,
                       stream, static_cast<bf16_t*>(h), static_cast<bf16_t*>(xn), nullptr, 1, 0,
                       nullptr, nullptr, nullptr, nullptr, d, 0, K, eps);
  }
  return hipGetLastError();
}

hipError_t launch_router_topk(const void* x, const void* Wg, int T, int d, int E, int K,
                              int dtype, int32_t* topk_idx, float* topk_w, float* logits,
                              hipStream_t stream) {
  // Few tokens: four wavefronts per token; many tokens: one.
  const bool wide = T < 1024;
  const bool vec = dtype == kBF16 && E % 8 == 0 && d % 8 == 0 &&
                   (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(Wg) & 15) == 0;
  if (dtype == kBF16 && vec && !wide && E == 8 && K <= 8) {
    const int per_block = kRouterTokPerGroup;
    hipLaunchKernelGGL(router_e8_kernel, dim3((T + per_block - 1) / per_block), dim3(256), 0,
                       stream, static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(Wg), T, d,
                       K, topk_idx, topk_w, logits);
    return hipGetLastError();
  }
  if (dtype == kBF16) {
    if (vec) {
      if (wide) launch_t<bf16_t, 256, true>(x, Wg, T, d, E, K, topk_idx, topk_w, logits, stream);
      else launch_t<bf16_t, 64, true>(x, Wg, T, d, E, K, topk_idx, topk_w, logits, stream);
    } else {
      if (wide) launch_t<bf16_t, 256, false>(x, Wg, T, d, E, K, topk_idx, topk_w, logits, stream);
      else launch_t<bf16_t, 64, false>(x, Wg, T, d, E, K, topk_idx, topk_w, logits, stream);
    }
  } else {
    if (wide) launch_t<float, 256, false>(x, Wg, T, d, E, K, topk_idx, topk_w, logits, stream);
    else launch_t<float, 64, false>(x, Wg, T, d, E, K, topk_idx, topk_w, logits, stream);
  }
  return hipGetLastError();
}

}  // namespace moe
