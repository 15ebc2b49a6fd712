// Weight-streaming grouped GEMMs for small batches (decode): every expert
// segment has at most 16*NJ rows, so the product is bound by reading each
// active expert's weights once from HBM.
//
// Same product as the LDS-tiled kernels ("从Mistral 7B到MoE模型Mixtral 8x7B
// 的全面解析" (aiqianji.com) section 3.2.4, code block D), organised for
// bandwidth:
//   * a wavefront owns 128 features and a k-range; each lane fetches an 8x8
//     (k x feature) block with eight 16-byte loads per weight matrix, lanes
//     0-15 covering 256 contiguous bytes of one weight row;
//   * the block is transposed in registers and used directly as the M-side
//     operand of v_mfma_f32_16x16x32_bf16 (instruction c takes feature
//     8*i + c at M-row i) -- no LDS round trip for the weights;
//   * the token operand (16 rows x 8 k per lane) is a 16-byte load of the
//     gathered activation row, L2-resident;
//   * loads for the next k-step are issued before the current step's
//     transposes and matrix instructions (two register stages);
//   * every wave streams one matrix: with two matrices (W1, W3) waves 0-1
//     take W1 and waves 2-3 take W3, each pair splitting the k-range; with
//     one matrix the four waves split it.  The waves' partial products are
//     summed in LDS in wave order;
//   * K is further split over `splits` workgroups (fp32 partial sums written
//     to separate slices, summed later in slice order), so results are
//     deterministic and the grid has thousands of workgroups.
// Epilogue: with one split and two matrices, H = bf16(SiLU(a) * b) is
// stored directly; otherwise the fp32 partial sums are stored and
// swiglu_finish_kernel (its own launch) adds the splits in order and applies
// SwiGLU.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

struct StreamArgs {
  const bf16_t* A;         // [rows, Kdim] activations
  const int32_t* gather;   // sorted_token for gathered rows, else null
  const int32_t* offsets;  // [E + 1]
  ExpertPtrs Wa;
  ExpertPtrs Wb;
  bf16_t* H;               // final H when DUAL and splits == 1
  float* part;             // [splits][mats][P][N] partial sums otherwise
  int Kdim;
  int N;
  int E;
  int P;
  int max_tiles;
  int splits;
};

__device__ __forceinline__ uint32_t perm_lo(uint32_t hi_src, uint32_t lo_src) {
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t hi_src, uint32_t lo_src) {
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u);
}
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// rows[r] = 8 bf16 of k-row r (features c = 0..7, two per dword); returns
// operand c = the 8 k-values of feature c.
__device__ __forceinline__ bf16x8_t column(const u32x4_t rows[8], int c) {
  const int q = c >> 1;
  u32x4_t v;
  if ((c & 1) == 0) {
    v[0] = perm_lo(rows[1][q], rows[0][q]);
    v[1] = perm_lo(rows[3][q], rows[2][q]);
    v[2] = perm_lo(rows[5][q], rows[4][q]);
    v[3] = perm_lo(rows[7][q], rows[6][q]);
  } else {
    v[0] = perm_hi(rows[1][q], rows[0][q]);
    v[1] = perm_hi(rows[3][q], rows[2][q]);
    v[2] = perm_hi(rows[5][q], rows[4][q]);
    v[3] = perm_hi(rows[7][q], rows[6][q]);
  }
  return __builtin_bit_cast(bf16x8_t, v);
}

constexpr int kWaves = 4;
constexpr int kFeat = 128;  // features per workgroup (and per wave)

template <int NJ, bool DUAL>
struct StreamCfg {
  static constexpr int kMats = DUAL ? 2 : 1;
  static constexpr int kKParts = kWaves / kMats;  // waves sharing one matrix
  // LDS for the wave reduction: [wave][c][j][lane] float4
  static constexpr int kRedFloats = kWaves * 8 * NJ * 64 * 4;
};

template <int NJ, bool DUAL>
__global__ __launch_bounds__(256) void stream_gemm_kernel(StreamArgs a) {
  using C = StreamCfg<NJ, DUAL>;
  constexpr int M = C::kMats;
  __shared__ float4 red[C::kRedFloats / 4];

  const int tiles_f = a.N / kFeat;
  int bid = blockIdx.x;
  const int ftile = bid % tiles_f;
  bid /= tiles_f;
  const int s = bid % a.splits;
  const int ttile = bid / a.splits;
  int e, row_begin, row_end;
  if (!find_tile(a.offsets, a.E, 16 * NJ, ttile, e, row_begin, row_end)) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int mat = wave / C::kKParts;
  const int kpart = wave % C::kKParts;
  const int lrow = lane & 15;
  const int lk = lane >> 4;
  const int f0 = ftile * kFeat;
  const int kc = a.Kdim / a.splits;
  const int kw = kc / C::kKParts;
  const int kbeg = s * kc + kpart * kw;
  const int nsteps = kw / 32;
  const int64_t N = a.N;

  const bf16_t* wsrc = static_cast<const bf16_t*>(mat == 0 ? a.Wa.p[e] : a.Wb.p[e]) +
                       (int64_t)(kbeg + 8 * lk) * N + f0 + 8 * lrow;
  const bf16_t* bsrc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int r = row_begin + j * 16 + lrow;
    bsrc[j] = nullptr;
    if (r < row_end) {
      const int64_t src_row = a.gather ? a.gather[r] : r;
      bsrc[j] = a.A + src_row * a.Kdim + kbeg + 8 * lk;
    }
  }

  f32x4_t acc[8][NJ];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[c][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t w0[8], w1[8];
  u32x4_t b0[NJ], b1[NJ];

  auto load = [&](u32x4_t (&w)[8], u32x4_t (&b)[NJ], int step) {
    const bf16_t* src = wsrc + (int64_t)step * 32 * N;
#pragma unroll
    for (int r = 0; r < 8; ++r)
      w[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + (int64_t)r * N));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      b[j] = bsrc[j] ? *reinterpret_cast<const u32x4_t*>(bsrc[j] + step * 32) : u32x4_t{0, 0, 0, 0};
  };
  auto compute = [&](const u32x4_t (&w)[8], const u32x4_t (&b)[NJ]) {
    bf16x8_t bo[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) bo[j] = __builtin_bit_cast(bf16x8_t, b[j]);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bf16x8_t op = column(w, c);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[c][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op, bo[j], acc[c][j], 0, 0, 0);
    }
  };

  if (nsteps > 0) load(w0, b0, 0);
  for (int i = 0; i < nsteps; i += 2) {
    if (i + 1 < nsteps) load(w1, b1, i + 1);
    compute(w0, b0);
    if (i + 2 < nsteps) load(w0, b0, i + 2);
    if (i + 1 < nsteps) compute(w1, b1);
  }

#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const f32x4_t v = acc[c][j];
      red[((wave * 8 + c) * NJ + j) * 64 + lane] = make_float4(v[0], v[1], v[2], v[3]);
    }
  __syncthreads();

  // Thread t produces 8 consecutive features (c = 0..7) of one token for
  // every (j, source lane L, q) -- NJ*256 outputs over 256 threads.
  const float* redf = reinterpret_cast<const float*>(red);
  for (int o = threadIdx.x; o < NJ * 256; o += 256) {
    const int L = o & 63;
    const int q = (o >> 6) & 3;
    const int j = o >> 8;
    const int r = row_begin + j * 16 + (L & 15);
    if (r >= row_end) continue;
    const int f = f0 + 8 * (4 * (L >> 4) + q);
    // matrix m is the sum of waves m*kKParts .. m*kKParts + kKParts - 1, in order
    float sum[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < C::kKParts; ++w)
          t += redf[((((m * C::kKParts + w) * 8 + c) * NJ + j) * 64 + L) * 4 + q];
        sum[m][c] = t;
      }
    if (DUAL && a.splits == 1) {
      uint4 h;
      h.x = pack_bf16x2(silu_f32(sum[0][0]) * sum[M - 1][0], silu_f32(sum[0][1]) * sum[M - 1][1]);
      h.y = pack_bf16x2(silu_f32(sum[0][2]) * sum[M - 1][2], silu_f32(sum[0][3]) * sum[M - 1][3]);
      h.z = pack_bf16x2(silu_f32(sum[0][4]) * sum[M - 1][4], silu_f32(sum[0][5]) * sum[M - 1][5]);
      h.w = pack_bf16x2(silu_f32(sum[0][6]) * sum[M - 1][6], silu_f32(sum[0][7]) * sum[M - 1][7]);
      *reinterpret_cast<uint4*>(a.H + (int64_t)r * N + f) = h;
    } else {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float* dst = a.part + (((int64_t)s * M + m) * a.P + r) * N + f;
        *reinterpret_cast<float4*>(dst) = make_float4(sum[m][0], sum[m][1], sum[m][2], sum[m][3]);
        *reinterpret_cast<float4*>(dst + 4) =
            make_float4(sum[m][4], sum[m][5], sum[m][6], sum[m][7]);
      }
    }
  }
}

// H[r][f] = bf16(SiLU(sum_s part[s][0][r][f]) * sum_s part[s][1][r][f]), slices
// summed in order.
__global__ __launch_bounds__(256) void swiglu_finish_kernel(const float* __restrict__ part,
                                                            int splits, int P, int N,
                                                            bf16_t* __restrict__ H) {
  const int64_t n4 = (int64_t)P * N / 4;
  const int64_t slice = (int64_t)P * N;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n4;
       g += (int64_t)gridDim.x * blockDim.x) {
    float4 av = reinterpret_cast<const float4*>(part)[g];
    float4 bv = reinterpret_cast<const float4*>(part + slice)[g];
    for (int s = 1; s < splits; ++s) {
      const float4 x = reinterpret_cast<const float4*>(part + (2 * s) * slice)[g];
      const float4 y = reinterpret_cast<const float4*>(part + (2 * s + 1) * slice)[g];
      av.x += x.x; av.y += x.y; av.z += x.z; av.w += x.w;
      bv.x += y.x; bv.y += y.y; bv.z += y.z; bv.w += y.w;
    }
    uint2 h;
    h.x = pack_bf16x2(silu_f32(av.x) * bv.x, silu_f32(av.y) * bv.y);
    h.y = pack_bf16x2(silu_f32(av.z) * bv.z, silu_f32(av.w) * bv.w);
    reinterpret_cast<uint2*>(H)[g] = h;
  }
}

template <int NJ, bool DUAL>
hipError_t launch_stream(const StreamArgs& in, hipStream_t stream) {
  StreamArgs a = in;
  a.max_tiles = (int)(((int64_t)a.P + (int64_t)a.E * (16 * NJ - 1)) / (16 * NJ));
  if (a.max_tiles <= 0) return hipSuccess;
  const int64_t grid = (int64_t)a.max_tiles * a.splits * (a.N / kFeat);
  hipLaunchKernelGGL((stream_gemm_kernel<NJ, DUAL>), dim3((unsigned)grid), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace

bool stream_gemm_supported(int Kdim, int N, int splits) {
  // one matrix: the k-range of a split is cut in four, two matrices: in two
  return splits >= 1 && N % kFeat == 0 && Kdim % (splits * kWaves * 32) == 0;
}

hipError_t launch_stream_swiglu_bf16(const void* x, const int32_t* sorted_token,
                                     const ExpertPtrs& W1, const ExpertPtrs& W3,
                                     const int32_t* offsets, int P, int d, int d_ff, int E,
                                     int splits, float* part, void* H, hipStream_t stream) {
  StreamArgs a{};
  a.A = static_cast<const bf16_t*>(x);
  a.gather = sorted_token;
  a.offsets = offsets;
  a.Wa = W1;
  a.Wb = W3;
  a.H = static_cast<bf16_t*>(H);
  a.part = part;
  a.Kdim = d;
  a.N = d_ff;
  a.E = E;
  a.P = P;
  a.splits = splits;
  return launch_stream<1, true>(a, stream);
}

hipError_t launch_swiglu_finish_bf16(const float* part, int splits, int P, int d_ff, void* H,
                                     hipStream_t stream) {
  const int64_t n4 = (int64_t)P * d_ff / 4;
  if (n4 == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 2048);
  hipLaunchKernelGGL(swiglu_finish_kernel, dim3(blocks), dim3(256), 0, stream, part, splits, P,
                     d_ff, static_cast<bf16_t*>(H));
  return hipGetLastError();
}

hipError_t launch_stream_down_bf16(const void* H, const ExpertPtrs& W2, const int32_t* offsets,
                                   int P, int d, int d_ff, int E, int splits, float* O,
                                   hipStream_t stream) {
  StreamArgs a{};
  a.A = static_cast<const bf16_t*>(H);
  a.gather = nullptr;
  a.offsets = offsets;
  a.Wa = W2;
  a.Wb = W2;
  a.H = nullptr;
  a.part = O;
  a.Kdim = d_ff;
  a.N = d;
  a.E = E;
  a.P = P;
  a.splits = splits;
  return launch_stream<1, false>(a, stream);
}

}  // namespace moe
