// Grouped bf16 matrix-core GEMMs of the SwiGLU experts (gfx950).
//
// "从Mistral 7B到MoE模型Mixtral 8x7B的全面解析" (aiqianji.com) section 3.2.4,
// code block D: an expert computes w2(act(w1 h) * w3 h) on the rows routed to
// it.  Rows arrive expert-sorted (segment [offsets[e], offsets[e+1]) belongs
// to expert e), so one launch serves every expert: a workgroup owns one
// (token tile, feature tile) and finds its expert from the offsets on the
// device -- no host readback of the counts, empty tiles exit at once.
//
// Orientation.  Weights are stored [k][n] (n contiguous, the pages' x . W
// form) while a matrix-core operand needs 8 consecutive k of one row or
// column per lane.  The kernel therefore computes the transposed product
//     D[feature][token] = sum_k W[k][feature] * A[token][k]
// with the weight tile as the M-side operand.  Each thread fetches an 8x8
// (k x feature) block of W with eight 16-byte loads, transposes it in
// registers with byte permutes, and writes eight 16-byte feature rows
// (k-contiguous) to LDS.  The token tile is already k-contiguous and is
// copied as is (gathered through sorted_token for the W1/W3 product).  The
// accumulator layout of v_mfma_f32_16x16x32_bf16 then gives every lane four
// consecutive features of one token, so the epilogue writes 8-byte (bf16 H)
// or 16-byte (fp32 O) vectors.
//
// SwiGLU fusion: the W1 and W3 tiles of the same features share the token
// operand; the lane holding a = x.W1[:, f] also holds b = x.W3[:, f], and
// the epilogue stores H = bf16(SiLU(a) * b) directly.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

struct GemmArgs {
  const bf16_t* A;         // [rows, Kdim] activations (x or H)
  const int32_t* gather;   // sorted_token when A rows are gathered, else null
  const int32_t* offsets;  // [E + 1]
  ExpertPtrs Wa;           // W1 (dual) or W2
  ExpertPtrs Wb;           // W3 (dual only)
  void* out;               // H bf16 [P, N] (dual) or O fp32 [P, N]
  int Kdim;                // reduction length
  int N;                   // features (d_ff for W1/W3, d for W2)
  int E;
  int max_tiles;           // worst-case number of token tiles
};

__device__ __forceinline__ uint32_t perm_lo(uint32_t hi_src, uint32_t lo_src) {
  // {lo16(lo_src), lo16(hi_src)}
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t hi_src, uint32_t lo_src) {
  // {hi16(lo_src), hi16(hi_src)}
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u);
}

__device__ __forceinline__ uint32_t comp(const uint4& v, int q) {
  return q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
}

// rows[r] holds 8 bf16 of row r (columns c = 0..7, two per dword); on return
// cols[c] holds 8 bf16 of column c (rows r = 0..7).
__device__ __forceinline__ void transpose8x8(const uint4 rows[8], uint4 cols[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    cols[2 * q] = make_uint4(perm_lo(comp(rows[1], q), comp(rows[0], q)),
                             perm_lo(comp(rows[3], q), comp(rows[2], q)),
                             perm_lo(comp(rows[5], q), comp(rows[4], q)),
                             perm_lo(comp(rows[7], q), comp(rows[6], q)));
    cols[2 * q + 1] = make_uint4(perm_hi(comp(rows[1], q), comp(rows[0], q)),
                                 perm_hi(comp(rows[3], q), comp(rows[2], q)),
                                 perm_hi(comp(rows[5], q), comp(rows[4], q)),
                                 perm_hi(comp(rows[7], q), comp(rows[6], q)));
  }
}

template <int BF, int BT, int BK, int WAVES_F, int WAVES_T, bool DUAL>
struct GemmCfg {
  static constexpr int kThreads = 64 * WAVES_F * WAVES_T;
  static constexpr int kMats = DUAL ? 2 : 1;
  static constexpr int kWF = BF / WAVES_F;  // features per wave
  static constexpr int kWT = BT / WAVES_T;  // tokens per wave
  static constexpr int kMI = kWF / 16;
  static constexpr int kNJ = kWT / 16;
  static constexpr int kStride = BK + 8;    // LDS row stride in bf16 (16-byte pad)
  static constexpr int kKB = BK / 8;        // 8-row blocks along k
  static constexpr int kWBlocks = kMats * kKB * (BF / 8);
  static constexpr int kWPerThread = (kWBlocks + kThreads - 1) / kThreads;
  static constexpr int kAChunks = BT * kKB;  // 16-byte chunks of the token tile
  static constexpr int kAPerThread = (kAChunks + kThreads - 1) / kThreads;
  static constexpr int kLdsW = kMats * BF * kStride;
  static constexpr int kLdsA = BT * kStride;
  static constexpr int kLdsBytes = 2 * (kLdsW + kLdsA) * 2;
  static_assert(BF % (16 * WAVES_F) == 0 && BT % (16 * WAVES_T) == 0, "wave tile");
  static_assert(BK % 32 == 0, "k step");
};

template <int BF, int BT, int BK, int WAVES_F, int WAVES_T, bool DUAL>
__global__ __launch_bounds__(64 * WAVES_F * WAVES_T) void grouped_gemm_bf16_kernel(GemmArgs args) {
  using C = GemmCfg<BF, BT, BK, WAVES_F, WAVES_T, DUAL>;
  extern __shared__ __align__(16) bf16_t lds[];

  const int tiles_f = args.N / BF;
  const int ttile = blockIdx.x % args.max_tiles;
  const int ftile = blockIdx.x / args.max_tiles;
  int e, row_begin, row_end;
  if (!find_tile(args.offsets, args.E, BT, ttile, e, row_begin, row_end)) return;
  if (ftile >= tiles_f) return;
  const int f0 = ftile * BF;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int fw = (wave % WAVES_F) * C::kWF;
  const int tw = (wave / WAVES_F) * C::kWT;

  const bf16_t* Wm[2];
  Wm[0] = static_cast<const bf16_t*>(args.Wa.p[e]);
  Wm[1] = DUAL ? static_cast<const bf16_t*>(args.Wb.p[e]) : Wm[0];
  const int64_t N = args.N;

  // Token rows this thread copies (fixed across k).
  const bf16_t* a_src[C::kAPerThread];
  int a_lds[C::kAPerThread];
#pragma unroll
  for (int i = 0; i < C::kAPerThread; ++i) {
    const int q = tid + i * C::kThreads;
    const int row = q / C::kKB;
    const int kc = q % C::kKB;
    const int r = row_begin + row;
    a_src[i] = nullptr;
    a_lds[i] = -1;
    if (q < C::kAChunks) {
      a_lds[i] = row * C::kStride + kc * 8;
      if (r < row_end) {
        const int64_t src_row = args.gather ? args.gather[r] : r;
        a_src[i] = args.A + src_row * args.Kdim + kc * 8;
      }
    }
  }

  uint4 wreg[C::kWPerThread][8];
  uint4 areg[C::kAPerThread];

  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::kWPerThread; ++i) {
      const int q = tid + i * C::kThreads;
      if (q < C::kWBlocks) {
        const int mat = q / (C::kKB * (BF / 8));
        const int rem = q % (C::kKB * (BF / 8));
        const int kb = rem % C::kKB;
        const int fb = rem / C::kKB;
        const bf16_t* src = Wm[mat] + (int64_t)(k0 + kb * 8) * N + f0 + fb * 8;
#pragma unroll
        for (int r = 0; r < 8; ++r) wreg[i][r] = *reinterpret_cast<const uint4*>(src + r * N);
      }
    }
#pragma unroll
    for (int i = 0; i < C::kAPerThread; ++i) {
      if (a_src[i])
        areg[i] = *reinterpret_cast<const uint4*>(a_src[i] + k0);
      else
        areg[i] = make_uint4(0, 0, 0, 0);
    }
  };

  auto store_tiles = [&](int buf) {
    bf16_t* sW = lds + buf * (C::kLdsW + C::kLdsA);
    bf16_t* sA = sW + C::kLdsW;
#pragma unroll
    for (int i = 0; i < C::kWPerThread; ++i) {
      const int q = tid + i * C::kThreads;
      if (q < C::kWBlocks) {
        const int mat = q / (C::kKB * (BF / 8));
        const int rem = q % (C::kKB * (BF / 8));
        const int kb = rem % C::kKB;
        const int fb = rem / C::kKB;
        uint4 cols[8];
        transpose8x8(wreg[i], cols);
        bf16_t* dst = sW + (mat * BF + fb * 8) * C::kStride + kb * 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) *reinterpret_cast<uint4*>(dst + c * C::kStride) = cols[c];
      }
    }
#pragma unroll
    for (int i = 0; i < C::kAPerThread; ++i)
      if (a_lds[i] >= 0) *reinterpret_cast<uint4*>(sA + a_lds[i]) = areg[i];
  };

  f32x4_t acc[C::kMats][C::kMI][C::kNJ];
#pragma unroll
  for (int m = 0; m < C::kMats; ++m)
#pragma unroll
    for (int i = 0; i < C::kMI; ++i)
#pragma unroll
      for (int j = 0; j < C::kNJ; ++j) acc[m][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = args.Kdim / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();

  const int lrow = lane & 15;
  const int lk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) * BK);
    const bf16_t* sW = lds + cur * (C::kLdsW + C::kLdsA);
    const bf16_t* sA = sW + C::kLdsW;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      bf16x8_t b[C::kNJ];
#pragma unroll
      for (int j = 0; j < C::kNJ; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(sA + (tw + j * 16 + lrow) * C::kStride + ks + lk);
#pragma unroll
      for (int m = 0; m < C::kMats; ++m) {
#pragma unroll
        for (int i = 0; i < C::kMI; ++i) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
              sW + (m * BF + fw + i * 16 + lrow) * C::kStride + ks + lk);
#pragma unroll
          for (int j = 0; j < C::kNJ; ++j)
            acc[m][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[m][i][j], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nk) store_tiles(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds features f .. f+3 of token column (lane & 15).
  const int fq = (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < C::kNJ; ++j) {
    const int r = row_begin + tw + j * 16 + lrow;
    if (r >= row_end) continue;
#pragma unroll
    for (int i = 0; i < C::kMI; ++i) {
      const int f = f0 + fw + i * 16 + fq;
      if constexpr (DUAL) {
        const f32x4_t a = acc[0][i][j];
        const f32x4_t bb = acc[1][i][j];
        uint2 v;
        v.x = pack_bf16x2(silu_f32(a[0]) * bb[0], silu_f32(a[1]) * bb[1]);
        v.y = pack_bf16x2(silu_f32(a[2]) * bb[2], silu_f32(a[3]) * bb[3]);
        *reinterpret_cast<uint2*>(static_cast<bf16_t*>(args.out) + (int64_t)r * N + f) = v;
      } else {
        const f32x4_t a = acc[0][i][j];
        *reinterpret_cast<float4*>(static_cast<float*>(args.out) + (int64_t)r * N + f) =
            make_float4(a[0], a[1], a[2], a[3]);
      }
    }
  }
}

template <int BF, int BT, int BK, int WAVES_F, int WAVES_T, bool DUAL>
hipError_t launch_cfg(const GemmArgs& args_in, int P, int E, hipStream_t stream) {
  using C = GemmCfg<BF, BT, BK, WAVES_F, WAVES_T, DUAL>;
  GemmArgs args = args_in;
  // sum_e ceil(n_e / BT) <= floor((P + E * (BT - 1)) / BT)
  args.max_tiles = (int)(((int64_t)P + (int64_t)E * (BT - 1)) / BT);
  if (args.max_tiles <= 0) return hipSuccess;
  const int tiles_f = args.N / BF;
  auto kern = grouped_gemm_bf16_kernel<BF, BT, BK, WAVES_F, WAVES_T, DUAL>;
  hipError_t err = allow_dynamic_lds(reinterpret_cast<const void*>(kern), C::kLdsBytes);
  if (err != hipSuccess) return err;
  dim3 grid((unsigned)args.max_tiles * (unsigned)tiles_f);
  hipLaunchKernelGGL(kern, grid, dim3(C::kThreads), C::kLdsBytes, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_swiglu_bf16(const void* x, const int32_t* sorted_token,
                                     const ExpertPtrs& W1, const ExpertPtrs& W3,
                                     const int32_t* offsets, int P, int d, int d_ff, int E,
                                     void* H, hipStream_t stream) {
  GemmArgs a{};
  a.A = static_cast<const bf16_t*>(x);
  a.gather = sorted_token;
  a.offsets = offsets;
  a.Wa = W1;
  a.Wb = W3;
  a.out = H;
  a.Kdim = d;
  a.N = d_ff;
  a.E = E;
  if (P <= 64) return launch_cfg<128, 16, 64, 4, 1, true>(a, P, E, stream);
  return launch_cfg<128, 128, 64, 2, 2, true>(a, P, E, stream);
}

hipError_t launch_expert_down_bf16(const void* H, const ExpertPtrs& W2, const int32_t* offsets,
                                   int P, int d, int d_ff, int E, float* O, hipStream_t stream) {
  GemmArgs a{};
  a.A = static_cast<const bf16_t*>(H);
  a.gather = nullptr;
  a.offsets = offsets;
  a.Wa = W2;
  a.Wb = W2;
  a.out = O;
  a.Kdim = d_ff;
  a.N = d;
  a.E = E;
  if (d % 256 == 0) {
    if (P <= 64) return launch_cfg<256, 16, 64, 4, 1, false>(a, P, E, stream);
    return launch_cfg<256, 128, 64, 2, 2, false>(a, P, E, stream);
  }
  if (P <= 64) return launch_cfg<128, 16, 64, 4, 1, false>(a, P, E, stream);
  return launch_cfg<128, 128, 64, 2, 2, false>(a, P, E, stream);
}

}  // namespace moe
