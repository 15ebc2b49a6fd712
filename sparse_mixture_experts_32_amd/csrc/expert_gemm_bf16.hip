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

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// rows[r] holds 8 bf16 of row r (columns c = 0..7, two per dword); on return
// cols[c] holds 8 bf16 of column c (rows r = 0..7).
__device__ __forceinline__ void transpose8x8(const u32x4_t rows[8], u32x4_t cols[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      cols[2 * q][m] = perm_lo(rows[2 * m + 1][q], rows[2 * m][q]);
      cols[2 * q + 1][m] = perm_hi(rows[2 * m + 1][q], rows[2 * m][q]);
    }
  }
}

// BF weight columns (both matrices together when DUAL: the first BF/2 LDS rows
// hold W1 features, the last BF/2 the same W3 features) x BT tokens per
// workgroup, BK reduction depth per stage; four waves in a 2 x 2 grid, each
// owning (BF/2) x (BT/2).
template <int BF, int BT, int BK, bool DUAL>
struct GemmCfg {
  static constexpr int kThreads = 256;
  static constexpr int kWF = BF / 2;        // weight columns per wave
  static constexpr int kWT = BT / 2;        // tokens per wave
  static constexpr int kMI = kWF / 16;
  static constexpr int kNJ = kWT / 16;
  static constexpr int kStride = BK + 8;    // LDS row stride in bf16 (16-byte pad)
  static constexpr int kKB = BK / 8;        // 8-row blocks along k
  static constexpr int kWBlocks = kKB * (BF / 8);
  static constexpr int kWPerThread = (kWBlocks + kThreads - 1) / kThreads;
  static constexpr int kAChunks = BT * kKB;  // 16-byte chunks of the token tile
  static constexpr int kAPerThread = (kAChunks + kThreads - 1) / kThreads;
  static constexpr int kLdsW = BF * kStride;
  static constexpr int kLdsA = BT * kStride;
  static constexpr int kLdsBytes = 2 * (kLdsW + kLdsA) * 2;
  static constexpr int kFeat = DUAL ? BF / 2 : BF;  // output features per workgroup
  static_assert(kWF % 16 == 0 && kWT % 16 == 0, "wave tile");
  static_assert(!DUAL || kMI % 2 == 0, "dual wave tile");
  static_assert(BK % 32 == 0, "k step");
  // Uneven splits of the copy work need guards (small tiles only).
  static constexpr bool kWGuard = kWBlocks % kThreads != 0;
  static_assert(kAChunks % kThreads == 0, "token copy split");
};

template <int BF, int BT, int BK, bool DUAL>
__global__ __launch_bounds__(256) void grouped_gemm_bf16_kernel(GemmArgs args) {
  using C = GemmCfg<BF, BT, BK, DUAL>;
  extern __shared__ __align__(16) bf16_t lds[];

  // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of (feature tile, token tile) so the token tiles that
  // share a weight tile run together and hit in that XCD's L2.
  const int G = gridDim.x;
  const int v = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
  const int tiles_f = args.N / C::kFeat;
  const int ftile = v / args.max_tiles;
  const int ttile = v % args.max_tiles;
  if (ftile >= tiles_f) return;
  int e, row_begin, row_end;
  if (!find_tile(args.offsets, args.E, BT, ttile, e, row_begin, row_end)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wf = wave & 1;
  const int wt = wave >> 1;
  const int64_t N = args.N;
  const int fbase = ftile * C::kFeat;  // first output feature of the tile

  const bf16_t* Wm[2];
  Wm[0] = static_cast<const bf16_t*>(args.Wa.p[e]);
  Wm[1] = DUAL ? static_cast<const bf16_t*>(args.Wb.p[e]) : Wm[0];

  // Token rows this thread copies (fixed across k); rows past the segment
  // read the segment's last row (their outputs are never stored).
  // (row index, not pointer, to save registers; the chunk column is the same
  // for all of a thread's rows)
  int a_row[C::kAPerThread];
  const int a_kc = (tid % C::kKB) * 8;
#pragma unroll
  for (int i = 0; i < C::kAPerThread; ++i) {
    const int q = tid + i * C::kThreads;
    const int r = min(row_begin + q / C::kKB, row_end - 1);
    a_row[i] = args.gather ? args.gather[r] : r;
  }
  const bf16_t* a_base = args.A + a_kc;
  // Weight 8x8 blocks this thread copies: k-block fastest so that eight
  // consecutive lanes fill one 128-byte LDS row segment.
  const bf16_t* w_src[C::kWPerThread];
  int w_lds[C::kWPerThread];
#pragma unroll
  for (int i = 0; i < C::kWPerThread; ++i) {
    const int q = min(tid + i * C::kThreads, C::kWBlocks - 1);
    const int kb = q % C::kKB;
    const int fb = q / C::kKB;  // 8-column block inside the tile
    const int mat = DUAL ? fb / (BF / 16) : 0;
    const int col = DUAL ? (fb % (BF / 16)) * 8 : fb * 8;
    w_lds[i] = fb * 8 * C::kStride + kb * 8;
    w_src[i] = Wm[mat] + (int64_t)(kb * 8) * N + fbase + col;
  }

  u32x4_t wreg[C::kWPerThread][8];
  u32x4_t areg[C::kAPerThread];

  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::kWPerThread; ++i) {
      if (C::kWGuard && tid + i * C::kThreads >= C::kWBlocks) continue;
      const bf16_t* src = w_src[i] + (int64_t)k0 * N;
#pragma unroll
      for (int r = 0; r < 8; ++r) wreg[i][r] = *reinterpret_cast<const u32x4_t*>(src + r * N);
    }
#pragma unroll
    for (int i = 0; i < C::kAPerThread; ++i)
      areg[i] = *reinterpret_cast<const u32x4_t*>(a_base + (int64_t)a_row[i] * args.Kdim + k0);
  };

  auto store_tiles = [&](int buf) {
    bf16_t* sW = lds + buf * (C::kLdsW + C::kLdsA);
    bf16_t* sA = sW + C::kLdsW;
#pragma unroll
    for (int i = 0; i < C::kWPerThread; ++i) {
      if (C::kWGuard && tid + i * C::kThreads >= C::kWBlocks) continue;
      u32x4_t cols[8];
      transpose8x8(wreg[i], cols);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<u32x4_t*>(sW + w_lds[i] + c * C::kStride) = cols[c];
    }
#pragma unroll
    for (int i = 0; i < C::kAPerThread; ++i)
      *reinterpret_cast<u32x4_t*>(sA + ((tid + i * C::kThreads) / C::kKB) * C::kStride + a_kc) =
          areg[i];
  };

  // LDS row of the wave's i-th 16-row group of weight columns.
  auto wrow = [&](int i) {
    if (DUAL) {
      constexpr int half = C::kMI / 2;
      return i < half ? wf * (C::kWF / 2) + 16 * i : BF / 2 + wf * (C::kWF / 2) + 16 * (i - half);
    }
    return wf * C::kWF + 16 * i;
  };

  f32x4_t acc[C::kMI][C::kNJ];
#pragma unroll
  for (int i = 0; i < C::kMI; ++i)
#pragma unroll
    for (int j = 0; j < C::kNJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

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
        b[j] = *reinterpret_cast<const bf16x8_t*>(sA + (wt * C::kWT + j * 16 + lrow) * C::kStride +
                                                  ks + lk);
#pragma unroll
      for (int i = 0; i < C::kMI; ++i) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(sW + (wrow(i) + lrow) * C::kStride + ks + lk);
#pragma unroll
        for (int j = 0; j < C::kNJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) store_tiles(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds features f .. f+3 of token column (lane & 15).
  const int fq = (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < C::kNJ; ++j) {
    const int r = row_begin + wt * C::kWT + j * 16 + lrow;
    if (r >= row_end) continue;
    if constexpr (DUAL) {
#pragma unroll
      for (int i = 0; i < C::kMI / 2; ++i) {
        const int f = fbase + wf * (C::kWF / 2) + i * 16 + fq;
        const f32x4_t a = acc[i][j];
        const f32x4_t bb = acc[i + C::kMI / 2][j];
        uint2 v2;
        v2.x = pack_bf16x2(silu_f32(a[0]) * bb[0], silu_f32(a[1]) * bb[1]);
        v2.y = pack_bf16x2(silu_f32(a[2]) * bb[2], silu_f32(a[3]) * bb[3]);
        *reinterpret_cast<uint2*>(static_cast<bf16_t*>(args.out) + (int64_t)r * N + f) = v2;
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::kMI; ++i) {
        const int f = fbase + wf * C::kWF + i * 16 + fq;
        const f32x4_t a = acc[i][j];
        *reinterpret_cast<float4*>(static_cast<float*>(args.out) + (int64_t)r * N + f) =
            make_float4(a[0], a[1], a[2], a[3]);
      }
    }
  }
}

template <int BF, int BT, int BK, bool DUAL>
hipError_t launch_cfg(const GemmArgs& args_in, int P, int E, hipStream_t stream) {
  using C = GemmCfg<BF, BT, BK, DUAL>;
  GemmArgs args = args_in;
  // sum_e ceil(n_e / BT) <= floor((P + E * (BT - 1)) / BT)
  args.max_tiles = (int)(((int64_t)P + (int64_t)E * (BT - 1)) / BT);
  if (args.max_tiles <= 0) return hipSuccess;
  const int tiles_f = args.N / C::kFeat;
  auto kern = grouped_gemm_bf16_kernel<BF, BT, BK, DUAL>;
  hipError_t err = allow_dynamic_lds(reinterpret_cast<const void*>(kern), C::kLdsBytes);
  if (err != hipSuccess) return err;
  int64_t blocks = (int64_t)args.max_tiles * tiles_f;
  blocks = (blocks + 7) / 8 * 8;  // whole XCD rounds for the remapped order
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(C::kThreads), C::kLdsBytes, stream, args);
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
  if (P <= 0) return hipSuccess;
  if (d_ff % 128 == 0) return launch_cfg<256, 256, 64, true>(a, P, E, stream);
  if (d_ff % 64 == 0) return launch_cfg<128, 256, 64, true>(a, P, E, stream);
  return hipErrorInvalidValue;
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
  if (d % 256 == 0) return launch_cfg<256, 256, 64, false>(a, P, E, stream);
  if (d % 128 == 0) return launch_cfg<128, 256, 64, false>(a, P, E, stream);
  return launch_cfg<64, 256, 64, false>(a, P, E, stream);
}

}  // namespace moe
