// Grouped bf16 matrix-core GEMMs for large batches (prefill), CDNA4 form.
//
// Same products as the other expert kernels ("从Mistral 7B到MoE模型Mixtral
// 8x7B的全面解析" (aiqianji.com) section 3.2.4, code block D): rows arrive
// expert-sorted, a workgroup owns one (token tile, feature tile) of one
// expert and finds it from the offsets on the device.
//
// Data path (gfx950):
//   * both operand tiles travel global -> LDS with global_load_lds_dwordx4
//     (each instruction lands 64 lanes x 16 bytes contiguously), no register
//     staging; a four-slot LDS ring keeps three k-stages in flight;
//   * the weight tile stays in its [k][feature] layout in LDS and the
//     matrix-core operand (8 consecutive k of one feature per lane) is read
//     with ds_read_b64_tr_b16: in each 16-lane group, lane i addresses 4
//     features of k-row (i / 4), and lane j receives element j % 4 of lanes
//     j / 4 + 4q, i.e. 4 consecutive k of one feature;
//   * 16-byte chunks are XOR-swizzled per row so the transposed reads and
//     the token-operand reads are free of LDS bank conflicts (the token
//     swizzle, chunk ^ (row / 2) mod 4 over 64-byte rows, is the one that
//     gfx950's bank-conflict counter reads as zero for the 16-row operand
//     read; (row / 4) mod 4 is 2-way conflicted there);
//   * each slot is its own __shared__ object and the k loop is unrolled over
//     the four slots, so the compiler can prove a slot's reads independent of
//     the loads in flight to the other slots; waits are explicit vmcnt counts
//     followed by a bare s_barrier;
//   * 256 weight columns x 256 tokens per workgroup (with W1/W3: 128 H
//     features of each), eight waves of 128 x 64 (two per SIMD),
//     v_mfma_f32_16x16x32_bf16 with fp32 accumulators; D is
//     [feature][token], so the epilogue writes 4 consecutive features per
//     lane (SiLU(a) * b fused for W1/W3);
//   * ping-pong: per k-stage a wave has a read phase (its LDS fragment
//     reads, then the stage's four load issues) and a matrix phase (its 32
//     matrix instructions), separated by barriers, and waves 4-7 run one
//     barrier behind waves 0-3, so on each SIMD one wave multiplies while
//     the other reads (3-4 % faster than all eight waves reading and then
//     multiplying together); the k loop is instantiated for both groups and
//     twice per group -- one straight block for tiles whose token groups are
//     all live, one that skips the groups lying wholly in the padding of an
//     expert's last tile;
//   * tile order: each XCD runs a contiguous range in which 4 feature tiles
//     are interleaved with the token tiles, so the ~32 workgroups it runs at
//     once share a few weight tiles and a few token tiles in its L2.
#include <type_traits>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void global_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBF = 256;       // weight columns per workgroup
constexpr int kBK = 32;        // k per stage
constexpr int kSlots = 4;      // LDS ring depth
constexpr int kWavesT = 4;     // waves along tokens (x 2 along weight columns)
constexpr int kGroupF = 4;     // feature tiles interleaved in the tile order
constexpr int kRowBytesW = kBF * 2;   // 512
constexpr int kRowBytesA = kBK * 2;   // 64

struct TiledArgs {
  const bf16_t* A;         // [rows, Kdim] activations
  const int32_t* gather;   // sorted_token, or null when A is already sorted
  const int32_t* offsets;  // [E + 1]
  ExpertPtrs Wa;
  ExpertPtrs Wb;
  void* out;               // H bf16 [P, N] (dual) or O fp32 [splits, P, N]
  int Kdim;
  int N;                   // output features (d_ff, or d)
  int E;
  int P;
  int max_tiles;
  int splits;              // K splits (one output slice each; 1 for W1/W3)
  int group_f;             // feature tiles interleaved in the tile order (divides N / feat)
};

// Chunk swizzles (16-byte chunks): weight rows hold 32 chunks, token rows 4.
__device__ __forceinline__ int swz_w(int r) { return 2 * (r & 3) + 8 * ((r >> 3) & 1); }
__device__ __forceinline__ int swz_a(int t) { return (t >> 1) & 3; }

__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((global_void_t*)src, (lds_void_t*)lds_dst, 16, 0, 0);
}

// s_waitcnt vmcnt(n) only (expcnt and lgkmcnt left at their maxima).
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) only.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

template <int BT, bool DUAL>
struct TiledCfg {
  static constexpr int kWaves = 2 * kWavesT;   // 2 along weight columns x 4 along tokens
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kWT = BT / kWavesT;     // tokens per wave
  static constexpr int kNJ = kWT / 16;
  static constexpr int kMI = 8;                // 128 weight columns per wave
  static constexpr int kSlotW = kBK * kRowBytesW;  // 16 KB
  static constexpr int kSlotA = BT * kRowBytesA;   // 16 KB at BT = 256
  static constexpr int kWInstr = kSlotW / 1024 / kWaves;  // per wave per stage
  static constexpr int kAInstr = kSlotA / 1024 / kWaves;
  static constexpr int kDmaPerStage = kWInstr + kAInstr;
  static constexpr int kFeat = DUAL ? kBF / 2 : kBF;
  static_assert(kSlotA % (1024 * kWaves) == 0 && kSlotW % (1024 * kWaves) == 0, "copy split");
};

template <int BT, bool DUAL>
__global__ __launch_bounds__(128 * kWavesT) void tiled_gemm_kernel(TiledArgs args) {
  using C = TiledCfg<BT, DUAL>;
  __shared__ __align__(1024) char sW0[C::kSlotW], sW1[C::kSlotW], sW2[C::kSlotW], sW3[C::kSlotW];
  __shared__ __align__(1024) char sA0[C::kSlotA], sA1[C::kSlotA], sA2[C::kSlotA], sA3[C::kSlotA];
  char* const sW[kSlots] = {sW0, sW1, sW2, sW3};
  char* const sA[kSlots] = {sA0, sA1, sA2, sA3};

  // Tile order.  Workgroup b runs on XCD b % 8; each XCD gets a contiguous
  // range of the order, in which group_f feature tiles are interleaved with
  // the token tiles (feature fastest), so the ~32 workgroups an XCD runs at
  // once span a few weight tiles and a few token tiles and both operands are
  // reused from that XCD's L2.
  const int G = gridDim.x;
  const int v = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
  const int tiles_f = args.N / C::kFeat;
  const int per_split = args.max_tiles * tiles_f;
  const int split = v / per_split;
  if (split >= args.splits) return;
  const int w = v % per_split;
  const int gf = args.group_f;
  const int ftile = (w / (gf * args.max_tiles)) * gf + w % gf;
  const int ttile = (w / gf) % args.max_tiles;
  int e, row_begin, row_end;
  if (!find_tile(args.offsets, args.E, BT, ttile, e, row_begin, row_end)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wf = wave & 1;
  const int wt = wave >> 1;
  const int64_t N = args.N;
  const int fbase = ftile * C::kFeat;
  (void)tid;

  // ---- copy assignment (fixed across k) ----
  // The weight slot holds kSub sub-tiles (W1 and W3 for the SwiGLU product)
  // of 32 k-rows x kSubCols features; one load instruction fills 1 KB, i.e.
  // 1024 / kRowB consecutive rows of one sub-tile, so its source matrix is
  // uniform and the address is a scalar base plus a 32-bit lane offset.
  constexpr int kSub = DUAL ? 2 : 1;
  constexpr int kSubCols = kBF / kSub;
  constexpr int kRowB = kSubCols * 2;          // bytes per LDS row of a sub-tile
  constexpr int kChunks = kRowB / 16;          // 16-byte chunks per row
  constexpr int kRowsPerInstr = 1024 / kRowB;
  uint32_t woff[C::kWInstr];
  const char* wbase[C::kWInstr];
#pragma unroll
  for (int u = 0; u < C::kWInstr; ++u) {
    const int ii = wave * C::kWInstr + u;                 // 0 .. 15
    const int sub = ii / (16 / kSub);
    const int r = (ii % (16 / kSub)) * kRowsPerInstr + lane / kChunks;
    const int c = (lane % kChunks) ^ swz_w(r);
    wbase[u] = static_cast<const char*>(sub == 0 ? args.Wa.p[e] : args.Wb.p[e]);
    woff[u] = (uint32_t)(((int64_t)r * N + fbase + 8 * c) * 2);
  }
  // token instruction u fills token rows 16*jj .. 16*jj+15 (jj = wave*kAInstr + u)
  uint32_t aoff[C::kAInstr];
#pragma unroll
  for (int u = 0; u < C::kAInstr; ++u) {
    const int jj = wave * C::kAInstr + u;
    const int t = 16 * jj + (lane >> 2);
    const int c = (lane & 3) ^ swz_a(t);
    const int r = min(row_begin + t, row_end - 1);   // rows past the segment: never stored
    const int64_t src_row = args.gather ? args.gather[r] : r;
    aoff[u] = (uint32_t)((src_row * args.Kdim + 8 * c) * 2);
  }
  const int64_t wstep = (int64_t)kBK * N * 2;   // bytes per stage along k
  const int astep = kBK * 2;
  const int ksplit = args.Kdim / args.splits;    // this split's k-range
  const char* abase = reinterpret_cast<const char*>(args.A) + (int64_t)split * ksplit * 2;
#pragma unroll
  for (int u = 0; u < C::kWInstr; ++u) wbase[u] += (int64_t)split * ksplit * N * 2;

  auto issue = [&](int stage, char* w_dst, char* a_dst) {
#pragma unroll
    for (int u = 0; u < C::kWInstr; ++u)
      dma16(wbase[u] + stage * wstep + woff[u], w_dst + (wave * C::kWInstr + u) * 1024);
#pragma unroll
    for (int u = 0; u < C::kAInstr; ++u)
      dma16(abase + stage * astep + aoff[u], a_dst + (wave * C::kAInstr + u) * 1024);
  };

  // ---- operand read offsets (bytes inside a slot) ----
  const int g = lane >> 4;
  const int j = lane & 15;
  // weight column group i of this wave: 16 columns of sub-tile sub from column n0
  int a_off[C::kMI][2];
#pragma unroll
  for (int i = 0; i < C::kMI; ++i) {
    int sub, n0;
    if (DUAL) {
      sub = i < 4 ? 0 : 1;
      n0 = wf * 64 + 16 * (i & 3);
    } else {
      sub = 0;
      n0 = wf * 128 + 16 * i;
    }
    const int n = n0 + 4 * (j & 3);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * g + 4 * h + (j >> 2);
      a_off[i][h] = sub * (kBK * kRowB) + r * kRowB + (((n >> 3) ^ swz_w(r)) << 4) + (n & 7) * 2;
    }
  }
  int b_off[C::kNJ];
#pragma unroll
  for (int jb = 0; jb < C::kNJ; ++jb) {
    const int t = wt * C::kWT + 16 * jb + j;
    b_off[jb] = t * kRowBytesA + ((g ^ swz_a(t)) << 4);
  }

  f32x4_t acc[C::kMI][C::kNJ];
#pragma unroll
  for (int i = 0; i < C::kMI; ++i)
#pragma unroll
    for (int jb = 0; jb < C::kNJ; ++jb) acc[i][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  bf16x8_t fa[C::kMI], fb[C::kNJ];
  auto read_fa = [&](int i, const char* w_src) {
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)((lds_char_t*)w_src + a_off[i][0]));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)((lds_char_t*)w_src + a_off[i][1]));
    const s16x4_t both[2] = {lo, hi};
    fa[i] = __builtin_bit_cast(bf16x8_t, both);
  };
  auto read_fb = [&](const char* a_src) {
#pragma unroll
    for (int jb = 0; jb < C::kNJ; ++jb)
      fb[jb] = *reinterpret_cast<const bf16x8_t*>(a_src + b_off[jb]);
  };
  auto read_frags = [&](const char* w_src, const char* a_src) {
    read_fb(a_src);
#pragma unroll
    for (int i = 0; i < C::kMI; ++i) read_fa(i, w_src);
  };
  // Token groups of the wave that lie wholly past the expert's segment (the
  // padding of its last tile) are skipped: their outputs are never stored.
  const int live_groups = min(C::kNJ, (row_end - row_begin - wt * C::kWT + 15) / 16);
  // FULL: every token group of the wave is live (all tiles but the last of
  // an expert), so the 32 matrix instructions form one straight block and a
  // load issue can go after every 8 of them; otherwise dead groups are skipped.
  auto mma = [&](auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    if constexpr (FULL) {
      // weight fragment outer: the first multiplies need only fb[] and fa[0]
#pragma unroll
      for (int i = 0; i < C::kMI; ++i)
#pragma unroll
        for (int jb = 0; jb < C::kNJ; ++jb)
          acc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[jb], acc[i][jb], 0, 0, 0);

    } else {
#pragma unroll
      for (int jb = 0; jb < C::kNJ; ++jb) {
        if (jb >= live_groups) break;
#pragma unroll
        for (int i = 0; i < C::kMI; ++i)
          acc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[jb], acc[i][jb], 0, 0, 0);
      }
    }
  };

  // nk is a multiple of kSlots (Kdim % 128 == 0 per split).  Every stage
  // issues the same number of loads -- past the end it reloads the last
  // k-stage into the free slot -- so a constant vmcnt marks "this stage has
  // landed" on every path, which keeps the compiler's own wait analysis exact.
  const int nk = ksplit / kBK;
#pragma unroll
  for (int s = 0; s < kSlots - 1; ++s) issue(s, sW[s], sA[s]);

  // Ping-pong: waves 0-3 (group A) and 4-7 (group B); with waves dealt to
  // the four SIMDs round-robin, each SIMD holds one wave of each group.  Each stage has a read phase (LDS reads, load
  // issues) and a matrix phase, separated by barriers; group B runs one
  // barrier behind group A, so on every SIMD one wave multiplies while the
  // other reads.  A workgroup barrier counts arrivals, so A's read barrier of
  // stage k pairs with B's matrix barrier of stage k-1, and B's read barrier
  // of stage k with A's matrix barrier of stage k.  Hence B's loads of stage
  // k+1 must have landed when B reaches its matrix barrier of stage k (A reads
  // stage k+1 right after it), and every wave's reads of a slot have returned
  // before the barrier that lets another wave refill it.
  const bool group_b = wave >= 4;
  constexpr int kLead = (kSlots - 2) * C::kDmaPerStage;
  if (group_b) {
    wait_vm<kLead>();                 // own stage 0 landed
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  auto k_loop = [&](auto full_tag, auto b_tag) {
    constexpr bool GB = decltype(b_tag)::value;
    for (int k0 = 0; k0 < nk; k0 += kSlots) {
#pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        const int kt = k0 + s;
        // A: own stage kt landed.  B: already true (waited before its last
        // matrix barrier); the no-op wait tells the compiler so.
        wait_vm<kLead>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(sW[s], sA[s]);
        __builtin_amdgcn_sched_barrier(0);
        issue(min(kt + kSlots - 1, nk - 1), sW[(s + kSlots - 1) % kSlots],
              sA[(s + kSlots - 1) % kSlots]);
        wait_lgkm0();                          // this wave's reads returned
        if constexpr (GB) wait_vm<kLead>();    // own stage kt+1 landed
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        mma(full_tag);
      }
    }
  };
  if (live_groups == C::kNJ) {
    if (group_b) k_loop(std::true_type{}, std::true_type{});
    else k_loop(std::true_type{}, std::false_type{});
  } else {
    if (group_b) k_loop(std::false_type{}, std::true_type{});
    else k_loop(std::false_type{}, std::false_type{});
  }
  if (!group_b) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();       // pairs with B's last matrix barrier
  }
  wait_vm<0>();  // no load may land in LDS after the workgroup ends

  // ---- epilogue: lane holds features f .. f+3 of token column j ----
  const int fq = g * 4;
#pragma unroll
  for (int jb = 0; jb < C::kNJ; ++jb) {
    const int r = row_begin + wt * C::kWT + jb * 16 + j;
    if (r >= row_end) continue;
    if constexpr (DUAL) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = fbase + wf * 64 + i * 16 + fq;
        const f32x4_t a = acc[i][jb];
        const f32x4_t bb = acc[i + 4][jb];
        uint2 v2;
        v2.x = pack_bf16x2(silu_f32(a[0]) * bb[0], silu_f32(a[1]) * bb[1]);
        v2.y = pack_bf16x2(silu_f32(a[2]) * bb[2], silu_f32(a[3]) * bb[3]);
        *reinterpret_cast<uint2*>(static_cast<bf16_t*>(args.out) + (int64_t)r * N + f) = v2;
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::kMI; ++i) {
        const int f = fbase + wf * 128 + i * 16 + fq;
        const f32x4_t a = acc[i][jb];
        float* o = static_cast<float*>(args.out) + ((int64_t)split * args.P + r) * N + f;
        *reinterpret_cast<float4*>(o) = make_float4(a[0], a[1], a[2], a[3]);
      }
    }
  }
}

template <int BT, bool DUAL>
hipError_t launch_tiled(const TiledArgs& in, int P, hipStream_t stream) {
  using C = TiledCfg<BT, DUAL>;
  TiledArgs a = in;
  a.max_tiles = (int)(((int64_t)P + (int64_t)a.E * (BT - 1)) / BT);
  if (a.max_tiles <= 0) return hipSuccess;
  const int tiles_f = a.N / C::kFeat;
  a.group_f = kGroupF;
  while (tiles_f % a.group_f != 0) --a.group_f;
  int64_t blocks = (int64_t)a.max_tiles * tiles_f * a.splits;
  blocks = (blocks + 7) / 8 * 8;  // whole XCD rounds for the remapped order
  hipLaunchKernelGGL((tiled_gemm_kernel<BT, DUAL>), dim3((unsigned)blocks),
                     dim3(C::kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool tiled_gemm_supported(int Kdim, int N, bool dual, int splits, int64_t a_rows) {
  // token-operand byte offsets are 32-bit per lane
  return splits >= 1 && Kdim % (kBK * kSlots * splits) == 0 && N % (dual ? kBF / 2 : kBF) == 0 &&
         a_rows * Kdim * 2 < (int64_t(1) << 32);
}

int tiled_gemm_tiles(int P, int E, int N, bool dual) {
  const int64_t mt = ((int64_t)P + (int64_t)E * 255) / 256;
  return (int)(mt * (N / (dual ? kBF / 2 : kBF)));
}

hipError_t launch_tiled_swiglu_bf16(const void* x, const int32_t* sorted_token,
                                    const ExpertPtrs& W1, const ExpertPtrs& W3,
                                    const int32_t* offsets, int P, int d, int d_ff, int E,
                                    void* H, hipStream_t stream) {
  TiledArgs a{};
  a.A = static_cast<const bf16_t*>(x);
  a.gather = sorted_token;
  a.offsets = offsets;
  a.Wa = W1;
  a.Wb = W3;
  a.out = H;
  a.Kdim = d;
  a.N = d_ff;
  a.E = E;
  a.P = P;
  a.splits = 1;
  return launch_tiled<256, true>(a, P, stream);
}

hipError_t launch_tiled_down_bf16(const void* H, const ExpertPtrs& W2, const int32_t* offsets,
                                  int P, int d, int d_ff, int E, int splits, float* O,
                                  hipStream_t stream) {
  TiledArgs a{};
  a.A = static_cast<const bf16_t*>(H);
  a.gather = nullptr;
  a.offsets = offsets;
  a.Wa = W2;
  a.Wb = W2;
  a.out = O;
  a.Kdim = d_ff;
  a.N = d;
  a.E = E;
  a.P = P;
  a.splits = splits;
  return launch_tiled<256, false>(a, P, stream);
}

}  // namespace moe
