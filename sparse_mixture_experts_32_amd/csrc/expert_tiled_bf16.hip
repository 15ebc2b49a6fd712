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
//     once share a few weight tiles and a few token tiles in its L2;
//   * where every expert holds about one token tile of rows, each weight
//     tile is read once and its copies are non-temporal (weights_read_once);
//     elsewhere so are those of any expert whose rows fit one token tile.
#include <algorithm>
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

constexpr int kBF = 256;       // weight columns per workgroup (W2; W1/W3 may take 512)
constexpr int kBK = 32;        // k per stage
constexpr int kSlots = 4;      // LDS ring depth
constexpr int kGroupF = 4;     // feature tiles interleaved in the tile order
// W1/W3 chooses the tile shape per expert (tiled_mixed_kernel) up to this
// average of rows per expert.  Against 256 x 256 tiles throughout, at Mixtral
// shape with 8 experts (one machine, 3 A/B pairs): 5.6, 7.3, 10.3, 11.2 and
// 5.7 % faster layers at 64, 128, 256, 384 and 512 tokens, level at 640 and
// 768.  (The 128 x 512 tile for every expert was 3.4 % slower at 512 tokens:
// three of the eight experts then hold more than 128 rows and would take a
// second, nearly empty tile.)
constexpr int kMixedRowsPerExpert = 192;
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
  // W2 with a tail split (null: none): partial sums of the tail pieces,
  // side_rows rows of [256] floats per piece, side_pieces pieces
  float* side;
  int side_rows;
  int side_pieces;
};

// A W2 launch with a tail split numbers the busy tiles densely, p = 0 ..
// nt-1 over the bt busy token tiles (group_f feature tiles interleaved with
// the token tiles, as the plain order).  The first Nw tiles, whole rounds of
// kTailRound workgroups, run over all of K and write O directly; the last nt
// - Nw (the partial round) are cut into S pieces along K, dispatched last,
// whose fp32 partial sums tail_fixup_kernel adds in piece order into O.  So
// the chip's last round holds S times as many, S times shorter workgroups
// instead of a few long ones, and O needs one slice.
constexpr int kTailRound = 256;   // compute units

__device__ __forceinline__ void tail_plan(const int32_t* offsets, int E, int tiles_f, int Kdim,
                                          int side_pieces, int& bt, int& nt, int& Nw, int& S) {
  bt = busy_tiles(offsets, E, 256);
  nt = bt * tiles_f;
  const int rem = nt % kTailRound;
  const int cap = min(kTailRound, side_pieces);
  const int quads = Kdim / (kBK * kSlots);   // a piece takes a multiple of kSlots stages
  S = 1;
  for (int s = 8; s >= 2; --s)
    if (quads % s == 0 && rem * s <= cap) {
      S = s;
      break;
    }
  Nw = S > 1 ? nt - rem : nt;
}

__device__ __forceinline__ void tail_tile(int p, int bt, int gf, int& ftile, int& ttile) {
  ftile = (p / (gf * bt)) * gf + p % gf;
  ttile = (p / gf) % bt;
}

// Feature tiles interleaved in the tile order: the largest divisor of
// tiles_f up to kGroupF.
int group_for(int tiles_f) {
  int g = kGroupF;
  while (tiles_f % g != 0) --g;
  return g;
}

// Chunk swizzles (16-byte chunks): weight rows hold 32 chunks, token rows 4.
__device__ __forceinline__ int swz_w(int r) { return 2 * (r & 3) + 8 * ((r >> 3) & 1); }
__device__ __forceinline__ int swz_a(int t) { return (t >> 1) & 3; }

__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((global_void_t*)src, (lds_void_t*)lds_dst, 16, 0, 0);
}

// The same copy with the non-temporal cache policy, for operands read once.
__device__ __forceinline__ void dma16_nt(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((global_void_t*)src, (lds_void_t*)lds_dst, 16, 0, 2);
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

// BT tokens x BF weight columns per workgroup: eight waves of 128 columns x
// 64 tokens, BF / 128 along the columns and the rest along the tokens.
template <int BT, bool DUAL, int BF>
struct TiledCfg {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kWavesF = BF / 128;     // along weight columns
  static constexpr int kWavesT = kWaves / kWavesF;
  static constexpr int kWT = BT / kWavesT;     // tokens per wave
  static constexpr int kNJ = kWT / 16;
  static constexpr int kMI = 8;                // 128 weight columns per wave
  static constexpr int kSlotW = kBK * BF * 2;      // 16 KB at BF = 256
  static constexpr int kSlotA = BT * kRowBytesA;   // 16 KB at BT = 256
  static constexpr int kInstrW = kSlotW / 1024;    // 1 KB load instructions per stage
  static constexpr int kWInstr = kInstrW / kWaves;  // per wave per stage
  static constexpr int kAInstr = kSlotA / 1024 / kWaves;
  static constexpr int kDmaPerStage = kWInstr + kAInstr;
  static constexpr int kFeat = DUAL ? BF / 2 : BF;
  static_assert(kWT == 64, "every wave holds 128 x 64");
  static_assert(kSlotA % (1024 * kWaves) == 0 && kSlotW % (1024 * kWaves) == 0, "copy split");
  static_assert(kSlots * (kSlotW + kSlotA) <= 160 * 1024, "LDS");
};

// One (token tile, feature tile, k-range) of a grouped product: the rows
// row_begin .. min(row_end, row_begin + BT) - 1 of expert e, features
// ftile * kFeat .., K slice `split` of `nsplit` (a tail piece of W2 when piece
// >= 0).  sW / sA: the four LDS slots of the weight and token operands.
template <int BT, bool DUAL, int BF, bool NT>
__device__ __forceinline__ void tile_body(const TiledArgs& args, char* const (&sW)[kSlots],
                                          char* const (&sA)[kSlots], int e, int row_begin,
                                          int row_end, int ftile, int split, int nsplit,
                                          int piece) {
  using C = TiledCfg<BT, DUAL, BF>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wf = wave % C::kWavesF;
  const int wt = wave / C::kWavesF;
  const int64_t N = args.N;
  const int fbase = ftile * C::kFeat;
  (void)tid;

  // ---- copy assignment (fixed across k) ----
  // The weight slot holds kSub sub-tiles (W1 and W3 for the SwiGLU product)
  // of 32 k-rows x kSubCols features; one load instruction fills 1 KB, i.e.
  // 1024 / kRowB consecutive rows of one sub-tile, so its source matrix is
  // uniform and the address is a scalar base plus a 32-bit lane offset.
  constexpr int kSub = DUAL ? 2 : 1;
  constexpr int kSubCols = BF / kSub;
  constexpr int kRowB = kSubCols * 2;          // bytes per LDS row of a sub-tile
  constexpr int kChunks = kRowB / 16;          // 16-byte chunks per row
  constexpr int kRowsPerInstr = 1024 / kRowB;
  uint32_t woff[C::kWInstr];
  const char* wbase[C::kWInstr];
#pragma unroll
  for (int u = 0; u < C::kWInstr; ++u) {
    const int ii = wave * C::kWInstr + u;                 // 0 .. kInstrW - 1
    const int sub = ii / (C::kInstrW / kSub);
    const int r = (ii % (C::kInstrW / kSub)) * kRowsPerInstr + lane / kChunks;
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
  const int ksplit = args.Kdim / nsplit;        // this split's k-range
  const char* abase = reinterpret_cast<const char*>(args.A) + (int64_t)split * ksplit * 2;
#pragma unroll
  for (int u = 0; u < C::kWInstr; ++u) wbase[u] += (int64_t)split * ksplit * N * 2;

  auto issue = [&](int stage, char* w_dst, char* a_dst) {
#pragma unroll
    for (int u = 0; u < C::kWInstr; ++u)
      if constexpr (NT)
        dma16_nt(wbase[u] + stage * wstep + woff[u], w_dst + (wave * C::kWInstr + u) * 1024);
      else
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
    } else if (piece >= 0) {
      // tail piece: fp32 partial sums of the tile, row r - row_begin
      float* dst = args.side + ((int64_t)piece * args.side_rows + (r - row_begin)) * BF;
#pragma unroll
      for (int i = 0; i < C::kMI; ++i) {
        const f32x4_t a = acc[i][jb];
        *reinterpret_cast<float4*>(dst + wf * 128 + i * 16 + fq) = make_float4(a[0], a[1], a[2], a[3]);
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

template <int BT, bool DUAL, int BF, bool NT>
__global__ __launch_bounds__(512) void tiled_gemm_kernel(TiledArgs args) {
  using C = TiledCfg<BT, DUAL, BF>;
  __shared__ __align__(1024) char sW0[C::kSlotW], sW1[C::kSlotW], sW2[C::kSlotW], sW3[C::kSlotW];
  __shared__ __align__(1024) char sA0[C::kSlotA], sA1[C::kSlotA], sA2[C::kSlotA], sA3[C::kSlotA];
  char* const sW[kSlots] = {sW0, sW1, sW2, sW3};
  char* const sA[kSlots] = {sA0, sA1, sA2, sA3};

  // Tile order.  Workgroup b runs on XCD b % 8; each XCD gets a contiguous
  // range of the order, in which group_f feature tiles are interleaved with
  // the token tiles (feature fastest), so the ~32 workgroups an XCD runs at
  // once span a few weight tiles and a few token tiles and both operands are
  // reused from that XCD's L2.
  const int tiles_f = args.N / C::kFeat;
  const int gf = args.group_f;
  int split = 0, nsplit = args.splits, ftile, ttile;
  int piece = -1;  // index of a tail piece in args.side, or -1
  if (!DUAL && args.side) {
    int bt, nt, Nw, S;
    tail_plan(args.offsets, args.E, tiles_f, args.Kdim, args.side_pieces, bt, nt, Nw, S);
    const int Gw = (Nw + 7) / 8 * 8;
    const int b = blockIdx.x;
    int p;
    if (b < Gw) {
      const int v = (b % 8) * (Gw / 8) + b / 8;
      if (v >= Nw) return;
      p = v;
      nsplit = 1;
    } else {
      piece = b - Gw;
      if (piece >= (nt - Nw) * S) return;
      p = Nw + piece / S;
      split = piece % S;
      nsplit = S;
    }
    tail_tile(p, bt, gf, ftile, ttile);
  } else {
    const int G = gridDim.x;
    const int v = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
    const int per_split = args.max_tiles * tiles_f;
    split = v / per_split;
    if (split >= args.splits) return;
    const int w = v % per_split;
    ftile = (w / (gf * args.max_tiles)) * gf + w % gf;
    ttile = (w / gf) % args.max_tiles;
  }
  int e, row_begin, row_end;
  if (!find_tile(args.offsets, args.E, BT, ttile, e, row_begin, row_end)) return;

  // An expert whose rows fit one token tile has each weight tile read once:
  // its copies are non-temporal even where the launch's are not.
  if (NT || args.offsets[e + 1] - args.offsets[e] <= BT)
    tile_body<BT, DUAL, BF, true>(args, sW, sA, e, row_begin, row_end, ftile, split, nsplit, piece);
  else
    tile_body<BT, DUAL, BF, false>(args, sW, sA, e, row_begin, row_end, ftile, split, nsplit, piece);
}

// W1/W3 with a tile shape per expert: experts of at most 128 rows take one
// 128 x 512 tile (256 features of each matrix) per feature tile, larger
// experts 256 x 256 tiles.  The units of each shape are numbered as the
// plain order numbers tiles (group_f feature tiles interleaved with the
// token tiles).  Workgroup b runs on XCD b % 8, and XCD x takes its equal
// share of the wide units first (the longer ones), then its share of the
// 256-row units, so the XCDs stay balanced and each reuses a few weight and
// token tiles from its L2.  The four 40 KB LDS slots hold either shape.  It
// runs only where weights_read_once holds; weight copies are non-temporal
// except for an expert of more than one 256-row tile (skewed routing), whose
// tiles share its weight tiles.
constexpr int kMixedSlot = 40 * 1024;

__global__ __launch_bounds__(512) void tiled_mixed_kernel(TiledArgs args) {
  __shared__ __align__(1024) char s0[kMixedSlot], s1[kMixedSlot], s2[kMixedSlot], s3[kMixedSlot];
  using CW = TiledCfg<128, true, 512>;
  using CS = TiledCfg<256, true, 256>;
  const int tiles_fw = args.N / CW::kFeat;
  const int tiles_fs = args.N / CS::kFeat;
  // wide experts (1 .. 128 rows) and 256-row token tiles of the others
  int nw = 0, ns = 0;
  for (int x = 0; x < args.E; ++x) {
    const int c = args.offsets[x + 1] - args.offsets[x];
    if (c > 0 && c <= 128) ++nw;
    else ns += (c + 255) / 256;
  }
  const int NW = nw * tiles_fw, NS = ns * tiles_fs;
  const int xcd = blockIdx.x % 8, l = blockIdx.x / 8;
  const int w0 = xcd * NW / 8, wn = (xcd + 1) * NW / 8 - w0;
  const int s0i = xcd * NS / 8, sn = (xcd + 1) * NS / 8 - s0i;
  const bool wide = l < wn;
  int u;
  if (wide) u = w0 + l;
  else if (l < wn + sn) u = s0i + (l - wn);
  else return;
  const int gf = args.group_f;   // divides tiles_fw and tiles_fs
  const int nt = wide ? nw : ns;
  const int ftile = (u / (gf * nt)) * gf + u % gf;
  int tt = (u / gf) % nt;        // the tt-th wide expert, or 256-row tile of the others
  int e = 0, row_begin = 0;
  for (; e < args.E; ++e) {
    const int b = args.offsets[e];
    const int c = args.offsets[e + 1] - b;
    const bool ew = c > 0 && c <= 128;
    if (wide && ew) {
      if (tt == 0) { row_begin = b; break; }
      --tt;
    } else if (!wide && !ew) {
      const int tiles = (c + 255) / 256;
      if (tt < tiles) { row_begin = b + 256 * tt; break; }
      tt -= tiles;
    }
  }
  if (e == args.E) return;   // not reached for a unit below NW + NS
  const int row_end = args.offsets[e + 1];
  if (wide) {
    char* const sW[kSlots] = {s0, s1, s2, s3};
    char* const sA[kSlots] = {s0 + CW::kSlotW, s1 + CW::kSlotW, s2 + CW::kSlotW, s3 + CW::kSlotW};
    tile_body<128, true, 512, true>(args, sW, sA, e, row_begin, row_end, ftile, 0, 1, -1);
  } else {
    char* const sW[kSlots] = {s0, s1, s2, s3};
    char* const sA[kSlots] = {s0 + CS::kSlotW, s1 + CS::kSlotW, s2 + CS::kSlotW, s3 + CS::kSlotW};
    if (row_end - args.offsets[e] <= 256)   // one token tile: weights read once
      tile_body<256, true, 256, true>(args, sW, sA, e, row_begin, row_end, ftile, 0, 1, -1);
    else
      tile_body<256, true, 256, false>(args, sW, sA, e, row_begin, row_end, ftile, 0, 1, -1);
  }
}

template <int BT, bool DUAL, int BF, bool NT>
hipError_t launch_tiled(const TiledArgs& in, int P, hipStream_t stream) {
  using C = TiledCfg<BT, DUAL, BF>;
  TiledArgs a = in;
  a.max_tiles = (int)(((int64_t)P + (int64_t)a.E * (BT - 1)) / BT);
  if (a.max_tiles <= 0) return hipSuccess;
  const int tiles_f = a.N / C::kFeat;
  a.group_f = group_for(tiles_f);
  int64_t blocks = (int64_t)a.max_tiles * tiles_f * a.splits;
  blocks = (blocks + 7) / 8 * 8;  // whole XCD rounds for the remapped order
  if (a.side) blocks += kTailRound;   // the tail pieces, after the whole tiles
  hipLaunchKernelGGL((tiled_gemm_kernel<BT, DUAL, BF, NT>), dim3((unsigned)blocks),
                     dim3(C::kThreads), 0, stream, a);
  return hipGetLastError();
}

// O rows of the tail tiles of a split W2 launch: the sum of the tile's S
// pieces in piece order.  A fixed grid of kFixupBlocks blocks, each reading
// the expert offsets into LDS and working out the tail plan once; items are
// (tail tile, 4 rows), a thread per 4 features, and a block takes items
// blockIdx.x + j gridDim.x four at a time, so that the loads of four items
// are in flight together.
constexpr int kFixupBlocks = 768;
constexpr int kFixupBatch = 4;

__global__ __launch_bounds__(256) void tail_fixup_kernel(const float* __restrict__ side,
                                                         int side_rows, int side_pieces,
                                                         const int32_t* __restrict__ offsets,
                                                         int E, int N, int Kdim, int group_f,
                                                         float* __restrict__ O) {
  constexpr int kRowsPerItem = 256 / (kBF / 4);
  __shared__ int32_t off[kMaxExperts + 1];
  if ((int)threadIdx.x <= E) off[threadIdx.x] = offsets[threadIdx.x];
  __syncthreads();
  const int tiles_f = N / kBF;
  int bt, nt, Nw, S;
  tail_plan(off, E, tiles_f, Kdim, side_pieces, bt, nt, Nw, S);
  if (S == 1) return;
  const int groups = (side_rows + kRowsPerItem - 1) / kRowsPerItem;
  const int items = (nt - Nw) * groups;
  const int sub = threadIdx.x / (kBF / 4);
  const int c = (threadIdx.x % (kBF / 4)) * 4;
  const int64_t piece_stride = (int64_t)side_rows * kBF;
  for (int i0 = blockIdx.x; i0 < items; i0 += kFixupBatch * gridDim.x) {
    float4 a[kFixupBatch];
    int64_t dst[kFixupBatch];
#pragma unroll
    for (int q = 0; q < kFixupBatch; ++q) {
      dst[q] = -1;
      const int item = i0 + q * gridDim.x;
      if (item >= items) continue;
      const int t = item / groups;   // tail tile
      const int i = (item % groups) * kRowsPerItem + sub;
      int ftile, ttile, e, rb, re;
      tail_tile(Nw + t, bt, group_f, ftile, ttile);
      if (!find_tile(off, E, 256, ttile, e, rb, re) || i >= min(256, re - rb)) continue;
      const float* src = side + ((int64_t)t * S * side_rows + i) * kBF + c;
      a[q] = *reinterpret_cast<const float4*>(src);
      for (int p = 1; p < S; ++p) {
        const float4 x = *reinterpret_cast<const float4*>(src + p * piece_stride);
        a[q].x += x.x; a[q].y += x.y; a[q].z += x.z; a[q].w += x.w;
      }
      dst[q] = (int64_t)(rb + i) * N + ftile * kBF + c;
    }
#pragma unroll
    for (int q = 0; q < kFixupBatch; ++q)
      if (dst[q] >= 0) *reinterpret_cast<float4*>(O + dst[q]) = a[q];
  }
}

}  // namespace

// Up to kMixedRowsPerExpert rows per expert on average, an expert's rows
// fill about one token tile, so each weight tile is read by one workgroup and
// the weight copies take the non-temporal cache policy (they would only push
// the token rows, which every feature tile re-reads, out of L2).  At Mixtral
// shape with 8 experts (one machine, 3 A/B rounds), against the default
// policy: layers 5.7, 4.5, 3.6 and 3.4 % faster at 128, 256, 512 and 768
// tokens, but 5.5 % slower at 1024 and 13 % slower at 4096, where token
// tiles of one expert share its weight tiles through L2.
bool weights_read_once(int64_t P, int E) {
  return P <= (int64_t)kMixedRowsPerExpert * E;
}

bool tiled_swiglu_mixed(int P, int E, int d_ff) {
  return d_ff % 256 == 0 && (int64_t)P <= (int64_t)kMixedRowsPerExpert * E;
}

size_t tiled_down_side_bytes(int P, int d, int d_ff) {
  // only where even the fewest busy token tiles P rows fill (one per 256)
  // make a whole round of W2 tiles; 256 pieces of min(256, P) rows x 256
  // fp32 features
  if (P <= 0 || !tiled_gemm_supported(d_ff, d, false, 1, P)) return 0;
  if ((int64_t)((P + 255) / 256) * (d / kBF) < kTailRound) return 0;
  return (size_t)kTailRound * std::min(256, P) * kBF * sizeof(float);
}

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
  // Experts of at most 128 rows take 128 tokens x 512 columns (256 features
  // of each matrix): each stage loads 32 KB of weights against 8 KB of tokens
  // instead of 16 against 16 (a compute unit's load rate is shared by both),
  // and the weight rows come in 512-byte segments instead of 256.
  if (tiled_swiglu_mixed(P, E, d_ff)) {
    const int tiles_fs = d_ff / TiledCfg<256, true, 256>::kFeat;
    a.group_f = group_for(tiles_fs / 2);   // divides both feature-tile counts
    // at most E wide experts of tiles_fs / 2 units, and the 256-row tiles of
    // the others (at most max_tiles) of tiles_fs units; 8 extra for the
    // XCD shares' rounding
    const int64_t max_tiles = ((int64_t)P + (int64_t)E * 255) / 256;
    const int64_t units = (int64_t)E * (tiles_fs / 2) + max_tiles * tiles_fs;
    const int64_t blocks = (units + 7) / 8 * 8 + 16;
    hipLaunchKernelGGL(tiled_mixed_kernel, dim3((unsigned)blocks), dim3(512), 0, stream, a);
    return hipGetLastError();
  }
  if (weights_read_once(P, E)) return launch_tiled<256, true, 256, true>(a, P, stream);
  return launch_tiled<256, true, 256, false>(a, P, stream);
}

hipError_t launch_tiled_down_bf16(const void* H, const ExpertPtrs& W2, const int32_t* offsets,
                                  int P, int d, int d_ff, int E, int splits, float* O,
                                  float* side, size_t side_bytes, hipStream_t stream) {
  TiledArgs a{};
  if (side && side_bytes > 0 && P > 0 && splits == 1) {
    a.side = side;
    a.side_rows = std::min(256, P);
    a.side_pieces =
        (int)std::min<size_t>(kTailRound, side_bytes / ((size_t)a.side_rows * kBF * 4));
    if (a.side_pieces < 2) a.side = nullptr;
  }
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
  if (weights_read_once(P, E)) return launch_tiled<256, false, 256, true>(a, P, stream);
  return launch_tiled<256, false, 256, false>(a, P, stream);
}

hipError_t launch_tiled_down_fixup(const float* side, size_t side_bytes, const int32_t* offsets,
                                   int P, int d, int d_ff, int E, float* O, hipStream_t stream) {
  if (!side || side_bytes == 0 || P <= 0) return hipSuccess;
  const int rows = std::min(256, P);
  const int pieces = (int)std::min<size_t>(kTailRound, side_bytes / ((size_t)rows * kBF * 4));
  if (pieces < 2) return hipSuccess;
  hipLaunchKernelGGL(tail_fixup_kernel, dim3(kFixupBlocks), dim3(256), 0, stream, side, rows,
                     pieces, offsets, E, d, d_ff, group_for(d / kBF), O);
  return hipGetLastError();
}

}  // namespace moe
