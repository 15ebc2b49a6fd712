// Weight-streaming grouped GEMMs for small batches (decode): every expert
// segment has at most 16*NJ rows, so the product is bound by reading each
// active expert's weights once from HBM.
//
// Same product as the LDS-tiled kernels ("从Mistral 7B到MoE模型Mixtral 8x7B
// 的全面解析" (aiqianji.com) section 3.2.4, code block D), organised for
// bandwidth:
//   * a wavefront owns 256 features and a k-range.  Every 16-byte load
//     instruction covers two 512-byte row segments: lanes 0-31 read 512
//     contiguous bytes of one weight row, lanes 32-63 the same columns eight
//     rows further down.  (Measured with a loads-only replica, two 512-byte
//     segments per instruction stream at ~6.9 TB/s, four 256-byte segments
//     at ~6.4 TB/s.)
//   * a k-step of 32 rows takes 16 loads per lane: rows 0-7 and 16-23 of the
//     step for lanes 0-31, 8-15 and 24-31 for lanes 32-63.  Each group of 8
//     loads is transposed in registers (v_perm_b32) into 8-k columns of one
//     feature; v_permlane16_swap then regroups the 16-lane rows so that one
//     register holds features 0-127 of the wave over four k-groups and the
//     other features 128-255.  Each is the M-side operand of
//     v_mfma_f32_16x16x32_bf16 (instruction c takes feature 8*i + c at
//     M-row i); no LDS round trip for the weights.  The k-groups sit in the
//     operand in the order 0, 16, 8, 24, and the token operand (16 rows x 8
//     k per lane, a 16-byte load of the gathered activation row, L2-resident)
//     follows the same order;
//   * loads for the next k-step are issued before the current step's
//     transposes and matrix instructions (two register stages).  The k loop is
//     straight-line (no data-dependent branch: padding rows of a token tile
//     load a real row), so the wait before a step covers only that step's
//     loads;
//   * a workgroup has eight waves (two per SIMD, one workgroup per compute
//     unit) and every wave streams one matrix.  The W2 product puts all
//     eight on W2, splitting the workgroup's k-range eight ways.  The W1/W3
//     product runs one of two ways: fused (stream_gemm_kernel) -- waves 0-3
//     on W1, 4-7 on W3, each four splitting the whole of K, and H =
//     bf16(SiLU(a) * b) stored by the epilogue -- or per matrix
//     (stream_sk_kernel) -- one matrix at a time over a persistent grid that
//     gives every compute unit the same number of weight rows, fp32 partial
//     sums of a and b stored for swiglu_finish_kernel (its own launch), which
//     adds the slices in order and applies SwiGLU.  The waves' partial
//     products meet in LDS and are added in wave order;
//   * K splits write fp32 partial sums to separate slices (non-temporal
//     stores), summed later in slice order, so results are deterministic.
//     Every partial byte written costs streaming time -- a loads-only
//     replica slowed by 13 % when its workgroups also wrote 1.6 % as many
//     bytes as they read -- so the launch form and split count are chosen
//     per batch size by how the workgroups fill the chip (pick_launch).
#include <cmath>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

struct StreamArgs {
  // W1/W3 launches of moe_forward: the routing table, from which every
  // workgroup builds the dispatch tables itself (at most 64 pairs) and
  // workgroup 0 writes them to offsets / gather / pos_out for the later
  // kernels; null when the caller passes the tables (gather, offsets)
  const int32_t* topk_idx;
  int K;
  int32_t* pos_out;
  const bf16_t* A;         // [rows, Kdim] activations
  const int32_t* gather;   // sorted_token for gathered rows, else null
  const int32_t* offsets;  // [E + 1]
  ExpertPtrs Wa;
  ExpertPtrs Wb;
  bf16_t* H;               // H of the fused W1/W3 launch
  float* part;             // [splits][slices][P][N] partial sums otherwise
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
// the 8 k-values of feature c.
__device__ __forceinline__ u32x4_t column(const u32x4_t* rows, int c) {
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
  return v;
}

// Buffer resource word 3 of the gfx9 family (32-bit data format, so untyped
// loads return data), and the cache-policy bit of a non-temporal load.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNonTemporal = 2;

constexpr int kWaves = 8;           // waves per workgroup (two per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kFeat = kStreamFeat;  // features per workgroup (and per wave)
// The launch choice (pick_launch) counts rounds of workgroups over the
// chip's 256 compute units.  Measured at 1-32 tokens (MI355X, every split
// count timed): a single round that fills at least ~55 % of the compute
// units beats more, shorter workgroups; without one, an unsplit product of
// at least 1.7 rounds (no partial sums, no finish launch) beats splitting,
// and otherwise about three rounds do best.  For Mixtral's shapes at 1, 2,
// 4, 8, 16, 32 tokens this gives W1/W3 per matrix, fused, per matrix, per
// matrix, fused, fused (the per-matrix form then runs over its persistent
// grid); W2 with 7, 4, 2, 2, 2, 2 splits.
constexpr double kComputeUnits = 256;
constexpr int kLoads = 16;          // 16-byte loads per lane per k-step of 32

// What a launch streams:
//   kDown:      one matrix (W2); partial sums to O slices.
//   kFused:     W1 and W3 in every workgroup (waves 0-3 / 4-7), no K split;
//               H = bf16(SiLU(a) * b) in the epilogue.
// (The per-matrix W1/W3 form is stream_sk_kernel below.)
enum StreamMode { kDown = 0, kFused = 1 };

template <int NJ, int MODE>
struct StreamCfg {
  static constexpr int kSlices = MODE == kDown ? 1 : 2;   // partial slices per split
  static constexpr int kMatsWG = MODE == kFused ? 2 : 1;  // matrices inside a workgroup
  static constexpr int kKParts = kWaves / kMatsWG;        // waves sharing one matrix
};

constexpr int kStreamMaxPairs = 64;   // the streaming plan takes T * K <= 64

// Workgroup 0 of a W1/W3 launch that built the dispatch tables writes them
// out for the finish, W2 and combine kernels (and for the caller).
__device__ __forceinline__ void publish_route(const StreamArgs& a, const int32_t* off,
                                              const int32_t* tok, const int32_t* pos) {
  const int t = threadIdx.x;
  if (t <= a.E) const_cast<int32_t*>(a.offsets)[t] = off[t];
  if (t < off[a.E]) const_cast<int32_t*>(a.gather)[t] = tok[t];
  if (t < a.P) a.pos_out[t] = pos[t];
}

// One k-step of 32 rows: the 16 loaded weight registers w are transposed
// into MFMA operands and multiplied with the token operand b.
//   t: k-rows 0-7 (lanes 0-31) / 8-15 (lanes 32-63); u: 16-23 / 24-31.
//   Lanes 0-15 and 32-47 hold features 0-127, lanes 16-31 and 48-63
//   features 128-255.
template <int NJ>
__device__ __forceinline__ void mma_step(const u32x4_t (&w)[kLoads], const u32x4_t (&b)[NJ],
                                         f32x4_t (&acc)[2][8][NJ]) {
  bf16x8_t bo[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) bo[j] = __builtin_bit_cast(bf16x8_t, b[j]);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const u32x4_t t = column(w, c);
    const u32x4_t u = column(w + 8, c);
    u32x4_t lo, hi;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const auto r = __builtin_amdgcn_permlane16_swap(t[v], u[v], false, false);
      lo[v] = r[0];  // rows t0, u0, t2, u2: features 0-127, k-groups 0, 16, 8, 24
      hi[v] = r[1];  // rows t1, u1, t3, u3: features 128-255, same k-groups
    }
    const bf16x8_t opl = __builtin_bit_cast(bf16x8_t, lo);
    const bf16x8_t oph = __builtin_bit_cast(bf16x8_t, hi);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      acc[0][c][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opl, bo[j], acc[0][c][j], 0, 0, 0);
      acc[1][c][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oph, bo[j], acc[1][c][j], 0, 0, 0);
    }
    // one column at a time: forming all eight operands first would hold
    // 64 more registers
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int NJ, int MODE>
__global__ __launch_bounds__(kThreads) void stream_gemm_kernel(StreamArgs a) {
  using C = StreamCfg<NJ, MODE>;
  constexpr int MW = C::kMatsWG;
  // one feature half (8 accumulators per token tile) of every wave
  __shared__ f32x4_t red[kWaves * 8 * NJ * 64];

  const int tiles_f = a.N / kFeat;
  int bid = blockIdx.x;
  const int ftile = bid % tiles_f;
  bid /= tiles_f;
  const int s = bid % a.splits;
  const int ttile = bid / a.splits;
  const int splits = a.splits;
  // dispatch tables: built here from the routing table, or the caller's
  __shared__ int32_t sh_off[kMaxExperts + 1];
  __shared__ int32_t sh_tok[kStreamMaxPairs];
  __shared__ int32_t sh_pos[kStreamMaxPairs];
  const int32_t* offsets = a.offsets;
  const int32_t* gather = a.gather;
  if (a.topk_idx) {
    if (threadIdx.x < 64) small_route(a.topk_idx, a.P, a.K, a.E, sh_off, sh_tok, sh_pos);
    __syncthreads();
    if (blockIdx.x == 0) publish_route(a, sh_off, sh_tok, sh_pos);
    offsets = sh_off;
    gather = sh_tok;
  }
  int e, row_begin, row_end;
  if (!find_tile(offsets, a.E, 16 * NJ, ttile, e, row_begin, row_end)) return;
  e = __builtin_amdgcn_readfirstlane(e);
  row_begin = __builtin_amdgcn_readfirstlane(row_begin);
  row_end = __builtin_amdgcn_readfirstlane(row_end);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mat = wave / C::kKParts;
  const int kpart = wave % C::kKParts;
  const int f0 = ftile * kFeat;
  const int kc = a.Kdim / splits;
  const int kw = kc / C::kKParts;
  const int kbeg = s * kc + kpart * kw;
  const int nsteps = kw / 32;
  const int64_t N = a.N;
  const int64_t row_bytes = N * 2;

  // Token operand: lane group g (16 lanes) carries k-group {0, 16, 8, 24}[g]
  // of the step, matching the weight operand after the lane swap.  Padding
  // rows (r >= row_end) read the tile's last row: their products land in
  // output columns that are never stored.
  const int kofs = 8 * ((lane >> 4) >> 1) + 16 * ((lane >> 4) & 1);
  int64_t src_row[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int r = min(row_begin + j * 16 + (lane & 15), row_end - 1);
    src_row[j] = gather ? gather[r] : r;
  }

  // Weight loads are buffer loads: a k-step's 32 rows as one resource (base
  // and size in scalar registers), the row offset in a scalar register, one
  // 32-bit per-lane offset.  The resource of the step after the last has
  // size 0, so the loop's final prefetch returns zeros without touching
  // memory and the loop needs no peeled tail.
  char* wrow = const_cast<char*>(reinterpret_cast<const char*>(mat == 0 ? a.Wa.p[e] : a.Wb.p[e])) +
               ((int64_t)kbeg * N + f0) * 2;
  const int lane_off = (lane >> 5) * 8 * (int)row_bytes + (lane & 31) * 16;

  f32x4_t acc[2][8][NJ];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[h][c][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t w0[kLoads], w1[kLoads];
  u32x4_t b0[NJ], b1[NJ];
  const bf16_t* bsrc[NJ];

  auto load_w = [&](u32x4_t (&w)[kLoads], int step) {
    const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
        wrow + (int64_t)step * 32 * row_bytes, (short)0, step < nsteps ? 32 * (int)row_bytes : 0,
        kBufferWord3);
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int row = (r & 7) + 16 * (r >> 3);
      w[r] = __builtin_amdgcn_raw_buffer_load_b128(res, lane_off, row * (int)row_bytes, kNonTemporal);
    }
  };
  auto load_b = [&](u32x4_t (&b)[NJ], int step) {
    const int st = min(step, nsteps - 1);  // past the end: reread the last step (unused)
#pragma unroll
    for (int j = 0; j < NJ; ++j) b[j] = *reinterpret_cast<const u32x4_t*>(bsrc[j] + st * 32);
    // keep the issue here: hoisting the next compute above these loads
    // would make its wait cover them too
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute = [&](const u32x4_t (&w)[kLoads], const u32x4_t (&b)[NJ]) {
    mma_step<NJ>(w, b, acc);
  };

  // The first weight loads need only the expert; the token rows wait for
  // the gather indices.
  load_w(w0, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NJ; ++j) bsrc[j] = a.A + src_row[j] * a.Kdim + kbeg + kofs;
  load_b(b0, 0);
  // Two register stages: the loads of step i+1 are in flight while step i
  // computes (nsteps is even).
  for (int i = 0; i < nsteps; i += 2) {
    load_w(w1, i + 1);
    load_b(b1, i + 1);
    compute(w0, b0);
    load_w(w0, i + 2);
    load_b(b0, i + 2);
    compute(w1, b1);
  }

  // Epilogue, one feature half at a time.  Thread t produces 8 consecutive
  // features (c = 0..7) of one token for every (j, source lane L, q) --
  // NJ*256 outputs over the workgroup's threads.
  const float* redf = reinterpret_cast<const float*>(red);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h) __syncthreads();  // the first half's reads are done
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int j = 0; j < NJ; ++j) red[((wave * 8 + c) * NJ + j) * 64 + lane] = acc[h][c][j];
    __syncthreads();
    for (int o = threadIdx.x; o < NJ * 256; o += kThreads) {
      const int L = o & 63;
      const int q = (o >> 6) & 3;
      const int j = o >> 8;
      const int r = row_begin + j * 16 + (L & 15);
      if (r >= row_end) continue;
      const int f = f0 + 128 * h + 8 * (4 * (L >> 4) + q);
      // matrix m of the workgroup is the sum of waves m*kKParts ..
      // m*kKParts + kKParts - 1, in order
      float sum[MW][8];
#pragma unroll
      for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float t = redf[(((m * C::kKParts * 8 + c) * NJ + j) * 64 + L) * 4 + q];
#pragma unroll
          for (int w = 1; w < C::kKParts; ++w)
            t += redf[((((m * C::kKParts + w) * 8 + c) * NJ + j) * 64 + L) * 4 + q];
          sum[m][c] = t;
        }
      if (MODE == kFused) {
        uint4 hv;
        hv.x = pack_bf16x2(silu_f32(sum[0][0]) * sum[MW - 1][0], silu_f32(sum[0][1]) * sum[MW - 1][1]);
        hv.y = pack_bf16x2(silu_f32(sum[0][2]) * sum[MW - 1][2], silu_f32(sum[0][3]) * sum[MW - 1][3]);
        hv.z = pack_bf16x2(silu_f32(sum[0][4]) * sum[MW - 1][4], silu_f32(sum[0][5]) * sum[MW - 1][5]);
        hv.w = pack_bf16x2(silu_f32(sum[0][6]) * sum[MW - 1][6], silu_f32(sum[0][7]) * sum[MW - 1][7]);
        *reinterpret_cast<uint4*>(a.H + (int64_t)r * N + f) = hv;
      } else {
#pragma unroll
        for (int m = 0; m < MW; ++m) {
          const int slice = s * C::kSlices + m;
          f32x4_t* dst = reinterpret_cast<f32x4_t*>(a.part + ((int64_t)slice * a.P + r) * N + f);
          __builtin_nontemporal_store(f32x4_t{sum[m][0], sum[m][1], sum[m][2], sum[m][3]}, dst);
          __builtin_nontemporal_store(f32x4_t{sum[m][4], sum[m][5], sum[m][6], sum[m][7]}, dst + 1);
        }
      }
    }
  }
}

// ---- per-matrix W1/W3 product over a persistent grid (stream-K) ----
//
// Work units are (busy token tile, feature tile of 256, matrix), numbered
// u = (tile * tiles_f + ftile) * 2 + matrix, each K = Kdim rows long and cut
// into chunks of kChunkRows rows (one k-step per wave).  With G = kSkGrid
// workgroups (one per compute unit on 7/8 of the compute units):
//   * U >= G units: workgroup w takes chunks [w C / G, (w+1) C / G) of the
//     C = U * (Kdim / kChunkRows) chunks in unit order, so every workgroup
//     streams the same number of weight bytes (to one chunk: for
//     Mixtral's shapes at 8 tokens, 56 chunks each) and no round of
//     workgroups is left nearly empty.  A unit is cut at most once; its head
//     piece goes to partial-sum slice 0, its tail to slice 1.
//   * U < G: every unit is cut into the same number s of pieces (the largest
//     power of two with U s <= G dividing the chunk count), piece i to
//     slice i.
// Inside a piece the eight waves split its rows evenly (one chunk's k-step
// each per chunk) and their partial products meet in LDS in wave order.
// The weight and token loads of the next piece's first k-step are issued
// before the current piece's epilogue, and the epilogue synchronises the
// waves through LDS only, so those loads stay in flight across it.
constexpr int kChunkRows = 32 * kWaves;
// Persistent workgroups of the stream-K launch.  Measured at Mixtral shape
// with 8 tokens (one machine, 3 A/B rounds each): 224 workgroups stream the
// W1/W3 weights 0.7-1 % faster than 256 (both divide Mixtral's chunk counts,
// busy experts x 1792, evenly), 240 (uneven shares) 0.3 % slower than 256,
// 168 and 112 8 % and 37 % slower.
constexpr int kSkGrid = 224;

__device__ __forceinline__ int sk_small_split(int U, int G, int cpu) {
  int s = 1;
  while (cpu % (2 * s) == 0 && (int64_t)U * 2 * s <= G) s *= 2;
  return s;
}

// Whether unit u of the stream-K layout (U >= G) is cut by a workgroup
// boundary: the boundaries are floor(w C / G); the owner of the unit's first
// chunk is the largest w with floor(w C / G) <= u cpu.
__device__ __forceinline__ bool sk_unit_split(int64_t u, int64_t C, int G, int cpu) {
  const int64_t c = u * cpu;
  const int64_t w0 = ((c + 1) * G + C - 1) / C - 1;
  return w0 + 1 < G && ((w0 + 1) * C) / G < c + cpu;
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__global__ __launch_bounds__(kThreads) void stream_sk_kernel(StreamArgs a) {
  constexpr int NJ = 1;
  __shared__ f32x4_t red[kWaves * 8 * NJ * 64];
  // the routing tables of the batch (at most 64 pairs), read once: later
  // reads come from LDS, not from memory the kernel also writes
  __shared__ int32_t sh_off[kMaxExperts + 1];
  __shared__ int32_t sh_tok[kStreamMaxPairs];
  if (a.topk_idx) {
    __shared__ int32_t sh_pos[kStreamMaxPairs];
    if (threadIdx.x < 64) small_route(a.topk_idx, a.P, a.K, a.E, sh_off, sh_tok, sh_pos);
    __syncthreads();
    if (blockIdx.x == 0) publish_route(a, sh_off, sh_tok, sh_pos);
  } else {
    if ((int)threadIdx.x <= a.E) sh_off[threadIdx.x] = a.offsets[threadIdx.x];
    if ((int)threadIdx.x < a.P) sh_tok[threadIdx.x] = a.gather[threadIdx.x];
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles_f = a.N / kFeat;
  const int G = gridDim.x;
  const int w = blockIdx.x;
  const int cpu = a.Kdim / kChunkRows;
  const int U = busy_tiles(sh_off, a.E, 16) * tiles_f * 2;
  int64_t c_beg, c_end;
  int small_slice = -1;
  if (U >= G) {
    const int64_t C = (int64_t)U * cpu;
    c_beg = (int64_t)w * C / G;
    c_end = (int64_t)(w + 1) * C / G;
  } else {
    const int s = sk_small_split(U, G, cpu);
    if (w >= U * s) return;
    const int per = cpu / s;
    small_slice = w % s;
    c_beg = (int64_t)(w / s) * cpu + small_slice * per;
    c_end = c_beg + per;
  }
  const int64_t N = a.N;
  const int64_t row_bytes = N * 2;
  const int lane_off = (lane >> 5) * 8 * (int)row_bytes + (lane & 31) * 16;
  const int kofs = 8 * ((lane >> 4) >> 1) + 16 * ((lane >> 4) & 1);

  struct Piece {
    const char* wbase;      // this wave's first weight row of the piece
    const bf16_t* bsrc;     // this lane's token row at the wave's first k
    int nsteps;             // k-steps of 32 rows per wave, one per chunk (0: no piece)
    int row_begin, row_end, f0, mat, slice;
    int64_t next;           // first chunk after the piece
  };
  auto make_piece = [&](int64_t c) {
    Piece p;
    const int64_t u = c / cpu;
    const int pc0 = (int)(c - u * cpu);
    const int pc1 = (int)min((int64_t)cpu, c_end - u * cpu);
    p.mat = (int)(u & 1);
    const int ftile = (int)((u >> 1) % tiles_f);
    const int bt = (int)((u >> 1) / tiles_f);
    int e = 0, rb = 0, re = 1;
    find_tile(sh_off, a.E, 16, bt, e, rb, re);
    p.row_begin = __builtin_amdgcn_readfirstlane(rb);
    p.row_end = __builtin_amdgcn_readfirstlane(re);
    e = __builtin_amdgcn_readfirstlane(e);
    p.f0 = ftile * kFeat;
    p.slice = small_slice >= 0 ? small_slice : (pc0 == 0 ? 0 : 1);
    const int kw = (pc1 - pc0) * (kChunkRows / kWaves);
    const int kbeg = pc0 * kChunkRows + wave * kw;
    p.nsteps = kw / 32;
    p.wbase = reinterpret_cast<const char*>(p.mat == 0 ? a.Wa.p[e] : a.Wb.p[e]) +
              ((int64_t)kbeg * N + p.f0) * 2;
    const int r = min(p.row_begin + (lane & 15), p.row_end - 1);
    p.bsrc = a.A + (int64_t)sh_tok[r] * a.Kdim + kbeg + kofs;
    p.next = u * cpu + pc1;
    return p;
  };

  f32x4_t acc[2][8][NJ];
  u32x4_t w0[kLoads], w1[kLoads];
  u32x4_t b0[NJ], b1[NJ];

  // weight rows of k-step `step` of a piece: a zero-size resource when the
  // piece is empty, so the loads return zeros without a memory access.  The
  // address and size are wave-uniform, but the compiler cannot see it through
  // the loop-carried piece and would wrap every load in a loop over distinct
  // resources; readfirstlane puts the resource in scalar registers.
  auto load_w = [&](u32x4_t (&wr)[kLoads], const char* base, int step, bool live) {
    const uint64_t addr = reinterpret_cast<uint64_t>(base) + (uint64_t)step * 32 * row_bytes;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    const int size = __builtin_amdgcn_readfirstlane(live ? 32 * (int)row_bytes : 0);
    const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<char*>(((uint64_t)hi << 32) | lo), (short)0, size, kBufferWord3);
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int row = (r & 7) + 16 * (r >> 3);
      wr[r] = __builtin_amdgcn_raw_buffer_load_b128(res, lane_off, row * (int)row_bytes,
                                                    kNonTemporal);
    }
  };
  auto load_b = [&](u32x4_t (&b)[NJ], const bf16_t* src) {
    b[0] = *reinterpret_cast<const u32x4_t*>(src);
    __builtin_amdgcn_sched_barrier(0);
  };

  Piece cur = make_piece(c_beg);
  load_w(w0, cur.wbase, 0, true);
  __builtin_amdgcn_sched_barrier(0);
  load_b(b0, cur.bsrc);
  while (true) {
    Piece nxt = cur;
    nxt.nsteps = 0;
    if (cur.next < c_end) nxt = make_piece(cur.next);
    const bool more = nxt.nsteps > 0;
    // past the last piece the token loads reread the current piece's last step
    const bf16_t* b_after = more ? nxt.bsrc : cur.bsrc + (cur.nsteps - 1) * 32;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[h][c][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Steps go in pairs; after an odd count the second of the last pair
    // loads zeros (zero-size resource) against the piece's last token step,
    // so it adds exactly nothing and reads no memory past the piece.
    for (int i = 0; i < cur.nsteps; i += 2) {
      load_w(w1, cur.wbase, i + 1, i + 1 < cur.nsteps);
      load_b(b1, cur.bsrc + min(i + 1, cur.nsteps - 1) * 32);
      mma_step<NJ>(w0, b0, acc);
      // k-step i + 2: this piece's, or the next piece's first
      const bool inside = i + 2 < cur.nsteps;
      load_w(w0, inside ? cur.wbase : nxt.wbase, inside ? i + 2 : 0, inside || more);
      load_b(b0, inside ? cur.bsrc + (i + 2) * 32 : b_after);
      mma_step<NJ>(w1, b1, acc);
    }

    // epilogue: the waves' partial products meet in LDS, added in wave
    // order; one feature half at a time
    const float* redf = reinterpret_cast<const float*>(red);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h) lds_barrier();  // the first half's reads are done
#pragma unroll
      for (int c = 0; c < 8; ++c) red[(wave * 8 + c) * 64 + lane] = acc[h][c][0];
      lds_barrier();
      for (int o = threadIdx.x; o < 256; o += kThreads) {
        const int L = o & 63;
        const int q = (o >> 6) & 3;
        const int r = cur.row_begin + (L & 15);
        if (r >= cur.row_end) continue;
        const int f = cur.f0 + 128 * h + 8 * (4 * (L >> 4) + q);
        float sum[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float t = redf[((c * 64) + L) * 4 + q];
#pragma unroll
          for (int v = 1; v < kWaves; ++v) t += redf[(((v * 8 + c) * 64) + L) * 4 + q];
          sum[c] = t;
        }
        const int slice = cur.slice * 2 + cur.mat;
        f32x4_t* dst = reinterpret_cast<f32x4_t*>(a.part + ((int64_t)slice * a.P + r) * N + f);
        __builtin_nontemporal_store(f32x4_t{sum[0], sum[1], sum[2], sum[3]}, dst);
        __builtin_nontemporal_store(f32x4_t{sum[4], sum[5], sum[6], sum[7]}, dst + 1);
      }
    }
    lds_barrier();  // before the next piece's epilogue writes the LDS again
    if (!more) break;
    cur = nxt;
  }
}

// H[r][f] = bf16(SiLU(a) * b), a and b the sums of their matrix's partial
// slices in slice order: the slices stream_sk_kernel wrote for the unit of
// (r, f), i.e. one, or two for a unit cut by a workgroup boundary, or the s
// equal pieces when there are fewer units than workgroups.  Rows past the
// last expert segment belong to no unit and are left alone.
__global__ __launch_bounds__(256) void swiglu_finish_kernel(const float* __restrict__ part,
                                                            const int32_t* __restrict__ offsets,
                                                            int E, int P, int N, int Kdim, int G,
                                                            bf16_t* __restrict__ H) {
  const int tiles_f = N / kFeat;
  const int U = busy_tiles(offsets, E, 16) * tiles_f * 2;
  const int cpu = Kdim / kChunkRows;
  const int s_small = U < G ? sk_small_split(U, G, cpu) : 0;
  const int64_t C = (int64_t)U * cpu;
  const int64_t n4 = (int64_t)P * N / 4;
  const int64_t slice = (int64_t)P * N;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n4;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(g / (N / 4));
    const int f = (int)(g % (N / 4)) * 4;
    int bt = 0, e = 0;
    for (; e < E; ++e) {
      const int lo = offsets[e], hi = offsets[e + 1];
      if (r < hi) {
        bt += (r - lo) / 16;
        break;
      }
      bt += (hi - lo + 15) / 16;
    }
    if (e == E) continue;
    const int64_t u = ((int64_t)bt * tiles_f + f / kFeat) * 2;
    const int na = s_small ? s_small : (sk_unit_split(u, C, G, cpu) ? 2 : 1);
    const int nb = s_small ? s_small : (sk_unit_split(u + 1, C, G, cpu) ? 2 : 1);
    float4 av = reinterpret_cast<const float4*>(part)[g];
    float4 bv = reinterpret_cast<const float4*>(part + slice)[g];
    for (int i = 1; i < na; ++i) {
      const float4 x = reinterpret_cast<const float4*>(part + (2 * i) * slice)[g];
      av.x += x.x; av.y += x.y; av.z += x.z; av.w += x.w;
    }
    for (int i = 1; i < nb; ++i) {
      const float4 y = reinterpret_cast<const float4*>(part + (2 * i + 1) * slice)[g];
      bv.x += y.x; bv.y += y.y; bv.z += y.z; bv.w += y.w;
    }
    uint2 h;
    h.x = pack_bf16x2(silu_f32(av.x) * bv.x, silu_f32(av.y) * bv.y);
    h.y = pack_bf16x2(silu_f32(av.z) * bv.z, silu_f32(av.w) * bv.w);
    reinterpret_cast<uint2*>(H)[g] = h;
  }
}

template <int NJ, int MODE>
hipError_t launch_stream(const StreamArgs& in, hipStream_t stream) {
  StreamArgs a = in;
  a.max_tiles = (int)(((int64_t)a.P + (int64_t)a.E * (16 * NJ - 1)) / (16 * NJ));
  if (a.max_tiles <= 0) return hipSuccess;
  const int64_t grid =
      (int64_t)a.max_tiles * a.splits * (a.N / kFeat);
  hipLaunchKernelGGL((stream_gemm_kernel<NJ, MODE>), dim3((unsigned)grid), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

namespace {

// A launch whose workgroups put `kparts` waves on one matrix, K split
// `splits` ways: every wave takes an even number of k-steps of 32 (and, when
// K is split, at least four), and a k-step's 32 weight rows stay under 2 GiB
// (32-bit buffer offsets).
bool stream_shape_ok(int Kdim, int N, int kparts, int splits) {
  return splits >= 1 && N % kFeat == 0 && Kdim % (splits * kparts * 64) == 0 &&
         (splits == 1 || Kdim / (splits * kparts) >= 128) &&
         (int64_t)32 * N * 2 < (int64_t(1) << 31);
}

// Picks among candidate launches, given as busy-workgroup counts in
// increasing order (index 0 = the unsplit launch):
//   * the largest candidate that is one round of workgroups (one per compute
//     unit) filling at least 55 % of the compute units;
//   * else the unsplit launch when it alone makes at least 1.7 rounds (no
//     partial sums at all);
//   * else the smallest candidate with at least 3 rounds (the largest if
//     none has).
int pick_launch(const double* wgs, int n) {
  int one = -1;
  for (int i = 0; i < n; ++i)
    if (wgs[i] <= kComputeUnits && wgs[i] >= 0.55 * kComputeUnits) one = i;
  if (one >= 0) return one;
  if (wgs[0] >= 1.7 * kComputeUnits) return 0;
  for (int i = 0; i < n; ++i)
    if (wgs[i] >= 3.0 * kComputeUnits) return i;
  return n - 1;
}

}  // namespace

// Partial-sum slices of the per-matrix W1/W3 product (stream_sk_kernel over
// kSkGrid workgroups): two for units cut by a workgroup boundary, or
// the equal pieces of units when there are fewer units than workgroups (most
// when a single token tile holds rows).
int sk_slices(int d, int d_ff) {
  const int cpu = d / kChunkRows;
  const int U = 2 * (d_ff / kFeat);
  int s = 1;
  while (cpu % (2 * s) == 0 && (int64_t)U * 2 * s <= (int64_t)kSkGrid) s *= 2;
  return std::max(2, s);
}

int stream_swiglu_splits(int d, int d_ff, double tiles) {
  if (!stream_shape_ok(d, d_ff, kWaves / 2, 1)) return -1;
  const double per = tiles * (d_ff / kFeat);  // busy workgroups of the fused launch
  double wgs[16];
  int split[16];
  int n = 0;
  wgs[n] = per;
  split[n++] = 0;
  for (int s = 1; s <= 64 && n < 16; ++s)
    if (stream_shape_ok(d, d_ff, kWaves, s)) {
      wgs[n] = 2.0 * s * per;
      split[n++] = s;
    }
  const int pick = split[pick_launch(wgs, n)];
  return pick == 0 ? 0 : sk_slices(d, d_ff);
}

int stream_down_splits(int d_ff, int d, double tiles) {
  if (!stream_shape_ok(d_ff, d, kWaves, 1)) return 0;
  const double per = tiles * (d / kFeat);
  double wgs[16];
  int split[16];
  int n = 0;
  for (int s = 1; s <= 64 && n < 16; ++s)
    if (stream_shape_ok(d_ff, d, kWaves, s)) {
      wgs[n] = s * per;
      split[n++] = s;
    }
  return split[pick_launch(wgs, n)];
}

hipError_t launch_stream_swiglu_bf16(const void* x, const int32_t* sorted_token,
                                     const ExpertPtrs& W1, const ExpertPtrs& W3,
                                     const int32_t* offsets, int P, int d, int d_ff, int E,
                                     int splits, float* part, void* H, const int32_t* topk_idx,
                                     int K, int32_t* pos, hipStream_t stream) {
  if (P > kStreamMaxPairs || E > kMaxExperts) return hipErrorInvalidValue;
  StreamArgs a{};
  a.topk_idx = topk_idx;
  a.K = K;
  a.pos_out = pos;
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
  if (splits == 0) {
    a.splits = 1;
    return launch_stream<1, kFused>(a, stream);
  }
  if (P == 0) return hipSuccess;
  hipLaunchKernelGGL(stream_sk_kernel, dim3((unsigned)kSkGrid), dim3(kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_swiglu_finish_bf16(const float* part, const int32_t* offsets, int P, int d,
                                     int d_ff, int E, void* H, hipStream_t stream) {
  const int64_t n4 = (int64_t)P * d_ff / 4;
  if (n4 == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 2048);
  hipLaunchKernelGGL(swiglu_finish_kernel, dim3(blocks), dim3(256), 0, stream, part, offsets, E,
                     P, d_ff, d, kSkGrid, static_cast<bf16_t*>(H));
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
  return launch_stream<1, kDown>(a, stream);
}

}  // namespace moe
