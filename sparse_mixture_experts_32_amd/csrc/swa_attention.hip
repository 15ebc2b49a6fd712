// Sliding-window grouped-query attention with a rolling-buffer key/value
// cache, one chunk of query tokens at a time (bf16 storage, fp32 arithmetic).
//
// What is computed ("从Mistral 7B到MoE模型Mixtral 8x7B的全面解析" (aiqianji.com),
// sections 1.1 and 1.2.1-1.2.3): query token t of sequence b sits at
// position p = pos0[b] + t and attends to the positions p - W + 1 .. p (at
// least 0), itself included; query head h reads key/value head
// h / (n_heads / n_kv_heads).  A key at position j < pos0[b] comes from the
// cache slot j mod W, a key at j >= pos0[b] from the chunk itself.  Scores
// are q.k / sqrt(128); weights are their softmax over the window.
//
// Kernel layout (gfx950):
//   * a workgroup owns one key/value head of one sequence, all G query heads
//     that share it and 16 * (4 / G) * kQSub query tokens: wave w takes query
//     head w % G and kQSub tiles of 16 tokens, so every key/value tile
//     staged in LDS serves all heads of the group;
//   * keys go in blocks of 64: K and V rows (256 bytes each) travel global ->
//     LDS with global_load_lds_dwordx4, double buffered; each
//     row's 16-byte chunks are XOR-swizzled so the operand reads are free of
//     bank conflicts; workgroups of one key/value head are placed on one XCD
//     so their overlapping windows share an L2;
//   * scores: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys on the M side,
//     queries on the N side), so a lane holds 8 keys of one query; scores
//     are masked only in blocks at the window's edges;
//   * online softmax per query with a lazily moved reference (exp2 with the
//     scale folded in; the O rescale happens only when the maximum grows by
//     more than 2^8); the probabilities are rounded to bf16 and are, as
//     held, the N-side operand of O^T = V^T P^T -- the matrix instruction's
//     k order is taken to be the lane's key order, and the V^T operand is
//     read in that same order with ds_read_b64_tr_b16 (4 keys of one column
//     per read); a ones operand against the same weights gives the sums;
//   * long windows with few query tiles (decode) split the key range over
//     workgroups; each writes its unnormalised output, reference and sum,
//     and a combine kernel merges the splits in split order.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void global_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int kHd = 128;              // head dimension
constexpr int kRowBytes = kHd * 2;    // 256 bytes per key or value row
constexpr int kKB = 64;               // keys per block
constexpr int kTile = kKB * kRowBytes;   // 16 KB per K or V tile
constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const bf16_t* q;        // [B, T, H, hd]
  const bf16_t* k_new;    // [B, T, KVH, hd]
  const bf16_t* v_new;
  const bf16_t* k_cache;  // [B, W, KVH, hd]
  const bf16_t* v_cache;
  const int32_t* pos0;    // [B]
  void* out;              // [B, T, H, hd] bf16 or fp32 (splits == 1)
  float* part_o;          // [B, T, H, splits, hd] (splits > 1)
  float* part_ml;         // [B, T, H, splits, 2]
  int B, T, W, H, KVH, G;
  int qtiles;             // query tiles per (sequence, kv head)
  int splits;             // key-range splits
  int out_f32;
};

__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((global_void_t*)src, (lds_void_t*)lds_dst, 16, 0, 0);
}

// 16-byte chunk swizzles of a 256-byte row: K rows are read 16 rows x one
// chunk per instruction, V rows by transposed reads of 4 rows x 2 chunks.
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v(int r) { return 2 * (r & 3) + 8 * ((r >> 2) & 1); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Max over the four 16-lane rows that hold the same query column: the
// permlane swaps exchange rows 0<->1, 2<->3 (16) and the halves (32); of the
// two results one is the lane's own value and one its partner's.
__device__ __forceinline__ float max_rows(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// two floats -> two bf16 (round to nearest even, the hardware conversion)
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// kQSub: 16-token query tiles per wave.  Two workgroups per CU (each wave
// has 256 registers), each with a 2-slot ring: one block of keys in flight
// while the other is consumed.
template <int kQSub>
__global__ __launch_bounds__(256, 2) void swa_attn_kernel(AttnArgs a) {
  __shared__ __align__(1024) char sK0[kTile], sV0[kTile], sK1[kTile], sV1[kTile];

  // ---- which (sequence, kv head, query tile, key split) ----
  // Work items are numbered split-fastest; consecutive items go to the same
  // XCD (the hardware deals workgroups round-robin over the 8 XCDs), so the
  // query tiles of one kv head, whose key windows overlap, share an L2.
  int bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
  const int split = bid % a.splits;
  bid /= a.splits;
  const int qt = bid % a.qtiles;
  bid /= a.qtiles;
  const int kv = bid % a.KVH;
  const int b = bid / a.KVH;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.G;
  const int h = kv * G + wave % G;                 // this wave's query head
  const int sub_per_head = kWaves / G;             // query tiles of 16 per head in the WG
  const int wg_tokens = 16 * kQSub * sub_per_head;
  const int t_base = qt * wg_tokens + (wave / G) * 16 * kQSub;  // first token of this wave
  const int T = a.T, W = a.W;
  const int pos0 = a.pos0[b];

  // key range of the whole workgroup, then this split's share (64-aligned)
  const int t_lo = qt * wg_tokens;
  const int t_hi = min(T, t_lo + wg_tokens) - 1;
  const int k_first = max(0, pos0 + t_lo - W + 1);
  const int k_last = pos0 + t_hi;
  const int nblk_all = (k_last - k_first + kKB) / kKB;
  const int per = (nblk_all + a.splits - 1) / a.splits;
  const int blk0 = split * per;
  const int nblk = max(0, min(nblk_all, blk0 + per) - blk0);
  const int k_lo = k_first + blk0 * kKB;                          // this split's keys
  const int k_hi = min(k_last, k_lo + nblk * kKB - 1);
  // positions of this wave's first and last (clamped) query rows
  const int wq_lo = pos0 + min(t_base, T - 1);
  const int wq_hi = pos0 + min(t_base + 16 * kQSub - 1, T - 1);

  const int g = lane >> 4;
  const int j = lane & 15;
  const int64_t kv_stride = (int64_t)a.KVH * kHd;                 // elements per position

  // ---- query operand (N side): lane holds q[t][h][32 s + 8 g .. +7] ----
  bf16x8_t qf[kQSub][4];
  int qpos[kQSub];
#pragma unroll
  for (int u = 0; u < kQSub; ++u) {
    const int t = min(t_base + 16 * u + j, T - 1);   // rows past the chunk: never stored
    qpos[u] = pos0 + t;
    const bf16_t* src = a.q + (((int64_t)b * T + t) * a.H + h) * kHd + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[u][s] = *reinterpret_cast<const bf16x8_t*>(src + 32 * s);
  }

  // ---- key/value tile loads: 32 instructions per block, 8 per wave ----
  // instruction u of wave w fills rows 32 (w mod 2) + 4 u .. +3 of the K
  // tile (waves 0, 1) or the V tile (waves 2, 3); lane l lands chunk l mod 16
  // of row 32 (w mod 2) + 4 u + l / 16.  A key at position kp < pos0 lies
  // within one window before pos0, so its cache slot is
  // kp - pos0 + (pos0 mod W), plus W when that is negative; a key at
  // kp >= pos0 is chunk row kp - pos0.
  const bool wave_v = wave >= 2;
  const int row_bytes = a.KVH * kRowBytes;                        // bytes per position
  const char* cache_base = reinterpret_cast<const char*>(wave_v ? a.v_cache : a.k_cache) +
                           (int64_t)b * W * row_bytes + kv * kRowBytes;
  const char* chunk_base = reinterpret_cast<const char*>(wave_v ? a.v_new : a.k_new) +
                           (int64_t)b * T * row_bytes + kv * kRowBytes;
  const int pos0_slot = pos0 % W;
  const int row_w = 32 * (wave & 1) + (lane >> 4);                // + 4 u
  uint32_t lane_off[8];                                           // within a block: row, chunk
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = row_w + 4 * u;
    const int c = (lane & 15) ^ (wave_v ? swz_v(row) : swz_k(row));
    lane_off[u] = (uint32_t)(row * row_bytes + 16 * c);
  }
  auto issue = [&](int blk, char* kdst, char* vdst) __attribute__((always_inline)) {
    const int kb = k_lo + blk * kKB;
    char* dst = wave_v ? vdst : kdst;
    const int e0 = kb - pos0;                          // first key relative to pos0
    const int slot0 = e0 + pos0_slot + (e0 + pos0_slot < 0 ? W : 0);
    const bool whole = kb + kKB - 1 <= k_hi;
    if (whole && (e0 >= 0 || (e0 + kKB <= 0 && slot0 + kKB <= W))) {
      // all 64 rows from one source, consecutive: a uniform base + fixed offsets
      const char* base = e0 >= 0 ? chunk_base + (int64_t)e0 * row_bytes
                                 : cache_base + (int64_t)slot0 * row_bytes;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        dma16(base + lane_off[u], dst + (8 * (wave & 1) + u) * 1024);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int row = row_w + 4 * u;
        const int c = (lane & 15) ^ (wave_v ? swz_v(row) : swz_k(row));
        const int e = min(kb + row, k_hi) - pos0;        // rows past the range: masked
        const int slot = e + pos0_slot + (e + pos0_slot < 0 ? W : 0);
        const bool cached = e < 0;
        const char* src = (cached ? cache_base : chunk_base) +
                          (int64_t)(cached ? slot : e) * row_bytes + 16 * c;
        dma16(src, dst + (8 * (wave & 1) + u) * 1024);
      }
    }
  };

  // Online softmax with a lazily moved reference: m is the exponent
  // reference (log2 units, scale folded in); it moves only when a score
  // exceeds it by more than kTau, so the weights 2^(s - m) stay below 2^kTau
  // and the O rescale is rare.  The result O / l does not depend on m.
  // The weight sums come from the matrix cores too (a ones operand against
  // the same bf16 weights), so every entry of lsum[u] is the column's sum.
  constexpr float kTau = 8.f;
  f32x4_t o[kQSub][8];
  f32x4_t lsum[kQSub];
  float m[kQSub];
#pragma unroll
  for (int u = 0; u < kQSub; ++u) {
    m[u] = -1e30f;
    lsum[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < 8; ++db) o[u][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3f803f80u, 0x3f803f80u,
                                                             0x3f803f80u, 0x3f803f80u});
  const float scale = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)
  const float neg_inf = -__builtin_inff();

  // K operand (M side) of key row r, k-step s: chunk 4 s + g of row r
  int koff[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = 16 * rb + j;
      koff[rb][s] = r * kRowBytes + (((4 * s + g) ^ swz_k(r)) << 4);
    }
  // V^T operand: transposed read of rows k0 + i / 4, columns 16 db + 4 (i mod 4);
  // the second 16 keys sit 16 rows (4 KB) further with the same swizzle
  int voff[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const int r = 4 * g + (j >> 2);
    const int col = 16 * db + 4 * (j & 3);
    voff[db] = r * kRowBytes + (((col >> 3) ^ swz_v(r)) << 4) + (col & 7) * 2;
  }

  // Operand reads of 32 keys: K rows as the M-side operand of the scores,
  // V^T (transposed reads) as the M-side operand of O^T.
  auto read_k = [&](const char* kt32, bf16x8_t (&kf)[2][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kf[rb][s] = *reinterpret_cast<const bf16x8_t*>(kt32 + koff[rb][s]);
  };
  auto read_v = [&](const char* vt32, bf16x8_t (&vf)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)((lds_char_t*)vt32 + voff[db]));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)((lds_char_t*)vt32 + voff[db] + 16 * kRowBytes));
      const s16x4_t both[2] = {lo, hi};
      vf[db] = __builtin_bit_cast(bf16x8_t, both);
    }
  };

  // 64 keys from one slot, as two halves of 32.  The reads of the second
  // half are issued behind the first half's score products (K) and behind
  // its P.V products (V), into the registers those products have consumed,
  // so their latency hides under the softmax and the matrix work.  edge:
  // the block holds keys that some query of this wave must not see (window
  // edges, causal edge, end of the split's range); only then are scores
  // masked.
  auto compute = [&](int n, const char* kt, const char* vt) __attribute__((always_inline)) {
    const int kb = k_lo + n * kKB;
    const bool edge = !(kb + kKB - 1 <= k_hi && kb + kKB - 1 <= wq_lo && kb > wq_hi - W);
    bf16x8_t kf[2][4];
    bf16x8_t vf[8];
    read_k(kt, kf);
    read_v(vt, vf);
#pragma unroll
    for (int half32 = 0; half32 < 2; ++half32) {       // 32 keys at a time
      // raw scores of keys 16 rb + 4 g + i for query column j, all tiles
      f32x4_t sc[kQSub][2];
#pragma unroll
      for (int u = 0; u < kQSub; ++u)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          sc[u][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s)
            sc[u][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[rb][s], qf[u][s], sc[u][rb], 0, 0, 0);
        }
      if (half32 == 0) {
        __builtin_amdgcn_sched_barrier(0);
        read_k(kt + 32 * kRowBytes, kf);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < kQSub; ++u) {
        if (edge) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int kp = kb + half32 * 32 + 16 * rb + 4 * g + i;
              const bool valid = kp <= k_hi && kp <= qpos[u] && kp > qpos[u] - W;
              sc[u][rb][i] = valid ? sc[u][rb][i] : neg_inf;
            }
        }
        float mx = fmaxf(fmaxf(fmaxf(sc[u][0][0], sc[u][0][1]), fmaxf(sc[u][0][2], sc[u][0][3])),
                         fmaxf(fmaxf(sc[u][1][0], sc[u][1][1]), fmaxf(sc[u][1][2], sc[u][1][3])));
        mx = max_rows(mx) * scale;
        const bool move = mx > m[u] + kTau;
        if (__builtin_amdgcn_ballot_w64(move) != 0) {   // rare after the first block
          const float m_new = move ? mx : m[u];
          const float corr = __builtin_amdgcn_exp2f(m[u] - m_new);
          m[u] = m_new;
          lsum[u] *= corr;
#pragma unroll
          for (int db = 0; db < 8; ++db) o[u][db] *= corr;
        }
        const float neg_m = -m[u];
        float p[8];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            p[4 * rb + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][rb][i], scale, neg_m));
        const u32x4_t pk = {cvt_bf16x2(p[0], p[1]), cvt_bf16x2(p[2], p[3]),
                            cvt_bf16x2(p[4], p[5]), cvt_bf16x2(p[6], p[7])};
        const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pk);
#pragma unroll
        for (int db = 0; db < 8; ++db)
          o[u][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pf, o[u][db], 0, 0, 0);
        lsum[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf, lsum[u], 0, 0, 0);
      }
      if (half32 == 0) {
        __builtin_amdgcn_sched_barrier(0);
        read_v(vt + 32 * kRowBytes, vf);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // block n sits in one slot while block n + 1 is loaded into the other.
  // The loop is unrolled over the two slots so that the compiler sees which
  // LDS object each read and each load touches.
  auto stage = [&](int n, const char* kt, const char* vt, char* kn, char* vn)
                   __attribute__((always_inline)) {
    wait_vm<0>();                      // block n has landed ...
    __builtin_amdgcn_s_barrier();      // ... for every wave; the other slot is free
    if (n + 1 < nblk) issue(n + 1, kn, vn);
    compute(n, kt, vt);
  };

  if (nblk > 0) issue(0, sK0, sV0);
  for (int n = 0; n < nblk; n += 2) {
    stage(n, sK0, sV0, sK1, sV1);
    if (n + 1 < nblk) stage(n + 1, sK1, sV1, sK0, sV0);
  }
  wait_vm<0>();                                          // no load lands after the end

  // ---- output: lane holds d = 16 db + 4 g .. +3 of query token t ----
#pragma unroll
  for (int u = 0; u < kQSub; ++u) {
    const float l = lsum[u][0];
    const int t = t_base + 16 * u + j;
    if (t >= T) continue;
    const int64_t row = ((int64_t)b * T + t) * a.H + h;
    if (a.splits == 1) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int d = 16 * db + 4 * g;
        const f32x4_t v = o[u][db] * inv;
        if (a.out_f32) {
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + row * kHd + d) =
              make_float4(v[0], v[1], v[2], v[3]);
        } else {
          uint2 w2;
          w2.x = pack_bf16x2(v[0], v[1]);
          w2.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(static_cast<bf16_t*>(a.out) + row * kHd + d) = w2;
        }
      }
    } else {
      const int64_t prow = row * a.splits + split;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int d = 16 * db + 4 * g;
        const f32x4_t v = o[u][db];
        *reinterpret_cast<float4*>(a.part_o + prow * kHd + d) = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (g == 0) {
        a.part_ml[prow * 2 + 0] = m[u];
        a.part_ml[prow * 2 + 1] = l;
      }
    }
  }
}

// Merge the key splits of each (sequence, token, head) in split order:
// o = sum_s 2^(m_s - m) o_s / sum_s 2^(m_s - m) l_s with m = max_s m_s.  A
// split that saw no key of the row has l_s = 0 and o_s = 0 and weighs 0.
// kSplits is a compile-time count, so every load is issued before the first
// use and the merge costs one memory latency.
template <int kSplits>
__global__ __launch_bounds__(128) void swa_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int rows, void* out, int out_f32) {
  const int row = blockIdx.x;
  const int d = threadIdx.x;
  if (row >= rows) return;
  const float* ml = part_ml + (int64_t)row * kSplits * 2;
  const float* po = part_o + (int64_t)row * kSplits * kHd + d;
  float ms[kSplits], ls[kSplits], os[kSplits];
#pragma unroll
  for (int s = 0; s < kSplits; ++s) {
    ms[s] = ml[2 * s];
    ls[s] = ml[2 * s + 1];
    os[s] = po[(int64_t)s * kHd];
  }
  float mmax = -1e30f;
#pragma unroll
  for (int s = 0; s < kSplits; ++s) mmax = ls[s] > 0.f ? fmaxf(mmax, ms[s]) : mmax;
  float num = 0.f, den = 0.f;
#pragma unroll
  for (int s = 0; s < kSplits; ++s) {
    const float w = ls[s] > 0.f ? __builtin_amdgcn_exp2f(ms[s] - mmax) : 0.f;
    num = __builtin_fmaf(w, os[s], num);
    den = __builtin_fmaf(w, ls[s], den);
  }
  const float v = den > 0.f ? num / den : 0.f;
  if (out_f32)
    static_cast<float*>(out)[(int64_t)row * kHd + d] = v;
  else
    static_cast<bf16_t*>(out)[(int64_t)row * kHd + d] = f32_to_bf16(v);
}

// Rolling-buffer append: position pos0[b] + t goes to slot (pos0[b] + t) mod W;
// one thread per 16 bytes of a key (and of a value) row.
__global__ __launch_bounds__(256) void swa_append_kernel(const bf16_t* __restrict__ k_new,
                                                         const bf16_t* __restrict__ v_new,
                                                         const int32_t* __restrict__ pos0,
                                                         int B, int T, int W, int KVH,
                                                         bf16_t* __restrict__ k_cache,
                                                         bf16_t* __restrict__ v_cache) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const int chunks = KVH * kHd / 8;               // 16-byte pieces per position
  const int64_t total = (int64_t)B * T * chunks;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % chunks);
    const int64_t bt = i / chunks;
    const int t = (int)(bt % T);
    const int b = (int)(bt / T);
    if (t < T - W) continue;                        // overwritten later in the same chunk
    const int slot = (pos0[b] + t) % W;
    const int64_t src = bt * chunks + c;
    const int64_t dst = ((int64_t)b * W + slot) * chunks + c;
    reinterpret_cast<u32x4_t*>(k_cache)[dst] = reinterpret_cast<const u32x4_t*>(k_new)[src];
    reinterpret_cast<u32x4_t*>(v_cache)[dst] = reinterpret_cast<const u32x4_t*>(v_new)[src];
  }
}

}  // namespace

int swa_head_dim() { return kHd; }

// Launch plan.  Chunks of 64 tokens or more: two 16-token tiles per wave
// (each K/V fragment read from LDS serves 32 query columns); shorter chunks
// (decode): one tile per wave.  Both run two workgroups per CU, so that each
// SIMD holds two waves -- the matrix work of one overlaps the softmax of the
// other, and eight waves per CU keep the loads of decode flowing.  (Measured
// alternatives: four tiles per wave need more than the 256 registers a wave
// has at that occupancy and ran slower at one workgroup per CU; decode with
// one workgroup per CU and 4 or 5 slots in flight was slower than two
// workgroups with 2 slots.)  Key splits (a power of two, at most 16) are
// added until 512 workgroups cover the chip, each split at least 4 blocks
// of 64 keys.

int swa_plan_splits(int B, int T, int W, int H, int KVH, int* qtiles_out, int* qsub_out) {
  const int G = H / KVH;
  const bool big = T >= 64;
  const int qsub = big ? 2 : 1;
  const int wg_tokens = 16 * qsub * (kWaves / G);
  const int qtiles = (T + wg_tokens - 1) / wg_tokens;
  const int64_t wgs = (int64_t)B * KVH * qtiles;
  const int64_t target = 512;
  const int keys = min(W, T) + W;                  // generous upper bound of a tile's range
  const int max_splits = min(16, max(1, keys / (4 * kKB)));
  int splits = 1;                                  // a power of two, at most 16
  while (2 * splits <= max_splits && wgs * splits < target) splits *= 2;
  if (qtiles_out) *qtiles_out = qtiles;
  if (qsub_out) *qsub_out = qsub;
  return splits;
}

hipError_t launch_swa_attention(const void* q, const void* k_new, const void* v_new,
                                const void* k_cache, const void* v_cache, const int32_t* pos0,
                                int B, int T, int W, int H, int KVH, void* out, int out_f32,
                                float* part_o, float* part_ml, hipStream_t stream) {
  int qtiles = 0, qsub = 1;
  const int splits = swa_plan_splits(B, T, W, H, KVH, &qtiles, &qsub);
  AttnArgs a{};
  a.q = static_cast<const bf16_t*>(q);
  a.k_new = static_cast<const bf16_t*>(k_new);
  a.v_new = static_cast<const bf16_t*>(v_new);
  a.k_cache = static_cast<const bf16_t*>(k_cache);
  a.v_cache = static_cast<const bf16_t*>(v_cache);
  a.pos0 = pos0;
  a.out = out;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.B = B;
  a.T = T;
  a.W = W;
  a.H = H;
  a.KVH = KVH;
  a.G = H / KVH;
  a.qtiles = qtiles;
  a.splits = splits;
  a.out_f32 = out_f32;
  const int64_t grid = (int64_t)B * KVH * qtiles * splits;
  if (grid == 0) return hipSuccess;
  if (qsub == 1)
    hipLaunchKernelGGL(swa_attn_kernel<1>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(swa_attn_kernel<2>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int rows = B * T * H;
  switch (splits) {
    case 2: hipLaunchKernelGGL(swa_combine_kernel<2>, dim3(rows), dim3(kHd), 0, stream, part_o,
                               part_ml, rows, out, out_f32); break;
    case 4: hipLaunchKernelGGL(swa_combine_kernel<4>, dim3(rows), dim3(kHd), 0, stream, part_o,
                               part_ml, rows, out, out_f32); break;
    case 8: hipLaunchKernelGGL(swa_combine_kernel<8>, dim3(rows), dim3(kHd), 0, stream, part_o,
                               part_ml, rows, out, out_f32); break;
    case 16: hipLaunchKernelGGL(swa_combine_kernel<16>, dim3(rows), dim3(kHd), 0, stream, part_o,
                                part_ml, rows, out, out_f32); break;
    default: return hipErrorInvalidValue;   // the plan only makes powers of two up to 16
  }
  return hipGetLastError();
}

hipError_t launch_swa_append(const void* k_new, const void* v_new, const int32_t* pos0, int B,
                             int T, int W, int KVH, void* k_cache, void* v_cache,
                             hipStream_t stream) {
  const int64_t total = (int64_t)B * T * KVH * kHd / 8;
  if (total == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(swa_append_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(k_new), static_cast<const bf16_t*>(v_new), pos0,
                     B, T, W, KVH, static_cast<bf16_t*>(k_cache), static_cast<bf16_t*>(v_cache));
  return hipGetLastError();
}

}  // namespace moe
