// C ABI of the MoE layer forward: host-side validation, workspace carving and
// the launch sequence.  Declarations and contracts: include/moe_mi355x.h.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <unordered_set>

#include "../../include/moe_mi355x.h"
#include "moe_internal.h"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

moe_status ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Status of a finished launch sequence: MOE_OK (and a cleared message) or MOE_EHIP.
moe_status finish(hipError_t e, const char* what) {
  return e == hipSuccess ? ok() : hip_status(e, what);
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t dtype_bytes(int32_t dt) { return dt == MOE_BF16 ? 2 : 4; }

moe_status check_dtype(int32_t dt, const char* name) {
  if (dt != MOE_F32 && dt != MOE_BF16) return fail(MOE_EINVAL, "unknown %s %d", name, dt);
  return MOE_OK;
}

moe_status check_shape(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K, int32_t dt) {
  moe_status s = check_dtype(dt, "dtype");
  if (s) return s;
  if (T < 0) return fail(MOE_EINVAL, "T = %lld < 0", (long long)T);
  if (d <= 0 || d_ff <= 0) return fail(MOE_EINVAL, "d and d_ff must be positive");
  if (E < 1 || E > MOE_MAX_EXPERTS)
    return fail(MOE_EINVAL, "E = %d outside [1, %d]", E, MOE_MAX_EXPERTS);
  if (K < 1 || K > E) return fail(MOE_EINVAL, "K = %d outside [1, E = %d]", K, E);
  if (T * (int64_t)K >= (int64_t(1) << 31)) return fail(MOE_EINVAL, "T*K must be < 2^31");
  if (d >= (int64_t(1) << 31) || d_ff >= (int64_t(1) << 31))
    return fail(MOE_EINVAL, "d and d_ff must be < 2^31");
  if (dt == MOE_BF16 && (d % 64 != 0 || d_ff % 64 != 0))
    return fail(MOE_EUNSUPPORTED, "bf16 path needs d %% 64 == 0 and d_ff %% 64 == 0");
  return MOE_OK;
}

struct Plan {
  int swiglu_splits = 0;
  int down_splits = 1;
  size_t scratch = 0;        // W1/W3 partial sums
  size_t down_scratch = 0;   // W2 tail pieces
  bool streaming = false;
  bool swiglu_mixed = false;  // tiled W1/W3 with a tile shape per expert
};

// Batches whose expert segments fit one 16-row token tile per expert in the
// common case (T*K <= 64) stream the weights; larger ones use the tiled
// matrix-core kernels, with the W2 product split over K when its grid would
// fill the chip fewer than ~4 times.
Plan make_plan(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K, int32_t dt) {
  Plan p;
  const int64_t P = T * K;
  if (dt != MOE_BF16 || P == 0) return p;
  if (P > 64) {
    // W2 of at least a whole round of tiles: whole-K tiles and a split tail
    // (one slice of O); smaller: K splits so that the grid fills the chip
    p.down_scratch = moe::tiled_down_side_bytes((int)P, (int)d, (int)d_ff);
    p.swiglu_mixed = moe::tiled_gemm_supported((int)d, (int)d_ff, true, 1, P) &&
                     moe::tiled_swiglu_mixed((int)P, E, (int)d_ff);
    if (p.down_scratch == 0 && moe::tiled_gemm_supported((int)d_ff, (int)d, false, 1, P)) {
      const int64_t tiles = moe::tiled_gemm_tiles((int)P, E, (int)d, false);
      for (int s = 2; s <= 4 && tiles * (s - 1) < 4 * 256; ++s)
        if (moe::tiled_gemm_supported((int)d_ff, (int)d, false, s, P)) p.down_splits = s;
    }
    return p;
  }
  // The split count is sized for the token tiles expected to hold rows: the
  // expected number of distinct experts among T tokens choosing K of E
  // uniformly, E (1 - (1 - K/E)^T), at least P/16, at most the worst case.
  const double busy = E * (1.0 - std::pow(1.0 - (double)K / E, (double)T));
  const double tiles = std::min<double>(std::max<double>(busy, P / 16.0),
                                        (double)((P + (int64_t)E * 15) / 16));
  const int s1 = moe::stream_swiglu_splits((int)d, (int)d_ff, tiles);
  const int s2 = moe::stream_down_splits((int)d_ff, (int)d, tiles);
  if (s1 < 0 || s2 == 0) return p;
  p.streaming = true;
  p.swiglu_splits = s1;
  p.down_splits = s2;
  if (p.swiglu_splits > 0) p.scratch = (size_t)p.swiglu_splits * 2 * P * d_ff * sizeof(float);
  return p;
}

void layout(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K, int32_t dt,
            size_t off[MOE_WS_COUNT], size_t* total) {
  const size_t P = (size_t)T * K;
  const Plan plan = make_plan(T, d, d_ff, E, K, dt);
  size_t o = 0;
  auto put = [&](int item, size_t bytes) {
    off[item] = o;
    o = align256(o + bytes);
  };
  put(MOE_WS_TOPK_IDX, P * 4);
  put(MOE_WS_TOPK_W, P * 4);
  put(MOE_WS_OFFSETS, (size_t)(E + 1) * 4);
  put(MOE_WS_SORTED_TOKEN, P * 4);
  put(MOE_WS_POS, P * 4);
  put(MOE_WS_H, P * (size_t)d_ff * dtype_bytes(dt));
  put(MOE_WS_O, (size_t)plan.down_splits * P * (size_t)d * 4);
  put(MOE_WS_SCRATCH, std::max(plan.scratch, plan.down_scratch));
  *total = o;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

moe_status fill_ptrs(const void* const* src, int32_t E, moe::ExpertPtrs& dst, const char* name,
                     bool need16) {
  if (!src) return fail(MOE_EINVAL, "%s is NULL", name);
  std::memset(&dst, 0, sizeof(dst));
  for (int e = 0; e < E; ++e) {
    if (!src[e]) return fail(MOE_EINVAL, "%s[%d] is NULL", name, e);
    if (need16 && !aligned16(src[e]))
      return fail(MOE_EUNSUPPORTED, "%s[%d] is not 16-byte aligned", name, e);
    dst.p[e] = src[e];
  }
  return MOE_OK;
}

}  // namespace

namespace moe {

hipError_t allow_dynamic_lds(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::unordered_set<uint64_t> done;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t key = (reinterpret_cast<uint64_t>(kernel) << 8) ^ (uint64_t)dev;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count(key)) return hipSuccess;
  err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (err == hipSuccess) done.insert(key);
  return err;
}

}  // namespace moe

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE";
    case MOE_EHIP: return "MOE_EHIP";
  }
  return "MOE_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

moe_status moe_plan_for(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K, int32_t dtype,
                        moe_plan* plan) {
  if (!plan) return fail(MOE_EINVAL, "plan is NULL");
  moe_status s = check_shape(T, d, d_ff, E, K, dtype);
  if (s) return s;
  const Plan p = make_plan(T, d, d_ff, E, K, dtype);
  plan->swiglu_splits = p.swiglu_splits;
  plan->down_splits = p.down_splits;
  plan->swiglu_scratch_bytes = p.scratch;
  plan->down_scratch_bytes = p.down_scratch;
  plan->swiglu_mixed = p.swiglu_mixed ? 1 : 0;
  plan->weights_nt = dtype == MOE_BF16 && !p.streaming && T > 0 && moe::weights_read_once(T * K, E);
  plan->streaming = p.streaming ? 1 : 0;
  return ok();
}

moe_status moe_workspace_size(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K,
                              int32_t dtype, size_t* bytes) {
  if (!bytes) return fail(MOE_EINVAL, "bytes is NULL");
  moe_status s = check_shape(T, d, d_ff, E, K, dtype);
  if (s) return s;
  size_t off[MOE_WS_COUNT];
  layout(T, d, d_ff, E, K, dtype, off, bytes);
  return ok();
}

moe_status moe_workspace_layout(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K,
                                int32_t dtype, size_t* offsets) {
  if (!offsets) return fail(MOE_EINVAL, "offsets is NULL");
  moe_status s = check_shape(T, d, d_ff, E, K, dtype);
  if (s) return s;
  size_t total;
  layout(T, d, d_ff, E, K, dtype, offsets, &total);
  return ok();
}

moe_status moe_router_topk(const void* x, const void* W_g, int64_t T, int64_t d, int32_t E,
                           int32_t K, int32_t dtype, int32_t* topk_idx, float* topk_w,
                           float* logits, void* stream) {
  moe_status s = check_dtype(dtype, "dtype");
  if (s) return s;
  if (T < 0 || d <= 0 || d >= (int64_t(1) << 31)) return fail(MOE_EINVAL, "bad T or d");
  if (E < 1 || E > MOE_MAX_EXPERTS || K < 1 || K > E) return fail(MOE_EINVAL, "bad E or K");
  if (T * (int64_t)K >= (int64_t(1) << 31)) return fail(MOE_EINVAL, "T*K must be < 2^31");
  if (T == 0) return ok();
  if (!x || !W_g || !topk_idx || !topk_w) return fail(MOE_EINVAL, "NULL pointer");
  return finish(moe::launch_router_topk(x, W_g, (int)T, (int)d, E, K, dtype, topk_idx,
                                            topk_w, logits, (hipStream_t)stream),
                    "router_topk");
}

moe_status moe_route_permute(const int32_t* topk_idx, int64_t T, int32_t E, int32_t K,
                             int32_t* offsets, int32_t* sorted_token, int32_t* pos,
                             void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "T < 0");
  if (E < 1 || E > MOE_MAX_EXPERTS || K < 1 || K > E) return fail(MOE_EINVAL, "bad E or K");
  if (T * (int64_t)K >= (int64_t(1) << 31)) return fail(MOE_EINVAL, "T*K must be < 2^31");
  if (!offsets) return fail(MOE_EINVAL, "offsets is NULL");
  if (T > 0 && (!topk_idx || !sorted_token || !pos)) return fail(MOE_EINVAL, "NULL pointer");
  return finish(moe::launch_route_permute(topk_idx, (int)T, E, K, offsets, sorted_token, pos,
                                              (hipStream_t)stream),
                    "route_permute");
}

moe_status moe_routing_stats(const int32_t* topk_idx, int64_t T, int32_t E, int32_t K,
                             int32_t* counts, int32_t* repeats, void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "T < 0");
  if (E < 1 || E > MOE_MAX_EXPERTS || K < 1 || K > E) return fail(MOE_EINVAL, "bad E or K");
  if (T * (int64_t)K >= (int64_t(1) << 31)) return fail(MOE_EINVAL, "T*K must be < 2^31");
  if (T == 0) return ok();
  if (!topk_idx || !counts || !repeats) return fail(MOE_EINVAL, "NULL pointer");
  return finish(moe::launch_routing_stats(topk_idx, (int)T, E, K, counts, repeats,
                                          (hipStream_t)stream),
                "routing_stats");
}

}  // extern "C"

namespace {

// With `route` (topk_idx, K, pos) the small-batch kernels build the dispatch
// tables themselves and write them to offsets, sorted_token and pos.
struct Route {
  const int32_t* topk_idx = nullptr;
  int K = 0;
  int32_t* pos = nullptr;
};

hipError_t run_swiglu(const Plan& plan, const void* x, const int32_t* sorted_token,
                      const moe::ExpertPtrs& p1, const moe::ExpertPtrs& p3, const int32_t* offsets,
                      int P, int d, int d_ff, int E, int32_t dtype, void* H, void* scratch,
                      hipStream_t st, const Route& route = Route()) {
  if (dtype != MOE_BF16)
    return moe::launch_expert_swiglu_f32(x, sorted_token, p1, p3, offsets, P, d, d_ff, E, H, st);
  if (plan.streaming)
    return moe::launch_stream_swiglu_bf16(x, sorted_token, p1, p3, offsets, P, d, d_ff, E,
                                          plan.swiglu_splits, static_cast<float*>(scratch), H,
                                          route.topk_idx, route.K, route.pos, st);
  if (moe::tiled_gemm_supported(d, d_ff, true, 1, P))
    return moe::launch_tiled_swiglu_bf16(x, sorted_token, p1, p3, offsets, P, d, d_ff, E, H, st);
  return moe::launch_expert_swiglu_bf16(x, sorted_token, p1, p3, offsets, P, d, d_ff, E, H, st);
}

hipError_t run_down(const Plan& plan, const void* H, const moe::ExpertPtrs& p2,
                    const int32_t* offsets, int P, int d, int d_ff, int E, int32_t dtype, float* O,
                    void* scratch, hipStream_t st) {
  if (dtype != MOE_BF16) return moe::launch_expert_down_f32(H, p2, offsets, P, d, d_ff, E, O, st);
  if (plan.streaming)
    return moe::launch_stream_down_bf16(H, p2, offsets, P, d, d_ff, E, plan.down_splits, O, st);
  if (moe::tiled_gemm_supported(d_ff, d, false, plan.down_splits, P)) {
    float* side = plan.down_scratch ? static_cast<float*>(scratch) : nullptr;
    hipError_t e = moe::launch_tiled_down_bf16(H, p2, offsets, P, d, d_ff, E, plan.down_splits,
                                               O, side, plan.down_scratch, st);
    if (e == hipSuccess && side)
      e = moe::launch_tiled_down_fixup(side, plan.down_scratch, offsets, P, d, d_ff, E, O, st);
    return e;
  }
  return moe::launch_expert_down_bf16(H, p2, offsets, P, d, d_ff, E, O, st);
}

// Intermediates of one layer inside a workspace laid out by layout().
struct Bufs {
  int32_t* topk_idx;
  float* topk_w;
  int32_t* offsets;
  int32_t* sorted_token;
  int32_t* pos;
  void* H;
  float* O;
  void* scratch;
};

Bufs carve(void* workspace, const size_t off[MOE_WS_COUNT]) {
  char* ws = static_cast<char*>(workspace);
  Bufs b;
  b.topk_idx = reinterpret_cast<int32_t*>(ws + off[MOE_WS_TOPK_IDX]);
  b.topk_w = reinterpret_cast<float*>(ws + off[MOE_WS_TOPK_W]);
  b.offsets = reinterpret_cast<int32_t*>(ws + off[MOE_WS_OFFSETS]);
  b.sorted_token = reinterpret_cast<int32_t*>(ws + off[MOE_WS_SORTED_TOKEN]);
  b.pos = reinterpret_cast<int32_t*>(ws + off[MOE_WS_POS]);
  b.H = ws + off[MOE_WS_H];
  b.O = reinterpret_cast<float*>(ws + off[MOE_WS_O]);
  b.scratch = ws + off[MOE_WS_SCRATCH];
  return b;
}

// The stack's workspace: one layer's intermediates, then the normalised block
// input xn [T, d] at *xn_off.  Returns the total size.
size_t stack_layout(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K, int32_t dt,
                    size_t off[MOE_WS_COUNT], size_t* xn_off) {
  size_t total;
  layout(T, d, d_ff, E, K, dt, off, &total);
  *xn_off = total;
  return align256(total + (size_t)T * d * dtype_bytes(dt));
}

// Dispatch tables, the W1/W3 product (+ finish) and the W2 product of one
// layer whose router has filled b.topk_idx.
moe_status run_experts(const Plan& plan, const void* x, const moe::ExpertPtrs& p1,
                       const moe::ExpertPtrs& p3, const moe::ExpertPtrs& p2, const Bufs& b,
                       int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K, int32_t dtype,
                       hipStream_t st) {
  const int P = (int)(T * K);
  hipError_t e = hipSuccess;
  // small batches: the W1/W3 kernels build the dispatch tables themselves
  Route route;
  if (plan.streaming) {
    route.topk_idx = b.topk_idx;
    route.K = K;
    route.pos = b.pos;
  } else {
    e = moe::launch_route_permute(b.topk_idx, (int)T, E, K, b.offsets, b.sorted_token, b.pos, st);
    if (e != hipSuccess) return hip_status(e, "route_permute");
  }
  e = run_swiglu(plan, x, b.sorted_token, p1, p3, b.offsets, P, (int)d, (int)d_ff, E, dtype, b.H,
                 b.scratch, st, route);
  if (e != hipSuccess) return hip_status(e, "expert_swiglu");
  if (plan.swiglu_splits > 0) {
    e = moe::launch_swiglu_finish_bf16(static_cast<const float*>(b.scratch), b.offsets, P,
                                       (int)d, (int)d_ff, E, b.H, st);
    if (e != hipSuccess) return hip_status(e, "swiglu_finish");
  }
  e = run_down(plan, b.H, p2, b.offsets, P, (int)d, (int)d_ff, E, dtype, b.O, b.scratch, st);
  if (e != hipSuccess) return hip_status(e, "expert_down");
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_expert_swiglu(const void* x, const void* const* W1, const void* const* W3,
                             int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K,
                             int32_t dtype, const int32_t* offsets, const int32_t* sorted_token,
                             void* H, void* scratch, size_t scratch_bytes, void* stream) {
  moe_status s = check_shape(T, d, d_ff, E, K, dtype);
  if (s) return s;
  if (T == 0) return ok();
  if (!x || !offsets || !sorted_token || !H) return fail(MOE_EINVAL, "NULL pointer");
  const bool bf16 = dtype == MOE_BF16;
  if (bf16 && (!aligned16(x) || !aligned16(H)))
    return fail(MOE_EUNSUPPORTED, "x and H must be 16-byte aligned");
  moe::ExpertPtrs p1, p3;
  if ((s = fill_ptrs(W1, E, p1, "W1", bf16))) return s;
  if ((s = fill_ptrs(W3, E, p3, "W3", bf16))) return s;
  const Plan plan = make_plan(T, d, d_ff, E, K, dtype);
  if (plan.scratch > 0) {
    if (!scratch || scratch_bytes < plan.scratch)
      return fail(MOE_EWORKSPACE, "scratch has %zu bytes, needs %zu", scratch ? scratch_bytes : 0,
                  plan.scratch);
    if (!aligned16(scratch)) return fail(MOE_EWORKSPACE, "scratch must be 16-byte aligned");
  }
  return finish(run_swiglu(plan, x, sorted_token, p1, p3, offsets, (int)(T * K), (int)d,
                           (int)d_ff, E, dtype, H, scratch, (hipStream_t)stream),
                "expert_swiglu");
}

moe_status moe_swiglu_finish(const void* scratch, int64_t T, int64_t d, int64_t d_ff, int32_t E,
                             int32_t K, int32_t dtype, const int32_t* offsets, void* H,
                             void* stream) {
  moe_status s = check_shape(T, d, d_ff, E, K, dtype);
  if (s) return s;
  const Plan plan = make_plan(T, d, d_ff, E, K, dtype);
  if (T == 0 || plan.swiglu_splits == 0) return ok();
  if (!scratch || !H || !offsets) return fail(MOE_EINVAL, "NULL pointer");
  if (!aligned16(scratch) || !aligned16(H))
    return fail(MOE_EUNSUPPORTED, "scratch and H must be 16-byte aligned");
  return finish(moe::launch_swiglu_finish_bf16(static_cast<const float*>(scratch), offsets,
                                               (int)(T * K), (int)d, (int)d_ff, E, H,
                                               (hipStream_t)stream),
                "swiglu_finish");
}

moe_status moe_expert_down(const void* H, const void* const* W2, int64_t T, int64_t d,
                           int64_t d_ff, int32_t E, int32_t K, int32_t dtype,
                           const int32_t* offsets, float* O, void* scratch, size_t scratch_bytes,
                           void* stream) {
  moe_status s = check_shape(T, d, d_ff, E, K, dtype);
  if (s) return s;
  if (T == 0) return ok();
  if (!H || !offsets || !O) return fail(MOE_EINVAL, "NULL pointer");
  const bool bf16 = dtype == MOE_BF16;
  if (bf16 && (!aligned16(H) || !aligned16(O)))
    return fail(MOE_EUNSUPPORTED, "H and O must be 16-byte aligned");
  moe::ExpertPtrs p2;
  if ((s = fill_ptrs(W2, E, p2, "W2", bf16))) return s;
  const Plan plan = make_plan(T, d, d_ff, E, K, dtype);
  if (plan.down_scratch > 0) {
    if (!scratch || scratch_bytes < plan.down_scratch)
      return fail(MOE_EWORKSPACE, "scratch has %zu bytes, needs %zu", scratch ? scratch_bytes : 0,
                  plan.down_scratch);
    if (!aligned16(scratch)) return fail(MOE_EWORKSPACE, "scratch must be 16-byte aligned");
  }
  return finish(run_down(plan, H, p2, offsets, (int)(T * K), (int)d, (int)d_ff, E, dtype, O,
                         scratch, (hipStream_t)stream),
                "expert_down");
}

moe_status moe_combine(const float* O, int32_t o_splits, const float* topk_w, const int32_t* pos,
                       int64_t T, int64_t d, int32_t K, void* y, int32_t y_dtype,
                       int32_t accumulate, void* stream) {
  moe_status s = check_dtype(y_dtype, "y_dtype");
  if (s) return s;
  if (T < 0 || d <= 0 || d >= (int64_t(1) << 31) || K < 1 || K > MOE_MAX_EXPERTS)
    return fail(MOE_EINVAL, "bad T, d or K");
  if (o_splits < 1 || o_splits > 64) return fail(MOE_EINVAL, "o_splits outside [1, 64]");
  if (T == 0) return ok();
  if (!O || !topk_w || !pos || !y) return fail(MOE_EINVAL, "NULL pointer");
  if (d % 4 == 0 && (!aligned16(O) || (y_dtype == MOE_F32 ? !aligned16(y) : ((uintptr_t)y & 7))))
    return fail(MOE_EUNSUPPORTED, "O must be 16-byte and y vector aligned");
  return finish(moe::launch_combine(O, o_splits, T * K * d, topk_w, pos, (int)T, (int)d, K, y,
                                    y_dtype, accumulate ? 1 : 0, (hipStream_t)stream),
                "combine");
}

moe_status moe_rmsnorm(const void* h, void* out, int64_t T, int64_t d, float eps, int32_t dtype,
                       void* stream) {
  moe_status s = check_dtype(dtype, "dtype");
  if (s) return s;
  if (T < 0 || d <= 0 || d >= (int64_t(1) << 31)) return fail(MOE_EINVAL, "bad T or d");
  if (!(eps >= 0.0f)) return fail(MOE_EINVAL, "eps must be >= 0");
  if (T == 0) return ok();
  if (!h || !out) return fail(MOE_EINVAL, "NULL pointer");
  const size_t bytes = (size_t)T * d * dtype_bytes(dtype);
  if (overlap(h, bytes, out, bytes)) return fail(MOE_EINVAL, "h and out overlap");
  return finish(moe::launch_rmsnorm(h, out, (int)T, (int)d, eps, dtype, (hipStream_t)stream),
                    "rmsnorm");
}

moe_status moe_forward(const void* x, const void* W_g, const void* const* W1,
                       const void* const* W3, const void* const* W2, int64_t T, int64_t d,
                       int64_t d_ff, int32_t E, int32_t K, int32_t dtype, void* y,
                       int32_t y_dtype, int32_t accumulate, void* workspace,
                       size_t workspace_bytes, void* stream) {
  moe_status s = check_shape(T, d, d_ff, E, K, dtype);
  if (s) return s;
  if ((s = check_dtype(y_dtype, "y_dtype"))) return s;
  if (dtype == MOE_F32 && y_dtype != MOE_F32)
    return fail(MOE_EUNSUPPORTED, "an fp32 layer writes fp32 y");
  if (T == 0) return ok();
  if (!x || !W_g || !y) return fail(MOE_EINVAL, "NULL pointer");
  const bool bf16 = dtype == MOE_BF16;
  moe::ExpertPtrs p1, p3, p2;
  if ((s = fill_ptrs(W1, E, p1, "W1", bf16))) return s;
  if ((s = fill_ptrs(W3, E, p3, "W3", bf16))) return s;
  if ((s = fill_ptrs(W2, E, p2, "W2", bf16))) return s;
  if (bf16 && (!aligned16(x) || !aligned16(y)))
    return fail(MOE_EUNSUPPORTED, "x and y must be 16-byte aligned");
  const size_t xbytes = (size_t)T * d * dtype_bytes(dtype);
  const size_t ybytes = (size_t)T * d * dtype_bytes(y_dtype);
  if (overlap(x, xbytes, y, ybytes)) return fail(MOE_EINVAL, "x and y overlap");
  size_t off[MOE_WS_COUNT], need;
  layout(T, d, d_ff, E, K, dtype, off, &need);
  if (!workspace) return fail(MOE_EWORKSPACE, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(MOE_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MOE_EWORKSPACE, "workspace must be 256-byte aligned");
  if (overlap(workspace, need, x, xbytes) || overlap(workspace, need, y, ybytes))
    return fail(MOE_EINVAL, "workspace overlaps x or y");

  const Bufs b = carve(workspace, off);
  hipStream_t st = (hipStream_t)stream;
  const Plan plan = make_plan(T, d, d_ff, E, K, dtype);
  hipError_t e = moe::launch_router_topk(x, W_g, (int)T, (int)d, E, K, dtype, b.topk_idx,
                                         b.topk_w, nullptr, st);
  if (e != hipSuccess) return hip_status(e, "router_topk");
  if ((s = run_experts(plan, x, p1, p3, p2, b, T, d, d_ff, E, K, dtype, st))) return s;
  e = moe::launch_combine(b.O, plan.down_splits, T * K * d, b.topk_w, b.pos, (int)T, (int)d, K, y,
                          y_dtype, accumulate ? 1 : 0, st);
  if (e != hipSuccess) return hip_status(e, "combine");
  return ok();
}

moe_status moe_stack_workspace_size(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t K,
                                    int32_t dtype, size_t* bytes) {
  if (!bytes) return fail(MOE_EINVAL, "bytes is NULL");
  moe_status s = check_shape(T, d, d_ff, E, K, dtype);
  if (s) return s;
  size_t off[MOE_WS_COUNT], xn_off;
  *bytes = stack_layout(T, d, d_ff, E, K, dtype, off, &xn_off);
  return ok();
}

moe_status moe_stack_forward(void* h, const void* const* W_g, const void* const* W1,
                             const void* const* W3, const void* const* W2, int32_t L, int64_t T,
                             int64_t d, int64_t d_ff, int32_t E, int32_t K, float eps,
                             int32_t dtype, int32_t* stats, void* workspace,
                             size_t workspace_bytes, void* stream) {
  moe_status s = check_shape(T, d, d_ff, E, K, dtype);
  if (s) return s;
  if (L < 0) return fail(MOE_EINVAL, "L = %d < 0", L);
  if (!(eps >= 0.0f)) return fail(MOE_EINVAL, "eps must be >= 0");
  if (T == 0 || L == 0) return ok();
  if (!h || !W_g || !W1 || !W3 || !W2) return fail(MOE_EINVAL, "NULL pointer");
  const bool bf16 = dtype == MOE_BF16;
  if (bf16 && !aligned16(h)) return fail(MOE_EUNSUPPORTED, "h must be 16-byte aligned");
  for (int l = 0; l < L; ++l) {
    if (!W_g[l]) return fail(MOE_EINVAL, "W_g[%d] is NULL", l);
    moe::ExpertPtrs p;
    if ((s = fill_ptrs(W1 + (size_t)l * E, E, p, "W1", bf16))) return s;
    if ((s = fill_ptrs(W3 + (size_t)l * E, E, p, "W3", bf16))) return s;
    if ((s = fill_ptrs(W2 + (size_t)l * E, E, p, "W2", bf16))) return s;
  }
  size_t off[MOE_WS_COUNT], xn_off;
  const size_t need = stack_layout(T, d, d_ff, E, K, dtype, off, &xn_off);
  if (!workspace) return fail(MOE_EWORKSPACE, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(MOE_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MOE_EWORKSPACE, "workspace must be 256-byte aligned");
  const size_t hbytes = (size_t)T * d * dtype_bytes(dtype);
  if (overlap(workspace, need, h, hbytes)) return fail(MOE_EINVAL, "workspace overlaps h");
  if (stats && overlap(stats, (size_t)L * (E + 1) * 4, h, hbytes))
    return fail(MOE_EINVAL, "stats overlaps h");

  const Bufs b = carve(workspace, off);
  void* xn = static_cast<char*>(workspace) + xn_off;
  hipStream_t st = (hipStream_t)stream;
  const Plan plan = make_plan(T, d, d_ff, E, K, dtype);
  const int64_t slice = T * K * d;
  // Small batches join the blocks with one glue launch (the previous block's
  // combine, RMSNorm, this block's router).  Otherwise the previous block's
  // combine and the RMSNorm share one launch where they can (bf16), and the
  // router follows; else all three are launched one by one.  All run the
  // same arithmetic.
  const bool glue = plan.streaming && moe::stack_glue_supported((int)T, (int)d, E, dtype);
  const bool norm = !glue && moe::stack_norm_supported((int)d, dtype);
  hipError_t e = hipSuccess;
  for (int l = 0; l < L; ++l) {
    moe::ExpertPtrs p1, p3, p2;
    fill_ptrs(W1 + (size_t)l * E, E, p1, "W1", bf16);
    fill_ptrs(W3 + (size_t)l * E, E, p3, "W3", bf16);
    fill_ptrs(W2 + (size_t)l * E, E, p2, "W2", bf16);
    if (glue) {
      e = moe::launch_stack_glue(h, xn, l > 0 ? b.O : nullptr, plan.down_splits, slice, b.topk_w,
                                 b.pos, b.topk_idx, W_g[l], (int)T, (int)d, E, K, eps, st);
      if (e != hipSuccess) return hip_status(e, "stack_glue");
    } else {
      e = norm ? moe::launch_stack_norm(h, xn, l > 0 ? b.O : nullptr, plan.down_splits, slice,
                                        b.topk_w, b.pos, (int)T, (int)d, K, eps, st)
               : moe::launch_rmsnorm(h, xn, (int)T, (int)d, eps, dtype, st);
      if (e != hipSuccess) return hip_status(e, "rmsnorm");
      e = moe::launch_router_topk(xn, W_g[l], (int)T, (int)d, E, K, dtype, b.topk_idx, b.topk_w,
                                  nullptr, st);
      if (e != hipSuccess) return hip_status(e, "router_topk");
    }
    if (stats) {
      int32_t* sl = stats + (size_t)l * (E + 1);
      e = moe::launch_routing_stats(b.topk_idx, (int)T, E, K, sl, sl + E, st);
      if (e != hipSuccess) return hip_status(e, "routing_stats");
    }
    if ((s = run_experts(plan, xn, p1, p3, p2, b, T, d, d_ff, E, K, dtype, st))) return s;
    if (!(glue || norm) || l == L - 1) {
      e = moe::launch_combine(b.O, plan.down_splits, slice, b.topk_w, b.pos, (int)T, (int)d, K, h,
                              dtype, 1, st);
      if (e != hipSuccess) return hip_status(e, "combine");
    }
  }
  return ok();
}

// ---- allocation-free variant of moe_forward ----

}  // extern "C"

// The scratch of moe_forward_noalloc: a device array of fixed size, one copy
// per device the library runs on, held until the process ends.  Host code
// never passes this name to a kernel (on the host it is only a stand-in for
// the symbol); the device address comes from hipGetSymbolAddress, once per
// device, and is kept in g_scratch_addr.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current.
moe_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EHIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u))
      return fail(MOE_EHIP, "static scratch has no 256-byte aligned device address");
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward_noalloc(const void* x, const void* W_g, const void* const* W1,
                               const void* const* W3, const void* const* W2, int64_t T,
                               int64_t d, int64_t d_ff, int32_t E, int32_t K, int32_t dtype,
                               void* y, int32_t y_dtype, int32_t accumulate, void* stream) {
  moe_status s = check_shape(T, d, d_ff, E, K, dtype);
  if (s) return s;
  if (T == 0)
    return moe_forward(x, W_g, W1, W3, W2, T, d, d_ff, E, K, dtype, y, y_dtype, accumulate,
                       nullptr, 0, stream);
  size_t off[MOE_WS_COUNT], need;
  layout(T, d, d_ff, E, K, dtype, off, &need);
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_EWORKSPACE,
                "moe_forward_noalloc: this shape needs %zu bytes of scratch, the static scratch "
                "holds %zu; call moe_forward with a workspace instead",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((s = scratch_address(&ws))) return s;
  return moe_forward(x, W_g, W1, W3, W2, T, d, d_ff, E, K, dtype, y, y_dtype, accumulate, ws,
                     (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

// ---- attention sub-block ----

namespace {

moe_status swa_check(int64_t B, int64_t T, int64_t W, int32_t H, int32_t KVH, int32_t hd) {
  if (B < 0 || T < 0) return fail(MOE_EINVAL, "B and T must be >= 0");
  if (W < 1 || W >= (int64_t(1) << 30)) return fail(MOE_EINVAL, "W = %lld out of range", (long long)W);
  if (H < 1 || KVH < 1 || H % KVH != 0)
    return fail(MOE_EINVAL, "n_heads must be a positive multiple of n_kv_heads");
  if (hd != moe::swa_head_dim()) return fail(MOE_EUNSUPPORTED, "head_dim must be 128");
  const int32_t G = H / KVH;
  if (G != 1 && G != 2 && G != 4)
    return fail(MOE_EUNSUPPORTED, "n_heads / n_kv_heads = %d, supported 1, 2, 4", G);
  if (T > W) return fail(MOE_EUNSUPPORTED, "a chunk is at most W tokens (T = %lld, W = %lld)",
                         (long long)T, (long long)W);
  if (B * T * H * hd >= (int64_t(1) << 31) || B * W * KVH * hd >= (int64_t(1) << 40))
    return fail(MOE_EUNSUPPORTED, "shape too large");
  return MOE_OK;
}

size_t swa_ws_bytes(int64_t B, int64_t T, int64_t W, int32_t H, int32_t KVH) {
  const int splits = moe::swa_plan_splits((int)B, (int)T, (int)W, H, KVH, nullptr, nullptr);
  if (splits <= 1 || B == 0 || T == 0) return 0;
  const size_t rows = (size_t)B * T * H * splits;
  const size_t o = (rows * 128 * sizeof(float) + 255) / 256 * 256;
  return o + rows * 2 * sizeof(float);
}

}  // namespace

moe_status swa_workspace_size(int64_t B, int64_t T, int64_t W, int32_t n_heads,
                              int32_t n_kv_heads, int32_t head_dim, size_t* bytes) {
  if (!bytes) return fail(MOE_EINVAL, "bytes is NULL");
  moe_status s = swa_check(B, T, W, n_heads, n_kv_heads, head_dim);
  if (s) return s;
  *bytes = swa_ws_bytes(B, T, W, n_heads, n_kv_heads);
  return ok();
}

moe_status swa_attention(const void* q, const void* k_new, const void* v_new,
                         const void* k_cache, const void* v_cache, const int32_t* pos0,
                         int64_t B, int64_t T, int64_t W, int32_t n_heads, int32_t n_kv_heads,
                         int32_t head_dim, void* out, int32_t out_dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  moe_status s = swa_check(B, T, W, n_heads, n_kv_heads, head_dim);
  if (s) return s;
  s = check_dtype(out_dtype, "out_dtype");
  if (s) return s;
  if (B == 0 || T == 0) return ok();
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !pos0 || !out)
    return fail(MOE_EINVAL, "NULL pointer");
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(out))
    return fail(MOE_EUNSUPPORTED, "q, k_new, v_new, caches and out must be 16-byte aligned");
  const size_t qbytes = (size_t)B * T * n_heads * head_dim * 2;
  const size_t obytes = (size_t)B * T * n_heads * head_dim * (out_dtype == MOE_F32 ? 4 : 2);
  const size_t nbytes = (size_t)B * T * n_kv_heads * head_dim * 2;
  const size_t cbytes = (size_t)B * W * n_kv_heads * head_dim * 2;
  if (overlap(out, obytes, q, qbytes) || overlap(out, obytes, k_new, nbytes) ||
      overlap(out, obytes, v_new, nbytes) || overlap(out, obytes, k_cache, cbytes) ||
      overlap(out, obytes, v_cache, cbytes))
    return fail(MOE_EINVAL, "out overlaps an input");
  const size_t need = swa_ws_bytes(B, T, W, n_heads, n_kv_heads);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(MOE_EWORKSPACE, "workspace has %zu bytes, needs %zu",
                  workspace ? workspace_bytes : 0, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(MOE_EWORKSPACE, "workspace must be 256-byte aligned");
    const int splits = moe::swa_plan_splits((int)B, (int)T, (int)W, n_heads, n_kv_heads,
                                            nullptr, nullptr);
    const size_t rows = (size_t)B * T * n_heads * splits;
    part_o = static_cast<float*>(workspace);
    part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       (rows * 128 * sizeof(float) + 255) / 256 * 256);
  }
  return finish(moe::launch_swa_attention(q, k_new, v_new, k_cache, v_cache, pos0, (int)B,
                                          (int)T, (int)W, n_heads, n_kv_heads, out,
                                          out_dtype == MOE_F32 ? 1 : 0, part_o, part_ml,
                                          (hipStream_t)stream),
                "swa_attention");
}

moe_status swa_cache_append(const void* k_new, const void* v_new, const int32_t* pos0,
                            int64_t B, int64_t T, int64_t W, int32_t n_kv_heads, int32_t head_dim,
                            void* k_cache, void* v_cache, void* stream) {
  if (B < 0 || T < 0) return fail(MOE_EINVAL, "B and T must be >= 0");
  if (W < 1 || W >= (int64_t(1) << 30)) return fail(MOE_EINVAL, "W out of range");
  if (n_kv_heads < 1) return fail(MOE_EINVAL, "n_kv_heads must be >= 1");
  if (head_dim != moe::swa_head_dim()) return fail(MOE_EUNSUPPORTED, "head_dim must be 128");
  if (B == 0 || T == 0) return ok();
  if (!k_new || !v_new || !pos0 || !k_cache || !v_cache) return fail(MOE_EINVAL, "NULL pointer");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(MOE_EUNSUPPORTED, "keys, values and caches must be 16-byte aligned");
  if (B * T * n_kv_heads * head_dim >= (int64_t(1) << 40)) return fail(MOE_EUNSUPPORTED, "too large");
  return finish(moe::launch_swa_append(k_new, v_new, pos0, (int)B, (int)T, (int)W, n_kv_heads,
                                       k_cache, v_cache, (hipStream_t)stream),
                "swa_cache_append");
}

}  // extern "C"
