// C ABI of the MoE library: argument validation, workspace layout and
// dispatch to the gfx950 kernels.  Every check runs on the host before any
// HIP call; no C++ exception crosses the boundary.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "launch.h"
#include "select.h"

namespace {

thread_local char g_detail[512] = "";
thread_local size_t g_required_ws = 0;

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_detail[0] = '\0';
  return MOE_OK;
}

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Smallest M tile of the grouped GEMM (sizes the tile list).
constexpr int kMinTileBM = 32;

struct WsLayout {
  size_t header, slots, tile_desc, chunk_hist, h_routed, h_shared, x16;
  size_t end_perm, end_ffn;
  size_t logits, end_route;
  size_t topk_idx, topk_w, counts, offsets, sorted_pair, pair_pos, slot_expert, y_sorted, shared_out, total;
  int64_t max_tiles;
};

WsLayout ws_layout(const moe_shape& s, int64_t T) {
  WsLayout L{};
  const int64_t P = T * s.top_k;
  const int64_t E = s.n_experts;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += up(bytes);
    return at;
  };
  L.max_tiles = (P + kMinTileBM - 1) / kMinTileBM + std::min<int64_t>(E, P) +
                (s.shared_inter > 0 ? (T + kMinTileBM - 1) / kMinTileBM : 0) + 2;
  L.header = take(moe::kHdrWords * 4);
  L.slots = take(size_t(E + 1) * 16);
  L.tile_desc = take(size_t(L.max_tiles) * 16);
  // chunk rows of the multi-workgroup permutation: moe_permute's (kPermChunk pairs each) or the
  // prefill layer's (moe::select_chunks: 16 tokens each, at least as many)
  const int64_t n_chunks =
      P > moe::kSmallPairs ? std::max<int64_t>((P + moe::kPermChunk - 1) / moe::kPermChunk, moe::select_chunks(T)) : 0;
  L.chunk_hist = take(size_t(n_chunks) * size_t(E + 1) * 4);
  L.end_perm = off;
  L.h_routed = take(size_t(P) * s.inter * 2);
  L.h_shared = take(size_t(T) * s.shared_inter * 2);
  L.x16 = take(size_t(T) * s.hidden * 2);
  L.end_ffn = off;
  L.logits = take(size_t(T) * E * 4);
  L.end_route = off;
  L.topk_idx = take(size_t(P) * 4);
  L.topk_w = take(size_t(P) * 4);
  L.counts = take(size_t(E) * 4);
  L.offsets = take(size_t(E + 1) * 4);
  L.sorted_pair = take(size_t(P) * 4);
  L.pair_pos = take(size_t(P) * 4);
  L.slot_expert = take(size_t(moe::kMaxTopK) * 4);
  L.y_sorted = take(size_t(P) * s.hidden * 4);
  L.shared_out = take(s.shared_inter > 0 ? size_t(T) * s.hidden * 4 : 0);
  L.total = off;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return MOE_OK;
  if (ws == nullptr || have < need) {
    g_required_ws = need;
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes is too small: %zu bytes needed (%zu MiB short)", have,
                need, (need - std::min(need, have) + (1u << 20) - 1) >> 20);
  }
  if (!aligned(ws, kAlign)) return fail(MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return MOE_OK;
}

int check_shape(const moe_shape* s) {
  if (!s) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (s->hidden <= 0 || s->hidden % 32) return fail(MOE_ERR_INVALID_ARG, "hidden=%d must be a positive multiple of 32", s->hidden);
  if (s->inter <= 0 || s->inter % 32) return fail(MOE_ERR_INVALID_ARG, "inter=%d must be a positive multiple of 32", s->inter);
  if (s->shared_inter < 0 || s->shared_inter % 32)
    return fail(MOE_ERR_INVALID_ARG, "shared_inter=%d must be 0 or a positive multiple of 32", s->shared_inter);
  if (s->n_experts < 1 || s->n_experts > moe::kMaxExperts)
    return fail(MOE_ERR_INVALID_ARG, "n_experts=%d must be in [1, %d]", s->n_experts, moe::kMaxExperts);
  if (s->top_k < 1 || s->top_k > std::min(s->n_experts, moe::kMaxTopK))
    return fail(MOE_ERR_INVALID_ARG, "top_k=%d must be in [1, min(n_experts, %d)]", s->top_k, moe::kMaxTopK);
  if (s->qbits < 2 || s->qbits > 4) return fail(MOE_ERR_UNSUPPORTED, "qbits=%d: only 2, 3 and 4 are supported", s->qbits);
  return MOE_OK;
}

int check_T(int64_t T, const moe_shape* s) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%lld must be >= 0", (long long)T);
  if (T * int64_t(s->top_k) > INT32_MAX) return fail(MOE_ERR_INVALID_ARG, "T*top_k exceeds 2^31-1");
  return MOE_OK;
}

// Router weights: fp32 or bf16.
int check_dtype(moe_dtype d, const char* what) {
  if (d != MOE_F32 && d != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "%s dtype %d is not MOE_F32 or MOE_BF16", what, int(d));
  return MOE_OK;
}

// Activations: fp32, bf16 or fp16.
int check_x_dtype(moe_dtype d) {
  if (d != MOE_F32 && d != MOE_BF16 && d != MOE_F16)
    return fail(MOE_ERR_INVALID_ARG, "x dtype %d is not MOE_F32, MOE_BF16 or MOE_F16", int(d));
  return MOE_OK;
}

int x_kind(moe_dtype d) { return d == MOE_BF16 ? moe::kXBF16 : d == MOE_F16 ? moe::kXF16 : moe::kXF32; }

int check_qw(const moe_qweights& q, const char* what, int n) {
  for (int m = 0; m < 3; ++m) {
    if (!q.codes[m] || !q.scales[m]) return fail(MOE_ERR_INVALID_ARG, "%s: codes/scales[%d] is NULL", what, m);
    if (!aligned(q.codes[m], 16)) return fail(MOE_ERR_INVALID_ARG, "%s: codes[%d] must be 16-byte aligned", what, m);
    if (!aligned(q.scales[m], 4)) return fail(MOE_ERR_INVALID_ARG, "%s: scales[%d] must be 4-byte aligned", what, m);
  }
  if (n > 1) {
    if (q.code_stride <= 0 || q.code_stride % 16)
      return fail(MOE_ERR_INVALID_ARG, "%s: code_stride=%lld must be a positive multiple of 16", what, (long long)q.code_stride);
    if (q.scale_stride <= 0 || q.scale_stride % 2)
      return fail(MOE_ERR_INVALID_ARG, "%s: scale_stride=%lld must be a positive even count", what, (long long)q.scale_stride);
  }
  return MOE_OK;
}

int check_layer(const moe_layer* L, const moe_shape* s, bool need_router, bool need_experts) {
  if (!L) return fail(MOE_ERR_INVALID_ARG, "layer is NULL");
  if (need_router) {
    if (!L->w_router) return fail(MOE_ERR_INVALID_ARG, "w_router is NULL");
    if (int r = check_dtype(L->router_dtype, "router")) return r;
  }
  if (need_experts) {
    if (int r = check_qw(L->experts, "experts", s->n_experts)) return r;
    if (s->shared_inter > 0)
      if (int r = check_qw(L->shared, "shared", 1)) return r;
  }
  return MOE_OK;
}

moe::QMat qmat(const moe_qweights& q, int m) { return moe::QMat{q.codes[m], q.scales[m], q.code_stride, q.scale_stride}; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

moe_algo pick_algo(const moe_options* o, int64_t T, const moe_shape* s) {
  const moe_algo a = o ? o->ffn_algo : MOE_ALGO_AUTO;
  if (a != MOE_ALGO_AUTO) return a;
  return T <= 16 && moe::gemv_lds_ok(T, s->hidden, s->inter, s->shared_inter) ? MOE_ALGO_GEMV : MOE_ALGO_GROUPED;
}

// The route tail skip's first tail rank (the pages' 7) when it applies: the
// option is set, the layer is one verify window (T <= 4) and the top-k has a
// tail (k > 7); else 0.
constexpr int kTailSkipRank = 7;
constexpr int64_t kVerifyWindow = 4;
int tail_skip_rank(const moe_options* o, int64_t T, const moe_shape* s) {
  const bool on = o && (o->flags & MOE_LAYER_ROUTE_TAIL_SKIP);
  return on && T <= kVerifyWindow && s->top_k > kTailSkipRank ? kTailSkipRank : 0;
}

int check_algo(moe_algo algo, int64_t T, const moe_shape* s) {
  if (algo == MOE_ALGO_GEMV && !moe::gemv_lds_ok(T, s->hidden, s->inter, s->shared_inter))
    return fail(MOE_ERR_UNSUPPORTED, "the GEMV kernels stage min(T, 16) token rows of hidden=%d and inter=%d in LDS, "
                "which does not fit at T=%lld; use MOE_ALGO_GROUPED", s->hidden, std::max(s->inter, s->shared_inter),
                (long long)T);
  return MOE_OK;
}

enum OptsFor { kOptsPlain, kOptsFfn, kOptsLayer };

int check_opts(const moe_options* o, OptsFor what = kOptsPlain) {
  if (!o) return MOE_OK;
  if (o->ffn_algo < MOE_ALGO_AUTO || o->ffn_algo > MOE_ALGO_GROUPED)
    return fail(MOE_ERR_INVALID_ARG, "ffn_algo=%d is not a moe_algo", int(o->ffn_algo));
  const int allowed = what == kOptsFfn     ? (MOE_FFN_REUSE_PLAN | MOE_FFN_SKIP_GATEUP | MOE_FFN_SKIP_DOWN)
                      : what == kOptsLayer ? MOE_LAYER_ROUTE_TAIL_SKIP
                                           : 0;
  if (o->flags & ~allowed) return fail(MOE_ERR_INVALID_ARG, "flags=0x%x not accepted by this call", unsigned(o->flags));
  return MOE_OK;
}

// ---- the steps, shared by the single-step entry points and layer_forward

// Router logits: bf16 x bf16 on MFMA (products exact, fp32 accumulation),
// anything with fp32 operands on the vector ALUs.
hipError_t route_logits(const void* x, moe_dtype xd, int64_t T, const moe_layer* L, const moe_shape* s,
                        float* logits, hipStream_t st) {
  if (xd == MOE_BF16 && L->router_dtype == MOE_BF16)
    return moe::launch_router_mfma(static_cast<const uint16_t*>(x), T, s->hidden,
                                   static_cast<const uint16_t*>(L->w_router), L->router_bias, s->n_experts, logits,
                                   st);
  return moe::launch_router_gemv(x, x_kind(xd), T, s->hidden, L->w_router, L->router_dtype == MOE_BF16,
                                 L->router_bias, s->n_experts, logits, st);
}

hipError_t do_route(const void* x, moe_dtype xd, int64_t T, const moe_layer* L, const moe_shape* s, float* logits,
                    int32_t* idx, float* w, hipStream_t st) {
  hipError_t e = route_logits(x, xd, T, L, s, logits, st);
  if (e != hipSuccess) return e;
  return moe::launch_topk(logits, T, s->n_experts, s->top_k, idx, w, st);
}

moe::FfnArgs ffn_args(const void* x, moe_dtype xd, int64_t T, const moe_layer* L, const moe_shape* s,
                      const int32_t* offsets, const int32_t* sorted_pair, float* y_sorted, float* shared_out,
                      void* ws, const WsLayout& W) {
  moe::FfnArgs a{};
  a.x = x;
  a.x_kind = x_kind(xd);
  a.T = T;
  a.H = s->hidden;
  a.I = s->inter;
  a.Is = s->shared_inter;
  a.k = s->top_k;
  a.E = s->n_experts;
  a.qbits = s->qbits;
  a.has_shared = s->shared_inter > 0 && shared_out != nullptr;
  a.rg = qmat(L->experts, 0);
  a.ru = qmat(L->experts, 1);
  a.rd = qmat(L->experts, 2);
  if (s->shared_inter > 0) {
    a.sg = qmat(L->shared, 0);
    a.su = qmat(L->shared, 1);
    a.sd = qmat(L->shared, 2);
  }
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.header = at<int32_t>(ws, W.header);
  a.slots = at<int4>(ws, W.slots);
  a.tile_desc = at<int4>(ws, W.tile_desc);
  a.h_routed = at<_Float16>(ws, W.h_routed);
  a.h_shared = at<_Float16>(ws, W.h_shared);
  a.x16 = at<_Float16>(ws, W.x16);
  a.y_sorted = y_sorted;
  a.shared_out = shared_out;
  return a;
}

hipError_t do_ffn(const void* x, moe_dtype xd, int64_t T, const moe_layer* L, const moe_shape* s,
                  const int32_t* offsets, const int32_t* sorted_pair, float* y_sorted, float* shared_out,
                  moe_algo algo, void* ws, const WsLayout& W, hipStream_t st, int flags = 0,
                  _Float16* y_sorted_h = nullptr, _Float16* shared_out_h = nullptr) {
  moe::FfnArgs a = ffn_args(x, xd, T, L, s, offsets, sorted_pair, y_sorted, shared_out, ws, W);
  a.y_sorted_h = y_sorted_h;
  a.shared_out_h = shared_out_h;
  const int tile_bm = algo == MOE_ALGO_GROUPED ? moe::grouped_tile_rows(T, s->top_k, s->n_experts) : 0;
  if (!(flags & MOE_FFN_REUSE_PLAN)) {
    hipError_t e = moe::launch_plan(offsets, s->n_experts, T, a.has_shared, tile_bm, at<int32_t>(ws, W.header),
                                    at<int4>(ws, W.slots), at<int4>(ws, W.tile_desc), sorted_pair, s->top_k, st);
    if (e != hipSuccess) return e;
    if (algo == MOE_ALGO_GROUPED) {  // the grouped gate/up GEMM reads x through its fp16 copy
      e = moe::launch_x16(a, st);
      if (e != hipSuccess) return e;
    }
  }
  const int phases = (flags & MOE_FFN_SKIP_GATEUP ? 0 : moe::kPhaseGateUp) | (flags & MOE_FFN_SKIP_DOWN ? 0 : moe::kPhaseDown);
  if (algo == MOE_ALGO_GROUPED) {
    const int64_t P = T * s->top_k, BM = tile_bm;
    const int64_t max_tiles = (P + BM - 1) / BM + std::min<int64_t>(s->n_experts, P) +
                              (a.has_shared ? (T + BM - 1) / BM : 0);
    return moe::launch_ffn_grouped(a, max_tiles, tile_bm, st, phases);
  }
  return moe::launch_ffn_gemv(a, st, phases);
}

// The decode layer in five launches: router, one-workgroup selection (top-k,
// permutation, slot table), gate/up GEMV, down GEMV, combine (with the stack
// glue).  No workgroup waits on another inside a kernel.
bool fused_decode_ok(int64_t T, const moe_shape* s, moe_algo algo) {
  return algo == MOE_ALGO_GEMV && T <= 16 && T * s->top_k <= 1024;
}

hipError_t fused_decode(const void* x, moe_dtype xd, int64_t T, const moe_layer* L, const moe_shape* s, float* out,
                        float* residual, uint16_t* next_in, int32_t* idx, float* w, void* ws, const WsLayout& W,
                        hipStream_t st, int kc) {
  float* logits = at<float>(ws, W.logits);
  hipError_t e = route_logits(x, xd, T, L, s, logits, st);
  if (e != hipSuccess) return e;
  int32_t* offsets = at<int32_t>(ws, W.offsets);
  int32_t* sorted_pair = at<int32_t>(ws, W.sorted_pair);
  int32_t* pair_pos = at<int32_t>(ws, W.pair_pos);
  float* y = at<float>(ws, W.y_sorted);
  float* s_out = s->shared_inter > 0 ? at<float>(ws, W.shared_out) : nullptr;
  moe::FfnArgs a = ffn_args(x, xd, T, L, s, offsets, sorted_pair, y, s_out, ws, W);
  const moe::SelOut so{logits, idx, w, at<int32_t>(ws, W.counts), offsets, sorted_pair, pair_pos,
                       at<int32_t>(ws, W.header), at<int4>(ws, W.slots), kc};
  // the gate/up kernel makes the selection itself where it can, else a selection launch first
  e = moe::launch_gateup_select(a, so, st);
  if (e == hipErrorNotSupported) {
    e = moe::launch_select_small(logits, int(T), s->n_experts, s->top_k, s_out != nullptr, idx, w,
                                 at<int32_t>(ws, W.counts), offsets, sorted_pair, pair_pos,
                                 at<int32_t>(ws, W.header), at<int4>(ws, W.slots), kc, st);
    if (e != hipSuccess) return e;
    e = moe::launch_ffn_gemv(a, st, moe::kPhaseGateUp);
  }
  if (e != hipSuccess) return e;
  e = moe::launch_ffn_gemv(a, st, moe::kPhaseDown);
  if (e != hipSuccess) return e;
  return moe::launch_combine(y, pair_pos, w, s_out, T, s->hidden, s->top_k, out, residual, next_in, st);
}

// The single-token decode layer in three launches (four with the stack
// glue): router logits; gate/up with the top-k made from the logits inside
// every workgroup (no selection kernel, no slot table); down projection of
// all selected experts and the shared expert with the combine done inside
// the workgroup; then the residual RMSNorm when next_in is asked for.
bool decode1_ok(int64_t T, const moe_shape* s, moe_algo algo) {
  return algo == MOE_ALGO_GEMV && T == 1 && s->n_experts <= moe::kDecode1MaxExperts &&
         moe::decode1_lds_ok(s->hidden, s->inter, s->shared_inter, s->top_k, s->shared_inter > 0);
}

hipError_t decode1(const void* x, moe_dtype xd, const moe_layer* L, const moe_shape* s, float* out, float* residual,
                   uint16_t* next_in, int32_t* idx, float* w, void* ws, const WsLayout& W, hipStream_t st, int kc) {
  float* logits = at<float>(ws, W.logits);
  hipError_t e = route_logits(x, xd, 1, L, s, logits, st);
  if (e != hipSuccess) return e;
  float* s_out = s->shared_inter > 0 ? at<float>(ws, W.shared_out) : nullptr;  // only marks the shared expert
  moe::FfnArgs a = ffn_args(x, xd, 1, L, s, nullptr, nullptr, nullptr, s_out, ws, W);
  const moe::Decode1Sel sel{logits, idx, w, at<int32_t>(ws, W.pair_pos), at<int32_t>(ws, W.slot_expert),
                            at<int32_t>(ws, W.header), kc};
  e = moe::launch_decode1_ffn(a, sel, out, residual, st);
  if (e != hipSuccess || !next_in) return e;
  return moe::launch_residual_rmsnorm(residual, 1, s->hidden, next_in, st);
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    case MOE_ERR_INDEX: return "MOE_ERR_INDEX";
    default: return "unknown moe_status";
  }
}

const char* moe_last_error_detail(void) { return g_detail; }
size_t moe_last_required_workspace(void) { return g_required_ws; }

size_t moe_workspace_bytes(const moe_shape* shape, int64_t T, const moe_options* opts) {
  if (check_shape(shape) || check_T(T, shape) || check_opts(opts)) return 0;
  return ws_layout(*shape, T).total;
}

int moe_route(const void* x, moe_dtype x_dtype, int64_t T, const moe_layer* layer, const moe_shape* shape,
              float* logits, int32_t* topk_idx, float* topk_w, void* workspace, size_t workspace_bytes,
              void* stream) {
  try {
    if (int r = check_shape(shape)) return r;
    if (int r = check_T(T, shape)) return r;
    if (int r = check_layer(layer, shape, true, false)) return r;
    if (int r = check_x_dtype(x_dtype)) return r;
    if (T == 0) return ok();
    if (!x || !topk_idx || !topk_w) return fail(MOE_ERR_INVALID_ARG, "x, topk_idx and topk_w must be non-NULL");
    const WsLayout W = ws_layout(*shape, T);
    if (!logits) {
      if (int r = check_ws(workspace, workspace_bytes, W.end_route)) return r;
      logits = at<float>(workspace, W.logits);
    }
    return device_status(do_route(x, x_dtype, T, layer, shape, logits, topk_idx, topk_w, as_stream(stream)),
                         "moe_route");
  } catch (...) {
    return fail(MOE_ERR_DEVICE, "moe_route: unexpected exception");
  }
}

int moe_permute(const int32_t* topk_idx, int64_t T, const moe_shape* shape, int32_t* counts, int32_t* offsets,
                int32_t* sorted_pair, int32_t* pair_pos, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (int r = check_shape(shape)) return r;
    if (int r = check_T(T, shape)) return r;
    if (!counts || !offsets) return fail(MOE_ERR_INVALID_ARG, "counts and offsets must be non-NULL");
    if (T > 0 && (!topk_idx || !sorted_pair || !pair_pos))
      return fail(MOE_ERR_INVALID_ARG, "topk_idx, sorted_pair and pair_pos must be non-NULL");
    const WsLayout W = ws_layout(*shape, T);
    if (int r = check_ws(workspace, workspace_bytes, W.end_perm)) return r;
    return device_status(moe::launch_permute(topk_idx, T * shape->top_k, shape->n_experts, counts, offsets,
                                             sorted_pair, pair_pos, at<int32_t>(workspace, W.header),
                                             at<int32_t>(workspace, W.chunk_hist), as_stream(stream)),
                         "moe_permute");
  } catch (...) {
    return fail(MOE_ERR_DEVICE, "moe_permute: unexpected exception");
  }
}

int moe_expert_ffn(const void* x, moe_dtype x_dtype, int64_t T, const moe_layer* layer, const moe_shape* shape,
                   const int32_t* offsets, const int32_t* sorted_pair, float* y_sorted, float* shared_out,
                   const moe_options* opts, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (int r = check_shape(shape)) return r;
    if (int r = check_T(T, shape)) return r;
    if (int r = check_opts(opts, kOptsFfn)) return r;
    if (int r = check_layer(layer, shape, false, true)) return r;
    if (int r = check_x_dtype(x_dtype)) return r;
    if (T == 0) return ok();
    if (!x || !offsets || !sorted_pair || !y_sorted)
      return fail(MOE_ERR_INVALID_ARG, "x, offsets, sorted_pair and y_sorted must be non-NULL");
    if (!aligned(x, 16) || !aligned(y_sorted, 16) || (shared_out && !aligned(shared_out, 16)))
      return fail(MOE_ERR_INVALID_ARG, "x, y_sorted and shared_out must be 16-byte aligned");
    const WsLayout W = ws_layout(*shape, T);
    if (int r = check_ws(workspace, workspace_bytes, W.end_ffn)) return r;
    const moe_algo algo = pick_algo(opts, T, shape);
    if (int r = check_algo(algo, T, shape)) return r;
    return device_status(do_ffn(x, x_dtype, T, layer, shape, offsets, sorted_pair, y_sorted, shared_out, algo,
                                workspace, W, as_stream(stream), opts ? opts->flags : 0),
                         "moe_expert_ffn");
  } catch (...) {
    return fail(MOE_ERR_DEVICE, "moe_expert_ffn: unexpected exception");
  }
}

int moe_combine(const float* y_sorted, const int32_t* pair_pos, const float* topk_w, const float* shared_out,
                int64_t T, const moe_shape* shape, float* out, float* residual, uint16_t* next_in_bf16,
                void* stream) {
  try {
    if (int r = check_shape(shape)) return r;
    if (int r = check_T(T, shape)) return r;
    if (T == 0) return ok();
    if (!y_sorted || !pair_pos || !topk_w) return fail(MOE_ERR_INVALID_ARG, "y_sorted, pair_pos and topk_w must be non-NULL");
    if (!out && !residual) return fail(MOE_ERR_INVALID_ARG, "one of out and residual must be non-NULL");
    if (next_in_bf16 && !residual) return fail(MOE_ERR_INVALID_ARG, "next_in_bf16 needs residual");
    for (const void* p : {(const void*)y_sorted, (const void*)shared_out, (const void*)out, (const void*)residual})
      if (p && !aligned(p, 16)) return fail(MOE_ERR_INVALID_ARG, "float tensors must be 16-byte aligned");
    return device_status(moe::launch_combine(y_sorted, pair_pos, topk_w, shared_out, T, shape->hidden,
                                             shape->top_k, out, residual, next_in_bf16, as_stream(stream)),
                         "moe_combine");
  } catch (...) {
    return fail(MOE_ERR_DEVICE, "moe_combine: unexpected exception");
  }
}

}  // extern "C"

namespace {

// Argument checks of the whole layer (both entry points), before any HIP call.
int check_layer_forward(const void* x, moe_dtype x_dtype, int64_t T, const moe_layer* layer, const moe_shape* shape,
                        const float* out, const float* residual, const uint16_t* next_in_bf16,
                        const moe_options* opts) {
  if (int r = check_shape(shape)) return r;
  if (int r = check_T(T, shape)) return r;
  if (int r = check_opts(opts, kOptsLayer)) return r;
  if (int r = check_layer(layer, shape, true, true)) return r;
  if (int r = check_x_dtype(x_dtype)) return r;
  if (T == 0) return MOE_OK;
  if (tail_skip_rank(opts, T, shape) && pick_algo(opts, T, shape) != MOE_ALGO_GEMV)
    return fail(MOE_ERR_UNSUPPORTED, "the route tail skip runs on the GEMV (decode) path; T=%lld takes the grouped "
                "GEMM here", (long long)T);
  if (!x) return fail(MOE_ERR_INVALID_ARG, "x is NULL");
  if (!out && !residual) return fail(MOE_ERR_INVALID_ARG, "one of out and residual must be non-NULL");
  if (next_in_bf16 && !residual) return fail(MOE_ERR_INVALID_ARG, "next_in_bf16 needs residual");
  for (const void* p : {(const void*)x, (const void*)out, (const void*)residual})
    if (p && !aligned(p, 16)) return fail(MOE_ERR_INVALID_ARG, "x, out and residual must be 16-byte aligned");
  return MOE_OK;
}

// The layer on a checked workspace of W.total bytes at ws.
int layer_forward_ws(const void* x, moe_dtype x_dtype, int64_t T, const moe_layer* layer, const moe_shape* shape,
                     float* out, float* residual, uint16_t* next_in_bf16, int32_t* topk_idx, float* topk_w,
                     const moe_options* opts, void* ws, const WsLayout& W, hipStream_t st) {
  {
    int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, W.topk_idx);
    float* w = topk_w ? topk_w : at<float>(ws, W.topk_w);
    const moe_algo algo = pick_algo(opts, T, shape);
    if (int r = check_algo(algo, T, shape)) return r;
    const int kc = tail_skip_rank(opts, T, shape);
    if (decode1_ok(T, shape, algo))
      return device_status(decode1(x, x_dtype, layer, shape, out, residual, next_in_bf16, idx, w, ws, W, st, kc),
                           "moe_layer_forward");
    if (fused_decode_ok(T, shape, algo))
      return device_status(fused_decode(x, x_dtype, T, layer, shape, out, residual, next_in_bf16, idx, w, ws, W, st,
                                        kc),
                           "moe_layer_forward");
    int32_t* offsets = at<int32_t>(ws, W.offsets);
    int32_t* sorted_pair = at<int32_t>(ws, W.sorted_pair);
    int32_t* pair_pos = at<int32_t>(ws, W.pair_pos);
    float* y = at<float>(ws, W.y_sorted);
    float* s_out = shape->shared_inter > 0 ? at<float>(ws, W.shared_out) : nullptr;
    // the grouped GEMM hands the routed and shared rows to the combine in fp16 (half the bytes of
    // the layer's largest intermediates); the stand-alone moe_expert_ffn / moe_combine keep fp32
    _Float16* yh = algo == MOE_ALGO_GROUPED ? reinterpret_cast<_Float16*>(y) : nullptr;
    _Float16* sh = algo == MOE_ALGO_GROUPED ? reinterpret_cast<_Float16*>(s_out) : nullptr;
    int ffn_flags = 0;
    hipError_t e;
    if (algo == MOE_ALGO_GROUPED && T * shape->top_k > moe::kSmallPairs) {
      // prefill: top-k, permutation, plan and the fp16 copy of x in three launches
      e = route_logits(x, x_dtype, T, layer, shape, at<float>(ws, W.logits), st);
      if (e != hipSuccess) return device_status(e, "moe_layer_forward/route");
      const moe::FfnArgs a = ffn_args(x, x_dtype, T, layer, shape, offsets, sorted_pair, y, s_out, ws, W);
      const moe::PlanOut plan{a.has_shared ? 1 : 0, moe::grouped_tile_rows(T, shape->top_k, shape->n_experts),
                              at<int32_t>(ws, W.header), at<int4>(ws, W.slots), at<int4>(ws, W.tile_desc)};
      e = moe::launch_select_plan(at<float>(ws, W.logits), x, x_kind(x_dtype), T, shape->hidden, shape->n_experts,
                                  shape->top_k, idx, w, at<int32_t>(ws, W.chunk_hist), at<int32_t>(ws, W.counts),
                                  offsets, sorted_pair, pair_pos, a.x16, plan, st);
      if (e != hipSuccess) return device_status(e, "moe_layer_forward/select");
      ffn_flags = MOE_FFN_REUSE_PLAN;
    } else {
      e = do_route(x, x_dtype, T, layer, shape, at<float>(ws, W.logits), idx, w, st);
      if (e != hipSuccess) return device_status(e, "moe_layer_forward/route");
      e = moe::launch_permute(idx, T * shape->top_k, shape->n_experts, at<int32_t>(ws, W.counts), offsets,
                              sorted_pair, pair_pos, at<int32_t>(ws, W.header), at<int32_t>(ws, W.chunk_hist), st);
      if (e != hipSuccess) return device_status(e, "moe_layer_forward/permute");
    }
    e = do_ffn(x, x_dtype, T, layer, shape, offsets, sorted_pair, y, s_out, algo, ws, W, st, ffn_flags, yh, sh);
    if (e != hipSuccess) return device_status(e, "moe_layer_forward/ffn");
    e = yh ? moe::launch_combine_f16y(yh, pair_pos, w, sh, T, shape->hidden, shape->top_k, out, residual,
                                      next_in_bf16, st)
           : moe::launch_combine(y, pair_pos, w, s_out, T, shape->hidden, shape->top_k, out, residual,
                                 next_in_bf16, st);
    return device_status(e, "moe_layer_forward/combine");
  }
}

// ---- the no-allocation variant: its workspace is a file-scope device array.
// In host code `scratch` names a host-side stand-in, never the device memory:
// only the address hipGetSymbolAddress returns for the current device is
// used (kernel arguments and every other host-side use).
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device, looked up once
// per device.
int scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "moe_layer_forward_noalloc/hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_status(e, "moe_layer_forward_noalloc/hipGetSymbolAddress");
    if (!p || !aligned(p, kAlign)) return fail(MOE_ERR_DEVICE, "scratch array address %p is not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer_forward(const void* x, moe_dtype x_dtype, int64_t T, const moe_layer* layer, const moe_shape* shape,
                      float* out, float* residual, uint16_t* next_in_bf16, int32_t* topk_idx, float* topk_w,
                      const moe_options* opts, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (int r = check_layer_forward(x, x_dtype, T, layer, shape, out, residual, next_in_bf16, opts)) return r;
    if (T == 0) return ok();
    const WsLayout W = ws_layout(*shape, T);
    if (int r = check_ws(workspace, workspace_bytes, W.total)) return r;
    return layer_forward_ws(x, x_dtype, T, layer, shape, out, residual, next_in_bf16, topk_idx, topk_w, opts,
                            workspace, W, as_stream(stream));
  } catch (...) {
    return fail(MOE_ERR_DEVICE, "moe_layer_forward: unexpected exception");
  }
}

int moe_layer_forward_noalloc(const void* x, moe_dtype x_dtype, int64_t T, const moe_layer* layer,
                              const moe_shape* shape, float* out, float* residual, uint16_t* next_in_bf16,
                              int32_t* topk_idx, float* topk_w, const moe_options* opts, void* stream) {
  try {
    if (int r = check_layer_forward(x, x_dtype, T, layer, shape, out, residual, next_in_bf16, opts)) return r;
    if (T == 0) return ok();
    const WsLayout W = ws_layout(*shape, T);
    if (W.total > kScratchBytes)
      return fail(MOE_ERR_UNSUPPORTED, "moe_layer_forward_noalloc: this shape needs %zu bytes of workspace at T=%lld; "
                  "the scratch array holds %zu (use moe_layer_forward with a workspace)", W.total, (long long)T,
                  kScratchBytes);
    void* ws = nullptr;
    if (int r = scratch_of_current_device(&ws)) return r;
    return layer_forward_ws(x, x_dtype, T, layer, shape, out, residual, next_in_bf16, topk_idx, topk_w, opts, ws, W,
                            as_stream(stream));
  } catch (...) {
    return fail(MOE_ERR_DEVICE, "moe_layer_forward_noalloc: unexpected exception");
  }
}

int moe_rmsnorm_bf16(const float* r, int64_t T, int32_t H, uint16_t* a, void* stream) {
  if (T < 0 || H <= 0 || H % 4) return fail(MOE_ERR_INVALID_ARG, "bad T=%lld or H=%d", (long long)T, H);
  if (T == 0) return ok();
  if (!r || !a) return fail(MOE_ERR_INVALID_ARG, "r and a must be non-NULL");
  return device_status(moe::launch_rmsnorm_bf16(r, T, H, a, as_stream(stream)), "moe_rmsnorm_bf16");
}

int moe_dequant(const uint8_t* codes, const uint16_t* scales, int64_t rows, int32_t cols, int32_t qbits, float* out,
                void* stream) {
  if (qbits < 2 || qbits > 4) return fail(MOE_ERR_UNSUPPORTED, "qbits=%d: only 2, 3 and 4 are supported", qbits);
  if (rows < 0 || cols <= 0 || cols % 32) return fail(MOE_ERR_INVALID_ARG, "rows=%lld cols=%d: cols must be a positive multiple of 32", (long long)rows, cols);
  if (rows == 0) return ok();
  if (!codes || !scales || !out) return fail(MOE_ERR_INVALID_ARG, "codes, scales and out must be non-NULL");
  if (!aligned(codes, 8) || !aligned(scales, 2) || !aligned(out, 16))
    return fail(MOE_ERR_INVALID_ARG, "codes must be 8-, scales 2- and out 16-byte aligned");
  return device_status(moe::launch_dequant(codes, scales, rows, cols, qbits, out, as_stream(stream)), "moe_dequant");
}

int moe_quantize(const float* w, int64_t rows, int32_t cols, int32_t qbits, uint8_t* codes, uint16_t* scales,
                 void* stream) {
  if (qbits < 2 || qbits > 4) return fail(MOE_ERR_UNSUPPORTED, "qbits=%d: only 2, 3 and 4 are supported", qbits);
  if (rows < 0 || cols <= 0 || cols % 32) return fail(MOE_ERR_INVALID_ARG, "rows=%lld cols=%d: cols must be a positive multiple of 32", (long long)rows, cols);
  if (rows == 0) return ok();
  if (!codes || !scales || !w) return fail(MOE_ERR_INVALID_ARG, "w, codes and scales must be non-NULL");
  if (!aligned(codes, 8) || !aligned(scales, 2) || !aligned(w, 16))
    return fail(MOE_ERR_INVALID_ARG, "codes must be 8-, scales 2- and w 16-byte aligned");
  return device_status(moe::launch_quantize(w, rows, cols, qbits, codes, scales, as_stream(stream)), "moe_quantize");
}

int moe_repack(const uint8_t* codes, const uint16_t* scales, int64_t rows, int32_t cols, int32_t qbits,
               uint8_t* packed_codes, uint16_t* packed_scales, void* stream) {
  if (qbits < 2 || qbits > 4) return fail(MOE_ERR_UNSUPPORTED, "qbits=%d: only 2, 3 and 4 are supported", qbits);
  if (rows < 0 || cols <= 0 || cols % 32) return fail(MOE_ERR_INVALID_ARG, "rows=%lld cols=%d: cols must be a positive multiple of 32", (long long)rows, cols);
  if (rows == 0) return ok();
  if (!codes || !scales || !packed_codes || !packed_scales)
    return fail(MOE_ERR_INVALID_ARG, "codes, scales, packed_codes and packed_scales must be non-NULL");
  if (!aligned(codes, 8) || !aligned(packed_codes, 8) || !aligned(scales, 2) || !aligned(packed_scales, 2))
    return fail(MOE_ERR_INVALID_ARG, "codes and packed_codes must be 8-, scales and packed_scales 2-byte aligned");
  const uintptr_t nc = uintptr_t(rows) * uintptr_t(cols) / 8 * uintptr_t(qbits), ns = uintptr_t(rows) * (cols / 32) * 2;
  const uintptr_t in[2][2] = {{uintptr_t(codes), uintptr_t(codes) + nc}, {uintptr_t(scales), uintptr_t(scales) + ns}};
  const uintptr_t out[2][2] = {{uintptr_t(packed_codes), uintptr_t(packed_codes) + nc},
                               {uintptr_t(packed_scales), uintptr_t(packed_scales) + ns}};
  for (const auto& a : in)
    for (const auto& b : out)
      if (a[0] < b[1] && b[0] < a[1]) return fail(MOE_ERR_INVALID_ARG, "moe_repack is out of place: outputs overlap inputs");
  return device_status(moe::launch_repack(codes, scales, rows, cols, qbits, packed_codes, packed_scales,
                                          as_stream(stream)),
                       "moe_repack");
}

int moe_read_error(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < 256) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL or too small");
  hipStream_t st = as_stream(stream);
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return device_status(e, "moe_read_error/sync");
  int32_t err = 0;
  e = hipMemcpy(&err, workspace, sizeof(err), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return device_status(e, "moe_read_error/copy");
  if (err == 0) return ok();
  const int32_t zero = 0;
  e = hipMemcpy(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice);
  if (e != hipSuccess) return device_status(e, "moe_read_error/clear");
  return fail(MOE_ERR_INDEX, "%d expert ids outside [0, n_experts) were skipped by the last permutation", err);
}

}  // extern "C"
