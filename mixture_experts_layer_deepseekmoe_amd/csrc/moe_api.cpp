// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace carving and the launch sequence.  Never allocates, frees or
// synchronises; every kernel goes on the caller's stream.
#include "moe.h"

#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace {

using moe::FMT_BF16;
using moe::FMT_E4M3;
using moe::FMT_F32;

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int elem_bytes(int dt) { return dt == MOE_DTYPE_F32 ? 4 : (dt == MOE_DTYPE_BF16 ? 2 : 1); }

int fmt_of(int dt) { return dt == MOE_DTYPE_F32 ? FMT_F32 : (dt == MOE_DTYPE_BF16 ? FMT_BF16 : FMT_E4M3); }

// Workspace map (byte offsets, each 256-byte aligned).
struct Layout {
  size_t hist, idx, gate, counts, offsets, perm, pos, mtiles, mtcount, uq, us, h, hs, y, scores, total;
  int nblk, max_mt;
  long long rows;   // grouped rows: T*K routed + N_s*T shared
};

Layout make_layout(const moe_shape& s) {
  Layout L{};
  const long long T = s.T, TK = T * s.top_k;
  L.nblk = moe::ceil_div(s.T, moe::GROUP_TB);
  L.max_mt = moe::max_mtiles(T, s.top_k, s.n_routed, s.n_shared, moe::gg_bm(fmt_of(s.w_dtype)));
  L.rows = TK + static_cast<long long>(s.n_shared) * T;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align_up(bytes); return at; };
  L.hist = take(static_cast<size_t>(L.nblk) * s.n_routed * 4);
  L.idx = take(TK * 4);
  L.gate = take(TK * 4);
  L.counts = take(static_cast<size_t>(s.n_routed) * 4);
  L.offsets = take(static_cast<size_t>(s.n_routed + 1) * 4);
  L.perm = take(TK * 4);
  L.pos = take(TK * 4);
  L.mtiles = take(static_cast<size_t>(L.max_mt) * 16);
  L.mtcount = take(4 * (2 + moe::MT_SEGMENTS));
  const bool fp8 = s.w_dtype == MOE_DTYPE_E4M3;
  L.uq = take(fp8 ? static_cast<size_t>(T) * s.d : 0);
  L.us = take(fp8 ? static_cast<size_t>(T) * (s.d / 128) * 4 : 0);
  L.h = take(static_cast<size_t>(L.rows) * s.inter * elem_bytes(s.w_dtype));
  L.hs = take(fp8 ? static_cast<size_t>(L.rows) * (s.inter / 128) * 4 : 0);
  L.y = take(static_cast<size_t>(L.rows) * s.d * (s.w_dtype == MOE_DTYPE_F32 ? 4 : 2));
  L.scores = take(static_cast<size_t>(moe::route_scratch_floats(fmt_of(s.x_dtype), T, s.d, s.n_routed)) * 4);
  L.total = o;
  return L;
}

int validate_shape(const moe_shape* s) {
  if (s == nullptr) return MOE_ERR_INVALID_ARG;
  if (s->T < 0 || s->d <= 0 || s->inter <= 0 || s->n_routed <= 0 || s->n_shared < 0 || s->top_k <= 0)
    return MOE_ERR_INVALID_ARG;
  if (s->top_k > s->n_routed) return MOE_ERR_INVALID_ARG;
  if (s->x_dtype != MOE_DTYPE_F32 && s->x_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (s->out_dtype != MOE_DTYPE_F32 && s->out_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  const bool combo_ok = (s->x_dtype == MOE_DTYPE_F32 && s->w_dtype == MOE_DTYPE_F32) ||
                        (s->x_dtype == MOE_DTYPE_BF16 && s->w_dtype == MOE_DTYPE_BF16) ||
                        (s->x_dtype == MOE_DTYPE_BF16 && s->w_dtype == MOE_DTYPE_E4M3);
  if (!combo_ok) return MOE_ERR_INVALID_ARG;
  if (s->n_routed > moe::MAX_ROUTED || s->n_shared > moe::MAX_SHARED || s->top_k > moe::MAX_TOPK)
    return MOE_ERR_UNSUPPORTED;
  const int kmult = s->w_dtype == MOE_DTYPE_F32 ? 32 : (s->w_dtype == MOE_DTYPE_BF16 ? 64 : 128);
  if (s->d % kmult != 0 || s->inter % kmult != 0) return MOE_ERR_UNSUPPORTED;
  const long long T = s->T;
  if (T * (s->top_k + s->n_shared) >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (s->w_dtype == MOE_DTYPE_E4M3 && (s->d > 32768 || s->inter > 32768)) return MOE_ERR_UNSUPPORTED;
  // the kernels address the activations and one expert's weight matrix with
  // 32-bit byte offsets
  const long long xes = s->x_dtype == MOE_DTYPE_F32 ? 4 : 2;
  const long long wes = s->w_dtype == MOE_DTYPE_F32 ? 4 : (s->w_dtype == MOE_DTYPE_BF16 ? 2 : 1);
  if (T * s->d * xes >= (1LL << 32) || 2LL * s->inter * s->d * wes >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  const long long gu_tiles =
      static_cast<long long>(moe::max_mtiles(T, s->top_k, s->n_routed, s->n_shared, moe::gg_bm(fmt_of(s->w_dtype)))) *
      moe::ceil_div(s->d > s->inter ? s->d : s->inter, 128);
  if (gu_tiles >= (1LL << 31) - 64) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

int check_launch(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

// Optional per-stage event records on the caller's stream.
struct Stages {
  const moe_trace* tr;
  hipStream_t st;
  void begin(int i) const {
    if (tr != nullptr && tr->start[i] != nullptr) (void)hipEventRecord(tr->start[i], st);
  }
  void end(int i) const {
    if (tr != nullptr && tr->stop[i] != nullptr) (void)hipEventRecord(tr->stop[i], st);
  }
};

// Route + group.  `mtiles` null: routing only (no GEMM tile list).
int run_route(const moe_shape& s, const void* u, const void* cen, const float* bias, int32_t* idx, float* gate,
              int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos, int32_t* hist, float* scores,
              int4* mtiles, int32_t* mtcount, hipStream_t st) {
  moe::RouteArgs ra{u,   cen,  bias,  s.T, s.d, s.n_routed, s.top_k, idx, gate, scores,
                    moe::route_ksplit(fmt_of(s.x_dtype), s.T, s.d, s.n_routed)};
  int rc = check_launch(moe::launch_route(fmt_of(s.x_dtype), ra, st));
  if (rc != MOE_OK) return rc;
  const int bm = moe::gg_bm(fmt_of(s.w_dtype));
  moe::GroupArgs ga{idx,     s.T,  s.top_k, s.n_routed, s.n_shared, hist, counts, offsets, perm, pos, mtiles, mtcount, bm,
                    moe::seg_cap(moe::max_mtiles(s.T, s.top_k, s.n_routed, s.n_shared, bm))};
  return check_launch(moe::launch_group(ga, st));
}

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: null pointer, bad shape, dtype combination or alignment";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape outside the library's limits";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH: kernel launch failed";
    default: return "unknown moe_status";
  }
}

const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

int moe_workspace_size(const moe_shape* shape, size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  const int rc = validate_shape(shape);
  if (rc != MOE_OK) return rc;
  *bytes = make_layout(*shape).total;
  return MOE_OK;
}

int moe_route(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
              const moe_routing* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = validate_shape(shape);
  if (rc != MOE_OK) return rc;
  const moe_shape& s = *shape;
  if (out == nullptr || out->topk_idx == nullptr || out->topk_gate == nullptr || out->expert_counts == nullptr ||
      out->expert_offsets == nullptr || out->perm_token == nullptr || out->pos == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (s.T > 0 && (u == nullptr || !aligned16(u))) return MOE_ERR_INVALID_ARG;
  if (centroids == nullptr || bias == nullptr || !aligned16(centroids)) return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(s);
  if (workspace == nullptr || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  return run_route(s, u, centroids, bias, out->topk_idx, out->topk_gate, out->expert_counts, out->expert_offsets,
                   out->perm_token, out->pos, at<int32_t>(workspace, L.hist), at<float>(workspace, L.scores),
                   nullptr, nullptr, stream);
}

int moe_forward(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
                const moe_weights* wt, void* y, const moe_routing* routing, void* workspace, size_t workspace_bytes,
                const moe_trace* trace, hipStream_t stream) {
  int rc = validate_shape(shape);
  if (rc != MOE_OK) return rc;
  const moe_shape& s = *shape;
  const bool fp8 = s.w_dtype == MOE_DTYPE_E4M3;
  if (wt == nullptr || centroids == nullptr || bias == nullptr || !aligned16(centroids)) return MOE_ERR_INVALID_ARG;
  if (s.T > 0 && (u == nullptr || y == nullptr || !aligned16(u) || !aligned16(y))) return MOE_ERR_INVALID_ARG;
  if (wt->w_gate_up == nullptr || wt->w_down == nullptr || !aligned16(wt->w_gate_up) || !aligned16(wt->w_down))
    return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && (wt->ws_gate_up == nullptr || wt->ws_down == nullptr || !aligned16(wt->ws_gate_up) ||
                         !aligned16(wt->ws_down)))
    return MOE_ERR_INVALID_ARG;
  if (fp8 && (wt->s_gate_up == nullptr || wt->s_down == nullptr ||
              (s.n_shared > 0 && (wt->ss_gate_up == nullptr || wt->ss_down == nullptr))))
    return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(s);
  if (workspace == nullptr || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;

  moe_routing r{};
  if (routing != nullptr) r = *routing;
  int32_t* idx = r.topk_idx ? r.topk_idx : at<int32_t>(workspace, L.idx);
  float* gate = r.topk_gate ? r.topk_gate : at<float>(workspace, L.gate);
  int32_t* counts = r.expert_counts ? r.expert_counts : at<int32_t>(workspace, L.counts);
  int32_t* offsets = r.expert_offsets ? r.expert_offsets : at<int32_t>(workspace, L.offsets);
  int32_t* perm = r.perm_token ? r.perm_token : at<int32_t>(workspace, L.perm);
  int32_t* pos = r.pos ? r.pos : at<int32_t>(workspace, L.pos);
  int4* mtiles = at<int4>(workspace, L.mtiles);
  int32_t* mtcount = at<int32_t>(workspace, L.mtcount);

  Stages stg{trace, stream};
  stg.begin(MOE_STAGE_ROUTE);
  moe::RouteArgs ra{u,    centroids, bias, s.T, s.d, s.n_routed, s.top_k, idx, gate, at<float>(workspace, L.scores),
                    moe::route_ksplit(fmt_of(s.x_dtype), s.T, s.d, s.n_routed)};
  rc = check_launch(moe::launch_route(fmt_of(s.x_dtype), ra, stream));
  if (rc != MOE_OK) return rc;
  stg.end(MOE_STAGE_ROUTE);
  stg.begin(MOE_STAGE_GROUP);
  moe::GroupArgs gra{idx,    s.T,    s.top_k, s.n_routed, s.n_shared, at<int32_t>(workspace, L.hist), counts,
                     offsets, perm, pos,      mtiles,     mtcount,    moe::gg_bm(fmt_of(s.w_dtype)), moe::seg_cap(L.max_mt)};
  rc = check_launch(moe::launch_group(gra, stream));
  if (rc != MOE_OK) return rc;
  stg.end(MOE_STAGE_GROUP);
  if (s.T == 0) {
    for (int i = MOE_STAGE_QUANT; i < MOE_NUM_STAGES; ++i) { stg.begin(i); stg.end(i); }
    return MOE_OK;
  }

  const void* x = u;
  const float* xs = nullptr;
  stg.begin(MOE_STAGE_QUANT);
  if (fp8) {
    rc = check_launch(moe::launch_quant_act(u, s.T, s.d, at<uint8_t>(workspace, L.uq), at<float>(workspace, L.us), stream));
    if (rc != MOE_OK) return rc;
    x = at<uint8_t>(workspace, L.uq);
    xs = at<float>(workspace, L.us);
  }
  stg.end(MOE_STAGE_QUANT);
  const int wf = fmt_of(s.w_dtype);
  const int TK = s.T * s.top_k;
  moe::GateUpArgs ga{x, xs, perm, s.T, TK, s.n_routed, s.d, s.inter, wt->w_gate_up, wt->ws_gate_up,
                     wt->s_gate_up, wt->ss_gate_up, mtiles, mtcount, L.max_mt,
                     at<void>(workspace, L.h), fp8 ? at<float>(workspace, L.hs) : nullptr};
  stg.begin(MOE_STAGE_GATE_UP);
  rc = check_launch(moe::launch_gateup(wf, ga, stream));
  if (rc != MOE_OK) return rc;
  stg.end(MOE_STAGE_GATE_UP);
  moe::DownArgs da{at<void>(workspace, L.h), fp8 ? at<float>(workspace, L.hs) : nullptr, s.n_routed, s.d, s.inter,
                   wt->w_down, wt->ws_down, wt->s_down, wt->ss_down, mtiles, mtcount, L.max_mt,
                   at<void>(workspace, L.y)};
  stg.begin(MOE_STAGE_DOWN);
  rc = check_launch(moe::launch_down(wf, da, stream));
  if (rc != MOE_OK) return rc;
  stg.end(MOE_STAGE_DOWN);
  moe::CombineArgs ca{u, at<void>(workspace, L.y), gate, pos, s.T, s.d, s.top_k, s.n_shared, TK, y};
  const int yf = s.w_dtype == MOE_DTYPE_F32 ? FMT_F32 : FMT_BF16;
  stg.begin(MOE_STAGE_COMBINE);
  rc = check_launch(moe::launch_combine(fmt_of(s.x_dtype), yf, fmt_of(s.out_dtype), ca, stream));
  if (rc != MOE_OK) return rc;
  stg.end(MOE_STAGE_COMBINE);
  return MOE_OK;
}

int moe_update_bias(float* bias, const int32_t* counts, int32_t n_routed, int64_t total_assignments, float gamma,
                    hipStream_t stream) {
  if (bias == nullptr || counts == nullptr || n_routed <= 0 || total_assignments < 0) return MOE_ERR_INVALID_ARG;
  if (n_routed > (1 << 24)) return MOE_ERR_UNSUPPORTED;
  return check_launch(moe::launch_bias_update(bias, counts, n_routed, total_assignments, gamma, stream));
}

int moe_quantize_weight_e4m3(const void* src, int32_t src_dtype, int64_t n, int32_t rows, int32_t cols,
                             uint8_t* codes, float* scales, hipStream_t stream) {
  if (n < 0 || rows <= 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (src_dtype != MOE_DTYPE_F32 && src_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (rows % 128 != 0 || cols % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (n * (rows / 128) * static_cast<long long>(cols / 128) >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (n == 0) return MOE_OK;
  if (src == nullptr || codes == nullptr || scales == nullptr || !aligned16(src) || !aligned16(codes))
    return MOE_ERR_INVALID_ARG;
  return check_launch(moe::launch_quant_weight(fmt_of(src_dtype), src, n, rows, cols, codes, scales, stream));
}

int moe_quantize_act_e4m3(const void* src, int32_t rows, int32_t cols, uint8_t* codes, float* scales,
                          hipStream_t stream) {
  if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (cols % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (src == nullptr || codes == nullptr || scales == nullptr || !aligned16(src) || !aligned16(codes))
    return MOE_ERR_INVALID_ARG;
  return check_launch(moe::launch_quant_act(src, rows, cols, codes, scales, stream));
}

}  // extern "C"
