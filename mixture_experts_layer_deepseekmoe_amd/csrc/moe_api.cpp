// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace carving and the launch sequence.  Never allocates, frees or
// synchronises; every kernel goes on the caller's stream.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <mutex>
#ifdef MOE_DEBUG
#include <cstdio>
#endif

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
  // training (moe_forward_train / moe_backward) only, after `total`
  size_t sel, gu, dys, xp, dgu, dx, dg, dz, dzr;
  size_t qr, qr_s, qa, qa_s, qb, qb_s;   // FP8 backward only (0 bytes otherwise)
  size_t hr;                             // FP8: bf16 H rows (the forward's H holds e4m3 codes)
  size_t total_train;
  long long kt;                          // columns of the FP8 Wgrad codes
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
  const size_t R = static_cast<size_t>(L.rows);
  L.sel = take(TK * 4);
  L.gu = take(R * 2 * s.inter * 2);
  L.dys = take(R * s.d * 2);
  L.xp = take(fp8 ? 0 : R * s.d * 2);   // the FP8 backward quantises u by token instead
  L.dgu = take(R * 2 * s.inter * 2);
  L.dx = take(R * s.d * 2);
  L.dg = take(TK * 4);
  L.dz = take(TK * 4);
  L.dzr = take(TK * 4);
  {
    const size_t dmax = static_cast<size_t>(s.d > 2 * s.inter ? s.d : 2 * s.inter);
    const size_t bmax = static_cast<size_t>(s.d > s.inter ? s.d : s.inter);
    L.kt = fp8 ? moe::wgrad8_kt(L.rows, s.n_routed + s.n_shared) : 0;
    const size_t kt = static_cast<size_t>(L.kt);
    L.qr = take(fp8 ? R * dmax : 0);
    L.qr_s = take(fp8 ? R * (dmax / 128) * 4 : 0);
    L.qa = take(dmax * kt);
    L.qa_s = take(dmax * (kt / 128) * 4);
    L.qb = take(bmax * kt);
    L.qb_s = take(bmax * (kt / 128) * 4);
    L.hr = take(fp8 ? R * s.inter * 2 : 0);
  }
  L.total_train = o;
  return L;
}

// Group-limited routing is on when 1 < topk_groups < n_groups; otherwise the
// kernels get n_groups = topk_groups = 1 (global top-K).
int groups_of(const moe_shape& s) { return s.n_groups > 1 && s.topk_groups < s.n_groups ? s.n_groups : 1; }
int topk_groups_of(const moe_shape& s) { return s.n_groups > 1 && s.topk_groups < s.n_groups ? s.topk_groups : 1; }

int validate_shape(const moe_shape* s);

// The training entry points: bf16 activations with bf16 or E4M3 weights.
// FP8: the Wgrad code arrays ([channel][kt], byte offsets in 32 bits, with
// room past them for the loads of padding rows) must fit.
int validate_train(const moe_shape& s) {
  if (s.x_dtype != MOE_DTYPE_BF16 || (s.w_dtype != MOE_DTYPE_BF16 && s.w_dtype != MOE_DTYPE_E4M3))
    return MOE_ERR_UNSUPPORTED;
  // the Wgrad addresses one group's bf16 rows ([dG dU], G|U: up to T rows of
  // 2I) with 32-bit byte offsets (the rows of d are covered by the check on u)
  if (static_cast<long long>(s.T) * 4LL * s.inter >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  if (s.w_dtype == MOE_DTYPE_E4M3) {
    const long long R = static_cast<long long>(s.T) * (s.top_k + s.n_shared);
    const long long kt = moe::wgrad8_kt(R, s.n_routed + s.n_shared);
    const long long cmax = s.d > 2LL * s.inter ? s.d : 2LL * s.inter;
    if (cmax * kt >= 0x7ff00000LL) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

int validate_shape(const moe_shape* s) {
  if (s == nullptr) return MOE_ERR_INVALID_ARG;
  if (s->n_groups < 0) return MOE_ERR_INVALID_ARG;
  if (s->n_groups > 1) {
    if (s->n_groups > 64) return MOE_ERR_UNSUPPORTED;
    if (s->n_routed <= 0 || s->n_routed % s->n_groups != 0 || s->topk_groups < 1 || s->topk_groups > s->n_groups)
      return MOE_ERR_INVALID_ARG;
    if (static_cast<long long>(s->topk_groups) * (s->n_routed / s->n_groups) < s->top_k) return MOE_ERR_INVALID_ARG;
  }
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

// Debug build (-DMOE_DEBUG): after an entry point's launches, wait for the
// stream and read every kernel file's index-check flag; a failed check turns
// the call's status into MOE_ERR_LAUNCH and is reported on stderr.  (The
// release build never synchronises.)
#ifdef MOE_DEBUG
int debug_status(int rc, hipStream_t st, const char* what) {
  if (rc != MOE_OK) return rc;
  if (hipStreamSynchronize(st) != hipSuccess) return MOE_ERR_LAUNCH;
  const int flags[5] = {moe::debug_take_route(), moe::debug_take_group(), moe::debug_take_ggemm(),
                        moe::debug_take_combine(), moe::debug_take_bwd()};
  for (const int f : flags) {
    if (f != 0) {
      std::fprintf(stderr, "moe debug build: %s: index check %d failed\n", what, f);
      return MOE_ERR_LAUNCH;
    }
  }
  return MOE_OK;
}
#else
inline int debug_status(int rc, hipStream_t, const char*) { return rc; }
#endif

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
                    moe::route_ksplit(fmt_of(s.x_dtype), s.T, s.d, s.n_routed), groups_of(s), topk_groups_of(s)};
  int rc = check_launch(moe::launch_route(fmt_of(s.x_dtype), ra, st));
  if (rc != MOE_OK) return rc;
  const int bm = moe::gg_bm(fmt_of(s.w_dtype));
  moe::GroupArgs ga{idx,     s.T,  s.top_k, s.n_routed, s.n_shared, hist, counts, offsets, perm, pos, mtiles, mtcount, bm,
                    moe::seg_cap(moe::max_mtiles(s.T, s.top_k, s.n_routed, s.n_shared, bm))};
  return check_launch(moe::launch_group(ga, st));
}

int validate_forward(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
                     const moe_weights* wt, const void* y);
int run_forward(const moe_shape& s, const Layout& L, const void* u, const void* centroids, const float* bias,
                const moe_weights* wt, void* y, const moe_routing* routing, void* workspace, const moe_trace* trace,
                hipStream_t stream, bool train = false);

// ---- the workspace of moe_forward_static
//
// A file-scope device array; every device the library runs on holds its own
// copy (at its own address) until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address comes
// from hipGetSymbolAddress, taken once per device (with that device current)
// on the device's first moe_forward_static call, and only that address is
// ever handed to a kernel.  Nothing in the forward needs the workspace to
// start at zero: every kernel writes what a later one reads in the same call.
constexpr size_t kStaticScratchBytes = MOE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_LAUNCH;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MOE_OK;
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

const char* moe_version(void) { return "moe-mi355x 0.2 (gfx950)"; }

int moe_workspace_size(const moe_shape* shape, size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  const int rc = validate_shape(shape);
  if (rc != MOE_OK) return rc;
  *bytes = make_layout(*shape).total;
  return MOE_OK;
}

int moe_workspace_layout(const moe_shape* shape, moe_workspace_map* map) {
  if (map == nullptr) return MOE_ERR_INVALID_ARG;
  const int rc = validate_shape(shape);
  if (rc != MOE_OK) return rc;
  const Layout L = make_layout(*shape);
  map->mtiles = L.mtiles;
  map->mt_count = L.mtcount;
  map->h = L.h;
  map->h_scale = L.hs;
  map->y = L.y;
  map->max_mtiles = L.max_mt;
  map->tile_rows = moe::gg_bm(fmt_of(shape->w_dtype));
  map->seg_cap = moe::seg_cap(L.max_mt);
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
  return debug_status(run_route(s, u, centroids, bias, out->topk_idx, out->topk_gate, out->expert_counts,
                                out->expert_offsets, out->perm_token, out->pos, at<int32_t>(workspace, L.hist),
                                at<float>(workspace, L.scores), nullptr, nullptr, stream),
                      stream, "moe_route");
}

int moe_forward(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
                const moe_weights* wt, void* y, const moe_routing* routing, void* workspace, size_t workspace_bytes,
                const moe_trace* trace, hipStream_t stream) {
  const int rc = validate_forward(shape, u, centroids, bias, wt, y);
  if (rc != MOE_OK) return rc;
  const Layout L = make_layout(*shape);
  if (workspace == nullptr || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  return debug_status(run_forward(*shape, L, u, centroids, bias, wt, y, routing, workspace, trace, stream), stream,
                      "moe_forward");
}

int moe_forward_static(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
                       const moe_weights* wt, void* y, const moe_routing* routing, const moe_trace* trace,
                       hipStream_t stream) {
  int rc = validate_forward(shape, u, centroids, bias, wt, y);
  if (rc != MOE_OK) return rc;
  const Layout L = make_layout(*shape);
  if (L.total > kStaticScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  rc = static_scratch(&ws);
  if (rc != MOE_OK) return rc;
  return debug_status(run_forward(*shape, L, u, centroids, bias, wt, y, routing, ws, trace, stream), stream,
                      "moe_forward_static");
}

}  // extern "C"

namespace {

int validate_forward(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
                     const moe_weights* wt, const void* y) {
  const int rc = validate_shape(shape);
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
  return MOE_OK;
}

// The whole forward on a workspace of at least L.total bytes (arguments
// already validated).
int run_forward(const moe_shape& s, const Layout& L, const void* u, const void* centroids, const float* bias,
                const moe_weights* wt, void* y, const moe_routing* routing, void* workspace, const moe_trace* trace,
                hipStream_t stream, bool train) {
  int rc = MOE_OK;
  const bool fp8 = s.w_dtype == MOE_DTYPE_E4M3;
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
                    moe::route_ksplit(fmt_of(s.x_dtype), s.T, s.d, s.n_routed), groups_of(s), topk_groups_of(s),
                    train ? at<float>(workspace, L.sel) : nullptr};
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
    for (int i = MOE_STAGE_QUANT; i <= MOE_STAGE_COMBINE; ++i) { stg.begin(i); stg.end(i); }
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
                     at<void>(workspace, L.h), fp8 ? at<float>(workspace, L.hs) : nullptr,
                     train ? at<uint16_t>(workspace, L.gu) : nullptr};
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

}  // namespace

extern "C" {

int moe_train_workspace_size(const moe_shape* shape, size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  const int rc = validate_shape(shape);
  if (rc != MOE_OK) return rc;
  const int rt = validate_train(*shape);
  if (rt != MOE_OK) return rt;
  *bytes = make_layout(*shape).total_train;
  return MOE_OK;
}

int moe_forward_train(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
                      const moe_weights* wt, void* y, void* workspace, size_t workspace_bytes, const moe_trace* trace,
                      hipStream_t stream) {
  const int rc = validate_forward(shape, u, centroids, bias, wt, y);
  if (rc != MOE_OK) return rc;
  const int rt = validate_train(*shape);
  if (rt != MOE_OK) return rt;
  const Layout L = make_layout(*shape);
  if (workspace == nullptr || workspace_bytes < L.total_train) return MOE_ERR_WORKSPACE;
  return debug_status(run_forward(*shape, L, u, centroids, bias, wt, y, nullptr, workspace, trace, stream, true),
                      stream, "moe_forward_train");
}

int moe_backward(const moe_shape* shape, const void* u, const void* centroids, const moe_weights* wt, const float* dy,
                 float* du, float* dcentroids, const moe_weight_grads* grads, void* workspace, size_t workspace_bytes,
                 const moe_trace* trace, hipStream_t stream) {
  const int rc = validate_shape(shape);
  if (rc != MOE_OK) return rc;
  const moe_shape& s = *shape;
  const int rt = validate_train(s);
  if (rt != MOE_OK) return rt;
  const bool fp8 = s.w_dtype == MOE_DTYPE_E4M3;
  if (wt == nullptr || grads == nullptr || centroids == nullptr || dcentroids == nullptr) return MOE_ERR_INVALID_ARG;
  if (fp8 && (wt->w_gate_up_t == nullptr || wt->w_down_t == nullptr || wt->s_gate_up_t == nullptr ||
              wt->s_down_t == nullptr || !aligned16(wt->w_gate_up_t) || !aligned16(wt->w_down_t) ||
              (s.n_shared > 0 && (wt->ws_gate_up_t == nullptr || wt->ws_down_t == nullptr ||
                                  wt->ss_gate_up_t == nullptr || wt->ss_down_t == nullptr ||
                                  !aligned16(wt->ws_gate_up_t) || !aligned16(wt->ws_down_t)))))
    return MOE_ERR_INVALID_ARG;
  if (s.T > 0 && (u == nullptr || dy == nullptr || du == nullptr || !aligned16(u) || !aligned16(dy) || !aligned16(du)))
    return MOE_ERR_INVALID_ARG;
  if (wt->w_gate_up == nullptr || wt->w_down == nullptr || grads->dw_gate_up == nullptr || grads->dw_down == nullptr ||
      !aligned16(wt->w_gate_up) || !aligned16(wt->w_down) || !aligned16(grads->dw_gate_up) ||
      !aligned16(grads->dw_down) || !aligned16(centroids) || !aligned16(dcentroids))
    return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && (wt->ws_gate_up == nullptr || wt->ws_down == nullptr || grads->dws_gate_up == nullptr ||
                         grads->dws_down == nullptr || !aligned16(wt->ws_gate_up) || !aligned16(wt->ws_down) ||
                         !aligned16(grads->dws_gate_up) || !aligned16(grads->dws_down)))
    return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(s);
  if (workspace == nullptr || workspace_bytes < L.total_train) return MOE_ERR_WORKSPACE;
  moe::BwdArgs a{};
  a.T = s.T;
  a.d = s.d;
  a.n_routed = s.n_routed;
  a.n_shared = s.n_shared;
  a.inter = s.inter;
  a.top_k = s.top_k;
  a.TK = static_cast<long long>(s.T) * s.top_k;
  a.R = L.rows;
  a.max_mtiles = L.max_mt;
  a.mtiles = at<int4>(workspace, L.mtiles);
  a.mt_count = at<int32_t>(workspace, L.mtcount);
  a.offsets = at<int32_t>(workspace, L.offsets);
  a.counts = at<int32_t>(workspace, L.counts);
  a.perm_token = at<int32_t>(workspace, L.perm);
  a.pos = at<int32_t>(workspace, L.pos);
  a.idx = at<int32_t>(workspace, L.idx);
  a.gate = at<float>(workspace, L.gate);
  a.sel_score = at<float>(workspace, L.sel);
  a.u = static_cast<const uint16_t*>(u);
  a.centroids = static_cast<const uint16_t*>(centroids);
  a.y = at<uint16_t>(workspace, L.y);
  a.dy = dy;
  a.w_gate_up = wt->w_gate_up;
  a.w_down = wt->w_down;
  a.ws_gate_up = wt->ws_gate_up;
  a.ws_down = wt->ws_down;
  a.gu = at<uint16_t>(workspace, L.gu);
  a.dys = at<uint16_t>(workspace, L.dys);
  a.xp = at<uint16_t>(workspace, L.xp);
  a.dgu = at<uint16_t>(workspace, L.dgu);
  // the forward's H is not needed any more: bf16, H is recomputed into it
  a.hr = at<uint16_t>(workspace, s.w_dtype == MOE_DTYPE_E4M3 ? L.hr : L.h);
  a.dx = at<uint16_t>(workspace, L.dx);
  a.dg = at<float>(workspace, L.dg);
  a.dz = at<float>(workspace, L.dz);
  a.dzr = at<float>(workspace, L.dzr);
  a.du = du;
  a.dcentroids = dcentroids;
  a.dw_gate_up = grads->dw_gate_up;
  a.dw_down = grads->dw_down;
  a.dws_gate_up = grads->dws_gate_up;
  a.dws_down = grads->dws_down;
  if (fp8) {
    a.fp8 = 1;
    a.w_gate_up_t = wt->w_gate_up_t;
    a.w_down_t = wt->w_down_t;
    a.ws_gate_up_t = wt->ws_gate_up_t;
    a.ws_down_t = wt->ws_down_t;
    a.s_gate_up_t = wt->s_gate_up_t;
    a.s_down_t = wt->s_down_t;
    a.ss_gate_up_t = wt->ss_gate_up_t;
    a.ss_down_t = wt->ss_down_t;
    a.qr = at<uint8_t>(workspace, L.qr);
    a.qr_s = at<float>(workspace, L.qr_s);
    a.kt = L.kt;
    a.qa = at<uint8_t>(workspace, L.qa);
    a.qa_s = at<float>(workspace, L.qa_s);
    a.qb = at<uint8_t>(workspace, L.qb);
    a.qb_s = at<float>(workspace, L.qb_s);
  }
  Stages stg{trace, stream};
  for (int st = 0; st < moe::BWD_STAGES; ++st) {
    stg.begin(MOE_STAGE_BWD_PREP + st);
    const int rc2 = check_launch(moe::launch_backward_stage(st, a, stream));
    if (rc2 != MOE_OK) return rc2;
    stg.end(MOE_STAGE_BWD_PREP + st);
  }
  return debug_status(MOE_OK, stream, "moe_backward");
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
