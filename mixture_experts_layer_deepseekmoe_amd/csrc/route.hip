// Router: affinity GEMM fused with sigmoid, bias add, wavefront top-K and
// gate normalisation (DeepSeek-V3 Technical Report summary, section 2:
// s_{i,t} = Sigmoid(u_t^T e_i); g'_{i,t} = s_{i,t} when s_{i,t} + b_i is among
// the K_r largest of {s_{j,t} + b_j}, else 0; g_{i,t} = g' normalised).
//
// One block routes 32 tokens against every expert: the logits of one chunk
// of 256 experts come from the pipelined MFMA tile core (fp32 accumulation);
// their sigmoids go to LDS (the logits never reach HBM); then each wave
// selects the top-K of its tokens, with the N_r scores of a token spread
// 1..8 per lane.  Small batches (too few such blocks to fill the chip) split
// the experts over blocks as well and pass the sigmoids through scratch;
// large bf16 batches take 256 x 256 tiles over slices of K instead and pass
// fp32 partial logits through scratch.
// Ordering is by v = s + b descending, exact ties to the lower expert index;
// a NaN score ranks below every number, so K distinct in-range experts are
// always produced.  Gates are s_k / sum of the K selected s, summed in
// selection order in fp32.
#include "gemm_core.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int RBT = ROUTE_BT;
constexpr int RCHUNK = 256;   // experts per MFMA pass

// Group-limited routing (the node-limited variant: a token's experts come
// from at most topk_groups of n_groups equal runs of consecutive experts).
// The groups are ranked by the sum of each group's q largest keys, the
// topk_groups best are kept (ties to the lower group), and the experts of the
// other groups are excluded before the top-K.  Returns a bit per group, set
// for the kept ones.  Lane g < n_groups scores group g; the keys are those of
// the top-K (s + b, NaN ranked as -inf).
__device__ __forceinline__ uint64_t keep_groups(const float* srow, const float* bias, int n_groups, int topk_groups,
                                                int gsize, int q) {
  const int lane = threadIdx.x & 63;
  float score = -INFINITY;
  if (lane < n_groups) {
    // the q largest keys of the group, largest first (key, then lower index
    // first among equal keys), summed in that order
    float sum = 0.f, pv = INFINITY;
    int pe = -1;
    for (int j = 0; j < q; ++j) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
      for (int m = 0; m < gsize; ++m) {
        const int e = lane * gsize + m;
        float x = srow[e] + bias[e];
        if (x != x) x = -INFINITY;
        const bool after = x < pv || (x == pv && e > pe);
        if (after && (x > bv || (x == bv && e < be))) { bv = x; be = e; }
      }
      sum += bv;
      pv = bv;
      pe = be;
    }
    score = sum;
  }
  uint64_t kept = 0;
  for (int j = 0; j < topk_groups; ++j) {
    const bool cand = lane < n_groups && !((kept >> lane) & 1ull);
    float bv = cand ? score : -INFINITY;
    int be = cand ? lane : 0x7fffffff;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    kept |= 1ull << be;
  }
  return kept;
}

// Top-K of one token by one wave: srow holds the token's N_r sigmoid scores
// (LDS or global), bq[q] the bias of expert lane + 64 q.  Lane k < K writes
// the k-th selected expert and its gate.  With grouped routing
// (1 < topk_groups < n_groups) only the kept groups' experts take part.
template <int NQ>
__device__ __forceinline__ void select_topk(const float* srow, const float (&bq)[NQ], const RouteArgs& a,
                                            int32_t* idx_out, float* gate_out) {
  const int lane = threadIdx.x & 63;
  const int n_routed = a.n_routed, top_k = a.top_k;
  float key[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = lane + 64 * q;
    float v = -INFINITY;
    if (e < n_routed) {
      v = srow[e] + bq[q];
      if (v != v) v = -INFINITY;
    }
    key[q] = v;
  }
  uint32_t taken = 0;   // bit q: expert lane + 64 q is chosen or excluded
  if (a.topk_groups < a.n_groups) {
    const int gsize = n_routed / a.n_groups;
    const int qg = min((top_k + a.topk_groups - 1) / a.topk_groups, gsize);
    const uint64_t kept = keep_groups(srow, a.bias, a.n_groups, a.topk_groups, gsize, qg);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = lane + 64 * q;
      if (e < n_routed && !((kept >> (e / gsize)) & 1ull)) taken |= 1u << q;
    }
  }
  int chosen = 0;     // lane k keeps the k-th selected expert
  float chosen_s = 0.f;
  float sum = 0.f;
  for (int k = 0; k < top_k; ++k) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = lane + 64 * q;
      const bool cand = e < n_routed && !((taken >> q) & 1u);
      if (cand && (key[q] > bv || (key[q] == bv && e < be))) { bv = key[q]; be = e; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    if (!MOE_CHECK(be >= 0 && be < n_routed, 101)) be = 0;
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    const float s_sel = srow[be];
    sum += s_sel;
    if (lane == k) { chosen = be; chosen_s = s_sel; }
  }
  if (lane < top_k) {
    idx_out[lane] = chosen;
    gate_out[lane] = chosen_s / sum;
    if (a.sel_score != nullptr) a.sel_score[(idx_out - a.idx) + lane] = chosen_s;
  }
}

template <int NQ>
__device__ __forceinline__ void load_bias(const float* bias, int n_routed, float (&bq)[NQ]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = lane + 64 * q;
    bq[q] = e < n_routed ? bias[e] : 0.f;
  }
}

// Every block streams all centroids (from L2) beside its own token rows, so
// the router is bound by the loads a CU keeps in flight.  Up to 256 experts
// it runs the wave-specialised paired pipeline (8 waves: whole-line L2
// requests, loads issued by their own waves); beyond, the score buffer
// leaves room only for the 4-wave single-stage pipeline on a 4-stage ring.
// NRMAX: the expert count rounded up to 64, 128, 256 or 512.  Experts go
// through the MFMAs in chunks of up to 256 (one chunk of NRMAX below), so
// no chunk loads centroid rows past the last expert.
template <int NRMAX>
struct RouteCfg {
  static constexpr bool WS = NRMAX <= 256;
  static constexpr int NW = WS ? 8 : 4;     // waves per block
  static constexpr int NST = WS ? 5 : 4;    // stage buffers
  static constexpr int CHUNK = NRMAX < RCHUNK ? NRMAX : RCHUNK;   // experts per MFMA pass
  static constexpr int EW = CHUNK / 4;      // experts per MFMA wave
};

template <int FMT, int NRMAX>
__global__ __launch_bounds__(64 * RouteCfg<NRMAX>::NW) void route_kernel(RouteArgs a) {
  using C = RouteCfg<NRMAX>;
  using P = Pipe<FMT, RBT, C::CHUNK, C::NST>;
  constexpr int SSTRIDE = NRMAX + 4;
  __shared__ __attribute__((aligned(1024))) uint8_t st0[P::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[P::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[P::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[P::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t st4[C::NST > 4 ? P::STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(16))) float sbuf[RBT * SSTRIDE];
  uint8_t* const all[5] = {st0, st1, st2, st3, st4};
  uint8_t* st[C::NST];   // a ring of separate LDS objects
#pragma unroll
  for (int i = 0; i < C::NST; ++i) st[i] = all[i];

  const int w = wave_id(), lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int t0 = blockIdx.x * RBT;
  const int es = FMT == FMT_F32 ? 4 : 2;
  const size_t row_bytes = static_cast<size_t>(a.d) * es;
  const int nk = static_cast<int>(row_bytes / P::SB);
  const WRows<0> wr{C::EW * (w & 3)};   // expert subtile j: rows EW w + 16 j of the chunk
  const int valid = min(RBT, a.T - t0);

  for (int ec = 0; ec < a.n_routed; ec += C::CHUNK) {
    P p;
    const rsrc_t ru = make_rsrc(static_cast<const uint8_t*>(a.u) + static_cast<size_t>(t0) * row_bytes,
                                static_cast<uint32_t>(valid * row_bytes));
    p.init(ru, [&](int r) { return static_cast<uint32_t>((r < valid ? r : 0) * row_bytes); },
           make_rsrc(a.centroids, static_cast<uint32_t>(a.n_routed * row_bytes)),
           [&](int r) { return static_cast<uint32_t>((ec + r < a.n_routed ? ec + r : 0) * row_bytes); },
           ru, [](int) { return 0u; });
    f32x4 acc[P::MI][P::NJ];
    zero_acc(acc);
    if constexpr (C::WS) {
      if (valid > 16)
        pipe_mainloop_ws<P, 2>(p, st, nk, wr, acc);
      else
        pipe_mainloop_ws<P, 1>(p, st, nk, wr, acc);
      if (w >= 4) continue;   // load waves hold no scores
    } else {
      if (valid > 16)
        pipe_mainloop<P, C::NST, 2>(p, st, nk, wr, acc);
      else
        pipe_mainloop<P, C::NST, 1>(p, st, nk, wr, acc);
    }

    // lane: token 16i + lr, experts ec + EW w + 16 j + 4lg .. +3
#pragma unroll
    for (int i = 0; i < P::MI; ++i)
#pragma unroll
      for (int j = 0; j < P::NJ; ++j) {
        const int e = ec + C::EW * w + 16 * j + 4 * lg;
        float* dst = sbuf + (16 * i + lr) * SSTRIDE + e;
        if (e + 3 < a.n_routed) {
          *reinterpret_cast<float4*>(dst) = make_float4(sigmoid_f32(acc[i][j][0]), sigmoid_f32(acc[i][j][1]),
                                                        sigmoid_f32(acc[i][j][2]), sigmoid_f32(acc[i][j][3]));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (e + r < a.n_routed) dst[r] = sigmoid_f32(acc[i][j][r]);
        }
      }
  }
  __syncthreads();

  // ---- top-K: wave w takes tokens w * RBT / NW .. of the block
  constexpr int NQ = NRMAX / 64;
  constexpr int TPW = RBT / C::NW;
  float bq[NQ];
  load_bias(a.bias, a.n_routed, bq);
  for (int tt = 0; tt < TPW; ++tt) {
    const int tl = w * TPW + tt;
    const int t = t0 + tl;
    if (t >= a.T) break;
    select_topk(sbuf + tl * SSTRIDE, bq, a, a.idx + static_cast<size_t>(t) * a.top_k,
                a.gate + static_cast<size_t>(t) * a.top_k);
  }
}

// ---- small batches: expert chunks of 64 over blocks too
constexpr int SCHUNK = 64;

// Scores of 32 tokens against 64 experts on the wave-specialised paired
// pipeline (each MFMA wave owns 16 experts), written to scratch.
template <int FMT>
__global__ __launch_bounds__(512) void route_scores_kernel(RouteArgs a) {
  using P = Pipe<FMT, RBT, SCHUNK, 5>;
  __shared__ __attribute__((aligned(1024))) uint8_t st0[P::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[P::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[P::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[P::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t st4[P::STAGE_BYTES];
  uint8_t* const st[5] = {st0, st1, st2, st3, st4};

  const int w = wave_id(), lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int t0 = blockIdx.x * RBT, ec = blockIdx.y * SCHUNK;
  const int es = FMT == FMT_F32 ? 4 : 2;
  const size_t row_bytes = static_cast<size_t>(a.d) * es;
  const int nk = static_cast<int>(row_bytes / P::SB);
  const int valid = min(RBT, a.T - t0);
  P p;
  const rsrc_t ru = make_rsrc(static_cast<const uint8_t*>(a.u) + static_cast<size_t>(t0) * row_bytes,
                              static_cast<uint32_t>(valid * row_bytes));
  p.init(ru, [&](int r) { return static_cast<uint32_t>((r < valid ? r : 0) * row_bytes); },
         make_rsrc(a.centroids, static_cast<uint32_t>(a.n_routed * row_bytes)),
         [&](int r) { return static_cast<uint32_t>((ec + r < a.n_routed ? ec + r : 0) * row_bytes); },
         ru, [](int) { return 0u; });
  const WRows<0> wr{16 * (w & 3)};   // this wave's 16 experts of the chunk
  f32x4 acc[P::MI][P::NJ];
  zero_acc(acc);
  if (valid > 16)
    pipe_mainloop_ws<P, 2>(p, st, nk, wr, acc);
  else
    pipe_mainloop_ws<P, 1>(p, st, nk, wr, acc);
  if (w >= 4) return;
  // lane: token 16 i + lr, experts ec + 16 w + 4 lg .. +3
  const int e = ec + 16 * w + 4 * lg;
#pragma unroll
  for (int i = 0; i < P::MI; ++i) {
    const int t = t0 + 16 * i + lr;
    if (t >= a.T) continue;
    float* dst = a.scores + static_cast<size_t>(t) * a.n_routed + e;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (e + r < a.n_routed) dst[r] = sigmoid_f32(acc[i][0][r]);
  }
}

// One wave per token: top-K over its scores in scratch.
template <int NRMAX>
__global__ __launch_bounds__(256) void route_topk_kernel(RouteArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  constexpr int NQ = NRMAX / 64;
  float bq[NQ];
  load_bias(a.bias, a.n_routed, bq);
  if (t >= a.T) return;
  select_topk(a.scores + static_cast<size_t>(t) * a.n_routed, bq, a, a.idx + static_cast<size_t>(t) * a.top_k,
              a.gate + static_cast<size_t>(t) * a.top_k);
}

// ---- large bf16 batches: K split over blocks
//
// A 32-token block streams every centroid beside its tokens, ~9x the bytes
// of its token rows at 256 experts; the CU's loads, not the matrix cores,
// bound it.  Here a block takes 256 tokens x 256 experts (the grouped
// GEMM's tile and pipeline: 8 MFMA waves, 4 load waves, 5-stage ring) over
// one slice of K, ~4x fewer bytes per logit, and the slices make up the
// block count.  The fp32 logits of slice s go to scores[s][T][N_r].
using KsPipe = Pipe<FMT_BF16, 256, 256, 5, 2, ACC_TIED, 8, 4>;
constexpr int KS_THREADS = 768;

__global__ __launch_bounds__(KS_THREADS, 1) void route_part_kernel(RouteArgs a) {
  using P = KsPipe;
  constexpr int WM = 2;
  __shared__ __attribute__((aligned(1024))) uint8_t ring_lds[5 * P::STAGE_BYTES];
  uint8_t* const st[5] = {ring_lds, ring_lds + P::STAGE_BYTES, ring_lds + 2 * P::STAGE_BYTES,
                          ring_lds + 3 * P::STAGE_BYTES, ring_lds + 4 * P::STAGE_BYTES};
  const int w = wave_id(), lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = w % WM, wn = w / WM;
  const int t0 = blockIdx.x * 256, slice = blockIdx.y;
  const int valid = min(256, a.T - t0);
  const size_t row_bytes = static_cast<size_t>(a.d) * 2;
  const int np = a.d / 64;                        // 128-byte pairs along K
  const int pps = ceil_div(np, a.ksplit);
  const int p0 = slice * pps, p1 = min(np, p0 + pps);   // non-empty: the host sizes ksplit so

  P p;
  const rsrc_t ru = make_rsrc(static_cast<const uint8_t*>(a.u) + static_cast<size_t>(t0) * row_bytes,
                              static_cast<uint32_t>(valid * row_bytes));
  p.init(ru, [&](int r) { return static_cast<uint32_t>((r < valid ? r : 0) * row_bytes); },
         make_rsrc(a.centroids, static_cast<uint32_t>(a.n_routed * row_bytes)),
         [&](int r) { return static_cast<uint32_t>((r < a.n_routed ? r : 0) * row_bytes); },
         ru, [](int) { return 0u; });
  p.krot = 2 * p0;   // K-step offset of the slice (no wrap: nks stays past every K-step)
  const WRows<0> wr{16 * P::NJ * wn};
  f32x4 acc[P::MI][P::NJ];
  zero_acc(acc);
  pipe_mainloop_ws<P, P::MI, P::MI>(p, st, 2 * (p1 - p0), wr, acc);
  if (w >= 8) return;   // load waves hold no logits

  // lane: token 16 (WM i + wm) + lr, experts 16 NJ wn + 16 j + 4 lg .. +3
  float* const part = a.scores + static_cast<size_t>(slice) * a.T * a.n_routed;
#pragma unroll
  for (int i = 0; i < P::MI; ++i) {
    const int row = 16 * (WM * i + wm) + lr;
    if (row >= valid) continue;
    float* const dst = part + static_cast<size_t>(t0 + row) * a.n_routed;
#pragma unroll
    for (int j = 0; j < P::NJ; ++j) {
      const int e = 16 * P::NJ * wn + 16 * j + 4 * lg;
      if (e < a.n_routed)   // n_routed % 4 == 0: all four or none
        *reinterpret_cast<float4*>(dst + e) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
  }
}

// One wave per token: the slices' logits summed in slice order, sigmoid,
// top-K.
template <int NRMAX>
__global__ __launch_bounds__(256) void route_finish_kernel(RouteArgs a) {
  constexpr int NQ = NRMAX / 64;
  __shared__ float srow_s[4][NRMAX];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wv;
  float bq[NQ];
  load_bias(a.bias, a.n_routed, bq);
  if (t >= a.T) return;
  float* const srow = srow_s[wv];
  const size_t slice_stride = static_cast<size_t>(a.T) * a.n_routed;
  const float* const src = a.scores + static_cast<size_t>(t) * a.n_routed;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = lane + 64 * q;
    if (e < a.n_routed) {
      float z = 0.f;
      for (int sl = 0; sl < a.ksplit; ++sl) z += src[sl * slice_stride + e];
      srow[e] = sigmoid_f32(z);
    }
  }
  __builtin_amdgcn_wave_barrier();
  select_topk(srow, bq, a, a.idx + static_cast<size_t>(t) * a.top_k, a.gate + static_cast<size_t>(t) * a.top_k);
}

template <int FMT, int NRMAX>
hipError_t launch_route_t(const RouteArgs& a, hipStream_t s) {
  if constexpr (FMT == FMT_BF16 && NRMAX == 256) {
    if (a.ksplit > 0 && a.scores != nullptr) {
      hipLaunchKernelGGL(route_part_kernel, dim3(ceil_div(a.T, 256), a.ksplit), dim3(KS_THREADS), 0, s, a);
      hipLaunchKernelGGL((route_finish_kernel<NRMAX>), dim3(ceil_div(a.T, 4)), dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  if (route_split(a.T) && a.scores != nullptr) {
    hipLaunchKernelGGL((route_scores_kernel<FMT>), dim3(ceil_div(a.T, RBT), ceil_div(a.n_routed, SCHUNK)), dim3(512),
                       0, s, a);
    hipLaunchKernelGGL((route_topk_kernel<NRMAX>), dim3(ceil_div(a.T, 4)), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((route_kernel<FMT, NRMAX>), dim3(ceil_div(a.T, RBT)), dim3(64 * RouteCfg<NRMAX>::NW), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

MOE_DEBUG_FILE(route)

hipError_t launch_route(int fmt, const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int nr = a.n_routed;
  if (fmt == FMT_BF16) {
    if (nr <= 64) return launch_route_t<FMT_BF16, 64>(a, s);
    if (nr <= 128) return launch_route_t<FMT_BF16, 128>(a, s);
    return nr <= 256 ? launch_route_t<FMT_BF16, 256>(a, s) : launch_route_t<FMT_BF16, 512>(a, s);
  }
  if (nr <= 64) return launch_route_t<FMT_F32, 64>(a, s);
  if (nr <= 128) return launch_route_t<FMT_F32, 128>(a, s);
  return nr <= 256 ? launch_route_t<FMT_F32, 256>(a, s) : launch_route_t<FMT_F32, 512>(a, s);
}

}  // namespace moe
