// Router: affinity GEMM fused with sigmoid, bias add, wavefront top-K and
// gate normalisation (DeepSeek-V3 Technical Report summary, section 2:
// s_{i,t} = Sigmoid(u_t^T e_i); g'_{i,t} = s_{i,t} when s_{i,t} + b_i is among
// the K_r largest of {s_{j,t} + b_j}, else 0; g_{i,t} = g' normalised).
//
// One block routes 32 tokens against every expert: the logits of one chunk
// of 256 experts come from the MFMA tile core (fp32 accumulation); their
// sigmoids go to LDS (the logits never reach HBM); then each wave selects
// the top-K of 8 tokens, with the N_r scores of a token spread 1..8 per lane.
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

template <int FMT, int NRMAX>
struct RouteSmem {
  static constexpr int SSTRIDE = NRMAX + 4;
  static constexpr size_t kTile = sizeof(TileSmem<RBT, RCHUNK>);
  static constexpr size_t kScores = sizeof(float) * RBT * SSTRIDE;
  // With a single expert chunk the score buffer reuses the staging buffers.
  static constexpr size_t kBytes = NRMAX <= RCHUNK ? (kTile > kScores ? kTile : kScores) : kTile + kScores;
  static constexpr size_t kScoreOff = NRMAX <= RCHUNK ? 0 : kTile;
};

template <int FMT, int NRMAX>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  using Core = GemmCore<FMT, RBT, RCHUNK>;
  using SM = RouteSmem<FMT, NRMAX>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[SM::kBytes];
  auto& tile = *reinterpret_cast<TileSmem<RBT, RCHUNK>*>(lds);
  float* sbuf = reinterpret_cast<float*>(lds + SM::kScoreOff);

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int t0 = blockIdx.x * RBT;
  const int es = FMT == FMT_F32 ? 4 : 2;
  const size_t row_bytes = static_cast<size_t>(a.d) * es;
  const int nk = static_cast<int>(row_bytes / KSTEP_BYTES);
  const int brow[4] = {64 * w, 64 * w + 16, 64 * w + 32, 64 * w + 48};
  const float* no_scale[4] = {nullptr, nullptr, nullptr, nullptr};
  const int nvalid = ceil_div(min(RBT, a.T - t0), 16);

  for (int ec = 0; ec < a.n_routed; ec += RCHUNK) {
    Core core;
    core.psa = nullptr;
    {
      int r = Core::slot_row(0);
      int t = t0 + r < a.T ? t0 + r : t0;
      core.pa[0] = static_cast<const uint8_t*>(a.u) + t * row_bytes + Core::slot_col();
#pragma unroll
      for (int i = 0; i < Core::NB; ++i) {
        int e = ec + Core::slot_row(i);
        if (e >= a.n_routed) e = 0;
        core.pb[i] = static_cast<const uint8_t*>(a.centroids) + e * row_bytes + Core::slot_col();
      }
    }
    f32x4 acc[RBT / 16][4];
#pragma unroll
    for (int i = 0; i < RBT / 16; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    gemm_mainloop<FMT, RBT, RCHUNK>(core, tile, nk, brow, nvalid, acc, no_scale);

#pragma unroll
    for (int i = 0; i < RBT / 16; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = ec + brow[j] + lr;
        if (e < a.n_routed) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sbuf[(16 * i + 4 * lg + r) * SM::SSTRIDE + e] = sigmoid_f32(acc[i][j][r]);
        }
      }
    __syncthreads();
  }

  // ---- top-K: wave w takes tokens 8w .. 8w+7 of the block
  constexpr int NQ = NRMAX / 64;
  float bq[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = lane + 64 * q;
    bq[q] = e < a.n_routed ? a.bias[e] : 0.f;
  }
  for (int tt = 0; tt < RBT / 4; ++tt) {
    const int tl = w * (RBT / 4) + tt;
    const int t = t0 + tl;
    if (t >= a.T) break;
    const float* srow = sbuf + tl * SM::SSTRIDE;
    float key[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = lane + 64 * q;
      float v = -INFINITY;
      if (e < a.n_routed) {
        v = srow[e] + bq[q];
        if (v != v) v = -INFINITY;
      }
      key[q] = v;
    }
    uint32_t taken = 0;
    int chosen = 0;     // lane k keeps the k-th selected expert
    float chosen_s = 0.f;
    float sum = 0.f;
    for (int k = 0; k < a.top_k; ++k) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int e = lane + 64 * q;
        const bool cand = e < a.n_routed && !((taken >> q) & 1u);
        if (cand && (key[q] > bv || (key[q] == bv && e < be))) { bv = key[q]; be = e; }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      const float s_sel = srow[be];
      sum += s_sel;
      if (lane == k) { chosen = be; chosen_s = s_sel; }
    }
    if (lane < a.top_k) {
      a.idx[static_cast<size_t>(t) * a.top_k + lane] = chosen;
      a.gate[static_cast<size_t>(t) * a.top_k + lane] = chosen_s / sum;
    }
  }
}

template <int FMT, int NRMAX>
hipError_t launch_route_t(const RouteArgs& a, hipStream_t s) {
  const int grid = ceil_div(a.T, RBT);
  hipLaunchKernelGGL((route_kernel<FMT, NRMAX>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(int fmt, const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const bool wide = a.n_routed > 256;
  if (fmt == FMT_BF16) return wide ? launch_route_t<FMT_BF16, 512>(a, s) : launch_route_t<FMT_BF16, 256>(a, s);
  return wide ? launch_route_t<FMT_F32, 512>(a, s) : launch_route_t<FMT_F32, 256>(a, s);
}

}  // namespace moe
