// Grouped expert GEMMs (DeepSeek-V3 Technical Report summary, section 2:
// every routed and shared expert is an FFN; the FFN is the SwiGLU operator
// named in the report's FP8 training section).
//
// Row space: grouped rows 0 .. T*K-1 hold the routed assignments in
// expert-major, token-ascending order; rows T*K + s*T + t hold shared expert
// s applied to token t.  A "group" is one routed expert or one shared expert.
// The m-tile list (group, first row, rows) comes from the scan kernel, so no
// host round trip is needed to size the groups.
//
// gate/up:  H[r, n] = SiLU(x_r . Wg[n]) * (x_r . Wu[n]), x_r = u[token(r)] is
//           gathered straight from u by the permutation (the permuted copy of
//           the activations is never written); H is bf16 (fp32 on the fp32
//           path) or, on the FP8 path, e4m3 codes with one fp32 scale per row
//           per 128 columns, quantised in the epilogue.
// down:     Y[r, c] = H_r . Wd[c], stored bf16 (fp32 on the fp32 path).
//
// Block tiles: 256 rows x 256 B rows (gate/up: 128 gate + 128 up rows =
// 128 h columns; down: 256 output columns).  Blocks are mapped to XCDs so
// that each XCD walks a contiguous run of the tile list (expert-major): the
// tiles of one expert run together on one XCD and share its L2 for the
// expert's weights and gathered rows.
#include "gemm_core.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int BM = GG_BM, BNW = GG_BNW;
constexpr int NXCD = 8;

// Logical tile index of this block, or -1 if the block has no work.
__device__ __forceinline__ int xcd_tile(int n_tiles) {
  const int bid = blockIdx.x;
  const int xcd = bid % NXCD, j = bid / NXCD;
  const int chunk = ceil_div(n_tiles, NXCD);
  if (j >= chunk) return -1;
  const int q = xcd * chunk + j;
  return q < n_tiles ? q : -1;
}

template <int FMT>
__global__ __launch_bounds__(256, 1) void gateup_kernel(GateUpArgs a) {
  using Core = GemmCore<FMT, BM, BNW>;
  __shared__ __attribute__((aligned(16))) TileSmem<BM, BNW> smem;
  __shared__ float red[4][BM];

  const int nb_n = ceil_div(a.inter, GG_HCOLS);
  const int q = xcd_tile(*a.mt_count * nb_n);
  if (q < 0) return;
  const int mt = q / nb_n, nb = q % nb_n;
  const int4 tl = a.mtiles[mt];
  const int g = tl.x, row0 = tl.y, rows = tl.z;
  const int n0 = nb * GG_HCOLS;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int es = FMT == FMT_F32 ? 4 : (FMT == FMT_BF16 ? 2 : 1);
  const size_t xrow = static_cast<size_t>(a.d) * es;
  const int nk = static_cast<int>(xrow / KSTEP_BYTES);
  const bool shared = g >= a.n_routed;
  const int gs = shared ? g - a.n_routed : g;
  const uint8_t* wbase = static_cast<const uint8_t*>(shared ? a.w_shared : a.w_routed) +
                         static_cast<size_t>(gs) * 2 * a.inter * xrow;
  auto token_of = [&](int r) -> int {
    const int gr = row0 + r;
    return shared ? gr - a.TK - gs * a.T : a.perm_token[gr];
  };

  Core core;
#pragma unroll
  for (int i = 0; i < Core::NA; ++i) {
    int r = Core::slot_row(i);
    if (r >= rows) r = 0;
    core.pa[i] = static_cast<const uint8_t*>(a.x) + static_cast<size_t>(token_of(r)) * xrow + Core::slot_col();
  }
#pragma unroll
  for (int i = 0; i < Core::NB; ++i) {
    const int rb = Core::slot_row(i);
    int n = n0 + (rb & 127);
    if (n >= a.inter) n = 0;
    const int wr = rb < 128 ? n : a.inter + n;
    core.pb[i] = wbase + static_cast<size_t>(wr) * xrow + Core::slot_col();
  }
  core.psa = nullptr;
  const float* sw_ptr[4] = {nullptr, nullptr, nullptr, nullptr};
  if constexpr (FMT == FMT_E4M3) {
    const int kb = a.d / 128;
    if (tid < BM) core.psa = a.x_scale + static_cast<size_t>(token_of(tid < rows ? tid : 0)) * kb;
    const float* sbase = (shared ? a.sw_shared : a.sw_routed) + static_cast<size_t>(gs) * (2 * a.inter / 128) * kb;
    sw_ptr[0] = sw_ptr[1] = sbase + static_cast<size_t>(n0 / 128) * kb;
    sw_ptr[2] = sw_ptr[3] = sbase + static_cast<size_t>((a.inter + n0) / 128) * kb;
  }

  // wave w: gate columns 32w..32w+31 (subtiles 0,1) and the same up columns (2,3)
  const int brow[4] = {32 * w, 32 * w + 16, 128 + 32 * w, 128 + 32 * w + 16};
  const int nvalid = ceil_div(rows, 16);
  f32x4 acc[BM / 16][4];
#pragma unroll
  for (int i = 0; i < BM / 16; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gemm_mainloop<FMT, BM, BNW>(core, smem, nk, brow, nvalid, acc, sw_ptr);

  // ---- epilogue: h = SiLU(gate) * up
  if constexpr (FMT != FMT_E4M3) {
#pragma unroll
    for (int i = 0; i < BM / 16; ++i) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int col = n0 + 32 * w + 16 * jj + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * i + 4 * lg + r;
          if (i < nvalid && col < a.inter && row < rows) {
            const float hv = silu_f32(acc[i][jj][r]) * acc[i][jj + 2][r];
            const size_t o = static_cast<size_t>(row0 + row) * a.inter + col;
            if constexpr (FMT == FMT_F32)
              static_cast<float*>(a.h)[o] = hv;
            else
              static_cast<uint16_t*>(a.h)[o] = f32_to_bf16(hv);
          }
        }
      }
    }
  } else {
    // 1x128 quantisation of h along I: the 128 columns of this tile are one
    // scale group; a row's amax is reduced across lanes and then waves.
    float hv[BM / 16][2][4];
#pragma unroll
    for (int i = 0; i < BM / 16; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[i][jj][r] = i < nvalid ? silu_f32(acc[i][jj][r]) * acc[i][jj + 2][r] : 0.f;
#pragma unroll
    for (int i = 0; i < BM / 16; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = fmaxf(fabsf(hv[i][0][r]), fabsf(hv[i][1][r]));
        m = wave_max_16(m);
        if (lr == 0) red[w][16 * i + 4 * lg + r] = m;
      }
    }
    __syncthreads();
    const int ncb = a.inter / 128;
#pragma unroll
    for (int i = 0; i < BM / 16; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * i + 4 * lg + r;
        if (i >= nvalid || row >= rows) continue;
        const float m = fmaxf(fmaxf(red[0][row], red[1][row]), fmaxf(red[2][row], red[3][row]));
        const float inv = m == 0.f ? 0.f : 448.f / m;
        const size_t grow = static_cast<size_t>(row0 + row);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int col = n0 + 32 * w + 16 * jj + lr;
          static_cast<uint8_t*>(a.h)[grow * a.inter + col] = static_cast<uint8_t>(f32_to_e4m3(hv[i][jj][r] * inv));
        }
        if (w == 0 && lr == 0) a.h_scale[grow * ncb + nb] = m == 0.f ? 1.f : m / 448.f;
      }
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(256, 1) void down_kernel(DownArgs a) {
  using Core = GemmCore<FMT, BM, BNW>;
  __shared__ __attribute__((aligned(16))) TileSmem<BM, BNW> smem;

  const int nb_n = ceil_div(a.d, BNW);
  const int q = xcd_tile(*a.mt_count * nb_n);
  if (q < 0) return;
  const int mt = q / nb_n, nb = q % nb_n;
  const int4 tl = a.mtiles[mt];
  const int g = tl.x, row0 = tl.y, rows = tl.z;
  const int n0 = nb * BNW;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int es = FMT == FMT_F32 ? 4 : (FMT == FMT_BF16 ? 2 : 1);
  const size_t hrow = static_cast<size_t>(a.inter) * es;
  const int nk = static_cast<int>(hrow / KSTEP_BYTES);
  const bool shared = g >= a.n_routed;
  const int gs = shared ? g - a.n_routed : g;
  const uint8_t* wbase = static_cast<const uint8_t*>(shared ? a.w_shared : a.w_routed) +
                         static_cast<size_t>(gs) * a.d * hrow;

  Core core;
#pragma unroll
  for (int i = 0; i < Core::NA; ++i) {
    int r = Core::slot_row(i);
    if (r >= rows) r = 0;
    core.pa[i] = static_cast<const uint8_t*>(a.h) + static_cast<size_t>(row0 + r) * hrow + Core::slot_col();
  }
#pragma unroll
  for (int i = 0; i < Core::NB; ++i) {
    int c = n0 + Core::slot_row(i);
    if (c >= a.d) c = 0;
    core.pb[i] = wbase + static_cast<size_t>(c) * hrow + Core::slot_col();
  }
  core.psa = nullptr;
  const float* sw_ptr[4] = {nullptr, nullptr, nullptr, nullptr};
  if constexpr (FMT == FMT_E4M3) {
    const int kb = a.inter / 128;
    if (tid < BM) core.psa = a.h_scale + static_cast<size_t>(row0 + (tid < rows ? tid : 0)) * kb;
    const float* sbase = (shared ? a.sw_shared : a.sw_routed) + static_cast<size_t>(gs) * (a.d / 128) * kb;
    const int cb = min(n0 + 64 * w, a.d - 1) / 128;
    sw_ptr[0] = sw_ptr[1] = sw_ptr[2] = sw_ptr[3] = sbase + static_cast<size_t>(cb) * kb;
  }

  const int brow[4] = {64 * w, 64 * w + 16, 64 * w + 32, 64 * w + 48};
  const int nvalid = ceil_div(rows, 16);
  f32x4 acc[BM / 16][4];
#pragma unroll
  for (int i = 0; i < BM / 16; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gemm_mainloop<FMT, BM, BNW>(core, smem, nk, brow, nvalid, acc, sw_ptr);

#pragma unroll
  for (int i = 0; i < BM / 16; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + 64 * w + 16 * j + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * i + 4 * lg + r;
        if (i < nvalid && col < a.d && row < rows) {
          const size_t o = static_cast<size_t>(row0 + row) * a.d + col;
          if constexpr (FMT == FMT_F32)
            static_cast<float*>(a.y)[o] = acc[i][j][r];
          else
            static_cast<uint16_t*>(a.y)[o] = f32_to_bf16(acc[i][j][r]);
        }
      }
    }
  }
}

int grid_for(int max_mtiles, int nb_n) {
  const long long tiles = static_cast<long long>(max_mtiles) * nb_n;
  return static_cast<int>(NXCD * ((tiles + NXCD - 1) / NXCD));
}

}  // namespace

hipError_t launch_gateup(int fmt, const GateUpArgs& a, hipStream_t s) {
  const int grid = grid_for(a.max_mtiles, ceil_div(a.inter, GG_HCOLS));
  if (grid == 0) return hipSuccess;
  if (fmt == FMT_BF16)
    hipLaunchKernelGGL(gateup_kernel<FMT_BF16>, dim3(grid), dim3(256), 0, s, a);
  else if (fmt == FMT_E4M3)
    hipLaunchKernelGGL(gateup_kernel<FMT_E4M3>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(gateup_kernel<FMT_F32>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down(int fmt, const DownArgs& a, hipStream_t s) {
  const int grid = grid_for(a.max_mtiles, ceil_div(a.d, BNW));
  if (grid == 0) return hipSuccess;
  if (fmt == FMT_BF16)
    hipLaunchKernelGGL(down_kernel<FMT_BF16>, dim3(grid), dim3(256), 0, s, a);
  else if (fmt == FMT_E4M3)
    hipLaunchKernelGGL(down_kernel<FMT_E4M3>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(down_kernel<FMT_F32>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
