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
// Tiles: BM rows (256; 128 on the FP8 and fp32 paths) x 256 W rows (gate/up: 128 gate + 128 up rows = 128 h columns; down:
// 256 output columns).  Blocks are mapped to XCDs so that each XCD walks a
// contiguous run of the tile list (expert-major): the tiles of one expert run
// together on one XCD and share its L2 for the expert's weights and gathered
// rows.
#include "gemm_core.hpp"
#include "kernels.hpp"
#include "tile_map.hpp"

namespace moe {

namespace {

constexpr int BNW = GG_BNW;

template <int FMT>
struct GG {
  // bf16: 256 rows, 8 MFMA waves (two per SIMD) laid out 2 x 4 (128 rows x
  // 64 W rows each: 8 x 4 accumulator subtiles) + 4 load waves, the
  // wave-specialised paired pipeline on a ring of 5 stage buffers (5 x 32
  // KB: all of the LDS).  Three waves per SIMD leave an MFMA wave 168
  // registers.  FP8: 128 rows, 4 MFMA waves (2 x 2) + 4 load waves, the
  // wave-specialised FP8 pipeline on a ring of 3 (128-byte K-steps).  fp32
  // (only small layers): 128 rows, 4 waves (2 x 2) that load and compute, the
  // single-stage pipeline on 5.
  static constexpr int BM = FMT == FMT_BF16 ? 256 : 128;
  static constexpr int NST = FMT == FMT_E4M3 ? 3 : 5;
  static constexpr int THREADS = FMT == FMT_BF16 ? 768 : (FMT == FMT_E4M3 ? 512 : 256);
  static constexpr int WM = 2;                          // wave rows
  static constexpr int NW = FMT == FMT_BF16 ? 8 : 4;   // computing waves
  static constexpr int LW = 4;                          // loading waves
  // bf16 accumulates in place through asm: with 128 accumulators in a
  // 168-register budget the builtin's accumulators get rotated and spilled
  using P = Pipe<FMT, BM, BNW, NST, WM, FMT == FMT_BF16 ? ACC_TIED : ACC_BUILTIN, NW, LW>;
  static constexpr int HW = 8 * P::NJ;                  // gate/up: h columns per wave
};

// make_pipe() returns the tile's initialised Pipe (the loads' per-lane
// state).  wr: the W rows of this wave's column subtiles.
template <int FMT, int NSUB, int NSUBC, class MK, class WR>
__device__ __forceinline__ void gg_mainloop(const MK& make_pipe, uint8_t* const (&st)[GG<FMT>::NST], int nk,
                                            const WR& wr, f32x4 (&acc)[GG<FMT>::P::MI][GG<FMT>::P::NJ],
                                            const float* sw_lds, int sw_stride) {
  using P = typename GG<FMT>::P;
  if constexpr (FMT == FMT_BF16)
    pipe_mainloop_ws<P, NSUB, NSUBC>(make_pipe(), st, nk, wr, acc);
  else if constexpr (FMT == FMT_E4M3)
    pipe_mainloop_ws8<P, NSUB>(make_pipe(), st, nk, wr, acc, sw_lds, sw_stride);
  else
    pipe_mainloop<P, GG<FMT>::NST, NSUB>(make_pipe(), st, nk, wr, acc, sw_lds, sw_stride);
}

// bf16: where a tile starts along K, in 64-byte K-steps (whole pairs): the
// n-blocks of an m-tile, which share its X rows, start 2 pairs apart.  It
// depends on the n-block only, so the order in which an output element's
// products are summed is the same for every row, whatever else the batch
// holds (a row's result does not depend on how many tokens share its
// expert, nor on which of the expert's m-tiles it falls in).
template <int FMT>
__device__ __forceinline__ int k_rotation(int nb, int nk) {
  if constexpr (FMT != FMT_BF16) {
    return 0;
  } else {
    const int np = nk / 2;
    return 2 * ((2 * nb) % np);
  }
}

constexpr int MAX_KB = 256;   // FP8: at most 256 scale blocks along K (d, I <= 32768)

// The stage ring: NST stage buffers, one after the other in one LDS array
// (the bf16 epilogue reuses it whole as its output tile).
template <int NST>
struct Ring {
  uint8_t* s[NST];
};

template <int NST, int SBY>
__device__ __forceinline__ Ring<NST> make_ring(uint8_t* base) {
  Ring<NST> r;
#pragma unroll
  for (int i = 0; i < NST; ++i) r.s[i] = base + i * SBY;
  return r;
}

// bf16 epilogue, second half: the block's output tile sits in LDS as rows of
// COLS bf16 (PITCH bytes apart); every wave of the block copies it out in
// 16-byte pieces, consecutive lanes along a row, so each store instruction
// writes whole 128-byte lines.  (Written straight from the accumulators,
// a store put 32 contiguous bytes per row and took ~14% of a down tile.)
template <int COLS, int PITCH, int THREADS>
__device__ __forceinline__ void store_tile_from_lds(const uint8_t* lds, int rows, int ncols, uint16_t* dst,
                                                    size_t stride) {
  constexpr int CPR = COLS / 8;   // 16-byte pieces per row
  const int npr = ncols / 8;
  for (int idx = threadIdx.x; idx < rows * CPR; idx += THREADS) {
    const int r = idx / CPR, c = idx - r * CPR;
    if (c < npr)
      *reinterpret_cast<uint4*>(dst + static_cast<size_t>(r) * stride + c * 8) =
          *reinterpret_cast<const uint4*>(lds + r * PITCH + c * 16);
  }
}

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2(bf16x2(a, b), bf16x2(c, d));
}

// Calls f.template operator()<NSUB>() with NSUB = the number of row subtiles
// the first of the WM wave rows computes: ceil(rows / (16 WM)), 1 .. MI.
template <int MI, int WM, int N = 1, class F>
__device__ __forceinline__ void dispatch_rows(int rows, F&& f) {
  if constexpr (N >= MI) {
    f.template operator()<MI>();
  } else {
    if (rows <= 16 * WM * N)
      f.template operator()<N>();
    else
      dispatch_rows<MI, WM, N + 1>(rows, f);
  }
}

// bf16: wave row wm computes the tile's 16-row subtiles wm, wm + WM, ...; when
// the last of them is past the tile's rows, its waves compute one fewer than
// the first wave row instead of a subtile of padding (the loads still cover
// the first wave row's rows).
template <int FMT>
__device__ __forceinline__ bool short_wave_row(int rows) {
  if constexpr (FMT != FMT_BF16) {
    return false;
  } else {
    constexpr int WM = GG<FMT>::WM;
    const int s = (rows + 15) / 16, nsub = (s + WM - 1) / WM;
    return wave_id() % WM + WM * (nsub - 1) >= s;
  }
}

// ------------------------------------------------------------------ gate/up

// Training: the SwiGLU inputs G and U of a gate/up tile (bf16, G in columns
// 0..I-1 of a row of gu, U in I..2I-1), kept for the backward pass, which
// recomputes H from them.  acc[i][jj] holds G and acc[i][jj + NJ/2] the
// matching U of the wave's h columns.
template <class P, int NSUBC, int WM, int HW>
__device__ __forceinline__ void store_gu(const GateUpArgs& a, const f32x4 (&acc)[P::MI][P::NJ], int row0, int rows,
                                         int n0, int wm, int wn) {
  constexpr int NJ2 = P::NJ / 2;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < NSUBC; ++i) {
    const int row = 16 * (WM * i + wm) + lr;
    if (row < rows) {
      uint16_t* const grow = a.gu + static_cast<size_t>(row0 + row) * 2 * a.inter;
#pragma unroll
      for (int jj = 0; jj < NJ2; ++jj) {
        const int col = n0 + HW * wn + 16 * jj + 4 * lg;
        if (col < a.inter) {
          *reinterpret_cast<uint2*>(grow + col) =
              pack_bf16x4(acc[i][jj][0], acc[i][jj][1], acc[i][jj][2], acc[i][jj][3]);
          *reinterpret_cast<uint2*>(grow + a.inter + col) =
              pack_bf16x4(acc[i][jj + NJ2][0], acc[i][jj + NJ2][1], acc[i][jj + NJ2][2], acc[i][jj + NJ2][3]);
        }
      }
    }
  }
}

template <int FMT, int NSUB, int NSUBC, class MK>
__device__ __forceinline__ void gateup_tile(const GateUpArgs& a, const MK& make_pipe, uint8_t* const (&st)[GG<FMT>::NST],
                                            const float* swl, int kb, int nk, int row0, int rows, int n0, int nb,
                                            float (*red)[GG<FMT>::BM]) {
  using P = typename GG<FMT>::P;
  const int w = wave_id(), lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int WM = GG<FMT>::WM, HW = GG<FMT>::HW, NJ2 = P::NJ / 2;
  const int wm = w % WM, wn = w / WM;
  // wave (wm, wn): h columns HW wn .. HW wn + HW - 1 of the tile -- gate
  // subtiles 0 .. NJ/2-1 and the matching up subtiles NJ/2 .. NJ-1 (gate rows
  // 0-127 of the stage, up rows 128-255) -- on row subtiles wm, wm + WM, ...
  const WRows<128 - HW> wr{HW * wn};
  f32x4 acc[P::MI][P::NJ];
  zero_acc(acc);
  gg_mainloop<FMT, NSUB, NSUBC>(make_pipe, st, nk, wr, acc, swl, kb);
  if constexpr (FMT == FMT_BF16) {
    if (a.gu != nullptr && w < GG<FMT>::NW) store_gu<P, NSUBC, WM, HW>(a, acc, row0, rows, n0, wm, wn);
    // H tile (rows x 128 columns, bf16) through LDS; every wave stores
    constexpr int PITCH = GG_HCOLS * 2 + 16;   // padded rows: the 16 rows of a subtile hit different banks
    static_assert(GG<FMT>::BM * PITCH <= GG<FMT>::NST * P::STAGE_BYTES, "output tile fits the stage ring");
    uint8_t* const lds = st[0];
    wait_vm_lgkm0<0>();
    block_barrier();   // every wave is done with the stage ring
    if (w < GG<FMT>::NW) {
#pragma unroll
      for (int i = 0; i < NSUBC; ++i) {
        const int row = 16 * (WM * i + wm) + lr;
#pragma unroll
        for (int jj = 0; jj < NJ2; ++jj) {
          const int col = HW * wn + 16 * jj + 4 * lg;
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = silu_f32(acc[i][jj][r]) * acc[i][jj + NJ2][r];
          *reinterpret_cast<uint2*>(lds + row * PITCH + col * 2) = pack_bf16x4(h[0], h[1], h[2], h[3]);
        }
      }
    }
    wait_vm_lgkm0<0>();
    block_barrier();
    store_tile_from_lds<GG_HCOLS, PITCH, GG<FMT>::THREADS>(lds, rows, min(GG_HCOLS, a.inter - n0),
                                                           static_cast<uint16_t*>(a.h) +
                                                               static_cast<size_t>(row0) * a.inter + n0,
                                                           a.inter);
    return;
  }
  // the load-only waves hold no results (the FP8 epilogue keeps them for its
  // barrier)
  if (FMT != FMT_E4M3 && w >= GG<FMT>::NW) return;

  if constexpr (FMT != FMT_E4M3) {
#pragma unroll
    for (int i = 0; i < NSUBC; ++i) {
      const int row = 16 * (WM * i + wm) + lr;
#pragma unroll
      for (int jj = 0; jj < NJ2; ++jj) {
        const int col = n0 + HW * wn + 16 * jj + 4 * lg;
        if (row < rows && col < a.inter) {
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = silu_f32(acc[i][jj][r]) * acc[i][jj + NJ2][r];
          const size_t o = static_cast<size_t>(row0 + row) * a.inter + col;
          if constexpr (FMT == FMT_F32) {
            *reinterpret_cast<float4*>(static_cast<float*>(a.h) + o) = make_float4(h[0], h[1], h[2], h[3]);
          } else {
            const uint32_t lo = bf16x2(h[0], h[1]);
            const uint32_t hi = bf16x2(h[2], h[3]);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.h) + o) = make_uint2(lo, hi);
          }
        }
      }
    }
  } else {
    // 1x128 quantisation of h along I: the 128 columns of this tile are one
    // scale group.  A row's amax is reduced over its lane's 16 values, the 4
    // lane groups, then the two waves (wn = 0, 1) that share the row.
    float hv[NSUBC][NJ2][4];
    const bool mw = w < 4;   // an MFMA wave
    if (mw && a.gu != nullptr) store_gu<P, NSUBC, WM, HW>(a, acc, row0, rows, n0, wm, wn);
    if (mw) {
#pragma unroll
      for (int i = 0; i < NSUBC; ++i) {
        float m = 0.f;
#pragma unroll
        for (int jj = 0; jj < NJ2; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            hv[i][jj][r] = silu_f32(acc[i][jj][r]) * acc[i][jj + NJ2][r];
            m = fmaxf(m, fabsf(hv[i][jj][r]));
          }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (lg == 0) red[wn][16 * (WM * i + wm) + lr] = m;
      }
    }
    __syncthreads();
    if (!mw) return;
    const int ncb = a.inter / 128;
#pragma unroll
    for (int i = 0; i < NSUBC; ++i) {
      const int row = 16 * (WM * i + wm) + lr;
      if (row < rows) {
        const float m = fmaxf(red[0][row], red[1][row]);
        const float inv = m == 0.f ? 0.f : 448.f / m;
        const size_t grow = static_cast<size_t>(row0 + row);
#pragma unroll
        for (int jj = 0; jj < NJ2; ++jj) {
          const int col = n0 + HW * wn + 16 * jj + 4 * lg;
          const uint32_t q =
              e4m3x4(hv[i][jj][0] * inv, hv[i][jj][1] * inv, hv[i][jj][2] * inv, hv[i][jj][3] * inv);
          *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(a.h) + grow * a.inter + col) = q;
        }
        if (wn == 0 && lg == 0) a.h_scale[grow * ncb + nb] = m == 0.f ? 1.f : m / 448.f;
      }
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(GG<FMT>::THREADS, 1) void gateup_kernel(GateUpArgs a) {
  using P = typename GG<FMT>::P;
  constexpr int NST = GG<FMT>::NST, BM = GG<FMT>::BM;
  __shared__ __attribute__((aligned(1024))) uint8_t ring_lds[NST * P::STAGE_BYTES];
  // FP8 only: the epilogue's row-amax exchange and the weight-block scales
  // (the bf16 ring takes all of the LDS)
  float (*red)[BM] = nullptr;
  float* swl = nullptr;
  if constexpr (FMT == FMT_E4M3) {
    __shared__ float red_s[2][BM];
    __shared__ float swl_s[2 * MAX_KB];
    red = red_s;
    swl = swl_s;
  }

  const int nb_n = ceil_div(a.inter, GG_HCOLS);
  const int q = xcd_tile(a.mt_count, nb_n);
  if (q < 0) return;
  int mt, nb, in_unit;
  tile_coords(a.mtiles, q, nb_n, mt, nb, in_unit);
  if (!MOE_CHECK(mt >= 0 && mt < a.mt_count[0] && nb < nb_n, 301)) return;
  const int4 tl = a.mtiles[mt];
  const int g = tl.x, row0 = tl.y, rows = tl.z;
  if (!MOE_CHECK(g >= 0 && rows >= 1 && rows <= GG<FMT>::BM && row0 >= 0, 302)) return;
  if (!MOE_CHECK(g < a.n_routed ? row0 + rows <= a.TK : (row0 >= a.TK && (row0 - a.TK) % a.T + rows <= a.T), 303))
    return;
  const int n0 = nb * GG_HCOLS;

  const int es = FMT == FMT_F32 ? 4 : (FMT == FMT_BF16 ? 2 : 1);
  const size_t xrow = static_cast<size_t>(a.d) * es;
  const int nk = static_cast<int>(xrow / P::SB);
  const bool shared = g >= a.n_routed;
  const int gs = shared ? g - a.n_routed : g;
  const uint8_t* wbase = static_cast<const uint8_t*>(shared ? a.w_shared : a.w_routed) +
                         static_cast<size_t>(gs) * 2 * a.inter * xrow;
  auto token_of = [&](int r) -> int {
    if (r >= rows) r = 0;
    const int gr = row0 + r;
    const int t = shared ? gr - a.TK - gs * a.T : a.perm_token[gr];
    return MOE_CHECK(t >= 0 && t < a.T, 304) ? t : 0;
  };
  const int kb = a.d / 128;

  // byte offsets fit 32 bits: T * d * element size < 2^32 is checked on the host
  auto make_pipe = [&]() {
    P p;
    p.init(make_rsrc(a.x, static_cast<uint32_t>(a.T * xrow)),
           // rows past the tile's: an offset past the resource, so their
           // loads return zeros without touching memory
           [&](int r) { return static_cast<uint32_t>((r < rows ? token_of(r) : a.T) * xrow); },
           make_rsrc(wbase, static_cast<uint32_t>(2 * a.inter * xrow)),
           [&](int r) {
             int n = n0 + (r & 127);
             if (n >= a.inter) n = 0;
             return static_cast<uint32_t>((r < 128 ? n : a.inter + n) * xrow);
           },
           FMT == FMT_E4M3 ? make_rsrc(a.x_scale, static_cast<uint32_t>(a.T * kb * 4)) : make_rsrc(a.x, 0),
           [&](int r) { return static_cast<uint32_t>(token_of(r) * kb * 4); });
    p.krot = k_rotation<FMT>(nb, nk);
    p.nks = nk;
    return p;
  };

  if constexpr (FMT == FMT_E4M3) {
    // this tile's weight-block scales: gate block n0/128 and up block (I+n0)/128, all K blocks
    const float* sb = (shared ? a.sw_shared : a.sw_routed) + static_cast<size_t>(gs) * (2 * a.inter / 128) * kb;
    for (int i = threadIdx.x; i < 2 * kb; i += GG<FMT>::THREADS)
      swl[i] = i < kb ? sb[static_cast<size_t>(n0 / 128) * kb + i] : sb[static_cast<size_t>((a.inter + n0) / 128) * kb + i - kb];
    __syncthreads();
  }

  const Ring<NST> ring = make_ring<NST, P::STAGE_BYTES>(ring_lds);
  const float* sw = FMT == FMT_E4M3 ? swl : nullptr;
  // the K loop instantiated for the tile's valid rows, in 32-row steps
  const bool short_row = short_wave_row<FMT>(rows);
  dispatch_rows<P::MI, GG<FMT>::WM>(rows, [&]<int NSUB>() {
    if (short_row)
      gateup_tile<FMT, NSUB, (FMT == FMT_BF16 ? NSUB - 1 : NSUB)>(a, make_pipe, ring.s, sw, kb, nk, row0, rows, n0, nb,
                                                                  red);
    else
      gateup_tile<FMT, NSUB, NSUB>(a, make_pipe, ring.s, sw, kb, nk, row0, rows, n0, nb, red);
  });
}

// ------------------------------------------------------------------ down

template <int FMT, int NSUB, int NSUBC, class MK>
__device__ __forceinline__ void down_tile(const DownArgs& a, const MK& make_pipe, uint8_t* const (&st)[GG<FMT>::NST],
                                          const float* swl, int kb, int nk, int row0, int rows, int n0) {
  using P = typename GG<FMT>::P;
  const int w = wave_id(), lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int WM = GG<FMT>::WM;
  const int wm = w % WM, wn = w / WM;
  // wave (wm, wn): output columns 16 NJ wn .. 16 NJ (wn + 1) - 1 of the tile
  // (FP8: 128 columns, one weight scale block), row subtiles wm, wm + WM, ...
  const WRows<0> wr{16 * P::NJ * wn};
  f32x4 acc[P::MI][P::NJ];
  zero_acc(acc);
  gg_mainloop<FMT, NSUB, NSUBC>(make_pipe, st, nk, wr, acc, FMT == FMT_E4M3 ? swl + wn * kb : nullptr, 0);
  if constexpr (FMT == FMT_BF16) {
    // Y tile (rows x 256 columns, bf16) through LDS; every wave stores
    constexpr int PITCH = BNW * 2 + 16;   // padded rows: the 16 rows of a subtile hit different banks
    static_assert(GG<FMT>::BM * PITCH <= GG<FMT>::NST * P::STAGE_BYTES, "output tile fits the stage ring");
    uint8_t* const lds = st[0];
    wait_vm_lgkm0<0>();
    block_barrier();   // every wave is done with the stage ring
    if (w < GG<FMT>::NW) {
#pragma unroll
      for (int i = 0; i < NSUBC; ++i) {
        const int row = 16 * (WM * i + wm) + lr;
#pragma unroll
        for (int j = 0; j < P::NJ; ++j) {
          const int col = 16 * P::NJ * wn + 16 * j + 4 * lg;
          *reinterpret_cast<uint2*>(lds + row * PITCH + col * 2) =
              pack_bf16x4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      }
    }
    wait_vm_lgkm0<0>();
    block_barrier();
    store_tile_from_lds<BNW, PITCH, GG<FMT>::THREADS>(lds, rows, min(BNW, a.d - n0),
                                                      static_cast<uint16_t*>(a.y) + static_cast<size_t>(row0) * a.d + n0,
                                                      a.d);
    return;
  }
  if (w >= GG<FMT>::NW) return;   // FP8: the load-only waves
#pragma unroll
  for (int i = 0; i < NSUBC; ++i) {
    const int row = 16 * (WM * i + wm) + lr;
#pragma unroll
    for (int j = 0; j < P::NJ; ++j) {
      const int col = n0 + 16 * P::NJ * wn + 16 * j + 4 * lg;
      if (row < rows && col < a.d) {
        const size_t o = static_cast<size_t>(row0 + row) * a.d + col;
        if constexpr (FMT == FMT_F32) {
          *reinterpret_cast<float4*>(static_cast<float*>(a.y) + o) =
              make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        } else {
          const uint32_t lo = bf16x2(acc[i][j][0], acc[i][j][1]);
          const uint32_t hi = bf16x2(acc[i][j][2], acc[i][j][3]);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y) + o) = make_uint2(lo, hi);
        }
      }
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(GG<FMT>::THREADS, 1) void down_kernel(DownArgs a) {
  using P = typename GG<FMT>::P;
  constexpr int NST = GG<FMT>::NST;
  __shared__ __attribute__((aligned(1024))) uint8_t ring_lds[NST * P::STAGE_BYTES];
  float* swl = nullptr;   // FP8 only: the weight-block scales
  if constexpr (FMT == FMT_E4M3) {
    __shared__ float swl_s[2 * MAX_KB];
    swl = swl_s;
  }

  const int nb_n = ceil_div(a.d, BNW);
  const int q = xcd_tile(a.mt_count, nb_n);
  if (q < 0) return;
  int mt, nb, in_unit;
  tile_coords(a.mtiles, q, nb_n, mt, nb, in_unit);
  if (!MOE_CHECK(mt >= 0 && mt < a.mt_count[0] && nb < nb_n, 305)) return;
  const int4 tl = a.mtiles[mt];
  const int g = tl.x, row0 = tl.y, rows = tl.z;
  if (!MOE_CHECK(g >= 0 && rows >= 1 && rows <= GG<FMT>::BM && row0 >= 0, 306)) return;
  const int n0 = nb * BNW;

  const int es = FMT == FMT_F32 ? 4 : (FMT == FMT_BF16 ? 2 : 1);
  const size_t hrow = static_cast<size_t>(a.inter) * es;
  const int nk = static_cast<int>(hrow / P::SB);
  const bool shared = g >= a.n_routed;
  const int gs = shared ? g - a.n_routed : g;
  const uint8_t* wbase = static_cast<const uint8_t*>(shared ? a.w_shared : a.w_routed) +
                         static_cast<size_t>(gs) * a.d * hrow;
  const int kb = a.inter / 128;

  // the tile's rows of H (and of its FP8 scales) as resources of their own
  auto make_pipe = [&]() {
    P p;
    p.init(make_rsrc(static_cast<const uint8_t*>(a.h) + static_cast<size_t>(row0) * hrow, static_cast<uint32_t>(rows * hrow)),
           [&](int r) { return static_cast<uint32_t>((r < rows ? r : rows) * hrow); },   // past the rows: zeros
           make_rsrc(wbase, static_cast<uint32_t>(a.d * hrow)),
           [&](int r) {
             int c = n0 + r;
             if (c >= a.d) c = 0;
             return static_cast<uint32_t>(c * hrow);
           },
           FMT == FMT_E4M3 ? make_rsrc(a.h_scale + static_cast<size_t>(row0) * kb, static_cast<uint32_t>(rows * kb * 4))
                           : make_rsrc(a.h, 0),
           [&](int r) { return static_cast<uint32_t>((r < rows ? r : 0) * kb * 4); });
    p.krot = k_rotation<FMT>(nb, nk);
    p.nks = nk;
    return p;
  };

  if constexpr (FMT == FMT_E4M3) {
    // weight-block scales of this tile's two 128-column blocks (the second
    // clamped at the matrix edge), all K blocks
    const float* sb = (shared ? a.sw_shared : a.sw_routed) + static_cast<size_t>(gs) * (a.d / 128) * kb;
    const int b0 = n0 / 128, b1 = min(n0 / 128 + 1, a.d / 128 - 1);
    for (int i = threadIdx.x; i < 2 * kb; i += GG<FMT>::THREADS)
      swl[i] = i < kb ? sb[static_cast<size_t>(b0) * kb + i] : sb[static_cast<size_t>(b1) * kb + i - kb];
    __syncthreads();
  }

  const Ring<NST> ring = make_ring<NST, P::STAGE_BYTES>(ring_lds);
  const float* sw = FMT == FMT_E4M3 ? swl : nullptr;
  const bool short_row = short_wave_row<FMT>(rows);
  dispatch_rows<P::MI, GG<FMT>::WM>(rows, [&]<int NSUB>() {
    if (short_row)
      down_tile<FMT, NSUB, (FMT == FMT_BF16 ? NSUB - 1 : NSUB)>(a, make_pipe, ring.s, sw, kb, nk, row0, rows, n0);
    else
      down_tile<FMT, NSUB, NSUB>(a, make_pipe, ring.s, sw, kb, nk, row0, rows, n0);
  });
}


}  // namespace

MOE_DEBUG_FILE(ggemm)

int gg_bm(int fmt) {
  return fmt == FMT_E4M3 ? GG<FMT_E4M3>::BM : (fmt == FMT_F32 ? GG<FMT_F32>::BM : GG<FMT_BF16>::BM);
}

hipError_t launch_gateup(int fmt, const GateUpArgs& a, hipStream_t s) {
  const int grid = mtile_grid(a.max_mtiles, ceil_div(a.inter, GG_HCOLS));
  if (grid == 0) return hipSuccess;
  if (fmt == FMT_BF16)
    hipLaunchKernelGGL(gateup_kernel<FMT_BF16>, dim3(grid), dim3(GG<FMT_BF16>::THREADS), 0, s, a);
  else if (fmt == FMT_E4M3)
    hipLaunchKernelGGL(gateup_kernel<FMT_E4M3>, dim3(grid), dim3(GG<FMT_E4M3>::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(gateup_kernel<FMT_F32>, dim3(grid), dim3(GG<FMT_F32>::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down(int fmt, const DownArgs& a, hipStream_t s) {
  const int grid = mtile_grid(a.max_mtiles, ceil_div(a.d, BNW));
  if (grid == 0) return hipSuccess;
  if (fmt == FMT_BF16)
    hipLaunchKernelGGL(down_kernel<FMT_BF16>, dim3(grid), dim3(GG<FMT_BF16>::THREADS), 0, s, a);
  else if (fmt == FMT_E4M3)
    hipLaunchKernelGGL(down_kernel<FMT_E4M3>, dim3(grid), dim3(GG<FMT_E4M3>::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(down_kernel<FMT_F32>, dim3(grid), dim3(GG<FMT_F32>::THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
