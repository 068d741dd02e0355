// MFMA tile pipeline: C[BM x BNW] += X[BM x K] * W[BNW x K]^T, both operands
// K-contiguous in global memory.
//
// Data movement: every K-step ("stage") moves SB bytes of K per row (64 bytes
// = 32 bf16 / 16 fp32, or 128 bytes = 128 e4m3) straight from global memory
// into LDS with global_load_lds_dwordx4 (no register staging).  NST stage
// buffers form a ring; loads run NST-2 stages ahead of the MFMAs.  Each stage
// buffer is its own __shared__ object, so the compiler's wait insertion can
// tell the asynchronous LDS writes of one stage from the reads of another; the
// waits on the asynchronous loads are explicit (vmcnt), and the per-stage
// barrier is a bare s_barrier.
//
// LDS layout: rows of SB bytes, unpadded; the 16-byte chunk j of row r sits at
// position j ^ swz(r), which makes the MFMA fragment reads bank-conflict free
// (see swz below).  The loader picks, for each lane, the global chunk that
// belongs at the LDS position the DMA writes it to.
//
// Compute: block = 4 waves laid out WM x (4/WM).  A wave owns NJ = 4*WM
// column subtiles of W (16 W rows each, offsets chosen by the caller) and
// every WM-th 16-row subtile of X starting at subtile wm = w % WM, so short
// tiles stay balanced across the wave rows.  The MFMA's first operand is the
// W fragment, its second the X fragment, so a lane's four accumulators are
// four consecutive output columns of one X row (row lane & 15 of a subtile).
// The K loop is instantiated for NSUB = number of the wave's leading row
// subtiles to compute, so a short expert group issues MFMAs only for its rows
// and the loop carries no branches.  2 x 2 (128 x 128 per wave) reads 20%
// fewer LDS bytes per MFMA than 1 x 4 and measured ~40% faster on gfx950.
//
// FP8 (OCP e4m3): a stage is exactly one 128-wide scale block along K; each
// 16x16x128 product is formed from zero and promoted into the fp32
// accumulator as acc += P * (s_x[row] * s_w[column block]) -- fine-grained
// scaling with FP32 promotion every 128 K-elements.
#pragma once

#include "moe_common.hpp"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

__device__ __forceinline__ void dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)g, (lds_void_ptr)l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)g, (lds_void_ptr)l, 4, 0, 0);
}

// s_waitcnt vmcnt(N) expcnt(any) lgkmcnt(0)  (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Chunk swizzle per row.  Chosen by measurement on gfx950 (SQ_LDS_BANK_CONFLICT
// over a sweep of lane->chunk permutations): a ds_read_b128 in which lane l
// reads row (l & 15) of a 16-row block at logical chunk (l >> 4) is free of
// bank conflicts with these two maps (64- and 128-byte rows), at every block
// base; plain row-major, 144-byte padded rows and several XOR maps that are
// conflict-free under a plain address-modulo bank model all conflict there.
template <int SB>
__device__ __forceinline__ int swz(int r) {
  if constexpr (SB == 64)
    return (r >> 1) & 3;
  else
    return (r ^ (r >> 3)) & 7;
}

template <int FMT, int BM, int BNW, int NST, int WM = 1>
struct Pipe {
  static constexpr int SB = FMT == FMT_E4M3 ? 128 : 64;
  static constexpr int CPR = SB / 16;            // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;           // rows per wave DMA instruction
  static constexpr int NIA = (BM + 4 * RPI - 1) / (4 * RPI);
  static constexpr int NIB = BNW / (4 * RPI);
  static constexpr int AROWS = NIA * 4 * RPI;
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = AROWS * SB;
  static constexpr int S_OFF = B_OFF + BNW * SB;
  static constexpr int STAGE_BYTES = S_OFF + (FMT == FMT_E4M3 ? 1024 : 0);
  static constexpr int NL = NIA + NIB + (FMT == FMT_E4M3 ? 1 : 0);   // DMA ops per lane per stage
  static constexpr int NJ = 4 * WM;                     // column subtiles per wave
  static constexpr int MI = (BM / 16 + WM - 1) / WM;     // row subtiles per wave
  static_assert(BNW % (4 * RPI) == 0, "W rows must fill whole DMA instructions");

  const uint8_t* pa[NIA];
  const uint8_t* pb[NIB];
  const float* psa;

  // a_row(r): first byte of X row r of the tile (r < AROWS; the caller clamps
  // rows past the valid ones to a valid row).  b_row(r): W row r (r < BNW).
  // sa_row(r): FP8 scale row of X row r (r < 256).
  template <class FA, class FB, class FS>
  __device__ __forceinline__ void init(FA a_row, FB b_row, FS sa_row) {
    const int w = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NIA; ++i) {
      const int r = RPI * (w + 4 * i) + lane / CPR;
      pa[i] = a_row(r) + ((lane % CPR) ^ swz<SB>(r)) * 16;
    }
#pragma unroll
    for (int i = 0; i < NIB; ++i) {
      const int r = RPI * (w + 4 * i) + lane / CPR;
      pb[i] = b_row(r) + ((lane % CPR) ^ swz<SB>(r)) * 16;
    }
    psa = nullptr;
    if constexpr (FMT == FMT_E4M3) psa = sa_row(64 * w + lane);
  }

  __device__ __forceinline__ void issue(uint8_t* st, int ks) const {
    const int w = wave_id();
    const size_t kofs = static_cast<size_t>(ks) * SB;
#pragma unroll
    for (int i = 0; i < NIA; ++i) dma16(pa[i] + kofs, st + A_OFF + RPI * (w + 4 * i) * SB);
#pragma unroll
    for (int i = 0; i < NIB; ++i) dma16(pb[i] + kofs, st + B_OFF + RPI * (w + 4 * i) * SB);
    if constexpr (FMT == FMT_E4M3) dma4(psa + ks, st + S_OFF + 256 * w);
  }

  __device__ __forceinline__ static uint4 frag16(const uint8_t* base, int r, int chunk) {
    return *reinterpret_cast<const uint4*>(base + r * SB + ((chunk ^ swz<SB>(r)) << 4));
  }

  // Fragments carried from one stage to the next: the W fragments of the
  // wave's column subtiles and the first two X fragments.
  static constexpr int XW = FMT == FMT_E4M3 ? 2 : 1;   // 16-byte pieces per fragment
  struct Frags {
    uint4 w[NJ * XW];
    uint4 x[2 * XW];
    float sx[2];
  };

  __device__ __forceinline__ static int xrow(int i) {   // first X row of the wave's i-th subtile
    return 16 * (WM * i + (WM > 1 ? wave_id() % WM : 0));
  }

  __device__ __forceinline__ static void load_x(const uint8_t* st, int i, uint4* x, float& sx) {
    const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
    const int r = xrow(i) + lr;
    if constexpr (FMT == FMT_E4M3) {
      x[0] = frag16(st + A_OFF, r, 2 * lg);
      x[1] = frag16(st + A_OFF, r, 2 * lg + 1);
      sx = reinterpret_cast<const float*>(st + S_OFF)[r];
    } else {
      x[0] = frag16(st + A_OFF, r, lg);
    }
  }

  // Reads of a stage's first fragments (issued at the end of the previous
  // stage, so each stage starts on MFMAs).
  template <int NSUB>
  __device__ __forceinline__ static void prefetch(const uint8_t* st, const int (&brow)[NJ], Frags& f) {
    const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if constexpr (FMT == FMT_E4M3) {
        f.w[2 * j] = frag16(st + B_OFF, brow[j] + lr, 2 * lg);
        f.w[2 * j + 1] = frag16(st + B_OFF, brow[j] + lr, 2 * lg + 1);
      } else {
        f.w[j] = frag16(st + B_OFF, brow[j] + lr, lg);
      }
    }
    load_x(st, 0, &f.x[0], f.sx[0]);
    if constexpr (NSUB > 1) load_x(st, 1, &f.x[XW], f.sx[1]);
  }

  // MFMAs of one stage for the wave's first NSUB row subtiles.  X fragments
  // are read two subtiles ahead of the MFMAs that use them: with one wave per
  // SIMD the MFMA issue blocks for the length of the previous MFMAs, so a read
  // issued after a group of MFMAs would expose its whole LDS latency.
  // sched_barrier pins that order.  sw[j]: FP8 weight scale of subtile j.
  template <int NSUB>
  __device__ __forceinline__ static void compute(const uint8_t* st, Frags& f, f32x4 (&acc)[MI][NJ], const float (&sw)[NJ]) {
    uint4 xc[XW], xnx[XW], xn[XW];
    float sc = f.sx[0], snx = f.sx[1], sn = 0.f;
#pragma unroll
    for (int q = 0; q < XW; ++q) { xc[q] = f.x[q]; xnx[q] = f.x[XW + q]; }
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
#pragma unroll
      for (int q = 0; q < XW; ++q) xn[q] = xnx[q];
      sn = snx;
      if (i + 2 < NSUB) load_x(st, i + 2, xn, sn);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if constexpr (FMT == FMT_BF16) {
          acc[i][j] = mfma_bf16(f.w[j], xc[0], acc[i][j]);
        } else if constexpr (FMT == FMT_F32) {
          acc[i][j] = mfma_f32(__uint_as_float(f.w[j].x), __uint_as_float(xc[0].x), acc[i][j]);
          acc[i][j] = mfma_f32(__uint_as_float(f.w[j].y), __uint_as_float(xc[0].y), acc[i][j]);
          acc[i][j] = mfma_f32(__uint_as_float(f.w[j].z), __uint_as_float(xc[0].z), acc[i][j]);
          acc[i][j] = mfma_f32(__uint_as_float(f.w[j].w), __uint_as_float(xc[0].w), acc[i][j]);
        } else {
          const i32x8 wv = {(int)f.w[2 * j].x, (int)f.w[2 * j].y, (int)f.w[2 * j].z, (int)f.w[2 * j].w,
                            (int)f.w[2 * j + 1].x, (int)f.w[2 * j + 1].y, (int)f.w[2 * j + 1].z, (int)f.w[2 * j + 1].w};
          const i32x8 xv = {(int)xc[0].x, (int)xc[0].y, (int)xc[0].z, (int)xc[0].w,
                            (int)xc[1].x, (int)xc[1].y, (int)xc[1].z, (int)xc[1].w};
          const f32x4 p = mfma_e4m3(wv, xv, f32x4{0.f, 0.f, 0.f, 0.f});
          acc[i][j] += p * (sc * sw[j]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < XW; ++q) { xc[q] = xnx[q]; xnx[q] = xn[q]; }
      sc = snx;
      snx = sn;
    }
  }
};

template <class P, int NST, int S, int NSUB, bool GUARD>
__device__ __forceinline__ void pipe_step(const P& p, uint8_t* const (&st)[NST], int ks, int nk,
                                          const int (&brow)[P::NJ], typename P::Frags& f,
                                          f32x4 (&acc)[P::MI][P::NJ], const float* sw_lds, int sw_stride) {
  if constexpr (GUARD) {
    if (ks >= nk) return;
  }
  // Every step issues exactly one stage of loads (clamped to the last K-step
  // past the end: it lands in a buffer nobody reads), so NST-3 stages newer
  // than ks+1 are always in flight here.  The wait makes stage ks+1 complete
  // for this wave; after the barrier it is complete for all, and nobody still
  // reads the buffer about to be refilled (that of stage ks-1).  Full rounds
  // of NST steps carry no branch: at a control-flow join the compiler loses
  // track of which stage buffer an LDS DMA targets and would wait for every
  // outstanding load before the next LDS read, serialising the pipeline.
  wait_vm_lgkm0<(NST - 3) * P::NL>();
  block_barrier();
  p.issue(st[(S + NST - 1) % NST], min(ks + NST - 1, nk - 1));
  float sw[P::NJ];
#pragma unroll
  for (int j = 0; j < P::NJ; ++j) sw[j] = 1.f;
  if constexpr (P::SB == 128) {
    // the first half of the column subtiles use scale row 0, the second row 1
#pragma unroll
    for (int j = 0; j < P::NJ; ++j) sw[j] = sw_lds[(j >= P::NJ / 2 ? sw_stride : 0) + ks];
  }
  P::template compute<NSUB>(st[S], f, acc, sw);
  // stage ks+1 (if any: past the end this reads a clamped, unused buffer)
  P::template prefetch<NSUB>(st[(S + 1) % NST], brow, f);
}

template <class P, int NST, int S, int NSUB, bool GUARD>
__device__ __forceinline__ void pipe_round(const P& p, uint8_t* const (&st)[NST], int base, int nk,
                                           const int (&brow)[P::NJ], typename P::Frags& f,
                                           f32x4 (&acc)[P::MI][P::NJ], const float* sw_lds, int sw_stride) {
  pipe_step<P, NST, S, NSUB, GUARD>(p, st, base + S, nk, brow, f, acc, sw_lds, sw_stride);
  if constexpr (S + 1 < NST) pipe_round<P, NST, S + 1, NSUB, GUARD>(p, st, base, nk, brow, f, acc, sw_lds, sw_stride);
}

// The whole K loop (unrolled by the ring size so every stage buffer is a
// compile-time object).  FP8: sw_lds holds the tile's weight-block scales,
// two rows (column subtiles 0-1 and 2-3) of sw_stride entries, one per stage.
template <class P, int NST, int NSUB>
__device__ __forceinline__ void pipe_mainloop(const P& p, uint8_t* const (&st)[NST], int nk,
                                              const int (&brow)[P::NJ], f32x4 (&acc)[P::MI][P::NJ],
                                              const float* sw_lds = nullptr, int sw_stride = 0) {
  static_assert(NST >= 3 && P::NL * (NST - 2) < 64, "stage ring");
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) p.issue(st[s], min(s, nk - 1));
  wait_vm_lgkm0<(NST - 2) * P::NL>();   // stage 0
  block_barrier();
  typename P::Frags f;
  P::template prefetch<NSUB>(st[0], brow, f);
  int base = 0;
  for (; base + NST <= nk; base += NST)
    pipe_round<P, NST, 0, NSUB, false>(p, st, base, nk, brow, f, acc, sw_lds, sw_stride);
  if (base < nk) pipe_round<P, NST, 0, NSUB, true>(p, st, base, nk, brow, f, acc, sw_lds, sw_stride);
  // drain the clamped tail loads; every wave is done with every buffer
  wait_vm_lgkm0<0>();
  block_barrier();
}

template <int MI, int NJ>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[MI][NJ]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

}  // namespace moe
