// MFMA tile pipeline: C[BM x BNW] += X[BM x K] * W[BNW x K]^T, both operands
// K-contiguous in global memory.
//
// Data movement: every K-step ("stage") moves SB bytes of K per row (64 bytes
// = 32 bf16 / 16 fp32, or 128 bytes = 128 e4m3) straight from global memory
// into LDS with buffer_load_dwordx4 ... lds (no register staging).  NST stage
// buffers form a ring and the loads run ahead of the MFMAs.  The DMA is
// issued through asm and the pipelines order it against the fragment reads
// themselves: explicit vmcnt waits by the loading waves, then a bare
// s_barrier.
//
// LDS layout: rows of SB bytes, unpadded; the 16-byte chunk j of row r sits at
// position j ^ swz(r), which makes the MFMA fragment reads bank-conflict free
// (see swz below).  The loader picks, for each lane, the global chunk that
// belongs at the LDS position the DMA writes it to.
//
// Compute: NW computing waves laid out WM x (NW/WM).  A wave owns NJ =
// BNW*WM/(16 NW) column subtiles of W (16 W rows each, offsets chosen by the
// caller) and every WM-th 16-row subtile of X starting at subtile wm = w % WM,
// so short tiles stay balanced across the wave rows.  The MFMA's first
// operand is the W fragment, its second the X fragment, so a lane's four
// accumulators are four consecutive output columns of one X row (row
// lane & 15 of a subtile).  The K loop is instantiated for NSUB = number of
// the wave's leading row subtiles to compute, so a short expert group issues
// MFMAs only for its rows and the loop carries no branches.
//
// FP8 (OCP e4m3): a stage is exactly one 128-wide scale block along K; each
// 16x16x128 product is formed from zero and promoted into the fp32
// accumulator as acc += P * (s_x[row] * s_w[column block]) -- fine-grained
// scaling with FP32 promotion every 128 K-elements.
#pragma once

#include "moe_common.hpp"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Raw buffer resource over [base, base + bytes): loads at offsets past the
// range return zeros instead of touching memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// buffer_load ... lds: each lane's 16 (4) bytes at voff + soff go to LDS at
// l + 16 * lane (4 * lane); soff and l (in M0) are wave-uniform.  Written as asm so that
// the compiler does not track these LDS writes: it cannot tell most fragment
// reads from the stage buffers being refilled, and before such a read it
// would wait for every load in flight (vmcnt(0)), loads just issued for
// stages two ahead included.  The pipelines order the DMA and the reads
// themselves (explicit vmcnt waits, then a barrier).  No register outputs:
// the instruction reads voff, r and soff at issue and writes only LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* l) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_ptr)const_cast<void*>(l)));
}
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, void* l) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff)),
                  "s"(__builtin_amdgcn_readfirstlane(lds_addr(l))) : "m0");
}
__device__ __forceinline__ void dma4(rsrc_t r, uint32_t voff, uint32_t soff, void* l) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff)),
                  "s"(__builtin_amdgcn_readfirstlane(lds_addr(l))) : "m0");
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
// reads row (l & 15) of a 16-row block at logical chunk (l >> 4) (64-byte
// rows; 2 (l >> 4) and 2 (l >> 4) + 1 for 128-byte rows) is free of bank
// conflicts with these two maps, at every block base; plain row-major,
// 144-byte padded rows and several maps that are conflict-free under a plain
// address-modulo bank model (e.g. (r >> 1) & 7 for 128-byte rows) conflict
// there.  Both depend on the row modulo 16 only, so every fragment of a
// 16-row subtile shares one lane address pattern.
template <int SB>
__device__ __forceinline__ int swz(int r) {
  if constexpr (SB == 64)
    return (r >> 1) & 3;
  else
    return (r & 7) ^ ((r >> 3) & 1);
}

// W rows read by one wave: subtile j covers rows base + 16 j, plus SPLIT
// for the second half of the subtiles (j >= NJ / 2).  base is wave-uniform
// and a multiple of 16, so a row's swizzle (a function of the row modulo 16)
// is fixed by the lane, and every fragment address is one register plus an
// immediate
// (given as a runtime array of rows, the compiler kept one address register
// per subtile and spilled them).
template <int SPLIT>
struct WRows {
  int base;
};

// NW waves compute, laid out WM x (NW / WM); LW waves issue the loads (the
// same waves, or as many load-only waves).
// ACC: how the bf16 MFMAs accumulate -- through the builtin (ACC_BUILTIN) or
// in place through asm (ACC_TIED).
enum : int { ACC_BUILTIN = 0, ACC_TIED = 1 };
template <int FMT, int BM, int BNW, int NST, int WM = 1, int ACC = ACC_BUILTIN, int NW = 4, int LW = NW>
struct Pipe {
  static constexpr int SB = FMT == FMT_E4M3 ? 128 : 64;
  static constexpr int CPR = SB / 16;            // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;           // rows per wave DMA instruction
  static constexpr int NIA = (BM + LW * RPI - 1) / (LW * RPI);
  static constexpr int NIB = BNW / (LW * RPI);
  static constexpr int AROWS = NIA * LW * RPI;
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = AROWS * SB;
  static constexpr int S_OFF = B_OFF + BNW * SB;
  static constexpr int STAGE_BYTES = S_OFF + (FMT == FMT_E4M3 ? 1024 : 0);
  static constexpr int NL = NIA + NIB + (FMT == FMT_E4M3 ? 1 : 0);   // DMA ops per lane per stage
  static constexpr int NJ = BNW * WM / (16 * NW);       // column subtiles per wave
  static constexpr int MI = (BM / 16 + WM - 1) / WM;     // row subtiles per wave
  static_assert(BNW % (LW * RPI) == 0, "W rows must fill whole DMA instructions");
  static_assert(NJ >= 1 && BNW * WM % (16 * NW) == 0, "whole column subtiles per wave");
  static_assert((NW == 4 || NW == 8) && NW % WM == 0 && (LW == 4 || LW == 8), "wave layout");
  static_assert(FMT != FMT_E4M3 || LW == 4, "FP8 scale loads: 4 loading waves");
  static constexpr int N_COMPUTE = NW;
  static_assert(ACC == ACC_BUILTIN || FMT == FMT_BF16, "asm accumulation: bf16 only");
  static constexpr int ACCM = ACC;

  rsrc_t ra, rb, rs;
  uint32_t oa[NIA];   // per-lane byte offsets of the lane's 16-byte piece, K-step 0
  uint32_t ob[NIB];
  uint32_t os;
  // K-step ks of the loop loads K-step (ks + krot) mod nks: tiles that read
  // the same rows start at different points of K, so one fetches a line and
  // the others find it in L2 later instead of all waiting on the same miss.
  // The sum over K is the same, in another order.  0 for FP8 (its scales
  // follow the loop's K-step).
  int krot = 0, nks = 1 << 30;

  // X rows come from resource a (a_off(r): byte offset of X row r of the
  // tile, r < AROWS; the caller maps rows past the valid ones to a valid
  // row), W rows from resource b (b_off(r), r < BNW), FP8 X scales from
  // resource s (s_off(r): byte offset of the scale row of X row r, r < 256).
  // The loads are spread over LW waves: loading wave w (its wave index
  // modulo LW) issues row groups w, w + LW, w + 2 LW, ...
  template <class FA, class FB, class FS>
  __device__ __forceinline__ void init(rsrc_t a, FA a_off, rsrc_t b, FB b_off, rsrc_t sc, FS s_off) {
    const int w = wave_id() % LW, lane = threadIdx.x & 63;
    ra = a;
    rb = b;
    rs = sc;
#pragma unroll
    for (int i = 0; i < NIA; ++i) {
      const int r = RPI * (w + LW * i) + lane / CPR;
      oa[i] = a_off(r) + ((lane % CPR) ^ swz<SB>(r)) * 16;
    }
#pragma unroll
    for (int i = 0; i < NIB; ++i) {
      const int r = RPI * (w + LW * i) + lane / CPR;
      ob[i] = b_off(r) + ((lane % CPR) ^ swz<SB>(r)) * 16;
    }
    os = 0;
    if constexpr (FMT == FMT_E4M3) os = s_off(64 * w + lane);
  }

  // X row-group DMA instructions a stage needs when each wave computes only
  // its first NSUB row subtiles (tile rows < 16 * WM * NSUB): the row groups
  // wholly past them are not loaded at all.
  template <int NSUB>
  static constexpr int nia_for() {
    constexpr int need = (16 * WM * NSUB + LW * RPI - 1) / (LW * RPI);
    return need < NIA ? need : NIA;
  }
  template <int NSUB>
  static constexpr int nl_for() {
    return nia_for<NSUB>() + NIB + (FMT == FMT_E4M3 ? 1 : 0);
  }

  // DMA instruction Q of a stage: NA X row groups, then the W row groups,
  // then (FP8) the X scales.
  template <int Q, int NA>
  __device__ __forceinline__ void issue_one(uint8_t* st, int ks) const {
    const int w = wave_id() % LW;
    int kr = ks + krot;
    if (kr >= nks) kr -= nks;
    const uint32_t kofs = static_cast<uint32_t>(kr) * SB;
    if constexpr (Q < NA)
      dma16(ra, oa[Q], kofs, st + A_OFF + RPI * (w + LW * Q) * SB);
    else if constexpr (Q < NA + NIB)
      dma16(rb, ob[Q - NA], kofs, st + B_OFF + RPI * (w + LW * (Q - NA)) * SB);
    else
      dma4(rs, os, static_cast<uint32_t>(ks) * 4, st + S_OFF + 256 * w);
  }
  template <int LO, int HI, int NA>
  __device__ __forceinline__ void issue_range(uint8_t* st, int ks) const {
    if constexpr (LO < HI) {
      issue_one<LO, NA>(st, ks);
      issue_range<LO + 1, HI, NA>(st, ks);
    }
  }
  // Instructions LO..HI-1 of K-steps ks (into st0) and ks+1 (into st1),
  // interleaved so that the two 64-byte halves of every 128-byte line are
  // requested back to back: the L1 then merges them into one L2 request.
  // With 64-byte pieces requested a K-step apart, each half costs a request
  // of its own, and the number of L2 requests a CU keeps in flight is what
  // limits the loads (measured: 25 vs 32 TB/s of L2 hits, 5.7 vs 6.2 TB/s
  // from HBM).
  template <int LO, int HI, int NA>
  __device__ __forceinline__ void issue_pair_range(uint8_t* st0, uint8_t* st1, int ks) const {
    if constexpr (LO < HI) {
      issue_one<LO, NA>(st0, ks);
      issue_one<LO, NA>(st1, ks + 1);
      issue_pair_range<LO + 1, HI, NA>(st0, st1, ks);
    }
  }

  // One 128-bit LDS read.  Fragments are vector values (i32x4), not i32x4
  // structs: a struct is split into four 32-bit loads that the backend merges
  // again, and the merged read loses the LDS object's alias information; the
  // wait insertion then cannot tell it from the stage buffers being refilled
  // by DMA and waits for every load in flight before it.
  __device__ __forceinline__ static i32x4 frag16(const uint8_t* base, int r, int chunk) {
    return *reinterpret_cast<const i32x4*>(base + r * SB + ((chunk ^ swz<SB>(r)) << 4));
  }

  // Fragments carried from one stage to the next: the W fragments of the
  // wave's column subtiles and the first two X fragments.
  static constexpr int XW = FMT == FMT_E4M3 ? 2 : 1;   // 16-byte pieces per fragment
  // X fragments are read XPD row subtiles ahead of their MFMAs: two with one
  // MFMA wave per SIMD, one with two (the other wave's MFMAs cover the read,
  // and the MFMA wave keeps 4 registers more in a 168-register budget).
  static constexpr int XPD = NW > 4 ? 1 : 2;
  struct Frags {
    i32x4 w[NJ * XW];
    i32x4 x[2 * XW];
    float sx[2];
  };

  __device__ __forceinline__ static int xrow(int i) {   // first X row of the wave's i-th subtile
    return 16 * (WM * i + (WM > 1 ? wave_id() % WM : 0));
  }

  __device__ __forceinline__ static void load_x(const uint8_t* st, int i, i32x4* x, float& sx) {
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
  template <int NSUB, int SPLIT>
  __device__ __forceinline__ static void prefetch(const uint8_t* st, WRows<SPLIT> wr, Frags& f) {
    const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
    const uint8_t* wst = st + B_OFF + wr.base * SB;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = 16 * j + (j >= NJ / 2 ? SPLIT : 0) + lr;
      if constexpr (FMT == FMT_E4M3) {
        f.w[2 * j] = frag16(wst, r, 2 * lg);
        f.w[2 * j + 1] = frag16(wst, r, 2 * lg + 1);
      } else {
        f.w[j] = frag16(wst, r, lg);
      }
    }
    load_x(st, 0, &f.x[0], f.sx[0]);
    if constexpr (NSUB > 1 && XPD == 2) load_x(st, 1, &f.x[XW], f.sx[1]);
  }

  // MFMAs of one stage for the wave's first NSUB row subtiles.  X fragments
  // are read two subtiles ahead of the MFMAs that use them: with one wave per
  // SIMD the MFMA issue blocks for the length of the previous MFMAs, so a read
  // issued after a group of MFMAs would expose its whole LDS latency.
  // sched_barrier pins that order.  sw[j]: FP8 weight scale of subtile j.
  //
  // hook<i>() runs after the MFMAs of subtile i: the pipelines below use it
  // to spread the loads of a refilled stage over the subtiles, a few after
  // each group of MFMAs -- issued back to back they fill the vector memory
  // queue and hold up the wave's MFMA issue.
  template <int NSUB, int I, class H>
  __device__ __forceinline__ static void compute_from(const uint8_t* st, Frags& f, f32x4 (&acc)[MI][NJ],
                                                      const float (&sw)[NJ], H& hook, i32x4 (&xc)[XW],
                                                      i32x4 (&xnx)[XW], float& sc, float& snx) {
    if constexpr (I < NSUB) {
      constexpr int i = I;
      i32x4 xn[XW];
      float sn = 0.f;
      if constexpr (XPD == 2) {
#pragma unroll
        for (int q = 0; q < XW; ++q) xn[q] = xnx[q];
        sn = snx;
        if constexpr (i + 2 < NSUB) load_x(st, i + 2, xn, sn);
      } else {
#pragma unroll
        for (int q = 0; q < XW; ++q) xn[q] = xc[q];
        if constexpr (i + 1 < NSUB) load_x(st, i + 1, xn, sn);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if constexpr (FMT == FMT_BF16) {
          if constexpr (ACC == ACC_TIED)
            mfma_bf16_tied(acc[i][j], f.w[j], xc[0]);
          else
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
      hook.template operator()<i>();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (XPD == 2) {
#pragma unroll
        for (int q = 0; q < XW; ++q) { xc[q] = xnx[q]; xnx[q] = xn[q]; }
        sc = snx;
        snx = sn;
      } else {
#pragma unroll
        for (int q = 0; q < XW; ++q) xc[q] = xn[q];
        sc = sn;
      }
      compute_from<NSUB, I + 1>(st, f, acc, sw, hook, xc, xnx, sc, snx);
    }
  }

  // ---- FP8, W-subtile-outer order (the wave-specialised FP8 pipeline).
  // The stage's X fragments and scales for all NSUB row subtiles are held in
  // registers; the W fragments stream two column subtiles ahead of their
  // MFMAs; the products of column subtile j are promoted while the MFMAs of
  // subtile j+1 run, and the last subtile's products (pp, with their scales
  // psc) are carried into the next stage.  About 250 registers, so that two
  // waves can share a SIMD.
  struct FragsJ {
    i32x4 x[MI][2];
    float sx[MI];
    i32x4 w[2][2];   // the stage's first two W subtiles
  };

  template <int SPLIT>
  __device__ __forceinline__ static void wfrag(const uint8_t* st, WRows<SPLIT> wr, int j, i32x4 (&w)[2]) {
    const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
    const uint8_t* wst = st + B_OFF + wr.base * SB;
    const int r = 16 * j + (j >= NJ / 2 ? SPLIT : 0) + lr;
    w[0] = frag16(wst, r, 2 * lg);
    w[1] = frag16(wst, r, 2 * lg + 1);
  }

  template <int NSUB, int SPLIT>
  __device__ __forceinline__ static void prefetch_jo(const uint8_t* st, WRows<SPLIT> wr, FragsJ& f) {
#pragma unroll
    for (int i = 0; i < NSUB; ++i) load_x(st, i, f.x[i], f.sx[i]);
    wfrag(st, wr, 0, f.w[0]);
    if constexpr (NJ > 1) wfrag(st, wr, 1, f.w[1]);
  }

  template <int NSUB, int J, int SPLIT, class H>
  __device__ __forceinline__ static void compute_jo_from(const uint8_t* st, WRows<SPLIT> wr, FragsJ& f,
                                                         f32x4 (&acc)[MI][NJ], const float (&sw)[NJ], H& hook,
                                                         i32x4 (&wc)[2], i32x4 (&wn1)[2], f32x4 (&pp)[MI],
                                                         float (&psc)[MI]) {
    if constexpr (J < NJ) {
      i32x4 wn2[2];
      if constexpr (J + 2 < NJ) wfrag(st, wr, J + 2, wn2);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 pn[MI];
      const i32x8 wv = {(int)wc[0].x, (int)wc[0].y, (int)wc[0].z, (int)wc[0].w,
                        (int)wc[1].x, (int)wc[1].y, (int)wc[1].z, (int)wc[1].w};
#pragma unroll
      for (int i = 0; i < NSUB; ++i) {
        const i32x8 xv = {(int)f.x[i][0].x, (int)f.x[i][0].y, (int)f.x[i][0].z, (int)f.x[i][0].w,
                          (int)f.x[i][1].x, (int)f.x[i][1].y, (int)f.x[i][1].z, (int)f.x[i][1].w};
        pn[i] = mfma_e4m3(wv, xv, f32x4{0.f, 0.f, 0.f, 0.f});
        // the previous column subtile's product (the previous stage's last, for J == 0)
        if constexpr (J == 0)
          acc[i][NJ - 1] += pp[i] * psc[i];
        else
          acc[i][J - 1] += pp[i] * (f.sx[i] * sw[J - 1]);
      }
#pragma unroll
      for (int i = 0; i < NSUB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // then one promotion
      }
      __builtin_amdgcn_sched_barrier(0);
      hook.template operator()<J>();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NSUB; ++i) pp[i] = pn[i];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        wc[q] = wn1[q];
        if constexpr (J + 2 < NJ) wn1[q] = wn2[q];
      }
      compute_jo_from<NSUB, J + 1>(st, wr, f, acc, sw, hook, wc, wn1, pp, psc);
    } else {
#pragma unroll
      for (int i = 0; i < NSUB; ++i) psc[i] = f.sx[i] * sw[NJ - 1];
    }
  }

  // hook.template operator()<j>() runs after the MFMAs of column subtile j.
  template <int NSUB, int SPLIT, class H>
  __device__ __forceinline__ static void compute_jo(const uint8_t* st, WRows<SPLIT> wr, FragsJ& f,
                                                    f32x4 (&acc)[MI][NJ], const float (&sw)[NJ], H&& hook,
                                                    f32x4 (&pp)[MI], float (&psc)[MI]) {
    i32x4 wc[2] = {f.w[0][0], f.w[0][1]};
    i32x4 wn1[2] = {f.w[1][0], f.w[1][1]};
    compute_jo_from<NSUB, 0>(st, wr, f, acc, sw, hook, wc, wn1, pp, psc);
  }

  // hook.template operator()<i>() runs after the MFMAs of row subtile i.
  template <int NSUB, class H>
  __device__ __forceinline__ static void compute(const uint8_t* st, Frags& f, f32x4 (&acc)[MI][NJ],
                                                 const float (&sw)[NJ], H&& hook) {
    i32x4 xc[XW], xnx[XW];
    float sc = f.sx[0], snx = f.sx[1];
#pragma unroll
    for (int q = 0; q < XW; ++q) { xc[q] = f.x[q]; xnx[q] = f.x[XW + q]; }
    static_assert(FMT != FMT_E4M3, "FP8 tiles run in W-subtile-outer order (compute_jo)");
    compute_from<NSUB, 0>(st, f, acc, sw, hook, xc, xnx, sc, snx);
  }
};

// ---------------------------------------------------------------------------
// Single-stage pipeline (NST >= 3 stage buffers; used with 128-byte K-steps,
// whose loads are whole lines already, and by the router).

template <class P, int NST, int S, int NSUB, bool GUARD, bool SPREAD, class WR>
__device__ __forceinline__ void pipe_step(const P& p, uint8_t* const (&st)[NST], int ks, int nk,
                                          const WR& wr, typename P::Frags& f,
                                          f32x4 (&acc)[P::MI][P::NJ], const float* sw_lds, int sw_stride) {
  if constexpr (GUARD) {
    if (ks >= nk) return;
  }
  constexpr int NA = P::template nia_for<NSUB>();
  constexpr int NL = P::template nl_for<NSUB>();
  // Every step issues exactly one stage of loads (clamped to the last K-step
  // past the end: it lands in a buffer nobody reads), so NST-3 stages newer
  // than ks+1 are always in flight here.  The wait makes stage ks+1 complete
  // for this wave; after the barrier it is complete for all, and nobody still
  // reads the buffer about to be refilled (that of stage ks-1).  Full rounds
  // of NST steps carry no branch: at a control-flow join the compiler loses
  // track of which stage buffer an LDS DMA targets and would wait for every
  // outstanding load before the next LDS read, serialising the pipeline.
  wait_vm_lgkm0<(NST - 3) * NL>();
  block_barrier();
  uint8_t* const dst = st[(S + NST - 1) % NST];
  const int kn = min(ks + NST - 1, nk - 1);
  if constexpr (!SPREAD) p.template issue_range<0, NL, NA>(dst, kn);
  float sw[P::NJ];
#pragma unroll
  for (int j = 0; j < P::NJ; ++j) sw[j] = 1.f;
  if constexpr (P::SB == 128) {
    // the first half of the column subtiles use scale row 0, the second row 1
#pragma unroll
    for (int j = 0; j < P::NJ; ++j) sw[j] = sw_lds[(j >= P::NJ / 2 ? sw_stride : 0) + ks];
  }
  P::template compute<NSUB>(st[S], f, acc, sw, [&]<int I>() {
    if constexpr (SPREAD) p.template issue_range<I * NL / NSUB, (I + 1) * NL / NSUB, NA>(dst, kn);
  });
  // stage ks+1 (if any: past the end this reads a clamped, unused buffer)
  P::template prefetch<NSUB>(st[(S + 1) % NST], wr, f);
}

template <class P, int NST, int S, int NSUB, bool GUARD, bool SPREAD, class WR>
__device__ __forceinline__ void pipe_round(const P& p, uint8_t* const (&st)[NST], int base, int nk,
                                           const WR& wr, typename P::Frags& f,
                                           f32x4 (&acc)[P::MI][P::NJ], const float* sw_lds, int sw_stride) {
  pipe_step<P, NST, S, NSUB, GUARD, SPREAD>(p, st, base + S, nk, wr, f, acc, sw_lds, sw_stride);
  if constexpr (S + 1 < NST)
    pipe_round<P, NST, S + 1, NSUB, GUARD, SPREAD>(p, st, base, nk, wr, f, acc, sw_lds, sw_stride);
}

// The whole K loop (unrolled by the ring size so every stage buffer is a
// compile-time object).  FP8: sw_lds holds the tile's weight-block scales,
// two rows (column subtiles 0-1 and 2-3) of sw_stride entries, one per stage.
template <class P, int NST, int NSUB, bool SPREAD = false, class WR>
__device__ __forceinline__ void pipe_mainloop(const P& p, uint8_t* const (&st)[NST], int nk,
                                              const WR& wr, f32x4 (&acc)[P::MI][P::NJ],
                                              const float* sw_lds = nullptr, int sw_stride = 0) {
  constexpr int NA = P::template nia_for<NSUB>();
  constexpr int NL = P::template nl_for<NSUB>();
  static_assert(NST >= 3 && NL * (NST - 2) < 64, "stage ring");
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) p.template issue_range<0, NL, NA>(st[s], min(s, nk - 1));
  wait_vm_lgkm0<(NST - 2) * NL>();   // stage 0
  block_barrier();
  typename P::Frags f;
  P::template prefetch<NSUB>(st[0], wr, f);
  int base = 0;
  for (; base + NST <= nk; base += NST)
    pipe_round<P, NST, 0, NSUB, false, SPREAD>(p, st, base, nk, wr, f, acc, sw_lds, sw_stride);
  if (base < nk) pipe_round<P, NST, 0, NSUB, true, SPREAD>(p, st, base, nk, wr, f, acc, sw_lds, sw_stride);
  // drain the clamped tail loads; every wave is done with every buffer
  wait_vm_lgkm0<0>();
  block_barrier();
}

// ---------------------------------------------------------------------------
// Wave-specialised paired pipeline (64-byte K-steps, a ring of 5 stage
// buffers, stage s in buffer s % 5).  Waves 0 .. N_COMPUTE-1 only read
// fragments and run the MFMAs; the waves after them only issue loads.  A wave
// that issues a load while the CU's memory requests are backed up (it keeps a
// bounded number in flight) stalls until the load is accepted; in a wave that
// also issues the MFMAs, that stall idles the matrix core for as long as the
// memory system is the bottleneck, serialising memory and math (measured:
// loads alone and MFMAs alone add up to the time of a tile whose MFMA waves
// issue their own loads).
//
// Per pair q (K-steps 2q, 2q+1), both roles pass two barriers:
//   A_q  the MFMA waves are done with stage 2q: the loader refills the
//        buffers of stages 2q-1 and 2q with pair q+2;
//   B_q  the loader's wait completed pair q+1: the MFMA waves read it.
// So pair q+2 has the MFMA time of K-steps 2q+1 .. 2q+3 to arrive.

template <class P, int Q, int NSUB, bool GUARD>
__device__ __forceinline__ void ws_load_pairs(const P& p, uint8_t* const (&st)[5], int q0, int np) {
  constexpr int NA = P::template nia_for<NSUB>();
  constexpr int NL = P::template nl_for<NSUB>();
  const int q = q0 + Q;
  if constexpr (GUARD) {
    if (q >= np) return;
  }
  block_barrier();   // A_q
  // Only the load waves issue loads and they read no LDS, so a branch costs
  // nothing here: the last two pairs issue none.
  if (q + 2 < np) {
    p.template issue_pair_range<0, NL, NA>(st[(2 * Q + 4) % 5], st[(2 * Q + 5) % 5], 2 * (q + 2));
    wait_vm_lgkm0<2 * NL>();   // pair q+1
  } else {
    wait_vm_lgkm0<0>();        // pair q+1 (if any) is the newest
  }
  block_barrier();   // B_q
  if constexpr (Q + 1 < 5) ws_load_pairs<P, Q + 1, NSUB, GUARD>(p, st, q0, np);
}

template <class P, int Q, int NSUB, bool GUARD, class WR>
__device__ __forceinline__ void ws_mfma_pairs(uint8_t* const (&st)[5], int q0, int np, const WR& wr,
                                              typename P::Frags& f, f32x4 (&acc)[P::MI][P::NJ]) {
  const int q = q0 + Q;
  if constexpr (GUARD) {
    if (q >= np) return;
  }
  const float sw[P::NJ] = {};
  P::template compute<NSUB>(st[(2 * Q) % 5], f, acc, sw, []<int I>() {});
  P::template prefetch<NSUB>(st[(2 * Q + 1) % 5], wr, f);
  block_barrier();   // A_q
  P::template compute<NSUB>(st[(2 * Q + 1) % 5], f, acc, sw, []<int I>() {});
  block_barrier();   // B_q
  P::template prefetch<NSUB>(st[(2 * Q + 2) % 5], wr, f);
  if constexpr (Q + 1 < 5) ws_mfma_pairs<P, Q + 1, NSUB, GUARD>(st, q0, np, wr, f, acc);
}

// Returns on every wave; only the computing waves hold results in acc.
// NSUB: the row subtiles loaded (the most any wave row computes); NSUBC:
// those this wave computes (one fewer for a wave row whose last subtile is
// past the tile's rows).
template <class P, int NSUB, int NSUBC = NSUB, class WR>
__device__ __forceinline__ void pipe_mainloop_ws(const P& p, uint8_t* const (&st)[5], int nk,
                                                 const WR& wr, f32x4 (&acc)[P::MI][P::NJ]) {
  static_assert(P::SB == 64, "pairs of 64-byte K-steps");
  constexpr int NA = P::template nia_for<NSUB>();
  constexpr int NL = P::template nl_for<NSUB>();
  static_assert(4 * NL < 64, "vmcnt range");
  const int np = nk / 2;
  if (wave_id() >= P::N_COMPUTE) {
    p.template issue_pair_range<0, NL, NA>(st[0], st[1], 0);
    if (np > 1) {
      p.template issue_pair_range<0, NL, NA>(st[2], st[3], 2);
      wait_vm_lgkm0<2 * NL>();   // pair 0
    } else {
      wait_vm_lgkm0<0>();
    }
    block_barrier();
    int q = 0;
    for (; q + 5 <= np; q += 5) ws_load_pairs<P, 0, NSUB, false>(p, st, q, np);
    if (q < np) ws_load_pairs<P, 0, NSUB, true>(p, st, q, np);
  } else {
    block_barrier();
    typename P::Frags f;
    P::template prefetch<NSUBC>(st[0], wr, f);
    if constexpr (P::ACCM == ACC_TIED) acc_fence(acc);
    int q = 0;
    for (; q + 5 <= np; q += 5) ws_mfma_pairs<P, 0, NSUBC, false>(st, q, np, wr, f, acc);
    if (q < np) ws_mfma_pairs<P, 0, NSUBC, true>(st, q, np, wr, f, acc);
    if constexpr (P::ACCM == ACC_TIED) acc_fence(acc);
  }
}

// ---------------------------------------------------------------------------
// Wave-specialised FP8 pipeline (8 waves, 128-byte K-steps = one scale block,
// a ring of 3 stage buffers, stage s in buffer s % 3).  Waves 4-7 issue the
// loads of stage k+2 as soon as stage k-1's buffer is free; waves 0-3 run the
// MFMAs in W-subtile-outer order.  Two barriers per stage, in this order:
//   B_k  (halfway through the MFMAs of stage k) stage k+1 has landed;
//   A_k  (after the MFMA waves read stage k+1's first fragments) nobody
//        reads stage k any more, and its buffer takes stage k+3.
// Stages k+1 and k+2 are in flight while stage k is computed (the 4-wave
// single-stage ring of 3 keeps one).

template <class P, int S, int NSUB, bool GUARD>
__device__ __forceinline__ void ws8_load_steps(const P& p, uint8_t* const (&st)[3], int k0, int nk) {
  constexpr int NA = P::template nia_for<NSUB>();
  constexpr int NL = P::template nl_for<NSUB>();
  const int ks = k0 + S;
  if constexpr (GUARD) {
    if (ks >= nk) return;
  }
  if (ks + 2 < nk) {
    p.template issue_range<0, NL, NA>(st[(S + 2) % 3], ks + 2);
    wait_vm_lgkm0<NL>();   // stage ks+1
  } else {
    wait_vm_lgkm0<0>();    // stage ks+1 (if any) is the newest
  }
  block_barrier();   // B_ks
  block_barrier();   // A_ks
  if constexpr (S + 1 < 3) ws8_load_steps<P, S + 1, NSUB, GUARD>(p, st, k0, nk);
}

template <class P, int S, int NSUB, bool GUARD, class WR>
__device__ __forceinline__ void ws8_mfma_steps(uint8_t* const (&st)[3], int k0, int nk, const WR& wr,
                                               typename P::FragsJ& f, f32x4 (&acc)[P::MI][P::NJ],
                                               f32x4 (&pp)[P::MI], float (&psc)[P::MI], const float* sw_lds,
                                               int sw_stride) {
  const int ks = k0 + S;
  if constexpr (GUARD) {
    if (ks >= nk) return;
  }
  float sw[P::NJ];
#pragma unroll
  for (int j = 0; j < P::NJ; ++j) sw[j] = sw_lds[(j >= P::NJ / 2 ? sw_stride : 0) + ks];
  P::template compute_jo<NSUB>(st[S], wr, f, acc, sw, []<int J>() {
    if constexpr (J == P::NJ / 2 - 1) block_barrier();   // B_ks
  }, pp, psc);
  // stage ks+1 (past the end: a stale buffer, read and unused)
  P::template prefetch_jo<NSUB>(st[(S + 1) % 3], wr, f);
  block_barrier();   // A_ks
  if constexpr (S + 1 < 3)
    ws8_mfma_steps<P, S + 1, NSUB, GUARD>(st, k0, nk, wr, f, acc, pp, psc, sw_lds, sw_stride);
}

// Returns on every wave; only waves 0-3 hold results in acc.
template <class P, int NSUB, class WR>
__device__ __forceinline__ void pipe_mainloop_ws8(const P& p, uint8_t* const (&st)[3], int nk, const WR& wr,
                                                  f32x4 (&acc)[P::MI][P::NJ], const float* sw_lds,
                                                  int sw_stride) {
  static_assert(P::SB == 128 && P::NJ >= 2, "FP8 stages");
  constexpr int NA = P::template nia_for<NSUB>();
  constexpr int NL = P::template nl_for<NSUB>();
  if (wave_id() >= 4) {
    p.template issue_range<0, NL, NA>(st[0], 0);
    if (nk > 1) {
      p.template issue_range<0, NL, NA>(st[1], 1);
      wait_vm_lgkm0<NL>();   // stage 0
    } else {
      wait_vm_lgkm0<0>();
    }
    block_barrier();
    int k = 0;
    for (; k + 3 <= nk; k += 3) ws8_load_steps<P, 0, NSUB, false>(p, st, k, nk);
    if (k < nk) ws8_load_steps<P, 0, NSUB, true>(p, st, k, nk);
  } else {
    block_barrier();
    typename P::FragsJ f;
    P::template prefetch_jo<NSUB>(st[0], wr, f);
    f32x4 pp[P::MI];
    float psc[P::MI];
#pragma unroll
    for (int i = 0; i < P::MI; ++i) {
      pp[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      psc[i] = 0.f;
    }
    int k = 0;
    for (; k + 3 <= nk; k += 3) ws8_mfma_steps<P, 0, NSUB, false>(st, k, nk, wr, f, acc, pp, psc, sw_lds, sw_stride);
    if (k < nk) ws8_mfma_steps<P, 0, NSUB, true>(st, k, nk, wr, f, acc, pp, psc, sw_lds, sw_stride);
#pragma unroll
    for (int i = 0; i < NSUB; ++i) acc[i][P::NJ - 1] += pp[i] * psc[i];
  }
}

template <int MI, int NJ>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[MI][NJ]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

}  // namespace moe
