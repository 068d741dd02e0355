// MFMA tile core: C[BM x BNW] += A[BM x K] * B[BNW x K]^T with both operands
// K-contiguous in global memory, staged through LDS 128 bytes of K at a time
// (a "K-step": 64 bf16, 32 fp32 or 128 e4m3 values), double-buffered, with
// the next K-step's global loads in flight while the current one is consumed.
//
// Block = 256 threads = 4 waves laid out 1 x 4: every wave covers all BM rows
// and a quarter of the B rows (four 16-wide column subtiles, whose B-row
// offsets the caller chooses).  Rows are processed in 16-row subtiles; a
// subtile wholly past the tile's valid rows issues no MFMA, so a short
// expert group costs MFMA time in proportion to its rows.
//
// FP8 (OCP e4m3): one K-step is exactly one 128-wide scale block along K, so
// each 16x16x128 MFMA product is formed from zero and promoted into the fp32
// accumulator as acc += P * (s_a[row] * s_b[col block]), which is the
// fine-grained scaling with fp32 promotion every 128 K-elements.
#pragma once

#include "moe_common.hpp"

namespace moe {

constexpr int KSTEP_BYTES = 128;
constexpr int LDS_ROW = KSTEP_BYTES + 16;   // padded row: conflict-free 16-byte fragment reads

template <int BM, int BNW>
struct TileSmem {
  uint8_t a[2][BM * LDS_ROW];
  uint8_t b[2][BNW * LDS_ROW];
  float sa[2][BM];
};

template <int FMT, int BM, int BNW>
struct GemmCore {
  static_assert(BM % 32 == 0 && BNW % 32 == 0, "tile rows must be multiples of 32");
  static constexpr int NA = BM / 32;   // 16-byte load slots per thread for A
  static constexpr int NB = BNW / 32;  // and for B
  static constexpr int MI = BM / 16;   // row subtiles per wave

  const uint8_t* pa[NA];
  const uint8_t* pb[NB];
  const float* psa;                    // FP8: this thread's A row scales (row = tid), or null
  uint4 ra[NA];
  uint4 rb[NB];
  float rsa;

  // Row (within the tile) that load slot i of this thread covers.
  __device__ static int slot_row(int i) { return (threadIdx.x >> 3) + 32 * i; }
  __device__ static int slot_col() { return (threadIdx.x & 7) * 16; }

  __device__ void load(int ks) {
    const size_t off = static_cast<size_t>(ks) * KSTEP_BYTES;
#pragma unroll
    for (int i = 0; i < NA; ++i) ra[i] = *reinterpret_cast<const uint4*>(pa[i] + off);
#pragma unroll
    for (int i = 0; i < NB; ++i) rb[i] = *reinterpret_cast<const uint4*>(pb[i] + off);
    if (FMT == FMT_E4M3 && psa != nullptr) rsa = psa[ks];
  }

  __device__ void store(TileSmem<BM, BNW>& s, int buf) const {
    const int c = slot_col();
#pragma unroll
    for (int i = 0; i < NA; ++i) *reinterpret_cast<uint4*>(&s.a[buf][slot_row(i) * LDS_ROW + c]) = ra[i];
#pragma unroll
    for (int i = 0; i < NB; ++i) *reinterpret_cast<uint4*>(&s.b[buf][slot_row(i) * LDS_ROW + c]) = rb[i];
    if (FMT == FMT_E4M3 && threadIdx.x < BM) s.sa[buf][threadIdx.x] = rsa;
  }

  // One K-step of MFMAs for this wave.  brow[j]: first B row (within the
  // tile) of column subtile j.  nvalid: number of row subtiles with any
  // valid row.  sw[j]: FP8 weight scale of column subtile j for this K-step.
  __device__ static void compute(const TileSmem<BM, BNW>& s, int buf, const int brow[4], int nvalid,
                                 f32x4 (&acc)[MI][4], const float sw[4]) {
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const uint8_t* A = s.a[buf];
    const uint8_t* B = s.b[buf];
    if constexpr (FMT == FMT_BF16 || FMT == FMT_F32) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int koff = c * 64 + lg * 16;
        uint4 bf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const uint4*>(&B[(brow[j] + lr) * LDS_ROW + koff]);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if (i < nvalid) {
            const uint4 af = *reinterpret_cast<const uint4*>(&A[(16 * i + lr) * LDS_ROW + koff]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if constexpr (FMT == FMT_BF16) {
                acc[i][j] = mfma_bf16(af, bf[j], acc[i][j]);
              } else {
                acc[i][j] = mfma_f32(__uint_as_float(af.x), __uint_as_float(bf[j].x), acc[i][j]);
                acc[i][j] = mfma_f32(__uint_as_float(af.y), __uint_as_float(bf[j].y), acc[i][j]);
                acc[i][j] = mfma_f32(__uint_as_float(af.z), __uint_as_float(bf[j].z), acc[i][j]);
                acc[i][j] = mfma_f32(__uint_as_float(af.w), __uint_as_float(bf[j].w), acc[i][j]);
              }
            }
          }
        }
      }
    } else {  // FMT_E4M3: one 16x16x128 MFMA per subtile covers the whole K-step
      const int koff = lg * 32;
      i32x8 bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 lo = *reinterpret_cast<const uint4*>(&B[(brow[j] + lr) * LDS_ROW + koff]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&B[(brow[j] + lr) * LDS_ROW + koff + 16]);
        bf[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        if (i < nvalid) {
          const uint4 lo = *reinterpret_cast<const uint4*>(&A[(16 * i + lr) * LDS_ROW + koff]);
          const uint4 hi = *reinterpret_cast<const uint4*>(&A[(16 * i + lr) * LDS_ROW + koff + 16]);
          const i32x8 af = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          const f32x4 sa = *reinterpret_cast<const f32x4*>(&s.sa[buf][16 * i + 4 * lg]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 p = mfma_e4m3(af, bf[j], zero);
            acc[i][j] += p * (sa * sw[j]);
          }
        }
      }
    }
  }
};

// Runs the whole K loop.  ``sw_ptr[j]`` (FP8 only) points at the weight
// scales of column subtile j, indexed by K-step.
template <int FMT, int BM, int BNW>
__device__ __forceinline__ void gemm_mainloop(GemmCore<FMT, BM, BNW>& core, TileSmem<BM, BNW>& smem, int nk,
                                              const int brow[4], int nvalid,
                                              f32x4 (&acc)[BM / 16][4], const float* const sw_ptr[4]) {
  float sw[4] = {1.f, 1.f, 1.f, 1.f};
  core.load(0);
  core.store(smem, 0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) core.load(ks + 1);
    if constexpr (FMT == FMT_E4M3) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sw[j] = sw_ptr[j][ks];
    }
    GemmCore<FMT, BM, BNW>::compute(smem, buf, brow, nvalid, acc, sw);
    if (ks + 1 < nk) core.store(smem, buf ^ 1);
    __syncthreads();
  }
}

}  // namespace moe
