// Shared device helpers for the gfx950 (CDNA4) DeepSeekMoE kernels:
// number formats, MFMA wrappers, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Element formats handled by the kernels.
enum : int { FMT_F32 = 0, FMT_BF16 = 1, FMT_E4M3 = 2 };

constexpr int WAVE = 64;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __bf16 bf16pair_t __attribute__((ext_vector_type(2)));
typedef float f32pair_t __attribute__((ext_vector_type(2)));

// Two values to two bf16 (the low half holds a) through the hardware
// conversion: round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32pair_t{a, b}, bf16pair_t));
}

// ---------------------------------------------------------------- OCP FP8 E4M3
//
// E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; largest finite 448,
// no infinities, S.1111.111 is NaN, subnormals m/8 * 2^-6.  Encoding rounds
// to nearest with ties to the even code and saturates at +-448 (values at
// or above the 464 midpoint go to 448; non-finite input is outside the
// contract).  The sign is kept, so -0 encodes as 0x80.
// Four values to four codes (byte r of the result = value r) through the
// hardware conversion, which rounds to nearest even and keeps subnormals.
// Inputs are clamped to +-448 first, so values past the largest finite code
// saturate instead of becoming NaN (fmin/fmax keep -0, which encodes as 0x80).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  auto cl = [](float x) { return fminf(fmaxf(x, -448.0f), 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), lo, true));
}

// ---------------------------------------------------------------- MFMA
//
// 16x16 output tiles on one wave.  Operand fragments: lane l supplies row
// (l & 15) of A (column (l & 15) of B) for a run of consecutive k chosen by
// lane group l >> 4; A and B use the same k assignment, so any fixed
// assignment gives the exact dot products.  Output: lane l holds rows
// 4*(l >> 4) + r, r = 0..3, of column (l & 15).

__device__ __forceinline__ f32x4 mfma_bf16(const i32x4 a, const i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

// The same product accumulated in place (acc tied to the MFMA's destination).
// Written through the builtin, accumulators under register pressure are
// rotated through other registers and copies, or spilled.  The compiler does
// not see this as an MFMA, so the code around it keeps the hazard distances
// itself: acc_fence() before the first and after the last such MFMA, and a
// VALU write of an operand is kept two wait states away by the s_nop in
// front.
__device__ __forceinline__ void mfma_bf16_tied(f32x4& acc, const i32x4 a, const i32x4 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// Pins the accumulators in registers at this point and waits out the MFMA
// dependency distances (at most 19 wait states on gfx950 for an 8-pass MFMA
// result read by VALU, 2 for a VALU write read by an MFMA).
template <int MI, int NJ>
__device__ __forceinline__ void acc_fence(f32x4 (&acc)[MI][NJ]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(acc[i][j]));
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// 16x16x128 OCP-e4m3 product with unit block scales (scale operands of zero
// select the unscaled instruction).
__device__ __forceinline__ f32x4 mfma_e4m3(const i32x8 a, const i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(const float a, const float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_max_16(float v) {  // over lanes sharing l >> 4
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  return v;
}

// SiLU(g) = g * sigmoid(g) through the hardware exp2 and reciprocal: a few
// ulp of fp32, far below the bf16 / e4m3 rounding of the H it feeds, and ~5
// instructions instead of ~30 for expf and an IEEE divide (the gate/up
// epilogue evaluates it for every element of H while its CU has no loads in
// flight).  g -> -inf: exp overflows to inf and the reciprocal to 0.
__device__ __forceinline__ float silu_f32(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

__device__ __forceinline__ float sigmoid_f32(float z) { return 1.0f / (1.0f + expf(-z)); }

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- debug build
//
// Built with -DMOE_DEBUG, MOE_CHECK(cond, id) tests an index at the points
// where a wrong routing result or tile list would send a kernel out of
// bounds; a failure records id (the first one) in this source file's device
// flag and the caller skips the access.  The host reads and clears the flags
// after each call (MOE_DEBUG_FILE below defines this file's reader).
// Without MOE_DEBUG the checks compile to `true`.
#ifdef MOE_DEBUG
static __device__ int g_moe_debug_flag = 0;
__device__ __forceinline__ bool moe_check(bool ok, int id) {
  if (!ok) atomicCAS(&g_moe_debug_flag, 0, id);
  return ok;
}
#define MOE_CHECK(cond, id) moe::moe_check(static_cast<bool>(cond), (id))
#define MOE_DEBUG_FILE(name)                                                                     \
  int debug_take_##name() {                                                                      \
    int v = 0, z = 0;                                                                            \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_moe_debug_flag), sizeof v) != hipSuccess) return -1; \
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_moe_debug_flag), &z, sizeof z) != hipSuccess) return -1;   \
    return v;                                                                                    \
  }
#else
#define MOE_CHECK(cond, id) true
#define MOE_DEBUG_FILE(name)
#endif

}  // namespace moe
