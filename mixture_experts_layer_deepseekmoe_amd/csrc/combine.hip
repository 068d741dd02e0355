// Combine (DeepSeek-V3 Technical Report summary, section 2):
//   h'_t = u_t + sum_s FFN^(s)_s(u_t) + sum_k g_{t,k} FFN^(r)_{idx[t,k]}(u_t)
// Each token's expert outputs are read from the grouped rows (shared expert s
// at row T*K + s*T + t, routed choice k at row pos[t,k]) and summed in fp32 in
// a fixed order: u, then the shared experts in order, then the routed choices
// in selection order.  No atomics: the result is bit-reproducible.
// One wave per token, 8 columns per lane per chunk (16-byte bf16 loads).
#include "kernels.hpp"
#include "moe_common.hpp"

namespace moe {

namespace {

// Every row is read once and y is written once: non-temporal loads and
// stores keep the streams from displacing each other in the caches
// (measured at d = 7168, 8 + 1 rows per token: 0.280 -> 0.240 ms, 5.9 TB/s).
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

template <int F>
__device__ __forceinline__ void load8(const void* base, size_t off, float v[8]) {
  if constexpr (F == FMT_F32) {
    const f32x4v* p = reinterpret_cast<const f32x4v*>(static_cast<const float*>(base) + off);
    const f32x4v a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const u32x4v r = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(static_cast<const uint16_t*>(base) + off));
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xffffu));
      v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
    }
  }
}

template <int XF, int YF, int OF>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  float gk = 0.f;
  int pk = 0;
  if (lane < a.top_k) {
    gk = a.gate[static_cast<size_t>(t) * a.top_k + lane];
    pk = a.pos[static_cast<size_t>(t) * a.top_k + lane];
    if (!MOE_CHECK(pk >= 0 && pk < a.TK, 401)) pk = 0;
  }
  // Broadcast the K gates and rows while every lane is still active.
  float gs[MAX_TOPK];
  int ps[MAX_TOPK];
#pragma unroll
  for (int k = 0; k < MAX_TOPK; ++k) {
    gs[k] = __shfl(gk, k);
    ps[k] = __shfl(pk, k);
  }
  // CC column chunks of 8 per lane at a time: the loads of one row are
  // independent of each other, so a wave keeps CC of them in flight (the
  // loop over the K choices has a runtime bound and runs in order).
  constexpr int CC = 4;
  const size_t d = a.d;
  for (int c0 = lane * 8; c0 < a.d; c0 += 64 * 8 * CC) {
    float acc[CC][8], v[CC][8];
#pragma unroll
    for (int u = 0; u < CC; ++u)
      if (c0 + 512 * u < a.d) load8<XF>(a.u, static_cast<size_t>(t) * d + c0 + 512 * u, acc[u]);
    for (int s = 0; s < a.n_shared; ++s) {
      const size_t row = static_cast<size_t>(a.TK + static_cast<long long>(s) * a.T + t) * d;
#pragma unroll
      for (int u = 0; u < CC; ++u)
        if (c0 + 512 * u < a.d) load8<YF>(a.yrows, row + c0 + 512 * u, v[u]);
#pragma unroll
      for (int u = 0; u < CC; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] += v[u][i];
    }
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k) {
      if (k >= a.top_k) break;
      const size_t row = static_cast<size_t>(ps[k]) * d;
#pragma unroll
      for (int u = 0; u < CC; ++u)
        if (c0 + 512 * u < a.d) load8<YF>(a.yrows, row + c0 + 512 * u, v[u]);
#pragma unroll
      for (int u = 0; u < CC; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = fmaf(gs[k], v[u][i], acc[u][i]);
    }
#pragma unroll
    for (int u = 0; u < CC; ++u) {
      const int c = c0 + 512 * u;
      if (c >= a.d) continue;
      if constexpr (OF == FMT_F32) {
        f32x4v* o = reinterpret_cast<f32x4v*>(static_cast<float*>(a.out) + static_cast<size_t>(t) * d + c);
        __builtin_nontemporal_store(f32x4v{acc[u][0], acc[u][1], acc[u][2], acc[u][3]}, o);
        __builtin_nontemporal_store(f32x4v{acc[u][4], acc[u][5], acc[u][6], acc[u][7]}, o + 1);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = bf16x2(acc[u][2 * i], acc[u][2 * i + 1]);
        __builtin_nontemporal_store(u32x4v{w[0], w[1], w[2], w[3]},
                                    reinterpret_cast<u32x4v*>(static_cast<uint16_t*>(a.out) + static_cast<size_t>(t) * d + c));
      }
    }
  }
}

template <int XF, int YF>
hipError_t launch_o(int ofmt, const CombineArgs& a, hipStream_t s) {
  const dim3 grid(ceil_div(a.T, 4)), block(256);
  if (ofmt == FMT_F32)
    hipLaunchKernelGGL((combine_kernel<XF, YF, FMT_F32>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((combine_kernel<XF, YF, FMT_BF16>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

MOE_DEBUG_FILE(combine)

hipError_t launch_combine(int xfmt, int yfmt, int ofmt, const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (xfmt == FMT_F32) return yfmt == FMT_F32 ? launch_o<FMT_F32, FMT_F32>(ofmt, a, s) : launch_o<FMT_F32, FMT_BF16>(ofmt, a, s);
  return yfmt == FMT_F32 ? launch_o<FMT_BF16, FMT_F32>(ofmt, a, s) : launch_o<FMT_BF16, FMT_BF16>(ofmt, a, s);
}

}  // namespace moe
