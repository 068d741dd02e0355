// Measured ceilings of the chip the MoE kernels run on, beside the published
// peaks: sustained MFMA throughput with random and with all-zero operands
// (the matrix cores' power draw, and so the clock the card holds, depends on
// the data), and HBM streaming read bandwidth through the LDS-DMA path the
// GEMMs use.  Prints one JSON object per measurement.
//
//   peak_probes            (run on the GPU; takes a few seconds)
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int NF = 8;         // operand fragments held per lane
constexpr int MFMA_GRID = 256 * 4;

// Each lane loads NF A and NF B fragments (16 bytes; 32 for fp8) from src at
// (block * 256 + thread) * 2 * NF * W, then runs iters rounds of 32
// independent MFMAs into 32 accumulator tiles, which are summed into out.
template <bool FP8>
__global__ __launch_bounds__(256) void mfma_loop(const uint4* __restrict__ src, float* out, int iters) {
  constexpr int W = FP8 ? 2 : 1;
  const size_t base = (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 2 * NF * W;
  uint4 a[NF * W], b[NF * W];
#pragma unroll
  for (int f = 0; f < NF * W; ++f) {
    a[f] = src[base + f];
    b[f] = src[base + NF * W + f];
  }
  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int fa = (i + j) % NF, fb = (3 * i + j) % NF;
        if constexpr (FP8) {
          const i32x8 av = {(int)a[2 * fa].x, (int)a[2 * fa].y, (int)a[2 * fa].z, (int)a[2 * fa].w,
                            (int)a[2 * fa + 1].x, (int)a[2 * fa + 1].y, (int)a[2 * fa + 1].z, (int)a[2 * fa + 1].w};
          const i32x8 bv = {(int)b[2 * fb].x, (int)b[2 * fb].y, (int)b[2 * fb].z, (int)b[2 * fb].w,
                            (int)b[2 * fb + 1].x, (int)b[2 * fb + 1].y, (int)b[2 * fb + 1].z, (int)b[2 * fb + 1].w};
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 0, 0, 0, 0, 0, 0);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[fa]),
                                                              __builtin_bit_cast(bf16x8, b[fb]), acc[i][j], 0, 0, 0);
        }
      }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// HBM read stream: block b reads its own slab of 256 rows x ROWB bytes, the
// two 64-byte halves of each 128-byte line back to back, into LDS (the
// access pattern of the grouped GEMMs' weight stream).  Offsets stay inside
// the slab (row < 256, k + 16 <= ROWB); LDS offsets < 32 KB.
constexpr int ROWB = 14336;
__global__ __launch_bounds__(256) void hbm_stream(const uint8_t* buf, uint32_t* out, int nslab) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2][16384];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(buf) + static_cast<size_t>(blockIdx.x % nslab) * 256 * ROWB, 0, 256 * ROWB, 0x00020000);
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (16 * (w + 4 * i) + lane / 4) * ROWB + (lane % 4) * 16;
  for (int s = 0; s < ROWB / 64; s += 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds[0] + (w + 4 * i) * 1024), 16, o[i], s * 64, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds[1] + (w + 4 * i) * 1024), 16, o[i], s * 64 + 64, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt((24 & 15) | (7 << 4) | ((24 >> 4) << 14));   // at most 24 loads in flight
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  out[blockIdx.x * 256 + threadIdx.x] = lds[0][threadIdx.x * 16] + lds[1][threadIdx.x * 16];
}

#define CHECK(x)                                                                 \
  do {                                                                           \
    if ((x) != hipSuccess) {                                                     \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(hipGetLastError())); \
      exit(1);                                                                   \
    }                                                                            \
  } while (0)

float time_ms(hipEvent_t e0, hipEvent_t e1) {
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  return ms;
}

// random bf16 / e4m3 bit patterns of N(0, ~0.01) scale
void fill_random(std::vector<uint4>& h, bool fp8) {
  srand(1);
  for (auto& v : h) {
    uint32_t w[4];
    for (int q = 0; q < 4; ++q) {
      if (fp8) {
        uint32_t x = 0;
        for (int k = 0; k < 4; ++k) x |= static_cast<uint32_t>(((rand() & 1) << 7) | ((rand() % 6 + 1) << 3) | (rand() & 7)) << (8 * k);
        w[q] = x;
      } else {
        const uint32_t lo = ((rand() & 1) << 15) | ((0x78 + rand() % 3) << 7) | (rand() & 0x7f);
        const uint32_t hi = ((rand() & 1) << 15) | ((0x78 + rand() % 3) << 7) | (rand() & 0x7f);
        w[q] = lo | (hi << 16);
      }
    }
    v = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

int main() {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float* out;
  CHECK(hipMalloc(&out, MFMA_GRID * 256 * sizeof(float)));
  // ---- MFMA
  for (int fp8 = 0; fp8 < 2; ++fp8) {
    const size_t n = static_cast<size_t>(MFMA_GRID) * 256 * 2 * NF * (fp8 ? 2 : 1);
    std::vector<uint4> h(n);
    fill_random(h, fp8);
    uint4* src;
    CHECK(hipMalloc(&src, n * sizeof(uint4)));
    const int iters = fp8 ? 5000 : 10000;
    const double flops = 2.0 * 16 * 16 * (fp8 ? 128 : 32) * 32.0 * iters * (MFMA_GRID * 4.0);
    for (int zero = 0; zero < 2; ++zero) {
      if (zero)
        CHECK(hipMemset(src, 0, n * sizeof(uint4)));
      else
        CHECK(hipMemcpy(src, h.data(), n * sizeof(uint4), hipMemcpyHostToDevice));
      float best = 1e30f, last = 0.f;
      for (int rep = 0; rep < 10; ++rep) {   // the first launches ramp the clocks
        CHECK(hipEventRecord(e0));
        if (fp8)
          hipLaunchKernelGGL(mfma_loop<true>, dim3(MFMA_GRID), dim3(256), 0, 0, src, out, iters);
        else
          hipLaunchKernelGGL(mfma_loop<false>, dim3(MFMA_GRID), dim3(256), 0, 0, src, out, iters);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        last = time_ms(e0, e1);
        best = last < best ? last : best;
      }
      printf("{\"probe\": \"mfma_%s_%s\", \"tflops_sustained\": %.1f, \"tflops_best\": %.1f, \"launch_ms\": %.2f}\n",
             fp8 ? "e4m3_16x16x128" : "bf16_16x16x32", zero ? "zero_operands" : "random_operands",
             flops / last / 1e9, flops / best / 1e9, last);
    }
    CHECK(hipFree(src));
  }
  // ---- HBM stream (2 GB, read once per launch)
  const int nslab = 512;
  const size_t bytes = static_cast<size_t>(nslab) * 256 * ROWB;
  uint8_t* buf;
  uint32_t* o2;
  CHECK(hipMalloc(&buf, bytes));
  CHECK(hipMalloc(&o2, nslab * 256 * sizeof(uint32_t)));
  CHECK(hipMemset(buf, 1, bytes));
  float best = 1e30f;
  for (int rep = 0; rep < 10; ++rep) {
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(hbm_stream, dim3(nslab), dim3(256), 0, 0, buf, o2, nslab);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    const float ms = time_ms(e0, e1);
    best = ms < best ? ms : best;
  }
  printf("{\"probe\": \"hbm_read_lds_dma_paired_64B\", \"gbs_best\": %.1f, \"bytes\": %zu}\n", bytes / best / 1e6, bytes);
  CHECK(hipDeviceSynchronize());
  return 0;
}
