// Grouping tokens by expert: a stable counting sort in three passes, plus the
// small kernels around it (FP8 quantisers, the aux-loss-free bias update).
//
//   hist    per block of 256 tokens, per-expert assignment counts (LDS atomics
//           only count, so the result is order independent)
//   scan    one block: per-(block, expert) exclusive prefix over blocks, the
//           expert counts and offsets (exclusive prefix over experts), and
//           the m-tile list of the grouped GEMMs
//   permute per token block again: a token's rank among the block's tokens
//           routed to the same expert comes from a per-expert bitmask of the
//           block's tokens (popcount of the lower bits), so grouped row
//           p = offsets[e] + base[block][e] + rank is the stable
//           (token-ascending) position.  No atomic decides any position.
#include "kernels.hpp"
#include "moe_common.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(GROUP_TB) void hist_kernel(GroupArgs a) {
  __shared__ int h[MAX_ROUTED];
  for (int e = threadIdx.x; e < a.n_routed; e += GROUP_TB) h[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * GROUP_TB + threadIdx.x;
  if (t < a.T) {
    for (int k = 0; k < a.top_k; ++k) {
      const int e = a.idx[static_cast<size_t>(t) * a.top_k + k];
      if (MOE_CHECK(e >= 0 && e < a.n_routed, 201)) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.n_routed; e += GROUP_TB)
    a.block_hist[static_cast<size_t>(blockIdx.x) * a.n_routed + e] = h[e];
}

constexpr int SCAN_THREADS = 1024;
static_assert(MAX_ROUTED + MT_SEGMENTS * MAX_SHARED < SCAN_THREADS, "one tile-list piece per scan thread");

// Inclusive prefix sum of one value per thread over the whole block: within
// each wave by shuffles, then over the 16 wave totals in the first wave.
// Three barriers, where a block-wide Hillis-Steele scan takes two per step.
// wsum: 16 ints of shared memory, free again when this returns.
__device__ __forceinline__ int block_incl_scan(int v, int* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  if (w == 0) {
    int s = lane < SCAN_THREADS / 64 ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < SCAN_THREADS / 64; off <<= 1) {
      const int t = __shfl_up(s, off);
      if (lane >= off) s += t;
    }
    if (lane < SCAN_THREADS / 64) wsum[lane] = s;
  }
  __syncthreads();
  if (w > 0) v += wsum[w - 1];
  __syncthreads();
  return v;
}

__global__ __launch_bounds__(SCAN_THREADS) void scan_kernel(GroupArgs a, int nblk) {
  __shared__ int sc[MAX_ROUTED + MAX_SHARED + 1];
  __shared__ int tmp[MAX_ROUTED + MAX_SHARED + 1];
  __shared__ int pc[MAX_ROUTED + MT_SEGMENTS * MAX_SHARED + 1];
  __shared__ int rb[MT_SEGMENTS + 1];
  __shared__ int rbs[2][MT_SEGMENTS + 1];
  __shared__ int cst[MAX_ROUTED];
  __shared__ int seg_mode;
  __shared__ int wsum[SCAN_THREADS / 64];
  const int tid = threadIdx.x;
  const int nr = a.n_routed;
  // 1. per-expert totals and per-block bases.  The counts of 16 blocks are
  //    loaded together before their bases are written back: a load, store,
  //    load chain per block kept a single load in flight.
  constexpr int HB = 16;
  for (int e = tid; e < nr; e += SCAN_THREADS) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += HB) {
      int h[HB];
#pragma unroll
      for (int j = 0; j < HB; ++j) h[j] = b0 + j < nblk ? a.block_hist[static_cast<size_t>(b0 + j) * nr + e] : 0;
#pragma unroll
      for (int j = 0; j < HB; ++j) {
        if (b0 + j < nblk) a.block_hist[static_cast<size_t>(b0 + j) * nr + e] = run;
        run += h[j];
      }
    }
    a.counts[e] = run;
    sc[e] = run;
  }
  __syncthreads();
  // 2. inclusive scan over experts (nr <= MAX_ROUTED < SCAN_THREADS: one per thread), then offsets
  {
    const int incl = block_incl_scan(tid < nr ? sc[tid] : 0, wsum);
    if (tid < nr) sc[tid] = incl;
  }
  __syncthreads();
  for (int e = tid; e <= nr; e += SCAN_THREADS) a.offsets[e] = e == 0 ? 0 : sc[e - 1];
  if (a.mtiles == nullptr) return;
  __syncthreads();
  // 3. m-tiles: group g (routed experts, then shared experts over all T
  //    tokens) is cut into ceil(M_g / BM) tiles of balanced size.  The tiles
  //    of a group read the same weight blocks at the same time and share
  //    them in L2 only while they run at the same speed; a short remainder
  //    tile would drift away from its partners (measured: 1.5x the HBM
  //    traffic of the grouped GEMM).
  //    The list is laid out in MT_SEGMENTS segments -- the GEMMs give each
  //    XCD an equal share of it, in order -- and each segment holds an equal
  //    share of the routed experts' m-tiles (whole experts) and of every
  //    shared expert's tiles.  With the shared experts' full tiles at the end
  //    of the list, the last XCD carried ~8% more work than the others and
  //    the rest idled for it.
  const int ns = a.n_shared;
  const int n_sh = ceil_div(a.T, a.bm);   // m-tiles of one shared expert
  const int np = nr + MT_SEGMENTS * ns;   // pieces: one per routed expert, one per (shared expert, segment)
  const long long TK = static_cast<long long>(a.T) * a.top_k;
  // Segment s takes routed experts rb[s] .. rb[s+1]-1, cut where the prefix
  // of a per-expert cost crosses s/MT_SEGMENTS of the total: expert g goes to
  // the segment of its first unit of cost, a monotone map.  The cost of an
  // expert is its m-tiles times BM (each tile streams a whole weight block)
  // plus its rows; each segment must fit the blocks the GEMMs give an XCD
  // (seg_cap m-tiles).  The other cut is by m-tile counts.  With the cost cut
  // the GEMMs give XCD x exactly segment x; with the count cut (or when the
  // cost cut does not fit) equal tile counts per XCD (mt_count[1] = -1).
  for (int g = tid; g < nr; g += SCAN_THREADS) {
    const int M = sc[g] - (g ? sc[g - 1] : 0), n = ceil_div(M, a.bm);
    tmp[g] = n;
    cst[g] = n * (a.bm / 16) + ceil_div(M, 16);   // in 16-row units: the prefix stays far below 2^31
  }
  __syncthreads();
  {   // inclusive prefixes of the m-tile counts and of the costs
    const int pt = block_incl_scan(tid < nr ? tmp[tid] : 0, wsum);
    const int pcst = block_incl_scan(tid < nr ? cst[tid] : 0, wsum);
    if (tid < nr) {
      tmp[tid] = pt;
      cst[tid] = pcst;
    }
  }
  __syncthreads();
  // rbs[0][.]: cut by cost, rbs[1][.]: cut by m-tile count
  for (int which = 0; which < 2; ++which) {
    const int* pre = which ? tmp : cst;
    const long long total = nr ? pre[nr - 1] : 0;
    // segment of expert g (g = nr: past the end).  Experts after the last
    // unit of cost (trailing experts without rows) stay in the last segment:
    // every expert 0 .. nr-1 lies in some segment, and rb[MT_SEGMENTS] = nr.
    auto seg_of = [&](int g) {
      if (g >= nr || total == 0) return g >= nr ? MT_SEGMENTS : 0;
      const long long before = g ? pre[g - 1] : 0;
      return static_cast<int>(min(before * MT_SEGMENTS / total, static_cast<long long>(MT_SEGMENTS - 1)));
    };
    if (tid == 0) rbs[which][0] = 0;
    for (int g = tid; g <= nr; g += SCAN_THREADS) {
      const int s1 = seg_of(g), s0 = g ? seg_of(g - 1) : 0;
      for (int x = s0 + 1; x <= s1; ++x) rbs[which][x] = g;
    }
  }
  __syncthreads();
  if (tid == 0) {
    // With few m-tiles per segment the GEMM tiles of an XCD run in a few
    // rounds over its CUs, and equal tile counts matter more than equal cost
    // (bf16 d = 2048, 160 m-tiles: the cost cut was 5% slower, at d = 7168
    // with ~400 m-tiles 1.5% faster).
    const int first = nr && tmp[nr - 1] >= 32 * MT_SEGMENTS ? 0 : 1;
    int pick = -1;
    for (int k = 0; k < 2 && pick < 0; ++k) {
      const int which = k ? 1 - first : first;
      bool fits = true;
      for (int x = 0; x < MT_SEGMENTS; ++x) {
        const int g0 = rbs[which][x], g1 = rbs[which][x + 1];
        const int routed = (g1 ? tmp[g1 - 1] : 0) - (g0 ? tmp[g0 - 1] : 0);
        const int shared = ns * ((x + 1) * n_sh / MT_SEGMENTS - x * n_sh / MT_SEGMENTS);
        fits = fits && routed + shared <= a.seg_cap;
      }
      if (fits) pick = which;
    }
    seg_mode = pick;
    for (int x = 0; x <= MT_SEGMENTS; ++x) rb[x] = rbs[pick < 0 ? 1 : pick][x];
  }
  __syncthreads();
  // piece p -> group, its m-tiles k0 .. k1-1, the group's m-tile count and rows
  auto piece = [&](int p, int& g, int& k0, int& k1, int& n, long long& M) {
    int seg = 0, base = 0;
    for (; seg < MT_SEGMENTS - 1; ++seg) {
      const int len = rb[seg + 1] - rb[seg] + ns;
      if (p < base + len) break;
      base += len;
    }
    const int r0 = rb[seg], rn = rb[seg + 1] - r0;
    const int loc = p - base;
    if (loc < rn) {
      g = r0 + loc;
      M = sc[g] - (g ? sc[g - 1] : 0);
      n = ceil_div(static_cast<int>(M), a.bm);
      k0 = 0;
      k1 = n;
    } else {
      g = nr + (loc - rn);
      M = a.T;
      n = n_sh;
      k0 = seg * n_sh / MT_SEGMENTS;
      k1 = (seg + 1) * n_sh / MT_SEGMENTS;
    }
  };
  for (int p = tid; p < np; p += SCAN_THREADS) {
    int g, k0, k1, n;
    long long M;
    piece(p, g, k0, k1, n, M);
    pc[p] = k1 - k0;
  }
  __syncthreads();
  // exclusive prefix of the pieces' m-tile counts (np <= 576 < SCAN_THREADS:
  // one piece per thread), pc[np] = the total
  {
    const int own = tid < np ? pc[tid] : 0;
    const int incl = block_incl_scan(own, wsum);
    if (tid < np) pc[tid] = incl - own;
    if (tid == np - 1) pc[np] = incl;
    if (np == 0 && tid == 0) pc[0] = 0;
  }
  __syncthreads();
  if (tid == 0) {
    const int run = pc[np];
    MOE_CHECK(run <= MT_SEGMENTS * a.seg_cap, 202);
    a.mt_count[0] = run;
    // the m-tile where each segment starts, for the GEMMs' XCD ranges
    // (cut by cost only: with the cut by m-tile counts, equal tile counts per
    // XCD -- mt_count[1] = -1 -- match the segments as closely and split an
    // expert's tiles between two XCDs where the counts do not divide evenly)
    for (int x = 0; x <= MT_SEGMENTS; ++x) a.mt_count[1 + x] = seg_mode != 0 ? -1 : pc[rb[x] + x * ns];
  }
  __syncthreads();
  // .w = (index within its unit << 8) | unit size: consecutive m-tiles of a
  // piece form units of at most MT_UNIT, whose tiles the GEMMs visit with the
  // m-tile index fastest, so the tiles sharing one weight block run together.
  for (int p = tid; p < np; p += SCAN_THREADS) {
    int g, k0, k1, n;
    long long M;
    piece(p, g, k0, k1, n, M);
    const long long first = g < nr ? (g ? sc[g - 1] : 0) : TK + static_cast<long long>(g - nr) * a.T;
    for (int k = k0; k < k1; ++k) {
      const long long r0 = k * M / n, r1 = (k + 1) * M / n;
      const int loc = k - k0, ustart = loc - loc % MT_UNIT;
      const int usize = min(MT_UNIT, (k1 - k0) - ustart);
      a.mtiles[pc[p] + loc] = make_int4(g, static_cast<int>(first + r0), static_cast<int>(r1 - r0),
                                        ((loc - ustart) << 8) | usize);
    }
  }
}

__global__ __launch_bounds__(GROUP_TB) void permute_kernel(GroupArgs a) {
  __shared__ uint32_t mask[MAX_ROUTED][GROUP_TB / 32];
  __shared__ int base_s[MAX_ROUTED];   // offsets[e] + this block's base for expert e
  const int nr = a.n_routed;
  for (int i = threadIdx.x; i < nr * (GROUP_TB / 32); i += GROUP_TB) (&mask[0][0])[i] = 0;
  for (int e = threadIdx.x; e < nr; e += GROUP_TB)
    base_s[e] = a.offsets[e] + a.block_hist[static_cast<size_t>(blockIdx.x) * nr + e];
  const int tl = threadIdx.x;
  const int t = blockIdx.x * GROUP_TB + tl;
  const bool live = t < a.T;
  const int word = tl >> 5;
  const uint32_t bit = 1u << (tl & 31);
  // the token's K choices, loaded together
  int ev[MAX_TOPK];
#pragma unroll
  for (int k = 0; k < MAX_TOPK; ++k) ev[k] = live && k < a.top_k ? a.idx[static_cast<size_t>(t) * a.top_k + k] : 0;
  __syncthreads();
  if (live) {
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k)
      if (k < a.top_k && MOE_CHECK(ev[k] >= 0 && ev[k] < nr, 203)) atomicOr(&mask[ev[k]][word], bit);
  }
  __syncthreads();
  if (live) {
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k) {
      if (k >= a.top_k) break;
      const int e = ev[k];
      if (!MOE_CHECK(e >= 0 && e < nr, 203)) continue;
      int rank = __popc(mask[e][word] & (bit - 1u));
      for (int wd = 0; wd < word; ++wd) rank += __popc(mask[e][wd]);
      const int p = base_s[e] + rank;
      if (!MOE_CHECK(p >= 0 && p < static_cast<long long>(a.T) * a.top_k, 204)) continue;
      a.pos[static_cast<size_t>(t) * a.top_k + k] = p;
      a.perm_token[p] = t;
    }
  }
}

// FP8 activation quantiser: per row, per 1x128 tile, scale = amax / 448,
// codes = E4M3(x * (448 / amax)); scale 1 and zero codes for an all-zero tile.
// One wave per row; each 16-lane group handles one 128-column tile at a time.
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                        uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int ntile = cols / 128;
  const int grp = lane >> 4, gl = lane & 15;
  for (int tb = 0; tb < ntile; tb += 4) {
    const int tile = tb + grp;
    const bool live = tile < ntile;
    const size_t off = static_cast<size_t>(row) * cols + tile * 128 + gl * 8;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (live) raw = *reinterpret_cast<const uint4*>(x + off);
    float v[8];
    const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(static_cast<uint16_t>(wds[i] & 0xffffu));
      v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(wds[i] >> 16));
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    m = wave_max_16(m);
    const float sc = m == 0.f ? 1.f : m / 448.f;
    const float inv = m == 0.f ? 0.f : 448.f / m;
    const uint32_t lo = e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    const uint32_t hi = e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    if (live) {
      *reinterpret_cast<uint2*>(q + off) = make_uint2(lo, hi);
      if (gl == 0) scale[static_cast<size_t>(row) * ntile + tile] = sc;
    }
  }
}

// FP8 weight quantiser: one block per 128x128 block of one matrix.
template <int FMT>
__global__ __launch_bounds__(256) void quant_weight_kernel(const void* __restrict__ w, int rows, int cols,
                                                           uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int rb = rows / 128, cb = cols / 128;
  const long long blk = blockIdx.x;
  const long long mat = blk / (rb * cb);
  const int bi = static_cast<int>((blk / cb) % rb), bj = static_cast<int>(blk % cb);
  const size_t base = static_cast<size_t>(mat) * rows * cols + static_cast<size_t>(bi) * 128 * cols + bj * 128;
  float v[8][8];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = threadIdx.x + 256 * i;
    const size_t off = base + static_cast<size_t>(c >> 4) * cols + (c & 15) * 8;
    if constexpr (FMT == FMT_BF16) {
      const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + off);
      const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[i][2 * j] = bf16_to_f32(static_cast<uint16_t>(wds[j] & 0xffffu));
        v[i][2 * j + 1] = bf16_to_f32(static_cast<uint16_t>(wds[j] >> 16));
      }
    } else {
      const float4 r0 = *reinterpret_cast<const float4*>(static_cast<const float*>(w) + off);
      const float4 r1 = *reinterpret_cast<const float4*>(static_cast<const float*>(w) + off + 4);
      v[i][0] = r0.x; v[i][1] = r0.y; v[i][2] = r0.z; v[i][3] = r0.w;
      v[i][4] = r1.x; v[i][5] = r1.y; v[i][6] = r1.z; v[i][7] = r1.w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[i][j]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = m == 0.f ? 1.f : m / 448.f;
  const float inv = m == 0.f ? 0.f : 448.f / m;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = threadIdx.x + 256 * i;
    const size_t off = base + static_cast<size_t>(c >> 4) * cols + (c & 15) * 8;
    const uint32_t lo = e4m3x4(v[i][0] * inv, v[i][1] * inv, v[i][2] * inv, v[i][3] * inv);
    const uint32_t hi = e4m3x4(v[i][4] * inv, v[i][5] * inv, v[i][6] * inv, v[i][7] * inv);
    *reinterpret_cast<uint2*>(q + off) = make_uint2(lo, hi);
  }
  if (threadIdx.x == 0) scale[blk] = sc;
}

// Aux-loss-free balancing (section 2 of the xyznot summary): an expert whose
// load is above the batch mean T*K/N_r (decided as N_r * count > T*K) gets
// b -= gamma, one below it b += gamma, one exactly at it is left alone.
__global__ void bias_update_kernel(float* bias, const int32_t* counts, int n_routed, long long total, float gamma) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n_routed) return;
  const long long diff = total - static_cast<long long>(n_routed) * counts[e];
  const float step = diff > 0 ? gamma : (diff < 0 ? -gamma : 0.f);
  bias[e] = bias[e] + step;
}

}  // namespace

MOE_DEBUG_FILE(group)

hipError_t launch_group(const GroupArgs& a, hipStream_t s) {
  const int nblk = ceil_div(a.T, GROUP_TB);
  if (nblk > 0) hipLaunchKernelGGL(hist_kernel, dim3(nblk), dim3(GROUP_TB), 0, s, a);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(SCAN_THREADS), 0, s, a, nblk);
  if (nblk > 0) hipLaunchKernelGGL(permute_kernel, dim3(nblk), dim3(GROUP_TB), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quant_act(const void* x, int rows, int cols, uint8_t* q, float* scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_act_kernel, dim3(ceil_div(rows, 4)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), rows, cols, q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_weight(int fmt, const void* w, long long n, int rows, int cols, uint8_t* q, float* scale,
                               hipStream_t s) {
  const long long nblk = n * (rows / 128) * (cols / 128);
  if (nblk == 0) return hipSuccess;
  if (fmt == FMT_BF16)
    hipLaunchKernelGGL(quant_weight_kernel<FMT_BF16>, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, w, rows,
                       cols, q, scale);
  else
    hipLaunchKernelGGL(quant_weight_kernel<FMT_F32>, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, w, rows,
                       cols, q, scale);
  return hipGetLastError();
}

hipError_t launch_bias_update(float* bias, const int32_t* counts, int n_routed, long long total, float gamma,
                              hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(ceil_div(n_routed, 256)), dim3(256), 0, s, bias, counts, n_routed,
                     total, gamma);
  return hipGetLastError();
}

}  // namespace moe
