// The MoE layer backward, bf16 or FP8 (the report's FP8 training section, as
// paraphrased on why-be.co.kr: the Linear operator's Fprop, Dgrad and Wgrad
// GEMMs, all three in FP8 in its Figure 6; the SwiGLU inputs are cached in
// the forward and its output is recomputed in the backward pass).  With the
// expert selection held fixed:
//
//   prep     grouped row r (token t, gate g; g = 1 for a shared expert):
//            dY_r = g dy_t and X_r = u_t as bf16 rows (X_r only for the bf16
//            Wgrad: the FP8 one quantises u by token), dg_{t,k} = dy_t . Y_r
//   dz       per token: S = sum of the selected sigmoids, ds_k = (dg_k -
//            sum_j g_j dg_j) / S, dz_k = ds_k s_k (1 - s_k)
//   dgrad    dH = dY W_down (per group), fused with the SwiGLU backward:
//   down     from the cached G, U: dG = dH U SiLU'(G), dU = dH SiLU(G),
//            and H = SiLU(G) U recomputed for the down Wgrad
//   dgrad    dX = [dG dU] W_gate_up
//   gate/up
//   wgrad    dW_down = dY^T H and dW_gate_up = [dG dU]^T X per group (fp32)
//   du       du_t = dy_t + shared dX rows + routed dX rows + sum_k dz_k e_k
//   dE       dE_e = sum over e's rows of dz u_t
//
// Every sum runs in a fixed order: the results are bit-reproducible.
//
// bf16 GEMM tiles: 256 x 256 outputs, 8 MFMA waves (2 x 4, 128 x 64 each,
// bf16 16x16x32 MFMAs accumulating in place) and 4 load waves that move 32-K
// stages into a ring of LDS buffers by DMA.  An operand is stored either
// K-contiguous (rows of K: the activations of Dgrad) or K-outer (rows along
// K, its M or N index contiguous: the weights of Dgrad, both operands of
// Wgrad).  K-outer fragments come from LDS transpose reads
// (ds_read_b64_tr_b16): lane 16 g + c of a read points at K-row 8 g + c / 4,
// columns 4 (c % 4) .. + 3, and receives the four K-rows 8 g .. 8 g + 3 of
// column 4 (c / 4)' ... -- i.e. each lane gets four consecutive K values of
// its own column; two reads give the eight a 16x16x32 MFMA operand holds.
#include "gemm_core.hpp"
#include "kernels.hpp"
#include "tile_map.hpp"

namespace moe {

namespace {

constexpr int BT = 256;                 // tile rows and columns
constexpr int NSTG = 5;                 // stage buffers (5 x 32 KB: all of the LDS)
constexpr int NMW = 8;                  // MFMA waves
constexpr int NLW = 4;                  // load waves
constexpr int THREADS = 64 * (NMW + NLW);
constexpr int OPB = 16384;              // bytes of one operand in a stage (256 x 32 bf16)
constexpr int STB = 2 * OPB;            // stage bytes (A then B)
constexpr int NLI = 4;                  // DMA instructions per operand per stage and load wave
constexpr int NLS = 2 * NLI;            // ... for both operands
constexpr int MI = 8, NJ = 4;           // accumulator subtiles per MFMA wave

enum : int { KC = 0, KO = 1 };

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// K-outer stage rows are 512 bytes (256 bf16); the 16-byte chunk of a row is
// xor-ed with a function of the K-row that gives the 16 rows one transpose
// read touches (8 g + j, g, j = 0..3) 16 different chunk positions.
__device__ __forceinline__ int xko(int k) { return (k & 3) | (((k >> 3) & 3) << 2); }

__device__ __forceinline__ i32x4 frag_kc(const uint8_t* op, int r0) {
  const int lane = threadIdx.x & 63;
  const int r = r0 + (lane & 15);
  return *reinterpret_cast<const i32x4*>(op + r * 64 + (((lane >> 4) ^ swz<64>(r)) << 4));
}

// The lane's constants for K-outer fragment reads.  Lane 16 g + c reads
// K-rows k0 = 8 g + c / 4 and k0 + 4, columns c0 + 4 (c % 4) .. + 3 of a
// 16-column subtile at c0 (a multiple of 16): byte (col % 8) * 2 = 8 (c % 2)
// of chunk col / 8 = c0 / 8 + (c % 4) / 2, stored at chunk position
// (col / 8) ^ xko(k0) (xko(k0 + 4) = xko(k0)); c0 / 8 is even, so that is
// (c0 / 8) ^ y with y = (c % 4) / 2 ^ xko(k0).
struct KoLane {
  int base;   // k0 * 512 + 8 (c % 2)
  int y;
};
__device__ __forceinline__ KoLane ko_lane() {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int k0 = 8 * g + (c >> 2);
  return {k0 * 512 + 8 * (c & 1), ((c & 3) >> 1) ^ xko(k0)};
}

__device__ __forceinline__ i32x4 frag_ko(const uint8_t* op, int c0, KoLane kl) {
  const uint8_t* p0 = op + kl.base + ((((c0 >> 3) ^ kl.y)) << 4);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(const_cast<uint8_t*>(p0)));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(const_cast<uint8_t*>(p0 + 4 * 512)));
  const i32x2 a = __builtin_bit_cast(i32x2, lo), b = __builtin_bit_cast(i32x2, hi);
  return i32x4{a.x, a.y, b.x, b.y};
}

// One operand's loads: a buffer resource over its valid bytes (reads past it
// return zeros), per-lane byte offsets of the lane's NLI 16-byte pieces at
// K-step 0, and the bytes one K-step advances.
struct Opnd {
  rsrc_t r;
  uint32_t off[NLI];
  uint32_t kstride;
};

// K-contiguous operand: tile row m at byte row_off(m) of the resource, its
// 32-K steps 64 bytes apart.
template <class F>
__device__ __forceinline__ Opnd opnd_kc(rsrc_t r, F row_off) {
  Opnd o;
  o.r = r;
  const int w = wave_id() - NMW, lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < NLI; ++q) {
    const int row = 16 * (w + NLW * q) + lane / 4;
    o.off[q] = row_off(row) + (((lane & 3) ^ swz<64>(row)) << 4);
  }
  o.kstride = 64;
  return o;
}

// K-outer operand: K-row k at byte k * ld, the tile's columns from col0; a
// K-step is 32 rows.
__device__ __forceinline__ Opnd opnd_ko(rsrc_t r, uint32_t ld, int col0) {
  Opnd o;
  o.r = r;
  const int w = wave_id() - NMW, lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < NLI; ++q) {
    const int k = 2 * (w + NLW * q) + lane / 32;
    o.off[q] = k * ld + col0 * 2 + (((lane & 31) ^ xko(k)) << 4);
  }
  o.kstride = 32 * ld;
  return o;
}

__device__ __forceinline__ void issue_stage(const Opnd& a, const Opnd& b, uint8_t* st, int ks) {
  const int w = wave_id() - NMW;
#pragma unroll
  for (int q = 0; q < NLI; ++q) {
    dma16(a.r, a.off[q], ks * a.kstride, st + 1024 * (w + NLW * q));
    dma16(b.r, b.off[q], ks * b.kstride, st + OPB + 1024 * (w + NLW * q));
  }
}

// acc[i][j][r] = C[16 (2 i + wm) + lane % 16][64 wn + 16 j + 4 (lane / 16) + r]
// summed over K-steps 0 .. nk-1 (A: the M side, B: the N side).  Returns on
// every wave; one barrier per K-step keeps the roles in step:
//   before barrier ks  stages ks and ks+1 have landed (the load waves waited
//                      for them);
//   after barrier ks   nobody reads stage ks-1 any more, and the load waves
//                      refill its buffers.
// So the MFMA waves read the next stage's first fragments (its weight side
// and first activation subtile) at the end of a stage, and within a stage
// read each activation fragment one subtile ahead of its MFMAs: no LDS read
// latency stands between a barrier and the first MFMA.
//
// The Dgrad K loop (A K-contiguous, B K-outer) with the A loads paired: a
// K-contiguous row moves 64 bytes per K-step, half a 128-byte line, and two
// halves requested a K-step apart cost an L2 request each, while requested
// back to back they merge into one (B's K-rows are whole lines already).  So
// A is loaded two K-steps at a time into a ring of 3 pair buffers (32 KB),
// B one K-step at a time into a ring of 4 (16 KB): 160 KB in all.  After
// barrier ks the load waves refill B's buffer of stage ks - 1 with
// stage ks + 3 and, for even ks, A's buffer of the pair (ks - 2, ks - 1) with
// the pair (ks + 4, ks + 5).  Loads complete in order, so the wait for stage
// ks + 2 allows exactly the loads issued after it: this step's B and, for an
// even ks (or the step before, for an odd one), the next A pair.
constexpr int PA_A = 0, PA_B = 3 * 2 * OPB;   // A pair buffers, then B buffers
static_assert(PA_B + 4 * OPB <= NSTG * STB, "paired ring fits the stage ring");

__device__ __forceinline__ void issue_a_pair(const Opnd& a, uint8_t* ring, int p, int nk) {
  const int w = wave_id() - NMW;
  uint8_t* st = ring + PA_A + (p % 3) * 2 * OPB;
  const int k0 = 2 * p, k1 = min(2 * p + 1, nk - 1);   // past the end: a clamped load nobody reads
#pragma unroll
  for (int q = 0; q < NLI; ++q) {
    dma16(a.r, a.off[q], k0 * a.kstride, st + 1024 * (w + NLW * q));
    dma16(a.r, a.off[q], k1 * a.kstride, st + OPB + 1024 * (w + NLW * q));
  }
}

__device__ __forceinline__ void issue_b(const Opnd& b, uint8_t* ring, int s) {
  const int w = wave_id() - NMW;
#pragma unroll
  for (int q = 0; q < NLI; ++q) dma16(b.r, b.off[q], s * b.kstride, ring + PA_B + (s % 4) * OPB + 1024 * (w + NLW * q));
}

__device__ __forceinline__ const uint8_t* pa_a(uint8_t* ring, int s) {
  return ring + PA_A + ((s / 2) % 3) * 2 * OPB + (s % 2) * OPB;
}
__device__ __forceinline__ const uint8_t* pa_b(uint8_t* ring, int s) { return ring + PA_B + (s % 4) * OPB; }

template <int NSUB = MI>
__device__ __forceinline__ void mainloop_pa(uint8_t* ring, const Opnd& a, const Opnd& b, int nk,
                                            f32x4 (&acc)[MI][NJ]) {
  static_assert(NSUB >= 1 && NSUB <= MI, "row subtiles");
  const int w = wave_id();
  if (nk <= 0) return;
  if (w >= NMW) {
    // A pair 0, B 0, B 1, A pair 1, B 2: stages 0 and 1 first
    issue_a_pair(a, ring, 0, nk);
    issue_b(b, ring, 0);
    if (nk > 1) issue_b(b, ring, 1);
    if (nk > 2) {
      issue_a_pair(a, ring, 1, nk);
      issue_b(b, ring, 2);
      wait_vm_lgkm0<3 * NLI>();   // A pair 1 and B 2 may be in flight
    } else {
      wait_vm_lgkm0<0>();
    }
    for (int ks = 0; ks < nk; ++ks) {
      block_barrier();
      const bool ib = ks + 3 < nk;
      if (ib) issue_b(b, ring, ks + 3);
      if ((ks & 1) == 0) {
        const bool ia = ks + 4 < nk;
        if (ia) issue_a_pair(a, ring, ks / 2 + 2, nk);
        if (ia)
          wait_vm_lgkm0<3 * NLI>();   // stage ks + 2; this step's B and A pair in flight
        else if (ib)
          wait_vm_lgkm0<NLI>();       // this step's B in flight
        else
          wait_vm_lgkm0<0>();
      } else {
        if (ib)
          wait_vm_lgkm0<3 * NLI>();   // the previous step's A pair and this step's B in flight
        else
          wait_vm_lgkm0<0>();
      }
    }
    return;
  }
  const int wm = w % 2, wn = w / 2;
  KoLane kl = ko_lane();
  i32x4 wf[NJ], xf;
  block_barrier();   // stages 0 and 1 have landed
  {
#pragma unroll
    for (int j = 0; j < NJ; ++j) wf[j] = frag_ko(pa_b(ring, 0), 64 * wn + 16 * j, kl);
    xf = frag_kc(pa_a(ring, 0), 16 * wm);
  }
  acc_fence(acc);
  for (int ks = 0; ks < nk; ++ks) {
    asm volatile("" : "+v"(kl.base), "+v"(kl.y));
    const uint8_t* sa = pa_a(ring, ks);
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      i32x4 xn;
      if (i + 1 < NSUB) xn = frag_kc(sa, 16 * (2 * (i + 1) + wm));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) mfma_bf16_tied(acc[i][j], wf[j], xf);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < NSUB) xf = xn;
    }
    if (ks + 1 < nk) {
      const uint8_t* nb = pa_b(ring, ks + 1);
#pragma unroll
      for (int j = 0; j < NJ; ++j) wf[j] = frag_ko(nb, 64 * wn + 16 * j, kl);
      xf = frag_kc(pa_a(ring, ks + 1), 16 * wm);
      block_barrier();
    }
  }
  acc_fence(acc);
}

// f.template operator()<NSUB>() with NSUB = the row subtiles wave row 0
// computes for a tile of `rows` rows (two wave rows of 16-row subtiles).
template <int N = 1, class F>
__device__ __forceinline__ void with_row_subtiles(int rows, F&& f) {
  if constexpr (N >= MI)
    f.template operator()<MI>();
  else if (rows <= 32 * N)
    f.template operator()<N>();
  else
    with_row_subtiles<N + 1>(rows, f);
}

__device__ __forceinline__ uint2 pack4(const f32x4& v) { return make_uint2(bf16x2(v[0], v[1]), bf16x2(v[2], v[3])); }

__device__ __forceinline__ void unpack4(uint2 p, float (&v)[4]) {
  v[0] = bf16_to_f32(static_cast<uint16_t>(p.x & 0xffffu));
  v[1] = bf16_to_f32(static_cast<uint16_t>(p.x >> 16));
  v[2] = bf16_to_f32(static_cast<uint16_t>(p.y & 0xffffu));
  v[3] = bf16_to_f32(static_cast<uint16_t>(p.y >> 16));
}

__device__ __forceinline__ float sigmoid_ref(float z) { return 1.0f / (1.0f + expf(-z)); }

// ------------------------------------------------------------------ Dgrad

// Group g's row range: routed expert g (g < N_r) or shared expert g - N_r.
struct GroupRows {
  int first, count;
};

// Dgrad tiles: (m-tile of the forward's list, n-block), laid out over the
// XCDs as the forward GEMMs lay out theirs (the list's per-XCD segments; the
// m-tiles of a unit, which read the same weight columns, back to back).
__device__ __forceinline__ bool dgrad_tile(const BwdArgs& a, int nb_n, int& row0, int& rows, int& g, int& n0) {
  const int q = xcd_tile(a.mt_count, nb_n);
  if (q < 0) return false;
  int mt, nb, in_unit;
  tile_coords(a.mtiles, q, nb_n, mt, nb, in_unit);
  if (!MOE_CHECK(mt >= 0 && mt < a.mt_count[0] && nb < nb_n, 501)) return false;
  const int4 t = a.mtiles[mt];
  g = t.x;
  row0 = t.y;
  rows = t.z;
  n0 = nb * BT;
  return MOE_CHECK(g >= 0 && g < a.n_routed + a.n_shared && rows >= 1 && rows <= BT && row0 >= 0 &&
                       row0 + rows <= a.R, 502);
}

// dH = dY W_down for the tile's rows, then the SwiGLU backward from the
// cached G and U: dG, dU (into dgu) and the recomputed H (into hr).
__global__ __launch_bounds__(THREADS, 1) void dgrad_down_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NSTG * STB];
  int row0, rows, g, n0;
  if (!dgrad_tile(a, ceil_div(a.inter, BT), row0, rows, g, n0)) return;
  const bool shared = g >= a.n_routed;
  const int gs = shared ? g - a.n_routed : g;
  const uint32_t ldy = a.d * 2, ldw = a.inter * 2;
  const uint8_t* wd = static_cast<const uint8_t*>(shared ? a.ws_down : a.w_down) + static_cast<size_t>(gs) * a.d * ldw;
  f32x4 acc[MI][NJ];
  zero_acc(acc);
  if (wave_id() >= NMW) {
    const Opnd oa = opnd_kc(make_rsrc(reinterpret_cast<const uint8_t*>(a.dys) + static_cast<size_t>(row0) * ldy,
                                      rows * ldy),
                            [&](int m) { return static_cast<uint32_t>((m < rows ? m : rows) * ldy); });   // past the rows: zeros
    const Opnd ob = opnd_ko(make_rsrc(wd, a.d * ldw), ldw, n0);
    mainloop_pa(ring, oa, ob, a.d / 32, acc);
    return;
  }
  with_row_subtiles(rows, [&]<int NS>() { mainloop_pa<NS>(ring, Opnd{}, Opnd{}, a.d / 32, acc); });
  const int w = wave_id(), lane = threadIdx.x & 63, wm = w % 2, wn = w / 2;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int row = 16 * (2 * i + wm) + (lane & 15);
    if (row >= rows) continue;
    const size_t r = static_cast<size_t>(row0 + row);
    const uint16_t* gu = a.gu + r * 2 * a.inter;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = n0 + 64 * wn + 16 * j + 4 * (lane >> 4);
      if (col >= a.inter) continue;
      float G[4], U[4], dG[4], dU[4], H[4];
      unpack4(*reinterpret_cast<const uint2*>(gu + col), G);
      unpack4(*reinterpret_cast<const uint2*>(gu + a.inter + col), U);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sg = sigmoid_ref(G[e]);
        const float silu = G[e] * sg;
        dG[e] = acc[i][j][e] * U[e] * (sg * (1.0f + G[e] * (1.0f - sg)));
        dU[e] = acc[i][j][e] * silu;
        H[e] = silu * U[e];
      }
      uint16_t* dgu = a.dgu + r * 2 * a.inter;
      *reinterpret_cast<uint2*>(dgu + col) = make_uint2(bf16x2(dG[0], dG[1]), bf16x2(dG[2], dG[3]));
      *reinterpret_cast<uint2*>(dgu + a.inter + col) = make_uint2(bf16x2(dU[0], dU[1]), bf16x2(dU[2], dU[3]));
      *reinterpret_cast<uint2*>(a.hr + r * a.inter + col) = make_uint2(bf16x2(H[0], H[1]), bf16x2(H[2], H[3]));
    }
  }
}

// dX = [dG dU] W_gate_up for the tile's rows (bf16 rows of dx).
__global__ __launch_bounds__(THREADS, 1) void dgrad_gateup_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NSTG * STB];
  int row0, rows, g, n0;
  if (!dgrad_tile(a, ceil_div(a.d, BT), row0, rows, g, n0)) return;
  const bool shared = g >= a.n_routed;
  const int gs = shared ? g - a.n_routed : g;
  const uint32_t ldg = a.inter * 4, ldw = a.d * 2;
  const uint8_t* wgu =
      static_cast<const uint8_t*>(shared ? a.ws_gate_up : a.w_gate_up) + static_cast<size_t>(gs) * 2 * a.inter * ldw;
  f32x4 acc[MI][NJ];
  zero_acc(acc);
  const int nk = 2 * a.inter / 32;
  if (wave_id() >= NMW) {
    const Opnd oa = opnd_kc(make_rsrc(reinterpret_cast<const uint8_t*>(a.dgu) + static_cast<size_t>(row0) * ldg,
                                      rows * ldg),
                            [&](int m) { return static_cast<uint32_t>((m < rows ? m : rows) * ldg); });   // past the rows: zeros
    const Opnd ob = opnd_ko(make_rsrc(wgu, 2 * a.inter * ldw), ldw, n0);
    mainloop_pa(ring, oa, ob, nk, acc);
    return;
  }
  with_row_subtiles(rows, [&]<int NS>() { mainloop_pa<NS>(ring, Opnd{}, Opnd{}, nk, acc); });
  const int w = wave_id(), lane = threadIdx.x & 63, wm = w % 2, wn = w / 2;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int row = 16 * (2 * i + wm) + (lane & 15);
    if (row >= rows) continue;
    uint16_t* dst = a.dx + static_cast<size_t>(row0 + row) * a.d;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = n0 + 64 * wn + 16 * j + 4 * (lane >> 4);
      if (col < a.d) *reinterpret_cast<uint2*>(dst + col) = pack4(acc[i][j]);
    }
  }
}

// ------------------------------------------------------------------ Wgrad

__device__ __forceinline__ GroupRows group_rows(const BwdArgs& a, int g) {
  if (g < a.n_routed) return {a.offsets[g], a.counts[g]};
  return {static_cast<int>(a.TK + static_cast<long long>(g - a.n_routed) * a.T), a.T};
}

// Wgrad tiles: per group, m-blocks x n-blocks (the n-block fastest), groups
// in order.  The routed groups' tiles are cut into NXCD contiguous chunks,
// one per XCD, so a group's tiles (which read its rows) share one L2; the
// shared groups' tiles, whose K runs over all T tokens, follow in chunks of
// their own, so every XCD gets an equal share of them too.  XCD x's list:
// its routed chunk, then its shared chunk.
//
// The kernel is persistent: P blocks per XCD (one per CU), block l of XCD x
// taking positions l, l + P, l + 2P, ... of x's list, so the tiles running
// at once on an XCD are neighbours in it.  A block's K-steps over all its
// tiles form one stream of stages: the load waves run on into the next
// tile's first stages while the MFMA waves store the finished tile's fp32
// gradients (a routed tile has only ~8 K-steps, and its 256 KB of stores
// would otherwise stall the CU).
struct WgradList {
  long long per_g, nr_t, cr, cs, r0, nr, s0, len;
  int l, P;

  __device__ WgradList(const BwdArgs& a, long long per_group) {
    per_g = per_group;
    nr_t = a.n_routed * per_g;
    const long long ns_t = a.n_shared * per_g;
    cr = (nr_t + NXCD - 1) / NXCD;
    cs = (ns_t + NXCD - 1) / NXCD;
    P = gridDim.x / NXCD;
    const int x = blockIdx.x % NXCD;
    l = blockIdx.x / NXCD;
    r0 = x * cr;
    nr = max(0LL, min(r0 + cr, nr_t) - r0);
    s0 = x * cs;
    const long long ns = max(0LL, min(s0 + cs, ns_t) - s0);
    len = nr + ns;
  }
  // tiles of this block
  __device__ long long count() const { return l < len ? (len - l + P - 1) / P : 0; }
  // the tile (index in the whole tile sequence) of this block's i-th tile
  __device__ long long tile(long long i) const {
    const long long p = l + i * P;
    return p < nr ? r0 + p : nr_t + s0 + (p - nr);
  }
};

// A group's tile rem -> (m-block, n-block): with RUN = 0, n-block fastest;
// else the n-blocks in runs of RUN, each run walked m-block by m-block (n
// fastest within the run).  Measured at d = 7168: the down Wgrad runs 9%
// (bf16, 28 x 8 blocks) and 11% (FP8, 28 x 16) faster in runs of 4; the
// gate/up Wgrad (16 x 28, 16 x 56) is fastest n-fastest (runs of 4 or 8:
// 1-11% slower).
template <int RUN>
__device__ __forceinline__ void wgrad_mn(int rem, int mb_n, int nb_n, int& mb, int& nb) {
  if (RUN == 0 || nb_n <= RUN) {
    mb = rem / nb_n;
    nb = rem % nb_n;
    return;
  }
  const int run = RUN * mb_n, r = rem / run, x = rem - r * run;
  const int w = min(RUN, nb_n - r * RUN);
  mb = x / w;
  nb = r * RUN + x % w;
}

inline int wgrad_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus < NXCD)
    cus = 256;
  return cus / NXCD * NXCD;
}

// A group's rows, checked against the grouped rows (debug build: a group out
// of range counts as empty, the same for every caller).
__device__ __forceinline__ GroupRows checked_rows(const BwdArgs& a, int g) {
  GroupRows gr = group_rows(a, g);
  if (!MOE_CHECK(gr.first >= 0 && gr.count >= 0 && gr.first + static_cast<long long>(gr.count) <= a.R, 504))
    gr = {0, 0};
  return gr;
}

// The rows of the group of a tile, cached: a block's consecutive tiles mostly
// share a group.
struct GroupCache {
  int g = -1;
  GroupRows gr{0, 0};
  __device__ const GroupRows& get(const BwdArgs& a, int g_new) {
    if (g_new != g) {
      g = g_new;
      gr = checked_rows(a, g);
    }
    return gr;
  }
};

// C[m][n] = sum over the group's rows r of A[r][m] B[r][n], both K-outer
// (rows r of M and N bf16), written as fp32 into the group's gradient.
template <int RUN>
__device__ __forceinline__ void wgrad_persistent(const BwdArgs& a, const uint16_t* A, int M, const uint16_t* B,
                                                 int N, float* routed_dst, float* shared_dst) {
  // 4 stage buffers, then 4 KB of store staging per MFMA wave (160 KB in all)
  constexpr int WN = 4;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[WN * STB + NMW * 4096];
  const int mb_n = ceil_div(M, BT), nb_n = ceil_div(N, BT);
  const long long per_g = static_cast<long long>(mb_n) * nb_n;
  const WgradList list(a, per_g);
  const long long ntiles = list.count();
  const uint32_t lda = M * 2, ldb = N * 2;
  const int w = wave_id(), lane = threadIdx.x & 63;

  // stages of the block's stream: the sum of its tiles' K-steps (lanes over tiles)
  long long total = 0;
  for (long long i = lane; i < ntiles; i += 64) {
    const int g = static_cast<int>(list.tile(i) / per_g);
    const GroupRows gr = checked_rows(a, g);
    total += gr.count > 0 ? ceil_div(gr.count, 32) : 0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) total += __shfl_xor(total, off);
  // the same in every lane: say so, so that the loops over it stay scalar
  total = static_cast<long long>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(total)))) |
          static_cast<long long>(__builtin_amdgcn_readfirstlane(static_cast<int>(total >> 32))) << 32;

  GroupCache gc;
  if (w >= NMW) {
    // ---- load waves: issue the stream WN - 1 stages ahead of the MFMAs
    long long it = -1;        // tile of the next stage to issue
    int ks = 0, nk = 0;       // that stage's K-step within it, and its K-steps
    Opnd oa{}, ob{};
    long long issued = 0;
    auto issue_next = [&]() {
      while (ks >= nk) {      // on to the next tile with rows
        ++it;
        const long long q = list.tile(it);
        const int g = static_cast<int>(q / per_g);
        const int rem = static_cast<int>(q - static_cast<long long>(g) * per_g);
        const GroupRows& gr = gc.get(a, g);
        nk = gr.count > 0 ? ceil_div(gr.count, 32) : 0;
        ks = 0;
        int mb, nb;
        wgrad_mn<RUN>(rem, mb_n, nb_n, mb, nb);
        oa = opnd_ko(make_rsrc(reinterpret_cast<const uint8_t*>(A) + static_cast<size_t>(gr.first) * lda,
                               gr.count * lda), lda, mb * BT);
        ob = opnd_ko(make_rsrc(reinterpret_cast<const uint8_t*>(B) + static_cast<size_t>(gr.first) * ldb,
                               gr.count * ldb), ldb, nb * BT);
      }
      issue_stage(oa, ob, ring + (issued % WN) * STB, ks);
      ++ks;
      ++issued;
    };
    const long long pre = min(total, static_cast<long long>(WN - 1));
    for (long long s = 0; s < pre; ++s) issue_next();
    if (pre == WN - 1)
      wait_vm_lgkm0<(WN - 3) * NLS>();   // stages 0 and 1
    else
      wait_vm_lgkm0<0>();
    for (long long S = 0; S < total; ++S) {
      block_barrier();
      if (S + WN - 1 < total) {
        issue_next();
        wait_vm_lgkm0<(WN - 3) * NLS>();   // stage S + 2
      } else {
        wait_vm_lgkm0<0>();
      }
    }
    return;
  }

  // ---- MFMA waves
  const int wm = w % 2, wn = w / 2;
  KoLane kl = ko_lane();
  f32x4 acc[MI][NJ];
  i32x4 wf[NJ], xf;
  long long S = 0;   // the next stage of the stream
  if (total > 0) block_barrier();   // #0: stages 0 and 1 have landed
  for (long long i = 0; i < ntiles; ++i) {
    const long long q = list.tile(i);
    const int g = static_cast<int>(q / per_g);
    const int rem = static_cast<int>(q - static_cast<long long>(g) * per_g);
    int mb, nb;
    wgrad_mn<RUN>(rem, mb_n, nb_n, mb, nb);
    const int m0 = mb * BT, n0 = nb * BT;
    const GroupRows& gr = gc.get(a, g);
    const int nk = gr.count > 0 ? ceil_div(gr.count, 32) : 0;
    zero_acc(acc);
    if (nk > 0) {
      {   // the tile's first stage (landed: this wave passed barrier #S)
        const uint8_t* st = ring + (S % WN) * STB;
#pragma unroll
        for (int j = 0; j < NJ; ++j) wf[j] = frag_ko(st + OPB, 64 * wn + 16 * j, kl);
        xf = frag_ko(st, 16 * wm, kl);
      }
      acc_fence(acc);
      for (int k = 0; k < nk; ++k) {
        asm volatile("" : "+v"(kl.base), "+v"(kl.y));
        const uint8_t* sa = ring + (S % WN) * STB;
        const uint8_t* na = ring + ((S + 1) % WN) * STB;
#pragma unroll
        for (int ii = 0; ii < MI; ++ii) {
          i32x4 xn;
          if (ii + 1 < MI) xn = frag_ko(sa, 16 * (2 * (ii + 1) + wm), kl);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < NJ; ++j) mfma_bf16_tied(acc[ii][j], wf[j], xf);
          __builtin_amdgcn_sched_barrier(0);
          if (ii + 1 < MI) xf = xn;
        }
        ++S;
        if (k + 1 < nk) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) wf[j] = frag_ko(na + OPB, 64 * wn + 16 * j, kl);
          xf = frag_ko(na, 16 * wm, kl);
          block_barrier();
        } else if (S < total) {
          block_barrier();   // the load waves go on into the next tile during the stores below
        }
      }
      acc_fence(acc);
    }
    float* dst = g < a.n_routed ? routed_dst + static_cast<size_t>(g) * M * N
                                : shared_dst + static_cast<size_t>(g - a.n_routed) * M * N;
    {
      // each 16-row subtile through the wave's 4 KB of staging: written as
      // the accumulators hold it (row lane & 15, 16-byte chunks 4 j + lane >> 4,
      // chunk positions xor-ed with the row), read back 4 rows x 256 bytes per
      // store instruction, so every store writes whole 128-byte lines, and
      // streamed past the caches (non-temporal): the gradient is not read
      // again here, and the group's operand rows stay in L2 for its other
      // tiles.  (64-byte pieces straight from the accumulators left the two
      // halves of each line to merge in L2, which the operands then lost.)
      uint8_t* sg = ring + WN * STB + 4096 * w;
      const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
      for (int ii = 0; ii < MI; ++ii) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          *reinterpret_cast<f32x4*>(sg + lr * 256 + (((4 * j + lg) ^ lr) << 4)) = acc[ii][j];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = 4 * q + (lane >> 4), c = lane & 15;
          const f32x4 v = *reinterpret_cast<const f32x4*>(sg + rr * 256 + ((c ^ rr) << 4));
          const int m = m0 + 16 * (2 * ii + wm) + rr, n = n0 + 64 * wn + 4 * c;
          if (m < M && n < N) {
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst + static_cast<size_t>(m) * N + n));
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  }
}

// dW_down[c][i] = sum_r dY[r][c] H[r][i]
__global__ __launch_bounds__(THREADS, 1) void wgrad_down_kernel(BwdArgs a) {
  wgrad_persistent<4>(a, a.dys, a.d, a.hr, a.inter, a.dw_down, a.dws_down);
}

// dW_gate_up[j][c] = sum_r [dG dU][r][j] X[r][c]
__global__ __launch_bounds__(THREADS, 1) void wgrad_gateup_kernel(BwdArgs a) {
  wgrad_persistent<0>(a, a.dgu, 2 * a.inter, a.xp, a.d, a.dw_gate_up, a.dws_gate_up);
}

// ------------------------------------------------------------------ FP8 backward
//
// Every GEMM of the backward takes E4M3 operands with fp32 scales per group
// of 128 along its inner dimension.  Dgrad: the 1x128 codes of dY (then of
// [dG dU]) times the weights' codes read transposed ([N][K] arrays with the
// same 128x128 blocks) -- the forward's FP8 row-times-weight GEMM.  Wgrad:
// both operands tiled 128x1 along the grouped rows, stored transposed
// ([channel][kt], group g's blocks from column koff_g) so that the GEMM reads
// them K-contiguous; each 16x16x128 product is promoted into the fp32
// accumulators with the row scale of A times the lane's four column scales
// of B.

__device__ __forceinline__ long long koff_of(const BwdArgs& a, int g, const GroupRows& gr) {
  return 128LL * (gr.first / 128 + 2LL * g);
}

// SwiGLU backward on the bf16 Dgrad output dH (in hr): dG = dH U SiLU'(G),
// dU = dH SiLU(G) into dgu, H = SiLU(G) U into hr (in place).  8 columns per
// thread.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(BwdArgs a) {
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = a.inter / 8;
  const long long r = idx / per_row;
  if (r >= a.R) return;
  const int c = static_cast<int>(idx - r * per_row) * 8;
  const uint16_t* gu = a.gu + r * 2 * a.inter;
  const uint4 dh = *reinterpret_cast<const uint4*>(a.hr + r * a.inter + c);
  const uint4 gv = *reinterpret_cast<const uint4*>(gu + c);
  const uint4 uv = *reinterpret_cast<const uint4*>(gu + a.inter + c);
  const uint32_t dw[4] = {dh.x, dh.y, dh.z, dh.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
  uint32_t og[4], ou[4], oh[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float dG[2], dU[2], H[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float d = bf16_to_f32(static_cast<uint16_t>(dw[q] >> (16 * h)));
      const float G = bf16_to_f32(static_cast<uint16_t>(gw[q] >> (16 * h)));
      const float U = bf16_to_f32(static_cast<uint16_t>(uw[q] >> (16 * h)));
      const float sg = sigmoid_ref(G);
      const float silu = G * sg;
      dG[h] = d * U * (sg * (1.0f + G * (1.0f - sg)));
      dU[h] = d * silu;
      H[h] = silu * U;
    }
    og[q] = bf16x2(dG[0], dG[1]);
    ou[q] = bf16x2(dU[0], dU[1]);
    oh[q] = bf16x2(H[0], H[1]);
  }
  uint16_t* dgu = a.dgu + r * 2 * a.inter;
  *reinterpret_cast<uint4*>(dgu + c) = make_uint4(og[0], og[1], og[2], og[3]);
  *reinterpret_cast<uint4*>(dgu + a.inter + c) = make_uint4(ou[0], ou[1], ou[2], ou[3]);
  *reinterpret_cast<uint4*>(a.hr + r * a.inter + c) = make_uint4(oh[0], oh[1], oh[2], oh[3]);
}

// The group of 128-row block kb of the transposed code arrays (-1: a gap):
// the last group whose koff is at most 128 kb, if kb falls in its blocks.
__device__ __forceinline__ int group_of_block(const BwdArgs& a, long long kb, GroupRows& gr, int& b) {
  int lo = 0, hi = a.n_routed + a.n_shared - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (koff_of(a, mid, group_rows(a, mid)) <= 128 * kb) lo = mid; else hi = mid - 1;
  }
  gr = checked_rows(a, lo);
  const long long k0 = koff_of(a, lo, gr) / 128;
  if (kb < k0 || kb >= k0 + ceil_div(gr.count, 128)) return -1;
  b = static_cast<int>(kb - k0);
  return lo;
}

// 128x1 quantiser, transposed output: block (kb, column range) takes rows
// 128 b .. 128 b + 127 of one group (b: kb's block in it; rows past the group
// are zero) and up to CQ_CHUNKS chunks of 64 columns of src [R][C] bf16 (with
// by_token, src is [T][C] and grouped row r reads the row of its token); per
// column, scale = amax / 448 and codes of x * (448 / amax) (scale 1, zero
// codes for an all-zero tile) into dst[c][128 kb ..] and dst_s[c][kb].  The
// block finds its group once, and loads the next chunk while it quantises
// the current one.
constexpr int CQ_CHUNKS = 8;
__global__ __launch_bounds__(256) void colquant_kernel(BwdArgs a, const uint16_t* __restrict__ src, int C,
                                                       bool by_token, uint8_t* __restrict__ dst,
                                                       float* __restrict__ dst_s) {
  __shared__ float tile[128][65];
  GroupRows gr;
  int b;
  const long long kb = blockIdx.x;
  if (group_of_block(a, kb, gr, b) < 0) return;
  const int t = threadIdx.x;
  const int r0 = gr.first + 128 * b, nr = min(128, gr.count - 128 * b);
  const int ch0 = blockIdx.y * CQ_CHUNKS, nch = min(CQ_CHUNKS, C / 64 - ch0);
  // thread t loads 32 columns (4 x 16 bytes) of row t / 2 of a chunk
  const int rr = t >> 1, cc = (t & 1) * 32;
  long long row = r0 + (rr < nr ? rr : 0);
  if (by_token) row = row < a.TK ? a.perm_token[row] : (row - a.TK) % a.T;
  const uint16_t* srow = src + static_cast<size_t>(row) * C + cc;
  uint4 v[4];
  auto load = [&](int ch) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = rr < nr ? *reinterpret_cast<const uint4*>(srow + 64 * ch + 8 * q) : make_uint4(0, 0, 0, 0);
  };
  load(ch0);
  // wave w takes columns 16 w .. 16 w + 15, two at a time: lane 8 c + k holds
  // rows 16 k .. 16 k + 15 of column 16 w + c (then + 8), so the eight lanes
  // of a column reduce its amax among themselves and one store instruction
  // writes 8 columns x 128 bytes, whole lines
  const int w = t >> 6, lane = t & 63, k = lane & 7;
  for (int i = 0; i < nch; ++i) {
    const int c0 = 64 * (ch0 + i);
    if (i > 0) __syncthreads();   // the previous chunk's tile reads are done
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t wd[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tile[rr][cc + 8 * q + 2 * e] = bf16_to_f32(static_cast<uint16_t>(wd[e] & 0xffffu));
        tile[rr][cc + 8 * q + 2 * e + 1] = bf16_to_f32(static_cast<uint16_t>(wd[e] >> 16));
      }
    }
    if (i + 1 < nch) load(ch0 + i + 1);
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 16 * w + 8 * h + (lane >> 3);
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(tile[16 * k + j][c]));
      m = fmaxf(m, __shfl_xor(m, 1));
      m = fmaxf(m, __shfl_xor(m, 2));
      m = fmaxf(m, __shfl_xor(m, 4));
      const float sc = m == 0.f ? 1.f : m / 448.f;
      const float inv = m == 0.f ? 0.f : 448.f / m;
      uint32_t wq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * k + 4 * j;
        wq[j] = e4m3x4(tile[r][c] * inv, tile[r + 1][c] * inv, tile[r + 2][c] * inv, tile[r + 3][c] * inv);
      }
      *reinterpret_cast<uint4*>(dst + static_cast<size_t>(c0 + c) * a.kt + 128 * kb + 16 * k) =
          make_uint4(wq[0], wq[1], wq[2], wq[3]);
      if (k == 0) dst_s[static_cast<size_t>(c0 + c) * (a.kt / 128) + kb] = sc;
    }
  }
}

// FP8 Wgrad tiles: 256 rows of A (M) x 128 rows of B (N), 8 MFMA waves (2 x
// 4: 128 x 32 each) and 4 load waves; a stage is one 128-row block of the
// group (K): A codes, B codes, A row scales, B row scales.
constexpr int W8_BM = 256, W8_BN = 128;
constexpr int W8_NSTG = 3;
constexpr int W8_A = 0, W8_B = 32768, W8_AS = 49152, W8_BS = 50176;
constexpr int W8_STB = 51200;
constexpr int W8_NL = 8 + 4 + 2;   // DMA ops per load wave per stage
static_assert(W8_NSTG * W8_STB + NMW * 1024 <= 160 * 1024, "ring and store staging fit the LDS");

struct Opnd8 {
  rsrc_t ra, rb, rsa, rsb;
  uint32_t oa[8], ob[4];
  uint32_t osa, osb;
};

// A lane's byte offsets in a 16-row subtile of 128-byte rows: row lane & 15,
// the two 16-byte chunks of K 32 (lane >> 4) .. + 31 (the swizzle depends on
// the row modulo 16 only, so they serve every subtile).
struct Lane8 {
  int lo, hi;
};
__device__ __forceinline__ Lane8 lane8() {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  return {lr * 128 + (((2 * lg) ^ swz<128>(lr)) << 4), lr * 128 + (((2 * lg + 1) ^ swz<128>(lr)) << 4)};
}

// The 32-byte fragment of the 16-row subtile at `sub` (a multiple of 16 rows).
__device__ __forceinline__ i32x8 frag8(const uint8_t* base, int sub, Lane8 l) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(base + sub * 128 + l.lo);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(base + sub * 128 + l.hi);
  return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// The load waves' operands for a tile of group g (its rows gr) at (m0, n0):
// A = qa rows m0.., B = qb rows n0.., from column koff_g; rows past M or N
// read past their resource (zeros).
__device__ __forceinline__ Opnd8 opnd8(const BwdArgs& a, const uint8_t* A, const float* As, int M, const uint8_t* B,
                                       const float* Bs, int N, long long koff, int m0, int n0) {
  const int w = wave_id() - NMW, lane = threadIdx.x & 63;
  const long long kt = a.kt, kbt = a.kt / 128, kb0 = koff / 128;
  Opnd8 o;
  o.ra = make_rsrc(A + koff, static_cast<uint32_t>(M * kt - koff));
  o.rb = make_rsrc(B + koff, static_cast<uint32_t>(N * kt - koff));
  o.rsa = make_rsrc(As + kb0, static_cast<uint32_t>((M * kbt - kb0) * 4));
  o.rsb = make_rsrc(Bs + kb0, static_cast<uint32_t>((N * kbt - kb0) * 4));
  const uint32_t far = 0x7ff00000u;   // past every resource: zeros
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = 8 * (w + NLW * q) + lane / 8;
    o.oa[q] = m0 + r < M ? static_cast<uint32_t>((m0 + r) * kt) + (((lane & 7) ^ swz<128>(r)) << 4) : far;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 8 * (w + NLW * q) + lane / 8;
    o.ob[q] = n0 + r < N ? static_cast<uint32_t>((n0 + r) * kt) + (((lane & 7) ^ swz<128>(r)) << 4) : far;
  }
  const int ra = 64 * w + lane, rb = (64 * w + lane) & (W8_BN - 1);
  o.osa = m0 + ra < M ? static_cast<uint32_t>((m0 + ra) * kbt * 4) : far;
  o.osb = n0 + rb < N ? static_cast<uint32_t>((n0 + rb) * kbt * 4) : far;
  return o;
}

__device__ __forceinline__ void issue8(const Opnd8& o, uint8_t* st, int ks) {
  const int w = wave_id() - NMW;
#pragma unroll
  for (int q = 0; q < 8; ++q) dma16(o.ra, o.oa[q], ks * 128, st + W8_A + 1024 * (w + NLW * q));
#pragma unroll
  for (int q = 0; q < 4; ++q) dma16(o.rb, o.ob[q], ks * 128, st + W8_B + 1024 * (w + NLW * q));
  dma4(o.rsa, o.osa, ks * 4, st + W8_AS + 256 * w);
  dma4(o.rsb, o.osb, ks * 4, st + W8_BS + 256 * w);
}

// C[m][n] = sum over the group's rows r of A[r][m] B[r][n] from the 128x1
// codes (qa: [M][kt], qb: [N][kt]), fp32 into the group's gradient.  The
// persistent stream of the bf16 Wgrad: the load waves run into the next
// tile's blocks while the MFMA waves store; "stage S landed" before barrier
// #S, and barrier #S+1 frees stage S's buffer for stage S + 3.
template <int RUN>
__device__ __forceinline__ void wgrad8_persistent(const BwdArgs& a, const uint8_t* A, const float* As, int M,
                                                  const uint8_t* B, const float* Bs, int N, float* routed_dst,
                                                  float* shared_dst) {
  // the stage ring, then 1 KB of store staging per MFMA wave
  __shared__ __attribute__((aligned(1024))) uint8_t ring[W8_NSTG * W8_STB + NMW * 1024];
  const int mb_n = ceil_div(M, W8_BM), nb_n = ceil_div(N, W8_BN);
  const long long per_g = static_cast<long long>(mb_n) * nb_n;
  const WgradList list(a, per_g);
  const long long ntiles = list.count();
  const int w = wave_id(), lane = threadIdx.x & 63;

  long long total = 0;
  for (long long i = lane; i < ntiles; i += 64) {
    const GroupRows gr = checked_rows(a, static_cast<int>(list.tile(i) / per_g));
    total += gr.count > 0 ? ceil_div(gr.count, 128) : 0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) total += __shfl_xor(total, off);
  total = static_cast<long long>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(total)))) |
          static_cast<long long>(__builtin_amdgcn_readfirstlane(static_cast<int>(total >> 32))) << 32;

  GroupCache gc;
  if (w >= NMW) {
    long long it = -1;
    int ks = 0, nk = 0;
    Opnd8 o{};
    long long issued = 0;
    auto issue_next = [&]() {
      while (ks >= nk) {
        ++it;
        const long long q = list.tile(it);
        const int g = static_cast<int>(q / per_g);
        const int rem = static_cast<int>(q - static_cast<long long>(g) * per_g);
        const GroupRows& gr = gc.get(a, g);
        nk = gr.count > 0 ? ceil_div(gr.count, 128) : 0;
        ks = 0;
        int mb, nb;
        wgrad_mn<RUN>(rem, mb_n, nb_n, mb, nb);
        o = opnd8(a, A, As, M, B, Bs, N, koff_of(a, g, gr), mb * W8_BM, nb * W8_BN);
      }
      issue8(o, ring + (issued % W8_NSTG) * W8_STB, ks);
      ++ks;
      ++issued;
    };
    const long long pre = min(total, 2LL);
    for (long long s = 0; s < pre; ++s) issue_next();
    if (pre == 2)
      wait_vm_lgkm0<W8_NL>();   // stage 0
    else
      wait_vm_lgkm0<0>();
    if (total > 0) block_barrier();   // #0
    for (long long S = 0; S + 1 < total; ++S) {
      if (S + 2 < total) {
        issue_next();
        wait_vm_lgkm0<W8_NL>();   // stage S + 1
      } else {
        wait_vm_lgkm0<0>();
      }
      block_barrier();   // #S+1
    }
    return;
  }

  const int wm = w % 2, wn = w / 2, lr = lane & 15, lg = lane >> 4;
  Lane8 l8 = lane8();
  int lsa = lr * 4, lsb = 4 * lg * 4;   // the lane's A row scale and B column scales in a stage
  f32x4 acc[MI][2];
  long long S = 0;
  if (total > 0) block_barrier();   // #0
  for (long long i = 0; i < ntiles; ++i) {
    const long long q = list.tile(i);
    const int g = static_cast<int>(q / per_g);
    const int rem = static_cast<int>(q - static_cast<long long>(g) * per_g);
    int mb, nb;
    wgrad_mn<RUN>(rem, mb_n, nb_n, mb, nb);
    const int m0 = mb * W8_BM, n0 = nb * W8_BN;
    const GroupRows& gr = gc.get(a, g);
    const int nk = gr.count > 0 ? ceil_div(gr.count, 128) : 0;
#pragma unroll
    for (int ii = 0; ii < MI; ++ii) acc[ii][0] = acc[ii][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < nk; ++k) {
      // the lane constants pass through an empty asm each stage, so the
      // per-subtile addresses stay one register plus an immediate
      asm volatile("" : "+v"(l8.lo), "+v"(l8.hi), "+v"(lsa), "+v"(lsb));
      const uint8_t* st = ring + (S % W8_NSTG) * W8_STB;
      const i32x8 b0 = frag8(st + W8_B, 32 * wn, l8), b1 = frag8(st + W8_B, 32 * wn + 16, l8);
      const f32x4 sb0 = *reinterpret_cast<const f32x4*>(st + W8_BS + 32 * wn * 4 + lsb);
      const f32x4 sb1 = *reinterpret_cast<const f32x4*>(st + W8_BS + (32 * wn + 16) * 4 + lsb);
      i32x8 xa = frag8(st + W8_A, 16 * wm, l8);
      float sa = *reinterpret_cast<const float*>(st + W8_AS + 16 * wm * 4 + lsa);
      f32x4 p0{}, p1{};
      float psa = 0.f;
#pragma unroll
      for (int ii = 0; ii < MI; ++ii) {
        i32x8 xn;
        float sn = 0.f;
        if (ii + 1 < MI) {   // the next row subtile's fragment, read one subtile ahead
          xn = frag8(st + W8_A, 16 * (2 * (ii + 1) + wm), l8);
          sn = *reinterpret_cast<const float*>(st + W8_AS + 16 * (2 * (ii + 1) + wm) * 4 + lsa);
        }
        __builtin_amdgcn_sched_barrier(0);
        const f32x4 n0p = mfma_e4m3(b0, xa, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 n1p = mfma_e4m3(b1, xa, f32x4{0.f, 0.f, 0.f, 0.f});
        if (ii > 0) {   // the previous row subtile's products, while these run
          acc[ii - 1][0] += p0 * (psa * sb0);
          acc[ii - 1][1] += p1 * (psa * sb1);
          // here, not sunk to the end of the stage (which would keep every
          // product live at once)
          asm volatile("" : "+v"(acc[ii - 1][0]), "+v"(acc[ii - 1][1]));
        }
        __builtin_amdgcn_sched_barrier(0);
        p0 = n0p;
        p1 = n1p;
        psa = sa;
        if (ii + 1 < MI) {
          xa = xn;
          sa = sn;
        }
      }
      acc[MI - 1][0] += p0 * (psa * sb0);
      acc[MI - 1][1] += p1 * (psa * sb1);
      ++S;
      if (S < total) block_barrier();   // #S: this stage's buffer is free
    }
    float* dst = g < a.n_routed ? routed_dst + static_cast<size_t>(g) * M * N
                                : shared_dst + static_cast<size_t>(g - a.n_routed) * M * N;
    // each half subtile (8 rows x 128 bytes) through the wave's staging, so
    // every store writes whole lines, streamed past the caches (as in the
    // bf16 Wgrad)
    uint8_t* sg = ring + W8_NSTG * W8_STB + 1024 * w;
#pragma unroll
    for (int ii = 0; ii < MI; ++ii) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if ((lr >> 3) == h) {
          const int r = lr & 7;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            *reinterpret_cast<f32x4*>(sg + r * 128 + (((4 * j + lg) ^ r) << 4)) = acc[ii][j];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int r = lane >> 3, c = lane & 7;
        const f32x4 v = *reinterpret_cast<const f32x4*>(sg + r * 128 + ((c ^ r) << 4));
        const int m = m0 + 16 * (2 * ii + wm) + 8 * h + r, n = n0 + 32 * wn + 4 * c;
        if (m < M && n < N) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst + static_cast<size_t>(m) * N + n));
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  }
}

// dW_down[c][i] = sum_r dY[r][c] H[r][i]   (qa: dY codes, qb: H codes)
__global__ __launch_bounds__(THREADS, 1) void wgrad8_down_kernel(BwdArgs a) {
  wgrad8_persistent<4>(a, a.qa, a.qa_s, a.d, a.qb, a.qb_s, a.inter, a.dw_down, a.dws_down);
}

// dW_gate_up[j][c] = sum_r [dG dU][r][j] X[r][c]   (qa: [dG dU] codes, qb: X codes)
__global__ __launch_bounds__(THREADS, 1) void wgrad8_gateup_kernel(BwdArgs a) {
  wgrad8_persistent<0>(a, a.qa, a.qa_s, 2 * a.inter, a.qb, a.qb_s, a.d, a.dw_gate_up, a.dws_gate_up);
}

// ------------------------------------------------------------------ elementwise passes

// One wave per token t, over all of its grouped rows r (the K routed rows, by
// pos, and the N_s shared rows): dY_r = g dy_t, X_r = u_t (bf16; the bf16
// Wgrad's operand, not written for the FP8 backward, whose quantiser reads u
// by token) and, for a routed row, dg_{t,k} = dy_t . Y_r (fp32; each lane
// sums its columns in order, then a butterfly over the lanes).  dy_t and u_t
// are read once for all of the token's rows.
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.T) return;
  const int K = a.top_k;
  int rk[MAX_TOPK];
  float gk[MAX_TOPK], dot[MAX_TOPK];
#pragma unroll
  for (int k = 0; k < MAX_TOPK; ++k) {
    rk[k] = -1;
    gk[k] = 0.f;
    dot[k] = 0.f;
    if (k < K) {
      const int r = a.pos[static_cast<size_t>(t) * K + k];
      if (MOE_CHECK(r >= 0 && r < a.TK && a.perm_token[r] == t, 503)) rk[k] = r;
      gk[k] = a.gate[static_cast<size_t>(t) * K + k];
    }
  }
  const float* dyt = a.dy + static_cast<size_t>(t) * a.d;
  const uint16_t* ut = a.u + static_cast<size_t>(t) * a.d;
  for (int c = 4 * lane; c < a.d; c += 256) {
    const float4 dv = *reinterpret_cast<const float4*>(dyt + c);
    const uint2 uv = *reinterpret_cast<const uint2*>(ut + c);
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k) {
      if (rk[k] < 0) continue;
      const size_t o = static_cast<size_t>(rk[k]) * a.d + c;
      const float g = gk[k];
      *reinterpret_cast<uint2*>(a.dys + o) = make_uint2(bf16x2(g * dv.x, g * dv.y), bf16x2(g * dv.z, g * dv.w));
      if (!a.fp8) *reinterpret_cast<uint2*>(a.xp + o) = uv;
      float yv[4];
      unpack4(*reinterpret_cast<const uint2*>(a.y + o), yv);
      dot[k] = fmaf(dv.x, yv[0], dot[k]);
      dot[k] = fmaf(dv.y, yv[1], dot[k]);
      dot[k] = fmaf(dv.z, yv[2], dot[k]);
      dot[k] = fmaf(dv.w, yv[3], dot[k]);
    }
    for (int j = 0; j < a.n_shared; ++j) {   // shared rows: g = 1
      const size_t o = (static_cast<size_t>(a.TK) + static_cast<size_t>(j) * a.T + t) * a.d + c;
      *reinterpret_cast<uint2*>(a.dys + o) = make_uint2(bf16x2(dv.x, dv.y), bf16x2(dv.z, dv.w));
      if (!a.fp8) *reinterpret_cast<uint2*>(a.xp + o) = uv;
    }
  }
#pragma unroll
  for (int k = 0; k < MAX_TOPK; ++k) {
    if (rk[k] < 0) continue;
    float v = dot[k];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) a.dg[static_cast<size_t>(t) * K + k] = v;
  }
}

// Per token: ds_k = (dg_k - sum_j g_j dg_j) / S, dz_k = ds_k s_k (1 - s_k);
// dz also by grouped row (for dE).
__global__ __launch_bounds__(256) void bwd_dz_kernel(BwdArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.T) return;
  const size_t o = static_cast<size_t>(t) * a.top_k;
  float S = 0.f, gd = 0.f;
  for (int k = 0; k < a.top_k; ++k) {
    S += a.sel_score[o + k];
    gd = fmaf(a.gate[o + k], a.dg[o + k], gd);
  }
  for (int k = 0; k < a.top_k; ++k) {
    const float s = a.sel_score[o + k];
    const float dz = (a.dg[o + k] - gd) / S * (s * (1.f - s));
    a.dz[o + k] = dz;
    a.dzr[a.pos[o + k]] = dz;
  }
}

// One wave per token: du_t = dy_t + the shared experts' dX rows + the K
// routed dX rows + sum_k dz_k e_k, in that order (fp32).  Each column chunk
// issues all of its row loads before the first add, so the wave waits on
// memory once per chunk, not once per row.
__global__ __launch_bounds__(256) void bwd_du_kernel(BwdArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.T) return;
  const size_t o = static_cast<size_t>(t) * a.top_k;
  const int K = a.top_k, NS = a.n_shared;
  size_t rowk[MAX_TOPK], cenk[MAX_TOPK];
  float dzk[MAX_TOPK];
#pragma unroll
  for (int k = 0; k < MAX_TOPK; ++k) {
    rowk[k] = cenk[k] = 0;
    dzk[k] = 0.f;
    if (k < K) {
      rowk[k] = static_cast<size_t>(a.pos[o + k]) * a.d;
      cenk[k] = static_cast<size_t>(a.idx[o + k]) * a.d;
      dzk[k] = a.dz[o + k];
    }
  }
  for (int c = 4 * lane; c < a.d; c += 256) {
    const float4 dv = *reinterpret_cast<const float4*>(a.dy + static_cast<size_t>(t) * a.d + c);
    uint2 xs[MAX_SHARED], xr[MAX_TOPK], xe[MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MAX_SHARED; ++j)
      if (j < NS)
        xs[j] = *reinterpret_cast<const uint2*>(a.dx + static_cast<size_t>(a.TK + static_cast<long long>(j) * a.T + t) * a.d + c);
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k)
      if (k < K) {
        xr[k] = *reinterpret_cast<const uint2*>(a.dx + rowk[k] + c);
        xe[k] = *reinterpret_cast<const uint2*>(a.centroids + cenk[k] + c);
      }
    float4 v = dv;
    float x[4];
#pragma unroll
    for (int j = 0; j < MAX_SHARED; ++j)
      if (j < NS) {
        unpack4(xs[j], x);
        v.x += x[0]; v.y += x[1]; v.z += x[2]; v.w += x[3];
      }
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k)
      if (k < K) {
        unpack4(xr[k], x);
        v.x += x[0]; v.y += x[1]; v.z += x[2]; v.w += x[3];
      }
#pragma unroll
    for (int k = 0; k < MAX_TOPK; ++k)
      if (k < K) {
        unpack4(xe[k], x);
        v.x = fmaf(dzk[k], x[0], v.x); v.y = fmaf(dzk[k], x[1], v.y);
        v.z = fmaf(dzk[k], x[2], v.z); v.w = fmaf(dzk[k], x[3], v.w);
      }
    *reinterpret_cast<float4*>(a.du + static_cast<size_t>(t) * a.d + c) = v;
  }
}

// dE_e[c] = sum over expert e's grouped rows (ascending) of dz_r u_{t(r)}[c];
// block (e, 1024-column chunk), 4 columns per thread; zero for an expert
// without rows.  The rows go in batches of 8 whose loads are all issued
// before the batch's first multiply-add.
__global__ __launch_bounds__(256) void bwd_de_kernel(BwdArgs a) {
  constexpr int NB = 8;
  const int e = blockIdx.y;
  const int c = blockIdx.x * 1024 + 4 * threadIdx.x;
  if (c >= a.d) return;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  const int r1 = a.offsets[e] + a.counts[e];
  for (int r = a.offsets[e]; r < r1; r += NB) {
    float dz[NB];
    int tok[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      dz[j] = r + j < r1 ? a.dzr[r + j] : 0.f;
      tok[j] = r + j < r1 ? a.perm_token[r + j] : 0;
    }
    uint2 xv[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (r + j < r1) xv[j] = *reinterpret_cast<const uint2*>(a.u + static_cast<size_t>(tok[j]) * a.d + c);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (r + j < r1) {
        float x[4];
        unpack4(xv[j], x);
        v.x = fmaf(dz[j], x[0], v.x); v.y = fmaf(dz[j], x[1], v.y);
        v.z = fmaf(dz[j], x[2], v.z); v.w = fmaf(dz[j], x[3], v.w);
      }
  }
  *reinterpret_cast<float4*>(a.dcentroids + static_cast<size_t>(e) * a.d + c) = v;
}

}  // namespace

MOE_DEBUG_FILE(bwd)

// FP8 stages 1-4 (a.fp8): the Dgrad GEMMs on the forward's FP8 row-times-
// weight kernel, the Wgrad GEMMs on the 128x1 codes.
hipError_t launch_backward_stage_fp8(int stage, const BwdArgs& a, hipStream_t s) {
  auto cq_grid = [](int C) { return static_cast<unsigned>(ceil_div(C / 64, CQ_CHUNKS)); };
  const int R = static_cast<int>(a.R);
  const unsigned kbt = static_cast<unsigned>(a.kt / 128);
  hipError_t e = hipSuccess;
  switch (stage) {
    case 1: {   // dH = q(dY) W_down (bf16 into hr), then the SwiGLU backward
      if (a.T == 0) break;
      if ((e = launch_quant_act(a.dys, R, a.d, a.qr, a.qr_s, s)) != hipSuccess) return e;
      const DownArgs da{a.qr, a.qr_s, a.n_routed, a.inter, a.d, a.w_down_t, a.ws_down_t, a.s_down_t, a.ss_down_t,
                        a.mtiles, a.mt_count, a.max_mtiles, a.hr};
      if ((e = launch_down(FMT_E4M3, da, s)) != hipSuccess) return e;
      const long long n = a.R * (a.inter / 8);
      hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, a);
      break;
    }
    case 2: {   // dX = q([dG dU]) W_gate_up
      if (a.T == 0) break;
      if ((e = launch_quant_act(a.dgu, R, 2 * a.inter, a.qr, a.qr_s, s)) != hipSuccess) return e;
      const DownArgs da{a.qr, a.qr_s, a.n_routed, a.d, 2 * a.inter, a.w_gate_up_t, a.ws_gate_up_t, a.s_gate_up_t,
                        a.ss_gate_up_t, a.mtiles, a.mt_count, a.max_mtiles, a.dx};
      if ((e = launch_down(FMT_E4M3, da, s)) != hipSuccess) return e;
      break;
    }
    case 3:     // dW_down from the 128x1 codes of dY and H
      if (a.T > 0) {
        hipLaunchKernelGGL(colquant_kernel, dim3(kbt, cq_grid(a.d)), dim3(256), 0, s, a, a.dys, a.d, false, a.qa,
                           a.qa_s);
        hipLaunchKernelGGL(colquant_kernel, dim3(kbt, cq_grid(a.inter)), dim3(256), 0, s, a, a.hr, a.inter, false, a.qb,
                           a.qb_s);
      }
      hipLaunchKernelGGL(wgrad8_down_kernel, dim3(wgrad_grid()), dim3(THREADS), 0, s, a);
      break;
    case 4:     // dW_gate_up from the 128x1 codes of [dG dU] and X
      if (a.T > 0) {
        hipLaunchKernelGGL(colquant_kernel, dim3(kbt, cq_grid(2 * a.inter)), dim3(256), 0, s, a, a.dgu, 2 * a.inter,
                           false, a.qa, a.qa_s);
        // X: the rows of u by token (the bf16 path's gathered copy is not written)
        hipLaunchKernelGGL(colquant_kernel, dim3(kbt, cq_grid(a.d)), dim3(256), 0, s, a, a.u, a.d, true, a.qb,
                           a.qb_s);
      }
      hipLaunchKernelGGL(wgrad8_gateup_kernel, dim3(wgrad_grid()), dim3(THREADS), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_backward_stage(int stage, const BwdArgs& a, hipStream_t s) {
  if (a.fp8 && stage >= 1 && stage <= 4) return launch_backward_stage_fp8(stage, a, s);
  switch (stage) {
    case 0:   // prep, dz
      if (a.T == 0) break;
      hipLaunchKernelGGL(bwd_prep_kernel, dim3(static_cast<unsigned>((a.T + 3) / 4)), dim3(256), 0, s, a);
      hipLaunchKernelGGL(bwd_dz_kernel, dim3(ceil_div(a.T, 256)), dim3(256), 0, s, a);
      break;
    case 1:   // Dgrad of the down GEMM, SwiGLU backward
      if (a.T == 0) break;
      hipLaunchKernelGGL(dgrad_down_kernel, dim3(mtile_grid(a.max_mtiles, ceil_div(a.inter, BT))), dim3(THREADS), 0,
                         s, a);
      break;
    case 2:   // Dgrad of the gate/up GEMM
      if (a.T == 0) break;
      hipLaunchKernelGGL(dgrad_gateup_kernel, dim3(mtile_grid(a.max_mtiles, ceil_div(a.d, BT))), dim3(THREADS), 0, s,
                         a);
      break;
    case 3:   // Wgrad of the down GEMM (every group: zeros where a group has no rows)
      hipLaunchKernelGGL(wgrad_down_kernel, dim3(wgrad_grid()), dim3(THREADS), 0, s, a);
      break;
    case 4:   // Wgrad of the gate/up GEMM
      hipLaunchKernelGGL(wgrad_gateup_kernel, dim3(wgrad_grid()), dim3(THREADS), 0, s, a);
      break;
    case 5:   // du, dcentroids (zeros for experts without rows)
      if (a.T > 0) hipLaunchKernelGGL(bwd_du_kernel, dim3(ceil_div(a.T, 4)), dim3(256), 0, s, a);
      if (a.n_routed > 0) hipLaunchKernelGGL(bwd_de_kernel, dim3(ceil_div(a.d, 1024), a.n_routed), dim3(256), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
