// Internal launcher interface between the C-ABI layer and the kernel files.
// Every launcher enqueues on the given stream and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_common.hpp"

namespace moe {

// B rows per grouped-GEMM tile: 128 gate + 128 up rows (128 h columns), or
// 256 output columns for the down projection.
constexpr int GG_BNW = 256;
constexpr int GG_HCOLS = 128;
constexpr int ROUTE_BT = 32;      // tokens per router block
constexpr int GROUP_TB = 256;     // tokens per histogram / permute block
constexpr int MAX_ROUTED = 512;
constexpr int MAX_SHARED = 8;
constexpr int MAX_TOPK = 16;
constexpr int MT_UNIT = 4;        // m-tiles of one group visited together by the grouped GEMMs
constexpr int MT_SEGMENTS = 8;    // segments of the m-tile list (one per XCD), each with a share of every group

struct RouteArgs {
  const void* u;          // [T][d] fmt
  const void* centroids;  // [N_r][d] fmt
  const float* bias;      // [N_r]
  int T, d, n_routed, top_k;
  int32_t* idx;           // [T][K]
  float* gate;            // [T][K]
  float* scores;          // scratch: [T][N_r] sigmoids (route_split), [ksplit][T][N_r] partial logits (ksplit > 0)
  int ksplit;             // route_ksplit(...) of this shape: 0, or the number of K slices
  int n_groups;           // group-limited routing: experts in n_groups equal runs, a token
  int topk_groups;        // takes experts from at most topk_groups of them (off: topk_groups >= n_groups)
  float* sel_score;       // null, or [T][K]: the selected experts' sigmoid scores s (training)
};

// Batches under 128 router blocks (T < 4096) spread the experts over blocks
// too: a score kernel writes the sigmoids to scratch, a second kernel selects.
constexpr int ROUTE_SPLIT_T = 4096;
inline bool route_split(long long T) { return T < ROUTE_SPLIT_T; }

// bf16 batches of 256-token tiles that, with d cut into K slices of at least
// 4 whole 128-byte pairs, give at least 128 blocks: 256-token x 256-expert
// tiles on the grouped GEMM's pipeline, fp32 partial logits per slice to
// scratch, then a kernel that sums the slices in order and selects.  Returns
// the number of slices (every slice non-empty), or 0 where it does not apply.
inline int route_ksplit(int fmt, long long T, long long d, int n_routed) {
  if (fmt != FMT_BF16 || T <= 0 || n_routed < 128 || n_routed > 256 || n_routed % 4 != 0 || d % 64 != 0) return 0;
  const long long tiles = (T + 255) / 256, np = d / 64;
  long long s = (256 + tiles - 1) / tiles;
  if (s > np / 4) s = np / 4;
  if (s < 1 || tiles * s < 128) return 0;
  const long long pps = (np + s - 1) / s;
  return static_cast<int>((np + pps - 1) / pps);
}

// Floats of router scratch a shape needs.
inline long long route_scratch_floats(int fmt, long long T, long long d, int n_routed) {
  const int ks = route_ksplit(fmt, T, d, n_routed);
  if (ks > 0) return ks * T * n_routed;
  return route_split(T) ? T * n_routed : 0;
}

struct GroupArgs {
  const int32_t* idx;     // [T][K]
  int T, top_k, n_routed, n_shared;
  int32_t* block_hist;    // [nblk][N_r] scratch
  int32_t* counts;        // [N_r]
  int32_t* offsets;       // [N_r + 1]
  int32_t* perm_token;    // [T*K]
  int32_t* pos;           // [T][K]
  int4* mtiles;           // [max_mtiles] (group, first grouped row, rows, unit info); null: routing only
  int32_t* mt_count;      // [2 + MT_SEGMENTS]: m-tile count, then each list segment's first m-tile (-1: none)
  int bm;                 // grouped-GEMM tile rows (m-tiles hold at most bm rows)
  int seg_cap;            // m-tiles one list segment may hold (the GEMM blocks of one XCD)
};

struct GateUpArgs {
  const void* x;          // GEMM input rows by token: u (f32/bf16) or its e4m3 codes
  const float* x_scale;   // e4m3: [T][d/128]
  const int32_t* perm_token;
  int T, TK, n_routed, d, inter;
  const void* w_routed;   // [N_r][2I][d]
  const void* w_shared;   // [N_s][2I][d]
  const float* sw_routed; // e4m3: [N_r][2I/128][d/128]
  const float* sw_shared;
  const int4* mtiles;
  const int32_t* mt_count;
  int max_mtiles;
  void* h;                // [R][I]: f32 / bf16 / e4m3 codes
  float* h_scale;         // e4m3: [R][I/128]
  uint16_t* gu;           // training only: [R][2I] the SwiGLU inputs G (columns 0..I-1) and U, bf16; else null
};

struct DownArgs {
  const void* h;          // [R][I]
  const float* h_scale;   // e4m3: [R][I/128]
  int n_routed, d, inter;
  const void* w_routed;   // [N_r][d][I]
  const void* w_shared;   // [N_s][d][I]
  const float* sw_routed; // e4m3: [N_r][d/128][I/128]
  const float* sw_shared;
  const int4* mtiles;
  const int32_t* mt_count;
  int max_mtiles;
  void* y;                // [R][d]: f32 (f32 path) or bf16
};

struct CombineArgs {
  const void* u;          // [T][d]
  const void* yrows;      // [R][d] expert outputs in grouped row order
  const float* gate;      // [T][K]
  const int32_t* pos;     // [T][K]
  int T, d, top_k, n_shared;
  long long TK;
  void* out;              // [T][d]
};

// The backward pass (bf16): what the training forward left in the workspace,
// the upstream gradient, and the gradient outputs.
struct BwdArgs {
  int T, d, n_routed, n_shared, inter, top_k;
  long long TK, R;                // T*K routed rows; R = T*K + N_s*T grouped rows
  int max_mtiles;
  const int4* mtiles;             // the forward's m-tile list
  const int32_t* mt_count;
  const int32_t* offsets;         // [N_r + 1]
  const int32_t* counts;          // [N_r]
  const int32_t* perm_token;      // [T*K]
  const int32_t* pos;             // [T][K]
  const int32_t* idx;             // [T][K]
  const float* gate;              // [T][K]
  const float* sel_score;         // [T][K] selected sigmoids
  const uint16_t* u;              // [T][d] bf16
  const uint16_t* centroids;      // [N_r][d] bf16
  const uint16_t* y;              // [R][d] bf16 expert outputs Y
  const float* dy;                // [T][d] upstream gradient
  const void* w_gate_up;          // [N_r][2I][d] bf16
  const void* w_down;             // [N_r][d][I]
  const void* ws_gate_up;         // [N_s][2I][d]
  const void* ws_down;            // [N_s][d][I]
  const uint16_t* gu;             // [R][2I] cached G | U
  uint16_t* dys;                  // [R][d] g dy rows
  uint16_t* xp;                   // [R][d] gathered u rows (bf16 backward only)
  uint16_t* dgu;                  // [R][2I] dG | dU
  uint16_t* hr;                   // [R][I] recomputed H
  uint16_t* dx;                   // [R][d] Dgrad of the gate/up GEMM
  float* dg;                      // [T][K]
  float* dz;                      // [T][K]
  float* dzr;                     // [T*K] dz by grouped row
  float* du;                      // [T][d]
  float* dcentroids;              // [N_r][d]
  float* dw_gate_up;              // [N_r][2I][d]
  float* dw_down;                 // [N_r][d][I]
  float* dws_gate_up;             // [N_s][2I][d]
  float* dws_down;                // [N_s][d][I]
  // FP8 backward (e4m3 weights; zero / null otherwise).  The weights' codes
  // transposed (the same 128x128 blocks, so the scales are transposed too):
  int fp8;
  const void* w_gate_up_t;        // [N_r][d][2I] e4m3
  const void* w_down_t;           // [N_r][I][d]
  const void* ws_gate_up_t;       // [N_s][d][2I]
  const void* ws_down_t;          // [N_s][I][d]
  const float* s_gate_up_t;       // [N_r][d/128][2I/128]
  const float* s_down_t;          // [N_r][I/128][d/128]
  const float* ss_gate_up_t;
  const float* ss_down_t;
  uint8_t* qr;                    // [R][max(d, 2I)] 1x128 codes of a Dgrad input: dY, then [dG dU]
  float* qr_s;                    // [R][max(d, 2I)/128]
  long long kt;                   // columns of the transposed 128x1 codes (wgrad8_kt)
  uint8_t* qa;                    // [max(d, 2I)][kt] Wgrad operand A, 128x1 codes transposed: dY, then [dG dU]
  float* qa_s;                    // [max(d, 2I)][kt/128]
  uint8_t* qb;                    // [max(I, d)][kt] Wgrad operand B: H, then X
  float* qb_s;                    // [max(I, d)][kt/128]
};

// FP8 Wgrad: group g's 128-row blocks of 128x1 codes, transposed, start at
// column koff_g = 128 (floor(first_g / 128) + 2 g) of the [channel][kt] code
// arrays (first_g: the group's first grouped row).  Consecutive groups start
// at least ceil(rows_g / 128) + 1 blocks apart, so each has room for its
// blocks; kt covers the last one.
inline long long wgrad8_kt(long long R, int n_groups) { return 128 * ((R + 127) / 128 + 2LL * n_groups + 1); }

hipError_t launch_route(int fmt, const RouteArgs& a, hipStream_t s);
// The backward in six stages, launched in order 0..5: prep and dz; Dgrad of
// the down GEMM (with the SwiGLU backward); Dgrad of the gate/up GEMM; Wgrad
// of the down GEMM; Wgrad of the gate/up GEMM; du and dcentroids.
constexpr int BWD_STAGES = 6;
hipError_t launch_backward_stage(int stage, const BwdArgs& a, hipStream_t s);
hipError_t launch_group(const GroupArgs& a, hipStream_t s);
hipError_t launch_quant_act(const void* x, int rows, int cols, uint8_t* q, float* scale, hipStream_t s);
hipError_t launch_quant_weight(int fmt, const void* w, long long n, int rows, int cols, uint8_t* q, float* scale,
                               hipStream_t s);
hipError_t launch_bias_update(float* bias, const int32_t* counts, int n_routed, long long total, float gamma,
                              hipStream_t s);
hipError_t launch_gateup(int fmt, const GateUpArgs& a, hipStream_t s);
hipError_t launch_down(int fmt, const DownArgs& a, hipStream_t s);
hipError_t launch_combine(int xfmt, int yfmt, int ofmt, const CombineArgs& a, hipStream_t s);

#ifdef MOE_DEBUG
// Debug build: each kernel file's first failed index check (0: none), cleared
// when read; -1 if it could not be read.  Check ids: 1xx route, 2xx group,
// 3xx grouped GEMMs, 4xx combine, 5xx backward.
int debug_take_route();
int debug_take_group();
int debug_take_ggemm();
int debug_take_combine();
int debug_take_bwd();
#endif

// Tile rows of the grouped GEMMs for a weight format (m-tiles hold at most this many rows).
int gg_bm(int fmt);

// m-tiles per XCD segment the GEMM grids cover
inline int seg_cap(int max_mt) { return (max_mt + MT_SEGMENTS - 1) / MT_SEGMENTS; }

inline int max_mtiles(long long T, int K, int n_routed, int n_shared, int bm) {
  // sum over groups of ceil(M_g / bm) <= (T*K)/bm + N_r + N_s * ceil(T/bm)
  return static_cast<int>((T * K) / bm + n_routed + n_shared * ((T + bm - 1) / bm));
}

}  // namespace moe
