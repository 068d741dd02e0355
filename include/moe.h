/*
 * moe.h - C ABI of the DeepSeekMoE layer for AMD Instinct MI355X (gfx950).
 *
 * What is computed (pages about the DeepSeek-V3 Technical Report):
 *   - "DeepSeek-V3 Technical Report" summary (xyznot.com), section 2,
 *     "DeepSeekMoE with Auxiliary-Loss-Free Balancing":
 *       h'_t    = u_t + sum_{i<=N_s} FFN^(s)_i(u_t) + sum_{i<=N_r} g_{i,t} FFN^(r)_i(u_t)
 *       s_{i,t} = Sigmoid(u_t^T e_i)
 *       g'_{i,t}= s_{i,t} if s_{i,t} + b_i is among the K_r largest of {s_{j,t} + b_j}, else 0
 *       g_{i,t} = g'_{i,t} normalised over the token's selected experts
 *       b_i    -= gamma when expert i is overloaded, += gamma when underloaded (gamma = 0.001)
 *     and, in its key-ideas list, the FP8 granularity: E4M3 for all tensors,
 *     1x128 activation tiles, 128x128 weight blocks, FP32 promotion every 128.
 *   - The same h' and g' formulas in the wenxiaobai explainer ("DeepSeek-V3深度解析"),
 *     items on DeepSeekMoE and on auxiliary-loss-free load balancing.
 *   - The expert FFN is the SwiGLU operator (the report's FP8 training section,
 *     as paraphrased on why-be.co.kr): FFN(x) = W_down (SiLU(W_gate x) * (W_up x)).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (HBM of the current HIP device),
 *     owned by the caller; the library never allocates, frees, synchronises
 *     or keeps state between calls.  Work is enqueued on `stream` (0 = the
 *     null stream) and the call returns without waiting for it.
 *   - Matrices are row-major and the reduction dimension is innermost
 *     ("K-contiguous").  Pointers must be 16-byte aligned.
 *   - Every call returns a moe_status.  Arguments are validated before any
 *     work is enqueued: on an error nothing is launched and no output is
 *     touched.  MOE_ERR_LAUNCH reports a failed kernel launch (the outputs
 *     are then undefined).
 *   - Inputs are expected to be finite.  Should a score be NaN the router
 *     still returns K distinct in-range experts per token.
 *   - Repeated calls with the same inputs give bit-identical outputs.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_DTYPE_F32 = 0,   /* IEEE binary32 */
  MOE_DTYPE_BF16 = 1,  /* bfloat16 (values rounded to nearest even) */
  MOE_DTYPE_E4M3 = 2   /* OCP FP8 E4M3 (bias 7, max 448, no inf) with fp32 block scales */
} moe_dtype;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, bad shape, bad dtype combination, misalignment */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but outside the library's limits (see moe_shape) */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than moe_workspace_size() */
  MOE_ERR_LAUNCH = 4        /* a kernel launch failed */
} moe_status;

/*
 * Layer shape and dtypes.
 *   T         tokens in the batch (>= 0; 0 is a no-op)
 *   d         hidden size
 *   n_routed  N_r routed experts, 1..512
 *   n_shared  N_s shared experts, 0..8
 *   inter     I, the intermediate size of every expert (shared and routed)
 *   top_k     K_r experts chosen per token, 1..min(N_r, 16)
 *   x_dtype   dtype of u and of the centroids e_i: F32 or BF16
 *   w_dtype   dtype of the expert weights and of the expert GEMMs:
 *               F32  (requires x_dtype F32)
 *               BF16 (requires x_dtype BF16)
 *               E4M3 (requires x_dtype BF16): the FP8 path.  u is quantised
 *                    per 1x128 tile and h per 1x128 tile on the fly, weights
 *                    come pre-quantised per 128x128 block (moe_quantize_weight_e4m3).
 *                    The router and the residual use the unquantised bf16 u.
 *   out_dtype dtype of y: F32 or BF16
 *   n_groups, topk_groups  group-limited (node-limited) routing: the experts
 *             form n_groups equal runs of consecutive experts (the devices or
 *             nodes they live on) and each token takes its experts from at
 *             most topk_groups of them.  Groups are ranked by the sum of each
 *             group's ceil(K / topk_groups) largest s + b (at most the group
 *             size), ties to the lower group; the top-K is then taken over
 *             the kept groups' experts.  A reading of the all-to-all
 *             paragraph of the xyznot summary (a token lands on a median of
 *             3.2 experts per node), which gives the effect but not the rule.
 *             Off (global top-K) when n_groups is 0 or 1 or topk_groups >=
 *             n_groups.  Otherwise n_groups divides n_routed, n_groups <= 64,
 *             and topk_groups * n_routed / n_groups >= top_k.
 * Limits: d and inter multiples of 64 (F32: 32 is enough; E4M3: 128, and
 * at most 32768); T * top_k and (top_k + n_shared) * T below 2^31; the
 * bytes of u (T * d * size of x_dtype) and of one expert's gate/up matrix
 * (2 * inter * d * size of w_dtype) below 2^32.  Outside them the calls
 * return MOE_ERR_UNSUPPORTED.
 */
typedef struct {
  int32_t T, d, n_routed, n_shared, inter, top_k;
  int32_t x_dtype, w_dtype, out_dtype;
  int32_t n_groups, topk_groups;
} moe_shape;

/*
 * Expert weights.  Gate and up projections of one expert are one [2I][d]
 * matrix, the I gate rows first.
 *   w_gate_up   [N_r][2I][d]     w_dtype
 *   w_down      [N_r][d][I]      w_dtype
 *   ws_gate_up  [N_s][2I][d]     w_dtype (may be null when N_s = 0)
 *   ws_down     [N_s][d][I]      w_dtype
 * E4M3 only (fp32 block scales, one per 128x128 block of the matrix above):
 *   s_gate_up   [N_r][2I/128][d/128]
 *   s_down      [N_r][d/128][I/128]
 *   ss_gate_up  [N_s][2I/128][d/128]
 *   ss_down     [N_s][d/128][I/128]
 * E4M3, moe_backward only (null otherwise): the same codes transposed, read
 * by the FP8 Dgrad GEMMs, with their block scales transposed (a 128x128
 * block has one scale in either orientation; moe_quantize_weight_e4m3 of the
 * transposed matrix gives exactly these):
 *   w_gate_up_t [N_r][d][2I]     s_gate_up_t [N_r][d/128][2I/128]
 *   w_down_t    [N_r][I][d]      s_down_t    [N_r][I/128][d/128]
 *   ws_gate_up_t, ws_down_t, ss_gate_up_t, ss_down_t: the shared experts'
 */
typedef struct {
  const void* w_gate_up;
  const void* w_down;
  const void* ws_gate_up;
  const void* ws_down;
  const float* s_gate_up;
  const float* s_down;
  const float* ss_gate_up;
  const float* ss_down;
  const void* w_gate_up_t;
  const void* w_down_t;
  const void* ws_gate_up_t;
  const void* ws_down_t;
  const float* s_gate_up_t;
  const float* s_down_t;
  const float* ss_gate_up_t;
  const float* ss_down_t;
} moe_weights;

/*
 * Routing results.
 *   topk_idx       [T][K] int32  selected experts, by descending s + b
 *                                (exact ties: lower index first)
 *   topk_gate      [T][K] fp32   g = s / (sum of the K selected s), same order
 *   expert_counts  [N_r]  int32  assignments per expert (sum = T*K)
 *   expert_offsets [N_r+1] int32 exclusive prefix sum of expert_counts
 *   perm_token     [T*K]  int32  token of each grouped row; grouped rows are
 *                                expert-major, tokens ascending within an expert
 *   pos            [T][K] int32  grouped row of assignment (t, k)
 */
typedef struct {
  int32_t* topk_idx;
  float* topk_gate;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* perm_token;
  int32_t* pos;
} moe_routing;

/* Human-readable name of a status code (static string). */
const char* moe_status_str(int status);

/* Library version string (static). */
const char* moe_version(void);

/*
 * Bytes of device workspace moe_route / moe_forward need for `shape`
 * (written to *bytes).  The same workspace serves both calls.
 */
int moe_workspace_size(const moe_shape* shape, size_t* bytes);

/*
 * Routing only: affinities, biased top-K, normalised gates, and the stable
 * grouping of assignments by expert.  Defined by the xyznot summary of the
 * DeepSeek-V3 Technical Report, section 2: s_{i,t} = Sigmoid(u_t^T e_i), the
 * top-K_r over s + b for g', and g = g' normalised over the selected experts.  Computes every field of `out` (all
 * must be non-null).  u: [T][d] x_dtype; centroids: [N_r][d] x_dtype;
 * bias: [N_r] fp32.  The affinity GEMM accumulates in fp32.
 */
int moe_route(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
              const moe_routing* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Where moe_forward keeps its intermediate results inside the workspace for
 * `shape` (byte offsets from the workspace's start), for tests and tools
 * that inspect them after a call; not an operation of the layer.
 *   mtiles      int32x4 [max_mtiles]  the grouped GEMMs' m-tile list: (group,
 *               first grouped row, rows, (index within its unit << 8) | unit
 *               size); groups 0..N_r-1 are the routed experts, N_r.. the
 *               shared ones (shared expert s holds grouped rows T*K + s*T + t)
 *   mt_count    int32 [2 + 8]  m-tile count, then the first m-tile of each
 *               of the 8 list segments and the count again (all -1 after the
 *               count when the list is not cut into per-XCD segments)
 *   h, h_scale  H [R][I] (w_dtype; fp32 scales [R][I/128] for E4M3) and
 *   y           Y [R][d] (fp32 for F32 weights, else bf16): the gate/up and
 *               down GEMM outputs by grouped row, R = T*K + N_s*T
 *   tile_rows   the most rows an m-tile holds
 *   seg_cap     the most m-tiles one list segment may hold
 * Returns MOE_OK, or the status moe_workspace_size() would return.
 */
typedef struct {
  size_t mtiles, mt_count, h, h_scale, y;
  int32_t max_mtiles, tile_rows, seg_cap;
} moe_workspace_map;
int moe_workspace_layout(const moe_shape* shape, moe_workspace_map* map);

/*
 * Optional per-stage timing: when a moe_trace is passed to moe_forward, the
 * library records start[i] on `stream` before stage i and stop[i] after it
 * (hipEventRecord; the events are created and owned by the caller).  A stage
 * that does not run for the given dtypes gets both events back to back.
 */
#define MOE_NUM_STAGES 12
typedef enum {
  MOE_STAGE_ROUTE = 0,    /* affinity GEMM + sigmoid + bias + top-K + gates */
  MOE_STAGE_GROUP = 1,    /* expert histogram, scan, stable permutation, m-tile list */
  MOE_STAGE_QUANT = 2,    /* FP8 only: 1x128 quantisation of u */
  MOE_STAGE_GATE_UP = 3,  /* grouped gate/up GEMM with the SwiGLU epilogue */
  MOE_STAGE_DOWN = 4,     /* grouped down-projection GEMM */
  MOE_STAGE_COMBINE = 5,  /* residual + shared + gate-weighted routed sum */
  /* moe_backward's stages */
  MOE_STAGE_BWD_PREP = 6,           /* scaled dy rows, gathered u rows, dg; dz */
  MOE_STAGE_BWD_DGRAD_DOWN = 7,     /* dH = dY W_down with the SwiGLU backward */
  MOE_STAGE_BWD_DGRAD_GATE_UP = 8,  /* dX = [dG dU] W_gate_up */
  MOE_STAGE_BWD_WGRAD_DOWN = 9,     /* dW_down = dY^T H */
  MOE_STAGE_BWD_WGRAD_GATE_UP = 10, /* dW_gate_up = [dG dU]^T X */
  MOE_STAGE_BWD_COMBINE = 11        /* du and dcentroids */
} moe_stage;
typedef struct {
  hipEvent_t start[MOE_NUM_STAGES];
  hipEvent_t stop[MOE_NUM_STAGES];
} moe_trace;

/*
 * The layer forward: y[T][d] (out_dtype) = h', the DeepSeekMoE layer output
 * of the xyznot summary, section 2 (u_t plus the shared experts' FFNs plus
 * the gate-weighted routed experts' FFNs; each FFN the SwiGLU operator of the
 * report's FP8 training section).  `routing` may be null, and so
 * may any of its fields; non-null fields receive the routing results.
 * Expert outputs are accumulated in fp32 and stored in bf16 between the
 * kernels (fp32 when w_dtype is F32); the final sum is fp32.  `trace` may be
 * null.
 */
int moe_forward(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
                const moe_weights* weights, void* y, const moe_routing* routing, void* workspace,
                size_t workspace_bytes, const moe_trace* trace, hipStream_t stream);

/*
 * moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels, bit-identical results, with no workspace
 * argument.  The intermediate results live in a device array of
 * MOE_STATIC_SCRATCH_BYTES inside the library, one per device, held from the
 * device's first call until the process ends; the call itself allocates,
 * frees and clears nothing.  A shape whose workspace (moe_workspace_size)
 * exceeds that returns MOE_ERR_WORKSPACE before any work is enqueued; 64 MiB
 * holds, e.g., decode batches of up to about 400 tokens at d = 7168, I = 2048,
 * K = 8 + 1 shared expert (bf16).  All calls on one device share its array:
 * calls that overlap on a device (different streams, or host threads) race
 * and must be serialised by the caller; calls on one stream are ordered.
 * The first call on each device also looks up the array's device address.
 */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
int moe_forward_static(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
                       const moe_weights* weights, void* y, const moe_routing* routing, const moe_trace* trace,
                       hipStream_t stream);

/*
 * Training: the layer backward (x_dtype = BF16 with w_dtype = BF16 or E4M3;
 * other dtypes return MOE_ERR_UNSUPPORTED).  The report's FP8 training
 * section (as paraphrased on why-be.co.kr, its Figure 6 passage) runs the
 * three GEMMs of a Linear operator, Fprop, Dgrad and Wgrad, in FP8, and
 * caches the inputs of the SwiGLU operator, recomputing its output in the
 * backward pass.  BF16: every GEMM in bf16 with fp32 accumulation.  E4M3:
 * every GEMM on E4M3 operands with fp32 scales per group of 128 along its
 * inner dimension and fp32 promotion per group -- the Dgrad inputs dY and
 * [dG dU] in 1x128 tiles along their columns against the weights' 128x128
 * blocks read transposed (moe_weights' *_t fields), both Wgrad operands in
 * 128x1 tiles along the grouped rows (blocks counted from each expert's first
 * row); the quantised tensors are the bf16 rows the backward stores.  The
 * weight gradients are fp32 either way.
 *
 * moe_train_workspace_size: bytes of the workspace moe_forward_train and
 * moe_backward share for `shape` (more than moe_workspace_size: the cached
 * SwiGLU inputs and the backward's intermediate rows).
 *
 * moe_forward_train: moe_forward (same y), keeping in the workspace what the
 * backward needs: the routing, the GEMM tile list, the selected experts'
 * sigmoid scores, the SwiGLU inputs G and U of every grouped row (bf16) and
 * the expert outputs.
 *
 * moe_backward: for the upstream gradient dy [T][d] (fp32) of y, with the
 * expert selection of the preceding moe_forward_train on this workspace (and
 * the same u, centroids and weights) held fixed:
 *   du          [T][d] fp32: through the residual, every expert and the router
 *               (gates g = s / sum s of the selected sigmoids s = Sigmoid(u . e))
 *   dcentroids  [N_r][d] fp32: through the router
 *   grads       fp32, the layouts of moe_weights; overwritten; experts that no
 *               token selected get zeros
 * Every sum runs in a fixed order (bit-reproducible).  `trace` (nullable)
 * records the MOE_STAGE_BWD_* stages.
 */
typedef struct {
  float* dw_gate_up;   /* [N_r][2I][d] */
  float* dw_down;      /* [N_r][d][I] */
  float* dws_gate_up;  /* [N_s][2I][d] (may be null when N_s = 0) */
  float* dws_down;     /* [N_s][d][I] */
} moe_weight_grads;
int moe_train_workspace_size(const moe_shape* shape, size_t* bytes);
int moe_forward_train(const moe_shape* shape, const void* u, const void* centroids, const float* bias,
                      const moe_weights* weights, void* y, void* workspace, size_t workspace_bytes,
                      const moe_trace* trace, hipStream_t stream);
int moe_backward(const moe_shape* shape, const void* u, const void* centroids, const moe_weights* weights,
                 const float* dy, float* du, float* dcentroids, const moe_weight_grads* grads, void* workspace,
                 size_t workspace_bytes, const moe_trace* trace, hipStream_t stream);

/*
 * Aux-loss-free bias update (xyznot summary, section 2: b_i is lowered by
 * gamma for an overloaded expert and raised by gamma for an underloaded one),
 * in place:
 *   bias[i] += gamma if n_routed * counts[i] <  total_assignments   (underloaded)
 *   bias[i] -= gamma if n_routed * counts[i] >  total_assignments   (overloaded)
 *   unchanged        if equal
 * total_assignments is T*K of the batch the counts were taken over (so the
 * threshold is the mean load T*K/N_r).  fp32 arithmetic; gamma = 0.001 in
 * DeepSeek-V3.
 */
int moe_update_bias(float* bias, const int32_t* counts, int32_t n_routed, int64_t total_assignments, float gamma,
                    hipStream_t stream);

/*
 * FP8 weight preparation (done once, offline; the 128x128 weight blocks of
 * the FP8 granularity in the xyznot summary's key-ideas list): quantise `n` row-major
 * [rows][cols] matrices (src_dtype F32 or BF16) to OCP E4M3 with one fp32
 * scale per 128x128 block: scale = amax/448, code = E4M3(x * (448/amax))
 * rounded to nearest even and saturated; scale 1 and zero codes for an
 * all-zero block.  codes: [n][rows][cols] uint8; scales: [n][rows/128][cols/128].
 * rows and cols must be multiples of 128.
 */
int moe_quantize_weight_e4m3(const void* src, int32_t src_dtype, int64_t n, int32_t rows, int32_t cols,
                             uint8_t* codes, float* scales, hipStream_t stream);

/*
 * FP8 activation quantisation, as moe_forward applies it to u (the 1x128
 * activation tiles of the same key-ideas list): per row, per 1x128 tile, scale = amax/448 and E4M3 codes (same rounding as above).
 * src: [rows][cols] bf16; codes: [rows][cols]; scales: [rows][cols/128].
 */
int moe_quantize_act_e4m3(const void* src, int32_t rows, int32_t cols, uint8_t* codes, float* scales,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
