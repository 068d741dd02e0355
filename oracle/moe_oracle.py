"""CPU oracle for the DeepSeekMoE layer forward pass and its aux-loss-free bias update.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it and shares no code with it.

It is a plain, slow, obviously-correct fp64 NumPy statement of what the layer
computes.  Sources (pages about the DeepSeek-V3 Technical Report):

* "DeepSeek-V3 Technical Report" summary on xyznot.com, section 2
  ("DeepSeekMoE with Auxiliary-Loss-Free Balancing"): the layer output
  h'_t = u_t + sum_i FFN^(s)_i(u_t) + sum_i g_{i,t} FFN^(r)_i(u_t), the
  affinity s_{i,t} = Sigmoid(u_t^T e_i), the biased top-K gate g'_{i,t}, the
  normalised gate g_{i,t}, and the bias rule b_i -/+ gamma with gamma = 0.001.
  Its key-ideas list gives the FP8 granularity: E4M3 everywhere, 1x128
  activation tiles, 128x128 weight blocks, FP32 promotion every N_c = 128.
* "DeepSeek-V3深度解析：FP8精度背后的科技力量" (wenxiaobai explainer), items
  "DeepSeekMoE架构" and Q2 (auxiliary-loss-free load balancing): the same h'
  and g' formulas.
* The why-be.co.kr paraphrase of the report's FP8 training section: the
  expert FFN is a SwiGLU operator; scaling is per group along the GEMM's
  inner dimension; partial sums are promoted to FP32.

Readings taken where the pages are silent:
* Expert FFN: W_down (SiLU(W_gate x) * (W_up x)), no biases; the gate/up
  weights are stored as one [2I, d] matrix, gate rows first.
* Gate normalisation: divide the K selected (unbiased) s by their sum.
* Top-K order: descending biased score v = s + b; exact ties go to the lower
  expert index.  Selection is global over all N_r experts, or, in the
  group-limited variant (the summary's all-to-all paragraph: a token lands
  on a median of 3.2 experts per node), confined to the topk_groups expert
  groups with the largest sums of their ceil(K / topk_groups) best v.
* Bias update: the load of expert i is its count over the batch of one
  routing call; it is overloaded when N_r * count_i > T * K, underloaded when
  below, unchanged at equality; b and gamma are fp32.
* FP8: scale = fl32(amax / 448), codes = E4M3_RNE_SATURATE(fl32(x * fl32(448 / amax))),
  scale 1 and codes 0 for an all-zero tile.  Both GEMMs of every expert are
  FP8; the router stays in the activation dtype; the residual u is unquantised;
  h is quantised 1x128 along I from fl32(h).
* FP8 backward (the Figure 6 passage: Fprop, Dgrad and Wgrad all in FP8):
  every operand is scaled per group of 128 along its GEMM's inner dimension,
  so the Dgrad activations (dY, [dG dU]) take 1x128 tiles along their
  columns, both Wgrad operands take 128x1 tiles along the rows (counted from
  each expert's first grouped row), and the weights keep their 128x128
  blocks.  Every row between two GEMMs (the cached G and U, dY, dH,
  [dG dU], H, x) is bf16, and each tensor is quantised from those values.

Everything is fp64 except where a reading fixes fp32 (scales, the bias).
"""

from __future__ import annotations

import math
from typing import Callable, Dict, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64
F32 = np.float32

GAMMA = F32(0.001)        # bias update speed (xyznot summary, section 2)
E4M3_MAX = 448.0          # largest finite OCP E4M3 value
QBLOCK = 128              # FP8 tile edge: 1x128 activations, 128x128 weights


# --------------------------------------------------------------------------
# Elementwise functions
# --------------------------------------------------------------------------

def sigmoid(z: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-z)) in fp64, the affinity nonlinearity of section 2."""
    z = np.asarray(z, dtype=F64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(a: np.ndarray) -> np.ndarray:
    """SiLU(a) = a * sigmoid(a), the gate nonlinearity of a SwiGLU FFN."""
    a = np.asarray(a, dtype=F64)
    return a * sigmoid(a)


# --------------------------------------------------------------------------
# Routing: affinities, biased top-K, gates  (xyznot summary, section 2)
# --------------------------------------------------------------------------

def affinities(u: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """s[t, i] = Sigmoid(u_t . e_i), fp64."""
    return sigmoid(np.asarray(u, F64) @ np.asarray(centroids, F64).T)


def select_topk(s: np.ndarray, bias: np.ndarray, k: int) -> Dict[str, np.ndarray]:
    """Biased top-K selection.

    v = s + b; a token keeps expert i when v_i is among its K largest.  The
    selected indices are listed in descending v, exact ties by ascending
    index.  ``gap`` is v_(K) - v_(K+1) (inf when K = N_r), the margin by
    which the K-th choice beat the first one left out.
    """
    s = np.asarray(s, F64)
    v = s + np.asarray(bias, F32).astype(F64)[None, :]
    T, n = v.shape
    idx = np.empty((T, k), dtype=np.int32)
    gap = np.full(T, np.inf)
    for t in range(T):
        order = np.argsort(-v[t], kind="stable")   # stable: equal v keep index order
        idx[t] = order[:k]
        if k < n:
            gap[t] = v[t, order[k - 1]] - v[t, order[k]]
    return {"idx": idx, "v": v, "gap": gap}


def group_scores(v: np.ndarray, n_groups: int, q: int) -> np.ndarray:
    """Score of each expert group for each token: the sum of the group's q
    largest biased scores v.  Groups are n_groups equal runs of consecutive
    experts (group g holds experts g*S .. g*S + S - 1, S = N_r / n_groups)."""
    T, n = v.shape
    S = n // n_groups
    out = np.empty((T, n_groups))
    for t in range(T):
        for g in range(n_groups):
            members = np.sort(v[t, g * S:(g + 1) * S])[::-1]
            out[t, g] = members[:q].sum()
    return out


def select_topk_grouped(s: np.ndarray, bias: np.ndarray, k: int, n_groups: int,
                        topk_groups: int) -> Dict[str, np.ndarray]:
    """Group-limited biased top-K (a token's experts come from at most
    topk_groups of the n_groups expert groups, e.g. the devices or nodes the
    experts live on).

    Reading (the pages give only the effect, a median of 3.2 experts per
    node, not the rule): a token ranks the groups by their score, the sum of
    the group's q = ceil(K / topk_groups) largest biased scores (at most the
    group size), keeps the topk_groups best groups (ties to the lower group
    index), then takes its K largest biased scores among those groups'
    experts, listed in descending v (ties to the lower expert index).
    ``gap`` is v_(K) - v_(K+1) among the kept groups' experts;
    ``group_gap`` is the margin of the last kept group's score over the
    first one left out (inf when every group is kept)."""
    s = np.asarray(s, F64)
    v = s + np.asarray(bias, F32).astype(F64)[None, :]
    T, n = v.shape
    S = n // n_groups
    q = min(math.ceil(k / topk_groups), S)
    gs = group_scores(v, n_groups, q)
    idx = np.empty((T, k), dtype=np.int32)
    gap = np.full(T, np.inf)
    group_gap = np.full(T, np.inf)
    groups = np.empty((T, topk_groups), dtype=np.int32)
    for t in range(T):
        gorder = np.argsort(-gs[t], kind="stable")           # stable: equal scores keep group order
        kept = np.sort(gorder[:topk_groups])
        groups[t] = gorder[:topk_groups]
        if topk_groups < n_groups:
            group_gap[t] = gs[t, gorder[topk_groups - 1]] - gs[t, gorder[topk_groups]]
        allowed = np.concatenate([np.arange(g * S, (g + 1) * S) for g in kept])   # ascending expert index
        order = allowed[np.argsort(-v[t, allowed], kind="stable")]
        idx[t] = order[:k]
        if k < len(allowed):
            gap[t] = v[t, order[k - 1]] - v[t, order[k]]
    return {"idx": idx, "v": v, "gap": gap, "group_gap": group_gap, "groups": groups, "group_score": gs}


def normalised_gates(s: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g_{t,k} = s_{t,idx[t,k]} / sum_k' s_{t,idx[t,k']}; the bias never enters."""
    sel = np.take_along_axis(np.asarray(s, F64), idx.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(u, centroids, bias, k: int, selection: Optional[np.ndarray] = None, n_groups: int = 1,
          topk_groups: int = 1) -> Dict[str, np.ndarray]:
    """Affinities, selection (or an imposed ``selection``), and gates.  With
    topk_groups < n_groups the selection is group-limited."""
    s = affinities(u, centroids)
    if topk_groups < n_groups:
        r = select_topk_grouped(s, bias, k, n_groups, topk_groups)
    else:
        r = select_topk(s, bias, k)
    if selection is not None:
        r["idx"] = np.asarray(selection, dtype=np.int32)
    r["s"] = s
    r["gate"] = normalised_gates(s, r["idx"])
    return r


# --------------------------------------------------------------------------
# Grouping tokens by expert (a counting sort, stable in token order)
# --------------------------------------------------------------------------

def group_by_expert(idx: np.ndarray, n_routed: int) -> Dict[str, np.ndarray]:
    """Expert-major row order, tokens ascending within an expert.

    counts[e] = number of (t, k) with idx[t, k] = e; offsets = exclusive
    prefix sum (length N_r + 1); perm_token[p] = token of grouped row p;
    pos[t, k] = grouped row of assignment (t, k).
    """
    T, k = idx.shape
    counts = np.zeros(n_routed, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            counts[idx[t, j]] += 1
    offsets = np.zeros(n_routed + 1, dtype=np.int64)
    for e in range(n_routed):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    perm_token = np.empty(T * k, dtype=np.int32)
    pos = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            p = fill[e]
            fill[e] += 1
            perm_token[p] = t
            pos[t, j] = p
    return {"counts": counts.astype(np.int32), "offsets": offsets.astype(np.int32),
            "perm_token": perm_token, "pos": pos}


# --------------------------------------------------------------------------
# Aux-loss-free bias update (xyznot summary, section 2; batch-level balance)
# --------------------------------------------------------------------------

def update_bias(bias: np.ndarray, counts: np.ndarray, total_assignments: int,
                gamma: np.float32 = GAMMA) -> np.ndarray:
    """b_i <- b_i - gamma if expert i is overloaded, + gamma if underloaded.

    Overloaded means count_i above the mean load T*K/N_r, decided exactly in
    integers as N_r * count_i > T * K.  Arithmetic in fp32.
    """
    bias = np.asarray(bias, F32)
    n = bias.shape[0]
    out = bias.copy()
    for i in range(n):
        diff = int(total_assignments) - n * int(counts[i])
        step = F32(0.0) if diff == 0 else (F32(gamma) if diff > 0 else -F32(gamma))
        out[i] = F32(bias[i] + step)
    return out


# --------------------------------------------------------------------------
# OCP FP8 E4M3 codec and fine-grained quantisation
# --------------------------------------------------------------------------

def _e4m3_value(code: np.ndarray) -> np.ndarray:
    """Value of OCP E4M3 codes: bias 7, 3 mantissa bits, no infinities,
    S.1111.111 = NaN, subnormals m/8 * 2^-6."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


_E4M3_TABLE = _e4m3_value(np.arange(256))      # the value of every code


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """Value of OCP E4M3 codes (a look-up in the table of all 256 values)."""
    return _E4M3_TABLE[np.asarray(code).astype(np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest E4M3 value, ties to the even code,
    saturating at +-448 (never producing NaN for finite input).  Returns
    uint8 codes.

    In the binade [2^E, 2^(E+1)), E >= -6, the E4M3 values are the multiples
    n * 2^(E-3), n = 8..15, with code 8 (E + 7) + (n - 8); below 2^-6 the
    subnormals are the multiples n * 2^-9, n = 0..7, with code n, which is
    the same formula at E = -6.  Rounding |x| to the nearest multiple of its
    binade's spacing, ties to the even multiple (an even n is an even code),
    is therefore round to nearest even on the E4M3 grid, and n = 16 (a value
    rounded up past its binade's top) lands on the next binade's first code.
    Codes past 126 (448) saturate.  Every step is exact in fp64."""
    x = np.asarray(x, dtype=F64)
    a = np.abs(x)
    _, e = np.frexp(a)                                 # a = f * 2^e, 0.5 <= f < 1 (e = 0 for a = 0)
    E = np.where(a < 2.0 ** -6, -6, e - 1)             # the binade of a; the subnormals share E = -6
    n = np.rint(np.ldexp(a, 3 - E)).astype(np.int64)   # a / 2^(E-3), ties to even
    code = np.minimum(8 * E + 48 + n, 126)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)   # sign kept, zero too


def _tile_scales(amax: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(scale, inverse scale) of each tile from its fp32 amax, both fp32:
    scale = fl32(amax / 448), inverse = fl32(448 / amax); an all-zero tile
    gets scale 1 and inverse 0 (zero codes)."""
    amax = np.asarray(amax, F32)
    zero = amax == 0
    safe = np.where(zero, F32(1.0), amax).astype(F32)
    scale = np.where(zero, F32(1.0), safe / F32(E4M3_MAX)).astype(F32)
    inv = np.where(zero, F32(0.0), F32(E4M3_MAX) / safe).astype(F32)
    return scale, inv


def quantize_act_1x128(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per row, per 128-column tile: codes [R, C] uint8 and scales [R, C/128] fp32.
    Each tile's codes are E4M3(fl32(x * inverse scale))."""
    x = np.asarray(x, F32)
    R, C = x.shape
    assert C % QBLOCK == 0
    tiles = x.reshape(R, C // QBLOCK, QBLOCK)                 # tile [r, j] = x[r, 128 j : 128 (j + 1)]
    scale, inv = _tile_scales(np.abs(tiles).max(axis=2) if R else np.zeros((0, C // QBLOCK), F32))
    q = e4m3_encode((tiles * inv[:, :, None]).astype(F32))
    return q.reshape(R, C), scale


def quantize_weight_128x128(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per 128x128 block: codes [R, C] uint8 and scales [R/128, C/128] fp32.
    Each block's codes are E4M3(fl32(w * inverse scale))."""
    w = np.asarray(w, F32)
    R, C = w.shape
    assert R % QBLOCK == 0 and C % QBLOCK == 0
    blocks = w.reshape(R // QBLOCK, QBLOCK, C // QBLOCK, QBLOCK)   # block [i, j] = blocks[i, :, j, :]
    scale, inv = _tile_scales(np.abs(blocks).max(axis=(1, 3)))
    q = e4m3_encode((blocks * inv[:, None, :, None]).astype(F32))
    return q.reshape(R, C), scale


def quantize_act_128x1(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per column, per 128-row tile counted from row 0 (the last tile may be
    short): codes [R, C] uint8 and scales [ceil(R/128), C] fp32.  The 1x128
    tiling of x's transpose: the tiles run along the rows, the inner
    dimension of a GEMM that contracts over them (a weight gradient)."""
    x = np.asarray(x, F32)
    R, C = x.shape
    Rp = -(-R // QBLOCK) * QBLOCK
    xt = np.zeros((C, Rp), F32)                 # zero rows do not change a tile's amax
    xt[:, :R] = x.T
    q, sc = quantize_act_1x128(xt)
    return q[:, :R].T.copy(), sc.T.copy()


def dequantize_act_128x1(q: np.ndarray, sc: np.ndarray) -> np.ndarray:
    R, C = q.shape
    rows = np.arange(R) // QBLOCK
    return e4m3_decode(q) * sc.astype(F64)[rows, :]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of fl32(x), as fp64: bit 16 of
    the fp32 pattern is the kept LSB; adding 0x7FFF plus that bit and
    clearing the low half rounds to nearest, ties to even."""
    b = np.asarray(x, F32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return b.view(F32).astype(F64)


def dequantize_act(q: np.ndarray, sc: np.ndarray) -> np.ndarray:
    R, C = q.shape
    return (e4m3_decode(q).reshape(R, C // QBLOCK, QBLOCK) * sc.astype(F64)[:, :, None]).reshape(R, C)


def dequantize_weight(q: np.ndarray, sc: np.ndarray) -> np.ndarray:
    R, C = q.shape
    blocks = e4m3_decode(q).reshape(R // QBLOCK, QBLOCK, C // QBLOCK, QBLOCK)
    return (blocks * sc.astype(F64)[:, None, :, None]).reshape(R, C)


# --------------------------------------------------------------------------
# Expert FFN and the layer
# --------------------------------------------------------------------------

def swiglu_ffn(x: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """FFN(x) = W_down (SiLU(W_gate x) * (W_up x)); w_gate_up is [2I, d], gate rows first."""
    x = np.asarray(x, F64)
    wgu = np.asarray(w_gate_up, F64)
    I = wgu.shape[0] // 2
    h = silu(x @ wgu[:I].T) * (x @ wgu[I:].T)
    return h @ np.asarray(w_down, F64).T


def swiglu_ffn_fp8(x_deq: np.ndarray, wgu_q, wgu_s, wd_q, wd_s) -> np.ndarray:
    """The FP8 expert: dequantised operands, fp64 products; h re-quantised 1x128."""
    wgu = dequantize_weight(wgu_q, wgu_s)
    I = wgu.shape[0] // 2
    h = silu(x_deq @ wgu[:I].T) * (x_deq @ wgu[I:].T)
    hq, hs = quantize_act_1x128(h.astype(F32))
    return dequantize_act(hq, hs) @ dequantize_weight(wd_q, wd_s).T


ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray]]


def layer_forward(u: np.ndarray, centroids: np.ndarray, bias: np.ndarray, k: int,
                  routed: ExpertFn, n_routed: int, shared: Sequence[Tuple[np.ndarray, np.ndarray]],
                  selection: Optional[np.ndarray] = None, fp8: bool = False,
                  fp8_weights: Optional[Callable[[str, int], Tuple]] = None, n_groups: int = 1,
                  topk_groups: int = 1) -> Dict[str, np.ndarray]:
    """h'_t = u_t + sum_s FFN^(s)_s(u_t) + sum_k g_{t,k} FFN^(r)_{idx[t,k]}(u_t).

    ``routed(e)`` returns expert e's (w_gate_up [2I, d], w_down [d, I]) as
    float arrays (exact upcasts of the stored values); ``shared`` lists the
    shared experts the same way.  With ``fp8``, the expert weights are
    quantised 128x128 here (or taken pre-quantised from ``fp8_weights(kind, e)``
    returning (gu_q, gu_s, d_q, d_s)), u is quantised 1x128 for the expert
    GEMMs, and the router and the residual use the unquantised u.  With
    topk_groups < n_groups the routing is group-limited (select_topk_grouped).
    """
    u64 = np.asarray(u, F64)
    r = route(u64, centroids, bias, k, selection, n_groups, topk_groups)
    idx, gate = r["idx"], r["gate"]
    T, d = u64.shape

    if fp8:
        uq, us = quantize_act_1x128(np.asarray(u, F32))
        x_in = dequantize_act(uq, us)
        r["u_q"], r["u_scale"] = uq, us

        def run(kind, e, wgu, wd, x):
            if fp8_weights is not None:
                gq, gs, dq, ds = fp8_weights(kind, e)
            else:
                gq, gs = quantize_weight_128x128(wgu)
                dq, ds = quantize_weight_128x128(wd)
            return swiglu_ffn_fp8(x, gq, gs, dq, ds)
    else:
        x_in = u64

        def run(kind, e, wgu, wd, x):
            return swiglu_ffn(x, wgu, wd)

    shared_sum = np.zeros((T, d), F64)
    for si, (wgu, wd) in enumerate(shared):
        shared_sum += run("shared", si, wgu, wd, x_in)

    routed_sum = np.zeros((T, d), F64)
    for e in range(n_routed):
        tok, slot = np.nonzero(idx == e)
        if tok.size == 0:
            continue
        wgu, wd = routed(e)
        out = run("routed", e, wgu, wd, x_in[tok])
        routed_sum[tok] += gate[tok, slot][:, None] * out

    r["y"] = u64 + shared_sum + routed_sum
    r["shared_sum"] = shared_sum
    r["routed_sum"] = routed_sum
    return r


# --------------------------------------------------------------------------
# Backward pass (the report's FP8 training section, as paraphrased on
# why-be.co.kr: the Linear operator's three GEMMs are Fprop, Dgrad and Wgrad,
# and the inputs of the SwiGLU operator are cached and its output recomputed
# in the backward pass).  Gradients of the forward above with the expert
# selection held fixed (the top-K is piecewise constant); fp64 throughout.
# --------------------------------------------------------------------------

def silu_grad(a: np.ndarray) -> np.ndarray:
    """d SiLU(a) / da = sigma(a) * (1 + a * (1 - sigma(a)))."""
    a = np.asarray(a, F64)
    sg = sigmoid(a)
    return sg * (1.0 + a * (1.0 - sg))


def swiglu_ffn_backward(x: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray,
                        dout: np.ndarray) -> Dict[str, np.ndarray]:
    """Backward of FFN(x) = W_down (SiLU(G) * U), G = x W_gate^T, U = x W_up^T,
    for the upstream gradient ``dout`` [n, d] of its n rows:
        H = SiLU(G) * U (recomputed from the cached G, U)
        dH = dout W_down,              dW_down = dout^T H
        dG = dH * U * SiLU'(G),        dU = dH * SiLU(G)
        dx = dG W_gate + dU W_up,      dW_gate = dG^T x,  dW_up = dU^T x
    Returns dx [n, d], dW_gate_up [2I, d] (gate rows first), dW_down [d, I]."""
    x = np.asarray(x, F64)
    wgu = np.asarray(w_gate_up, F64)
    wd = np.asarray(w_down, F64)
    dout = np.asarray(dout, F64)
    I = wgu.shape[0] // 2
    G = x @ wgu[:I].T
    U = x @ wgu[I:].T
    H = silu(G) * U
    dH = dout @ wd
    dG = dH * U * silu_grad(G)
    dU = dH * silu(G)
    dGU = np.concatenate([dG, dU], axis=1)
    return {"dx": dGU @ wgu, "dW_gate_up": dGU.T @ x, "dW_down": dout.T @ H}


def swiglu_ffn_backward_fp8(x: np.ndarray, x_deq: np.ndarray, wgu_q, wgu_s, wd_q, wd_s,
                            dout: np.ndarray) -> Dict[str, np.ndarray]:
    """The FP8 backward of one expert over its n rows (in grouped order): the
    same steps as swiglu_ffn_backward with every GEMM on E4M3 operands and
    fp64 products of the dequantised values (FP32 promotion per 128-element
    block, exact here).  Scaling is per group of 128 along each GEMM's inner
    dimension:
        Dgrad  dH = q(dout) Wd            dout tiled 1x128 along d
               dx = q([dG dU]) Wgu        [dG dU] tiled 1x128 along 2I
        Wgrad  dW_down = q(dout)^T q(H)           both tiled 128x1 along the
               dW_gate_up = q([dG dU])^T q(x)     rows, from the group's first
    The weights keep their forward 128x128 blocks (read transposed).  G and U
    are the FP8 forward's products from the dequantised input x_deq, cached
    as bf16 (the cached SwiGLU inputs); H = SiLU(G) U is recomputed.  Every
    row between two GEMMs is bf16 (dout, the Dgrad output dH, [dG dU], H and
    x), so each quantiser decides its codes from the bf16 values the kernels
    store."""
    wgu = dequantize_weight(wgu_q, wgu_s)
    wd = dequantize_weight(wd_q, wd_s)
    I = wgu.shape[0] // 2
    x_deq = np.asarray(x_deq, F64)
    G = round_bf16(x_deq @ wgu[:I].T)
    U = round_bf16(x_deq @ wgu[I:].T)
    dout_b = round_bf16(dout)
    dH = round_bf16(dequantize_act(*quantize_act_1x128(dout_b)) @ wd)
    dG = dH * U * silu_grad(G)
    dU = dH * silu(G)
    dGU_b = round_bf16(np.concatenate([dG, dU], axis=1))
    H_b = round_bf16(silu(G) * U)
    dx = dequantize_act(*quantize_act_1x128(dGU_b)) @ wgu
    dW_down = dequantize_act_128x1(*quantize_act_128x1(dout_b)).T @ dequantize_act_128x1(*quantize_act_128x1(H_b))
    dW_gu = (dequantize_act_128x1(*quantize_act_128x1(dGU_b)).T
             @ dequantize_act_128x1(*quantize_act_128x1(round_bf16(x))))
    return {"dx": dx, "dW_gate_up": dW_gu, "dW_down": dW_down}


def layer_backward(u: np.ndarray, centroids: np.ndarray, bias: np.ndarray, k: int,
                   routed: ExpertFn, n_routed: int, shared: Sequence[Tuple[np.ndarray, np.ndarray]],
                   dy: np.ndarray, selection: Optional[np.ndarray] = None, n_groups: int = 1,
                   topk_groups: int = 1, weight_grads: bool = True, fp8: bool = False,
                   fp8_weights: Optional[Callable[[str, int], Tuple]] = None) -> Dict[str, np.ndarray]:
    """Gradients of h' = u + sum_s FFN_s(u) + sum_k g_k FFN_{e_k}(u) for the
    upstream gradient dy [T, d], the selection held fixed:
      routed expert e, its rows (t, k): upstream g_{t,k} dy_t through FFN_e;
      shared expert s: upstream dy_t through FFN_s;
      gates g_k = s_k / S (S = sum of the selected s): dg_k = dy_t . FFN_{e_k}(u_t),
        ds_j = (dg_j - sum_k g_k dg_k) / S, and through s = Sigmoid(z),
        dz_j = ds_j s_j (1 - s_j), with z_j = u_t . e_j;
      du_t = dy_t + sum_s dx_s + sum_k dx_{t,k} + sum_k dz_k e_{e_k};
      dE_e = sum over e's rows of dz u_t.
    Returns du [T, d], dE [N_r, d], dg and dz [T, K], and (weight_grads)
    dW_gate_up / dW_down: dicts expert -> gradient (experts without rows
    have zero gradients and are left out), dWs_gate_up / dWs_down: lists
    over the shared experts.

    With ``fp8`` the layer is the FP8 one of layer_forward (weights quantised
    128x128 here or taken from ``fp8_weights``, u quantised 1x128 for the
    expert GEMMs) and every expert's backward is swiglu_ffn_backward_fp8;
    dg uses the FP8 expert outputs.  The router's gradient (dz, dE and the
    dz e terms of du) is the same in both."""
    u64 = np.asarray(u, F64)
    E64 = np.asarray(centroids, F64)
    dy = np.asarray(dy, F64)
    r = route(u64, E64, bias, k, selection, n_groups, topk_groups)
    idx, gate, s = r["idx"], r["gate"], r["s"]
    T, d = u64.shape
    if fp8:
        x_deq = dequantize_act(*quantize_act_1x128(np.asarray(u, F32)))

        def expert(kind, e, wgu, wd, rows, dout):
            if fp8_weights is not None:
                gq, gs, dq, ds = fp8_weights(kind, e)
            else:
                gq, gs = quantize_weight_128x128(wgu)
                dq, ds = quantize_weight_128x128(wd)
            ye = swiglu_ffn_fp8(x_deq[rows], gq, gs, dq, ds)
            return ye, swiglu_ffn_backward_fp8(u64[rows], x_deq[rows], gq, gs, dq, ds, dout)
    else:
        def expert(kind, e, wgu, wd, rows, dout):
            x = u64[rows]
            return swiglu_ffn(x, wgu, wd), swiglu_ffn_backward(x, wgu, wd, dout)
    du = dy.copy()
    dWs_gu, dWs_d = [], []
    for si, (wgu, wd) in enumerate(shared):
        _, b = expert("shared", si, wgu, wd, np.arange(T), dy)
        du += b["dx"]
        dWs_gu.append(b["dW_gate_up"])
        dWs_d.append(b["dW_down"])
    dg = np.zeros((T, k))
    dW_gu, dW_d = {}, {}
    for e in range(n_routed):
        tok, slot = np.nonzero(idx == e)
        if tok.size == 0:
            continue
        wgu, wd = routed(e)
        # FFN_e(u_t) of the rows, and the backward with upstream g dy
        ye, b = expert("routed", e, wgu, wd, tok, gate[tok, slot][:, None] * dy[tok])
        dg[tok, slot] = np.sum(dy[tok] * ye, axis=1)
        du[tok] += b["dx"]
        if weight_grads:
            dW_gu[e] = b["dW_gate_up"]
            dW_d[e] = b["dW_down"]
    sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    S = sel.sum(axis=1, keepdims=True)
    ds = (dg - np.sum(gate * dg, axis=1, keepdims=True)) / S
    dz = ds * sel * (1.0 - sel)
    dE = np.zeros((n_routed, d))
    for t in range(T):
        for j in range(k):
            du[t] += dz[t, j] * E64[idx[t, j]]
            dE[idx[t, j]] += dz[t, j] * u64[t]
    return {"du": du, "dE": dE, "dg": dg, "dz": dz, "idx": idx, "gate": gate,
            "dW_gate_up": dW_gu, "dW_down": dW_d, "dWs_gate_up": dWs_gu, "dWs_down": dWs_d}


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("annotations", "math")]
