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
  expert index.  Selection is global over all N_r experts.
* Bias update: the load of expert i is its count over the batch of one
  routing call; it is overloaded when N_r * count_i > T * K, underloaded when
  below, unchanged at equality; b and gamma are fp32.
* FP8: scale = fl32(amax / 448), codes = E4M3_RNE_SATURATE(fl32(x * fl32(448 / amax))),
  scale 1 and codes 0 for an all-zero tile.  Both GEMMs of every expert are
  FP8; the router stays in the activation dtype; the residual u is unquantised;
  h is quantised 1x128 along I from fl32(h).

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


def normalised_gates(s: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g_{t,k} = s_{t,idx[t,k]} / sum_k' s_{t,idx[t,k']}; the bias never enters."""
    sel = np.take_along_axis(np.asarray(s, F64), idx.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(u, centroids, bias, k: int, selection: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Affinities, selection (or an imposed ``selection``), and gates."""
    s = affinities(u, centroids)
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

def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """Value of OCP E4M3 codes: bias 7, 3 mantissa bits, no infinities,
    S.1111.111 = NaN, subnormals m/8 * 2^-6."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


_POS_VALUES = e4m3_decode(np.arange(0, 127))   # the finite non-negative values, ascending


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest E4M3 value, ties to the even code,
    saturating at +-448 (never producing NaN).  Returns uint8 codes."""
    x = np.asarray(x, dtype=F64)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 1, 126)
    lo = hi - 1
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 126, code)                  # saturate
    code = np.where(a <= _POS_VALUES[0], 0, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)   # sign kept, zero too


def _tile_scale(amax: np.float32) -> Tuple[np.float32, np.float32]:
    """(scale, inverse scale) of one tile, both fp32."""
    if amax == 0:
        return F32(1.0), F32(0.0)
    return F32(F32(amax) / F32(E4M3_MAX)), F32(F32(E4M3_MAX) / F32(amax))


def quantize_act_1x128(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per row, per 128-column tile: codes [R, C] uint8 and scales [R, C/128] fp32."""
    x = np.asarray(x, F32)
    R, C = x.shape
    assert C % QBLOCK == 0
    q = np.empty((R, C), dtype=np.uint8)
    sc = np.empty((R, C // QBLOCK), dtype=F32)
    for r in range(R):
        for j in range(C // QBLOCK):
            tile = x[r, j * QBLOCK:(j + 1) * QBLOCK]
            scale, inv = _tile_scale(F32(np.max(np.abs(tile))))
            q[r, j * QBLOCK:(j + 1) * QBLOCK] = e4m3_encode((tile * inv).astype(F32))
            sc[r, j] = scale
    return q, sc


def quantize_weight_128x128(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per 128x128 block: codes [R, C] uint8 and scales [R/128, C/128] fp32."""
    w = np.asarray(w, F32)
    R, C = w.shape
    assert R % QBLOCK == 0 and C % QBLOCK == 0
    q = np.empty((R, C), dtype=np.uint8)
    sc = np.empty((R // QBLOCK, C // QBLOCK), dtype=F32)
    for i in range(R // QBLOCK):
        for j in range(C // QBLOCK):
            blk = w[i * QBLOCK:(i + 1) * QBLOCK, j * QBLOCK:(j + 1) * QBLOCK]
            scale, inv = _tile_scale(F32(np.max(np.abs(blk))))
            q[i * QBLOCK:(i + 1) * QBLOCK, j * QBLOCK:(j + 1) * QBLOCK] = e4m3_encode((blk * inv).astype(F32))
            sc[i, j] = scale
    return q, sc


def dequantize_act(q: np.ndarray, sc: np.ndarray) -> np.ndarray:
    return e4m3_decode(q) * np.repeat(sc.astype(F64), QBLOCK, axis=1)


def dequantize_weight(q: np.ndarray, sc: np.ndarray) -> np.ndarray:
    s = np.repeat(np.repeat(sc.astype(F64), QBLOCK, axis=0), QBLOCK, axis=1)
    return e4m3_decode(q) * s


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
                  fp8_weights: Optional[Callable[[str, int], Tuple]] = None) -> Dict[str, np.ndarray]:
    """h'_t = u_t + sum_s FFN^(s)_s(u_t) + sum_k g_{t,k} FFN^(r)_{idx[t,k]}(u_t).

    ``routed(e)`` returns expert e's (w_gate_up [2I, d], w_down [d, I]) as
    float arrays (exact upcasts of the stored values); ``shared`` lists the
    shared experts the same way.  With ``fp8``, the expert weights are
    quantised 128x128 here (or taken pre-quantised from ``fp8_weights(kind, e)``
    returning (gu_q, gu_s, d_q, d_s)), u is quantised 1x128 for the expert
    GEMMs, and the router and the residual use the unquantised u.
    """
    u64 = np.asarray(u, F64)
    r = route(u64, centroids, bias, k, selection)
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


def near_tie_mask(gap: np.ndarray, band: float = 1e-6) -> np.ndarray:
    """Tokens whose K-th and (K+1)-th biased scores lie within ``band``."""
    return np.asarray(gap) <= band


def flops_per_token(d: int, n_routed: int, inter: int, k: int, n_shared: int) -> int:
    return 2 * d * n_routed + 6 * d * inter * (k + n_shared)


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("annotations", "math")]
