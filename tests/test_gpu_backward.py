"""GPU parity of the layer backward (moe_forward_train + moe_backward, bf16
and FP8, through the C ABI) against the oracle's fp64 layer_backward.

Bar (the pages state none for the backward; derived from the arithmetic):
the backward's GEMMs take bf16 operands (the scaled upstream rows, the
cached G and U, the SwiGLU gradients, the recomputed H), each rounded once
(unit roundoff 2^-9, error std 2^-9/sqrt(3)), about four roundings on the
longest path into a weight gradient, so a normwise relative error near
sqrt(4) * 2^-9 / sqrt(3) ~ 2e-3 is expected; the bound is 1e-2, per block,
so that a defect confined to one tile or row cannot hide in an average:
every 256 x 256 tile of each expert's dW_gate_up and dW_down, and every row
of du, within ||grad_gpu - grad_oracle||_F <= 1e-2 ||grad_oracle||_F; each
row of dcentroids within 1e-2 of the magnitude of its terms (see _de_err:
the router's ds is a difference that can cancel).  Experts that no token
selected must get exactly zero.  The oracle
adopts the GPU's expert selection (its own routing is checked by the
forward tests).

FP8 (e4m3 weights): the oracle runs the same FP8 backward -- the same
tiles, and codes decided from the same bf16 rows (the cached G and U, dY,
dH, [dG dU], H, x are bf16 on both sides) -- so a code differs only where
the GPU's fp32 and the oracle's fp64 evaluation of a row land on different
bf16 values (relative error ~1e-6 against a bf16 spacing of 2^-8: about one
element in 4000).  Such a flip moves one code, unless the element is the
largest of its 1x128 or 128x1 tile: then the tile's scale moves and every
code of the tile is decided afresh, each by up to one E4M3 step (2^-4).  In
an expert with few rows one such tile is a large share of a weight
gradient's block: the oracle against itself, with dy perturbed by 1e-7 to
1e-6 relative (the size of fp32 evaluation error), drifts by up to 1.3e-2
per block on the random shapes below.  The FP8 bound is 3e-2 per block.
"""

import numpy as np
import pytest
import torch

import mixture_experts_layer_deepseekmoe_amd as moe
from moe_workloads import CONFIGS, PARITY_CONFIGS, make_inputs, to_numpy_f32
from oracle import moe_oracle as O
from tests.parity import check_routing, expert_fns, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-2
TOL8 = 3e-2


def _maxrel(got: np.ndarray, ref: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    return float(np.abs(got.astype(np.float64) - ref).max()) / (rms or 1.0)


def _blocks(a: np.ndarray, bm: int, bn: int):
    """Blocks of the last two axes (bm x bn; bm = 1 for rows)."""
    a = a.reshape((-1,) + a.shape[-2:])
    for m in range(a.shape[0]):
        for i in range(0, a.shape[1], bm):
            for j in range(0, a.shape[2], bn):
                yield m, i, j, a[m, i:i + bm, j:j + bn]


def _err(got: np.ndarray, ref: np.ndarray, bm: int = 256, bn: int = 256) -> float:
    """The largest normwise relative error over blocks: max over blocks of
    ||grad_gpu - grad_oracle||_F / ||grad_oracle||_F (256 x 256 tiles of a
    weight gradient, single rows of du and dcentroids)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    worst = 0.0
    for (_, _, _, g), (_, _, _, r) in zip(_blocks(got, bm, bn), _blocks(ref, bm, bn)):
        nr = float(np.linalg.norm(r))
        worst = max(worst, float(np.linalg.norm(g - r)) / (nr or 1.0))
    return worst


def _de_err(got: np.ndarray, ref: dict, u: np.ndarray, E: np.ndarray, n_routed: int) -> float:
    """Worst row of dcentroids, its error measured against the magnitude of
    the terms it is made of.  ds_k = (dg_k - sum_j g_j dg_j) / S is a
    difference, and where it cancels (an expert with a single row, a token
    whose dg_k sits near the gated mean) its relative error grows by the
    cancellation factor whatever the precision; so the yardstick is
    |dz|-magnitude_k = (|dg_k| + sum_j g_j |dg_j|) / S * s_k (1 - s_k),
    summed like dz into each row: mag_e = sum over e's rows of mag_k |u_t|.
    Returns max over experts of ||dE_gpu,e - dE_e|| / ||mag_e||."""
    idx, g, dg = ref["idx"], ref["gate"], ref["dg"]
    s = np.take_along_axis(O.affinities(u, E), idx.astype(np.int64), axis=1)
    S = s.sum(axis=1, keepdims=True)
    mag = (np.abs(dg) + np.sum(g * np.abs(dg), axis=1, keepdims=True)) / S * s * (1 - s)
    magE = np.zeros((n_routed, u.shape[1]))
    for t in range(idx.shape[0]):
        for k in range(idx.shape[1]):
            magE[idx[t, k]] += mag[t, k] * np.abs(u[t].astype(np.float64))
    worst = 0.0
    for e in range(n_routed):
        nm = float(np.linalg.norm(magE[e]))
        if nm > 0:
            worst = max(worst, float(np.linalg.norm(got[e] - ref["dE"][e])) / nm)
        else:
            assert not got[e].any()
    return worst


def _dy(cfg):
    g = torch.Generator().manual_seed(1000 + cfg.cfg_id)
    return torch.randn((cfg.T, cfg.d), generator=g, dtype=torch.float32)


def _train_step(cfg, inp, dy, weights=None):
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = (t.to(DEV).contiguous() for t in (inp.u, inp.centroids, inp.bias))
    w = moe.prepare_weights(cfg, inp, train=True) if weights is None else weights
    ws = moe.alloc_train_workspace(shape)
    y = moe.moe_forward_train(shape, u, E, b, w, ws)
    du, dE, grads = moe.moe_backward(shape, u, E, w, dy.to(DEV).contiguous(), ws)
    torch.cuda.synchronize()
    return y, du, dE, grads, ws, w


def _compare(cfg, inp, dy_t, du, dE, grads, gi):
    u, E, b = to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy()
    routed, shared = expert_fns(inp, False)
    ref = O.layer_backward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared, dy_t.numpy(), selection=gi,
                           fp8=cfg.w_dtype == "e4m3")
    errs = {"du": _err(du.cpu().numpy(), ref["du"], 1, du.shape[1]),
            "dE": _de_err(dE.cpu().numpy(), ref, u, E, cfg.n_routed)}
    say("  max|d|/rms (information): du %.2e dE %.2e" % (_maxrel(du.cpu().numpy(), ref["du"]),
                                                        _maxrel(dE.cpu().numpy(), ref["dE"])))
    dgu = grads.dw_gate_up.cpu().numpy()
    dd = grads.dw_down.cpu().numpy()
    touched = sorted(ref["dW_gate_up"])
    untouched = [e for e in range(cfg.n_routed) if e not in ref["dW_gate_up"]]
    assert not dgu[untouched].any() and not dd[untouched].any(), "experts without rows must get zero gradients"
    if touched:
        errs["dW_gate_up"] = _err(dgu[touched], np.stack([ref["dW_gate_up"][e] for e in touched]))
        errs["dW_down"] = _err(dd[touched], np.stack([ref["dW_down"][e] for e in touched]))
    for s in range(cfg.n_shared):
        errs[f"dWs_gate_up{s}"] = _err(grads.dws_gate_up[s].cpu().numpy(), ref["dWs_gate_up"][s])
        errs[f"dWs_down{s}"] = _err(grads.dws_down[s].cpu().numpy(), ref["dWs_down"][s])
    return errs, len(untouched)


BWD_CASES = {
    "small_bf16": PARITY_CONFIGS["small_bf16"],
    "small_bf16_ns2": PARITY_CONFIGS["small_bf16_ns2"],
    "small_bf16_ns0": PARITY_CONFIGS["small_bf16_ns0"],
    "dense_k_eq_n": PARITY_CONFIGS["dense_k_eq_n"],
    "one_token": PARITY_CONFIGS["one_token"],
    "wide_router": PARITY_CONFIGS["wide_router"],
    "small_bf16_g4k2": PARITY_CONFIGS["small_bf16"].replace(name="small_bf16_g4k2", n_groups=4, topk_groups=2),
}


@pytest.mark.parametrize("name", list(BWD_CASES))
def test_backward_parity(name):
    cfg = BWD_CASES[name]
    say(f"case: moe_forward_train + moe_backward {name}")
    inp = make_inputs(cfg, 0)
    dy = _dy(cfg)
    y, du, dE, grads, ws, w = _train_step(cfg, inp, dy)
    # the training forward computes the same y as moe_forward
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = (t.to(DEV).contiguous() for t in (inp.u, inp.centroids, inp.bias))
    routing = moe.alloc_routing(shape)
    y_inf = moe.moe_forward(shape, u, E, b, w, routing=routing)
    torch.cuda.synchronize()
    assert torch.equal(y, y_inf)
    check_routing(routing, to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy(), cfg.top_k,
                  cfg.n_routed, cfg.n_groups, cfg.topk_groups)
    errs, empty = _compare(cfg, inp, dy, du, dE, grads, routing["topk_idx"].cpu().numpy())
    say("  worst block ||d||/||ref||: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f"; {empty} experts without rows")
    for k, v in errs.items():
        assert v <= TOL, (k, v)


def _random_train_shapes(n=8, seed=77):
    """Seeded small training shapes: bf16 or e4m3 weights, ragged T, N_r on
    both sides of the 128-row FP8 code blocks' group count, K up to 16, 0-3
    shared experts, d and I any multiple of 64 (bf16) or 128 (e4m3), bf16 or
    fp32 y; sizes bounded so the fp64 oracle backward stays quick."""
    rs = np.random.RandomState(seed)
    out = []
    for i in range(n):
        w = ["bf16", "e4m3"][i % 2]
        kmult = 64 if w == "bf16" else 128
        n_routed = int(rs.choice([int(rs.randint(1, 40)), int(rs.randint(40, 300))]))
        top_k = int(rs.randint(1, min(16, n_routed) + 1))
        d = kmult * int(rs.randint(1, 768 // kmult + 1))
        inter = kmult * int(rs.randint(1, 512 // kmult + 1))
        while n_routed * d * inter > (1 << 23):   # keep the oracle's weights small
            if d >= inter and d > kmult:
                d -= kmult
            elif inter > kmult:
                inter -= kmult
            else:
                n_routed = max(top_k, n_routed // 2)
        T = int(rs.randint(1, 600))
        out.append(PARITY_CONFIGS["small_bf16"].replace(
            name=f"train{i}_{w}_T{T}_d{d}_I{inter}_Nr{n_routed}_K{top_k}", T=T, d=d, n_routed=n_routed,
            n_shared=int(rs.randint(0, 4)), inter=inter, top_k=top_k, w_dtype=w,
            out_dtype=["f32", "bf16"][rs.randint(2)], w_std=0.03, e_std=0.05, b_std=0.02, cfg_id=200 + i))
    return out


RANDOM_TRAIN_SHAPES = _random_train_shapes()


@pytest.mark.parametrize("cfg", RANDOM_TRAIN_SHAPES, ids=[c.name for c in RANDOM_TRAIN_SHAPES])
def test_backward_random_shapes(cfg):
    """Seeded random training shapes, bf16 and FP8, against the oracle's
    backward (bf16 or FP8) at the same per-block bound."""
    say(f"case: moe_forward_train + moe_backward {cfg.name}")
    inp = make_inputs(cfg, 0)
    dy = _dy(cfg)
    y, du, dE, grads, ws, w = _train_step(cfg, inp, dy)
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = (t.to(DEV).contiguous() for t in (inp.u, inp.centroids, inp.bias))
    routing = moe.alloc_routing(shape)
    y_inf = moe.moe_forward(shape, u, E, b, w, routing=routing)
    torch.cuda.synchronize()
    assert torch.equal(y, y_inf)
    errs, empty = _compare(cfg, inp, dy, du, dE, grads, routing["topk_idx"].cpu().numpy())
    say("  worst block ||d||/||ref||: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f"; {empty} experts without rows")
    for k, v in errs.items():
        assert v <= (TOL8 if cfg.w_dtype == "e4m3" else TOL), (k, v)


def test_backward_deterministic_and_empty_batch():
    cfg = PARITY_CONFIGS["small_bf16_ns2"]
    say("case: moe_backward determinism, and T = 0")
    inp = make_inputs(cfg, 0)
    dy = _dy(cfg)
    _, du1, dE1, g1, _, w = _train_step(cfg, inp, dy)
    _, du2, dE2, g2, _, _ = _train_step(cfg, inp, dy, w)
    assert torch.equal(du1, du2) and torch.equal(dE1, dE2)
    for a, b in ((g1.dw_gate_up, g2.dw_gate_up), (g1.dw_down, g2.dw_down), (g1.dws_gate_up, g2.dws_gate_up),
                 (g1.dws_down, g2.dws_down)):
        assert torch.equal(a, b)
    # an empty batch: every gradient is zero
    c0 = cfg.replace(T=0)
    inp0 = make_inputs(c0, 0)
    _, du0, dE0, g0, _, _ = _train_step(c0, inp0, torch.zeros((0, c0.d)))
    assert du0.shape == (0, c0.d) and not dE0.any()
    assert not g0.dw_gate_up.any() and not g0.dw_down.any() and not g0.dws_gate_up.any() and not g0.dws_down.any()


def test_backward_full_d2048():
    """The d = 2048 layer (T = 4096, 64 + 2 experts, K = 6; every expert spans
    two m-tiles) in full: every gradient against the oracle."""
    cfg = CONFIGS["bf16_d2048"]
    say("case: moe_backward bf16_d2048 full size, every gradient")
    inp = make_inputs(cfg, 0)
    dy = _dy(cfg)
    y, du, dE, grads, ws, w = _train_step(cfg, inp, dy)
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = (t.to(DEV).contiguous() for t in (inp.u, inp.centroids, inp.bias))
    routing = moe.moe_route(shape, u, E, b)
    torch.cuda.synchronize()
    errs, empty = _compare(cfg, inp, dy, du, dE, grads, routing["topk_idx"].cpu().numpy())
    say("  worst block ||d||/||ref||: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    del w, ws, grads
    torch.cuda.empty_cache()


def test_backward_full_d7168_sampled():
    """The DeepSeek-V3 layer (T = 8192, d = 7168, 256 + 1 experts, K = 8):
    du on sampled tokens, and dW of the shared expert and of sampled routed
    experts (the largest, the smallest and a median one), against the oracle."""
    cfg = CONFIGS["bf16_d7168"]
    say("case: moe_backward bf16_d7168 full size, sampled")
    inp = make_inputs(cfg, 0, weights_device=DEV)
    dy = _dy(cfg)
    y, du, dE, grads, ws, w = _train_step(cfg, inp, dy)
    assert torch.isfinite(du).all() and torch.isfinite(dE).all()
    shape = moe.LayerShape.from_config(cfg)
    u_d, E_d, b_d = (t.to(DEV).contiguous() for t in (inp.u, inp.centroids, inp.bias))
    routing = moe.moe_route(shape, u_d, E_d, b_d)
    torch.cuda.synchronize()
    gi = routing["topk_idx"].cpu().numpy()
    gates = routing["topk_gate"].cpu().numpy().astype(np.float64)
    counts = routing["expert_counts"].cpu().numpy()
    u, E, b = to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy()
    routed, shared = expert_fns(inp, True)
    sample = np.array([0, 1, 255, 256, 4095, 4096, 8190, 8191])
    ref = O.layer_backward(u[sample], E, b, cfg.top_k, routed, cfg.n_routed, shared, dy.numpy()[sample],
                           selection=gi[sample], weight_grads=False)
    errs = {"du(sampled tokens)": _err(du.cpu().numpy()[sample], ref["du"], 1, cfg.d)}
    order = np.argsort(counts)
    for e in (int(order[-1]), int(order[0]), int(order[len(order) // 2])):
        tok, slot = np.nonzero(gi == e)
        # the expert's rows and their gates: the oracle recomputes the gates
        # from its own affinities for the GPU's selection
        r = O.route(u[tok], E, b, cfg.top_k, selection=gi[tok])
        bb = O.swiglu_ffn_backward(u[tok], *routed(e), r["gate"][np.arange(len(tok)), slot][:, None] * dy.numpy()[tok])
        errs[f"dW_gate_up[{e}] ({len(tok)} rows)"] = _err(grads.dw_gate_up[e].cpu().numpy(), bb["dW_gate_up"])
        errs[f"dW_down[{e}]"] = _err(grads.dw_down[e].cpu().numpy(), bb["dW_down"])
    bs = O.swiglu_ffn_backward(u, *shared[0], dy.numpy())
    errs["dWs_gate_up"] = _err(grads.dws_gate_up[0].cpu().numpy(), bs["dW_gate_up"])
    errs["dWs_down"] = _err(grads.dws_down[0].cpu().numpy(), bs["dW_down"])
    say("  worst block ||d||/||ref||: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    del w, ws, grads, inp
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ FP8 backward

FP8_CASES = {
    "small_fp8": PARITY_CONFIGS["small_fp8"],
    "small_fp8_ns2": PARITY_CONFIGS["small_fp8_ns2"],
    "small_fp8_ns0": PARITY_CONFIGS["small_fp8_ns2"].replace(name="small_fp8_ns0", n_shared=0),
    # experts without rows and groups of one or two rows in the 128x1 code layout
    "one_token_fp8": PARITY_CONFIGS["one_token"].replace(name="one_token_fp8", w_dtype="e4m3"),
    "wide_router_fp8": PARITY_CONFIGS["wide_router"].replace(name="wide_router_fp8", w_dtype="e4m3"),
}


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_backward_fp8_parity(name):
    """The FP8 backward (every GEMM on E4M3 operands) against the oracle's."""
    cfg = FP8_CASES[name]
    say(f"case: FP8 moe_forward_train + moe_backward {name}")
    inp = make_inputs(cfg, 0)
    dy = _dy(cfg)
    y, du, dE, grads, ws, w = _train_step(cfg, inp, dy)
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = (t.to(DEV).contiguous() for t in (inp.u, inp.centroids, inp.bias))
    routing = moe.alloc_routing(shape)
    y_inf = moe.moe_forward(shape, u, E, b, w, routing=routing)
    torch.cuda.synchronize()
    assert torch.equal(y, y_inf)
    errs, empty = _compare(cfg, inp, dy, du, dE, grads, routing["topk_idx"].cpu().numpy())
    say("  worst block ||d||/||ref||: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f"; {empty} experts without rows")
    for k, v in errs.items():
        assert v <= TOL8, (k, v)


def test_backward_fp8_transposed_weights_and_determinism():
    """The transposed codes the FP8 Dgrad reads are the forward's codes
    transposed (one scale per 128x128 block in either orientation), and two
    FP8 training steps give bit-identical gradients."""
    cfg = PARITY_CONFIGS["small_fp8_ns2"]
    say("case: FP8 transposed weight codes, determinism")
    inp = make_inputs(cfg, 0)
    dy = _dy(cfg)
    _, du1, dE1, g1, _, w = _train_step(cfg, inp, dy)
    for a, b in ((w.w_gate_up, w.w_gate_up_t), (w.w_down, w.w_down_t), (w.ws_gate_up, w.ws_gate_up_t),
                 (w.ws_down, w.ws_down_t), (w.s_gate_up, w.s_gate_up_t), (w.s_down, w.s_down_t)):
        assert torch.equal(a.transpose(-1, -2), b)
    _, du2, dE2, g2, _, _ = _train_step(cfg, inp, dy, w)
    assert torch.equal(du1, du2) and torch.equal(dE1, dE2)
    for a, b in ((g1.dw_gate_up, g2.dw_gate_up), (g1.dw_down, g2.dw_down), (g1.dws_gate_up, g2.dws_gate_up),
                 (g1.dws_down, g2.dws_down)):
        assert torch.equal(a, b)


def test_backward_fp8_full_d2048():
    """The FP8 d = 2048 layer (T = 4096, 64 + 2 experts, K = 6; every expert
    spans several 128-row m-tiles and Wgrad blocks) in full: every gradient."""
    cfg = CONFIGS["fp8_d2048"]
    say("case: FP8 moe_backward fp8_d2048 full size, every gradient")
    inp = make_inputs(cfg, 0)
    dy = _dy(cfg)
    y, du, dE, grads, ws, w = _train_step(cfg, inp, dy)
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = (t.to(DEV).contiguous() for t in (inp.u, inp.centroids, inp.bias))
    routing = moe.moe_route(shape, u, E, b)
    torch.cuda.synchronize()
    errs, empty = _compare(cfg, inp, dy, du, dE, grads, routing["topk_idx"].cpu().numpy())
    say("  worst block ||d||/||ref||: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL8, (k, v)
    del w, ws, grads
    torch.cuda.empty_cache()


def test_backward_fp8_full_d7168_sampled():
    """The FP8 DeepSeek-V3 layer (T = 8192, d = 7168, 256 + 1 experts, K = 8):
    du on sampled tokens, and dW of the shared expert and of sampled routed
    experts (the largest, the smallest and a median one), against the
    oracle's FP8 backward."""
    cfg = CONFIGS["fp8_d7168"]
    say("case: FP8 moe_backward fp8_d7168 full size, sampled")
    inp = make_inputs(cfg, 0, weights_device=DEV)
    dy = _dy(cfg)
    y, du, dE, grads, ws, w = _train_step(cfg, inp, dy)
    assert torch.isfinite(du).all() and torch.isfinite(dE).all()
    shape = moe.LayerShape.from_config(cfg)
    u_d, E_d, b_d = (t.to(DEV).contiguous() for t in (inp.u, inp.centroids, inp.bias))
    routing = moe.moe_route(shape, u_d, E_d, b_d)
    torch.cuda.synchronize()
    gi = routing["topk_idx"].cpu().numpy()
    counts = routing["expert_counts"].cpu().numpy()
    u, E, b = to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy()
    routed, shared = expert_fns(inp, True)
    x_deq = O.dequantize_act(*O.quantize_act_1x128(u))

    def expert_bwd(wgu, wd, rows, dout):
        gq, gs = O.quantize_weight_128x128(wgu)
        dq, ds = O.quantize_weight_128x128(wd)
        return O.swiglu_ffn_backward_fp8(u[rows], x_deq[rows], gq, gs, dq, ds, dout)

    sample = np.array([0, 1, 255, 256, 4095, 4096, 8190, 8191])
    ref = O.layer_backward(u[sample], E, b, cfg.top_k, routed, cfg.n_routed, shared, dy.numpy()[sample],
                           selection=gi[sample], weight_grads=False, fp8=True)
    errs = {"du(sampled tokens)": _err(du.cpu().numpy()[sample], ref["du"], 1, cfg.d)}
    order = np.argsort(counts)
    for e in (int(order[-1]), int(order[0]), int(order[len(order) // 2])):
        tok, slot = np.nonzero(gi == e)
        r = O.route(u[tok], E, b, cfg.top_k, selection=gi[tok])
        bb = expert_bwd(*routed(e), tok, r["gate"][np.arange(len(tok)), slot][:, None] * dy.numpy()[tok])
        errs[f"dW_gate_up[{e}] ({len(tok)} rows)"] = _err(grads.dw_gate_up[e].cpu().numpy(), bb["dW_gate_up"])
        errs[f"dW_down[{e}]"] = _err(grads.dw_down[e].cpu().numpy(), bb["dW_down"])
    bs = expert_bwd(*shared[0], np.arange(cfg.T), dy.numpy())
    errs["dWs_gate_up"] = _err(grads.dws_gate_up[0].cpu().numpy(), bs["dW_gate_up"])
    errs["dWs_down"] = _err(grads.dws_down[0].cpu().numpy(), bs["dW_down"])
    say("  worst block ||d||/||ref||: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL8, (k, v)
    del w, ws, grads, inp
    torch.cuda.empty_cache()
