"""Pins for the CPU oracle: each check ties it to something other than itself
(hand-worked values, closed forms, library routines, brute force, invariants),
chosen so that a dropped term, a wrong sign or index, or a transposed operand
in the oracle fails at least one of them."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as O
from moe_workloads import CONFIGS, PARITY_CONFIGS, make_inputs, to_numpy_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LN3 = math.log(3.0)


def _num(x):
    if isinstance(x, str):
        return {"ln3": LN3, "-ln3": -LN3}[x]
    if isinstance(x, list):
        return [_num(v) for v in x]
    return x


def _np_inputs(inp):
    routed = lambda e: (to_numpy_f32(inp.w_gate_up[e]), to_numpy_f32(inp.w_down[e]))
    n_sh = inp.ws_gate_up.shape[0] if inp.ws_gate_up.dim() == 3 else 0
    shared = [(to_numpy_f32(inp.ws_gate_up[s]), to_numpy_f32(inp.ws_down[s])) for s in range(n_sh)]
    return to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy(), routed, shared


# ---------------------------------------------------------------- golden

def test_hand_worked_layer():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_layer.json")))
    u = np.array(_num(g["u"]))
    E = np.array(_num(g["centroids"]))
    b = np.array(g["bias"], np.float32)
    wgu = np.array(_num(g["w_gate_up"]))
    wd = np.array(_num(g["w_down"]))
    shared = [(np.array(_num(g["ws_gate_up"][0])), np.array(_num(g["ws_down"][0])))]
    r = O.layer_forward(u, E, b, g["top_k"], lambda e: (wgu[e], wd[e]), g["n_routed"], shared)
    ex = g["expected"]
    assert r["idx"].tolist() == ex["idx"]
    np.testing.assert_allclose(r["gate"], ex["gate"], rtol=1e-14)
    np.testing.assert_allclose(r["y"], ex["y"], rtol=1e-13)
    grp = O.group_by_expert(r["idx"], g["n_routed"])
    assert grp["counts"].tolist() == ex["counts"]
    assert grp["offsets"].tolist() == ex["offsets"]
    assert grp["perm_token"].tolist() == ex["perm_token"]
    assert grp["pos"].tolist() == ex["pos"]
    nb = O.update_bias(b, grp["counts"], g["T"] * g["top_k"])
    assert nb.dtype == np.float32
    assert [float(x) for x in nb] == ex["bias_after"]


# ---------------------------------------------------------------- elementwise

def test_sigmoid_closed_forms_and_library():
    assert O.sigmoid(0.0) == 0.5
    assert abs(O.sigmoid(LN3) - 0.75) < 1e-15
    assert abs(O.sigmoid(-LN3) - 0.25) < 1e-15
    z = np.random.default_rng(0).normal(0, 5, 10000)
    np.testing.assert_allclose(O.sigmoid(z), scipy.special.expit(z), rtol=1e-14, atol=0)
    np.testing.assert_allclose(O.sigmoid(z) + O.sigmoid(-z), 1.0, atol=1e-15)


def test_silu_closed_forms_and_library():
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(LN3) - 0.75 * LN3) < 1e-15
    a = np.random.default_rng(1).normal(0, 4, 10000)
    ref = torch.nn.functional.silu(torch.from_numpy(a)).numpy()
    np.testing.assert_allclose(O.silu(a), ref, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(O.silu(a) - O.silu(-a), a, atol=1e-13)


# ---------------------------------------------------------------- routing

def test_affinities_special_case_unit_vectors():
    E = np.random.default_rng(2).normal(0, 1, (6, 4))
    s = O.affinities(np.eye(4), E)
    np.testing.assert_allclose(s, scipy.special.expit(E.T), rtol=1e-15)


def test_topk_brute_force_tiny_config():
    cfg = CONFIGS["tiny_fp32"]
    inp = make_inputs(cfg, 0)
    u, E, b, _, _ = _np_inputs(inp)
    s = O.affinities(u, E)
    r = O.select_topk(s, b, cfg.top_k)
    v = s + b.astype(np.float64)
    for t in range(cfg.T):
        best = max(itertools.combinations(range(cfg.n_routed), cfg.top_k),
                   key=lambda c: (sum(v[t, j] for j in c), tuple(-j for j in c)))
        assert set(r["idx"][t]) == set(best)
        sel = list(r["idx"][t])
        assert all(v[t, sel[i]] >= v[t, sel[i + 1]] for i in range(len(sel) - 1))
        uns = [j for j in range(cfg.n_routed) if j not in sel]
        assert min(v[t, sel]) >= max(v[t, uns])
        assert r["gap"][t] == pytest.approx(min(v[t, sel]) - max(v[t, uns]), abs=0)


def test_topk_exact_ties_go_to_lower_index():
    s = np.array([[0.5, 0.7, 0.5, 0.7, 0.5]])
    r = O.select_topk(s, np.zeros(5, np.float32), 3)
    assert r["idx"][0].tolist() == [1, 3, 0]
    assert r["gap"][0] == 0.0


def test_bias_enters_selection_only():
    rng = np.random.default_rng(3)
    s = O.sigmoid(rng.normal(0, 1, (50, 8)))
    J = [6, 1, 3]
    b = np.zeros(8, np.float32)
    b[J] = 10.0
    r = O.select_topk(s, b, 3)
    for t in range(50):
        assert set(r["idx"][t]) == set(J)
    g = O.normalised_gates(s, r["idx"])
    sel = np.take_along_axis(s, r["idx"].astype(np.int64), 1)
    np.testing.assert_allclose(g, sel / s[:, J].sum(axis=1, keepdims=True), rtol=1e-15)
    # A common shift of all biases changes nothing (the scores here are far from ties).
    b2 = rng.normal(0, 0.1, 8).astype(np.float32)
    r1 = O.select_topk(s, b2, 3)
    r2 = O.select_topk(s, (b2 + np.float32(0.25)).astype(np.float32), 3)
    far = r1["gap"] > 1e-6
    assert (r1["idx"][far] == r2["idx"][far]).all()


def test_gate_invariants():
    rng = np.random.default_rng(4)
    s = O.sigmoid(rng.normal(0, 2, (100, 16)))
    idx = O.select_topk(s, rng.normal(0, 0.1, 16).astype(np.float32), 5)["idx"]
    g = O.normalised_gates(s, idx)
    np.testing.assert_allclose(g.sum(axis=1), 1.0, atol=1e-15)
    assert (g > 0).all() and (g <= 1).all()
    sel = np.take_along_axis(s, idx.astype(np.int64), 1)
    np.testing.assert_allclose(g[:, 0] / g[:, 1], sel[:, 0] / sel[:, 1], rtol=1e-14)


# ---------------------------------------------------------------- grouping

@pytest.mark.parametrize("T,N,K", [(1, 4, 2), (37, 8, 3), (300, 16, 4), (64, 4, 4)])
def test_group_by_expert_against_library_sort(T, N, K):
    rng = np.random.default_rng(T * 100 + N)
    idx = np.stack([rng.permutation(N)[:K] for _ in range(T)]).astype(np.int32)
    g = O.group_by_expert(idx, N)
    assert g["counts"].tolist() == np.bincount(idx.ravel(), minlength=N).tolist()
    assert g["offsets"].tolist() == [0] + np.cumsum(np.bincount(idx.ravel(), minlength=N)).tolist()
    assert g["counts"].sum() == T * K
    order = np.argsort(idx.ravel(), kind="stable")       # t-major flattening -> stable by token
    assert (g["perm_token"] == order // K).all()
    inv = np.empty_like(order)
    inv[order] = np.arange(T * K)
    assert (g["pos"].ravel() == inv).all()
    assert sorted(g["pos"].ravel().tolist()) == list(range(T * K))


# ---------------------------------------------------------------- bias update

def test_bias_update_closed_form():
    counts = np.array([0, 5, 10, 11, 40])     # T*K = 50, N_r = 5: mean load 10
    b = O.update_bias(np.zeros(5, np.float32), counts, 50)
    g = np.float32(0.001)
    assert b.tolist() == [g, g, 0.0, -g, -g]
    # Constant counts for n steps: the fp32 sum of n identical increments.
    x = np.zeros(5, np.float32)
    ref = np.zeros(5, np.float32)
    for _ in range(100):
        x = O.update_bias(x, counts, 50)
        ref = (ref + np.array([g, g, 0, -g, -g], np.float32)).astype(np.float32)
    assert (x == ref).all()
    assert abs(float(x[0]) - 0.1) < 1e-5


def test_bias_update_moves_load_toward_mean():
    cfg = PARITY_CONFIGS["small_bf16"]
    inp = make_inputs(cfg, 0, with_weights=False)
    u, E, b, _, _ = _np_inputs(inp)
    s = O.affinities(u, E)
    counts0 = O.group_by_expert(O.select_topk(s, b, cfg.top_k)["idx"], cfg.n_routed)["counts"]
    bb = b.copy()
    for _ in range(200):
        c = O.group_by_expert(O.select_topk(s, bb, cfg.top_k)["idx"], cfg.n_routed)["counts"]
        bb = O.update_bias(bb, c, cfg.T * cfg.top_k)
    c = O.group_by_expert(O.select_topk(s, bb, cfg.top_k)["idx"], cfg.n_routed)["counts"]
    assert c.max() < counts0.max()


# ---------------------------------------------------------------- expert FFN and layer

def _torch_swiglu(x, wgu, wd):
    x, wgu, wd = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, wgu, wd))
    I = wgu.shape[0] // 2
    gate, up = torch.nn.functional.linear(x, wgu[:I]), torch.nn.functional.linear(x, wgu[I:])
    return torch.nn.functional.linear(torch.nn.functional.silu(gate) * up, wd).numpy()


def test_swiglu_scalar_closed_form():
    # d = I = 1: FFN(u) = wd * SiLU(wg u) * (wu u); with wg u = ln 3, SiLU = 0.75 ln 3.
    u = np.array([[2.0]])
    out = O.swiglu_ffn(u, np.array([[LN3 / 2], [3.0]]), np.array([[0.5]]))
    assert out[0, 0] == pytest.approx(0.5 * 0.75 * LN3 * 6.0, rel=1e-15)


def test_swiglu_against_library_mlp():
    rng = np.random.default_rng(5)
    x, wgu, wd = rng.normal(0, 1, (33, 40)), rng.normal(0, 0.2, (2 * 24, 40)), rng.normal(0, 0.2, (40, 24))
    np.testing.assert_allclose(O.swiglu_ffn(x, wgu, wd), _torch_swiglu(x, wgu, wd), rtol=1e-12, atol=1e-14)


def test_single_expert_layer_is_residual_mlp():
    rng = np.random.default_rng(6)
    u, E = rng.normal(0, 1, (20, 16)), rng.normal(0, 1, (1, 16))
    wgu, wd = rng.normal(0, 0.3, (2 * 8, 16)), rng.normal(0, 0.3, (16, 8))
    r = O.layer_forward(u, E, np.zeros(1, np.float32), 1, lambda e: (wgu, wd), 1, [])
    np.testing.assert_allclose(r["gate"], 1.0)
    np.testing.assert_allclose(r["y"], u + _torch_swiglu(u, wgu, wd), rtol=1e-12, atol=1e-13)


def test_dense_mixture_when_k_equals_n():
    cfg = PARITY_CONFIGS["dense_k_eq_n"]
    inp = make_inputs(cfg, 0)
    u, E, b, routed, shared = _np_inputs(inp)
    r = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared)
    s = scipy.special.expit(u.astype(np.float64) @ E.astype(np.float64).T)
    w = s / s.sum(axis=1, keepdims=True)
    ref = u.astype(np.float64) + sum(_torch_swiglu(u, *sh) for sh in shared)
    for e in range(cfg.n_routed):
        ref = ref + w[:, e:e + 1] * _torch_swiglu(u, *routed(e))
    np.testing.assert_allclose(r["y"], ref, rtol=1e-11, atol=1e-12)


def test_layer_linearity_and_zero_routed():
    cfg = PARITY_CONFIGS["small_bf16_ns2"].replace(T=40)
    inp = make_inputs(cfg, 0)
    u, E, b, routed, shared = _np_inputs(inp)
    base = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared)
    zero = O.layer_forward(u, E, b, cfg.top_k, lambda e: (routed(e)[0], 0 * routed(e)[1]), cfg.n_routed, shared)
    ref_shared = sum(_torch_swiglu(u, *sh) for sh in shared)
    np.testing.assert_allclose(zero["y"], u + ref_shared, rtol=1e-12, atol=1e-12)
    tri = O.layer_forward(u, E, b, cfg.top_k, lambda e: (routed(e)[0], 3 * routed(e)[1]), cfg.n_routed, shared)
    np.testing.assert_allclose(tri["routed_sum"], 3 * base["routed_sum"], rtol=1e-12, atol=1e-13)


def test_layer_expert_permutation_equivariance():
    cfg = PARITY_CONFIGS["small_bf16"].replace(T=30)
    inp = make_inputs(cfg, 0)
    u, E, b, routed, shared = _np_inputs(inp)
    base = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared)
    perm = np.random.default_rng(7).permutation(cfg.n_routed)
    r = O.layer_forward(u, E[perm], b[perm], cfg.top_k, lambda e: routed(perm[e]), cfg.n_routed, shared)
    ok = base["gap"] > 1e-9
    np.testing.assert_allclose(r["y"][ok], base["y"][ok], rtol=1e-12, atol=1e-12)
    assert (perm[r["idx"][ok]] == base["idx"][ok]).all()


def test_layer_tokens_are_independent():
    cfg = PARITY_CONFIGS["small_bf16"].replace(T=40)
    inp = make_inputs(cfg, 0)
    u, E, b, routed, shared = _np_inputs(inp)
    full = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared)
    sub = [3, 17, 39]
    part = O.layer_forward(u[sub], E, b, cfg.top_k, routed, cfg.n_routed, shared)
    np.testing.assert_allclose(part["y"], full["y"][sub], rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- FP8 codec and quantisation

def test_e4m3_decode_all_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all() and nan.sum() == 2     # 0x7F and 0xFF
    assert (ours[~nan] == ref[~nan]).all()
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e4m3_encode_against_torch_and_midpoints():
    vals = O.e4m3_decode(np.arange(0, 127))
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(8)
    x = np.concatenate([vals, mids, -mids, rng.normal(0, 100, 20000), rng.normal(0, 0.01, 20000),
                        np.nextafter(mids, 0), np.nextafter(mids, 1000)]).astype(np.float32)
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (O.e4m3_encode(x) == ref).all()
    # Midpoints go to the even code: e.g. between 1.0 (0x38) and 1.125 (0x39) -> 0x38.
    assert O.e4m3_encode(np.float32(1.0625)) == 0x38
    assert O.e4m3_encode(np.float32(1.1875)) == 0x3A


def test_e4m3_encode_saturates():
    x = np.array([464.0001, 500.0, 1e30, -1e30, 448.0, -470.0], np.float32)
    assert O.e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE]


def test_quantize_act_properties():
    rng = np.random.default_rng(9)
    x = rng.normal(0, 3, (7, 384)).astype(np.float32)
    x[2, 128:256] = 0
    q, sc = O.quantize_act_1x128(x)
    assert sc.shape == (7, 3) and sc.dtype == np.float32
    assert sc[2, 1] == 1.0 and (q[2, 128:256] & 0x7F == 0).all()
    deq = O.dequantize_act(q, sc)
    for r in range(7):
        for j in range(3):
            tile = x[r, j * 128:(j + 1) * 128].astype(np.float64)
            if not tile.any():
                continue
            a = np.argmax(np.abs(tile))
            assert q[r, j * 128 + a] & 0x7F == 0x7E                      # amax hits 448
            assert abs(abs(deq[r, j * 128 + a]) - abs(tile[a])) <= np.spacing(np.float32(abs(tile[a])))
            normal = np.abs(tile) * (448 / np.abs(tile).max()) >= 2 ** -6
            err = np.abs(deq[r, j * 128:(j + 1) * 128] - tile)[normal]
            assert (err <= 2.0 ** -4 * np.abs(tile[normal]) * 1.0001).all()


def test_quantize_weight_block_layout():
    rng = np.random.default_rng(10)
    w = rng.normal(0, 1, (256, 384)).astype(np.float32)
    w[128:, :128] *= 1000.0                    # one block far larger than the rest
    q, sc = O.quantize_weight_128x128(w)
    assert sc.shape == (2, 3)
    big = sc[1, 0]
    assert big > 100 * sc[0, 0] and big > 100 * sc[1, 1]
    deq = O.dequantize_weight(q, sc)
    np.testing.assert_allclose(deq, w, rtol=2 ** -4, atol=2 ** -9 * sc.max())


def test_fp8_gemm_blockwise_promotion_identity():
    """sum_kb (sa * sw) * sum_{k in kb} qa * qw equals the dequantised product."""
    rng = np.random.default_rng(11)
    a = rng.normal(0, 1, (9, 384)).astype(np.float32)
    w = rng.normal(0, 0.05, (256, 384)).astype(np.float32)
    qa, sa = O.quantize_act_1x128(a)
    qw, sw = O.quantize_weight_128x128(w)
    da, dw = O.e4m3_decode(qa), O.e4m3_decode(qw)
    acc = np.zeros((9, 256))
    for kb in range(3):
        part = da[:, kb * 128:(kb + 1) * 128] @ dw[:, kb * 128:(kb + 1) * 128].T
        acc += part * (sa[:, kb:kb + 1].astype(np.float64) * np.repeat(sw[:, kb].astype(np.float64), 128)[None, :])
    ref = O.dequantize_act(qa, sa) @ O.dequantize_weight(qw, sw).T
    np.testing.assert_allclose(acc, ref, rtol=1e-12, atol=1e-12)
    # and it is close to the unquantised product
    exact = a.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(ref - exact).max() < 0.1 * np.abs(exact).max()


def test_fp8_layer_close_to_bf16_layer():
    cfg = PARITY_CONFIGS["small_fp8"].replace(T=24)
    inp = make_inputs(cfg, 0)
    u, E, b, routed, shared = _np_inputs(inp)
    r8 = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared, fp8=True)
    r16 = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared)
    assert (r8["idx"] == r16["idx"]).all()            # the router is not quantised
    branch = r16["y"] - u
    err = np.abs(r8["y"] - r16["y"]).max()
    assert err < 0.1 * np.sqrt(np.mean(branch ** 2)) * 10
    assert err > 0                                      # quantisation did happen


def test_fp8_ffn_against_torch_float8_composition():
    """The FP8 expert, rebuilt independently: torch's float8_e4m3fn cast for
    every quantisation (values are scaled below 464 first, where its
    round-to-nearest-even agrees with a saturating encoder), float64 matmuls
    and torch's SiLU."""
    rng = np.random.default_rng(12)
    x = rng.normal(0, 1, (5, 256)).astype(np.float32)
    wgu = rng.normal(0, 0.05, (2 * 128, 256)).astype(np.float32)
    wd = rng.normal(0, 0.05, (256, 128)).astype(np.float32)

    xd, gd, dd = _tq_act(torch.from_numpy(x)), _tq_w(torch.from_numpy(wgu)), _tq_w(torch.from_numpy(wd))
    g, u = xd @ gd[:128].T, xd @ gd[128:].T
    h = (torch.nn.functional.silu(g) * u).to(torch.float32)
    ref = (_tq_act(h) @ dd.T).numpy()

    xq, xs = O.quantize_act_1x128(x)
    gq, gs = O.quantize_weight_128x128(wgu)
    dq, ds = O.quantize_weight_128x128(wd)
    out = O.swiglu_ffn_fp8(O.dequantize_act(xq, xs), gq, gs, dq, ds)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- the FP8 layer, composed independently

def _tq_act(a: torch.Tensor) -> torch.Tensor:
    """1x128 tiles through torch's float8_e4m3fn cast: scale = amax / 448 and
    codes of a * (448 / amax), in the tensor's own precision (float32 for the
    layer; the values are scaled to at most 448, where the cast rounds to
    nearest even like a saturating encoder).  Both quotients are
    tensor / tensor divisions, which torch rounds correctly (its
    scalar / tensor form multiplies by a reciprocal and can land one ulp
    off).  Returns the dequantised values in float64."""
    t = a.view(a.shape[0], -1, 128)
    amax = t.abs().amax(-1, keepdim=True)
    c448 = torch.full_like(amax, 448.0)
    q = (t * (c448 / amax)).to(torch.float8_e4m3fn).to(torch.float64)
    return (q * (amax / c448).to(torch.float64)).view(a.shape)


def _tq_w(w: torch.Tensor) -> torch.Tensor:
    """128x128 blocks through torch's float8_e4m3fn cast (float32 scales), dequantised to float64."""
    R, C = w.shape
    t = w.view(R // 128, 128, C // 128, 128)
    amax = t.abs().amax(dim=(1, 3), keepdim=True)
    c448 = torch.full_like(amax, 448.0)
    q = (t * (c448 / amax)).to(torch.float8_e4m3fn).to(torch.float64)
    return (q * (amax / c448).to(torch.float64)).view(R, C)


def _torch_fp8_layer(u, E, b, k, routed, n_routed, shared, slip=None):
    """The whole FP8 layer from torch pieces only: router and residual on the
    bf16 u (float64 sigmoid of the float64 logits, torch.topk on s + b,
    gates s / sum s); every expert's two GEMMs on the 1x128-quantised u and
    the 128x128-quantised weights in float64; h rounded to float32 and
    quantised 1x128 before the down GEMM.  ``slip`` plants one plausible
    mistake, for the checks that the pin would catch it."""
    u32 = torch.from_numpy(np.asarray(u, np.float32))
    u64 = u32.double()
    x_router = _tq_act(u32) if slip == "router_on_fp8_u" else u64
    s = torch.sigmoid(x_router @ torch.from_numpy(np.asarray(E, np.float64)).T)
    v = s + torch.from_numpy(np.asarray(b, np.float32)).double()
    idx = torch.topk(v, k, dim=1).indices
    sel = torch.gather(s, 1, idx)
    gate = sel / sel.sum(dim=1, keepdim=True)
    xq = _tq_act(u32)

    def ffn(x, wgu, wd):
        g = _tq_w(torch.from_numpy(np.asarray(wgu, np.float32)))
        dn = _tq_w(torch.from_numpy(np.asarray(wd, np.float32)))
        I = g.shape[0] // 2
        h = torch.nn.functional.silu(x @ g[:I].T) * (x @ g[I:].T)
        hq = _tq_act(h) if slip == "h_not_rounded_to_f32" else _tq_act(h.to(torch.float32))
        return hq @ dn.T

    y = (xq if slip == "quantised_residual" else u64).clone()
    for wgu, wd in shared:
        y += ffn(u64 if slip == "shared_on_bf16_u" else xq, wgu, wd)
    for t in range(u64.shape[0]):
        for j in range(k):
            y[t] += gate[t, j] * ffn(xq[t:t + 1], *routed(int(idx[t, j])))[0]
    return y.numpy(), idx.numpy()


def test_fp8_layer_against_torch_float8_composition():
    """layer_forward(fp8=True) against the FP8 layer composed from torch's
    float8_e4m3fn casts (two 128-tiles along d and along I, a shared expert,
    K = 2), and every plausible mistake in the FP8 assembly moves the
    result by far more than the comparison's tolerance: the shared expert
    fed the bf16 u, a quantised residual, h quantised without its fp32
    rounding, the router on the quantised u."""
    from moe_workloads import MoEConfig
    cfg = MoEConfig("fp8_layer_pin", T=12, d=256, n_routed=6, n_shared=1, inter=256, top_k=2,
                    x_dtype="bf16", w_dtype="e4m3", out_dtype="bf16", w_std=0.05, e_std=0.05, b_std=0.02,
                    cfg_id=90)
    inp = make_inputs(cfg, 0)
    u, E, b, routed, shared = _np_inputs(inp)
    r = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared, fp8=True)
    assert (r["gap"] > 1e-6).all()
    ref, idx = _torch_fp8_layer(u, E, b, cfg.top_k, routed, cfg.n_routed, shared)
    assert (np.sort(idx, 1) == np.sort(r["idx"], 1)).all()
    np.testing.assert_allclose(r["y"], ref, rtol=1e-12, atol=1e-12)
    branch = float(np.abs(r["y"] - u).max())
    for slip in ("shared_on_bf16_u", "quantised_residual", "h_not_rounded_to_f32", "router_on_fp8_u"):
        bad, _ = _torch_fp8_layer(u, E, b, cfg.top_k, routed, cfg.n_routed, shared, slip=slip)
        assert np.abs(bad - r["y"]).max() > 1e-9 * branch, slip


# ---------------------------------------------------------------- group-limited routing

def test_grouped_selection_hand_worked():
    """8 experts in 4 groups of 2, K = 3.  With 2 groups kept, q = 2 and a
    group's score is the sum of both members: groups 1 (0.5 + 0.6 = 1.1) and
    0 (0.9 + 0.1 = 1.0) beat group 2 (0.85), so expert 4 (0.8, the second
    best overall) is left out: [0, 3, 2].  With 3 groups kept, q = 1 (the
    group's best member): groups 0, 2, 1 -> the global top-3 [0, 4, 3]."""
    v = np.array([[0.9, 0.1, 0.5, 0.6, 0.8, 0.05, 0.3, 0.35]])
    r = O.select_topk_grouped(v, np.zeros(8, np.float32), 3, 4, 2)
    assert r["idx"][0].tolist() == [0, 3, 2]
    np.testing.assert_allclose(r["group_score"][0], [1.0, 1.1, 0.85, 0.65], rtol=1e-15)
    assert sorted(r["groups"][0].tolist()) == [0, 1]
    assert r["gap"][0] == pytest.approx(0.5 - 0.1, abs=1e-15)       # best expert left in the kept groups: 1 (0.1)
    assert r["group_gap"][0] == pytest.approx(1.0 - 0.85, abs=1e-15)
    r3 = O.select_topk_grouped(v, np.zeros(8, np.float32), 3, 4, 3)
    assert r3["idx"][0].tolist() == [0, 4, 3] == O.select_topk(v, np.zeros(8, np.float32), 3)["idx"][0].tolist()


def test_grouped_selection_special_cases():
    rng = np.random.default_rng(21)
    s = O.sigmoid(rng.normal(0, 1, (60, 24)))
    b = rng.normal(0, 0.05, 24).astype(np.float32)
    full = O.select_topk(s, b, 5)
    # every group kept: the global selection
    allg = O.select_topk_grouped(s, b, 5, 6, 6)
    assert (allg["idx"] == full["idx"]).all()
    # one expert per group, at least K groups kept: q = 1, the kept groups are the best experts
    single = O.select_topk_grouped(s, b, 5, 24, 7)
    assert (single["idx"] == full["idx"]).all()


def test_grouped_selection_brute_force():
    """Tiny inputs: the kept groups maximise the total group score over all
    subsets of topk_groups groups, and the K experts maximise the sum of v
    over all K-subsets of the kept groups' experts; the selection spans at
    most topk_groups groups and beats every other expert of those groups."""
    rng = np.random.default_rng(22)
    n, G, M, K = 12, 4, 2, 3
    S = n // G
    s = O.sigmoid(rng.normal(0, 1.5, (40, n)))
    b = rng.normal(0, 0.1, n).astype(np.float32)
    r = O.select_topk_grouped(s, b, K, G, M)
    v = s + b.astype(np.float64)
    q = math.ceil(K / M)
    for t in range(40):
        gsc = [sorted(v[t, g * S:(g + 1) * S], reverse=True)[:q] for g in range(G)]
        gsum = [sum(x) for x in gsc]
        best = max(itertools.combinations(range(G), M), key=lambda c: (sum(gsum[g] for g in c), tuple(-g for g in c)))
        assert set(r["groups"][t].tolist()) == set(best)
        allowed = [e for g in best for e in range(g * S, (g + 1) * S)]
        pick = max(itertools.combinations(allowed, K), key=lambda c: (sum(v[t, e] for e in c), tuple(-e for e in c)))
        assert set(r["idx"][t].tolist()) == set(pick)
        assert len({e // S for e in r["idx"][t]}) <= M
        rest = [e for e in allowed if e not in r["idx"][t]]
        assert min(v[t, r["idx"][t]]) >= max(v[t, rest])


def test_grouped_layer_matches_layer_with_the_grouped_selection():
    cfg = PARITY_CONFIGS["small_bf16"].replace(T=20)
    inp = make_inputs(cfg, 0)
    u, E, b, routed, shared = _np_inputs(inp)
    rg = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared, n_groups=4, topk_groups=2)
    sel = O.select_topk_grouped(O.affinities(u, E), b, cfg.top_k, 4, 2)["idx"]
    assert (rg["idx"] == sel).all()
    assert all(len({e // 4 for e in row}) <= 2 for row in rg["idx"])
    ref = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared, selection=sel)
    np.testing.assert_allclose(rg["y"], ref["y"], rtol=1e-15, atol=0)


# ---------------------------------------------------------------- backward

def _torch_layer(u, E, b, idx, routed, shared, n_routed):
    """The layer as torch float64 modules with the selection fixed, for autograd."""
    u_t = torch.tensor(u, dtype=torch.float64, requires_grad=True)
    E_t = torch.tensor(np.asarray(E, np.float64), requires_grad=True)
    W = {e: [torch.tensor(np.asarray(w, np.float64), requires_grad=True) for w in routed(e)] for e in range(n_routed)}
    Ws = [[torch.tensor(np.asarray(w, np.float64), requires_grad=True) for w in sh] for sh in shared]
    s = torch.sigmoid(u_t @ E_t.T)
    it = torch.tensor(idx, dtype=torch.int64)
    sel = torch.gather(s, 1, it)
    g = sel / sel.sum(dim=1, keepdim=True)

    def ffn(x, wgu, wd):
        I = wgu.shape[0] // 2
        return torch.nn.functional.linear(torch.nn.functional.silu(x @ wgu[:I].T) * (x @ wgu[I:].T), wd)

    y = u_t
    for wgu, wd in Ws:
        y = y + ffn(u_t, wgu, wd)
    for t in range(u.shape[0]):
        for j in range(idx.shape[1]):
            y = y + torch.nn.functional.pad(g[t, j] * ffn(u_t[t:t + 1], *W[int(idx[t, j])]),
                                            (0, 0, t, u.shape[0] - t - 1))
    return y, u_t, E_t, W, Ws


def test_backward_against_torch_autograd():
    """Every gradient of layer_backward against torch autograd in float64 on
    the same layer (selection fixed): du, dE, each routed expert's and each
    shared expert's dW, and zero weight gradients for experts without rows."""
    cfg = PARITY_CONFIGS["small_bf16_ns2"].replace(T=14, d=64, inter=32, n_routed=6, top_k=2)
    inp = make_inputs(cfg, 0)
    u, E, b, routed, shared = _np_inputs(inp)
    dy = np.random.default_rng(30).normal(0, 1, u.shape)
    r = O.layer_backward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared, dy)
    y, u_t, E_t, W, Ws = _torch_layer(u, E, b, r["idx"], routed, shared, cfg.n_routed)
    fwd = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared)
    np.testing.assert_allclose(y.detach().numpy(), fwd["y"], rtol=1e-12, atol=1e-12)
    y.backward(torch.tensor(dy))
    np.testing.assert_allclose(r["du"], u_t.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dE"], E_t.grad.numpy(), rtol=1e-10, atol=1e-13)
    for e in range(cfg.n_routed):
        if e in r["dW_gate_up"]:
            np.testing.assert_allclose(r["dW_gate_up"][e], W[e][0].grad.numpy(), rtol=1e-10, atol=1e-13)
            np.testing.assert_allclose(r["dW_down"][e], W[e][1].grad.numpy(), rtol=1e-10, atol=1e-13)
        else:
            assert W[e][0].grad is None or not W[e][0].grad.any()
    for si in range(cfg.n_shared):
        np.testing.assert_allclose(r["dWs_gate_up"][si], Ws[si][0].grad.numpy(), rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(r["dWs_down"][si], Ws[si][1].grad.numpy(), rtol=1e-10, atol=1e-13)


def test_backward_finite_differences():
    """Central differences of <dy, y> along random directions of u, of the
    centroids and of one expert's weights (selection fixed, away from ties)."""
    cfg = PARITY_CONFIGS["small_bf16"].replace(T=6, d=64, inter=32, n_routed=5, top_k=2)
    inp = make_inputs(cfg, 0)
    u, E, b, routed, shared = _np_inputs(inp)
    rng = np.random.default_rng(31)
    dy = rng.normal(0, 1, u.shape)
    r = O.layer_backward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared, dy)
    sel = r["idx"]
    eps = 1e-6

    def f(uu=u, EE=E, rt=routed):
        return float(np.sum(dy * O.layer_forward(uu, EE, b, cfg.top_k, rt, cfg.n_routed, shared, selection=sel)["y"]))

    for _ in range(3):
        v = rng.normal(0, 1, u.shape)
        num = (f(uu=u + eps * v) - f(uu=u - eps * v)) / (2 * eps)
        assert num == pytest.approx(float(np.sum(r["du"] * v)), rel=1e-6, abs=1e-8)
        v = rng.normal(0, 1, E.shape)
        num = (f(EE=E + eps * v) - f(EE=E - eps * v)) / (2 * eps)
        assert num == pytest.approx(float(np.sum(r["dE"] * v)), rel=1e-6, abs=1e-8)
    e = int(sel[0, 0])
    for which in (0, 1):
        v = rng.normal(0, 1, routed(e)[which].shape)

        def rt(sign):
            def fn(j):
                w = list(routed(j))
                if j == e:
                    w[which] = w[which] + sign * eps * v
                return tuple(w)
            return fn
        num = (f(rt=rt(1)) - f(rt=rt(-1))) / (2 * eps)
        ana = float(np.sum((r["dW_gate_up"] if which == 0 else r["dW_down"])[e] * v))
        assert num == pytest.approx(ana, rel=1e-6, abs=1e-8)


def test_backward_single_expert_is_residual_mlp_backward():
    """N_r = K = 1 (gate 1, so no routing gradient) and no shared expert:
    du = dy + the plain SwiGLU MLP's input gradient (torch.func.vjp)."""
    rng = np.random.default_rng(32)
    u, E = rng.normal(0, 1, (9, 16)), rng.normal(0, 1, (1, 16))
    wgu, wd = rng.normal(0, 0.3, (16, 16)), rng.normal(0, 0.3, (16, 8))
    dy = rng.normal(0, 1, u.shape)
    r = O.layer_backward(u, E, np.zeros(1, np.float32), 1, lambda e: (wgu, wd), 1, [], dy)
    assert not r["dz"].any() and not r["dE"].any()

    def mlp(x):
        g, up = x @ torch.tensor(wgu[:8]).T, x @ torch.tensor(wgu[8:]).T
        return torch.nn.functional.silu(g) * up @ torch.tensor(wd).T
    _, vjp = torch.func.vjp(mlp, torch.tensor(u))
    np.testing.assert_allclose(r["du"], dy + vjp(torch.tensor(dy))[0].numpy(), rtol=1e-12, atol=1e-12)


def test_silu_grad_closed_form():
    assert O.silu_grad(0.0) == 0.5
    a = np.random.default_rng(33).normal(0, 3, 1000)
    t = torch.tensor(a, requires_grad=True)
    torch.nn.functional.silu(t).sum().backward()
    np.testing.assert_allclose(O.silu_grad(a), t.grad.numpy(), rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------ FP8 backward

def test_round_bf16_matches_torch():
    """round_bf16 against torch's float32 -> bfloat16 conversion (nearest,
    ties to even), on random values and on exact ties."""
    rng = np.random.default_rng(40)
    x = np.concatenate([rng.normal(0, 1, 4000), rng.normal(0, 1e-30, 100), rng.normal(0, 1e30, 100)]).astype(np.float32)
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)   # half-way between two bf16
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1.0])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x)
    assert np.array_equal(got, ref)


def test_quantize_act_128x1_tiles_rows_from_row_zero():
    """The 128x1 tiling: tile (b, c) holds rows 128 b .. 128 b + 127 of column
    c (the last tile short); each tile is an independent 1x128 tile of the
    transpose.  A column whose rows differ in magnitude tile by tile, a zero
    column and a short last tile."""
    rng = np.random.default_rng(41)
    x = rng.normal(0, 1, (300, 5)).astype(np.float32)
    x[:128, 1] *= 1000.0
    x[:, 3] = 0.0
    q, sc = O.quantize_act_128x1(x)
    assert q.shape == x.shape and sc.shape == (3, 5)
    for b0 in range(3):
        rows = slice(128 * b0, min(128 * (b0 + 1), 300))
        for c in range(5):
            col = x[rows, c]
            tq, ts = O.quantize_act_1x128(np.pad(col, (0, 128 - col.size))[None, :])
            assert (q[rows, c] == tq[0, :col.size]).all() and sc[b0, c] == ts[0, 0]
    assert sc[0, 1] > 100 * sc[1, 1]               # the scaled rows are in tile 0 only
    assert (q[:, 3] == 0).all() and (sc[:, 3] == 1).all()
    deq = O.dequantize_act_128x1(q, sc)
    assert np.all(np.abs(deq - x) <= np.abs(x) * 2.0 ** -4 + sc[np.arange(300) // 128, :] * 2.0 ** -9)


def _tq_rows(a: torch.Tensor) -> torch.Tensor:
    """128x1 tiles (along the rows, from row 0) through torch's cast: the 1x128
    tiling of the zero-padded transpose.  Dequantised, float64."""
    R, C = a.shape
    Rp = -(-R // 128) * 128
    t = torch.zeros((C, Rp), dtype=a.dtype)
    t[:, :R] = a.T
    return _tq_act(t)[:, :R].T


def _torch_fp8_expert_backward(x, wgu, wd, dout, slip=None):
    """One FP8 expert's backward from torch pieces: float8_e4m3fn casts, torch
    bf16 rounding, float64 products.  ``slip`` plants one plausible mistake."""
    bf = lambda t: t.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    x32 = torch.from_numpy(np.asarray(x, np.float32))
    g = _tq_w(torch.from_numpy(np.asarray(wgu, np.float32)))
    dn = _tq_w(torch.from_numpy(np.asarray(wd, np.float32)))
    I = g.shape[0] // 2
    xq = _tq_act(x32)
    G, U = xq @ g[:I].T, xq @ g[I:].T
    if slip != "cache_not_bf16":
        G, U = bf(G), bf(U)
    do = torch.from_numpy(np.asarray(dout, np.float64))
    do_b = do if slip == "no_bf16_before_quantising" else bf(do)
    dH = bf(_tq_act(do_b.to(torch.float32)) @ dn)
    sg = torch.sigmoid(G)
    dG, dU = dH * U * sg * (1 + G * (1 - sg)), dH * torch.nn.functional.silu(G)
    dGU = bf(torch.cat([dG, dU], dim=1))
    H = bf(torch.nn.functional.silu(G) * U)
    dx = _tq_act(dGU.to(torch.float32)) @ g
    along_rows = (lambda t: _tq_act(t.to(torch.float32))) if slip == "wgrad_tiles_along_columns" else \
        (lambda t: _tq_rows(t.to(torch.float32)))
    xw = xq if slip == "wgrad_x_from_forward_codes" else x32.double()
    dW_down = along_rows(do_b).T @ along_rows(H)
    dW_gu = along_rows(dGU).T @ along_rows(xw)
    return {"dx": dx.numpy(), "dW_gate_up": dW_gu.numpy(), "dW_down": dW_down.numpy()}


def test_fp8_expert_backward_pinned_to_torch_fp8():
    """swiglu_ffn_backward_fp8 against the same steps built from torch's
    float8_e4m3fn and bfloat16 conversions (200 rows: one full and one short
    128-row Wgrad tile; two 128-blocks along d and I).  Each planted slip
    moves the torch result away from the oracle's."""
    rng = np.random.default_rng(42)
    n, d, I = 200, 256, 256
    x = torch.from_numpy(rng.normal(0, 1, (n, d))).to(torch.bfloat16).double().numpy()
    wgu = torch.from_numpy(rng.normal(0, 0.05, (2 * I, d))).to(torch.bfloat16).double().numpy()
    wd = torch.from_numpy(rng.normal(0, 0.05, (d, I))).to(torch.bfloat16).double().numpy()
    dout = rng.normal(0, 1, (n, d)).astype(np.float32).astype(np.float64)
    gq, gs = O.quantize_weight_128x128(wgu)
    dq, ds = O.quantize_weight_128x128(wd)
    x_deq = O.dequantize_act(*O.quantize_act_1x128(x.astype(np.float32)))
    got = O.swiglu_ffn_backward_fp8(x, x_deq, gq, gs, dq, ds, dout)
    ref = _torch_fp8_expert_backward(x, wgu, wd, dout)
    for key in ("dx", "dW_gate_up", "dW_down"):
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-11, atol=1e-11 * np.abs(ref[key]).max())
    for slip, key in (("no_bf16_before_quantising", "dx"), ("wgrad_tiles_along_columns", "dW_down"),
                      ("wgrad_x_from_forward_codes", "dW_gate_up"), ("cache_not_bf16", "dW_down")):
        bad = _torch_fp8_expert_backward(x, wgu, wd, dout, slip)
        assert np.abs(bad[key] - got[key]).max() > 1e-6 * np.abs(got[key]).max(), slip


def test_fp8_layer_backward_close_to_exact():
    """The FP8 backward of a small layer stays within the FP8 rounding of the
    exact one (normwise ~2^-4 at most), on every output."""
    cfg = PARITY_CONFIGS["small_fp8_ns2"] if "small_fp8_ns2" in PARITY_CONFIGS else CONFIGS["small_fp8"]
    inp = make_inputs(cfg, 3)
    u, E, b = to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy()
    wgu_all, wd_all = to_numpy_f32(inp.w_gate_up), to_numpy_f32(inp.w_down)
    routed = lambda e: (wgu_all[e], wd_all[e])
    shared = [(to_numpy_f32(inp.ws_gate_up[s]), to_numpy_f32(inp.ws_down[s])) for s in range(cfg.n_shared)]
    dy = np.random.default_rng(43).normal(0, 1, u.shape).astype(np.float32)
    r8 = O.layer_backward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared, dy, fp8=True)
    r = O.layer_backward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared, dy, selection=r8["idx"])
    rel = lambda a, c: np.linalg.norm(a - c) / np.linalg.norm(c)
    assert rel(r8["du"] - dy, r["du"] - dy) < 0.1
    for e in r["dW_down"]:
        assert rel(r8["dW_down"][e], r["dW_down"][e]) < 0.15
        assert rel(r8["dW_gate_up"][e], r["dW_gate_up"][e]) < 0.15
    for s in range(cfg.n_shared):
        assert rel(r8["dWs_down"][s], r["dWs_down"][s]) < 0.15
    assert rel(r8["dE"], r["dE"]) < 0.15
