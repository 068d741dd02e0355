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

    def tq_act(a):          # 1x128 tiles
        a = torch.from_numpy(a)
        t = a.view(a.shape[0], -1, 128)
        amax = t.abs().amax(-1, keepdim=True)
        scale = amax / 448.0
        q = (t * (448.0 / amax)).to(torch.float8_e4m3fn).to(torch.float64)
        return (q * scale.to(torch.float64)).view_as(a).to(torch.float64)

    def tq_w(w):            # 128x128 blocks
        w = torch.from_numpy(w)
        R, C = w.shape
        t = w.view(R // 128, 128, C // 128, 128)
        amax = t.abs().amax(dim=(1, 3), keepdim=True)
        q = (t * (448.0 / amax)).to(torch.float8_e4m3fn).to(torch.float64)
        return (q * (amax / 448.0).to(torch.float64)).view(R, C)

    xd, gd, dd = tq_act(x), tq_w(wgu), tq_w(wd)
    g, u = xd @ gd[:128].T, xd @ gd[128:].T
    h = (torch.nn.functional.silu(g) * u).to(torch.float32).numpy()
    ref = (tq_act(h) @ dd.T).numpy()

    xq, xs = O.quantize_act_1x128(x)
    gq, gs = O.quantize_weight_128x128(wgu)
    dq, ds = O.quantize_weight_128x128(wd)
    out = O.swiglu_ffn_fp8(O.dequantize_act(xq, xs), gq, gs, dq, ds)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
