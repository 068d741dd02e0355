"""GPU parity: the HIP library (called through its C ABI) against the CPU oracle.

Bar: expert indices, counts, offsets, perm_token and pos bit-exact (near ties
within 1e-6 of the K-th biased score allowed and counted); gates to fp32
rounding; FP8 codes and scales of the quantisers bit-exact; outputs within
max|y_gpu - y_oracle| <= 1e-2 * rms(y_oracle) (bf16 and fp32 configs, beyond
the final rounding of a bf16-stored output: at most 2^-8 |y| per element) or
4e-2 * rms(y_oracle) on the raw error (FP8, whose bound is stated for a bf16
output); see tests/parity.py.  The full-size layers compare every token
routed to the first or last grouped row of any m-tile, and check the m-tile
list itself.
"""

import numpy as np
import pytest
import torch

import mixture_experts_layer_deepseekmoe_amd as moe
from moe_workloads import CONFIGS, PARITY_CONFIGS, MoEConfig, make_inputs, to_numpy_f32
from oracle import moe_oracle as O
from tests.parity import check_routing, expert_fns, output_errors, rows_of, say

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-2, "e4m3": 4e-2}
DEV = "cuda"


def _dev(inp):
    return (inp.u.to(DEV).contiguous(), inp.centroids.to(DEV).contiguous(), inp.bias.to(DEV).contiguous())


def _run_forward(cfg, inp, weights=None):
    """One forward through the C ABI; the routing dict also keeps the call's
    workspace (key "workspace"), for checks of the m-tile list."""
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = _dev(inp)
    w = moe.prepare_weights(cfg, inp) if weights is None else weights
    routing = moe.alloc_routing(shape)
    ws = moe.alloc_workspace(shape)
    y = moe.moe_forward(shape, u, E, b, w, routing=routing, workspace=ws)
    torch.cuda.synchronize()
    routing["workspace"] = ws
    return y, routing, w


# ------------------------------------------------------------------ quantisers

def test_quantize_weight_e4m3_bitexact():
    say("case: quantize_weight_e4m3 [3,256,384] bf16")
    g = torch.Generator().manual_seed(1)
    w = (torch.randn((3, 256, 384), generator=g) * 0.02).to(torch.bfloat16)
    w[1, :128, 128:256] = 0
    w[2, 128:, :128] *= 1000
    codes, scales = moe.moe_quantize_weight_e4m3(w.to(DEV))
    torch.cuda.synchronize()
    for m in range(3):
        q, s = O.quantize_weight_128x128(to_numpy_f32(w[m]))
        assert (codes[m].cpu().numpy() == q).all()
        assert (scales[m].cpu().numpy() == s).all()


def test_quantize_weight_e4m3_f32_source():
    say("case: quantize_weight_e4m3 [128,256] f32")
    g = torch.Generator().manual_seed(2)
    w = torch.randn((128, 256), generator=g) * 3
    codes, scales = moe.moe_quantize_weight_e4m3(w.to(DEV))
    torch.cuda.synchronize()
    q, s = O.quantize_weight_128x128(w.numpy())
    assert (codes.cpu().numpy() == q).all() and (scales.cpu().numpy() == s).all()


def test_quantize_act_e4m3_bitexact():
    say("case: quantize_act_e4m3 [37,640] bf16")
    g = torch.Generator().manual_seed(3)
    x = (torch.randn((37, 640), generator=g) * 2).to(torch.bfloat16)
    x[5, 128:256] = 0
    x[9, :] *= 1e-3
    codes, scales = moe.moe_quantize_act_e4m3(x.to(DEV))
    torch.cuda.synchronize()
    q, s = O.quantize_act_1x128(to_numpy_f32(x))
    assert (codes.cpu().numpy() == q).all()
    assert (scales.cpu().numpy() == s).all()


def test_quantize_act_e4m3_rounding_grid():
    """Tiles whose largest magnitude is 448 quantise with scale 1, so the
    codes are the conversion itself: every finite E4M3 value of both signs,
    every midpoint between neighbours (ties to the even code), each midpoint
    one bf16 step above and below, subnormal ties, and -0."""
    say("case: quantize_act_e4m3 rounding grid (scale 1)")
    mags = O.e4m3_decode(np.arange(0, 127)).astype(np.float64)
    mids = (mags[:-1] + mags[1:]) / 2
    ulp = np.exp2(np.floor(np.log2(np.maximum(mids, 2.0 ** -9))) - 7)   # bf16 step at the midpoint
    vals = np.concatenate([mags, mids, mids + ulp, mids - ulp, [2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -11]])
    vals = np.concatenate([vals, -vals, [-0.0]])
    xb = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)
    assert (xb.float().double().numpy() == vals).all()   # every value is a bf16 value
    per = 127
    ntiles = (len(vals) + per - 1) // per
    x = torch.zeros((ntiles, 128), dtype=torch.bfloat16)
    x[:, 0] = 448.0
    flat = torch.zeros(ntiles * per, dtype=torch.bfloat16)
    flat[: len(vals)] = xb
    x[:, 1:] = flat.view(ntiles, per)
    x = x.reshape(1, ntiles * 128).repeat(2, 1).contiguous()
    codes, scales = moe.moe_quantize_act_e4m3(x.to(DEV))
    torch.cuda.synchronize()
    q, sc = O.quantize_act_1x128(to_numpy_f32(x))
    assert (sc == 1.0).all()
    assert (scales.cpu().numpy() == sc).all()
    got = codes.cpu().numpy()
    bad = np.nonzero(got != q)
    assert bad[0].size == 0, [(float(to_numpy_f32(x)[r, c]), int(got[r, c]), int(q[r, c])) for r, c in zip(*bad)][:10]


# ------------------------------------------------------------------ routing

ROUTE_CASES = ["tiny_fp32"] + list(PARITY_CONFIGS)


@pytest.mark.parametrize("name", ROUTE_CASES)
def test_route_parity(name):
    cfg = CONFIGS.get(name) or PARITY_CONFIGS[name]
    say(f"case: moe_route {name}")
    inp = make_inputs(cfg, 0, with_weights=False)
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = _dev(inp)
    out = moe.moe_route(shape, u, E, b)
    torch.cuda.synchronize()
    r = check_routing(out, to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy(), cfg.top_k, cfg.n_routed)
    say(f"  near ties {r['near_ties']}, descending order {r['order_ok']}")


# Shapes on the router's K-split path (256-token tiles over slices of d):
# a ragged last token tile with 160 experts, and 67 pairs of K cut into 14
# slices whose last one holds 2 pairs.
ROUTE_KSPLIT_CASES = {
    "ksplit_ragged": MoEConfig("ksplit_ragged", T=5000, d=2048, n_routed=160, n_shared=1, inter=128, top_k=6,
                               x_dtype="bf16", w_dtype="bf16", out_dtype="f32", e_std=0.05, b_std=0.02, cfg_id=21),
    "ksplit_uneven": MoEConfig("ksplit_uneven", T=2100, d=4288, n_routed=256, n_shared=1, inter=128, top_k=8,
                               x_dtype="bf16", w_dtype="bf16", out_dtype="f32", e_std=0.02, b_std=0.01, cfg_id=22),
}


@pytest.mark.parametrize("name", list(ROUTE_KSPLIT_CASES))
def test_route_ksplit_parity(name):
    cfg = ROUTE_KSPLIT_CASES[name]
    say(f"case: moe_route {name} T={cfg.T} d={cfg.d} N_r={cfg.n_routed}")
    inp = make_inputs(cfg, 0, with_weights=False)
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = _dev(inp)
    out = moe.moe_route(shape, u, E, b)
    torch.cuda.synchronize()
    r = check_routing(out, to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy(), cfg.top_k, cfg.n_routed)
    say(f"  near ties {r['near_ties']}, descending order {r['order_ok']}")


# ------------------------------------------------------------------ forward, small

FWD_CASES = ["tiny_fp32"] + list(PARITY_CONFIGS)


@pytest.mark.parametrize("name", FWD_CASES)
def test_forward_parity(name):
    cfg = CONFIGS.get(name) or PARITY_CONFIGS[name]
    say(f"case: moe_forward {name}")
    inp = make_inputs(cfg, 0)
    y, routing, _ = _run_forward(cfg, inp)
    u, E, b = to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy()
    r = check_routing(routing, u, E, b, cfg.top_k, cfg.n_routed)
    routed, shared = expert_fns(inp, False)
    ref = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared,
                          selection=routing["topk_idx"].cpu().numpy(), fp8=cfg.fp8)
    err = output_errors(rows_of(y), ref["y"], u, cfg.out_dtype, cfg.w_dtype)
    say(f"  {err} near ties {r['near_ties']}")
    assert err["rel_to_rms"] <= TOL[cfg.w_dtype], err
    check_tile_list(cfg, moe.LayerShape.from_config(cfg), routing["workspace"], routing)


@pytest.mark.parametrize("name", ["small_bf16", "wide_router"])
def test_forward_trailing_experts_empty(name):
    """All tokens on experts 0..K-1: the experts after them hold no rows and
    must still fall inside the tile list's segments."""
    cfg = PARITY_CONFIGS[name]
    say(f"case: moe_forward {name}, all tokens on experts 0..K-1")
    inp = make_inputs(cfg, 0)
    _force_first_k(cfg, inp)
    y, routing, _ = _run_forward(cfg, inp)
    u, E, b = to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy()
    check_routing(routing, u, E, b, cfg.top_k, cfg.n_routed)
    counts = routing["expert_counts"].cpu().numpy()
    assert (counts[: cfg.top_k] == cfg.T).all() and (counts[cfg.top_k:] == 0).all()
    check_tile_list(cfg, moe.LayerShape.from_config(cfg), routing["workspace"], routing)
    routed, shared = expert_fns(inp, False)
    ref = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared,
                          selection=routing["topk_idx"].cpu().numpy(), fp8=cfg.fp8)
    err = output_errors(rows_of(y), ref["y"], u, cfg.out_dtype, cfg.w_dtype)
    say(f"  {err}")
    assert err["rel_to_rms"] <= TOL[cfg.w_dtype], err


def _random_shapes(n=16, seed=2024):
    """Seeded small layer shapes across the library's envelope: ragged T,
    N_r on both sides of 256, K up to 16, 0-3 shared experts, every dtype
    path; sizes bounded so the fp64 oracle stays quick."""
    rs = np.random.RandomState(seed)
    out = []
    for i in range(n):
        w = ["bf16", "bf16", "e4m3", "e4m3", "f32"][rs.randint(5)]
        x = "f32" if w == "f32" else "bf16"
        kmult = {"f32": 32, "bf16": 64, "e4m3": 128}[w]
        n_routed = int(rs.choice([int(rs.randint(1, 40)), int(rs.randint(40, 300))]))
        top_k = int(rs.randint(1, min(16, n_routed) + 1))
        d = kmult * int(rs.randint(1, 1024 // kmult + 1))
        inter = kmult * int(rs.randint(1, 768 // kmult + 1))
        while n_routed * d * inter > (1 << 24):   # keep the oracle's weights small
            if d >= inter and d > kmult:
                d -= kmult
            elif inter > kmult:
                inter -= kmult
            else:
                n_routed = max(top_k, n_routed // 2)
        T = int(rs.randint(1, 700))
        out.append(MoEConfig(f"rand{i}_{w}_T{T}_d{d}_I{inter}_Nr{n_routed}_K{top_k}", T=T, d=d,
                             n_routed=n_routed, n_shared=int(rs.randint(0, 4)), inter=inter, top_k=top_k,
                             x_dtype=x, w_dtype=w, out_dtype=["f32", "bf16"][rs.randint(2)],
                             w_std=0.03, e_std=0.05, b_std=0.02, cfg_id=100 + i))
    # the edges the draw may miss: more than 256 experts (two router chunks), a single expert
    out.append(MoEConfig("edge_bf16_T333_Nr300_K16", T=333, d=128, n_routed=300, n_shared=1, inter=128, top_k=16,
                         x_dtype="bf16", w_dtype="bf16", out_dtype="f32", w_std=0.03, e_std=0.05, b_std=0.02,
                         cfg_id=100 + n))
    out.append(MoEConfig("edge_bf16_T50_Nr1_K1", T=50, d=64, n_routed=1, n_shared=0, inter=64, top_k=1,
                         x_dtype="bf16", w_dtype="bf16", out_dtype="bf16", w_std=0.03, e_std=0.05, b_std=0.02,
                         cfg_id=101 + n))
    return out


RANDOM_SHAPES = _random_shapes()


@pytest.mark.parametrize("cfg", RANDOM_SHAPES, ids=[c.name for c in RANDOM_SHAPES])
def test_forward_random_shapes(cfg):
    say(f"case: moe_forward {cfg}")
    inp = make_inputs(cfg, 0)
    y, routing, _ = _run_forward(cfg, inp)
    u, E, b = to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy()
    r = check_routing(routing, u, E, b, cfg.top_k, cfg.n_routed)
    routed, shared = expert_fns(inp, False)
    ref = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared,
                          selection=routing["topk_idx"].cpu().numpy(), fp8=cfg.fp8)
    err = output_errors(rows_of(y), ref["y"], u, cfg.out_dtype, cfg.w_dtype)
    say(f"  T={cfg.T} N_s={cfg.n_shared} out={cfg.out_dtype}: {err} near ties {r['near_ties']}")
    assert err["rel_to_rms"] <= TOL[cfg.w_dtype], err
    check_tile_list(cfg, moe.LayerShape.from_config(cfg), routing["workspace"], routing)


def test_forward_replays_from_a_hip_graph():
    """The forward allocates, clears and synchronises nothing, so it can be
    captured into a HIP graph: each replay, with eager launches and host
    synchronisation between replays, matches the eager result bit for bit."""
    cfg = PARITY_CONFIGS["small_bf16_ns2"]
    say("case: moe_forward captured in a HIP graph, small_bf16_ns2")
    inp = make_inputs(cfg, 0)
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = _dev(inp)
    w = moe.prepare_weights(cfg, inp)
    ws = moe.alloc_workspace(shape)
    routing = moe.alloc_routing(shape)
    y = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device=DEV)
    moe.moe_forward(shape, u, E, b, w, y=y, routing=routing, workspace=ws)
    torch.cuda.synchronize()
    y_ref = y.clone()
    idx_ref = routing["topk_idx"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm up on the capture stream
        moe.moe_forward(shape, u, E, b, w, y=y, routing=routing, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(shape, u, E, b, w, y=y, routing=routing, workspace=ws)
    for rep in range(3):
        y.zero_()
        routing["topk_idx"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), rep
        assert torch.equal(routing["topk_idx"], idx_ref), rep
        # eager work between replays
        y2 = moe.moe_forward(shape, u, E, b, w)
        torch.cuda.synchronize()
        assert torch.equal(y2, y_ref), rep


def test_forward_empty_batch():
    cfg = PARITY_CONFIGS["small_bf16"].replace(T=0)
    say("case: moe_forward T=0")
    inp = make_inputs(cfg, 0)
    y, routing, _ = _run_forward(cfg, inp)
    assert y.shape == (0, cfg.d)
    assert (routing["expert_counts"].cpu() == 0).all()
    assert (routing["expert_offsets"].cpu() == 0).all()


def test_forward_deterministic_and_batch_invariant():
    cfg = PARITY_CONFIGS["small_bf16"]
    say("case: determinism / batch invariance small_bf16")
    inp = make_inputs(cfg, 0)
    y1, _, w = _run_forward(cfg, inp)
    y2, _, _ = _run_forward(cfg, inp, w)
    assert torch.equal(y1, y2)
    sub = torch.tensor([0, 5, 77, 299])
    inp_s = make_inputs(cfg, 0, with_weights=False)
    inp_s.u = inp.u[sub].contiguous()
    y3, _, _ = _run_forward(cfg.replace(T=len(sub)), inp_s, w)
    assert torch.equal(y3, y1[sub.to(DEV)])


def _check_grouping_valid(cfg, out):
    """Counts, offsets, perm_token and pos form a valid stable grouping of
    whatever selection the GPU made."""
    T, K, N = cfg.T, cfg.top_k, cfg.n_routed
    idx = out["topk_idx"].cpu().numpy()
    assert ((idx >= 0) & (idx < N)).all()
    assert all(len(set(row)) == K for row in idx.tolist())
    grp = O.group_by_expert(idx, N)
    for key, ref in (("expert_counts", grp["counts"]), ("expert_offsets", grp["offsets"]),
                     ("perm_token", grp["perm_token"]), ("pos", grp["pos"])):
        assert (out[key].cpu().numpy() == ref).all(), key


NAN_ROUTE_CASES = {
    "split_f32": CONFIGS["tiny_fp32"],                      # scores through scratch, f32 path
    "split_bf16": PARITY_CONFIGS["small_bf16"],             # scores through scratch
    "fused_bf16": CONFIGS["bf16_d2048"],                    # one kernel, logits in LDS
    "ksplit_bf16": ROUTE_KSPLIT_CASES["ksplit_ragged"],     # K slices summed in order
}


@pytest.mark.parametrize("name", list(NAN_ROUTE_CASES))
def test_route_nan_scores_give_k_distinct_experts(name):
    """A NaN in a token's activations makes all its scores NaN; the router
    still gives it K distinct in-range experts (a NaN score ranks below
    every number, so the K lowest indices win), the grouping stays a valid
    permutation, and every other token is routed exactly as the oracle
    routes it."""
    cfg = NAN_ROUTE_CASES[name]
    say(f"case: moe_route {name} with NaN tokens")
    inp = make_inputs(cfg, 0, with_weights=False)
    nan_tok = sorted({0, 7, cfg.T // 2, cfg.T - 1})
    inp.u = inp.u.clone()
    inp.u[nan_tok, 3] = float("nan")
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = _dev(inp)
    out = moe.moe_route(shape, u, E, b)
    torch.cuda.synchronize()
    _check_grouping_valid(cfg, out)
    idx = out["topk_idx"].cpu().numpy()
    assert (idx[nan_tok] == np.arange(cfg.top_k)[None, :]).all(), idx[nan_tok]
    ok = np.setdiff1d(np.arange(cfg.T), nan_tok)
    un = to_numpy_f32(inp.u)[ok]
    r = O.route(un, to_numpy_f32(inp.centroids), inp.bias.numpy(), cfg.top_k)
    from tests.parity import check_selection
    near = check_selection(r["v"], r["gap"], r["idx"], idx[ok], cfg.top_k)
    say(f"  {len(nan_tok)} NaN tokens on experts 0..K-1; the other {len(ok)} match the oracle ({near} near ties)")


def test_forward_nan_tokens_leave_the_others_exact():
    """The forward with NaN tokens: no out-of-range row anywhere, and the
    other tokens' outputs still match the oracle."""
    cfg = PARITY_CONFIGS["small_bf16"]
    say("case: moe_forward small_bf16 with NaN tokens")
    inp = make_inputs(cfg, 0)
    nan_tok = [0, 150, 299]
    inp.u = inp.u.clone()
    inp.u[nan_tok, 11] = float("nan")
    y, routing, _ = _run_forward(cfg, inp)
    _check_grouping_valid(cfg, routing)
    ok = np.setdiff1d(np.arange(cfg.T), nan_tok)
    u, E, b = to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy()
    routed, shared = expert_fns(inp, False)
    gi = routing["topk_idx"].cpu().numpy()
    ref = O.layer_forward(u[ok], E, b, cfg.top_k, routed, cfg.n_routed, shared, selection=gi[ok])
    err = output_errors(rows_of(y)[ok], ref["y"], u[ok], cfg.out_dtype, cfg.w_dtype)
    say(f"  {err}")
    assert err["rel_to_rms"] <= TOL[cfg.w_dtype], err


@pytest.mark.parametrize("name", ["bf16_d2048", "fp8_d2048"])
def test_forward_batch_invariant_with_multi_tile_experts(name):
    """At d = 2048 every expert holds ~384 rows, two m-tiles (three FP8
    ones); the same tokens run alone (one m-tile per expert, another router
    kernel with the same summation order) give bit-identical outputs."""
    cfg = CONFIGS[name]
    say(f"case: batch invariance {name} (several m-tiles per expert) vs 37 tokens alone")
    inp = make_inputs(cfg, 0, weights_device=DEV)
    y_full, routing, w = _run_forward(cfg, inp)
    counts = routing["expert_counts"].cpu().numpy()
    bm = moe.workspace_layout(moe.LayerShape.from_config(cfg))["tile_rows"]
    assert counts.max() > bm           # several experts span more than one m-tile
    sub = torch.tensor(sorted({0, 1, 5, 100, 255, 256, 511, 1000, 2047, 2048, 3001, 4094, 4095} |
                              set(range(1200, 1224))))
    inp_s = make_inputs(cfg, 0, with_weights=False)
    inp_s.u = inp.u[sub].contiguous()
    y_sub, r_sub, _ = _run_forward(cfg.replace(T=len(sub)), inp_s, w)
    assert torch.equal(r_sub["topk_idx"], routing["topk_idx"][sub.to(DEV)])
    assert torch.equal(y_sub, y_full[sub.to(DEV)])
    del w
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ bias update

def test_update_bias_bitexact():
    say("case: moe_update_bias")
    g = torch.Generator().manual_seed(4)
    n, TK = 256, 2048
    counts = torch.randint(0, 17, (n,), generator=g, dtype=torch.int32)
    counts[:5] = 8     # exactly the mean: unchanged
    bias = (torch.randn(n, generator=g) * 0.01).float()
    bd = bias.to(DEV)
    moe.moe_update_bias(bd, counts.to(DEV), TK, 0.001)
    torch.cuda.synchronize()
    ref = O.update_bias(bias.numpy(), counts.numpy(), TK)
    assert (bd.cpu().numpy() == ref).all()


def test_skewed_bias_loop_stepwise():
    """100 route + update steps on the decode-like skewed batch; every step
    is checked against the oracle from the GPU's own bias (step-wise parity)."""
    cfg = CONFIGS["skew_decode_d7168"]
    say("case: skew_decode_d7168 bias loop, 100 steps")
    inp = make_inputs(cfg, 0, with_weights=False)
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = _dev(inp)
    un, En = to_numpy_f32(inp.u), to_numpy_f32(inp.centroids)
    s = O.affinities(un, En)
    TK = cfg.T * cfg.top_k
    ratios = []
    near_total = 0
    for step in range(100):
        b_before = b.cpu().numpy().copy()
        out = moe.moe_route(shape, u, E, b)
        moe.moe_update_bias(b, out["expert_counts"], TK, 0.001)
        torch.cuda.synchronize()
        gi = out["topk_idx"].cpu().numpy()
        sel = O.select_topk(s, b_before, cfg.top_k)
        from tests.parity import check_selection
        near_total += check_selection(sel["v"], sel["gap"], sel["idx"], gi, cfg.top_k)
        counts = O.group_by_expert(gi, cfg.n_routed)["counts"]
        assert (out["expert_counts"].cpu().numpy() == counts).all()
        assert (b.cpu().numpy() == O.update_bias(b_before, counts, TK)).all(), f"step {step}"
        ratios.append(counts.max() / counts.mean())
    say(f"  max/mean load: step0 {ratios[0]:.2f} step10 {ratios[10]:.2f} step50 {ratios[50]:.2f} "
        f"step99 {ratios[-1]:.2f}; near ties {near_total}")
    assert ratios[0] >= 9.0
    assert ratios[-1] < ratios[0] / 2


# ------------------------------------------------------------------ full-size workloads

def _force_first_k(cfg, inp):
    """Every token selects experts 0..K-1 (a bias of +4 on them; sigmoid
    scores lie in (0, 1)), so all later experts get no rows."""
    inp.bias = inp.bias.clone()
    inp.bias[: cfg.top_k] += 4.0


def read_tile_list(shape, ws):
    """The grouped GEMMs' m-tile list and its segment starts, from the
    workspace of the last moe_forward call."""
    lay = moe.workspace_layout(shape)
    mt = ws[lay["mtiles"]: lay["mtiles"] + 16 * lay["max_mtiles"]].cpu().view(torch.int32).numpy().reshape(-1, 4)
    mc = ws[lay["mt_count"]: lay["mt_count"] + 40].cpu().view(torch.int32).numpy()
    n = int(mc[0])
    assert 0 <= n <= lay["max_mtiles"], (n, lay)
    return mt[:n].copy(), mc[1:10].copy(), lay


def check_tile_list(cfg, shape, ws, routing):
    """The m-tile list partitions every group's grouped rows into balanced
    tiles of at most tile_rows rows, units hold consecutive tiles of one
    group, and the segment starts (when the list is cut per XCD) are
    monotone, cover the list and fit the grid; returns the list."""
    tiles, seg, lay = read_tile_list(shape, ws)
    N, S, T, K = cfg.n_routed, cfg.n_shared, cfg.T, cfg.top_k
    bm = lay["tile_rows"]
    counts = routing["expert_counts"].cpu().numpy()
    offsets = routing["expert_offsets"].cpu().numpy()
    g, r0, rows, w = tiles[:, 0], tiles[:, 1], tiles[:, 2], tiles[:, 3]
    assert ((g >= 0) & (g < N + S)).all(), "group out of range"
    assert ((rows >= 1) & (rows <= bm)).all(), "tile rows out of range"
    for grp in range(N + S):
        first, M = (int(offsets[grp]), int(counts[grp])) if grp < N else (T * K + (grp - N) * T, T)
        idx = np.nonzero(g == grp)[0]
        assert len(idx) == -(-M // bm), (grp, len(idx), M)
        if M == 0:
            continue
        sel = tiles[idx[np.argsort(r0[idx])]]
        assert sel[0, 1] == first and sel[-1, 1] + sel[-1, 2] == first + M, grp
        assert (sel[:-1, 1] + sel[:-1, 2] == sel[1:, 1]).all(), grp
        assert sel[:, 2].max() - sel[:, 2].min() <= 1, grp          # balanced split
    idx_in, usz = w >> 8, w & 0xFF
    i = 0
    while i < len(tiles):
        k = int(usz[i])
        assert idx_in[i] == 0 and 1 <= k <= 4, i
        assert (idx_in[i:i + k] == np.arange(k)).all() and (usz[i:i + k] == k).all() and (g[i:i + k] == g[i]).all()
        assert (np.diff(r0[i:i + k]) > 0).all()
        i += k
    if seg[0] >= 0:
        assert seg[0] == 0 and seg[8] == len(tiles) and (np.diff(seg) >= 0).all(), seg
        assert (np.diff(seg) <= lay["seg_cap"]).all(), (seg, lay["seg_cap"])
        where = np.searchsorted(seg, np.arange(len(tiles)), side="right") - 1
        for grp in range(N):                                         # whole routed experts per segment
            assert len(set(where[g == grp].tolist())) <= 1, grp
    else:
        assert (seg == -1).all(), seg
    return tiles


def boundary_tokens(cfg, tiles, routing):
    """Tokens at the first and the last grouped row of every m-tile."""
    perm = routing["perm_token"].cpu().numpy()
    TK = cfg.T * cfg.top_k
    rows = np.unique(np.concatenate([tiles[:, 1], tiles[:, 1] + tiles[:, 2] - 1]))
    tok = np.where(rows < TK, perm[np.minimum(rows, TK - 1)] if TK else 0, (rows - TK) % max(cfg.T, 1))
    return np.unique(tok)


def _fp8_weight_fn(inp, n_routed, n_shared, routed_needed):
    """The oracle's 128x128 quantisation of every needed expert, computed in
    a thread pool (the oracle's own functions; NumPy releases the GIL) and
    handed to layer_forward through its fp8_weights hook."""
    import concurrent.futures
    import os

    def one(kind, e):
        src = (inp.w_gate_up, inp.w_down) if kind == "routed" else (inp.ws_gate_up, inp.ws_down)
        gq, gs = O.quantize_weight_128x128(to_numpy_f32(src[0][e]))
        dq, ds = O.quantize_weight_128x128(to_numpy_f32(src[1][e]))
        return gq, gs, dq, ds

    jobs = [("routed", int(e)) for e in routed_needed] + [("shared", s) for s in range(n_shared)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        done = dict(zip(jobs, ex.map(lambda j: one(*j), jobs)))
    return lambda kind, e: done[(kind, e)]


def _full_forward(name, first_k=False, extra=()):
    """A full-size layer in the launch configuration bench.py times: routing
    parity on every token, the m-tile list checked, and the oracle's output
    compared on the tokens at the first and last grouped row of every m-tile
    (plus ``extra``)."""
    cfg = CONFIGS[name]
    say(f"case: moe_forward {name} full size{' (all tokens on experts 0..K-1)' if first_k else ''}")
    inp = make_inputs(cfg, 0, weights_device=DEV)
    if first_k:
        _force_first_k(cfg, inp)
    shape = moe.LayerShape.from_config(cfg)
    u_d, E_d, b_d = _dev(inp)
    w = moe.prepare_weights(cfg, inp)
    ws = moe.alloc_workspace(shape)
    routing = moe.alloc_routing(shape)
    y = moe.moe_forward(shape, u_d, E_d, b_d, w, routing=routing, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    u, E, b = to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy()
    r = check_routing(routing, u, E, b, cfg.top_k, cfg.n_routed, cfg.n_groups, cfg.topk_groups)
    tiles = check_tile_list(cfg, shape, ws, routing)
    sample = np.unique(np.concatenate([boundary_tokens(cfg, tiles, routing), np.asarray(extra, np.int64)]))
    gi = routing["topk_idx"].cpu().numpy()
    say(f"  near ties {r['near_ties']}; {len(tiles)} m-tiles; oracle on {len(sample)} tokens "
        f"(first and last row of every m-tile)")
    fp8_w = None
    routed, shared = expert_fns(inp, True)
    if cfg.fp8:
        fp8_w = _fp8_weight_fn(inp, cfg.n_routed, cfg.n_shared, np.unique(gi[sample]))
        routed = lambda e: (None, None)
        shared = [(None, None)] * cfg.n_shared
    ref = O.layer_forward(u[sample], E, b, cfg.top_k, routed, cfg.n_routed, shared, selection=gi[sample],
                          fp8=cfg.fp8, fp8_weights=fp8_w)
    yg = rows_of(y[torch.as_tensor(sample, device=DEV)])
    err = output_errors(yg, ref["y"], u[sample], cfg.out_dtype, cfg.w_dtype)
    say(f"  sampled output error {err}")
    assert err["rel_to_rms"] <= TOL[cfg.w_dtype], err
    if first_k:
        counts = routing["expert_counts"].cpu().numpy()
        assert (counts[: cfg.top_k] == cfg.T).all() and (counts[cfg.top_k:] == 0).all()
    del w, inp, ws
    torch.cuda.empty_cache()


def test_full_bf16_d2048():
    _full_forward("bf16_d2048", extra=[0, 4095])


def test_full_bf16_d7168():
    _full_forward("bf16_d7168", extra=[0, 8191])


def test_full_bf16_d7168_trailing_experts_empty():
    # 8 experts with 8192 rows each: 256 routed m-tiles, the cost-cut segments
    _full_forward("bf16_d7168", first_k=True)


def test_full_fp8_d2048():
    _full_forward("fp8_d2048", extra=[0, 4095])


def test_full_fp8_d7168():
    _full_forward("fp8_d7168", extra=[0, 8191])


def test_full_skew_decode_d7168():
    _full_forward("skew_decode_d7168", extra=[0, 255])


def test_full_bf16_d7168_group_limited():
    # 8 groups of 32 experts, at most 4 per token (q = 2)
    _full_forward("bf16_d7168_g8", extra=[0, 8191])


# ------------------------------------------------------------------ group-limited routing, small

GROUPED_CASES = {
    "small_bf16_g4k2": PARITY_CONFIGS["small_bf16"].replace(name="small_bf16_g4k2", n_groups=4, topk_groups=2),
    "small_bf16_ns2_g6k3": PARITY_CONFIGS["small_bf16_ns2"].replace(name="small_bf16_ns2_g6k3", n_groups=6,
                                                                     topk_groups=3),
    "small_fp32_g5k2": PARITY_CONFIGS["small_fp32"].replace(name="small_fp32_g5k2", n_groups=5, topk_groups=2),
    "small_fp8_g8k3": PARITY_CONFIGS["small_fp8"].replace(name="small_fp8_g8k3", n_groups=8, topk_groups=3),
    "wide_router_g16k4": PARITY_CONFIGS["wide_router"].replace(name="wide_router_g16k4", n_groups=16, topk_groups=4),
    "ksplit_ragged_g8k3": ROUTE_KSPLIT_CASES["ksplit_ragged"].replace(name="ksplit_ragged_g8k3", n_groups=8,
                                                                      topk_groups=3),
    "fused_d2048_g8k2": CONFIGS["bf16_d2048"].replace(name="fused_d2048_g8k2", n_groups=8, topk_groups=2),
}


@pytest.mark.parametrize("name", list(GROUPED_CASES))
def test_route_group_limited(name):
    """Group-limited routing on every router path (scores through scratch,
    the fused kernel, the K-split kernels; fp32 and bf16; 512 experts)."""
    cfg = GROUPED_CASES[name]
    say(f"case: moe_route {name} (groups {cfg.n_groups}, keep {cfg.topk_groups})")
    inp = make_inputs(cfg, 0, with_weights=False)
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = _dev(inp)
    out = moe.moe_route(shape, u, E, b)
    torch.cuda.synchronize()
    r = check_routing(out, to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy(), cfg.top_k,
                      cfg.n_routed, cfg.n_groups, cfg.topk_groups)
    glob = O.route(to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy(), cfg.top_k)["idx"]
    differ = int((np.sort(glob, 1) != np.sort(out["topk_idx"].cpu().numpy(), 1)).any(1).sum())
    say(f"  near ties {r['near_ties']}; {differ} of {cfg.T} tokens select otherwise than global top-K")


@pytest.mark.parametrize("name", ["small_bf16_g4k2", "small_fp8_g8k3", "small_fp32_g5k2"])
def test_forward_group_limited(name):
    cfg = GROUPED_CASES[name]
    say(f"case: moe_forward {name}")
    inp = make_inputs(cfg, 0)
    y, routing, _ = _run_forward(cfg, inp)
    u, E, b = to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy()
    check_routing(routing, u, E, b, cfg.top_k, cfg.n_routed, cfg.n_groups, cfg.topk_groups)
    routed, shared = expert_fns(inp, False)
    ref = O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared,
                          selection=routing["topk_idx"].cpu().numpy(), fp8=cfg.fp8)
    err = output_errors(rows_of(y), ref["y"], u, cfg.out_dtype, cfg.w_dtype)
    say(f"  {err}")
    assert err["rel_to_rms"] <= TOL[cfg.w_dtype], err
    check_tile_list(cfg, moe.LayerShape.from_config(cfg), routing["workspace"], routing)
