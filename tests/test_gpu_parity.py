"""GPU parity: the HIP library (called through its C ABI) against the CPU oracle.

Bar: expert indices, counts, offsets, perm_token and pos bit-exact (near ties
within 1e-6 of the K-th biased score allowed and counted); gates to fp32
rounding; FP8 codes and scales of the quantisers bit-exact; outputs within
max|y_gpu - y_oracle| <= 1e-2 * rms(y_oracle) (bf16 and fp32 configs) or
4e-2 * rms(y_oracle) (FP8), beyond the final rounding of a bf16-stored output
(at most 2^-8 |y| per element; see tests/parity.py).
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
    shape = moe.LayerShape.from_config(cfg)
    u, E, b = _dev(inp)
    w = moe.prepare_weights(cfg, inp) if weights is None else weights
    routing = moe.alloc_routing(shape)
    y = moe.moe_forward(shape, u, E, b, w, routing=routing)
    torch.cuda.synchronize()
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


def _sampled_forward(name, sample, first_k=False):
    cfg = CONFIGS[name]
    say(f"case: moe_forward {name} full size{' (all tokens on experts 0..K-1)' if first_k else ''}, "
        f"oracle on tokens {sample}")
    inp = make_inputs(cfg, 0, weights_device=DEV)
    if first_k:
        _force_first_k(cfg, inp)
    y, routing, w = _run_forward(cfg, inp)
    u, E, b = to_numpy_f32(inp.u), to_numpy_f32(inp.centroids), inp.bias.numpy()
    r = check_routing(routing, u, E, b, cfg.top_k, cfg.n_routed)
    routed, shared = expert_fns(inp, True)
    gi = routing["topk_idx"].cpu().numpy()
    ref = O.layer_forward(u[sample], E, b, cfg.top_k, routed, cfg.n_routed, shared, selection=gi[sample],
                          fp8=cfg.fp8)
    yg = rows_of(y[torch.tensor(sample, device=DEV)])
    err = output_errors(yg, ref["y"], u[sample], cfg.out_dtype, cfg.w_dtype)
    say(f"  near ties {r['near_ties']}; sampled output error {err}")
    assert err["rel_to_rms"] <= TOL[cfg.w_dtype], err
    assert torch.isfinite(y).all()
    if first_k:
        counts = routing["expert_counts"].cpu().numpy()
        assert (counts[: cfg.top_k] == cfg.T).all() and (counts[cfg.top_k:] == 0).all()
    del w, inp
    torch.cuda.empty_cache()


def test_full_bf16_d2048():
    _sampled_forward("bf16_d2048", [0, 1, 2047, 4095, 1234, 3000])


def test_full_bf16_d7168():
    _sampled_forward("bf16_d7168", [0, 4097, 8191, 2500])


def test_full_bf16_d7168_trailing_experts_empty():
    # 8 experts with 8192 rows each: 256 routed m-tiles, the cost-cut segments
    _sampled_forward("bf16_d7168", [0, 8191, 1000], first_k=True)


def test_full_fp8_d2048():
    _sampled_forward("fp8_d2048", [0, 4095, 777])


def test_full_fp8_d7168():
    _sampled_forward("fp8_d7168", [0, 8191, 3333])


def test_full_skew_decode_d7168():
    _sampled_forward("skew_decode_d7168", [0, 100, 255])
