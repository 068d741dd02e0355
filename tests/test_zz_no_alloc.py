"""moe_forward_static (the entry point that allocates nothing; its workspace
is the library's per-device scratch array) against moe_forward on the same
inputs: bit-identical outputs and routing, on two calls in a row whose
second is smaller (the array keeps the first call's contents), for the bf16,
FP8 and fp32 paths and the decode-sized d = 7168 layer."""

import numpy as np
import pytest
import torch

import mixture_experts_layer_deepseekmoe_amd as moe
from mixture_experts_layer_deepseekmoe_amd import binding as B
from moe_workloads import CONFIGS, PARITY_CONFIGS, make_inputs
from tests.parity import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(cfg, inp, w, T):
    shape = moe.LayerShape.from_config(cfg, T=T)
    u = inp.u[:T].to(DEV).contiguous()
    E, b = inp.centroids.to(DEV).contiguous(), inp.bias.to(DEV).contiguous()
    ydt = torch.float32 if cfg.out_dtype == "f32" else torch.bfloat16
    r_ref, r_st = moe.alloc_routing(shape), moe.alloc_routing(shape)
    y_ref = moe.moe_forward(shape, u, E, b, w, routing=r_ref)
    y_st = torch.full((T, cfg.d), float("nan"), dtype=ydt, device=DEV)
    moe.moe_forward_static(shape, u, E, b, w, y_st, routing=r_st)
    torch.cuda.synchronize()
    assert torch.equal(y_st, y_ref), (cfg.name, T)
    for k in r_ref:
        assert torch.equal(r_st[k], r_ref[k]), (cfg.name, T, k)


@pytest.mark.parametrize("name,T1,T2", [("small_bf16", 300, 129), ("small_fp8_ns2", 517, 200),
                                        ("small_fp32", 200, 37), ("skew_decode_d7168", 256, 64)])
def test_forward_static_matches_forward(name, T1, T2):
    cfg = CONFIGS.get(name) or PARITY_CONFIGS[name]
    say(f"case: moe_forward_static vs moe_forward, {name}, T = {T1} then {T2}")
    inp = make_inputs(cfg, 0, weights_device=DEV)
    w = moe.prepare_weights(cfg, inp)
    assert moe.workspace_size(moe.LayerShape.from_config(cfg, T=T1)) <= B.STATIC_SCRATCH_BYTES
    _pair(cfg, inp, w, T1)
    _pair(cfg, inp, w, T2)
    del w, inp
    torch.cuda.empty_cache()


def test_forward_static_rejects_a_shape_beyond_its_scratch():
    cfg = CONFIGS["bf16_d7168"]
    shape = moe.LayerShape.from_config(cfg)
    assert moe.workspace_size(shape) > B.STATIC_SCRATCH_BYTES
    say("case: moe_forward_static rejects the 8192-token d = 7168 layer")
    inp = make_inputs(cfg.replace(T=1), 0, with_weights=False)
    u = torch.zeros((cfg.T, cfg.d), dtype=torch.bfloat16, device=DEV)
    E, b = inp.centroids.to(DEV), inp.bias.to(DEV)
    dummy = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    w = moe.ExpertWeights(dummy, dummy, dummy, dummy)
    y = torch.zeros((cfg.T, cfg.d), dtype=torch.float32, device=DEV)
    with pytest.raises(moe.MoEError) as e:
        moe.moe_forward_static(shape, u, E, b, w, y)
    assert e.value.code == B.MOE_ERR_WORKSPACE
