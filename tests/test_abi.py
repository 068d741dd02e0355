"""C-ABI contract on the CPU: the library loads, exports every entry point that
include/moe.h declares, and rejects bad arguments before any GPU work (no
call here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

import mixture_experts_layer_deepseekmoe_amd as moe
from mixture_experts_layer_deepseekmoe_amd import binding as B
from moe_workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(moe_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert _declared() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = moe.load_library()
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    assert moe.status_str(0) == "MOE_OK"
    for c in range(1, 5):
        assert moe.status_str(c).startswith("MOE_ERR")
    assert "unknown" in moe.status_str(99)
    assert "gfx950" in moe.version()


def _shape(**kw):
    base = dict(T=64, d=128, n_routed=8, n_shared=1, inter=128, top_k=2, x_dtype="bf16", w_dtype="bf16",
                out_dtype="f32")
    base.update(kw)
    return moe.LayerShape(**base)


def _ws_rc(shape):
    n = ctypes.c_size_t(0)
    return moe.load_library().moe_workspace_size(ctypes.byref(shape.c()), ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,code", [
    (dict(top_k=9), B.MOE_ERR_INVALID_ARG),           # K > N_r
    (dict(top_k=0), B.MOE_ERR_INVALID_ARG),
    (dict(T=-1), B.MOE_ERR_INVALID_ARG),
    (dict(d=0), B.MOE_ERR_INVALID_ARG),
    (dict(x_dtype="f32"), B.MOE_ERR_INVALID_ARG),      # f32 activations with bf16 weights
    (dict(x_dtype="e4m3", w_dtype="e4m3"), B.MOE_ERR_INVALID_ARG),
    (dict(out_dtype="e4m3"), B.MOE_ERR_INVALID_ARG),
    (dict(n_routed=600, top_k=2), B.MOE_ERR_UNSUPPORTED),
    (dict(n_routed=64, top_k=17), B.MOE_ERR_UNSUPPORTED),
    (dict(n_shared=9), B.MOE_ERR_UNSUPPORTED),
    (dict(d=96), B.MOE_ERR_UNSUPPORTED),               # bf16 needs d % 64 == 0
    (dict(w_dtype="e4m3", d=192), B.MOE_ERR_UNSUPPORTED),   # e4m3 needs d % 128 == 0
    (dict(w_dtype="e4m3", inter=64), B.MOE_ERR_UNSUPPORTED),
    (dict(T=2 ** 28, top_k=8), B.MOE_ERR_UNSUPPORTED),       # T*K beyond int32
    (dict(T=299_594, d=7168, top_k=1), B.MOE_ERR_UNSUPPORTED),   # bytes of u reach 2^32 (32-bit offsets)
    (dict(inter=65_536, d=16_384, top_k=1), B.MOE_ERR_UNSUPPORTED),   # one expert's gate/up matrix reaches 2^32 bytes
])
def test_shape_validation(kw, code):
    rc, _ = _ws_rc(_shape(**kw))
    assert rc == code


def test_training_shape_validation():
    def rc(shape):
        n = ctypes.c_size_t(0)
        return moe.load_library().moe_train_workspace_size(ctypes.byref(shape.c()), ctypes.byref(n))
    assert rc(_shape()) == B.MOE_OK
    assert rc(_shape(w_dtype="e4m3", inter=128)) == B.MOE_OK
    assert rc(_shape(x_dtype="f32", w_dtype="f32")) == B.MOE_ERR_UNSUPPORTED   # training takes bf16 activations
    # a group's [dG dU] rows (T x 2I bf16) reach 2^32 bytes, though the forward's
    # own 32-bit offsets (u, one expert's weights) still fit
    big = _shape(T=131_072, d=1024, inter=8192, top_k=1)
    assert _ws_rc(big)[0] == B.MOE_OK and rc(big) == B.MOE_ERR_UNSUPPORTED
    assert rc(_shape(T=131_071, d=1024, inter=8192, top_k=1)) == B.MOE_OK


def test_largest_activation_within_32_bit_offsets_is_accepted():
    # T * d * 2 bytes just below 2^32
    rc, _ = _ws_rc(_shape(T=299_593, d=7168, top_k=1))
    assert rc == B.MOE_OK


def test_valid_shapes_and_workspace_monotone():
    sizes = []
    for T in (0, 1, 64, 4096):
        rc, n = _ws_rc(_shape(T=T))
        assert rc == 0
        sizes.append(n)
    assert sizes == sorted(sizes) and sizes[-1] > sizes[0]
    for cfg in CONFIGS.values():
        assert _ws_rc(moe.LayerShape.from_config(cfg))[0] == 0
    rc, _ = _ws_rc(_shape(x_dtype="f32", w_dtype="f32", d=32, inter=32))
    assert rc == 0


def test_workspace_holds_the_router_scratch():
    # d = 7168, 256 experts: 8192 tokens take the K-split router (8 slices of fp32 logits), 4096 tokens 16
    # slices, 256 tokens the expert-split router (one [T][N_r] block of sigmoids)
    def ws(T):
        return _ws_rc(_shape(T=T, d=7168, n_routed=256, top_k=8, inter=2048))[1]
    assert ws(8192) >= 8 * 8192 * 256 * 4
    assert ws(4096) >= 16 * 4096 * 256 * 4
    assert ws(256) >= 256 * 256 * 4
    # 254 experts (not a multiple of 4) stay on the fused router: no slice logits, the rest of the layout nearly equal
    n254 = _ws_rc(_shape(T=8192, d=7168, n_routed=254, top_k=8, inter=2048))[1]
    assert ws(8192) - n254 >= 8 * 8192 * 256 * 4 - (1 << 20)


FAKE = 1 << 20          # 16-byte aligned, never dereferenced: every call below fails validation


def test_route_rejects_bad_arguments_before_launch():
    lib = moe.load_library()
    sh = _shape()
    r = B.Routing(*[FAKE] * 6)
    ws_need = _ws_rc(sh)[1]
    # missing workspace / too small
    assert lib.moe_route(ctypes.byref(sh.c()), FAKE, FAKE, FAKE, ctypes.byref(r), None, 0, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(sh.c()), FAKE, FAKE, FAKE, ctypes.byref(r), FAKE, ws_need - 1,
                         None) == B.MOE_ERR_WORKSPACE
    # null outputs, misaligned input
    r2 = B.Routing(FAKE, None, FAKE, FAKE, FAKE, FAKE)
    assert lib.moe_route(ctypes.byref(sh.c()), FAKE, FAKE, FAKE, ctypes.byref(r2), FAKE, ws_need,
                         None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(sh.c()), FAKE + 4, FAKE, FAKE, ctypes.byref(r), FAKE, ws_need,
                         None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route(None, FAKE, FAKE, FAKE, ctypes.byref(r), FAKE, ws_need, None) == B.MOE_ERR_INVALID_ARG


def test_forward_rejects_bad_arguments_before_launch():
    lib = moe.load_library()
    sh = _shape()
    ws_need = _ws_rc(sh)[1]
    w = B.Weights(FAKE, FAKE, FAKE, FAKE, None, None, None, None)
    fwd = lambda shape, weights, ws=FAKE, wsb=ws_need, u=FAKE, y=FAKE: lib.moe_forward(
        ctypes.byref(shape.c()), u, FAKE, FAKE, ctypes.byref(weights) if weights else None, y, None, ws, wsb, None,
        None)
    assert fwd(sh, None) == B.MOE_ERR_INVALID_ARG
    assert fwd(sh, B.Weights(FAKE, FAKE, None, None, None, None, None, None)) == B.MOE_ERR_INVALID_ARG  # N_s=1
    assert fwd(sh, w, wsb=ws_need - 256) == B.MOE_ERR_WORKSPACE
    assert fwd(sh, w, y=FAKE + 8) == B.MOE_ERR_INVALID_ARG
    sh8 = _shape(w_dtype="e4m3", out_dtype="bf16")
    assert fwd(sh8, w, wsb=_ws_rc(sh8)[1]) == B.MOE_ERR_INVALID_ARG    # e4m3 needs the scale arrays
    assert fwd(_shape(top_k=20), w) == B.MOE_ERR_INVALID_ARG


def test_other_entry_points_validate():
    lib = moe.load_library()
    assert lib.moe_update_bias(None, FAKE, 8, 16, 0.001, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_update_bias(FAKE, FAKE, 0, 16, 0.001, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_update_bias(FAKE, FAKE, 8, -1, 0.001, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_weight_e4m3(FAKE, B.BF16, 1, 100, 128, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_quantize_weight_e4m3(FAKE, B.E4M3, 1, 128, 128, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_weight_e4m3(FAKE, B.BF16, 0, 128, 128, FAKE, FAKE, None) == B.MOE_OK   # nothing to do
    assert lib.moe_quantize_act_e4m3(FAKE, 4, 100, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_quantize_act_e4m3(None, 4, 128, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        B._ptr(torch.zeros(4))


@pytest.mark.parametrize("name", list(CONFIGS))
def test_workspace_layout_lies_inside_the_workspace(name):
    cfg = CONFIGS[name]
    shape = moe.LayerShape.from_config(cfg)
    total = moe.workspace_size(shape)
    lay = moe.workspace_layout(shape)
    R = cfg.T * cfg.top_k + cfg.n_shared * cfg.T
    es = {"f32": 4, "bf16": 2, "e4m3": 1}[cfg.w_dtype]
    ys = 4 if cfg.w_dtype == "f32" else 2
    spans = [(lay["mtiles"], 16 * lay["max_mtiles"]), (lay["mt_count"], 40), (lay["h"], R * cfg.inter * es),
             (lay["y"], R * cfg.d * ys)]
    if cfg.fp8:
        spans.append((lay["h_scale"], R * (cfg.inter // 128) * 4))
    for off, n in spans:
        assert off % 256 == 0 and off + n <= total, (off, n, total)
    spans.sort()
    for (o0, n0), (o1, _) in zip(spans, spans[1:]):
        assert o0 + n0 <= o1                      # no two of them overlap
    assert lay["tile_rows"] == (256 if cfg.w_dtype == "bf16" else 128)
    assert lay["seg_cap"] * 8 >= lay["max_mtiles"]


@pytest.mark.parametrize("kw,code", [
    (dict(n_routed=256, top_k=8, n_groups=8, topk_groups=4), B.MOE_OK),
    (dict(n_routed=256, top_k=8, n_groups=8, topk_groups=8), B.MOE_OK),      # every group kept: global top-K
    (dict(n_routed=256, top_k=8, n_groups=0, topk_groups=0), B.MOE_OK),      # off
    (dict(n_routed=256, top_k=8, n_groups=7, topk_groups=3), B.MOE_ERR_INVALID_ARG),    # 7 does not divide 256
    (dict(n_routed=256, top_k=8, n_groups=8, topk_groups=0), B.MOE_ERR_INVALID_ARG),
    (dict(n_routed=256, top_k=8, n_groups=8, topk_groups=9), B.MOE_ERR_INVALID_ARG),
    (dict(n_routed=32, top_k=8, n_groups=16, topk_groups=3), B.MOE_ERR_INVALID_ARG),    # 3 groups of 2 < K
    (dict(n_routed=256, top_k=8, n_groups=128, topk_groups=8), B.MOE_ERR_UNSUPPORTED),  # more than 64 groups
    (dict(n_routed=256, top_k=8, n_groups=-1, topk_groups=1), B.MOE_ERR_INVALID_ARG),
])
def test_group_limited_routing_validation(kw, code):
    rc, _ = _ws_rc(_shape(**kw))
    assert rc == code
