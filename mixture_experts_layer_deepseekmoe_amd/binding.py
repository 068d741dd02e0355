"""ctypes binding over libmoe_mi355x.so (the C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch tensors provide device memory and the current HIP stream;
outputs and the workspace are allocated here with torch when the caller does
not pass them.  There is no fallback: if the library is missing, loading
fails with an error telling how to build it.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

# moe_dtype
F32, BF16, E4M3 = 0, 1, 2
DTYPE_CODE = {"f32": F32, "bf16": BF16, "e4m3": E4M3}
_TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16}

# moe_status
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH = range(5)

EXPORTED = ("moe_status_str", "moe_version", "moe_workspace_size", "moe_workspace_layout", "moe_route",
            "moe_forward", "moe_forward_static", "moe_train_workspace_size", "moe_forward_train", "moe_backward",
            "moe_update_bias", "moe_quantize_weight_e4m3", "moe_quantize_act_e4m3")

STATIC_SCRATCH_BYTES = 64 << 20   # MOE_STATIC_SCRATCH_BYTES


class MoEError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_str(code)} ({code})")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "d", "n_routed", "n_shared", "inter", "top_k", "x_dtype", "w_dtype", "out_dtype",
                 "n_groups", "topk_groups")]


WEIGHT_FIELDS = ("w_gate_up", "w_down", "ws_gate_up", "ws_down", "s_gate_up", "s_down", "ss_gate_up", "ss_down",
                 "w_gate_up_t", "w_down_t", "ws_gate_up_t", "ws_down_t",
                 "s_gate_up_t", "s_down_t", "ss_gate_up_t", "ss_down_t")


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


NUM_STAGES = 12
STAGES = ("route", "group", "quant", "gate_up", "down", "combine",
          "bwd_prep", "bwd_dgrad_down", "bwd_dgrad_gate_up", "bwd_wgrad_down", "bwd_wgrad_gate_up", "bwd_combine")
FORWARD_STAGES = STAGES[:6]
BACKWARD_STAGES = STAGES[6:]


class Trace(ctypes.Structure):
    _fields_ = [("start", ctypes.c_void_p * NUM_STAGES), ("stop", ctypes.c_void_p * NUM_STAGES)]


class WorkspaceMap(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("mtiles", "mt_count", "h", "h_scale", "y")] + \
               [(n, ctypes.c_int32) for n in ("max_mtiles", "tile_rows", "seg_cap")]


class WeightGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dw_gate_up", "dw_down", "dws_gate_up", "dws_down")]


class Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_gate", "expert_counts", "expert_offsets", "perm_token", "pos")]


DEBUG_LIB_PATH = os.path.join(_PKG, "libmoe_mi355x_debug.so")

_lib = None


def use_library(path: str) -> Optional[ctypes.CDLL]:
    """Make the binding call the library at ``path`` (e.g. DEBUG_LIB_PATH,
    the bounds-checked build); returns the previously loaded one."""
    global _lib
    prev = _lib
    _lib = _open(path)
    return prev


def restore_library(prev: Optional[ctypes.CDLL]) -> None:
    global _lib
    _lib = prev


def load_library() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m mixture_experts_layer_deepseekmoe_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_status_str.argtypes = [ctypes.c_int]
    lib.moe_version.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_workspace_size.restype = ctypes.c_int
    lib.moe_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(sz)]
    lib.moe_workspace_layout.restype = ctypes.c_int
    lib.moe_workspace_layout.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(WorkspaceMap)]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_route.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, ctypes.POINTER(Routing), vp, sz, vp]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, ctypes.POINTER(Weights), vp,
                                ctypes.POINTER(Routing), vp, sz, ctypes.POINTER(Trace), vp]
    lib.moe_forward_static.restype = ctypes.c_int
    lib.moe_forward_static.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, ctypes.POINTER(Weights), vp,
                                       ctypes.POINTER(Routing), ctypes.POINTER(Trace), vp]
    lib.moe_train_workspace_size.restype = ctypes.c_int
    lib.moe_train_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(sz)]
    lib.moe_forward_train.restype = ctypes.c_int
    lib.moe_forward_train.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, ctypes.POINTER(Weights), vp, vp, sz,
                                      ctypes.POINTER(Trace), vp]
    lib.moe_backward.restype = ctypes.c_int
    lib.moe_backward.argtypes = [ctypes.POINTER(Shape), vp, vp, ctypes.POINTER(Weights), vp, vp, vp,
                                 ctypes.POINTER(WeightGrads), vp, sz, ctypes.POINTER(Trace), vp]
    lib.moe_update_bias.restype = ctypes.c_int
    lib.moe_update_bias.argtypes = [vp, vp, i32, i64, ctypes.c_float, vp]
    lib.moe_quantize_weight_e4m3.restype = ctypes.c_int
    lib.moe_quantize_weight_e4m3.argtypes = [vp, i32, i64, i32, i32, vp, vp, vp]
    lib.moe_quantize_act_e4m3.restype = ctypes.c_int
    lib.moe_quantize_act_e4m3.argtypes = [vp, i32, i32, vp, vp, vp]
    return lib


def status_str(code: int) -> str:
    return load_library().moe_status_str(code).decode()


def version() -> str:
    return load_library().moe_version().decode()


def _check(code: int, what: str):
    if code != MOE_OK:
        raise MoEError(code, what)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the MoE library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclass
class LayerShape:
    T: int
    d: int
    n_routed: int
    n_shared: int
    inter: int
    top_k: int
    x_dtype: str = "bf16"
    w_dtype: str = "bf16"
    out_dtype: str = "f32"
    n_groups: int = 1        # group-limited routing: off unless 1 < topk_groups < n_groups
    topk_groups: int = 1

    @classmethod
    def from_config(cls, cfg, T: Optional[int] = None) -> "LayerShape":
        return cls(cfg.T if T is None else T, cfg.d, cfg.n_routed, cfg.n_shared, cfg.inter, cfg.top_k,
                   cfg.x_dtype, cfg.w_dtype, cfg.out_dtype, cfg.n_groups, cfg.topk_groups)

    def c(self) -> Shape:
        return Shape(self.T, self.d, self.n_routed, self.n_shared, self.inter, self.top_k,
                     DTYPE_CODE[self.x_dtype], DTYPE_CODE[self.w_dtype], DTYPE_CODE[self.out_dtype],
                     self.n_groups, self.topk_groups)


def workspace_size(shape: LayerShape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().moe_workspace_size(ctypes.byref(shape.c()), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def workspace_layout(shape: LayerShape) -> Dict[str, int]:
    """Byte offsets of moe_forward's intermediate results inside its workspace
    (the m-tile list, H, Y), with the list's capacity and tile size."""
    m = WorkspaceMap()
    _check(load_library().moe_workspace_layout(ctypes.byref(shape.c()), ctypes.byref(m)), "moe_workspace_layout")
    return {n: getattr(m, n) for n, _ in WorkspaceMap._fields_}


def alloc_workspace(shape: LayerShape, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_size(shape), 1), dtype=torch.uint8, device=device)


def alloc_routing(shape: LayerShape, device="cuda") -> Dict[str, torch.Tensor]:
    T, K, N = shape.T, shape.top_k, shape.n_routed
    i32 = torch.int32
    return {
        "topk_idx": torch.empty((T, K), dtype=i32, device=device),
        "topk_gate": torch.empty((T, K), dtype=torch.float32, device=device),
        "expert_counts": torch.empty((N,), dtype=i32, device=device),
        "expert_offsets": torch.empty((N + 1,), dtype=i32, device=device),
        "perm_token": torch.empty((T * K,), dtype=i32, device=device),
        "pos": torch.empty((T, K), dtype=i32, device=device),
    }


def _routing_struct(r: Optional[Dict[str, torch.Tensor]]) -> Optional[Routing]:
    if r is None:
        return None
    return Routing(*[_ptr(r.get(n)) for n, _ in Routing._fields_])


def moe_route(shape: LayerShape, u: torch.Tensor, centroids: torch.Tensor, bias: torch.Tensor,
              out: Optional[Dict[str, torch.Tensor]] = None,
              workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Routing only (affinities, biased top-K, gates, grouping).  Returns the routing tensors."""
    lib = load_library()
    out = alloc_routing(shape, u.device) if out is None else out
    ws = alloc_workspace(shape, u.device) if workspace is None else workspace
    rc = lib.moe_route(ctypes.byref(shape.c()), _ptr(u), _ptr(centroids), _ptr(bias),
                       ctypes.byref(_routing_struct(out)), _ptr(ws), ws.numel(), _stream())
    _check(rc, "moe_route")
    return out


@dataclass
class ExpertWeights:
    """Device expert weights (bf16/f32), or e4m3 codes (uint8) plus fp32 block
    scales; for the FP8 backward also the codes and scales transposed (*_t)."""
    w_gate_up: torch.Tensor
    w_down: torch.Tensor
    ws_gate_up: Optional[torch.Tensor] = None
    ws_down: Optional[torch.Tensor] = None
    s_gate_up: Optional[torch.Tensor] = None
    s_down: Optional[torch.Tensor] = None
    ss_gate_up: Optional[torch.Tensor] = None
    ss_down: Optional[torch.Tensor] = None
    w_gate_up_t: Optional[torch.Tensor] = None
    w_down_t: Optional[torch.Tensor] = None
    ws_gate_up_t: Optional[torch.Tensor] = None
    ws_down_t: Optional[torch.Tensor] = None
    s_gate_up_t: Optional[torch.Tensor] = None
    s_down_t: Optional[torch.Tensor] = None
    ss_gate_up_t: Optional[torch.Tensor] = None
    ss_down_t: Optional[torch.Tensor] = None

    def c(self) -> Weights:
        f = lambda t: None if t is None or t.numel() == 0 else _ptr(t)
        return Weights(*[f(getattr(self, n)) for n in WEIGHT_FIELDS])


def moe_forward(shape: LayerShape, u: torch.Tensor, centroids: torch.Tensor, bias: torch.Tensor,
                weights: ExpertWeights, y: Optional[torch.Tensor] = None,
                routing: Optional[Dict[str, torch.Tensor]] = None,
                workspace: Optional[torch.Tensor] = None, trace: Optional[Trace] = None) -> torch.Tensor:
    """The layer forward.  Returns y [T, d] in shape.out_dtype.  ``trace``: optional
    per-stage hipEvent pairs (see HipEvents)."""
    lib = load_library()
    if y is None:
        y = torch.empty((shape.T, shape.d), dtype=_TORCH_DT[DTYPE_CODE[shape.out_dtype]], device=u.device)
    ws = alloc_workspace(shape, u.device) if workspace is None else workspace
    rs = _routing_struct(routing)
    rc = lib.moe_forward(ctypes.byref(shape.c()), _ptr(u), _ptr(centroids), _ptr(bias),
                         ctypes.byref(weights.c()), _ptr(y), ctypes.byref(rs) if rs is not None else None,
                         _ptr(ws), ws.numel(), ctypes.byref(trace) if trace is not None else None, _stream())
    _check(rc, "moe_forward")
    return y


def moe_forward_static(shape: LayerShape, u: torch.Tensor, centroids: torch.Tensor, bias: torch.Tensor,
                       weights: ExpertWeights, y: torch.Tensor, routing: Optional[Dict[str, torch.Tensor]] = None,
                       trace: Optional[Trace] = None) -> torch.Tensor:
    """The layer forward on the library's own per-device scratch array (no
    workspace argument; the library allocates nothing).  ``y`` must be given
    (this call is for callers that cannot allocate).  Calls that overlap on
    one device race on that array."""
    lib = load_library()
    rs = _routing_struct(routing)
    rc = lib.moe_forward_static(ctypes.byref(shape.c()), _ptr(u), _ptr(centroids), _ptr(bias),
                                ctypes.byref(weights.c()), _ptr(y), ctypes.byref(rs) if rs is not None else None,
                                ctypes.byref(trace) if trace is not None else None, _stream())
    _check(rc, "moe_forward_static")
    return y


def train_workspace_size(shape: LayerShape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().moe_train_workspace_size(ctypes.byref(shape.c()), ctypes.byref(n)),
           "moe_train_workspace_size")
    return n.value


def alloc_train_workspace(shape: LayerShape, device="cuda") -> torch.Tensor:
    return torch.empty(max(train_workspace_size(shape), 1), dtype=torch.uint8, device=device)


def moe_forward_train(shape: LayerShape, u: torch.Tensor, centroids: torch.Tensor, bias: torch.Tensor,
                      weights: ExpertWeights, workspace: torch.Tensor, y: Optional[torch.Tensor] = None,
                      trace: Optional[Trace] = None) -> torch.Tensor:
    """The forward for training (bf16 activations; bf16 or e4m3 weights): y, and
    in ``workspace`` what moe_backward needs."""
    if y is None:
        y = torch.empty((shape.T, shape.d), dtype=_TORCH_DT[DTYPE_CODE[shape.out_dtype]], device=u.device)
    rc = load_library().moe_forward_train(ctypes.byref(shape.c()), _ptr(u), _ptr(centroids), _ptr(bias),
                                          ctypes.byref(weights.c()), _ptr(y), _ptr(workspace), workspace.numel(),
                                          ctypes.byref(trace) if trace is not None else None, _stream())
    _check(rc, "moe_forward_train")
    return y


@dataclass
class WeightGradTensors:
    """fp32 weight gradients in the layouts of ExpertWeights."""
    dw_gate_up: torch.Tensor
    dw_down: torch.Tensor
    dws_gate_up: Optional[torch.Tensor] = None
    dws_down: Optional[torch.Tensor] = None

    def c(self) -> WeightGrads:
        f = lambda t: None if t is None or t.numel() == 0 else _ptr(t)
        return WeightGrads(f(self.dw_gate_up), f(self.dw_down), f(self.dws_gate_up), f(self.dws_down))


def alloc_weight_grads(shape: LayerShape, device="cuda") -> WeightGradTensors:
    f32, I, d = torch.float32, shape.inter, shape.d
    return WeightGradTensors(torch.empty((shape.n_routed, 2 * I, d), dtype=f32, device=device),
                             torch.empty((shape.n_routed, d, I), dtype=f32, device=device),
                             torch.empty((shape.n_shared, 2 * I, d), dtype=f32, device=device),
                             torch.empty((shape.n_shared, d, I), dtype=f32, device=device))


def moe_backward(shape: LayerShape, u: torch.Tensor, centroids: torch.Tensor, weights: ExpertWeights,
                 dy: torch.Tensor, workspace: torch.Tensor, grads: Optional[WeightGradTensors] = None,
                 trace: Optional[Trace] = None):
    """Gradients for dy (fp32 [T, d]) after moe_forward_train on ``workspace``:
    returns (du [T, d] fp32, dcentroids [N_r, d] fp32, weight grads)."""
    du = torch.empty((shape.T, shape.d), dtype=torch.float32, device=u.device)
    dE = torch.empty((shape.n_routed, shape.d), dtype=torch.float32, device=u.device)
    grads = alloc_weight_grads(shape, u.device) if grads is None else grads
    rc = load_library().moe_backward(ctypes.byref(shape.c()), _ptr(u) if shape.T else None, _ptr(centroids),
                                     ctypes.byref(weights.c()), _ptr(dy) if shape.T else None,
                                     _ptr(du) if shape.T else None, _ptr(dE), ctypes.byref(grads.c()),
                                     _ptr(workspace), workspace.numel(),
                                     ctypes.byref(trace) if trace is not None else None, _stream())
    _check(rc, "moe_backward")
    return du, dE, grads


def moe_update_bias(bias: torch.Tensor, counts: torch.Tensor, total_assignments: int, gamma: float = 0.001):
    """In-place aux-loss-free bias update on the GPU."""
    rc = load_library().moe_update_bias(_ptr(bias), _ptr(counts), bias.numel(), int(total_assignments),
                                        float(gamma), _stream())
    _check(rc, "moe_update_bias")
    return bias


def moe_quantize_weight_e4m3(w: torch.Tensor):
    """[n, rows, cols] (or [rows, cols]) f32/bf16 -> (uint8 codes, fp32 scales [n, rows/128, cols/128])."""
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    n, rows, cols = w3.shape
    codes = torch.empty((n, rows, cols), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, rows // 128, cols // 128), dtype=torch.float32, device=w.device)
    code = {torch.float32: F32, torch.bfloat16: BF16}[w.dtype]
    rc = load_library().moe_quantize_weight_e4m3(_ptr(w3) if n else None, code, n, rows, cols,
                                                 _ptr(codes) if n else None, _ptr(scales) if n else None, _stream())
    _check(rc, "moe_quantize_weight_e4m3")
    return (codes[0], scales[0]) if squeeze else (codes, scales)


def moe_quantize_act_e4m3(x: torch.Tensor):
    """[rows, cols] bf16 -> (uint8 codes, fp32 scales [rows, cols/128])."""
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, cols // 128), dtype=torch.float32, device=x.device)
    rc = load_library().moe_quantize_act_e4m3(_ptr(x) if rows else None, rows, cols,
                                              _ptr(codes) if rows else None, _ptr(scales) if rows else None,
                                              _stream())
    _check(rc, "moe_quantize_act_e4m3")
    return codes, scales


def prepare_weights(cfg, inputs, train: bool = False) -> ExpertWeights:
    """Device weights for moe_forward from seeded inputs (quantised on the GPU
    for e4m3 configs).  ``train`` (e4m3): also the transposed codes and scales
    the FP8 backward reads, quantised from the transposed matrices (the same
    128x128 blocks)."""
    dev = torch.device("cuda")
    mv = lambda t: t.to(dev).contiguous()
    if cfg.w_dtype != "e4m3":
        return ExpertWeights(mv(inputs.w_gate_up), mv(inputs.w_down),
                             mv(inputs.ws_gate_up) if cfg.n_shared else None,
                             mv(inputs.ws_down) if cfg.n_shared else None)

    def q(t, transposed=False):
        t = t.to(dev)
        return moe_quantize_weight_e4m3((t.transpose(-1, -2) if transposed else t).contiguous())

    names = [("w_gate_up", "s_gate_up", inputs.w_gate_up), ("w_down", "s_down", inputs.w_down)]
    if cfg.n_shared:
        names += [("ws_gate_up", "ss_gate_up", inputs.ws_gate_up), ("ws_down", "ss_down", inputs.ws_down)]
    kw = {}
    for wn, sn, t in names:
        kw[wn], kw[sn] = q(t)
        if train:
            kw[wn + "_t"], kw[sn + "_t"] = q(t, True)
    return ExpertWeights(**kw)


class HipEvents:
    """Per-stage hipEvent pairs for moe_forward's trace argument, created
    through the HIP runtime (the same events the library records on its
    stream), with elapsed-time readout."""

    def __init__(self, stages=FORWARD_STAGES):
        """stages: the stage names to time (the library records no event
        for the others)."""
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.trace = Trace()
        self.idx = [STAGES.index(n) for n in stages]
        for i in self.idx:
            for arr in (self.trace.start, self.trace.stop):
                ev = ctypes.c_void_p()
                if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                arr[i] = ev.value

    def elapsed_ms(self) -> Dict[str, float]:
        out = {}
        for i in self.idx:
            name = STAGES[i]
            self.hip.hipEventSynchronize(self.trace.stop[i])
            ms = ctypes.c_float(0)
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.trace.start[i], self.trace.stop[i]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out[name] = ms.value
        return out

    def close(self):
        for i in self.idx:
            self.hip.hipEventDestroy(self.trace.start[i])
            self.hip.hipEventDestroy(self.trace.stop[i])
