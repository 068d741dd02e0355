"""Seeded input generators.

Every tensor is drawn from its own stream, keyed by (seed, config id, tensor
id, expert), so any one expert's weights can be drawn again on its own and the
order in which tensors are created does not matter.  Values are drawn in fp32
from N(0, std) and rounded to nearest-even into the config's storage dtype
(torch's fp32 -> bf16 cast rounds to nearest even).

Activations, centroids and biases are always drawn on the CPU with torch's
CPU generator (they are small).  Expert weights are drawn on ``weights_device``:
the CPU for small cases, the GPU for the full-size layers, whose weights run
to 22.5 GB at the DeepSeek-V3 shape.  The same seed gives the same values on a
given device kind; CPU and GPU streams differ from each other.
"""

from __future__ import annotations

import dataclasses
import json
import os
from typing import Optional

import numpy as np
import torch

from .configs import MoEConfig

_TENSOR_IDS = {
    "u": 1, "centroids": 2, "bias": 3, "w_gate_up": 4, "w_down": 5,
    "ws_gate_up": 6, "ws_down": 7, "zipf_rank": 8,
}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.bfloat16}

_SKEW_FILE = os.path.join(os.path.dirname(__file__), "skew_calibration.json")


def seed_for(seed: int, cfg_id: int, tensor: str, expert: int = -1) -> int:
    """A 63-bit seed for one tensor (or one expert's slice of it)."""
    ss = np.random.SeedSequence([seed, cfg_id, _TENSOR_IDS[tensor], expert + 1])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def _gen(device: torch.device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _normal(shape, std: float, s: int, dtype: torch.dtype, device="cpu") -> torch.Tensor:
    device = torch.device(device)
    x = torch.randn(shape, generator=_gen(device, s), dtype=torch.float32, device=device)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def skew_scale(cfg: MoEConfig, seed: int = 0) -> Optional[torch.Tensor]:
    """Per-expert centroid norm multipliers 1 + c * rank^(-s) for a Zipf-skewed router.

    Ranks 1..N_r are a seeded permutation over experts.  The constant c is the
    one stored in skew_calibration.json for this config and seed (it is tuned
    so that the initial max/mean expert load is about 10).
    """
    if cfg.zipf_s is None:
        return None
    g = _gen(torch.device("cpu"), seed_for(seed, cfg.cfg_id, "zipf_rank"))
    rank = torch.randperm(cfg.n_routed, generator=g).to(torch.float64) + 1.0
    c = load_skew_constant(cfg, seed)
    return 1.0 + c * rank.pow(-cfg.zipf_s)


def load_skew_constant(cfg: MoEConfig, seed: int = 0) -> float:
    key = f"{cfg.name}/seed{seed}"
    if os.path.exists(_SKEW_FILE):
        with open(_SKEW_FILE) as f:
            table = json.load(f)
        if key in table:
            return float(table[key]["c"])
    raise KeyError(f"no skew calibration stored for {key}; run oracle/calibrate_skew.py")


def make_centroids(cfg: MoEConfig, seed: int = 0, skew_c: Optional[float] = None) -> torch.Tensor:
    """Expert affinity vectors e_i, [N_r, d] in x_dtype (CPU)."""
    dt = _DT[cfg.x_dtype]
    e = _normal((cfg.n_routed, cfg.d), cfg.e_std, seed_for(seed, cfg.cfg_id, "centroids"), torch.float32)
    if cfg.zipf_s is not None:
        if skew_c is None:
            scale = skew_scale(cfg, seed)
        else:
            g = _gen(torch.device("cpu"), seed_for(seed, cfg.cfg_id, "zipf_rank"))
            rank = torch.randperm(cfg.n_routed, generator=g).to(torch.float64) + 1.0
            scale = 1.0 + skew_c * rank.pow(-cfg.zipf_s)
        e = (e.to(torch.float64) * scale[:, None]).to(torch.float32)
    return e.to(dt)


def make_expert_weights(cfg: MoEConfig, kind: str, n: int, rows: int, cols: int, seed: int = 0,
                        device="cpu", experts=None) -> torch.Tensor:
    """[n, rows, cols] weights, each expert from its own stream; bf16 for e4m3 configs."""
    dt = _DT[cfg.w_dtype]
    device = torch.device(device)
    ids = range(n) if experts is None else experts
    out = torch.empty((len(ids), rows, cols), dtype=dt, device=device)
    for j, e in enumerate(ids):
        out[j] = _normal((rows, cols), cfg.w_std, seed_for(seed, cfg.cfg_id, kind, e), dt, device)
    return out


@dataclasses.dataclass
class MoEInputs:
    cfg: MoEConfig
    u: torch.Tensor           # [T, d] x_dtype, CPU
    centroids: torch.Tensor   # [N_r, d] x_dtype, CPU
    bias: torch.Tensor        # [N_r] fp32, CPU
    w_gate_up: torch.Tensor   # [N_r, 2I, d]: rows 0..I-1 gate, I..2I-1 up
    w_down: torch.Tensor      # [N_r, d, I]
    ws_gate_up: torch.Tensor  # [N_s, 2I, d]
    ws_down: torch.Tensor     # [N_s, d, I]


def make_inputs(cfg: MoEConfig, seed: int = 0, weights_device="cpu", with_weights: bool = True) -> MoEInputs:
    dt = _DT[cfg.x_dtype]
    u = _normal((cfg.T, cfg.d), cfg.u_std, seed_for(seed, cfg.cfg_id, "u"), dt)
    cen = make_centroids(cfg, seed)
    if cfg.b_std > 0:
        b = _normal((cfg.n_routed,), cfg.b_std, seed_for(seed, cfg.cfg_id, "bias"), torch.float32)
    else:
        b = torch.zeros(cfg.n_routed, dtype=torch.float32)
    I, d = cfg.inter, cfg.d
    if with_weights:
        wgu = make_expert_weights(cfg, "w_gate_up", cfg.n_routed, 2 * I, d, seed, weights_device)
        wd = make_expert_weights(cfg, "w_down", cfg.n_routed, d, I, seed, weights_device)
        wsgu = make_expert_weights(cfg, "ws_gate_up", cfg.n_shared, 2 * I, d, seed, weights_device)
        wsd = make_expert_weights(cfg, "ws_down", cfg.n_shared, d, I, seed, weights_device)
    else:
        e = torch.empty(0)
        wgu = wd = wsgu = wsd = e
    return MoEInputs(cfg, u, cen, b, wgu, wd, wsgu, wsd)


def to_numpy_f32(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of an f32/bf16 tensor to a float32 numpy array on the host."""
    return t.detach().to(torch.float32).cpu().numpy()
