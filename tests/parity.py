"""Helpers for comparing the GPU library with the CPU oracle.

Routing comparison (selection is discrete, so it must match exactly except
where the biased scores are within 1e-6 of a tie):
  * tokens whose oracle gap v_(K) - v_(K+1) exceeds 1e-6: the GPU's set of
    experts equals the oracle's;
  * near-tie tokens: the GPU's set holds every expert with v > v_(K) + 1e-6
    and only experts with v >= v_(K) - 1e-6; they are counted and reported.
The oracle then adopts the GPU's selection, so grouping (counts, offsets,
perm_token, pos) is compared bit-exactly and outputs element-wise.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

from moe_workloads import to_numpy_f32
from oracle import moe_oracle as O

BAND = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_selection(v: np.ndarray, gap: np.ndarray, oracle_idx: np.ndarray, gpu_idx: np.ndarray, k: int) -> int:
    """Assert the selection rule; return the number of near-tie tokens."""
    T = v.shape[0]
    near = gap <= BAND
    n = v.shape[1]
    for t in range(T):
        g = gpu_idx[t]
        assert len(set(g.tolist())) == k, f"token {t}: repeated experts {g}"
        assert ((g >= 0) & (g < n)).all(), f"token {t}: out of range {g}"
        if not near[t]:
            assert set(g.tolist()) == set(oracle_idx[t].tolist()), \
                f"token {t}: gpu {sorted(g.tolist())} oracle {sorted(oracle_idx[t].tolist())} gap {gap[t]}"
        else:
            vk = v[t, oracle_idx[t, k - 1]]
            must = set(np.nonzero(v[t] > vk + BAND)[0].tolist())
            may = set(np.nonzero(v[t] >= vk - BAND)[0].tolist())
            gs = set(g.tolist())
            assert must <= gs <= may, f"near-tie token {t}: {gs} not within [{must}, {may}]"
    return int(near.sum())


def check_selection_grouped(r: dict, gpu_idx: np.ndarray, k: int, n_groups: int, topk_groups: int) -> int:
    """The group-limited selection rule; returns the number of near-tie tokens.

    A token is a near tie when its K-th and (K+1)-th biased scores among the
    kept groups' experts lie within 1e-6, or when its last kept group's score
    lies within q * 1e-6 of the first one left out (a group score sums q fp32
    values).  Other tokens: the GPU's set equals the oracle's.  Near ties: K
    distinct in-range experts from at most topk_groups groups and, where the
    kept groups are certain, the 1e-6 band of check_selection."""
    v, T = r["v"], r["v"].shape[0]
    n = v.shape[1]
    S = n // n_groups
    q = min(-(-k // topk_groups), S)
    near_g = r["group_gap"] <= q * BAND
    near_e = r["gap"] <= BAND
    for t in range(T):
        g = gpu_idx[t]
        assert len(set(g.tolist())) == k, f"token {t}: repeated experts {g}"
        assert ((g >= 0) & (g < n)).all(), f"token {t}: out of range {g}"
        assert len({int(e) // S for e in g}) <= topk_groups, f"token {t}: {g} spans more than {topk_groups} groups"
        if not near_g[t] and not near_e[t]:
            assert set(g.tolist()) == set(r["idx"][t].tolist()), \
                f"token {t}: gpu {sorted(g.tolist())} oracle {sorted(r['idx'][t].tolist())}"
        elif not near_g[t]:
            kept = set(r["groups"][t].tolist())
            assert {int(e) // S for e in g} <= kept, f"token {t}: {g} outside the kept groups {kept}"
            allowed = np.array([e for e in range(n) if e // S in kept])
            vk = v[t, r["idx"][t, k - 1]]
            must = set(allowed[v[t, allowed] > vk + BAND].tolist())
            may = set(allowed[v[t, allowed] >= vk - BAND].tolist())
            assert must <= set(g.tolist()) <= may, f"near-tie token {t}"
    return int((near_g | near_e).sum())


def check_routing(out: dict, u: np.ndarray, E: np.ndarray, b: np.ndarray, k: int, n_routed: int,
                  n_groups: int = 1, topk_groups: int = 1) -> dict:
    """Full routing parity (group-limited when 1 < topk_groups < n_groups).
    Returns the oracle route (with the GPU's selection adopted)."""
    gpu_idx = out["topk_idx"].cpu().numpy()
    if 1 < topk_groups < n_groups:
        r = O.route(u, E, b, k, n_groups=n_groups, topk_groups=topk_groups)
        near = check_selection_grouped(r, gpu_idx, k, n_groups, topk_groups)
    else:
        r = O.route(u, E, b, k)
        near = check_selection(r["v"], r["gap"], r["idx"], gpu_idx, k)
    r = O.route(u, E, b, k, selection=gpu_idx)
    gates = out["topk_gate"].cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(gates, r["gate"], rtol=2e-6, atol=2e-7)
    np.testing.assert_allclose(gates.sum(axis=1), 1.0, atol=2e-6)
    # informational: the GPU lists a token's experts in descending v
    vsel = np.take_along_axis(r["v"], gpu_idx.astype(np.int64), 1)
    order_ok = (np.diff(vsel, axis=1) <= BAND).all()
    grp = O.group_by_expert(gpu_idx, n_routed)
    for key in ("expert_counts", "expert_offsets", "perm_token", "pos"):
        ref = grp[{"expert_counts": "counts", "expert_offsets": "offsets"}.get(key, key)]
        got = out[key].cpu().numpy()
        assert got.shape == ref.shape and (got == ref).all(), f"{key} differs"
    r["near_ties"] = near
    r["order_ok"] = bool(order_ok)
    return r


BF16_UNIT_ROUNDOFF = 2.0 ** -8   # |bf16(x) - x| <= 2^-8 |x| under round to nearest (8 significant bits)


def output_errors(y_gpu: np.ndarray, y_orc: np.ndarray, u: np.ndarray, out_dtype: str = "f32",
                  w_dtype: str = "bf16") -> dict:
    """Max-abs error of the layer output against the oracle, relative to rms(y).

    The 1e-2 * rms bound of the bf16 and fp32 layers is a bound on the
    layer's arithmetic: where such a layer stores y in bf16, the output's
    own final rounding (up to 2^-8 |y| per element) is allowed on top, and
    ``rel_to_rms`` counts only the excess over it.  The FP8 bound
    (4e-2 * rms) is stated for a bf16 output and gets no allowance:
    ``rel_to_rms`` is the raw max-abs error / rms there.  ``raw_rel_to_rms``
    is always the raw figure."""
    err = np.abs(y_gpu.astype(np.float64) - y_orc)
    if out_dtype == "bf16" and w_dtype != "e4m3":
        excess = np.maximum(err - BF16_UNIT_ROUNDOFF * 1.01 * np.abs(y_orc), 0.0)
    else:
        excess = err
    rms = float(np.sqrt(np.mean(y_orc ** 2))) if err.size else 0.0
    branch = y_orc - u.astype(np.float64)
    brms = float(np.sqrt(np.mean(branch ** 2))) if err.size else 0.0
    brms = brms or 1.0
    return {"max_abs": float(err.max()) if err.size else 0.0, "rms": rms,
            "rel_to_rms": float(excess.max() / rms) if err.size else 0.0,
            "raw_rel_to_rms": float(err.max() / rms) if err.size else 0.0,
            "branch_rel": float(err.max() / brms) if err.size else 0.0}


def expert_fns(inp, device_weights: bool):
    """Oracle-side accessors of the expert weights (downloaded on demand)."""
    def routed(e):
        return to_numpy_f32(inp.w_gate_up[e]), to_numpy_f32(inp.w_down[e])
    shared = [(to_numpy_f32(inp.ws_gate_up[s]), to_numpy_f32(inp.ws_down[s])) for s in range(inp.cfg.n_shared)]
    return routed, shared


def rows_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()
