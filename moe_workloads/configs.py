"""Workload configurations.

Shapes follow the DeepSeek-V3 MoE layer as the DeepSeek-V3 Technical Report
pages describe it: hidden size 7168 (wenxiaobai explainer, "hyper-parameter
settings"), 1 shared + 256 routed experts with 8 routed experts active per
token (xyznot summary, "key ideas" and section 2).  The smaller shapes are
synthetic parity cases; the skewed decode case mimics a trained router's
uneven expert load.

dtype names: "f32", "bf16" and "e4m3" (OCP FP8 E4M3, the FP8 path).  For the
FP8 path the activations and centroids are still given in bf16 (the router
stays bf16), the expert weights are bf16 values that are quantised to e4m3
with 128x128 block scales before use, and the output is bf16.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens in the batch
    d: int            # hidden size
    n_routed: int     # N_r
    n_shared: int     # N_s
    inter: int        # expert intermediate size I (shared and routed alike)
    top_k: int        # K_r
    x_dtype: str      # dtype of u and the centroids: "f32" | "bf16"
    w_dtype: str      # expert weight / GEMM dtype: "f32" | "bf16" | "e4m3"
    out_dtype: str    # dtype of y: "f32" | "bf16"
    u_std: float = 1.0
    w_std: float = 0.006
    e_std: float = 0.02
    b_std: float = 0.0
    # Zipf skew of the centroid norms (decode-like load imbalance); None = off.
    zipf_s: Optional[float] = None
    cfg_id: int = 0   # folded into every seed so configs draw unrelated streams
    # group-limited routing: experts in n_groups equal runs, at most
    # topk_groups of them per token (off when topk_groups >= n_groups)
    n_groups: int = 1
    topk_groups: int = 1

    @property
    def grouped(self) -> bool:
        return 1 < self.topk_groups < self.n_groups

    @property
    def fp8(self) -> bool:
        return self.w_dtype == "e4m3"

    @property
    def assignments(self) -> int:
        return self.T * self.top_k

    def flops(self) -> float:
        """Algorithmic flops of one forward: router GEMM + 3 GEMMs per active expert."""
        per_tok = 2 * self.d * self.n_routed + 6 * self.d * self.inter * (self.top_k + self.n_shared)
        return float(per_tok) * self.T

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# The five workloads the build is measured and checked on.
CONFIGS: Dict[str, MoEConfig] = {
    # Tiny, fp32 throughout; small enough for brute force.
    "tiny_fp32": MoEConfig("tiny_fp32", T=64, d=64, n_routed=8, n_shared=1, inter=32, top_k=2,
                           x_dtype="f32", w_dtype="f32", out_dtype="f32",
                           u_std=1.0, w_std=0.02, e_std=0.02, b_std=0.1, cfg_id=1),
    # Mid-size bf16 layer (DeepSeek-V2-like widths).
    "bf16_d2048": MoEConfig("bf16_d2048", T=4096, d=2048, n_routed=64, n_shared=2, inter=1408, top_k=6,
                            x_dtype="bf16", w_dtype="bf16", out_dtype="f32",
                            w_std=0.006, e_std=0.02, b_std=0.0, cfg_id=2),
    # The DeepSeek-V3 layer shape: the throughput workload.
    "bf16_d7168": MoEConfig("bf16_d7168", T=8192, d=7168, n_routed=256, n_shared=1, inter=2048, top_k=8,
                            x_dtype="bf16", w_dtype="bf16", out_dtype="f32",
                            w_std=0.006, e_std=0.02, b_std=0.01, cfg_id=3),
    # FP8 (e4m3, fine-grained scaling) at the mid-size shape, bf16 output.
    "fp8_d2048": MoEConfig("fp8_d2048", T=4096, d=2048, n_routed=64, n_shared=2, inter=1408, top_k=6,
                           x_dtype="bf16", w_dtype="e4m3", out_dtype="bf16",
                           w_std=0.006, e_std=0.02, b_std=0.0, cfg_id=4),
    # FP8 at the DeepSeek-V3 shape (secondary FP8 case).
    "fp8_d7168": MoEConfig("fp8_d7168", T=8192, d=7168, n_routed=256, n_shared=1, inter=2048, top_k=8,
                           x_dtype="bf16", w_dtype="e4m3", out_dtype="bf16",
                           w_std=0.006, e_std=0.02, b_std=0.01, cfg_id=6),
    # The DeepSeek-V3 layer with group-limited routing: 8 groups of 32 experts
    # (e.g. the nodes of an expert-parallel deployment), at most 4 per token.
    "bf16_d7168_g8": MoEConfig("bf16_d7168_g8", T=8192, d=7168, n_routed=256, n_shared=1, inter=2048, top_k=8,
                               x_dtype="bf16", w_dtype="bf16", out_dtype="f32",
                               w_std=0.006, e_std=0.02, b_std=0.01, cfg_id=3, n_groups=8, topk_groups=4),
    # Decode-like batch with a skewed router, used for the bias-update loop.
    "skew_decode_d7168": MoEConfig("skew_decode_d7168", T=256, d=7168, n_routed=256, n_shared=1, inter=2048,
                                   top_k=8, x_dtype="bf16", w_dtype="bf16", out_dtype="f32",
                                   w_std=0.006, e_std=0.02, b_std=0.0, zipf_s=1.2, cfg_id=5),
}

# Small cases the oracle finishes in seconds; they span several GEMM tiles
# and leave ragged tails (T, per-expert row counts, and N not tile multiples).
PARITY_CONFIGS: Dict[str, MoEConfig] = {
    "small_bf16": MoEConfig("small_bf16", T=300, d=512, n_routed=16, n_shared=1, inter=384, top_k=4,
                            x_dtype="bf16", w_dtype="bf16", out_dtype="f32",
                            w_std=0.02, e_std=0.05, b_std=0.01, cfg_id=11),
    "small_bf16_ns2": MoEConfig("small_bf16_ns2", T=517, d=256, n_routed=24, n_shared=2, inter=192, top_k=6,
                                x_dtype="bf16", w_dtype="bf16", out_dtype="f32",
                                w_std=0.03, e_std=0.05, b_std=0.02, cfg_id=12),
    "small_bf16_ns0": MoEConfig("small_bf16_ns0", T=129, d=384, n_routed=12, n_shared=0, inter=320, top_k=3,
                                x_dtype="bf16", w_dtype="bf16", out_dtype="bf16",
                                w_std=0.03, e_std=0.05, b_std=0.02, cfg_id=13),
    "small_fp32": MoEConfig("small_fp32", T=200, d=128, n_routed=10, n_shared=1, inter=96, top_k=3,
                            x_dtype="f32", w_dtype="f32", out_dtype="f32",
                            w_std=0.05, e_std=0.05, b_std=0.05, cfg_id=14),
    "small_fp8": MoEConfig("small_fp8", T=300, d=512, n_routed=16, n_shared=1, inter=384, top_k=4,
                           x_dtype="bf16", w_dtype="e4m3", out_dtype="bf16",
                           w_std=0.02, e_std=0.05, b_std=0.01, cfg_id=15),
    "small_fp8_ns2": MoEConfig("small_fp8_ns2", T=517, d=256, n_routed=24, n_shared=2, inter=256, top_k=6,
                               x_dtype="bf16", w_dtype="e4m3", out_dtype="f32",
                               w_std=0.03, e_std=0.05, b_std=0.02, cfg_id=16),
    # K = N_r: every expert active, a dense mixture.
    "dense_k_eq_n": MoEConfig("dense_k_eq_n", T=70, d=128, n_routed=4, n_shared=1, inter=64, top_k=4,
                              x_dtype="bf16", w_dtype="bf16", out_dtype="f32",
                              w_std=0.05, e_std=0.05, b_std=0.05, cfg_id=17),
    # A single token; most experts receive no rows.
    "one_token": MoEConfig("one_token", T=1, d=256, n_routed=32, n_shared=1, inter=128, top_k=8,
                           x_dtype="bf16", w_dtype="bf16", out_dtype="f32",
                           w_std=0.03, e_std=0.05, b_std=0.01, cfg_id=18),
    # Many experts (N_r = 512, the library's upper limit) and K = 16.
    "wide_router": MoEConfig("wide_router", T=96, d=256, n_routed=512, n_shared=1, inter=128, top_k=16,
                             x_dtype="bf16", w_dtype="bf16", out_dtype="f32",
                             w_std=0.03, e_std=0.05, b_std=0.01, cfg_id=19),
}


def get_config(name: str) -> MoEConfig:
    if name in CONFIGS:
        return CONFIGS[name]
    if name in PARITY_CONFIGS:
        return PARITY_CONFIGS[name]
    raise KeyError(f"unknown workload {name!r}")
