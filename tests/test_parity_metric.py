"""CPU checks of the output-error metric the GPU parity tests apply."""

import numpy as np
import torch

from tests.parity import output_errors


def _bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def test_bf16_output_rounding_alone_is_not_an_error():
    rs = np.random.RandomState(0)
    y = rs.randn(64, 512)
    y[0, 0] = 4.7                        # bf16(4.7) = 4.6875: the rounding alone exceeds 1e-2 * rms
    u = np.zeros_like(y)
    e = output_errors(_bf16(y), y, u, "bf16")
    assert e["rel_to_rms"] == 0.0
    assert e["max_abs"] > 1e-2 * e["rms"]    # the raw difference would have failed a plain bound
    assert output_errors(_bf16(y), y, u, "f32")["rel_to_rms"] > 1e-2


def test_error_beyond_the_rounding_is_counted():
    rs = np.random.RandomState(1)
    y = rs.randn(32, 256)
    u = np.zeros_like(y)
    yg = _bf16(y)
    yg[3, 7] += 0.05                          # far beyond 2^-8 |y| at any |y| here
    e = output_errors(yg, y, u, "bf16")
    assert e["rel_to_rms"] * e["rms"] > 0.04


def test_fp8_output_gets_no_rounding_allowance():
    """The FP8 bound is stated for a bf16 output: the raw error is what counts."""
    rs = np.random.RandomState(2)
    y = rs.randn(64, 512)
    y[0, 0] = 4.7
    u = np.zeros_like(y)
    e = output_errors(_bf16(y), y, u, "bf16", "e4m3")
    assert e["rel_to_rms"] == e["raw_rel_to_rms"] == e["max_abs"] / e["rms"]
    assert e["rel_to_rms"] > 0
    e16 = output_errors(_bf16(y), y, u, "bf16", "bf16")
    assert e16["rel_to_rms"] == 0.0 and e16["raw_rel_to_rms"] == e["raw_rel_to_rms"]
