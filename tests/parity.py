"""Comparison protocol between the HIP path and the CPU oracle.

* Kept masks and counts must agree bit-exactly, except on elements whose
  oracle post-softmax value lies within 1e-5 relative of theta (ambiguous:
  float32 scores on the GPU may land on either side).
* Outputs are compared against the oracle re-evaluated with the GPU's own
  decisions on those ambiguous elements: max-abs <= 1e-2 for bfloat16 inputs,
  and per row max|o - r| <= 1e-5 * max(|r|_inf, 1e-30) for float32 inputs.
  A bfloat16 output is stored in bfloat16 (the input type), so on top of the
  1e-2 it may differ from the exact value by the rounding of that value to
  bfloat16, half a unit in its last place (0.0156 for values in [4, 8)).
"""
import numpy as np
import torch

import oracle

AMBIG_REL = 1e-5
TOL_BF16_ABS = 1e-2
TOL_F32_REL = 1e-5


def device():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    return torch.device("cuda:0")


def ambiguous(s, theta):
    s = np.asarray(s, dtype=np.float64)
    if not np.isfinite(theta):
        return np.zeros(s.shape, dtype=bool)
    return np.abs(s - theta) <= AMBIG_REL * abs(theta)


def check_row_mask(gpu_keep, s, theta, where=""):
    """Assert mask parity outside the ambiguity band; return the band size."""
    gpu_keep = np.asarray(gpu_keep, dtype=bool)
    ref = np.asarray(s) >= theta
    amb = ambiguous(s, theta)
    bad = (gpu_keep != ref) & ~amb
    assert not bad.any(), f"mask mismatch {where}: keys {np.flatnonzero(bad)[:10]}"
    return int(amb.sum())


def bf16_half_ulp(x):
    """Half the spacing of bfloat16 values (8 significant bits) at |x|: the
    largest error of rounding x to bfloat16."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(x)                   # x = m * 2**e, 0.5 <= m < 1
    return np.where(x > 0, np.ldexp(1.0, e - 9), 0.0)


def check_out(gpu, ref, dtype, where=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if dtype == torch.bfloat16:
        err = (np.abs(gpu - ref) - bf16_half_ulp(ref)).max() if gpu.size else 0.0
        assert err <= TOL_BF16_ABS, f"bf16 max-abs error beyond output rounding {err:.3g} {where}"
    else:
        err = np.abs(gpu - ref).max()
        scale = max(np.abs(ref).max(), 1e-30)
        assert err <= TOL_F32_REL * scale, f"f32 rel error {err / scale:.3g} {where}"


def theta_of(theta_table, h, p):
    return oracle.theta_row(theta_table, h, p)
