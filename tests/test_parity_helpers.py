"""Host checks of the comparison helpers used by the GPU parity tests."""
import numpy as np
import torch

from parity import ambiguous, bf16_half_ulp


def test_bf16_half_ulp_bounds_torch_rounding():
    """The allowance for storing an exact value in bfloat16 bounds torch's
    round-to-nearest-even conversion, and is reached (tight) up to a few %."""
    rng = np.random.default_rng(0)
    # float32 values (one rounding to bfloat16, as the kernels' float32 results get)
    x = (rng.standard_normal(200000) * np.exp2(rng.uniform(-20, 20, 200000))).astype(np.float32)
    r = torch.tensor(x).to(torch.bfloat16).double().numpy()
    x = x.astype(np.float64)
    err = np.abs(r - x)
    bound = bf16_half_ulp(x)
    assert (err <= bound).all()
    assert (err / bound).max() > 0.97


def test_ambiguity_band():
    s = np.array([0.1, 0.1 * (1 + 0.9e-5), 0.1 * (1 + 1.1e-5), 0.2])
    assert ambiguous(s, 0.1).tolist() == [True, True, False, False]
    assert not ambiguous(s, -np.inf).any()
