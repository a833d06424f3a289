"""The bf16 spacing function behind the elementwise bar (host only)."""
import numpy as np
import torch

from gpu_common import bf16_ulp


def test_bf16_ulp_is_the_bf16_spacing():
    x = torch.tensor(np.random.default_rng(1).uniform(-1e3, 1e3, 1000), dtype=torch.bfloat16)
    x = torch.cat([x, torch.tensor([2.0 ** k for k in range(-20, 20)], dtype=torch.bfloat16)]).abs()
    up = torch.nextafter(x, torch.full_like(x, float("inf")))
    np.testing.assert_array_equal(bf16_ulp(x.float().numpy()), (up.float() - x.float()).double().numpy())
