"""The spacing functions behind the elementwise bars (host only)."""
import numpy as np
import torch

from gpu_common import bf16_ulp, fp32_ulp


def test_fp32_ulp_is_the_fp32_spacing():
    x = np.concatenate([np.ldexp(1.0, np.arange(-20, 20)), np.random.default_rng(0).uniform(-1e3, 1e3, 1000)])
    x = x.astype(np.float32)
    np.testing.assert_array_equal(fp32_ulp(x), np.spacing(np.abs(x)).astype(np.float64))


def test_bf16_ulp_is_the_bf16_spacing():
    x = torch.tensor(np.random.default_rng(1).uniform(-1e3, 1e3, 1000), dtype=torch.bfloat16)
    x = torch.cat([x, torch.tensor([2.0 ** k for k in range(-20, 20)], dtype=torch.bfloat16)]).abs()
    up = torch.nextafter(x, torch.full_like(x, float("inf")))
    np.testing.assert_array_equal(bf16_ulp(x.float().numpy()), (up.float() - x.float()).double().numpy())
