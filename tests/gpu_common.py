"""Shared helpers of the GPU parity tests (host side only)."""
import numpy as np

import oracle

# tolerance bars, per output tensor
BF16_MAX_ABS = 1e-2
BF16_REL_FRO = 5e-3
FP32_MAX_ABS = 1e-5
LSE_ABS = {"bf16": 1e-3, "fp32": 1e-5}


def torch_mod():
    import torch
    return torch


def to_device(x: np.ndarray, dtype: str, device="cuda"):
    """Host array (uint16 bf16 bits or float32) -> device tensor with the same bits."""
    torch = torch_mod()
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def to_host_bits(t) -> np.ndarray:
    """Device tensor -> host array of its raw bits (uint16 for bf16, float32 otherwise)."""
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def to_f64(t_or_bits, dtype: str) -> np.ndarray:
    bits = t_or_bits if isinstance(t_or_bits, np.ndarray) else to_host_bits(t_or_bits)
    return oracle.to_f64(bits, dtype)


def round_f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Exact values rounded to the nearest bf16 (ties to even), kept as float64.

    A bf16 output cannot be closer to the exact value than this; for |x| >= 4
    the spacing of bf16 (2^-5) alone exceeds an absolute error of 1e-2.
    """
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(m * 256.0), e - 8)


def check_close(name, got, want, dtype, max_abs=None, rel_fro=None):
    """bf16: max |got - bf16(want)| <= 1e-2 and ||got - want||_F / ||want||_F <= 5e-3;
    fp32: max |got - want| <= 1e-5. `want` is the fp64 oracle value."""
    st = oracle.error_stats(got, want)
    if dtype == "bf16":
        ma = BF16_MAX_ABS if max_abs is None else max_abs
        rf = BF16_REL_FRO if rel_fro is None else rel_fro
        st["max_abs_vs_rounded"] = oracle.error_stats(got, round_f64_to_bf16(want))["max_abs"]
        ok = st["max_abs_vs_rounded"] <= ma and st["rel_fro"] <= rf
    else:
        ma = FP32_MAX_ABS if max_abs is None else max_abs
        ok = st["max_abs"] <= ma
    assert ok, f"{name}: {st} exceeds the {dtype} bar"
    return st
