"""Shared helpers of the GPU parity tests (host side only)."""
import os
from concurrent.futures import ThreadPoolExecutor

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


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits): 2^(e-8) for |x| in [2^(e-1), 2^e)."""
    _, e = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    return np.ldexp(1.0, e - 8)


# every comparison check_close made in this process, for the end-of-run summary
RECORDS = []


def check_close(name, got, want, dtype, max_abs=None, rel_fro=None, fro=True, allowed=None, abs_sum=None):
    """Compare a kernel output with the fp64 oracle value `want`.

    bf16 outputs: every element within max(1e-2, one bf16 ulp of the exact
    value) -- the two differ only for |x| >= 2, where bf16 spacing alone
    (2^-6 and up) exceeds 1e-2 -- and ||got - want||_F / ||want||_F <= 5e-3.
    fp32 outputs: every element within 1e-5. With fro=False only the
    elementwise bar applies (for hand-picked rows, whose norm says nothing
    about the whole tensor's relative Frobenius error). `allowed`, when given,
    replaces the elementwise bar with a per-element array (sums of several
    outputs' budgets, see shared_head_allowed). `abs_sum`, when given (bf16),
    adds 2^-8 * abs_sum to the elementwise bar: the bound on rounding the
    probabilities (or dS) to bf16 before they enter the products, from the
    oracle's absolute sums (oracle.attn_abs_sums_head).

    The returned stats always carry the raw figures beside the pass/fail result:
    max_abs, n_over_flat (elements more than 1e-2 (bf16) or 1e-5 (fp32)
    off), and max_err_over_unwidened (the worst error over max(1e-2, ulp),
    or over 1e-5) next to max_err_over_allowed (over the bar the test
    applied, widened by `allowed` or `abs_sum` where given).
    """
    st = oracle.error_stats(got, want)
    err = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
    st["n"] = int(err.size)
    if dtype == "bf16":
        ma = BF16_MAX_ABS if max_abs is None else max_abs
        rf = BF16_REL_FRO if rel_fro is None else rel_fro
        plain = np.maximum(ma, bf16_ulp(want))
        if allowed is None:
            allowed = plain
        if abs_sum is not None:
            allowed = allowed + 2.0 ** -8 * np.asarray(abs_sum, dtype=np.float64)
        st["max_err_over_allowed"] = float(np.max(err / allowed)) if err.size else 0.0
        st["max_err_over_unwidened"] = float(np.max(err / plain)) if err.size else 0.0
        st["n_over_flat"] = int(np.count_nonzero(err > ma))
        ok = st["max_err_over_allowed"] <= 1.0 and (st["rel_fro"] <= rf or not fro)
    else:
        ma = FP32_MAX_ABS if max_abs is None else max_abs
        plain = np.full(np.shape(err), ma)
        if allowed is None:
            allowed = plain
        st["max_err_over_allowed"] = float(np.max(err / allowed)) if err.size else 0.0
        st["max_err_over_unwidened"] = float(np.max(err / plain)) if err.size else 0.0
        st["n_over_flat"] = int(np.count_nonzero(err > ma))
        ok = st["max_err_over_allowed"] <= 1.0
    RECORDS.append((name, dtype, st))
    assert ok, f"{name}: {st} exceeds the {dtype} bar"
    return st


def shared_head_allowed(parts, want, dtype):
    """Per-element bar of a gradient that sums several attention outputs.

    A K/V head shared by G query heads (or replicated on R ranks) receives
    the sum of G (or R) gradients, each of which carries the rounding of one
    attention output. The budget is the sum of the parts' own bars plus one
    rounding of the total: sum_g max(1e-2, ulp(part_g)) + ulp(total) for bf16,
    G * 1e-5 + 2^-23 |total| for fp32. `parts` stacks the oracle's per-part
    gradients along axis 0, aligned with `want`.
    """
    parts = np.asarray(parts, dtype=np.float64)
    if dtype == "bf16":
        return np.sum(np.maximum(BF16_MAX_ABS, bf16_ulp(parts)), axis=0) + bf16_ulp(want)
    return parts.shape[0] * FP32_MAX_ABS + 2.0 ** -23 * np.abs(want)


def host_cores() -> int:
    """Host threads this process may use (the host's CPU share when OMP_NUM_THREADS states it)."""
    n = len(os.sched_getaffinity(0))
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(1, n)


def host_parallel(fn, items, max_workers=16):
    """fn over items in host threads (numpy's loops release the interpreter
    lock, so oracle calls on independent heads or row ranges run side by
    side). Results in order. BLAS runs one thread per worker: concurrent
    calls into a multithreaded OpenBLAS from several threads were measured
    to return wrong products (an fp64 dK off by 1.8e-3 on a 32K-token head),
    while one BLAS thread per calling thread gave results bit-identical to a
    sequential run."""
    from threadpoolctl import threadpool_limits
    items = list(items)
    workers = max(1, min(len(items), max_workers, host_cores()))
    with threadpool_limits(1):
        with ThreadPoolExecutor(workers) as ex:
            return list(ex.map(fn, items))


def causal_row_ranges(L, parts, block=256):
    """Cut rows 0..L-1 into `parts` ranges of about equal causal work (row i
    costs ~i), at multiples of `block`."""
    cuts = [0]
    for p in range(1, parts):
        c = int(round(L * (p / parts) ** 0.5 / block)) * block
        cuts.append(min(L, max(cuts[-1], c)))
    cuts.append(L)
    return [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
