"""The backward entry point that allocates nothing (ulysses_attn_bwd_noalloc).

It takes no workspace: delta and the partial sums of split walks live in the
library's fixed per-device scratch. Each case makes two calls in a row, the
second on a smaller input (the scratch keeps the first call's contents), and
compares both with ulysses_attn_bwd on the same inputs and with the fp64
oracle, within the bf16 / fp32 bars. The first case is a launch whose split
dK/dV walks need more partial-sum room than the scratch has, so the capped
plan takes other kernels than the workspace entry point.
"""
import numpy as np
import pytest

import exact_attention_ulysses_amd as U
import oracle
from workloads import custom, host_tensor

from gpu_common import check_close, to_device, to_f64, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    U.lib()


def _backward_both_ways(B, L, H, d, P, causal, dtype, index):
    torch = torch_mod()
    Hh = H // P
    wl = custom(B, L, Hh, d, 1, dtype=dtype, causal=causal, index=index)
    host = {n: host_tensor(wl, n).reshape(B, L, Hh, d) for n in ("q", "k", "v", "do")}
    q, k, v, do = (to_device(host[n], dtype) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hh, L), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd(q, k, v, o, lse, B, L, H, d, P, causal)
    ws = torch.empty(U.ulysses_attn_bwd_workspace_bytes(B, L, H, d, P, causal, U.dtype_code(q)),
                     dtype=torch.uint8, device="cuda")
    ref = [torch.empty_like(q) for _ in range(3)]
    U.ulysses_attn_bwd(q, k, v, o, do, lse, *ref, ws, B, L, H, d, P, causal)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    print(f"noalloc B={B} L={L} H={H} d={d} P={P} causal={causal} {dtype}", flush=True)
    U.ulysses_attn_bwd_noalloc(q, k, v, o, do, lse, *got, B, L, H, d, P, causal)
    torch.cuda.synchronize()
    f = {n: oracle.to_f64(host[n], dtype) for n in ("q", "k", "v", "do")}
    want = oracle.attn_bwd(f["q"], f["k"], f["v"], f["do"], causal)[:3]
    for name, g, r, w in zip(("dQ", "dK", "dV"), got, ref, want):
        check_close(f"{name} no-alloc vs workspace entry", to_f64(g, dtype), to_f64(r, dtype), dtype)
        check_close(f"{name} no-alloc vs oracle", to_f64(g, dtype), w, dtype)


@pytest.mark.parametrize("first,second", [
    # 8K x 4 heads: the split dK/dV walks would need 64 MiB of partial sums
    ((1, 8192, 8, 128, 2, True, "bf16"), (2, 1000, 4, 64, 2, True, "bf16")),
    ((1, 2048, 8, 128, 2, False, "bf16"), (1, 513, 2, 128, 1, False, "bf16")),
    ((1, 300, 4, 64, 2, True, "fp32"), (1, 77, 2, 64, 1, True, "fp32")),
])
def test_noalloc_backward_matches_workspace_entry(first, second):
    _backward_both_ways(*first, index=600)
    _backward_both_ways(*second, index=601)
