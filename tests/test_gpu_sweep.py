"""A seeded sweep of small attention problems against the fp64 oracle.

Each case draws its own sizes: batch, query and key lengths (ragged, from a
single token up), query and K/V head counts over 1 or 2 virtual ranks, head
dim 64 or 128, causal or bidirectional (cross-attention when the lengths
differ), bf16 or fp32. Most of them are small launches, which the kernels
run with split key and query walks; the wide cases (many heads over few
tokens) reach the single-walk schedules at sizes the oracle still finishes
in a moment. 120 cases in all, and three fp32 ones with few keys and many
queries (dK and dV sum thousands of sizeable products in fp32); 36 more
run block layouts (a window, global and random blocks per row, some block
rows emptied; bf16, self-attention).
The gradient of a K/V head shared by several query heads is held to the
sum of its parts' bars in both element types (gpu_common.shared_head_allowed).
Forward and backward go through the generalised entry points
and are held to the same bars as every other parity test, with the bf16
elementwise bar widened by the bound on rounding P and dS to bf16 inside the
products (2^-8 times the oracle's absolute sums): without it the dV of the
heaviest causal keys in case 17 (256 heads of 272 tokens) has elements just
past one ulp, and a CPU emulation of the same bf16-operand, fp32-accumulate
arithmetic on the same inputs gives the same worst element.
"""
import numpy as np
import pytest

import exact_attention_ulysses_amd as U
import oracle
from workloads import block_layout, custom, host_tensor

from gpu_common import LSE_ABS, check_close, shared_head_allowed, to_device, to_f64, torch_mod

pytestmark = pytest.mark.gpu


def _draw_case(i):
    rng = np.random.default_rng(7000 + i)
    wide = i % 6 == 5
    causal = bool(rng.integers(0, 2))
    P = int(rng.integers(1, 3))
    Hkl = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4]))
    if wide:   # many heads over few tokens: launches above the split thresholds
        B, Hkl, G = int(rng.integers(4, 9)), 32, 1
        Lq = int(rng.integers(200, 400))
    else:
        B = int(rng.integers(1, 4))
        Lq = int(rng.integers(1, 700))
    Lk = Lq if causal else int(rng.integers(1, 900))
    d = int(rng.choice([64, 128]))
    dtype = "fp32" if (not wide and i % 7 == 3) else "bf16"
    Hq, Hkv = Hkl * G * P, Hkl * P   # global counts: the K/V heads split evenly over the ranks
    return B, Lq, Lk, Hq, Hkv, d, P, causal, dtype


# few keys, many queries, fp32: dK and dV sum thousands of products of size
# ~0.1-0.25 (P is ~1/L_k), so their largest elements reach 10-50
LONG_FP32_SUMS = [(3, 1550, 14, 1, 1, 128, 1, False, "fp32"), (1, 8000, 10, 2, 2, 128, 1, False, "fp32"),
                  (2, 4000, 4, 4, 4, 64, 2, False, "fp32")]
CASES = [_draw_case(i) for i in range(120)] + LONG_FP32_SUMS


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    U.lib()


def _draw(B, L, H, d, dtype, name, index):
    wl = custom(B, L, H, d, 1, dtype=dtype, index=index)
    return host_tensor(wl, name).reshape(B, L, H, d)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_sweep_parity(case):
    B, Lq, Lk, Hq, Hkv, d, P, causal, dtype = CASES[case]
    torch = torch_mod()
    Hql, Hkl = Hq // P, U.kv_local_heads(Hkv, P)
    G = Hql // Hkl
    base = 5000 + case
    host = {n: _draw(B, Lq, Hql, d, dtype, n, base) for n in ("q", "do")}
    host.update({n: _draw(B, Lk, Hkl, d, dtype, n, base) for n in ("k", "v")})
    dev = {n: to_device(host[n], dtype) for n in host}
    o = torch.empty_like(dev["q"])
    lse = torch.empty((B, Hql, Lq), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd_gqa(dev["q"], dev["k"], dev["v"], o, lse, B, Lq, Lk, Hq, Hkv, d, P, causal)
    dq = torch.empty_like(dev["q"])
    dk, dv = torch.empty_like(dev["k"]), torch.empty_like(dev["v"])
    dc = U.BF16 if dtype == "bf16" else U.FP32
    ws = torch.empty(U.ulysses_attn_bwd_gqa_workspace_bytes(B, Lq, Lk, Hq, Hkv, d, P, causal, dc),
                     dtype=torch.uint8, device="cuda")
    U.ulysses_attn_bwd_gqa(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, dq, dk, dv, ws, B, Lq, Lk, Hq, Hkv, d,
                           P, causal)
    torch.cuda.synchronize()
    tag = f"case {case} {CASES[case]}"
    f = {n: oracle.to_f64(host[n], dtype) for n in host}
    # bf16: the elementwise bars include the bound on rounding P and dS to
    # bf16 inside the products (their absolute sums, per output element)
    asum = {n: None for n in ("o", "dq", "dk", "dv")}
    if dtype == "bf16":
        asum = {"o": np.zeros(f["q"].shape), "dq": np.zeros(f["q"].shape),
                "dk": np.zeros(f["k"].shape), "dv": np.zeros(f["v"].shape)}
        for b in range(B):
            for h in range(Hql):
                a_dq, a_dk, a_dv, a_o = oracle.attn_abs_sums_head(f["q"][b, :, h], f["k"][b, :, h // G],
                                                                  f["v"][b, :, h // G], f["do"][b, :, h], causal)
                asum["o"][b, :, h], asum["dq"][b, :, h] = a_o, a_dq
                asum["dk"][b, :, h // G] += a_dk
                asum["dv"][b, :, h // G] += a_dv
    o_r, lse_r = oracle.attn_fwd_gqa(f["q"], f["k"], f["v"], causal)
    check_close(f"O {tag}", to_f64(o, dtype), o_r, dtype, abs_sum=asum["o"])
    assert np.max(np.abs(lse.cpu().numpy() - lse_r)) <= LSE_ABS[dtype], f"LSE {tag}"
    dq_r, dk_r, dv_r = oracle.attn_bwd_gqa(f["q"], f["k"], f["v"], f["do"], causal)
    check_close(f"dQ {tag}", to_f64(dq, dtype), dq_r, dtype, abs_sum=asum["dq"])
    if G == 1:
        check_close(f"dK {tag}", to_f64(dk, dtype), dk_r, dtype, abs_sum=asum["dk"])
        check_close(f"dV {tag}", to_f64(dv, dtype), dv_r, dtype, abs_sum=asum["dv"])
        return
    # a K/V head shared by G query heads gets the sum of their gradients
    parts = {"dK": np.zeros((G,) + dk_r.shape), "dV": np.zeros((G,) + dv_r.shape)}
    for b in range(B):
        for h in range(Hql):
            r = oracle.attn_bwd_head(f["q"][b, :, h], f["k"][b, :, h // G], f["v"][b, :, h // G], f["do"][b, :, h],
                                     causal)
            parts["dK"][h % G, b, :, h // G] = r[1]
            parts["dV"][h % G, b, :, h // G] = r[2]
    for name, got, want in (("dK", dk, dk_r), ("dV", dv, dv_r)):
        check_close(f"{name} {tag}", to_f64(got, dtype), want, dtype,
                    allowed=shared_head_allowed(parts[name], want, dtype), abs_sum=asum[name.lower()])


def _draw_sparse_case(i):
    rng = np.random.default_rng(9000 + i)
    causal = bool(rng.integers(0, 2))
    P = int(rng.integers(1, 3))
    Hkl = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 3))
    L = int(rng.integers(1, 1500))
    d = int(rng.choice([64, 128]))
    lay = (int(rng.integers(1, 5)), int(rng.integers(0, 3)), int(rng.integers(0, 4)), bool(rng.integers(0, 2)))
    return B, L, Hkl * G * P, Hkl * P, d, P, causal, lay   # lay: window, global, random, empty rows


SPARSE_CASES = [_draw_sparse_case(i) for i in range(36)]


@pytest.mark.parametrize("case", range(len(SPARSE_CASES)))
def test_sweep_block_sparse_parity(case):
    """Block layouts over random sizes: a window, global and random blocks per
    row (and, in some cases, block rows emptied), bf16."""
    B, L, Hq, Hkv, d, P, causal, (window, n_global, n_random, empty) = SPARSE_CASES[case]
    torch = torch_mod()
    Hql, Hkl = Hq // P, U.kv_local_heads(Hkv, P)
    G = Hql // Hkl
    BLOCK = U.SPARSE_BLOCK
    base = 8000 + case
    host = {n: _draw(B, L, Hql, d, "bf16", n, base) for n in ("q", "do")}
    host.update({n: _draw(B, L, Hkl, d, "bf16", n, base) for n in ("k", "v")})
    lay = block_layout(custom(B, L, Hql, d, 1, causal=causal, index=base, block=BLOCK, window=window,
                              n_global=n_global, n_random=n_random))
    nb = lay.shape[1]
    if empty:   # rows that see nothing: zero output, LSE -inf, no gradient through them
        lay[:, nb // 2, :] = 0
    dev = {n: to_device(host[n], "bf16") for n in host}
    layout = torch.from_numpy(lay).to("cuda")
    o = torch.empty_like(dev["q"])
    lse = torch.empty((B, Hql, L), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd_block_sparse(dev["q"], dev["k"], dev["v"], o, lse, layout, B, L, Hq, Hkv, d, P, causal)
    dq = torch.empty_like(dev["q"])
    dk, dv = torch.empty_like(dev["k"]), torch.empty_like(dev["v"])
    ws = torch.empty(U.ulysses_attn_bwd_block_sparse_workspace_bytes(B, L, Hq, Hkv, d, P, causal),
                     dtype=torch.uint8, device="cuda")
    U.ulysses_attn_bwd_block_sparse(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, dq, dk, dv, layout, ws, B, L,
                                    Hq, Hkv, d, P, causal)
    torch.cuda.synchronize()
    tag = f"sparse case {case} {SPARSE_CASES[case]}"
    f = {n: oracle.to_f64(host[n], "bf16") for n in host}
    kr, vr = np.repeat(f["k"], G, axis=2), np.repeat(f["v"], G, axis=2)
    o_r, lse_r = oracle.attn_fwd_block_sparse(f["q"], kr, vr, lay, BLOCK, causal)
    dq_r, dk_rep, dv_rep = oracle.attn_bwd_block_sparse(f["q"], kr, vr, f["do"], lay, BLOCK, causal)
    asum = {"o": np.zeros(f["q"].shape), "dq": np.zeros(f["q"].shape),
            "dk": np.zeros(f["k"].shape), "dv": np.zeros(f["v"].shape)}
    for b in range(B):
        for h in range(Hql):
            a_dq, a_dk, a_dv, a_o = oracle.attn_abs_sums_block_sparse_head(
                f["q"][b, :, h], f["k"][b, :, h // G], f["v"][b, :, h // G], f["do"][b, :, h], lay[h], BLOCK, causal)
            asum["o"][b, :, h], asum["dq"][b, :, h] = a_o, a_dq
            asum["dk"][b, :, h // G] += a_dk
            asum["dv"][b, :, h // G] += a_dv
    check_close(f"O {tag}", to_f64(o, "bf16"), o_r, "bf16", abs_sum=asum["o"])
    lse_g = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(lse_g), np.isneginf(lse_r)), f"LSE -inf rows {tag}"
    fin = np.isfinite(lse_r)
    assert np.max(np.abs(lse_g[fin] - lse_r[fin]), initial=0.0) <= LSE_ABS["bf16"], f"LSE {tag}"
    check_close(f"dQ {tag}", to_f64(dq, "bf16"), dq_r, "bf16", abs_sum=asum["dq"])
    for name, rep in (("dK", dk_rep), ("dV", dv_rep)):
        parts = np.moveaxis(rep.reshape(B, L, Hkl, G, d), 3, 0)   # [G, B, L, Hkl, d]
        want = parts.sum(axis=0)
        allowed = None if G == 1 else shared_head_allowed(parts, want, "bf16")
        check_close(f"{name} {tag}", to_f64(dk if name == "dK" else dv, "bf16"), want, "bf16", allowed=allowed,
                    abs_sum=asum[name.lower()])
