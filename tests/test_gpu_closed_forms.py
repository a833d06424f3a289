"""Closed forms and exact identities of the attention kernels, at full size.

None of these checks needs the oracle: they hold for exact attention
O = softmax(Q K^T / sqrt(d_h)) V with an optional causal mask (paper-graph
summary of arXiv 2309.14509, sections 3.4.1 and 3.4.5) and for its exact
gradient, the reading the oracle takes of a backward the pages leave unwritten.

Zero queries. Every visible score is 0, so each query row spreads its
probability evenly over its visible keys; O, LSE, dQ and dV then have the
closed forms of tests/closed_forms.py (formed on the host in fp64 with
running sums, checked against the oracle on the CPU), and dK is exactly 0.

Exact scaling. Every step of the kernels is linear in V (forward) and in dO
(backward, O held fixed), and multiplying by a power of two commutes with
every rounding on the way (no value here is near overflow or the subnormal
range), so V -> 2V doubles O bit for bit and leaves the LSE bits alone, and
dO -> 2 dO doubles dQ, dK and dV bit for bit; dO = 0 gives exact zeros.

Shapes: one rank's share of the 131,072-token workload (32 heads over 8
ranks: 4 local heads of 128, causal) launched as the benchmark launches it,
and smaller bidirectional, d_h = 64, cross-attention, grouped-query,
block-sparse and fp32 cases.
"""
import numpy as np
import pytest

import exact_attention_ulysses_amd as U
from workloads import block_layout, custom

from closed_forms import zero_query_attention
from gpu_common import LSE_ABS, check_close, to_f64, to_host_bits, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    U.lib()


class Case:
    """One attention problem: global sizes as the entry points take them."""

    def __init__(self, B, Lq, Lk, Hq, Hkv, d, P, causal, dtype="bf16", sparse=None):
        self.B, self.Lq, self.Lk, self.Hq, self.Hkv, self.d, self.P = B, Lq, Lk, Hq, Hkv, d, P
        self.causal, self.dtype, self.sparse = causal, dtype, sparse
        self.Hql, self.Hkl = Hq // P, U.kv_local_heads(Hkv, P)
        self.G = self.Hql // self.Hkl
        self.plain = Hq == Hkv and Lq == Lk and sparse is None

    def __repr__(self):
        return (f"B{self.B}-Lq{self.Lq}-Lk{self.Lk}-Hq{self.Hq}-Hkv{self.Hkv}-d{self.d}-P{self.P}-"
                f"{'causal' if self.causal else 'full'}-{self.dtype}{'-sparse' if self.sparse else ''}")

    def tdtype(self):
        torch = torch_mod()
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def draw(self, name, seed, scale):
        torch = torch_mod()
        rows, heads = (self.Lq, self.Hql) if name in ("q", "do") else (self.Lk, self.Hkl)
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        x = torch.randn((self.B, rows, heads, self.d), generator=g, device="cuda", dtype=torch.float32) * scale
        return x.to(self.tdtype())

    def layout(self):
        wl = custom(self.B, self.Lq, self.Hql, self.d, 1, causal=self.causal, index=self.sparse,
                    block=U.SPARSE_BLOCK, window=3, n_global=1, n_random=2)
        return torch_mod().from_numpy(block_layout(wl)).to("cuda")

    def fwd(self, q, k, v, layout=None):
        torch = torch_mod()
        o = torch.empty_like(q)
        lse = torch.empty((self.B, self.Hql, self.Lq), dtype=torch.float32, device="cuda")
        if layout is not None:
            U.ulysses_attn_fwd_block_sparse(q, k, v, o, lse, layout, self.B, self.Lq, self.Hq, self.Hkv, self.d,
                                            self.P, self.causal)
        elif self.plain:
            U.ulysses_attn_fwd(q, k, v, o, lse, self.B, self.Lq, self.Hq, self.d, self.P, self.causal)
        else:
            U.ulysses_attn_fwd_gqa(q, k, v, o, lse, self.B, self.Lq, self.Lk, self.Hq, self.Hkv, self.d, self.P,
                                   self.causal)
        return o, lse

    def bwd(self, q, k, v, o, do, lse, layout=None):
        torch = torch_mod()
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dc = U.BF16 if self.dtype == "bf16" else U.FP32
        if layout is not None:
            n = U.ulysses_attn_bwd_block_sparse_workspace_bytes(self.B, self.Lq, self.Hq, self.Hkv, self.d, self.P,
                                                                self.causal)
        elif self.plain:
            n = U.ulysses_attn_bwd_workspace_bytes(self.B, self.Lq, self.Hq, self.d, self.P, self.causal, dc)
        else:
            n = U.ulysses_attn_bwd_gqa_workspace_bytes(self.B, self.Lq, self.Lk, self.Hq, self.Hkv, self.d, self.P,
                                                       self.causal, dc)
        assert n > 0, f"no workspace size for {self}"
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        if layout is not None:
            U.ulysses_attn_bwd_block_sparse(q, k, v, o, do, lse, dq, dk, dv, layout, ws, self.B, self.Lq, self.Hq,
                                            self.Hkv, self.d, self.P, self.causal)
        elif self.plain:
            U.ulysses_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, self.B, self.Lq, self.Hq, self.d, self.P,
                               self.causal)
        else:
            U.ulysses_attn_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, ws, self.B, self.Lq, self.Lk, self.Hq, self.Hkv,
                                   self.d, self.P, self.causal)
        return dq, dk, dv


HEADLINE = Case(1, 131072, 131072, 32, 32, 128, 8, True)
ZERO_Q_CASES = [
    HEADLINE,
    Case(2, 8192, 8192, 4, 4, 64, 1, False),            # bidirectional, d_h = 64, two batch entries
    Case(1, 4096, 65536, 4, 4, 128, 1, False),          # cross-attention
    Case(1, 32768, 32768, 8, 2, 128, 1, True),          # four query heads per K/V head
    Case(1, 1000, 1000, 4, 4, 64, 2, True),             # ragged last tiles
    Case(1, 256, 256, 8, 8, 64, 4, True, dtype="fp32"),
]


@pytest.mark.parametrize("case", ZERO_Q_CASES, ids=repr)
def test_zero_queries_closed_forms(case):
    torch = torch_mod()
    k = case.draw("k", 11, 0.5)
    v = case.draw("v", 12, 0.5)
    do = case.draw("do", 13, 1.0)
    q = torch.zeros((case.B, case.Lq, case.Hql, case.d), dtype=case.tdtype(), device="cuda")
    o, lse = case.fwd(q, k, v)
    dq, dk, dv = case.bwd(q, k, v, o, do, lse)
    torch.cuda.synchronize()
    dt = case.dtype
    assert np.all(to_f64(dk, dt) == 0), f"dK {case} is not zero"
    kh, vh, doh = (to_f64(t, dt) for t in (k, v, do))
    oh, dqh, dvh = (to_f64(t, dt) for t in (o, dq, dv))
    lseh = lse.cpu().numpy()
    for b in range(case.B):
        dv_want = np.zeros((case.Hkl, case.Lk, case.d))
        for h in range(case.Hql):
            j = h // case.G
            r = zero_query_attention(kh[b, :, j], vh[b, :, j], doh[b, :, h], case.causal, case.Lq)
            tag = f"{case} b{b} h{h}"
            check_close(f"O {tag}", oh[b, :, h], r["o"], dt)
            assert np.max(np.abs(lseh[b, h] - r["lse"])) <= LSE_ABS[dt], f"LSE {tag}"
            check_close(f"dQ {tag}", dqh[b, :, h], r["dq"], dt)
            dv_want[j] += r["dv"]
        for j in range(case.Hkl):
            check_close(f"dV {case} b{b} kv{j}", dvh[b, :, j], dv_want[j], dt)


SCALE_CASES = [
    HEADLINE,
    Case(1, 32768, 32768, 8, 2, 128, 1, True),
    Case(1, 16384, 16384, 4, 4, 128, 1, True, sparse=731),
    Case(1, 12288, 12288, 4, 4, 64, 1, False, sparse=733),
    Case(1, 4096, 65536, 4, 4, 64, 1, False),
    Case(1, 256, 256, 8, 8, 64, 4, True, dtype="fp32"),
]


@pytest.mark.parametrize("case", SCALE_CASES, ids=repr)
def test_power_of_two_scaling_is_exact(case):
    torch = torch_mod()
    q = case.draw("q", 21, 0.5)
    k = case.draw("k", 22, 0.5)
    v = case.draw("v", 23, 0.5)
    do = case.draw("do", 24, 1.0)
    layout = case.layout() if case.sparse else None
    o, lse = case.fwd(q, k, v, layout)
    o2, lse2 = case.fwd(q, k, v * 2, layout)
    grads = case.bwd(q, k, v, o, do, lse, layout)
    grads2 = case.bwd(q, k, v, o, do * 2, lse, layout)
    grads0 = case.bwd(q, k, v, o, torch.zeros_like(do), lse, layout)
    torch.cuda.synchronize()
    dt = case.dtype
    np.testing.assert_array_equal(to_host_bits(lse2), to_host_bits(lse), err_msg=f"LSE {case}")
    assert np.array_equal(to_f64(o2, dt), 2 * to_f64(o, dt)), f"O(2V) != 2 O(V) for {case}"
    for name, g, g2, g0 in zip(("dQ", "dK", "dV"), grads, grads2, grads0):
        a, a2 = to_f64(g, dt), to_f64(g2, dt)
        assert np.any(a != 0), f"{name} {case} is all zero"
        assert np.array_equal(a2, 2 * a), f"{name}(2 dO) != 2 {name}(dO) for {case}"
        assert np.all(to_f64(g0, dt) == 0), f"{name}(dO = 0) is not zero for {case}"
