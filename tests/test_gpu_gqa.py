"""GPU parity of grouped-query attention, the K/V layout change and
cross-attention, at sizes the full oracle finishes in seconds.

Every case calls the library through the C ABI (the Python binding) and
compares with the fp64 oracle on the same input bits: the K/V layout change
bit-exact, the replica sum to one bf16 rounding, attention within the bf16 /
fp32 bars. Shapes cover several tiles and ragged tails, query groups of 1 to
8 heads, replicated and split K/V heads, queries shorter and longer than the
keys, and a single query.
"""
import numpy as np
import pytest

import exact_attention_ulysses_amd as U
import oracle
from workloads import custom, host_tensor

from gpu_common import (check_close, LSE_ABS, bf16_ulp, shared_head_allowed, to_device, to_f64, to_host_bits,
                        torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    U.lib()


def _draw(B, L, H, d, dtype, name, index):
    """Seeded [B, L, H, d] tensor (bf16 bits or fp32) from the shared generators."""
    wl = custom(B, L, H, d, 1, dtype=dtype, index=index)
    return host_tensor(wl, name).reshape(B, L, H, d)


# ---------------------------------------------------------------------------
# K/V layout change: bit-exact; replica sum: one rounding
# ---------------------------------------------------------------------------

KV_SHAPES = [  # B, L, Hkv, d, P, dtype
    (1, 64, 2, 128, 8, "bf16"), (2, 48, 1, 64, 4, "bf16"), (1, 96, 8, 128, 4, "bf16"),
    (3, 40, 2, 64, 4, "fp32"), (1, 256, 1, 128, 16, "bf16"), (2, 30, 3, 64, 3, "fp32"),
]


@pytest.mark.parametrize("B,L,Hkv,d,P,dtype", KV_SHAPES)
def test_kv_layout_change_bit_exact(B, L, Hkv, d, P, dtype):
    torch = torch_mod()
    rng = np.random.default_rng(L * 31 + Hkv)
    if dtype == "bf16":
        seq = rng.integers(0, 2 ** 16, size=(P, B, L // P, Hkv, d), dtype=np.uint16)
        seq.reshape(-1)[:4] = [0x7FC1, 0xFF80, 0x8000, 0x0001]
    else:
        seq = rng.integers(0, 2 ** 32, size=(P, B, L // P, Hkv, d), dtype=np.uint32).view(np.float32)
    Hl = U.kv_local_heads(Hkv, P)
    xs = to_device(seq, dtype)
    xh = torch.empty((P, B, L, Hl, d), dtype=xs.dtype, device="cuda")
    U.ulysses_seq_to_head_kv(xs, xh, B, L, Hkv, d, P)
    raw = np.uint16 if dtype == "bf16" else np.uint32
    want = oracle.seq_to_head_kv(seq.view(raw), B, L, Hkv, d, P)
    np.testing.assert_array_equal(to_host_bits(xh).view(raw), want)


@pytest.mark.parametrize("B,L,Hkv,d,P,dtype", KV_SHAPES)
def test_kv_gradient_sums_replicas(B, L, Hkv, d, P, dtype):
    torch = torch_mod()
    Hl = U.kv_local_heads(Hkv, P)
    R = P * Hl // Hkv
    g = _draw(P * B, L, Hl, d, dtype, "do", index=300 + L + Hkv)       # [P*B, L, Hl, d]
    gh = g.reshape(P, B, L, Hl, d)
    dev = to_device(gh, dtype)
    out = torch.empty((P, B, L // P, Hkv, d), dtype=dev.dtype, device="cuda")
    U.ulysses_head_to_seq_kv_grad(dev, out, B, L, Hkv, d, P)
    want = oracle.head_to_seq_kv_grad(oracle.to_f64(gh, dtype), B, L, Hkv, d, P)
    got = to_f64(out, dtype)
    if R == 1:   # a pure permutation: bits copied
        np.testing.assert_array_equal(got, want)
        return
    # fp32 accumulation of R terms, then one rounding to the element type
    mag = oracle.head_to_seq_kv_grad(np.abs(oracle.to_f64(gh, dtype)), B, L, Hkv, d, P)
    acc_err = (R - 1) * 2.0 ** -24 * mag
    if dtype == "bf16":   # the fp32 sum y lies within acc_err of want; RNE moves it by half a spacing at |y|
        allowed = 0.5 * bf16_ulp(np.abs(want) + acc_err) + acc_err
    else:
        allowed = acc_err
    assert np.all(np.abs(got - want) <= allowed + 1e-300)


# ---------------------------------------------------------------------------
# attention: grouped-query and cross-attention against the full oracle
# ---------------------------------------------------------------------------

ATTN_CASES = [  # B, Lq, Lkv, Hq, Hkv, d, P, causal, dtype   (global head counts)
    (1, 333, 333, 32, 8, 128, 8, True, "bf16"),      # 4 query heads per K/V head
    (2, 200, 200, 16, 8, 128, 4, True, "bf16"),      # 2 local K/V heads, groups of 2
    (1, 517, 517, 8, 2, 64, 8, True, "bf16"),        # replicated K/V head, 1 query head
    (1, 1000, 1000, 8, 1, 128, 2, False, "bf16"),    # multi-query: 4 heads share one
    (1, 700, 700, 64, 8, 128, 8, True, "bf16"),      # groups of 8
    (1, 300, 1000, 4, 4, 128, 1, False, "bf16"),     # cross: fewer queries than keys
    (2, 1000, 77, 8, 2, 128, 4, False, "bf16"),      # cross + GQA: more queries than keys
    (1, 1, 2048, 2, 2, 128, 1, False, "bf16"),       # a single query
    (1, 129, 64, 2, 1, 64, 1, False, "bf16"),
    (1, 130, 130, 8, 2, 64, 2, True, "fp32"),
    (1, 100, 250, 4, 2, 128, 2, False, "fp32"),
]


def _gqa_inputs(B, Lq, Lkv, Hq, Hkv, d, P, dtype):
    Hql, Hkl = Hq // P, U.kv_local_heads(Hkv, P)
    base = 400 + Lq + 3 * Lkv + 5 * Hq + Hkv + d
    h = {n: _draw(B, Lq, Hql, d, dtype, n, base) for n in ("q", "do")}
    h.update({n: _draw(B, Lkv, Hkl, d, dtype, n, base) for n in ("k", "v")})
    return h


def _fwd(host, B, Lq, Lkv, Hq, Hkv, d, P, causal, dtype):
    torch = torch_mod()
    q, k, v = (to_device(host[n], dtype) for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq // P, Lq), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd_gqa(q, k, v, o, lse, B, Lq, Lkv, Hq, Hkv, d, P, causal)
    return q, k, v, o, lse


@pytest.mark.parametrize("B,Lq,Lkv,Hq,Hkv,d,P,causal,dtype", ATTN_CASES)
def test_gqa_forward_parity(B, Lq, Lkv, Hq, Hkv, d, P, causal, dtype):
    host = _gqa_inputs(B, Lq, Lkv, Hq, Hkv, d, P, dtype)
    _, _, _, o, lse = _fwd(host, B, Lq, Lkv, Hq, Hkv, d, P, causal, dtype)
    f = {n: oracle.to_f64(host[n], dtype) for n in "qkv"}
    o_ref, lse_ref = oracle.attn_fwd_gqa(f["q"], f["k"], f["v"], causal)
    check_close("O", to_f64(o, dtype), o_ref, dtype)
    lse_err = np.max(np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref))
    assert lse_err <= LSE_ABS[dtype], lse_err


@pytest.mark.parametrize("B,Lq,Lkv,Hq,Hkv,d,P,causal,dtype", ATTN_CASES)
def test_gqa_backward_parity(B, Lq, Lkv, Hq, Hkv, d, P, causal, dtype):
    torch = torch_mod()
    host = _gqa_inputs(B, Lq, Lkv, Hq, Hkv, d, P, dtype)
    q, k, v, o, lse = _fwd(host, B, Lq, Lkv, Hq, Hkv, d, P, causal, dtype)
    do = to_device(host["do"], dtype)
    dq = torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(U.ulysses_attn_bwd_gqa_workspace_bytes(B, Lq, Lkv, Hq, Hkv, d, P, causal, U.dtype_code(q)),
                     dtype=torch.uint8, device="cuda")
    U.ulysses_attn_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, ws, B, Lq, Lkv, Hq, Hkv, d, P, causal)
    f = {n: oracle.to_f64(host[n], dtype) for n in ("q", "k", "v", "do")}
    dq_r, dk_r, dv_r = oracle.attn_bwd_gqa(f["q"], f["k"], f["v"], f["do"], causal)
    check_close("dQ", to_f64(dq, dtype), dq_r, dtype)
    G = (Hq // P) // U.kv_local_heads(Hkv, P)
    if G == 1:
        check_close("dK", to_f64(dk, dtype), dk_r, dtype)
        check_close("dV", to_f64(dv, dtype), dv_r, dtype)
        return
    # each K/V head sums the gradients of its G query heads: the bar is the
    # sum of the G parts' bars (one attention output each) plus one rounding
    parts_k = np.zeros((G,) + dk_r.shape)
    parts_v = np.zeros((G,) + dv_r.shape)
    for b in range(B):
        for h in range(Hq // P):
            r = oracle.attn_bwd_head(f["q"][b, :, h], f["k"][b, :, h // G], f["v"][b, :, h // G],
                                     f["do"][b, :, h], causal)
            parts_k[h % G, b, :, h // G] = r[1]
            parts_v[h % G, b, :, h // G] = r[2]
    np.testing.assert_allclose(parts_k.sum(0), dk_r, rtol=0, atol=1e-12)   # the parts add up to the oracle's sum
    check_close("dK", to_f64(dk, dtype), dk_r, dtype, allowed=shared_head_allowed(parts_k, dk_r, dtype))
    check_close("dV", to_f64(dv, dtype), dv_r, dtype, allowed=shared_head_allowed(parts_v, dv_r, dtype))


def test_plain_entry_points_equal_generalised_ones():
    # H_q == H_kv and L_q == L_kv: the two forms run the same kernels bit for bit
    torch = torch_mod()
    B, L, H, d, P = 1, 600, 8, 128, 4
    host = _gqa_inputs(B, L, L, H, H, d, P, "bf16")
    q, k, v, o, lse = _fwd(host, B, L, L, H, H, d, P, True, "bf16")
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    U.ulysses_attn_fwd(q, k, v, o2, lse2, B, L, H, d, P, True)
    do = to_device(host["do"], "bf16")
    grads = []
    for fn in ("gqa", "plain"):
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        ws = torch.empty(U.ulysses_attn_bwd_workspace_bytes(B, L, H, d, P), dtype=torch.uint8, device="cuda")
        if fn == "gqa":
            U.ulysses_attn_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, ws, B, L, L, H, H, d, P, True)
        else:
            U.ulysses_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, B, L, H, d, P, True)
        grads.append([to_host_bits(t) for t in (dq, dk, dv)])
    np.testing.assert_array_equal(to_host_bits(o), to_host_bits(o2))
    np.testing.assert_array_equal(to_host_bits(lse), to_host_bits(lse2))
    for a, b in zip(*grads):
        np.testing.assert_array_equal(a, b)


def test_gqa_leaves_guard_regions_untouched():
    torch = torch_mod()
    B, Lq, Lkv, Hq, Hkv, d, P = 1, 333, 333, 8, 2, 128, 2
    host = _gqa_inputs(B, Lq, Lkv, Hq, Hkv, d, P, "bf16")
    q, k, v = (to_device(host[x], "bf16") for x in "qkv")
    do = to_device(host["do"], "bf16")
    g = 8192
    nq, nk = q.numel(), k.numel()
    bufs = [torch.full((n + 2 * g,), 0x3C3C, dtype=torch.int16, device="cuda") for n in (nq, nq, nk, nk)]
    o, dq = (b_[g:g + nq].view(torch.bfloat16).view(q.shape) for b_ in bufs[:2])
    dk, dv = (b_[g:g + nk].view(torch.bfloat16).view(k.shape) for b_ in bufs[2:])
    nl = B * (Hq // P) * Lq
    lbuf = torch.full((nl + 2 * g,), -7.0, dtype=torch.float32, device="cuda")
    lse = lbuf[g:g + nl]
    U.ulysses_attn_fwd_gqa(q, k, v, o, lse, B, Lq, Lkv, Hq, Hkv, d, P, True)
    ws = torch.empty(U.ulysses_attn_bwd_gqa_workspace_bytes(B, Lq, Lkv, Hq, Hkv, d, P), dtype=torch.uint8,
                     device="cuda")
    U.ulysses_attn_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, ws, B, Lq, Lkv, Hq, Hkv, d, P, True)
    torch.cuda.synchronize()
    for b_, n in zip(bufs, (nq, nq, nk, nk)):
        assert bool((b_[:g] == 0x3C3C).all()) and bool((b_[g + n:] == 0x3C3C).all())
    assert bool((lbuf[:g] == -7.0).all()) and bool((lbuf[g + nl:] == -7.0).all())


# ---------------------------------------------------------------------------
# the whole per-rank pipeline with grouped-query attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,L,Hq,Hkv,d,P,dtype", [(1, 256, 16, 4, 128, 4, "bf16"), (1, 256, 16, 2, 128, 8, "bf16"),
                                                  (2, 96, 8, 1, 64, 4, "fp32")])
def test_gqa_pipeline_against_single_device_attention(B, L, Hq, Hkv, d, P, dtype):
    """seq_to_head (Q, dO), seq_to_head_kv (K, V), attention on all P head groups
    at once (batch B*P), head_to_seq (O, dQ), head_to_seq_kv_grad (dK, dV);
    against GQA attention on the unsharded tensors."""
    torch = torch_mod()
    wl = custom(B, L, Hq, d, P, dtype=dtype, Hkv=Hkv, index=500 + L + Hkv)
    host = {n: host_tensor(wl, n) for n in ("q", "k", "v", "do")}
    Hql, Hl = Hq // P, U.kv_local_heads(Hkv, P)
    dev = {n: to_device(host[n], dtype) for n in host}
    hq = {}
    for n in ("q", "do"):
        hq[n] = torch.empty((P, B, L, Hql, d), dtype=dev[n].dtype, device="cuda")
        U.ulysses_seq_to_head(dev[n], hq[n], B, L, Hq, d, P)
    for n in ("k", "v"):
        hq[n] = torch.empty((P, B, L, Hl, d), dtype=dev[n].dtype, device="cuda")
        U.ulysses_seq_to_head_kv(dev[n], hq[n], B, L, Hkv, d, P)
    BP = B * P
    o = torch.empty_like(hq["q"])
    lse = torch.empty((BP, Hql, L), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd_gqa(hq["q"], hq["k"], hq["v"], o, lse, BP, L, L, Hq, Hkv, d, P, True)
    dq, dk, dv = torch.empty_like(hq["q"]), torch.empty_like(hq["k"]), torch.empty_like(hq["v"])
    ws = torch.empty(U.ulysses_attn_bwd_gqa_workspace_bytes(BP, L, L, Hq, Hkv, d, P, True, U.dtype_code(o)),
                     dtype=torch.uint8, device="cuda")
    U.ulysses_attn_bwd_gqa(hq["q"], hq["k"], hq["v"], o, hq["do"], lse, dq, dk, dv, ws, BP, L, L, Hq, Hkv, d, P,
                           True)
    out = {}
    for n, t in (("o", o), ("dq", dq)):
        out[n] = torch.empty_like(dev["q"])
        U.ulysses_head_to_seq(t, out[n], B, L, Hq, d, P)
    for n, t in (("dk", dk), ("dv", dv)):
        out[n] = torch.empty_like(dev["k"])
        U.ulysses_head_to_seq_kv_grad(t, out[n], B, L, Hkv, d, P)

    f = {n: oracle.to_f64(host[n], dtype) for n in host}
    glob = lambda a: np.concatenate(list(a), axis=1)  # noqa: E731  [P,B,L/P,..] -> [B,L,..]
    o_r, _ = oracle.attn_fwd_gqa(glob(f["q"]), glob(f["k"]), glob(f["v"]), True)
    dq_r, dk_r, dv_r = oracle.attn_bwd_gqa(glob(f["q"]), glob(f["k"]), glob(f["v"]), glob(f["do"]), True)
    check_close("O", glob(to_f64(out["o"], dtype)), o_r, dtype)
    check_close("dQ", glob(to_f64(out["dq"], dtype)), dq_r, dtype)
    R = P * Hl // Hkv
    # dK/dV with replicas: R per-rank gradients, each within the bar of one
    # attention output, summed and rounded once more
    qh = oracle.seq_to_head(f["q"], B, L, Hq, d, P)
    doh = oracle.seq_to_head(f["do"], B, L, Hq, d, P)
    kh = oracle.seq_to_head_kv(f["k"], B, L, Hkv, d, P)
    vh = oracle.seq_to_head_kv(f["v"], B, L, Hkv, d, P)
    G = Hql // Hl
    for name, idx, want in (("dK", 1, dk_r), ("dV", 2, dv_r)):
        # split each rank's K/V gradient into its query heads' parts, then gather
        # the parts of every replica: R * G parts per K/V head in seq layout
        per_head = []
        for g in range(G):
            rank_parts = np.zeros((P, B, L, Hl, d))
            for p in range(P):
                for b in range(B):
                    for j in range(Hl):
                        h = j * G + g
                        r = oracle.attn_bwd_head(qh[p, b, :, h], kh[p, b, :, j], vh[p, b, :, j], doh[p, b, :, h],
                                                 True)
                        rank_parts[p, b, :, j] = r[idx]
            for rep in range(R):   # replica rep of each K/V head, alone
                only = np.zeros_like(rank_parts)
                for p in range(P):
                    if p % R == rep:
                        only[p] = rank_parts[p]
                per_head.append(glob(oracle.head_to_seq_kv_grad(only, B, L, Hkv, d, P)))
        np.testing.assert_allclose(np.sum(per_head, axis=0), want, rtol=0, atol=1e-12)
        check_close(name, glob(to_f64(out[name.lower()], dtype)), want, dtype,
                    allowed=shared_head_allowed(per_head, want, dtype))
