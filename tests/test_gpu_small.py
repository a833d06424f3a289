"""GPU parity at sizes the full oracle finishes in seconds.

Every case calls the library through the C ABI (the Python binding) and
compares element by element with the fp64 oracle on the same input bits:
permutations bit-exact; attention within the bf16 / fp32 bars. Shapes cover
several tiles, ragged tails, a single token, both head dims, causal and
bidirectional, several batches and head groups.
"""
import numpy as np
import pytest

import exact_attention_ulysses_amd as U
import oracle
from workloads import custom, host_tensor

from gpu_common import check_close, LSE_ABS, to_device, to_f64, to_host_bits, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    U.lib()


# ---------------------------------------------------------------------------
# permutations: bit-exact
# ---------------------------------------------------------------------------

PERM_SHAPES = [  # B, L, H, d, P, dtype
    (1, 64, 8, 128, 4, "bf16"), (2, 48, 6, 64, 3, "bf16"), (3, 40, 8, 64, 8, "fp32"),
    (1, 256, 8, 64, 4, "fp32"), (1, 96, 12, 128, 4, "bf16"), (2, 32, 4, 128, 1, "bf16"),
    (1, 1024, 32, 128, 8, "bf16"), (1, 520, 40, 64, 5, "fp32"), (4, 16, 16, 128, 16, "bf16"),
]


def _bits(shape, dtype, seed):
    rng = np.random.default_rng(seed)
    if dtype == "bf16":
        x = rng.integers(0, 2 ** 16, size=shape, dtype=np.uint16)
        x.reshape(-1)[:8] = [0x7FC1, 0xFFC3, 0x7F81, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x807F]  # NaN payloads, inf, -0, subnormal
        return x
    x = rng.integers(0, 2 ** 32, size=shape, dtype=np.uint32)
    x.reshape(-1)[:4] = [0x7FC00001, 0xFF800000, 0x80000000, 0x00000001]
    return x.view(np.float32)


@pytest.mark.parametrize("B,L,H,d,P,dtype", PERM_SHAPES)
def test_permutations_bit_exact(B, L, H, d, P, dtype):
    torch = torch_mod()
    seq = _bits((P, B, L // P, H, d), dtype, seed=B * 1000 + L + H)
    xs = to_device(seq, dtype)
    xh = torch.empty_like(xs).view(P, B, L, H // P, d)
    U.ulysses_seq_to_head(xs, xh, B, L, H, d, P)
    want = oracle.seq_to_head(seq.view(np.uint16 if dtype == "bf16" else np.uint32), B, L, H, d, P)
    got = to_host_bits(xh).view(np.uint16 if dtype == "bf16" else np.uint32)
    np.testing.assert_array_equal(got, want)
    back = torch.empty_like(xs)
    U.ulysses_head_to_seq(xh, back, B, L, H, d, P)
    np.testing.assert_array_equal(to_host_bits(back).view(got.dtype), seq.view(got.dtype))
    # head_to_seq on independent bits
    hb = _bits((P, B, L, H // P, d), dtype, seed=7 + L)
    y = torch.empty_like(xs)
    U.ulysses_head_to_seq(to_device(hb, dtype), y, B, L, H, d, P)
    np.testing.assert_array_equal(to_host_bits(y).view(got.dtype),
                                  oracle.head_to_seq(hb.view(got.dtype), B, L, H, d, P))


def test_permutation_leaves_guard_regions_untouched():
    torch = torch_mod()
    B, L, H, d, P = 1, 64, 8, 128, 4
    n = B * L * H * d
    guard = 4096
    buf = torch.full((n + 2 * guard,), 0x5A5A, dtype=torch.int16, device="cuda")
    src = to_device(_bits((P, B, L // P, H, d), "bf16", 3), "bf16")
    out = buf[guard:guard + n].view(torch.bfloat16)
    U.ulysses_seq_to_head(src, out, B, L, H, d, P)
    torch.cuda.synchronize()
    assert bool((buf[:guard] == 0x5A5A).all()) and bool((buf[guard + n:] == 0x5A5A).all())


# ---------------------------------------------------------------------------
# attention forward / backward against the full oracle
# ---------------------------------------------------------------------------

ATTN_CASES = [  # B, L, H, d, P, causal, dtype
    (1, 1, 1, 128, 1, True, "bf16"),
    (1, 64, 1, 128, 1, True, "bf16"),
    (1, 200, 2, 128, 1, True, "bf16"),
    (2, 333, 2, 128, 1, False, "bf16"),
    (1, 1024, 4, 128, 1, True, "bf16"),
    (1, 777, 8, 128, 4, True, "bf16"),
    (1, 517, 1, 64, 1, True, "bf16"),
    (3, 256, 2, 64, 1, False, "bf16"),
    (1, 2048, 1, 128, 1, False, "bf16"),
    (1, 256, 2, 64, 1, True, "fp32"),
    (2, 100, 1, 128, 1, False, "fp32"),
    (1, 1, 1, 64, 1, True, "fp32"),
    (1, 300, 4, 128, 2, True, "fp32"),
]


def _inputs(B, L, H, d, P, dtype, backward):
    Hh = H // P
    wl = custom(B, L, Hh, d, 1, dtype=dtype, index=200 + L + 7 * Hh + d)
    names = ["q", "k", "v"] + (["do"] if backward else [])
    host = {n: host_tensor(wl, n).reshape(B, L, Hh, d) for n in names}
    return host


def _run_fwd(host, B, L, H, d, P, causal, dtype):
    torch = torch_mod()
    q, k, v = (to_device(host[n], dtype) for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((B, H // P, L), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd(q, k, v, o, lse, B, L, H, d, P, causal)
    return q, k, v, o, lse


@pytest.mark.parametrize("B,L,H,d,P,causal,dtype", ATTN_CASES)
def test_forward_parity(B, L, H, d, P, causal, dtype):
    host = _inputs(B, L, H, d, P, dtype, backward=False)
    _, _, _, o, lse = _run_fwd(host, B, L, H, d, P, causal, dtype)
    f = {n: oracle.to_f64(host[n], dtype) for n in "qkv"}
    o_ref, lse_ref = oracle.attn_fwd(f["q"], f["k"], f["v"], causal)
    check_close("O", to_f64(o, dtype), o_ref, dtype)
    lse_err = np.max(np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref))
    assert lse_err <= LSE_ABS[dtype], lse_err


@pytest.mark.parametrize("B,L,H,d,P,causal,dtype", ATTN_CASES)
def test_backward_parity(B, L, H, d, P, causal, dtype):
    torch = torch_mod()
    host = _inputs(B, L, H, d, P, dtype, backward=True)
    q, k, v, o, lse = _run_fwd(host, B, L, H, d, P, causal, dtype)
    do = to_device(host["do"], dtype)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(U.ulysses_attn_bwd_workspace_bytes(B, L, H, d, P, causal, U.dtype_code(q)),
                     dtype=torch.uint8, device="cuda")
    U.ulysses_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, B, L, H, d, P, causal)
    f = {n: oracle.to_f64(host[n], dtype) for n in ("q", "k", "v", "do")}
    dq_r, dk_r, dv_r, *_ = oracle.attn_bwd(f["q"], f["k"], f["v"], f["do"], causal)
    check_close("dQ", to_f64(dq, dtype), dq_r, dtype)
    check_close("dK", to_f64(dk, dtype), dk_r, dtype)
    check_close("dV", to_f64(dv, dtype), dv_r, dtype)


def test_results_are_bitwise_reproducible():
    torch = torch_mod()
    B, L, H, d, P, causal = 1, 1000, 2, 128, 1, True
    host = _inputs(B, L, H, d, P, "bf16", backward=True)
    outs = []
    for _ in range(2):
        q, k, v, o, lse = _run_fwd(host, B, L, H, d, P, causal, "bf16")
        do = to_device(host["do"], "bf16")
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        ws = torch.empty(U.ulysses_attn_bwd_workspace_bytes(B, L, H, d, P), dtype=torch.uint8, device="cuda")
        U.ulysses_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, B, L, H, d, P, causal)
        outs.append([to_host_bits(t) for t in (o, lse, dq, dk, dv)])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


def test_attention_leaves_guard_regions_untouched():
    torch = torch_mod()
    B, L, H, d, P = 1, 333, 2, 128, 1
    host = _inputs(B, L, H, d, P, "bf16", backward=True)
    n = B * L * H * d
    g = 8192
    q, k, v = (to_device(host[x], "bf16") for x in "qkv")
    do = to_device(host["do"], "bf16")
    bufs = [torch.full((n + 2 * g,), 0x3C3C, dtype=torch.int16, device="cuda") for _ in range(4)]
    o, dq, dk, dv = (b_[g:g + n].view(torch.bfloat16).view(B, L, H, d) for b_ in bufs)
    lbuf = torch.full((B * H * L + 2 * g,), -7.0, dtype=torch.float32, device="cuda")
    lse = lbuf[g:g + B * H * L]
    U.ulysses_attn_fwd(q, k, v, o, lse, B, L, H, d, P, True)
    ws = torch.empty(U.ulysses_attn_bwd_workspace_bytes(B, L, H, d, P), dtype=torch.uint8, device="cuda")
    U.ulysses_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, B, L, H, d, P, True)
    torch.cuda.synchronize()
    for b_ in bufs:
        assert bool((b_[:g] == 0x3C3C).all()) and bool((b_[g + n:] == 0x3C3C).all())
    assert bool((lbuf[:g] == -7.0).all()) and bool((lbuf[g + B * H * L:] == -7.0).all())


def test_tiny_fp32_workload_end_to_end():
    """L=256, H=8, d=64, P=4 in fp32: seq_to_head, causal attention on all four
    head groups at once (batch B*P), head_to_seq; against the oracle pipeline."""
    torch = torch_mod()
    from workloads import WORKLOADS
    wl = WORKLOADS["tiny-fp32-L256"]
    B, L, H, d, P = wl.B, wl.L, wl.H, wl.d, wl.P
    host = {n: host_tensor(wl, n) for n in "qkv"}
    heads = {}
    for n in "qkv":
        xs = to_device(host[n], "fp32")
        xh = torch.empty((P, B, L, H // P, d), dtype=torch.float32, device="cuda")
        U.ulysses_seq_to_head(xs, xh, B, L, H, d, P)
        heads[n] = xh
    oh = torch.empty_like(heads["q"])
    lse = torch.empty((P * B, H // P, L), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd(heads["q"], heads["k"], heads["v"], oh, lse, B * P, L, H, d, P, True)
    o_seq = torch.empty((P, B, L // P, H, d), dtype=torch.float32, device="cuda")
    U.ulysses_head_to_seq(oh, o_seq, B, L, H, d, P)
    f = {n: host[n].astype(np.float64) for n in "qkv"}
    o_ref, lse_ref = oracle.ulysses_attention_fwd(f["q"], f["k"], f["v"], B, L, H, d, P, True)
    check_close("O (seq layout)", o_seq.cpu().numpy().astype(np.float64), o_ref, "fp32")
    assert np.max(np.abs(lse.cpu().numpy().reshape(P, B, H // P, L) - lse_ref)) <= 1e-5
