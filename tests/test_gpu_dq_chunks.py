"""GPU parity of backward launches that cut their walks into balanced chunks.

Launches of few 128-row query blocks split every block's walk over its key
tiles between several workgroups, whose fp32 partial sums a reduce kernel
adds in chunk order (tests/plans.py restates the plan). Every case below is
one the host cuts (asserted), with several chunks per block: ragged
sequence ends, both head dims, grouped-query heads, bidirectional and
cross-attention. Causal dK/dV launches of few key-block columns likewise cut
key block kb into parts of near-equal length (the last test). dQ, dK and dV
are compared element by element with the fp64 oracle on the same input bits;
a chunked launch is bitwise repeatable. The forward of the smallest launches
shares each 64-row block's key walk among four wave groups; its O and LSE
are checked the same way.
"""
import numpy as np
import pytest

import exact_attention_ulysses_amd as U
import oracle
from workloads import custom, host_tensor

from gpu_common import LSE_ABS, check_close, shared_head_allowed, to_device, to_f64, to_host_bits, torch_mod
from plans import dkdv_chunk_t, dq_chunk_items, fwd_groups

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    U.lib()


CASES = [  # B, Lq, Lk, Hq, Hkv, d, causal
    (1, 2000, 2000, 1, 1, 128, True),      # 16 chunks in the last block, ragged end
    (1, 3000, 3000, 2, 2, 64, True),
    (2, 2000, 2000, 2, 1, 128, True),      # two query heads per K/V head, two batch entries
    (1, 1000, 1000, 1, 1, 128, False),     # 8 chunks per block
    (1, 300, 20000, 2, 2, 128, False),     # cross-attention: 63 chunks per block
]


def _inputs(B, Lq, Lk, Hq, Hkv, d):
    base = 900 + Lq + 3 * Lk + 5 * Hq + Hkv + d
    draw = lambda L, H, n: host_tensor(custom(B, L, H, d, 1, dtype="bf16", index=base), n).reshape(B, L, H, d)
    host = {n: draw(Lq, Hq, n) for n in ("q", "do")}
    host.update({n: draw(Lk, Hkv, n) for n in ("k", "v")})
    return host


def _run(host, B, Lq, Lk, Hq, Hkv, d, causal):
    torch = torch_mod()
    q, k, v, do = (to_device(host[n], "bf16") for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd_gqa(q, k, v, o, lse, B, Lq, Lk, Hq, Hkv, d, 1, causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(U.ulysses_attn_bwd_gqa_workspace_bytes(B, Lq, Lk, Hq, Hkv, d, 1, causal),
                     dtype=torch.uint8, device="cuda")
    U.ulysses_attn_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, ws, B, Lq, Lk, Hq, Hkv, d, 1, causal)
    return dq, dk, dv


def _check_against_oracle(B, Lq, Lk, Hq, Hkv, d, causal):
    host = _inputs(B, Lq, Lk, Hq, Hkv, d)
    dq, dk, dv = _run(host, B, Lq, Lk, Hq, Hkv, d, causal)
    f = {n: oracle.to_f64(host[n], "bf16") for n in host}
    dq_r, dk_r, dv_r = oracle.attn_bwd_gqa(f["q"], f["k"], f["v"], f["do"], causal)
    check_close("dQ", to_f64(dq, "bf16"), dq_r, "bf16")
    G = Hq // Hkv
    allowed = {"dK": None, "dV": None}
    if G > 1:   # a shared K/V head sums its G query heads' gradients
        parts = {"dK": np.zeros((G,) + dk_r.shape), "dV": np.zeros((G,) + dv_r.shape)}
        for b in range(B):
            for h in range(Hq):
                r = oracle.attn_bwd_head(f["q"][b, :, h], f["k"][b, :, h // G], f["v"][b, :, h // G],
                                         f["do"][b, :, h], causal)
                parts["dK"][h % G, b, :, h // G] = r[1]
                parts["dV"][h % G, b, :, h // G] = r[2]
        allowed = {nm: shared_head_allowed(parts[nm], want, "bf16") for nm, want in (("dK", dk_r), ("dV", dv_r))}
    check_close("dK", to_f64(dk, "bf16"), dk_r, "bf16", allowed=allowed["dK"])
    check_close("dV", to_f64(dv, "bf16"), dv_r, "bf16", allowed=allowed["dV"])


@pytest.mark.parametrize("B,Lq,Lk,Hq,Hkv,d,causal", CASES)
def test_chunked_dq_matches_oracle(B, Lq, Lk, Hq, Hkv, d, causal):
    assert dq_chunk_items(B, Lq, Lk, Hq, causal) > 0, "the host no longer cuts this launch"
    _check_against_oracle(B, Lq, Lk, Hq, Hkv, d, causal)


DKDV_CASES = [  # B, L, Hq, Hkv, d: causal, all with a balanced dK/dV split
    (1, 2000, 2, 1, 128),     # two query heads per K/V head, ragged end: parts of at most 12 tiles
    (2, 1500, 2, 2, 64),
    (1, 4096, 4, 4, 128),     # the 4K x 4 heads shape: 252 parts of at most 22 tiles
]


@pytest.mark.parametrize("B,L,Hq,Hkv,d", DKDV_CASES)
def test_balanced_dkdv_split_matches_oracle(B, L, Hq, Hkv, d):
    assert dkdv_chunk_t(B, L, Hkv, True) > 0, "the host no longer cuts this launch"
    _check_against_oracle(B, L, L, Hq, Hkv, d, True)


def _draw_chunked_case(i):
    """Seeded shape (seed 9500 + i) that the host cuts: 1.5K-6K tokens, 1-4
    query heads over 1 or 2 K/V heads, causal or bidirectional, either head
    dim; redrawn until the dQ launch is chunked."""
    rng = np.random.default_rng(9500 + i)
    while True:
        L = int(rng.integers(1500, 6001))
        Hkv = int(rng.choice([1, 2]))
        Hq = Hkv * int(rng.choice([1, 2]))
        d = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        if dq_chunk_items(1, L, L, Hq, causal) > 0:
            return 1, L, L, Hq, Hkv, d, causal


@pytest.mark.parametrize("i", range(8))
def test_random_chunked_launches_match_oracle(i):
    B, Lq, Lk, Hq, Hkv, d, causal = _draw_chunked_case(i)
    print(f"case {i}: B={B} L={Lq} Hq={Hq} Hkv={Hkv} d={d} causal={causal} "
          f"dQ items={dq_chunk_items(B, Lq, Lk, Hq, causal)} dK/dV t={dkdv_chunk_t(B, Lk, Hkv, causal)}", flush=True)
    _check_against_oracle(B, Lq, Lk, Hq, Hkv, d, causal)


FWD4_CASES = [  # B, L, Hq, Hkv, d, causal: launches the forward splits among four wave groups
    (1, 4096, 4, 4, 128, True),
    (1, 2000, 4, 2, 128, True),      # grouped-query, ragged end
    (2, 3000, 2, 2, 64, False),
    (1, 100, 1, 1, 128, True),       # groups left without key tiles
]


@pytest.mark.parametrize("B,L,Hq,Hkv,d,causal", FWD4_CASES)
def test_four_group_forward_matches_oracle(B, L, Hq, Hkv, d, causal):
    assert fwd_groups(B, L, Hq, causal) == 4, "the host no longer uses four groups here"
    torch = torch_mod()
    host = _inputs(B, L, L, Hq, Hkv, d)
    q, k, v = (to_device(host[n], "bf16") for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd_gqa(q, k, v, o, lse, B, L, L, Hq, Hkv, d, 1, causal)
    f = {n: oracle.to_f64(host[n], "bf16") for n in ("q", "k", "v")}
    o_r, lse_r = oracle.attn_fwd_gqa(f["q"], f["k"], f["v"], causal)
    check_close("O", to_f64(o, "bf16"), o_r, "bf16")
    assert np.max(np.abs(lse.cpu().numpy() - lse_r)) <= LSE_ABS["bf16"]


def test_chunked_dq_is_bitwise_repeatable():
    B, Lq, Lk, Hq, Hkv, d, causal = CASES[0]
    host = _inputs(B, Lq, Lk, Hq, Hkv, d)
    first = [to_host_bits(t) for t in _run(host, B, Lq, Lk, Hq, Hkv, d, causal)]
    second = [to_host_bits(t) for t in _run(host, B, Lq, Lk, Hq, Hkv, d, causal)]
    for name, a, b in zip(("dQ", "dK", "dV"), first, second):
        np.testing.assert_array_equal(a, b, err_msg=name)
