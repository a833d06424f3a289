"""GPU parity of the dense backward's one-walk dK/dV launches.

Launches of many key-block columns (batch x local K/V heads x 128-token key
blocks: at least 512 causal, more than 128 bidirectional) give each column
one workgroup that walks every query tile of its key block, the schedule of
the long-sequence workloads. The cases below are such launches (asserted) at
sizes the fp64 oracle finishes in seconds: ragged sequence ends (the last
query tile partly past the end), grouped-query heads (a shared K/V head sums
its query heads' gradients), bidirectional and cross-attention, both head
dims. dQ, dK and dV are compared element by element with the oracle on the
same input bits, and a second call must repeat the first bit for bit.
"""
import numpy as np
import pytest

import exact_attention_ulysses_amd as U
import oracle
from workloads import custom, host_tensor

from gpu_common import check_close, shared_head_allowed, to_device, to_f64, to_host_bits, torch_mod
from plans import dkdv_whole_walks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    U.lib()


CASES = [  # B, Lq, Lk, Hq, Hkv, d, causal
    (4, 4096, 4096, 4, 4, 128, True),      # 512 columns of 32 key blocks
    (4, 4000, 4000, 8, 4, 128, True),      # two query heads per K/V head, ragged end
    (8, 4100, 4100, 2, 2, 128, True),      # a last query tile of 4 valid rows
    (2, 2100, 2100, 4, 4, 128, False),     # bidirectional, 136 columns
    (1, 1000, 9000, 4, 2, 128, False),     # cross-attention, G = 2
    (4, 4096, 4096, 4, 4, 64, True),       # d_h = 64
]


def _inputs(B, Lq, Lk, Hq, Hkv, d):
    base = 1300 + Lq + 3 * Lk + 5 * Hq + Hkv + d + B
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


@pytest.mark.parametrize("B,Lq,Lk,Hq,Hkv,d,causal", CASES)
def test_one_walk_dkdv_matches_oracle(B, Lq, Lk, Hq, Hkv, d, causal):
    assert dkdv_whole_walks(B, Lk, Hkv, causal), "the host splits this launch"
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


def test_one_walk_dkdv_is_bitwise_repeatable():
    B, Lq, Lk, Hq, Hkv, d, causal = CASES[1]
    host = _inputs(B, Lq, Lk, Hq, Hkv, d)
    first = [to_host_bits(t) for t in _run(host, B, Lq, Lk, Hq, Hkv, d, causal)]
    second = [to_host_bits(t) for t in _run(host, B, Lq, Lk, Hq, Hkv, d, causal)]
    for name, a, b in zip(("dQ", "dK", "dV"), first, second):
        np.testing.assert_array_equal(a, b, err_msg=name)
