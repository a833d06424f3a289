"""GPU parity of block-sparse attention at sizes the full oracle finishes in seconds.

Every case calls the library through the C ABI (the Python binding) with a
seeded window + global + random block layout and compares with the fp64
oracle on the same input bits. A full layout reproduces the dense kernels
bit for bit where both walk the keys the same way; block rows left empty
must give zero output, LSE -inf and no gradient.
"""
import numpy as np
import pytest

import exact_attention_ulysses_amd as U
import oracle
from workloads import block_layout, custom, host_tensor

from gpu_common import (check_close, LSE_ABS, shared_head_allowed, to_device, to_f64, to_host_bits, torch_mod)

pytestmark = pytest.mark.gpu
BLOCK = U.SPARSE_BLOCK


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    U.lib()


def _draw(B, L, H, d, name, index):
    wl = custom(B, L, H, d, 1, dtype="bf16", index=index)
    return host_tensor(wl, name).reshape(B, L, H, d)


def _case(B, L, Hq, Hkv, d, P, causal, window, n_global, n_random):
    Hql, Hkl = Hq // P, U.kv_local_heads(Hkv, P)
    base = 600 + L + 7 * Hq + Hkv + d + window
    host = {n: _draw(B, L, Hql, d, n, base) for n in ("q", "do")}
    host.update({n: _draw(B, L, Hkl, d, n, base) for n in ("k", "v")})
    lay = block_layout(custom(B, L, Hql, d, 1, causal=causal, index=base, block=BLOCK, window=window,
                              n_global=n_global, n_random=n_random))
    return host, lay


def _run(host, lay, B, L, Hq, Hkv, d, P, causal, backward=True):
    torch = torch_mod()
    dev = {n: to_device(host[n], "bf16") for n in host}
    layout = torch.from_numpy(lay).to("cuda")
    o = torch.empty_like(dev["q"])
    lse = torch.empty((B, Hq // P, L), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd_block_sparse(dev["q"], dev["k"], dev["v"], o, lse, layout, B, L, Hq, Hkv, d, P, causal)
    out = {"o": o, "lse": lse}
    if backward:
        dq = torch.empty_like(dev["q"])
        dk, dv = torch.empty_like(dev["k"]), torch.empty_like(dev["v"])
        ws = torch.empty(U.ulysses_attn_bwd_block_sparse_workspace_bytes(B, L, Hq, Hkv, d, P, causal),
                         dtype=torch.uint8, device="cuda")
        U.ulysses_attn_bwd_block_sparse(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, dq, dk, dv, layout, ws, B,
                                        L, Hq, Hkv, d, P, causal)
        out.update(dq=dq, dk=dk, dv=dv)
    return out


CASES = [  # B, L, Hq, Hkv, d, P, causal, window, n_global, n_random
    (1, 1000, 8, 8, 128, 4, True, 3, 1, 1),      # ragged last block
    (2, 640, 4, 4, 64, 1, True, 2, 0, 2),
    (1, 1024, 8, 2, 128, 2, True, 2, 1, 1),      # 4 query heads share a K/V head
    (1, 777, 4, 4, 128, 1, False, 3, 1, 2),      # bidirectional, ragged
    (1, 2048, 2, 2, 128, 1, True, 4, 1, 3),
]


@pytest.mark.parametrize("B,L,Hq,Hkv,d,P,causal,window,n_global,n_random", CASES)
def test_block_sparse_parity(B, L, Hq, Hkv, d, P, causal, window, n_global, n_random):
    host, lay = _case(B, L, Hq, Hkv, d, P, causal, window, n_global, n_random)
    out = _run(host, lay, B, L, Hq, Hkv, d, P, causal)
    f = {n: oracle.to_f64(host[n], "bf16") for n in host}
    G = (Hq // P) // U.kv_local_heads(Hkv, P)
    # grouped-query attention is multi-head attention on repeated K/V heads
    kr, vr = np.repeat(f["k"], G, axis=2), np.repeat(f["v"], G, axis=2)
    o_r, lse_r = oracle.attn_fwd_block_sparse(f["q"], kr, vr, lay, BLOCK, causal)
    check_close("O", to_f64(out["o"], "bf16"), o_r, "bf16")
    assert np.max(np.abs(out["lse"].cpu().numpy() - lse_r)) <= LSE_ABS["bf16"]
    dq_r, dk_rep, dv_rep = oracle.attn_bwd_block_sparse(f["q"], kr, vr, f["do"], lay, BLOCK, causal)
    check_close("dQ", to_f64(out["dq"], "bf16"), dq_r, "bf16")
    for name, rep in (("dK", dk_rep), ("dV", dv_rep)):
        B_, L_, Hq_, d_ = rep.shape
        parts = np.moveaxis(rep.reshape(B_, L_, Hq_ // G, G, d_), 3, 0)   # [G, B, L, Hkl, d]
        want = parts.sum(axis=0)
        allowed = None if G == 1 else shared_head_allowed(parts, want, "bf16")
        check_close(name, to_f64(out[name.lower()], "bf16"), want, "bf16", allowed=allowed)


@pytest.mark.parametrize("causal", [True, False])
def test_full_layout_equals_dense_kernels_bitwise(causal):
    """Every row goes through the same operations in the block-layout kernels
    and in the dense ones whenever the dense forward walks each query block's
    keys in one pass (grids of 1024 or more 256-row query blocks; smaller
    grids split the walk and round differently, checked against the oracle
    elsewhere) and no layout column is long enough to be split: 4 batch
    entries x 64 local heads x 4 query blocks, 8 key blocks per column."""
    torch = torch_mod()
    B, L, H, d, P = 4, 900, 128, 128, 2
    host, _ = _case(B, L, H, H, d, P, causal, 1, 0, 0)
    nb = -(-L // BLOCK)
    lay = np.ones((H // P, nb, nb), np.uint8)
    sp = _run(host, lay, B, L, H, H, d, P, causal)
    dev = {n: to_device(host[n], "bf16") for n in host}
    o = torch.empty_like(dev["q"])
    lse = torch.empty((B, H // P, L), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd(dev["q"], dev["k"], dev["v"], o, lse, B, L, H, d, P, causal)
    dq, dk, dv = (torch.empty_like(dev["q"]) for _ in range(3))
    ws = torch.empty(U.ulysses_attn_bwd_workspace_bytes(B, L, H, d, P, causal), dtype=torch.uint8, device="cuda")
    U.ulysses_attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, dq, dk, dv, ws, B, L, H, d, P, causal)
    for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_array_equal(to_host_bits(sp[name]), to_host_bits(t), err_msg=name)


def test_empty_block_rows():
    B, L, H, d, P = 1, 640, 2, 128, 1
    host, lay = _case(B, L, H, H, d, P, True, 2, 1, 0)
    lay[:, 2] = 0            # query block 2 sees nothing
    lay[1, 4, :] = 0         # head 1: block 4 neither
    out = _run(host, lay, B, L, H, H, d, P, True)
    o, lse, dq = (to_f64(out[n], "bf16") if n != "lse" else out[n].cpu().numpy() for n in ("o", "lse", "dq"))
    assert np.all(o[:, 256:384] == 0) and np.all(np.isneginf(lse[:, :, 256:384]))
    assert np.all(o[:, 512:640, 1] == 0) and np.all(np.isneginf(lse[:, 1, 512:640]))
    assert np.all(dq[:, 256:384] == 0) and np.all(dq[:, 512:640, 1] == 0)
    f = {n: oracle.to_f64(host[n], "bf16") for n in host}
    o_r, lse_r = oracle.attn_fwd_block_sparse(f["q"], f["k"], f["v"], lay, BLOCK, True)
    check_close("O", o, o_r, "bf16")
    dq_r, dk_r, dv_r = oracle.attn_bwd_block_sparse(f["q"], f["k"], f["v"], f["do"], lay, BLOCK, True)
    check_close("dQ", dq, dq_r, "bf16")
    check_close("dK", to_f64(out["dk"], "bf16"), dk_r, "bf16")
    check_close("dV", to_f64(out["dv"], "bf16"), dv_r, "bf16")


@pytest.mark.parametrize("B,L,Hq,Hkv,d,causal", [(1, 4096, 8, 2, 128, True), (2, 2048, 4, 1, 64, False)])
def test_heavy_columns_are_split_and_match(B, L, Hq, Hkv, d, causal):
    """Global key blocks seen by every query block of four query heads (64 to
    128 pairs) are cut into chunks whose partial sums are added in a fixed
    order: the result matches the oracle and is the same on every run (the
    second case splits columns of both batch entries)."""
    P = 1
    host, lay = _case(B, L, Hq, Hkv, d, P, causal, 2, 3, 2)
    out = _run(host, lay, B, L, Hq, Hkv, d, P, causal)
    again = _run(host, lay, B, L, Hq, Hkv, d, P, causal)
    for n in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(to_host_bits(out[n]), to_host_bits(again[n]), err_msg=n)
    f = {n: oracle.to_f64(host[n], "bf16") for n in host}
    G = Hq // Hkv
    kr, vr = np.repeat(f["k"], G, axis=2), np.repeat(f["v"], G, axis=2)
    dq_r, dk_rep, dv_rep = oracle.attn_bwd_block_sparse(f["q"], kr, vr, f["do"], lay, BLOCK, causal)
    check_close("dQ", to_f64(out["dq"], "bf16"), dq_r, "bf16")
    for name, rep in (("dK", dk_rep), ("dV", dv_rep)):
        parts = np.moveaxis(rep.reshape(B, L, Hkv, G, d), 3, 0)
        want = parts.sum(axis=0)
        check_close(name, to_f64(out[name.lower()], "bf16"), want, "bf16",
                    allowed=shared_head_allowed(parts, want, "bf16"))


def test_columns_beyond_the_partial_slots_stay_whole():
    """A full bidirectional layout over 128 key blocks and 4 heads asks for 2048
    partial-sum slots; the first 512 split the columns of head 0, the columns of
    heads 1-3 are walked whole. Sampled key columns of both kinds, and sampled
    query rows, match the oracle."""
    B, L, H, d, P, causal = 1, 16384, 4, 64, 1, False
    nb = L // BLOCK
    host = {n: _draw(B, L, H, d, n, 913) for n in ("q", "k", "v", "do")}
    lay = np.ones((H, nb, nb), np.uint8)
    out = _run(host, lay, B, L, H, H, d, P, causal)
    f = {n: oracle.to_f64(host[n], "bf16") for n in host}
    cols = [0, 127, 5000, 16383]
    for h in (0, 1):
        _, dk_r, dv_r = oracle.attn_dkv_cols_block_sparse(f["q"][0, :, h], f["k"][0, :, h], f["v"][0, :, h],
                                                          f["do"][0, :, h], cols, lay[h], BLOCK, causal)
        check_close(f"dK head {h}", to_f64(out["dk"][0, cols, h], "bf16"), dk_r, "bf16", fro=False)
        check_close(f"dV head {h}", to_f64(out["dv"][0, cols, h], "bf16"), dv_r, "bf16", fro=False)
    rows = [1, 4096, 16383]
    r = oracle.attn_rows_block_sparse(f["q"][0, :, 3], f["k"][0, :, 3], f["v"][0, :, 3], rows, lay[3], BLOCK,
                                      causal, do=f["do"][0, :, 3])
    check_close("O rows", to_f64(out["o"][0, rows, 3], "bf16"), r["o"], "bf16", fro=False)
    check_close("dQ rows", to_f64(out["dq"][0, rows, 3], "bf16"), r["dq"], "bf16", fro=False)
