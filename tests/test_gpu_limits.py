"""GPU parity at the largest sizes the entry points accept.

* Layout change at the 32 GiB tensor limit (2^31 - 8192 words of 16 bytes;
  B = 1, P = 8, H = 64, d_h = 128, L = 2^21 - 8, bf16 random bit patterns):
  every element of seq_to_head against the oracle's row map (the oracle's
  index arithmetic, applied with a device gather), and head_to_seq of the
  result back to the input bit for bit.
* The K/V layout change at the same limit on its head side (each of 2 K/V
  heads replicated on 4 of 8 ranks, L = 2^24 - 8): every element against
  the oracle's row map, and its gradient form (the 4 replicas summed back
  into their token shards) on every element within the rounding bound of an
  fp32 sum of 4 terms and one bf16 rounding.
* Attention at the 32-bit byte-offset limit of one batch entry's rows
  ((Lk + 256) * H_kv * d_h * 2 bytes just below 2^32): 256 queries against
  1,048,319 keys (a ragged last key tile) on 16 heads, bidirectional, forward
  and backward; every element of O, LSE, dQ, dK and dV of the first and the
  last head (whose rows sit at the highest offsets) against the fp64 oracle.
* Block layouts at the backward's pair-list limit: G query heads per K/V
  head times nb query blocks = 8192 listed (query head, query block) pairs
  in the two global key-block columns (G = 8 at 131,072 tokens; G = 1 at
  1,048,576 tokens, where query block indices reach 8191), whose chunks take
  all 512 partial-sum slots; sampled rows and key columns (the global
  blocks', a window block's, the last block's) against the fp64 oracle. A
  global column's dK and dV sum up to a million products, each carrying the
  rounding of P or dS to bf16 before the MFMAs: their elementwise bar adds
  2^-8 of the oracle's absolute sums of those products (the bound on that
  rounding), as the random-shape sweep does.
"""
import gc

import numpy as np
import pytest

import exact_attention_ulysses_amd as U
import oracle

from workloads import block_layout, custom

from gpu_common import LSE_ABS, check_close, host_parallel, shared_head_allowed, to_f64, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    U.lib()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _random_bits(shape, seed):
    """bf16 tensor of uniformly random 16-bit patterns (NaN and Inf patterns included), drawn per leading index."""
    torch = torch_mod()
    out = torch.empty(shape, dtype=torch.int16, device="cuda")
    g = torch.Generator(device="cuda")
    for i in range(shape[0]):
        g.manual_seed(seed + i)
        out[i].random_(-32768, 32768, generator=g)
    return out.view(torch.bfloat16)


def test_layout_change_at_the_tensor_size_limit():
    torch = torch_mod()
    B, P, H, d = 1, 8, 64, 128
    L = (1 << 21) - 8
    words = B * L * H * d * 2 // 16
    assert words == (1 << 31) - 8192   # the library's bound is 2^31 words per tensor
    Hp, Lp = H // P, L // P
    print(f"[limits] layout change L={L} H={H} P={P}: {words * 16 / 2**30:.3f} GiB", flush=True)
    x = _random_bits((P, B, Lp, H, d), 900)
    y = torch.empty((P, B, L, Hp, d), dtype=torch.bfloat16, device="cuda")
    U.ulysses_seq_to_head(x, y, B, L, H, d, P)
    # the oracle's map: destination row -> source row, applied by a plain gather
    rows = torch.from_numpy(oracle.seq_to_head_source_rows(B, L, H, P)).to("cuda")
    want = x.view(torch.int16).view(-1, d).index_select(0, rows)
    del rows
    assert torch.equal(want, y.view(torch.int16).view(-1, d)), "seq_to_head differs from the oracle's row map"
    # head_to_seq brings every bit back (into the gather's buffer)
    back = want.view(torch.bfloat16).view(P, B, Lp, H, d)
    U.ulysses_head_to_seq(y, back, B, L, H, d, P)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), x.view(torch.int16)), "head_to_seq(seq_to_head(x)) != x"
    del x, y, want, back
    gc.collect()
    torch.cuda.empty_cache()


def test_kv_layout_change_at_the_tensor_size_limit():
    torch = torch_mod()
    B, P, Hkv, d = 1, 8, 2, 128
    R = P // Hkv
    L = (1 << 24) - 8
    head_words = P * B * L * d * 2 // 16
    assert head_words == (1 << 31) - 1024   # the head side is R times the seq side
    Lp = L // P
    print(f"[limits] K/V layout change L={L} Hkv={Hkv} P={P}: head side {head_words * 16 / 2**30:.3f} GiB", flush=True)
    x = _random_bits((P, B, Lp, Hkv, d), 700)
    y = torch.empty((P, B, L, 1, d), dtype=torch.bfloat16, device="cuda")
    U.ulysses_seq_to_head_kv(x, y, B, L, Hkv, d, P)
    torch.cuda.synchronize()
    rows = torch.from_numpy(oracle.seq_to_head_kv_source_rows(B, L, Hkv, P)).to("cuda")
    xr, yr = x.view(torch.int16).view(-1, d), y.view(torch.int16).view(-1, d)
    step = 1 << 24
    for c0 in range(0, rows.numel(), step):
        assert torch.equal(xr.index_select(0, rows[c0:c0 + step]), yr[c0:c0 + step]), f"rows from {c0}"
    del x, y, rows, xr, yr
    gc.collect()
    torch.cuda.empty_cache()
    # the gradient form: dY random normal in the head layout, summed back over the replicas
    g = torch.Generator(device="cuda")
    dy = torch.empty((P, B, L, 1, d), dtype=torch.bfloat16, device="cuda")
    for p in range(P):
        g.manual_seed(710 + p)
        dy[p].copy_(torch.randn((B, L, 1, d), generator=g, device="cuda", dtype=torch.float32))
    out = torch.empty((P, B, Lp, Hkv, d), dtype=torch.bfloat16, device="cuda")
    U.ulysses_head_to_seq_kv_grad(dy, out, B, L, Hkv, d, P)
    torch.cuda.synchronize()
    grows = torch.from_numpy(oracle.head_to_seq_kv_grad_source_rows(B, L, Hkv, P)).to("cuda")
    assert grows.shape[0] == R
    dyr, outr = dy.view(-1, d), out.view(-1, d)
    worst = 0.0
    step = 1 << 22   # rows per fp64 check (4 GiB per operand)
    for c0 in range(0, grows.shape[1], step):
        parts = [dyr.index_select(0, grows[j, c0:c0 + step]).double() for j in range(R)]
        want = sum(parts)
        err = (R - 1) * 2.0 ** -24 * sum(t.abs() for t in parts)   # fp32 sum of R terms
        _, e = torch.frexp(want.abs() + err)
        bar = 0.5 * torch.ldexp(torch.ones_like(want), e - 8) + err   # one bf16 rounding of the sum
        ratio = ((outr[c0:c0 + step].double() - want).abs() / bar).max().item()
        worst = max(worst, ratio)
        assert ratio <= 1.0, f"rows from {c0}: {ratio}"
        del parts, want, err, e, bar
    print(f"[limits] K/V gradient form: worst error {worst:.3f} of the bound", flush=True)
    del dy, out, grows, dyr, outr
    gc.collect()
    torch.cuda.empty_cache()


def test_attention_at_the_row_offset_limit():
    torch = torch_mod()
    B, Lq, H, d, P = 1, 256, 16, 128, 1
    Lk = (1 << 32) // (H * d * 2) - 256 - 1      # (Lk + 256) rows of one batch entry just below 2^32 bytes
    assert (Lk + 256) * H * d * 2 < (1 << 32) <= (Lk + 257) * H * d * 2 and Lk % 64 != 0
    print(f"[limits] attention Lq={Lq} Lk={Lk} H={H}: K, V {Lk * H * d * 2 / 2**30:.3f} GiB each", flush=True)
    g = torch.Generator(device="cuda")

    def draw(shape, seed, scale):
        g.manual_seed(seed)
        return (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * scale).to(torch.bfloat16)

    q = draw((B, Lq, H, d), 11, 1.0)
    do = draw((B, Lq, H, d), 14, 1.0)
    k = torch.empty((B, Lk, H, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    for t, seed in ((k, 12), (v, 13)):   # in slabs, to bound the fp32 temporaries
        for h0 in range(0, H, 4):
            t[:, :, h0:h0 + 4].copy_(draw((B, Lk, 4, d), seed * 100 + h0, 1.0))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd_gqa(q, k, v, o, lse, B, Lq, Lk, H, H, d, P, False)
    dq = torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(U.ulysses_attn_bwd_gqa_workspace_bytes(B, Lq, Lk, H, H, d, P, False), dtype=torch.uint8,
                     device="cuda")
    U.ulysses_attn_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, ws, B, Lq, Lk, H, H, d, P, False)
    torch.cuda.synchronize()
    print("[limits] attention device pass done", flush=True)
    for h in (0, H - 1):
        qh, kh, vh, doh = (to_f64(t[0, :, h].contiguous(), "bf16") for t in (q, k, v, do))
        dq_r, dk_r, dv_r, o_r, lse_r, _ = oracle.attn_bwd_head(qh, kh, vh, doh, False)
        del qh, kh, vh, doh
        check_close(f"O head {h}", to_f64(o[0, :, h].contiguous(), "bf16"), o_r, "bf16")
        assert np.max(np.abs(lse[0, h].cpu().numpy() - lse_r)) <= LSE_ABS["bf16"]
        check_close(f"dQ head {h}", to_f64(dq[0, :, h].contiguous(), "bf16"), dq_r, "bf16")
        check_close(f"dK head {h}", to_f64(dk[0, :, h].contiguous(), "bf16"), dk_r, "bf16")
        check_close(f"dV head {h}", to_f64(dv[0, :, h].contiguous(), "bf16"), dv_r, "bf16")
        del dq_r, dk_r, dv_r, o_r, lse_r
        gc.collect()
        print(f"[limits] head {h} checked", flush=True)
    del q, k, v, do, o, lse, dq, dk, dv, ws
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("L,Hq", [(131072, 8), (1 << 20, 1)])
def test_block_layout_at_the_pair_list_limit(L, Hq):
    torch = torch_mod()
    B, Hkv, d, P, block = 1, 1, 128, 1, U.SPARSE_BLOCK
    nb, G = L // block, Hq // Hkv
    assert G * nb == 8192   # the most (query head, query block) pairs a key block's list holds
    print(f"[limits] block layout L={L} G={G}: {G * nb} pairs per global column", flush=True)
    lay = block_layout(custom(B, L, Hq, d, 1, causal=True, index=950 + Hq, block=block, window=2, n_global=2,
                              n_random=1))
    g = torch.Generator(device="cuda")

    def draw(shape, seed):
        g.manual_seed(seed)
        return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)

    q, do = draw((B, L, Hq, d), 21), draw((B, L, Hq, d), 24)
    k, v = draw((B, L, Hkv, d), 22), draw((B, L, Hkv, d), 23)
    layout = torch.from_numpy(lay).to("cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd_block_sparse(q, k, v, o, lse, layout, B, L, Hq, Hkv, d, P, True)
    dq = torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(U.ulysses_attn_bwd_block_sparse_workspace_bytes(B, L, Hq, Hkv, d, P, True), dtype=torch.uint8,
                     device="cuda")
    U.ulysses_attn_bwd_block_sparse(q, k, v, o, do, lse, dq, dk, dv, layout, ws, B, L, Hq, Hkv, d, P, True)
    torch.cuda.synchronize()
    print("[limits] block layout device pass done", flush=True)
    kf, vf = (to_f64(t[0, :, 0].contiguous(), "bf16") for t in (k, v))
    qf = {h: to_f64(q[0, :, h].contiguous(), "bf16") for h in range(Hq)}
    dof = {h: to_f64(do[0, :, h].contiguous(), "bf16") for h in range(Hq)}
    rows = [0, 1, 127, 128, 129, L // 2, L - 129, L - 128, L - 1]
    for h in sorted({0, Hq - 1}):
        r = oracle.attn_rows_block_sparse(qf[h], kf, vf, rows, lay[h], block, True, do=dof[h])
        check_close(f"O rows head {h}", to_f64(o[0, rows, h], "bf16"), r["o"], "bf16", fro=False)
        check_close(f"dQ rows head {h}", to_f64(dq[0, rows, h], "bf16"), r["dq"], "bf16", fro=False)
        assert np.max(np.abs(lse[0, h, rows].cpu().numpy() - r["lse"])) <= LSE_ABS["bf16"]
    # key columns of the two global blocks, a middle block and the last block;
    # the K/V head's gradient sums its G query heads' columns
    cols = [0, 1, 127, 128, 255, L // 2 + 3, L - 128, L - 1]
    # (head, range of query blocks) work items on the host's cores; a head's ranges add up
    ranges = [(h, (nb * j // 16, nb * (j + 1) // 16)) for h in range(Hq) for j in range(16)]
    got_parts = host_parallel(lambda it: oracle.attn_dkv_cols_block_sparse(qf[it[0]], kf, vf, dof[it[0]], cols,
                                                                           lay[it[0]], block, True,
                                                                           row_blocks=it[1], abs_sums=True)[1:],
                              ranges)
    parts = [[sum(p[i] for (h2, _), p in zip(ranges, got_parts) if h2 == h) for i in range(4)] for h in range(Hq)]
    # the global columns sum a million products each: their bar adds the bound
    # on rounding dS and P to bf16 before the products, 2^-8 of the absolute sums
    for name, got, i in (("dK", dk, 0), ("dV", dv, 1)):
        stack = np.stack([p[i] for p in parts])
        want = stack.sum(axis=0)
        abs_sum = sum(p[i + 2] for p in parts)
        allowed = shared_head_allowed(stack, want, "bf16") if G > 1 else None
        check_close(f"{name} columns", to_f64(got[0, cols, 0], "bf16"), want, "bf16", fro=False, allowed=allowed,
                    abs_sum=abs_sum)
    del q, k, v, do, o, lse, dq, dk, dv, ws, layout
    gc.collect()
    torch.cuda.empty_cache()
