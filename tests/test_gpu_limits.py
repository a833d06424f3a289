"""GPU parity at the largest sizes the entry points accept.

* Layout change at the 32 GiB tensor limit (2^31 - 8192 words of 16 bytes;
  B = 1, P = 8, H = 64, d_h = 128, L = 2^21 - 8, bf16 random bit patterns):
  every element of seq_to_head against the oracle's row map (the oracle's
  index arithmetic, applied with a device gather), and head_to_seq of the
  result back to the input bit for bit.
* Attention at the 32-bit byte-offset limit of one batch entry's rows
  ((Lk + 256) * H_kv * d_h * 2 bytes just below 2^32): 256 queries against
  1,048,319 keys (a ragged last key tile) on 16 heads, bidirectional, forward
  and backward; every element of O, LSE, dQ, dK and dV of the first and the
  last head (whose rows sit at the highest offsets) against the fp64 oracle.
"""
import gc

import numpy as np
import pytest

import exact_attention_ulysses_amd as U
import oracle

from gpu_common import LSE_ABS, check_close, to_f64, torch_mod

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
