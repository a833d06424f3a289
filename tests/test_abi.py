"""The C ABI: the library loads, exports every symbol include/ulysses.h declares,
and rejects bad arguments before any HIP call (so these run without a GPU).

Pointers below are fabricated addresses: validation must return its status
before anything dereferences them.
"""
import ctypes
import os
import re

import pytest

import exact_attention_ulysses_amd as U
from plans import dq_chunk_items as _dq_chunk_items

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ulysses.h")

A = 0x7F0000000000          # a 256-byte aligned fake address
GB = 1 << 30


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ulysses_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_exports():
    assert _declared_functions() == sorted(U.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = U.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = U.lib()
    for code, name in U.STATUS_NAMES.items():
        assert lib.ulysses_status_string(code).decode() == name
    assert lib.ulysses_status_string(99).decode() == "ULYSSES_UNKNOWN_STATUS"
    assert lib.ulysses_last_hip_error().decode() == ""


def s2h(src, dst, B=1, L=64, H=8, d=128, P=4, dtype=U.BF16):
    return U.lib().ulysses_seq_to_head(src, dst, B, L, H, d, P, dtype, None)


def h2s(src, dst, B=1, L=64, H=8, d=128, P=4, dtype=U.BF16):
    return U.lib().ulysses_head_to_seq(src, dst, B, L, H, d, P, dtype, None)


@pytest.mark.parametrize("fn", [s2h, h2s])
def test_permutation_validation(fn):
    assert fn(None, A + GB) == 1
    assert fn(A, None) == 1
    for bad in ({"B": 0}, {"L": -1}, {"H": 0}, {"d": 0}, {"P": 0}):
        assert fn(A, A + GB, **bad) == 1, bad
    assert fn(A, A + GB, H=6, P=4) == 2              # H % P
    assert fn(A, A + GB, L=66, P=4) == 2             # L % P
    assert fn(A, A + GB, d=96) == 3                  # head dim
    assert fn(A, A + GB, dtype=7) == 3               # dtype
    assert fn(A + 8, A + GB) == 4                    # misaligned source
    assert fn(A, A + GB + 4) == 4                    # misaligned destination
    assert fn(A, A + 16) == 5                        # overlapping buffers
    assert fn(A, A, dtype=U.FP32) == 5
    assert fn(A, A + 64 * GB, L=1 << 24, H=1024, P=4) == 3   # 32 GiB and above
    # sizes whose byte count overflows 64 bits are rejected, not wrapped
    assert fn(A, A + GB, B=1 << 30, L=1 << 30, H=1, d=64, P=1) == 3
    assert fn(A, A + GB, B=1 << 30, L=1 << 30, H=1 << 4, P=1 << 4) == 3


def fwd(q=A, k=A + GB, v=A + 2 * GB, o=A + 3 * GB, lse=A + 4 * GB, B=1, L=1024, H=8, d=128, P=4, causal=1,
        dtype=U.BF16):
    return U.lib().ulysses_attn_fwd(q, k, v, o, lse, B, L, H, d, P, causal, dtype, None)


def test_forward_validation():
    for ptr in ("q", "k", "v", "o", "lse"):
        assert fwd(**{ptr: None}) == 1, ptr
    assert fwd(L=0) == 1
    assert fwd(causal=2) == 1
    assert fwd(H=6, P=4) == 2
    assert fwd(d=32) == 3
    assert fwd(dtype=3) == 3
    assert fwd(q=A + 4) == 4
    assert fwd(o=A + 3 * GB + 8) == 4
    assert fwd(lse=A + 4 * GB + 2) == 4
    assert fwd(o=A + 1024) == 5                      # output overlaps q
    assert fwd(lse=A + 3 * GB + 64) == 5             # lse overlaps o
    assert fwd(lse=A + 2 * GB) == 5                  # lse overlaps v
    # one head's rows span 4 GiB: past the kernels' 32-bit row offsets
    assert fwd(L=1 << 20, H=16, P=1, q=A, k=A + 8 * GB, v=A + 16 * GB, o=A + 24 * GB, lse=A + 32 * GB) == 3


def bwd(ws_bytes=None, B=1, L=1024, H=8, d=128, P=4, causal=1, dtype=U.BF16, **ptrs):
    names = ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws"]
    p = {n: A + i * GB for i, n in enumerate(names)}
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = U.lib().ulysses_attn_bwd_workspace_bytes(B, L, H, d, P, causal, dtype)
    return U.lib().ulysses_attn_bwd(*[p[n] for n in names], ws_bytes, B, L, H, d, P, causal, dtype, None)


def test_backward_validation():
    for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws"):
        assert bwd(**{n: None}) == 1, n
    assert bwd(B=-2) == 1
    assert bwd(H=8, P=3) == 2
    assert bwd(d=256) == 3
    assert bwd(dk=A + 7 * GB + 2) == 4
    assert bwd(ws=A + 9 * GB + 4) == 4
    assert bwd(ws_bytes=16) == 6
    assert bwd(dq=A + 64) == 5                       # dq overlaps q
    assert bwd(dv=A + 7 * GB + 256) == 5             # dv overlaps dk
    assert bwd(ws=A + 5 * GB) == 5                   # workspace overlaps lse


def bwd_noalloc(B=1, L=1024, H=8, d=128, P=4, causal=1, dtype=U.BF16, **ptrs):
    names = ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"]
    p = {n: A + i * GB for i, n in enumerate(names)}
    p.update(ptrs)
    return U.lib().ulysses_attn_bwd_noalloc(*[p[n] for n in names], B, L, H, d, P, causal, dtype, None)


def test_backward_noalloc_validation():
    # every rejection happens before the first HIP call (the device lookup)
    for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert bwd_noalloc(**{n: None}) == 1, n
    assert bwd_noalloc(B=0) == 1
    assert bwd_noalloc(causal=3) == 1
    assert bwd_noalloc(H=8, P=3) == 2
    assert bwd_noalloc(d=96) == 3
    assert bwd_noalloc(dtype=5) == 3
    assert bwd_noalloc(dk=A + 7 * GB + 2) == 4
    assert bwd_noalloc(lse=A + 5 * GB + 2) == 4
    assert bwd_noalloc(dq=A + 64) == 5                   # dq overlaps q
    assert bwd_noalloc(dv=A + 7 * GB + 256) == 5         # dv overlaps dk
    # delta [B][H/P][L] fp32 must fit the 64 MiB scratch: 3 x 2 x 2^22 rows do not
    big = {n: A + i * 8 * GB for i, n in enumerate(["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"])}
    assert bwd_noalloc(B=3, L=1 << 22, H=4, P=2, **big) == 6


def test_workspace_size():
    lib = U.lib()
    # delta [B][H/P][L] fp32, rounded up to 256 bytes
    assert lib.ulysses_attn_bwd_workspace_bytes(1, 131072, 32, 128, 8, 1, U.BF16) == 4 * 131072 * 4
    assert lib.ulysses_attn_bwd_workspace_bytes(2, 100, 4, 64, 2, 0, U.FP32) == (2 * 2 * 100 * 4 + 255) // 256 * 256
    assert lib.ulysses_attn_bwd_workspace_bytes(1, 100, 6, 64, 4, 1, U.BF16) == 0   # invalid sizes


def _r256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("B,L,H,causal,chunked", [
    (1, 4096, 4, True, True), (1, 8192, 4, True, True), (1, 16384, 2, True, True),
    (1, 65536, 1, True, True),            # 512 blocks: four rounds of chunks
    (1, 32768, 4, True, False),           # 1024 blocks: whole walks
    (1, 131072, 4, True, False),
    (1, 4096, 8, True, False),            # 256 blocks: two wave groups per block rank better
    (1, 16384, 1, False, True), (2, 4096, 2, False, True), (2, 1000, 3, False, False),
    (2, 3000, 3, True, True), (1, 1, 1, True, False),
])
def test_dense_workspace_holds_dq_chunks(B, L, H, causal, chunked):
    """bf16 dQ launches of few query blocks cut the blocks' key walks into
    chunks, one [128][d_h] fp32 partial-sum slot each, after delta and any
    dK/dV partial sums; the item count the library sizes its workspace for
    is the one planned above."""
    lib = U.lib()
    for d in (64, 128):
        items = _dq_chunk_items(B, L, L, H, causal)
        assert (items > 0) == chunked
        base = lib.ulysses_attn_bwd_workspace_bytes(B, L, H, d, 1, causal, U.FP32)   # delta only
        ncol = B * H * -(-L // 128)
        kv = _r256(2 * ncol * 2 * 128 * d * 4) if (ncol < 512 if causal else ncol <= 128) else 0
        want = base + kv + _r256(items * 128 * d * 4)
        assert lib.ulysses_attn_bwd_workspace_bytes(B, L, H, d, 1, causal, U.BF16) == want, (d, items)


@pytest.mark.parametrize("B,L,H,d,P,causal,split", [
    (1, 1024, 8, 128, 4, 1, True),        # 16 key-block columns
    (1, 65408, 1, 128, 1, 1, True),       # 511 columns: causal split below 512
    (1, 65536, 1, 128, 1, 1, False),      # 512 columns
    (1, 16384, 1, 64, 1, 0, True),        # 128 columns: bidirectional split up to 128
    (1, 16512, 1, 64, 1, 0, False),       # 129 columns
])
def test_dense_workspace_holds_split_partials(B, L, H, d, P, causal, split):
    """bf16 launches of few key-block columns (batch x local K/V heads x
    128-token key blocks) split each column's walk in two and need two
    [dK | dV][128][d_h] fp32 partial sums per column after delta (and the dQ
    chunks' partial sums after those)."""
    lib = U.lib()
    ncol = B * (H // P) * -(-L // 128)
    want = _r256(B * (H // P) * L * 4) + (_r256(2 * ncol * 2 * 128 * d * 4) if split else 0)
    want += _r256(_dq_chunk_items(B, L, L, H // P, causal) * 128 * d * 4)
    assert lib.ulysses_attn_bwd_workspace_bytes(B, L, H, d, P, causal, U.BF16) == want
    # fp32 never splits
    assert lib.ulysses_attn_bwd_workspace_bytes(B, L, H, d, P, causal, U.FP32) == _r256(B * (H // P) * L * 4)


def test_python_binding_rejects_mismatched_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(10)
    with pytest.raises(ValueError):
        U.ulysses_seq_to_head(x, x, 1, 8, 4, 64, 2)   # host tensors are refused before any call


def s2h_kv(src, dst, B=1, L=64, Hkv=2, d=128, P=8, dtype=U.BF16):
    return U.lib().ulysses_seq_to_head_kv(src, dst, B, L, Hkv, d, P, dtype, None)


def h2s_kv(src, dst, B=1, L=64, Hkv=2, d=128, P=8, dtype=U.BF16):
    return U.lib().ulysses_head_to_seq_kv_grad(src, dst, B, L, Hkv, d, P, dtype, None)


@pytest.mark.parametrize("fn", [s2h_kv, h2s_kv])
def test_kv_layout_validation(fn):
    assert fn(None, A + GB) == 1
    assert fn(A, A + GB, Hkv=0) == 1
    assert fn(A, A + GB, Hkv=3, P=2) == 2            # neither divides the other
    assert fn(A, A + GB, Hkv=4, P=6) == 2
    assert fn(A, A + GB, L=60, P=8) == 2             # L % P
    assert fn(A, A + GB, d=80) == 3
    assert fn(A, A + GB, dtype=5) == 3
    assert fn(A + 4, A + GB) == 4
    # the head side is R = P / Hkv = 4 times the seq side: 64*2*128*2 B seq, 4x on the head side
    seq_bytes, head_bytes = 64 * 2 * 128 * 2, 4 * 64 * 2 * 128 * 2
    if fn is s2h_kv:
        assert fn(A + seq_bytes, A) == 5             # destination [A, A+head_bytes) covers the source
    else:
        assert fn(A, A + head_bytes - 16) == 5       # source (head side) overlaps destination
    assert fn(A, A + GB, B=1 << 20, L=1 << 14, Hkv=1, P=16) == 3   # replicated head tensor past 32 GiB
    assert fn(A, A + GB, B=1 << 30, L=1 << 30, Hkv=1, d=64, P=1) == 3      # byte counts past 64 bits
    assert fn(A, A + GB, B=1 << 28, L=1 << 30, Hkv=1, P=1 << 20) == 3


def fwd_gqa(q=A, k=A + GB, v=A + 2 * GB, o=A + 3 * GB, lse=A + 4 * GB, B=1, Lq=1024, Lkv=1024, Hq=32, Hkv=8, d=128,
            P=8, causal=1, dtype=U.BF16):
    return U.lib().ulysses_attn_fwd_gqa(q, k, v, o, lse, B, Lq, Lkv, Hq, Hkv, d, P, causal, dtype, None)


def test_gqa_forward_validation():
    for ptr in ("q", "k", "v", "o", "lse"):
        assert fwd_gqa(**{ptr: None}) == 1, ptr
    assert fwd_gqa(Lkv=0) == 1
    assert fwd_gqa(Hkv=0) == 1
    assert fwd_gqa(Hq=30, Hkv=6, P=8) == 2           # Hq % P
    assert fwd_gqa(Hq=32, Hkv=6, P=8) == 2           # Hq % Hkv
    assert fwd_gqa(Hq=48, Hkv=12, P=8) == 2          # neither Hkv % P nor P % Hkv
    assert fwd_gqa(Lq=1024, Lkv=512) == 3            # causal cross-attention
    assert fwd_gqa(Lq=1024, Lkv=512, causal=0, d=96) == 3
    assert fwd_gqa(k=A + GB + 2) == 4
    # k holds Lkv * Hl * d elements: with Hl = 1 (Hkv = 8, P = 8) that is 256 KiB here
    assert fwd_gqa(o=A + GB + 4096) == 5             # o overlaps k
    assert fwd_gqa(o=A + GB + 256 * 1024 - 16) == 5  # o overlaps the last row of k
    assert fwd_gqa(lse=A + 2 * GB + 64) == 5         # lse overlaps v
    # shapes validation accepts (the workspace query runs the same checks without launching)
    ws = U.lib().ulysses_attn_bwd_gqa_workspace_bytes
    for B, Lq, Lkv, Hq, Hkv, P, causal in ((1, 1000, 3000, 32, 8, 8, 0), (2, 5, 7, 4, 1, 4, 0),
                                          (1, 64, 64, 64, 2, 16, 1), (1, 64, 64, 8, 8, 8, 1)):
        assert ws(B, Lq, Lkv, Hq, Hkv, 128, P, causal, U.BF16) > 0


def bwd_gqa(ws_bytes=None, B=1, Lq=1024, Lkv=1024, Hq=32, Hkv=2, d=128, P=8, causal=1, dtype=U.BF16, **ptrs):
    names = ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws"]
    p = {n: A + i * GB for i, n in enumerate(names)}
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = U.lib().ulysses_attn_bwd_gqa_workspace_bytes(B, Lq, Lkv, Hq, Hkv, d, P, causal, dtype)
    return U.lib().ulysses_attn_bwd_gqa(*[p[n] for n in names], ws_bytes, B, Lq, Lkv, Hq, Hkv, d, P, causal,
                                        dtype, None)


def test_gqa_backward_validation():
    for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws"):
        assert bwd_gqa(**{n: None}) == 1, n
    assert bwd_gqa(Hkv=3) == 2
    assert bwd_gqa(Lkv=100) == 3                     # causal needs equal lengths
    assert bwd_gqa(ws_bytes=64) == 6
    assert bwd_gqa(dk=A + GB + 512) == 5             # dk overlaps k
    assert bwd_gqa(dv=A + 7 * GB + 16) == 5          # dv overlaps dk
    assert bwd_gqa(ws=A + 9 * GB + 8) == 4


def test_gqa_workspace_and_reductions():
    lib = U.lib()
    # delta [B][Hq/P][Lq] fp32 only: the key side does not change the workspace
    assert lib.ulysses_attn_bwd_gqa_workspace_bytes(1, 131072, 131072, 32, 8, 128, 8, 1, U.BF16) == 4 * 131072 * 4
    assert lib.ulysses_attn_bwd_gqa_workspace_bytes(2, 100, 333, 8, 2, 64, 4, 0, U.FP32) == \
        (2 * 2 * 100 * 4 + 255) // 256 * 256
    assert lib.ulysses_attn_bwd_gqa_workspace_bytes(1, 100, 333, 8, 2, 64, 4, 1, U.BF16) == 0
    # with H_q == H_kv and L_q == L_kv the generalised entry points are the plain ones
    assert lib.ulysses_attn_bwd_gqa_workspace_bytes(1, 4096, 4096, 16, 16, 128, 4, 1, U.BF16) == \
        lib.ulysses_attn_bwd_workspace_bytes(1, 4096, 16, 128, 4, 1, U.BF16)
    assert U.kv_local_heads(8, 8) == 1 and U.kv_local_heads(16, 8) == 2
    assert U.kv_local_heads(2, 8) == 1 and U.kv_local_heads(3, 8) == 0


def fwd_bs(layout=A + 6 * GB, block=128, B=1, L=1024, Hq=32, Hkv=8, d=128, P=8, causal=1, dtype=U.BF16, **ptrs):
    p = dict(q=A, k=A + GB, v=A + 2 * GB, o=A + 3 * GB, lse=A + 4 * GB)
    p.update(ptrs)
    return U.lib().ulysses_attn_fwd_block_sparse(p["q"], p["k"], p["v"], p["o"], p["lse"], layout, block, B, L, Hq,
                                                 Hkv, d, P, causal, dtype, None)


def bwd_bs(layout=A + 12 * GB, block=128, ws_bytes=None, B=1, L=1024, Hq=32, Hkv=8, d=128, P=8, causal=1,
           dtype=U.BF16, **ptrs):
    names = ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws"]
    p = {n: A + i * GB for i, n in enumerate(names)}
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = U.lib().ulysses_attn_bwd_block_sparse_workspace_bytes(B, L, Hq, Hkv, d, P, block, causal, dtype)
    return U.lib().ulysses_attn_bwd_block_sparse(p["q"], p["k"], p["v"], p["o"], p["do"], p["lse"], p["dq"], p["dk"],
                                                 p["dv"], layout, block, p["ws"], ws_bytes, B, L, Hq, Hkv, d, P,
                                                 causal, dtype, None)


def test_block_sparse_validation():
    assert fwd_bs(layout=None) == 1
    assert bwd_bs(layout=None) == 1
    assert fwd_bs(block=64) == 3                     # 128-token blocks only
    assert bwd_bs(block=256) == 3
    assert fwd_bs(dtype=U.FP32) == 3                 # bf16 only
    assert fwd_bs(Hkv=3) == 2
    assert fwd_bs(q=None) == 1
    assert bwd_bs(ws_bytes=8) == 6
    # the dense workspace (delta only) is too small for the block-sparse plan
    dense = U.lib().ulysses_attn_bwd_gqa_workspace_bytes(1, 1024, 1024, 32, 8, 128, 8, 1, U.BF16)
    assert bwd_bs(ws_bytes=dense) == 6
    # the layout is an input: an output over it is refused (o and lse, dq and dv)
    assert fwd_bs(layout=A + 3 * GB + 256) == 5
    assert fwd_bs(layout=A + 4 * GB) == 5
    assert bwd_bs(layout=A + 6 * GB + 100) == 5
    assert bwd_bs(layout=A + 8 * GB) == 5
    # the dK/dV kernel lists at most 8192 (query head, query block) pairs per key block
    assert bwd_bs(L=1 << 20, Hq=64, Hkv=8, P=8) == 3     # 8 x 8192 pairs
    assert bwd_bs(Hq=64, Hkv=4, P=4) == 3                # 16 query heads per K/V head


def test_block_sparse_workspace_size():
    ws = U.lib().ulysses_attn_bwd_block_sparse_workspace_bytes
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731  (256-byte alignment of each part)
    for B, L, Hq, Hkv, d, P in ((1, 1024, 32, 8, 128, 8), (2, 1000, 8, 2, 64, 2), (1, 131072, 32, 32, 128, 8)):
        Hql, Hkl = Hq // P, U.kv_local_heads(Hkv, P)
        nb = -(-L // 128)
        ncol = B * Hkl * nb
        # delta, pair counts and pair lists of the layout columns (uint16, G * nb per column), plan header,
        # work items, three tables of at most 256 split columns, 512 partial-sum slots
        want = (r(B * Hql * L * 4) + r(Hkl * nb * 4) + r(Hkl * nb * (Hql // Hkl) * nb * 2) + r(16)
                + r((ncol + 512) * 16) + 3 * r(256 * 4) + 512 * 2 * 128 * d * 4)
        assert ws(B, L, Hq, Hkv, d, P, 128, 1, U.BF16) == want
        assert ws(B, L, Hq, Hkv, d, P, 128, 0, U.BF16) == want
    assert ws(1, 1024, 32, 8, 128, 8, 64, 1, U.BF16) == 0       # 128-token blocks only
    assert ws(1, 1024, 32, 8, 128, 8, 128, 1, U.FP32) == 0      # bf16 only
    assert ws(1, 1024, 64, 4, 128, 4, 128, 1, U.BF16) == 0      # 16 query heads per K/V head
    assert ws(1, 1024, 32, 3, 128, 8, 128, 1, U.BF16) == 0      # indivisible heads
