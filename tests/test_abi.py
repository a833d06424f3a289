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


def test_workspace_size():
    lib = U.lib()
    # delta [B][H/P][L] fp32, rounded up to 256 bytes
    assert lib.ulysses_attn_bwd_workspace_bytes(1, 131072, 32, 128, 8, 1, U.BF16) == 4 * 131072 * 4
    assert lib.ulysses_attn_bwd_workspace_bytes(2, 100, 4, 64, 2, 0, U.FP32) == (2 * 2 * 100 * 4 + 255) // 256 * 256
    assert lib.ulysses_attn_bwd_workspace_bytes(1, 100, 6, 64, 4, 1, U.BF16) == 0   # invalid sizes


def test_python_binding_rejects_mismatched_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(10)
    with pytest.raises(ValueError):
        U.ulysses_seq_to_head(x, x, 1, 8, 4, 64, 2)   # host tensors are refused before any call
