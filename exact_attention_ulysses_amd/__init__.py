"""Python binding of libulysses, the HIP (gfx950) library of the Ulysses per-rank hot path.

Argument marshalling only: every step runs in the library's kernels. The
functions carry the C names (see include/ulysses.h) and take torch tensors
for device memory; the stream is torch's current stream unless one is given.
Before calling into the library each function checks that every tensor is a
contiguous CUDA tensor of the right dtype holding exactly the number of
elements the sizes imply, so the kernels never see a buffer smaller than
their sizes. A missing library raises at the first call: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; ULYSSES_LIB_PATH may name another build of the same library
# (kernel variants compared side by side).
LIB_PATH = os.environ.get("ULYSSES_LIB_PATH") or os.path.join(_HERE, "libulysses.so")

BF16 = 0
FP32 = 1

OK = 0
STATUS_NAMES = {0: "ULYSSES_OK", 1: "ULYSSES_INVALID_ARGUMENT", 2: "ULYSSES_NOT_DIVISIBLE",
                3: "ULYSSES_UNSUPPORTED", 4: "ULYSSES_MISALIGNED", 5: "ULYSSES_ALIASING",
                6: "ULYSSES_WORKSPACE_TOO_SMALL", 7: "ULYSSES_HIP_ERROR"}

EXPORTS = ("ulysses_seq_to_head", "ulysses_head_to_seq", "ulysses_seq_to_head_kv", "ulysses_head_to_seq_kv_grad",
           "ulysses_attn_fwd", "ulysses_attn_bwd", "ulysses_attn_bwd_workspace_bytes", "ulysses_attn_bwd_noalloc",
           "ulysses_attn_fwd_gqa", "ulysses_attn_bwd_gqa", "ulysses_attn_bwd_gqa_workspace_bytes",
           "ulysses_attn_fwd_block_sparse", "ulysses_attn_bwd_block_sparse",
           "ulysses_attn_bwd_block_sparse_workspace_bytes",
           "ulysses_status_string", "ulysses_last_hip_error")


class UlyssesError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}" + (f" ({detail})" if detail else ""))


_lib = None


def lib() -> ctypes.CDLL:
    """Load libulysses.so (built in-tree by exact_attention_ulysses_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_attention_ulysses_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, ci, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    for name in ("ulysses_seq_to_head", "ulysses_head_to_seq", "ulysses_seq_to_head_kv",
                 "ulysses_head_to_seq_kv_grad"):
        f = getattr(L, name)
        f.argtypes = [vp, vp, i64, i64, i64, i64, i64, ci, vp]
        f.restype = ci
    L.ulysses_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ci, ci, vp]
    L.ulysses_attn_fwd.restype = ci
    L.ulysses_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i64, i64, ci, ci, vp]
    L.ulysses_attn_bwd.restype = ci
    L.ulysses_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ci, ci, vp]
    L.ulysses_attn_bwd_noalloc.restype = ci
    L.ulysses_attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, ci, ci]
    L.ulysses_attn_bwd_workspace_bytes.restype = sz
    L.ulysses_attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, ci, vp]
    L.ulysses_attn_fwd_gqa.restype = ci
    L.ulysses_attn_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                       i64, i64, i64, i64, i64, i64, i64, ci, ci, vp]
    L.ulysses_attn_bwd_gqa.restype = ci
    L.ulysses_attn_bwd_gqa_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i64, ci, ci]
    L.ulysses_attn_bwd_gqa_workspace_bytes.restype = sz
    L.ulysses_attn_fwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ci, ci, vp]
    L.ulysses_attn_fwd_block_sparse.restype = ci
    L.ulysses_attn_bwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, sz,
                                                i64, i64, i64, i64, i64, i64, ci, ci, vp]
    L.ulysses_attn_bwd_block_sparse.restype = ci
    L.ulysses_attn_bwd_block_sparse_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i64, ci, ci]
    L.ulysses_attn_bwd_block_sparse_workspace_bytes.restype = sz
    L.ulysses_status_string.argtypes = [ci]
    L.ulysses_status_string.restype = ctypes.c_char_p
    L.ulysses_last_hip_error.argtypes = []
    L.ulysses_last_hip_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _dev(t, name: str, numel: int, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the sizes imply {numel}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != OK:
        detail = lib().ulysses_last_hip_error().decode() if status == 7 else ""
        raise UlyssesError(status, where, detail)


def ulysses_seq_to_head(x_seq, x_head, B: int, L: int, H: int, d_h: int, P: int, stream=None) -> None:
    """x_seq [P][B][L/P][H][d_h] -> x_head [P][B][L][H/P][d_h] (first all-to-all)."""
    n = B * L * H * d_h
    st = lib().ulysses_seq_to_head(_dev(x_seq, "x_seq", n), _dev(x_head, "x_head", n, x_seq.dtype),
                                   B, L, H, d_h, P, dtype_code(x_seq), _stream(stream))
    _check(st, "ulysses_seq_to_head")


def ulysses_head_to_seq(x_head, x_seq, B: int, L: int, H: int, d_h: int, P: int, stream=None) -> None:
    """x_head [P][B][L][H/P][d_h] -> x_seq [P][B][L/P][H][d_h] (second all-to-all)."""
    n = B * L * H * d_h
    st = lib().ulysses_head_to_seq(_dev(x_head, "x_head", n), _dev(x_seq, "x_seq", n, x_head.dtype),
                                   B, L, H, d_h, P, dtype_code(x_head), _stream(stream))
    _check(st, "ulysses_head_to_seq")


def kv_local_heads(H_kv: int, P: int) -> int:
    """K/V heads per rank after ulysses_seq_to_head_kv (0 if H_kv and P are incompatible)."""
    if H_kv % P == 0:
        return H_kv // P
    return 1 if P % H_kv == 0 else 0


def _kv_sizes(where: str, B: int, L: int, H_kv: int, d_h: int, P: int):
    hl = kv_local_heads(H_kv, P)
    if hl == 0:
        raise UlyssesError(2, where)
    return B * L * H_kv * d_h, P * B * L * hl * d_h


def ulysses_seq_to_head_kv(x_seq, x_head, B: int, L: int, H_kv: int, d_h: int, P: int, stream=None) -> None:
    """K/V x_seq [P][B][L/P][H_kv][d_h] -> x_head [P][B][L][Hl][d_h] (K/V heads replicated when P > H_kv)."""
    ns, nh = _kv_sizes("ulysses_seq_to_head_kv", B, L, H_kv, d_h, P)
    st = lib().ulysses_seq_to_head_kv(_dev(x_seq, "x_seq", ns), _dev(x_head, "x_head", nh, x_seq.dtype),
                                      B, L, H_kv, d_h, P, dtype_code(x_seq), _stream(stream))
    _check(st, "ulysses_seq_to_head_kv")


def ulysses_head_to_seq_kv_grad(dx_head, dx_seq, B: int, L: int, H_kv: int, d_h: int, P: int, stream=None) -> None:
    """Gradient of ulysses_seq_to_head_kv: dx_head [P][B][L][Hl][d_h] -> dx_seq [P][B][L/P][H_kv][d_h]."""
    ns, nh = _kv_sizes("ulysses_head_to_seq_kv_grad", B, L, H_kv, d_h, P)
    st = lib().ulysses_head_to_seq_kv_grad(_dev(dx_head, "dx_head", nh), _dev(dx_seq, "dx_seq", ns, dx_head.dtype),
                                           B, L, H_kv, d_h, P, dtype_code(dx_head), _stream(stream))
    _check(st, "ulysses_head_to_seq_kv_grad")


def _gqa_sizes(where: str, B: int, L_q: int, L_kv: int, H_q: int, H_kv: int, d_h: int, P: int):
    hl = kv_local_heads(H_kv, P)
    if H_q % P or H_q % H_kv or hl == 0:
        raise UlyssesError(2, where)
    return B * L_q * (H_q // P) * d_h, B * L_kv * hl * d_h, B * (H_q // P) * L_q


def ulysses_attn_fwd_gqa(q, k, v, o, lse, B: int, L_q: int, L_kv: int, H_q: int, H_kv: int, d_h: int, P: int,
                         causal: bool = True, stream=None) -> None:
    """Attention with H_q query heads sharing H_kv K/V heads, queries and keys of lengths L_q, L_kv:
    q, o [B][L_q][H_q/P][d_h]; k, v [B][L_kv][Hl][d_h]; lse [B][H_q/P][L_q] fp32."""
    torch = _torch()
    nq, nk, nl = _gqa_sizes("ulysses_attn_fwd_gqa", B, L_q, L_kv, H_q, H_kv, d_h, P)
    st = lib().ulysses_attn_fwd_gqa(_dev(q, "q", nq), _dev(k, "k", nk, q.dtype), _dev(v, "v", nk, q.dtype),
                                    _dev(o, "o", nq, q.dtype), _dev(lse, "lse", nl, torch.float32),
                                    B, L_q, L_kv, H_q, H_kv, d_h, P, int(bool(causal)), dtype_code(q),
                                    _stream(stream))
    _check(st, "ulysses_attn_fwd_gqa")


def ulysses_attn_bwd_gqa_workspace_bytes(B: int, L_q: int, L_kv: int, H_q: int, H_kv: int, d_h: int, P: int,
                                         causal: bool = True, dtype: int = BF16) -> int:
    return int(lib().ulysses_attn_bwd_gqa_workspace_bytes(B, L_q, L_kv, H_q, H_kv, d_h, P, int(bool(causal)),
                                                          dtype))


def ulysses_attn_bwd_gqa(q, k, v, o, d_o, lse, dq, dk, dv, workspace, B: int, L_q: int, L_kv: int, H_q: int,
                         H_kv: int, d_h: int, P: int, causal: bool = True, stream=None) -> None:
    """dQ, dK, dV of ulysses_attn_fwd_gqa (a shared K/V head gets the sum over its query heads)."""
    torch = _torch()
    nq, nk, nl = _gqa_sizes("ulysses_attn_bwd_gqa", B, L_q, L_kv, H_q, H_kv, d_h, P)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    wbytes = workspace.numel() * workspace.element_size()
    st = lib().ulysses_attn_bwd_gqa(
        _dev(q, "q", nq), _dev(k, "k", nk, q.dtype), _dev(v, "v", nk, q.dtype), _dev(o, "o", nq, q.dtype),
        _dev(d_o, "d_o", nq, q.dtype), _dev(lse, "lse", nl, torch.float32),
        _dev(dq, "dq", nq, q.dtype), _dev(dk, "dk", nk, q.dtype), _dev(dv, "dv", nk, q.dtype),
        workspace.data_ptr(), wbytes, B, L_q, L_kv, H_q, H_kv, d_h, P, int(bool(causal)), dtype_code(q),
        _stream(stream))
    _check(st, "ulysses_attn_bwd_gqa")


SPARSE_BLOCK = 128


def _layout(layout, H_q: int, P: int, L: int, block: int) -> int:
    torch = _torch()
    if block <= 0:
        raise ValueError("block must be positive")
    nb = -(-L // block)
    return _dev(layout, "layout", (H_q // P) * nb * nb, torch.uint8)


def ulysses_attn_fwd_block_sparse(q, k, v, o, lse, layout, B: int, L: int, H_q: int, H_kv: int, d_h: int, P: int,
                                  causal: bool = True, block: int = SPARSE_BLOCK, stream=None) -> None:
    """Attention restricted to the blocks a uint8 layout [H_q/P][nb][nb] marks (bf16)."""
    torch = _torch()
    nq, nk, nl = _gqa_sizes("ulysses_attn_fwd_block_sparse", B, L, L, H_q, H_kv, d_h, P)
    st = lib().ulysses_attn_fwd_block_sparse(
        _dev(q, "q", nq), _dev(k, "k", nk, q.dtype), _dev(v, "v", nk, q.dtype), _dev(o, "o", nq, q.dtype),
        _dev(lse, "lse", nl, torch.float32), _layout(layout, H_q, P, L, block), block, B, L, H_q, H_kv, d_h, P,
        int(bool(causal)), dtype_code(q), _stream(stream))
    _check(st, "ulysses_attn_fwd_block_sparse")


def ulysses_attn_bwd_block_sparse(q, k, v, o, d_o, lse, dq, dk, dv, layout, workspace, B: int, L: int, H_q: int,
                                  H_kv: int, d_h: int, P: int, causal: bool = True, block: int = SPARSE_BLOCK,
                                  stream=None) -> None:
    """dQ, dK, dV of ulysses_attn_fwd_block_sparse; workspace of ulysses_attn_bwd_block_sparse_workspace_bytes."""
    torch = _torch()
    nq, nk, nl = _gqa_sizes("ulysses_attn_bwd_block_sparse", B, L, L, H_q, H_kv, d_h, P)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    wbytes = workspace.numel() * workspace.element_size()
    st = lib().ulysses_attn_bwd_block_sparse(
        _dev(q, "q", nq), _dev(k, "k", nk, q.dtype), _dev(v, "v", nk, q.dtype), _dev(o, "o", nq, q.dtype),
        _dev(d_o, "d_o", nq, q.dtype), _dev(lse, "lse", nl, torch.float32),
        _dev(dq, "dq", nq, q.dtype), _dev(dk, "dk", nk, q.dtype), _dev(dv, "dv", nk, q.dtype),
        _layout(layout, H_q, P, L, block), block, workspace.data_ptr(), wbytes, B, L, H_q, H_kv, d_h, P,
        int(bool(causal)), dtype_code(q), _stream(stream))
    _check(st, "ulysses_attn_bwd_block_sparse")


def ulysses_attn_bwd_block_sparse_workspace_bytes(B: int, L: int, H_q: int, H_kv: int, d_h: int, P: int,
                                                  causal: bool = True, dtype: int = BF16,
                                                  block: int = SPARSE_BLOCK) -> int:
    return int(lib().ulysses_attn_bwd_block_sparse_workspace_bytes(B, L, H_q, H_kv, d_h, P, block,
                                                                   int(bool(causal)), dtype))


def ulysses_attn_fwd(q, k, v, o, lse, B: int, L: int, H: int, d_h: int, P: int, causal: bool = True,
                     stream=None) -> None:
    """O = softmax(Q K^T / sqrt(d_h)) V on one rank's head block [B][L][H/P][d_h]; lse [B][H/P][L] fp32."""
    torch = _torch()
    if H % P:
        raise UlyssesError(2, "ulysses_attn_fwd")
    n = B * L * (H // P) * d_h
    nl = B * (H // P) * L
    st = lib().ulysses_attn_fwd(_dev(q, "q", n), _dev(k, "k", n, q.dtype), _dev(v, "v", n, q.dtype),
                                _dev(o, "o", n, q.dtype), _dev(lse, "lse", nl, torch.float32),
                                B, L, H, d_h, P, int(bool(causal)), dtype_code(q), _stream(stream))
    _check(st, "ulysses_attn_fwd")


def ulysses_attn_bwd_workspace_bytes(B: int, L: int, H: int, d_h: int, P: int, causal: bool = True,
                                     dtype: int = BF16) -> int:
    return int(lib().ulysses_attn_bwd_workspace_bytes(B, L, H, d_h, P, int(bool(causal)), dtype))


def ulysses_attn_bwd(q, k, v, o, d_o, lse, dq, dk, dv, workspace, B: int, L: int, H: int, d_h: int, P: int,
                     causal: bool = True, stream=None) -> None:
    """dQ, dK, dV of the attention above; workspace is a uint8 device tensor of at least
    ulysses_attn_bwd_workspace_bytes(...) bytes."""
    torch = _torch()
    if H % P:
        raise UlyssesError(2, "ulysses_attn_bwd")
    n = B * L * (H // P) * d_h
    nl = B * (H // P) * L
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    wbytes = workspace.numel() * workspace.element_size()
    st = lib().ulysses_attn_bwd(
        _dev(q, "q", n), _dev(k, "k", n, q.dtype), _dev(v, "v", n, q.dtype), _dev(o, "o", n, q.dtype),
        _dev(d_o, "d_o", n, q.dtype), _dev(lse, "lse", nl, torch.float32),
        _dev(dq, "dq", n, q.dtype), _dev(dk, "dk", n, q.dtype), _dev(dv, "dv", n, q.dtype),
        workspace.data_ptr(), wbytes, B, L, H, d_h, P, int(bool(causal)), dtype_code(q), _stream(stream))
    _check(st, "ulysses_attn_bwd")


def ulysses_attn_bwd_noalloc(q, k, v, o, d_o, lse, dq, dk, dv, B: int, L: int, H: int, d_h: int, P: int,
                             causal: bool = True, stream=None) -> None:
    """ulysses_attn_bwd without a workspace: the library's fixed per-device scratch holds delta and
    the split walks' partial sums (no device allocation; calls on one device must not overlap)."""
    torch = _torch()
    if H % P:
        raise UlyssesError(2, "ulysses_attn_bwd_noalloc")
    n = B * L * (H // P) * d_h
    nl = B * (H // P) * L
    st = lib().ulysses_attn_bwd_noalloc(
        _dev(q, "q", n), _dev(k, "k", n, q.dtype), _dev(v, "v", n, q.dtype), _dev(o, "o", n, q.dtype),
        _dev(d_o, "d_o", n, q.dtype), _dev(lse, "lse", nl, torch.float32),
        _dev(dq, "dq", n, q.dtype), _dev(dk, "dk", n, q.dtype), _dev(dv, "dv", n, q.dtype),
        B, L, H, d_h, P, int(bool(causal)), dtype_code(q), _stream(stream))
    _check(st, "ulysses_attn_bwd_noalloc")


__all__ = ["lib", "LIB_PATH", "BF16", "FP32", "UlyssesError", "EXPORTS", "kv_local_heads", "ulysses_seq_to_head",
           "ulysses_head_to_seq", "ulysses_seq_to_head_kv", "ulysses_head_to_seq_kv_grad", "ulysses_attn_fwd",
           "ulysses_attn_bwd", "ulysses_attn_bwd_workspace_bytes", "ulysses_attn_bwd_noalloc", "ulysses_attn_fwd_gqa", "ulysses_attn_bwd_gqa",
           "ulysses_attn_bwd_gqa_workspace_bytes", "ulysses_attn_fwd_block_sparse", "ulysses_attn_bwd_block_sparse",
           "ulysses_attn_bwd_block_sparse_workspace_bytes",
           "SPARSE_BLOCK"]
