"""Seeded synthetic inputs for the Ulysses per-rank hot path.

This module holds workload shapes and random draws only. It holds none of the
method's arithmetic: no permutation, no attention, no gradient. Both sides of a
parity check take their inputs from here -- the fp64 CPU oracle (``oracle/``)
and the HIP library -- so that they consume identical bits.

Shapes follow the token-sharded layout of "Ulysses Sequence Parallelism: A
Temporary Change of Layout" (pinyu.ai, section "One attention block, end to
end"): every rank holds ``[B, L/P, H, d_h]``. On one GPU the P virtual ranks
sit rank-major in one buffer ``[P, B, L/P, H, d_h]``.

The pages train on "synthesized training data" (paper-graph summary of arXiv
2309.14509, section 5) and name no dataset; the sequence lengths below are the
ones the pages measure at (Fig 3's 32K and ~1M points, Table 2/3's 131,072 and
262,144 tokens), the head shapes are GPT-like.

Draws:
  * bf16 tensors are drawn in float32 and rounded to bf16 with round-to-nearest-
    even; the raw uint16 patterns are what both sides see.
  * host draws use numpy's PCG64 from ``SeedSequence(ROOT_SEED, spawn_key=...)``,
    chunked along the rank axis so big tensors can be drawn piecewise;
  * device draws (large workloads) use torch's seeded generator on the GPU;
    the oracle then reads the same bits back from device memory.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

ROOT_SEED = 230914509

# tensor identities used in spawn keys (stable numbering; never reorder)
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3, "fill_o": 4, "fill_dq": 5,
              "fill_dk": 6, "fill_dv": 7, "stress": 8, "layout": 9}


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    index: int          # stable id used in spawn keys
    B: int
    L: int
    H: int
    d: int
    P: int
    dtype: str          # "fp32" or "bf16"
    backward: bool
    causal: bool = True
    qk_scale: float = 0.5     # Q, K ~ qk_scale * N(0,1)
    v_dist: str = "normal"    # "normal" (v_scale*N(0,1)) or "uniform" (U(-1,1))
    v_scale: float = 0.5
    stress_rows: bool = False  # one seeded token row per head of Q and of K scaled by 8
    attn_all_ranks: bool = False  # True: attention on every virtual rank's head group
    Lkv: int = 0        # key/value tokens when they differ from L (cross-attention); 0 = L
    Hkv: int = 0        # key/value heads when fewer than H (grouped-query attention); 0 = H
    block: int = 0      # block-sparse attention: tokens per layout block (0 = dense)
    window: int = 0     # ... each query block sees its `window` latest key blocks (itself included),
    n_global: int = 0   # ... the first `n_global` key blocks,
    n_random: int = 0   # ... and `n_random` further earlier blocks drawn per (head, block row)
    doc: str = ""

    @property
    def Lk(self) -> int:
        return self.Lkv or self.L

    @property
    def Hk(self) -> int:
        return self.Hkv or self.H

    @property
    def Hkp(self) -> int:
        """K/V heads a rank holds after the layout change (1 when replicated)."""
        return self.Hk // self.P if self.Hk % self.P == 0 else 1

    @property
    def Hp(self) -> int:
        return self.H // self.P

    @property
    def Lp(self) -> int:
        return self.L // self.P

    @property
    def seq_shape(self) -> Tuple[int, ...]:
        return (self.P, self.B, self.Lp, self.H, self.d)

    @property
    def head_shape(self) -> Tuple[int, ...]:
        return (self.P, self.B, self.L, self.Hp, self.d)

    def shape_of(self, name: str) -> Tuple[int, ...]:
        """Seq-layout shape of a drawn tensor (head layout for filler)."""
        kv = name in ("k", "v", "fill_dk", "fill_dv")
        L, H = (self.Lk, self.Hk) if kv else (self.L, self.H)
        if name.startswith("fill_"):
            return (self.P, self.B, L, self.Hkp if kv else self.Hp, self.d)
        return (self.P, self.B, L // self.P, H, self.d)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    @property
    def tensor_bytes(self) -> int:
        return self.B * self.L * self.H * self.d * self.elem_bytes


WORKLOADS = {
    w.key: w for w in [
        Workload("tiny-fp32-L256", 0, B=1, L=256, H=8, d=64, P=4, dtype="fp32",
                 backward=False, qk_scale=1.0, v_scale=1.0, attn_all_ranks=True,
                 doc="tiny fp32 case, all 4 head groups, forward only"),
        Workload("gpt1.2b-L32k-fwd", 1, B=1, L=32768, H=16, d=128, P=8, dtype="bf16",
                 backward=False, doc="GPT ~1.2B shape, 32K tokens, 2 local heads, forward"),
        Workload("gpt7b-L131k", 2, B=1, L=131072, H=32, d=128, P=8, dtype="bf16",
                 backward=True, doc="GPT 7B shape, 131,072 tokens, 4 local heads, fwd+bwd"),
        Workload("gpt30b-L262k", 3, B=1, L=262144, H=64, d=128, P=16, dtype="bf16",
                 backward=True, v_dist="uniform", stress_rows=True,
                 doc="GPT 30B shape, 262,144 tokens, 4 local heads, stress rows, fwd+bwd"),
        Workload("L1m", 4, B=1, L=1048576, H=32, d=128, P=32, dtype="bf16",
                 backward=True, doc="1,048,576 tokens, 1 local head, fwd+bwd"),
        Workload("gqa8-L131k", 5, B=1, L=131072, H=32, Hkv=8, d=128, P=8, dtype="bf16",
                 backward=True, doc="grouped-query attention with 8 K/V heads (LLaMA-3-8B shape) at "
                                    "the largest pure Ulysses degree P = 8: 4 query heads share 1 K/V head"),
        Workload("gqa2-L131k", 6, B=1, L=131072, H=32, Hkv=2, d=128, P=8, dtype="bf16",
                 backward=True, doc="2 K/V heads over P = 8: each K/V head replicated on 4 ranks"),
        Workload("cross-L16k-L131k", 7, B=1, L=16384, Lkv=131072, H=32, d=128, P=8, dtype="bf16",
                 backward=True, causal=False,
                 doc="cross-attention: 16,384 queries over 131,072 keys, bidirectional, 4 local heads"),
        Workload("bsparse-L131k", 8, B=1, L=131072, H=32, d=128, P=8, dtype="bf16", backward=True,
                 block=128, window=16, n_global=1, n_random=2,
                 doc="blocked sparse causal attention, GPT 7B shape (Figs 6-7): 128-token blocks, a window of "
                     "16 blocks, 1 global block and 2 random earlier blocks per block row and head"),
        Workload("gpt7b-L8k", 9, B=1, L=8192, H=32, d=128, P=8, dtype="bf16", backward=True,
                 doc="GPT 7B shape at a short context of 8,192 tokens, 4 local heads: launches small "
                     "enough that every attention kernel splits its walks"),
    ]
}

HEADLINE = "L1m"


def custom(B, L, H, d, P, dtype="bf16", causal=True, backward=True, index=100,
           qk_scale=0.5, v_scale=0.5, v_dist="normal", stress_rows=False, Lkv=0, Hkv=0,
           block=0, window=0, n_global=0, n_random=0) -> Workload:
    """A workload outside the named table (parity sweeps, edge cases)."""
    return Workload(f"custom-{B}x{L}x{Lkv}x{H}x{Hkv}x{d}x{P}-{dtype}", index, B=B, L=L, H=H, d=d, P=P,
                    dtype=dtype, backward=backward, causal=causal, qk_scale=qk_scale,
                    v_scale=v_scale, v_dist=v_dist, stress_rows=stress_rows, Lkv=Lkv, Hkv=Hkv,
                    block=block, window=window, n_global=n_global, n_random=n_random)


def block_layout(wl: Workload, heads=None) -> np.ndarray:
    """Block layout of a block-sparse workload: uint8 [H, nb, nb] over the global
    heads (or the listed ones), nb = ceil(L / block); entry (h, i, j) = 1 when
    query block i of head h attends key block j.

    Row i holds its `window` latest blocks i-window+1 .. i, the first `n_global`
    blocks, and `n_random` further blocks drawn without replacement from the
    earlier ones (seeded per head). Bidirectional workloads mirror the window
    (i-window+1 .. i+window-1) and draw random blocks from the whole row. The
    structure -- not the arithmetic -- of the pages' "blocked sparse attention"
    workload, whose pattern they leave open.
    """
    assert wl.block > 0
    nb = -(-wl.L // wl.block)
    heads = range(wl.H) if heads is None else heads
    out = np.zeros((len(heads), nb, nb), dtype=np.uint8)
    for n, h in enumerate(heads):
        rng = np.random.Generator(np.random.PCG64(_seed_seq(wl, "layout", h)))
        for i in range(nb):
            lo = max(0, i - wl.window + 1)
            hi = i + 1 if wl.causal else min(nb, i + wl.window)
            out[n, i, lo:hi] = 1
            out[n, i, :min(wl.n_global, nb)] = 1
            pool = np.flatnonzero(out[n, i, :(i + 1 if wl.causal else nb)] == 0)
            if wl.n_random and pool.size:
                pick = rng.choice(pool, size=min(wl.n_random, pool.size), replace=False)
                out[n, i, pick] = 1
    return out


# ---------------------------------------------------------------------------
# bf16 encoding of generated values (input preparation, not the method)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even) and return uint16 bits.

    NaN inputs are not produced by the generators; they are not handled here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def _seed_seq(wl: Workload, name: str, *extra: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(ROOT_SEED, spawn_key=(wl.index, TENSOR_IDS[name]) + tuple(extra))


def stress_positions(wl: Workload, name: str) -> Optional[np.ndarray]:
    """Global token index t(h) of the stressed row of each global head, or None.

    One seeded row per head in each of Q and K (independent draws).
    """
    if not wl.stress_rows or name not in ("q", "k"):
        return None
    rng = np.random.Generator(np.random.PCG64(_seed_seq(wl, "stress", TENSOR_IDS[name])))
    P, B, Lp, H, _ = wl.shape_of(name)
    return rng.integers(0, P * Lp, size=(B, H), dtype=np.int64)


def _dist(wl: Workload, name: str) -> Tuple[str, float]:
    if name in ("q", "k"):
        return "normal", wl.qk_scale
    if name == "v":
        return (wl.v_dist, wl.v_scale)
    return "normal", 1.0  # dO and filler ~ N(0,1)


def host_tensor(wl: Workload, name: str) -> np.ndarray:
    """Draw a full seq-layout tensor ``[P, B, L/P, H, d]`` on the host.

    Returns float32 for fp32 workloads and uint16 bf16 bit patterns otherwise.
    Filler tensors (``fill_*``) have the head layout's element count and are
    returned in head layout ``[P, B, L, H/P, d]``.
    """
    shape = wl.shape_of(name)
    dist, scale = _dist(wl, name)
    out_f32 = np.empty(shape, dtype=np.float32)
    # one spawned child per leading (rank) slice, so the draw is chunkable
    for p in range(shape[0]):
        rng = np.random.Generator(np.random.PCG64(_seed_seq(wl, name, p)))
        sub = shape[1:]
        if dist == "normal":
            out_f32[p] = rng.standard_normal(sub, dtype=np.float32) * np.float32(scale)
        else:
            out_f32[p] = rng.uniform(-1.0, 1.0, size=sub).astype(np.float32)
    pos = stress_positions(wl, name)
    if pos is not None:
        Lp = shape[2]
        for b in range(pos.shape[0]):
            for h in range(pos.shape[1]):
                t = int(pos[b, h])
                out_f32[t // Lp, b, t % Lp, h, :] *= np.float32(8.0)
    if wl.dtype == "fp32":
        return out_f32
    return f32_to_bf16_bits(out_f32)


def device_tensor(wl: Workload, name: str, device="cuda"):
    """Draw the same kind of tensor as :func:`host_tensor` directly on a GPU.

    Uses torch's seeded device generator (Philox); the values differ from the
    host draw but are equally seeded and reproducible. Returned as a torch
    tensor of dtype bfloat16/float32 in seq layout (or head layout for filler).
    """
    import torch
    shape = wl.shape_of(name)
    dist, scale = _dist(wl, name)
    tdtype = torch.float32 if wl.dtype == "fp32" else torch.bfloat16
    out = torch.empty(shape, dtype=tdtype, device=device)
    g = torch.Generator(device=device)
    for p in range(shape[0]):
        seed = int(_seed_seq(wl, name, p).generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))
        g.manual_seed(seed)
        if dist == "normal":
            x = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32) * scale
        else:
            x = torch.rand(shape[1:], generator=g, device=device, dtype=torch.float32) * 2.0 - 1.0
        out[p].copy_(x)  # rounds to bf16 with round-to-nearest-even
        del x
    pos = stress_positions(wl, name)
    if pos is not None:
        Lp = shape[2]
        for b in range(pos.shape[0]):
            for h in range(pos.shape[1]):
                t = int(pos[b, h])
                row = out[t // Lp, b, t % Lp, h, :]
                # re-draw the stressed row in fp32 so the x8 is applied before rounding
                seed = int(_seed_seq(wl, name, 1000 + b, h).generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))
                g.manual_seed(seed)
                x = torch.randn((wl.d,), generator=g, device=device, dtype=torch.float32) * (scale * 8.0)
                row.copy_(x)
    return out
