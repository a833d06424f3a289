"""Plain fp64 CPU oracle of the Ulysses per-rank hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library and imports nothing from it.

What it computes (citations name a page and the passage on it):

* seq_to_head / head_to_seq -- the two all-to-all layout changes over P ranks.
  "Ulysses Sequence Parallelism: A Temporary Change of Layout" (pinyu.ai),
  section "Use the other independent axis": every sender splits its local heads
  into P groups, every receiver gathers one group from each sender and
  concatenates the token blocks along the sequence; the shape goes
  [B, L/P, H, d_h] -> [B, L, H/P, d_h] and back (section "One attention block,
  end to end", steps 2 and 4). Rank i owns tokens [i N/P, (i+1) N/P) before
  and heads [i h/P, (i+1) h/P) after (paper-graph summary of arXiv 2309.14509,
  section 3.4.1). Implemented as index arithmetic on d_h-element rows; values
  are moved as raw bits (any dtype).

* attn_fwd -- per-head exact attention O = softmax(Q K^T / sqrt(d_h)) V over the
  full sequence, with an optional causal mask (paper-graph summary, sections
  3.4.1 and 3.4.5; pinyu.ai, section "The layout that saves memory breaks at
  attention"; papers.chlience.com reading note, section 5.1). Two-pass
  softmax per block of rows in fp64: row max, then sum of exponentials.
  The log-sum-exp of each row's scaled scores is returned alongside O.

* attn_bwd -- the exact gradient of attn_fwd (the pages train with the method
  but do not write the backward out; the reading taken is the gradient of the
  exact attention above). With P = softmax(S), S = Q K^T / sqrt(d_h):
      dV = P^T dO,  dP = dO V^T,  D_i = sum_e dO_ie O_ie,
      dS = P o (dP - D),  dQ = dS K / sqrt(d_h),  dK = dS^T Q / sqrt(d_h).

* attn_fwd_gqa / attn_bwd_gqa -- grouped-query attention: H_q query heads share
  H_kv < H_q key/value heads (pinyu.ai, section "Head-count constraints";
  paper-graph summary, section 6.4). Query head h uses KV head h div (H_q/H_kv);
  the gradient of a shared KV head is the sum over its query heads.
  seq_to_head_kv / head_to_seq_kv_grad -- the K/V layout change: the ordinary
  one when H_kv % P == 0, otherwise (P % H_kv == 0) every rank gathers the one
  KV head its query heads use, so P/H_kv consecutive ranks hold a replica of it
  (the replication the "Head-count constraints" section mentions); the
  gradient map is the adjoint of that gather (replicas summed).

* attn_fwd_block_sparse / attn_bwd_block_sparse -- attention restricted to the
  (query block, key block) pairs a per-head block layout marks, plus the
  causal mask inside them (paper-graph summary, section 3.4 and Figs 6-7 run
  "blocked sparse attention" after the same all-to-all; the pages leave the
  pattern open, so the layout is an input). A row that sees no key has zero
  output, LSE -inf and zero gradients.

* cross-attention -- attn_fwd_head / attn_bwd_head take keys of another length
  than the queries (papers.chlience.com note, section 5.4 lists cross-attention
  among the supported kinds); bidirectional only.

Readings of points the pages leave open (kept in one place):
  * causal means key j is visible to query i iff j <= i (the diagonal is kept);
    positions are global token indices after the layout change;
  * masked keys are excluded from the softmax sum (equivalent to -inf logits);
  * the scale is exactly 1/sqrt(d_h); no dropout, bias or soft-cap;
  * the virtual ranks of one GPU sit rank-major in one buffer:
    seq layout [P, B, L/P, H, d_h], head layout [P, B, L, H/P, d_h].
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

# Rows of the score matrix handled per block: bounds host memory to about
# ROW_BLOCK * L * 8 bytes per temporary.
ROW_BLOCK = 256


# ---------------------------------------------------------------------------
# decoding of the raw input bits (exact widening)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    u32 = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact value of the kernel's input bits as float64 (bf16 bits or fp32)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# the two layout changes (pinyu.ai "Use the other independent axis";
# paper-graph summary section 3.4.1)
# ---------------------------------------------------------------------------

def check_divisible(L: int, H: int, P: int) -> None:
    """The head count and the length must split evenly over P ranks
    (pinyu.ai, "Head-count constraints": H % P == 0)."""
    if P <= 0 or H % P != 0 or L % P != 0:
        raise ValueError(f"H={H} and L={L} must both be divisible by P={P}")


def seq_to_head_source_rows(B: int, L: int, H: int, P: int) -> np.ndarray:
    """For every destination row of the head layout, the source row of the seq layout.

    Rows are d_h-element vectors. Destination row (p, b, n, j) of
    [P, B, L, H/P] takes the row of sender rank r = n div (L/P), local token
    t = n mod (L/P), global head p*(H/P) + j, i.e. row (r, b, t, p*(H/P) + j)
    of [P, B, L/P, H].
    """
    check_divisible(L, H, P)
    Lp, Hp = L // P, H // P
    p = np.arange(P, dtype=np.int64)[:, None, None, None]
    b = np.arange(B, dtype=np.int64)[None, :, None, None]
    n = np.arange(L, dtype=np.int64)[None, None, :, None]
    j = np.arange(Hp, dtype=np.int64)[None, None, None, :]
    r, t = n // Lp, n % Lp
    src = ((r * B + b) * Lp + t) * H + (p * Hp + j)
    return src.reshape(-1)


def head_to_seq_source_rows(B: int, L: int, H: int, P: int) -> np.ndarray:
    """For every destination row of the seq layout, the source row of the head layout.

    Destination row (r, b, t, h) of [P, B, L/P, H] takes the row of head-group
    rank p = h div (H/P), local head j = h mod (H/P), global token
    n = r*(L/P) + t, i.e. row (p, b, n, j) of [P, B, L, H/P].
    """
    check_divisible(L, H, P)
    Lp, Hp = L // P, H // P
    r = np.arange(P, dtype=np.int64)[:, None, None, None]
    b = np.arange(B, dtype=np.int64)[None, :, None, None]
    t = np.arange(Lp, dtype=np.int64)[None, None, :, None]
    h = np.arange(H, dtype=np.int64)[None, None, None, :]
    p, j = h // Hp, h % Hp
    n = r * Lp + t
    src = ((p * B + b) * L + n) * Hp + j
    return src.reshape(-1)


def _move_rows(x: np.ndarray, rows: np.ndarray, d: int, out_shape) -> np.ndarray:
    flat = np.ascontiguousarray(x).reshape(-1, d)
    return np.take(flat, rows, axis=0).reshape(out_shape)


def seq_to_head(x: np.ndarray, B: int, L: int, H: int, d: int, P: int) -> np.ndarray:
    """[P, B, L/P, H, d] -> [P, B, L, H/P, d] (first all-to-all). Bits are moved, not values."""
    rows = seq_to_head_source_rows(B, L, H, P)
    return _move_rows(x, rows, d, (P, B, L, H // P, d))


def head_to_seq(y: np.ndarray, B: int, L: int, H: int, d: int, P: int) -> np.ndarray:
    """[P, B, L, H/P, d] -> [P, B, L/P, H, d] (second all-to-all). Bits are moved, not values."""
    rows = head_to_seq_source_rows(B, L, H, P)
    return _move_rows(y, rows, d, (P, B, L // P, H, d))


def seq_to_head_part(x: np.ndarray, B: int, L: int, H: int, d: int, P: int, p: int) -> np.ndarray:
    """Destination rank p's block [B, L, H/P, d] of seq_to_head, for bounded host memory."""
    rows = seq_to_head_source_rows(B, L, H, P).reshape(P, -1)[p]
    return _move_rows(x, rows, d, (B, L, H // P, d))


def head_to_seq_part(y: np.ndarray, B: int, L: int, H: int, d: int, P: int, r: int) -> np.ndarray:
    """Token-rank r's block [B, L/P, H, d] of head_to_seq, for bounded host memory."""
    rows = head_to_seq_source_rows(B, L, H, P).reshape(P, -1)[r]
    return _move_rows(y, rows, d, (B, L // P, H, d))


# ---------------------------------------------------------------------------
# exact attention, forward (definition written out, fp64, two-pass softmax)
# ---------------------------------------------------------------------------

def _visible_keys(i1: int, Lkv: int, causal: bool) -> int:
    return min(i1, Lkv) if causal else Lkv


def _scores(qb: np.ndarray, kk: np.ndarray, i0: int, causal: bool, scale: float) -> np.ndarray:
    """Scaled scores of a row block, masked keys set to -inf (excluded from the sum)."""
    s = (qb @ kk.T) * scale
    if causal:
        rows = np.arange(i0, i0 + qb.shape[0])[:, None]
        cols = np.arange(kk.shape[0])[None, :]
        s = np.where(cols <= rows, s, -np.inf)
    return s


def _softmax_rows(s: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Two-pass softmax: returns probabilities and the log-sum-exp of each row."""
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    return e / l, (m + np.log(l))[:, 0]


def attn_fwd_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool,
                  row_block: int = ROW_BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """One head: q [Lq, d], k, v [Lkv, d] float64 -> O [Lq, d], LSE [Lq].

    Lq != Lkv is cross-attention (bidirectional only: the pages pair the
    causal mask with self-attention).
    """
    L, d = q.shape
    Lkv = k.shape[0]
    if causal and Lkv != L:
        raise ValueError("causal attention needs Lq == Lkv")
    scale = 1.0 / math.sqrt(d)
    o = np.empty((L, d), dtype=np.float64)
    lse = np.empty((L,), dtype=np.float64)
    for i0 in range(0, L, row_block):
        i1 = min(L, i0 + row_block)
        nk = _visible_keys(i1, Lkv, causal)
        s = _scores(q[i0:i1], k[:nk], i0, causal, scale)
        p, lse[i0:i1] = _softmax_rows(s)
        o[i0:i1] = p @ v[:nk]
    return o, lse


def attn_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool = True,
             row_block: int = ROW_BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """Heads are independent: q, k, v [B, L, Hh, d] float64 -> O [B, L, Hh, d], LSE [B, Hh, L]."""
    B, L, Hh, d = q.shape
    o = np.empty_like(q, dtype=np.float64)
    lse = np.empty((B, Hh, L), dtype=np.float64)
    for b in range(B):
        for h in range(Hh):
            o[b, :, h], lse[b, h] = attn_fwd_head(q[b, :, h], k[b, :, h], v[b, :, h], causal, row_block)
    return o, lse


# ---------------------------------------------------------------------------
# exact attention, backward (explicit formula, fp64)
# ---------------------------------------------------------------------------

def attn_bwd_head(q, k, v, do, causal: bool, row_block: int = ROW_BLOCK,
                  rows: Optional[Tuple[int, int]] = None):
    """One head: the exact gradient of <dO, O> w.r.t. q, k, v (float64; q, do
    [Lq, d], k, v [Lkv, d]).

    Per row block the probabilities are formed once and used for O, D, dP,
    dS and the three products; dK and dV accumulate over the row blocks.
    Returns (dq, dk, dv, o, lse, D). With rows = (r0, r1) only query rows
    r0 <= i < r1 are processed: their dq, o, lse and D are filled (the other
    rows stay 0), and dk, dv hold those rows' terms alone, so the dk, dv of
    a partition of the rows add up to the whole.
    """
    L, d = q.shape
    Lkv = k.shape[0]
    if causal and Lkv != L:
        raise ValueError("causal attention needs Lq == Lkv")
    scale = 1.0 / math.sqrt(d)
    r0, r1 = (0, L) if rows is None else (max(0, int(rows[0])), min(L, int(rows[1])))
    dq = np.zeros((L, d))
    dk = np.zeros((Lkv, d))
    dv = np.zeros((Lkv, d))
    o = np.zeros((L, d))
    lse = np.zeros((L,))
    D = np.zeros((L,))
    for i0 in range(r0, r1, row_block):
        i1 = min(r1, i0 + row_block)
        nk = _visible_keys(i1, Lkv, causal)
        s = _scores(q[i0:i1], k[:nk], i0, causal, scale)
        p, lse[i0:i1] = _softmax_rows(s)
        ob = p @ v[:nk]
        o[i0:i1] = ob
        dob = do[i0:i1]
        Db = np.sum(dob * ob, axis=1)
        D[i0:i1] = Db
        dp = dob @ v[:nk].T
        ds = p * (dp - Db[:, None])
        dq[i0:i1] = (ds @ k[:nk]) * scale
        dk[:nk] += (ds.T @ q[i0:i1]) * scale
        dv[:nk] += p.T @ dob
    return dq, dk, dv, o, lse, D


def attn_abs_sums_head(q, k, v, do, causal: bool, row_block: int = ROW_BLOCK):
    """One head: the absolute-value sums behind each output of attn_bwd_head.

    Every output element is a sum of products whose one factor a bf16
    computation has to round (P in O = P V and dV = P^T dO, dS in dQ and
    dK): for O_ie = sum_j P_ij v_je the sum is A_ie = sum_j P_ij |v_je|, and
    likewise sum_i P_ij |dO_ie| for dV, sum_j |dS_ij| |k_je| / sqrt(d) for dQ
    and sum_i |dS_ij| |q_ie| / sqrt(d) for dK. Rounding that factor to a
    format with unit roundoff u changes the element by at most u * A (the
    standard bound for a dot product with one perturbed factor). Returns
    (a_dq, a_dk, a_dv, a_o), shaped like (dq, dk, dv, o). Test
    infrastructure: it bounds rounding, it is not part of the method.
    """
    L, d = q.shape
    Lkv = k.shape[0]
    if causal and Lkv != L:
        raise ValueError("causal attention needs Lq == Lkv")
    scale = 1.0 / math.sqrt(d)
    a_dq = np.zeros((L, d))
    a_dk = np.zeros((Lkv, d))
    a_dv = np.zeros((Lkv, d))
    a_o = np.empty((L, d))
    for i0 in range(0, L, row_block):
        i1 = min(L, i0 + row_block)
        nk = _visible_keys(i1, Lkv, causal)
        s = _scores(q[i0:i1], k[:nk], i0, causal, scale)
        p, _ = _softmax_rows(s)
        a_o[i0:i1] = p @ np.abs(v[:nk])
        dob = do[i0:i1]
        ob = p @ v[:nk]
        Db = np.sum(dob * ob, axis=1)
        ads = np.abs(p * (dob @ v[:nk].T - Db[:, None]))
        a_dq[i0:i1] = (ads @ np.abs(k[:nk])) * scale
        a_dk[:nk] += (ads.T @ np.abs(q[i0:i1])) * scale
        a_dv[:nk] += p.T @ np.abs(dob)
    return a_dq, a_dk, a_dv, a_o


def attn_bwd(q, k, v, do, causal: bool = True, row_block: int = ROW_BLOCK):
    """[B, L, Hh, d] float64 each -> (dq, dk, dv) [B, L, Hh, d], plus o, lse [B,Hh,L], D [B,Hh,L]."""
    B, L, Hh, d = q.shape
    dq = np.empty((B, L, Hh, d))
    dk = np.empty((B, L, Hh, d))
    dv = np.empty((B, L, Hh, d))
    o = np.empty((B, L, Hh, d))
    lse = np.empty((B, Hh, L))
    D = np.empty((B, Hh, L))
    for b in range(B):
        for h in range(Hh):
            r = attn_bwd_head(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], causal, row_block)
            dq[b, :, h], dk[b, :, h], dv[b, :, h], o[b, :, h], lse[b, h], D[b, h] = r
    return dq, dk, dv, o, lse, D


# ---------------------------------------------------------------------------
# grouped-query attention: fewer K/V heads than query heads
# (pinyu.ai, "Head-count constraints": GQA/MQA have fewer KV heads; a rank's
# KV heads follow its query heads, replicated when P exceeds the KV heads)
# ---------------------------------------------------------------------------

def check_gqa(Hq: int, Hkv: int) -> int:
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"query heads {Hq} must be a multiple of KV heads {Hkv}")
    return Hq // Hkv


def attn_fwd_gqa(q, k, v, causal: bool = True, row_block: int = ROW_BLOCK):
    """q [B, Lq, Hq, d], k, v [B, Lkv, Hkv, d]: query head h attends with KV head
    h div (Hq/Hkv). Returns O [B, Lq, Hq, d], LSE [B, Hq, Lq]."""
    B, Lq, Hq, d = q.shape
    G = check_gqa(Hq, k.shape[2])
    o = np.empty((B, Lq, Hq, d))
    lse = np.empty((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            o[b, :, h], lse[b, h] = attn_fwd_head(q[b, :, h], k[b, :, h // G], v[b, :, h // G], causal, row_block)
    return o, lse


def attn_bwd_gqa(q, k, v, do, causal: bool = True, row_block: int = ROW_BLOCK):
    """Gradient of attn_fwd_gqa: dQ per query head; dK, dV of a KV head are the
    sums over the query heads that share it. Returns (dq, dk, dv)."""
    B, Lq, Hq, d = q.shape
    Hkv = k.shape[2]
    G = check_gqa(Hq, Hkv)
    dq = np.empty_like(q, dtype=np.float64)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            r = attn_bwd_head(q[b, :, h], k[b, :, h // G], v[b, :, h // G], do[b, :, h], causal, row_block)
            dq[b, :, h] = r[0]
            dk[b, :, h // G] += r[1]
            dv[b, :, h // G] += r[2]
    return dq, dk, dv


def kv_replication(Hkv: int, P: int) -> int:
    """Ranks per KV head group: 1 if the KV heads split evenly over P ranks,
    P / Hkv if every rank needs one KV head replicated from a smaller set."""
    if Hkv % P == 0:
        return 1
    if P % Hkv == 0:
        return P // Hkv
    raise ValueError(f"KV heads {Hkv} and P={P}: neither divides the other")


def seq_to_head_kv(x: np.ndarray, B: int, L: int, Hkv: int, d: int, P: int) -> np.ndarray:
    """K/V layout change. Hkv % P == 0: the ordinary seq_to_head over Hkv heads.
    P % Hkv == 0: rank p receives KV head p div (P/Hkv) from every sender,
    concatenated along the sequence -> [P, B, L, 1, d]."""
    R = kv_replication(Hkv, P)
    if R == 1:
        return seq_to_head(x, B, L, Hkv, d, P)
    out = np.empty((P, B, L, 1, d), dtype=x.dtype)
    Lp = L // P
    for p in range(P):
        for r in range(P):
            out[p, :, r * Lp:(r + 1) * Lp, 0] = x[r, :, :, p // R]
    return out


def seq_to_head_kv_source_rows(B: int, L: int, Hkv: int, P: int) -> np.ndarray:
    """For every destination row of the K/V head layout, the source row of the
    seq layout (seq_to_head_kv as index arithmetic). With replication
    (R = P / Hkv ranks per KV head) destination row (p, b, n, 0) of
    [P, B, L, 1] takes row (r, b, t, p div R) of [P, B, L/P, Hkv], r = n div
    (L/P), t = n mod (L/P); without it the map is seq_to_head's."""
    R = kv_replication(Hkv, P)
    if R == 1:
        return seq_to_head_source_rows(B, L, Hkv, P)
    Lp = L // P
    p = np.arange(P, dtype=np.int64)[:, None, None]
    b = np.arange(B, dtype=np.int64)[None, :, None]
    n = np.arange(L, dtype=np.int64)[None, None, :]
    r, t = n // Lp, n % Lp
    return (((r * B + b) * Lp + t) * Hkv + p // R).reshape(-1)


def head_to_seq_kv_grad_source_rows(B: int, L: int, Hkv: int, P: int) -> np.ndarray:
    """[R, rows of the seq layout]: the R head-layout rows whose sum is each
    destination row of head_to_seq_kv_grad (R = 1: head_to_seq's map).
    Destination row (r, b, t, h) of [P, B, L/P, Hkv] sums rows
    (h R + j, b, r (L/P) + t, 0) of [P, B, L, 1], j = 0 .. R-1."""
    R = kv_replication(Hkv, P)
    if R == 1:
        return head_to_seq_source_rows(B, L, Hkv, P)[None, :]
    Lp = L // P
    r = np.arange(P, dtype=np.int64)[:, None, None, None]
    b = np.arange(B, dtype=np.int64)[None, :, None, None]
    t = np.arange(Lp, dtype=np.int64)[None, None, :, None]
    h = np.arange(Hkv, dtype=np.int64)[None, None, None, :]
    return np.stack([(((h * R + j) * B + b) * L + r * Lp + t).reshape(-1) for j in range(R)])


def head_to_seq_kv_grad(y: np.ndarray, B: int, L: int, Hkv: int, d: int, P: int) -> np.ndarray:
    """Adjoint of seq_to_head_kv for dK/dV (float64): with replication the R
    copies of a KV head are summed back into its token shards."""
    R = kv_replication(Hkv, P)
    if R == 1:
        return head_to_seq(y, B, L, Hkv, d, P)
    Lp = L // P
    out = np.zeros((P, B, Lp, Hkv, d))
    for p in range(P):
        for r in range(P):
            out[r, :, :, p // R] += y[p, :, r * Lp:(r + 1) * Lp, 0]
    return out


# ---------------------------------------------------------------------------
# block-sparse attention (paper-graph summary, section 3.4 and Figs 6-7: the
# sparse pattern is applied locally after the all-to-all; pinyu.ai: each rank
# holds the full sequence of its heads, so it can build the whole pattern)
# ---------------------------------------------------------------------------

def block_visible(layout_row: np.ndarray, block: int, i0: int, i1: int, L: int, causal: bool) -> np.ndarray:
    """Token visibility of query rows i0..i1-1 (one block row or part of one)
    under a block layout row: key j is visible to query i iff the layout marks
    (i // block, j // block), and, when causal, j <= i."""
    cols = np.arange(L)
    vis = np.repeat(np.asarray(layout_row, dtype=bool), block)[:L][None, :].repeat(i1 - i0, axis=0)
    if causal:
        rows = np.arange(i0, i1)[:, None]
        vis &= cols[None, :] <= rows
    return vis


def _masked_softmax_rows(s: np.ndarray, vis: np.ndarray):
    """Softmax over the visible entries of each row; a row with no visible key
    gets all-zero probabilities and LSE -inf."""
    s = np.where(vis, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    any_vis = np.isfinite(m)
    m = np.where(any_vis, m, 0.0)
    e = np.where(vis, np.exp(s - m), 0.0)
    l = np.sum(e, axis=1, keepdims=True)
    p = np.where(any_vis, e / np.where(any_vis, l, 1.0), 0.0)
    lse = np.where(any_vis[:, 0], (m + np.log(np.where(any_vis, l, 1.0)))[:, 0], -np.inf)
    return p, lse


def attn_fwd_block_sparse_head(q, k, v, layout, block: int, causal: bool):
    """One head: O and LSE of softmax(Q K^T / sqrt(d)) V restricted to the
    visible (query, key) pairs of the block layout [nb, nb]."""
    L, d = q.shape
    scale = 1.0 / math.sqrt(d)
    o = np.zeros((L, d))
    lse = np.empty(L)
    for bi, i0 in enumerate(range(0, L, block)):
        i1 = min(L, i0 + block)
        vis = block_visible(layout[bi], block, i0, i1, L, causal)
        s = (q[i0:i1] @ k.T) * scale
        p, lse[i0:i1] = _masked_softmax_rows(s, vis)
        o[i0:i1] = p @ v
    return o, lse


def attn_bwd_block_sparse_head(q, k, v, do, layout, block: int, causal: bool):
    """One head: exact gradient of the block-sparse attention above (the
    masked entries are constants -inf, so dS = P o (dP - D) on the visible
    pairs and 0 elsewhere). Returns (dq, dk, dv, o, lse, D)."""
    L, d = q.shape
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = np.zeros((L, d)), np.zeros((L, d)), np.zeros((L, d))
    o, lse, D = np.zeros((L, d)), np.empty(L), np.empty(L)
    for bi, i0 in enumerate(range(0, L, block)):
        i1 = min(L, i0 + block)
        vis = block_visible(layout[bi], block, i0, i1, L, causal)
        s = (q[i0:i1] @ k.T) * scale
        p, lse[i0:i1] = _masked_softmax_rows(s, vis)
        ob = p @ v
        o[i0:i1] = ob
        Db = np.sum(do[i0:i1] * ob, axis=1)
        D[i0:i1] = Db
        dp = do[i0:i1] @ v.T
        ds = p * (dp - Db[:, None])
        dv += p.T @ do[i0:i1]
        dq[i0:i1] = (ds @ k) * scale
        dk += (ds.T @ q[i0:i1]) * scale
    return dq, dk, dv, o, lse, D


def attn_abs_sums_block_sparse_head(q, k, v, do, layout, block: int, causal: bool):
    """attn_abs_sums_head under a block layout: the absolute-value sums of the
    products behind each output of attn_bwd_block_sparse_head (P for O and
    dV, dS for dQ and dK, over the visible pairs). Test infrastructure."""
    L, d = q.shape
    scale = 1.0 / math.sqrt(d)
    a_dq, a_dk, a_dv, a_o = np.zeros((L, d)), np.zeros((L, d)), np.zeros((L, d)), np.zeros((L, d))
    for bi, i0 in enumerate(range(0, L, block)):
        i1 = min(L, i0 + block)
        vis = block_visible(layout[bi], block, i0, i1, L, causal)
        s = (q[i0:i1] @ k.T) * scale
        p, _ = _masked_softmax_rows(s, vis)
        a_o[i0:i1] = p @ np.abs(v)
        ob = p @ v
        Db = np.sum(do[i0:i1] * ob, axis=1)
        ads = np.abs(p * (do[i0:i1] @ v.T - Db[:, None]))
        a_dv += p.T @ np.abs(do[i0:i1])
        a_dq[i0:i1] = (ads @ np.abs(k)) * scale
        a_dk += (ads.T @ np.abs(q[i0:i1])) * scale
    return a_dq, a_dk, a_dv, a_o


def attn_fwd_block_sparse(q, k, v, layout, block: int, causal: bool = True):
    """q, k, v [B, L, H, d] (one rank's heads); layout [H, nb, nb] shared by the
    batch. Returns O [B, L, H, d] and LSE [B, H, L]."""
    B, L, H, d = q.shape
    o = np.empty((B, L, H, d))
    lse = np.empty((B, H, L))
    for b in range(B):
        for h in range(H):
            o[b, :, h], lse[b, h] = attn_fwd_block_sparse_head(q[b, :, h], k[b, :, h], v[b, :, h], layout[h],
                                                               block, causal)
    return o, lse


def attn_bwd_block_sparse(q, k, v, do, layout, block: int, causal: bool = True):
    """Gradients (dq, dk, dv) of attn_fwd_block_sparse."""
    B, L, H, d = q.shape
    dq, dk, dv = (np.empty((B, L, H, d)) for _ in range(3))
    for b in range(B):
        for h in range(H):
            r = attn_bwd_block_sparse_head(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], layout[h], block, causal)
            dq[b, :, h], dk[b, :, h], dv[b, :, h] = r[0], r[1], r[2]
    return dq, dk, dv


def _active_keys(layout_row: np.ndarray, block: int, L: int) -> np.ndarray:
    """Token indices of the key blocks a layout row marks, ascending. Keys of
    the other blocks are invisible to the row's queries, so the softmax and
    every product over them may be formed over these keys alone."""
    act = np.nonzero(np.asarray(layout_row))[0]
    if len(act) == 0:
        return np.empty(0, dtype=np.int64)
    return np.concatenate([np.arange(jb * block, min(L, (jb + 1) * block), dtype=np.int64) for jb in act])


def attn_rows_block_sparse(q, k, v, rows, layout, block: int, causal: bool = True, do=None):
    """Forward (and with dO the dQ row) of selected query rows of one head under a
    block layout; each row is formed over the keys of its layout row's active
    blocks. Returns dict o, lse (and D, dq)."""
    L, d = k.shape
    scale = 1.0 / math.sqrt(d)
    rows = list(rows)
    out = {"o": np.zeros((len(rows), d)), "lse": np.empty(len(rows))}
    if do is not None:
        out["D"] = np.empty(len(rows))
        out["dq"] = np.zeros((len(rows), d))
    for n, i in enumerate(rows):
        keys = _active_keys(layout[i // block], block, L)
        if len(keys) == 0:   # a block row the layout leaves empty: no keys, O = 0, LSE = -inf
            out["lse"][n] = -np.inf
            if do is not None:
                out["D"][n] = 0.0
            continue
        vis = (keys <= i) if causal else np.ones(len(keys), bool)
        kk = np.asarray(k[keys], dtype=np.float64).reshape(len(keys), d)
        vv = np.asarray(v[keys], dtype=np.float64).reshape(len(keys), d)
        s = (kk @ np.asarray(q[i], dtype=np.float64)) * scale
        p, lse = _masked_softmax_rows(s[None, :], vis[None, :])
        out["lse"][n] = lse[0]
        oi = p[0] @ vv
        out["o"][n] = oi
        if do is not None:
            doi = np.asarray(do[i], dtype=np.float64)
            Di = float(doi @ oi)
            dp = vv @ doi
            out["D"][n] = Di
            out["dq"][n] = ((p[0] * (dp - Di)) @ kk) * scale
    return out


def attn_dkv_cols_block_sparse(q, k, v, do, cols, layout, block: int, causal: bool = True,
                               row_blocks: Optional[Tuple[int, int]] = None, abs_sums: bool = False):
    """dK and dV of selected key columns of one head under a block layout: only
    the block rows whose layout row reaches a selected column's block are
    formed, each over all keys of its active blocks (for its LSE and D).
    With row_blocks = (b0, b1) only the terms of query blocks b0 <= bi < b1
    are summed, so the sums of a partition of the blocks add up to the whole.
    Returns (cols, dk, dv), and with abs_sums also the sums of the absolute
    values of the products behind them (as attn_abs_sums_block_sparse_head:
    |dS| |q| for dK, P |dO| for dV). Test infrastructure."""
    L, d = k.shape
    scale = 1.0 / math.sqrt(d)
    cols = np.asarray(sorted(set(int(c) for c in cols)), dtype=np.int64)
    cblocks = np.unique(cols // block)
    dk = np.zeros((len(cols), d))
    dv = np.zeros((len(cols), d))
    a_dk = np.zeros((len(cols), d))
    a_dv = np.zeros((len(cols), d))
    vc = np.asarray(v[cols], dtype=np.float64)
    nbq = -(-L // block)
    b0, b1 = (0, nbq) if row_blocks is None else (max(0, int(row_blocks[0])), min(nbq, int(row_blocks[1])))
    for bi in range(b0, b1):
        i0 = bi * block
        i1 = min(L, i0 + block)
        if not np.any(np.asarray(layout[bi])[cblocks]) or (causal and i1 - 1 < cols.min()):
            continue
        keys = _active_keys(layout[bi], block, L)
        qb = np.asarray(q[i0:i1], dtype=np.float64)
        dob = np.asarray(do[i0:i1], dtype=np.float64)
        kk = np.asarray(k[keys], dtype=np.float64).reshape(len(keys), d)
        vv = np.asarray(v[keys], dtype=np.float64).reshape(len(keys), d)
        vis = np.ones((i1 - i0, len(keys)), bool)
        if causal:
            vis &= keys[None, :] <= np.arange(i0, i1)[:, None]
        p, _ = _masked_softmax_rows((qb @ kk.T) * scale, vis)
        Db = np.sum(dob * (p @ vv), axis=1)
        # probabilities of the selected columns (0 for a column outside the active
        # blocks; the row block marks at least one block, so keys is not empty)
        pos = np.minimum(np.searchsorted(keys, cols), len(keys) - 1)
        present = keys[pos] == cols
        pc = np.zeros((i1 - i0, len(cols)))
        pc[:, present] = p[:, pos[present]]
        dsc = pc * (dob @ vc.T - Db[:, None])
        dk += (dsc.T @ qb) * scale
        dv += pc.T @ dob
        if abs_sums:
            a_dk += (np.abs(dsc).T @ np.abs(qb)) * scale
            a_dv += pc.T @ np.abs(dob)
    if abs_sums:
        return cols, dk, dv, a_dk, a_dv
    return cols, dk, dv


# ---------------------------------------------------------------------------
# sampled evaluation for sizes where the full quadratic oracle is too slow
# ---------------------------------------------------------------------------

def attn_rows(q, k, v, rows: Sequence[int], causal: bool = True, do=None):
    """Forward (and, with dO, the dQ row) of selected query rows of one head.

    q, k, v, do: [L, d] float64 (any array supporting row slicing, e.g. a
    memory map). Each row costs O(i d). Returns dict with o [n, d], lse [n],
    and with dO also D [n] and dq [n, d].
    """
    L, d = k.shape
    scale = 1.0 / math.sqrt(d)
    rows = list(rows)
    out = {"o": np.empty((len(rows), d)), "lse": np.empty(len(rows))}
    if do is not None:
        out["D"] = np.empty(len(rows))
        out["dq"] = np.empty((len(rows), d))
    for n, i in enumerate(rows):
        nk = i + 1 if causal else L
        kk = np.asarray(k[:nk], dtype=np.float64)
        vv = np.asarray(v[:nk], dtype=np.float64)
        qi = np.asarray(q[i], dtype=np.float64)
        s = (kk @ qi) * scale
        m = np.max(s)
        e = np.exp(s - m)
        l = np.sum(e)
        p = e / l
        oi = p @ vv
        out["o"][n] = oi
        out["lse"][n] = m + math.log(l)
        if do is not None:
            doi = np.asarray(do[i], dtype=np.float64)
            Di = float(doi @ oi)
            dp = vv @ doi
            ds = p * (dp - Di)
            out["D"][n] = Di
            out["dq"][n] = (ds @ kk) * scale
    return out


def attn_dkv_cols(q, k, v, do, cols: Sequence[int], causal: bool = True,
                  row_block: int = ROW_BLOCK, rows: Optional[Tuple[int, int]] = None):
    """dK and dV of selected key columns j of one head.

    dK_j = (1/sqrt d) sum_{i sees j} dS_ij q_i and dV_j = sum_{i sees j} P_ij dO_i.
    Every row i that sees some selected column needs its own LSE_i and D_i,
    which are formed here from the full row (no value comes from elsewhere).
    Cost O(#rows-that-see-the-columns * L * d); cheap for columns near the end
    of a causal sequence. With rows = (r0, r1) only the terms of query rows
    r0 <= i < r1 are summed, so the sums of a partition of the rows add up to
    the whole (callers may form the parts concurrently).
    """
    Lk, d = k.shape
    Lq = q.shape[0]
    if causal and Lq != Lk:
        raise ValueError("causal attention needs Lq == Lkv")
    scale = 1.0 / math.sqrt(d)
    cols = np.asarray(sorted(set(int(c) for c in cols)), dtype=np.int64)
    r0, r1 = (0, Lq) if rows is None else (max(0, int(rows[0])), min(Lq, int(rows[1])))
    first_row = max(r0, int(cols.min())) if causal else r0
    dk = np.zeros((len(cols), d))
    dv = np.zeros((len(cols), d))
    kc = np.asarray(k[cols], dtype=np.float64)
    vc = np.asarray(v[cols], dtype=np.float64)
    for i0 in range(first_row, r1, row_block):
        i1 = min(r1, i0 + row_block)
        nk = _visible_keys(i1, Lk, causal)
        qb = np.asarray(q[i0:i1], dtype=np.float64)
        dob = np.asarray(do[i0:i1], dtype=np.float64)
        kk = np.asarray(k[:nk], dtype=np.float64)
        vv = np.asarray(v[:nk], dtype=np.float64)
        s = _scores(qb, kk, i0, causal, scale)
        p, _ = _softmax_rows(s)
        ob = p @ vv
        Db = np.sum(dob * ob, axis=1)
        pc = p[:, cols[cols < nk]] if causal else p[:, cols]
        sel = cols < nk if causal else np.ones(len(cols), bool)
        dpc = dob @ vc[sel].T
        dsc = pc * (dpc - Db[:, None])
        dk[sel] += (dsc.T @ qb) * scale
        dv[sel] += pc.T @ dob
    return cols, dk, dv


# ---------------------------------------------------------------------------
# the whole per-layer attention block over P virtual ranks (forward)
# ---------------------------------------------------------------------------

def ulysses_attention_fwd(q_seq, k_seq, v_seq, B, L, H, d, P, causal=True):
    """seq_to_head on Q, K, V; attention on every rank's head group; head_to_seq on O.

    Inputs float64 [P, B, L/P, H, d]; returns O in the same layout and the LSE
    of every rank [P, B, H/P, L]. (pinyu.ai, "One attention block, end to end".)
    """
    qh = seq_to_head(q_seq, B, L, H, d, P)
    kh = seq_to_head(k_seq, B, L, H, d, P)
    vh = seq_to_head(v_seq, B, L, H, d, P)
    oh = np.empty_like(qh)
    lse = np.empty((P, B, H // P, L))
    for p in range(P):
        oh[p], lse[p] = attn_fwd(qh[p], kh[p], vh[p], causal)
    return head_to_seq(oh, B, L, H, d, P), lse


def monolithic_attention_fwd(q_seq, k_seq, v_seq, B, L, H, d, P, causal=True):
    """All H heads on the whole sequence on one device, no layout change.

    The seq buffer [P, B, L/P, H, d] is viewed as the global [B, L, H, d]
    (rank r's tokens are positions r*L/P ...), attention is run per head, and
    the result is cut back into the seq buffer.
    """
    def glob(x):
        return np.ascontiguousarray(x.transpose(1, 0, 2, 3, 4)).reshape(B, L, H, d)
    o, _ = attn_fwd(glob(q_seq), glob(k_seq), glob(v_seq), causal)
    return np.ascontiguousarray(o.reshape(B, P, L // P, H, d).transpose(1, 0, 2, 3, 4))


# ---------------------------------------------------------------------------
# comparison helpers used by the parity tests
# ---------------------------------------------------------------------------

def error_stats(x: np.ndarray, ref: np.ndarray) -> Dict[str, float]:
    """max |x - ref| and ||x - ref||_F / ||ref||_F in float64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = x - ref
    nref = float(np.linalg.norm(ref.ravel()))
    return {"max_abs": float(np.max(np.abs(diff))) if diff.size else 0.0,
            "rel_fro": float(np.linalg.norm(diff.ravel()) / nref) if nref > 0 else float(np.linalg.norm(diff.ravel()))}
