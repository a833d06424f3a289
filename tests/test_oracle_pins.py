"""Pins of the fp64 oracle to facts outside itself (no GPU needed).

Each test ties the oracle to something other than its own formulas: the
pages' procedural description of the all-to-all, a hand-drawn ownership grid
(tests/golden), closed forms, invariants of softmax attention, finite
differences, and library routines (torch's CPU attention and autograd in
float64). A plausible slip -- a swapped index, a dropped term, a wrong sign,
scale or mask edge -- breaks at least one of them.
"""
import math
import os

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, custom, f32_to_bf16_bits, host_tensor

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# the all-to-all layout changes
# ---------------------------------------------------------------------------

def _s2h_by_procedure(x, B, L, H, d, P):
    """Sender/receiver procedure of pinyu.ai "Use the other independent axis".

    Each sender splits its local heads into P groups; receiver p collects
    group p from every sender and concatenates the token blocks along the
    sequence in sender order. Written with explicit lists, no index formula.
    """
    Hp = H // P
    groups = [[x[r][:, :, g * Hp:(g + 1) * Hp, :] for g in range(P)] for r in range(P)]
    return np.stack([np.concatenate([groups[r][p] for r in range(P)], axis=1) for p in range(P)])


def _h2s_by_procedure(y, B, L, H, d, P):
    """Inverse procedure: each head-group owner cuts its full sequence into P
    token blocks; token-rank r concatenates block r of every owner along heads."""
    Lp = L // P
    blocks = [[y[p][:, r * Lp:(r + 1) * Lp] for r in range(P)] for p in range(P)]
    return np.stack([np.concatenate([blocks[p][r] for p in range(P)], axis=2) for r in range(P)])


SHAPES = [(1, 8, 4, 2, 2), (2, 12, 6, 3, 3), (3, 16, 8, 4, 4), (1, 6, 3, 5, 1), (2, 10, 10, 1, 5),
          (1, 32, 16, 2, 8)]


@pytest.mark.parametrize("B,L,H,d,P", SHAPES)
def test_s2h_h2s_match_sender_receiver_procedure(B, L, H, d, P):
    rng = np.random.default_rng(1)
    x = rng.integers(0, 2**16, size=(P, B, L // P, H, d), dtype=np.uint16)
    y = oracle.seq_to_head(x, B, L, H, d, P)
    assert y.shape == (P, B, L, H // P, d)
    np.testing.assert_array_equal(y, _s2h_by_procedure(x, B, L, H, d, P))
    z = rng.integers(0, 2**16, size=(P, B, L, H // P, d), dtype=np.uint16)
    np.testing.assert_array_equal(oracle.head_to_seq(z, B, L, H, d, P), _h2s_by_procedure(z, B, L, H, d, P))


@pytest.mark.parametrize("B,L,H,d,P", SHAPES)
def test_round_trips_and_bijection(B, L, H, d, P):
    rng = np.random.default_rng(2)
    x = rng.integers(0, 2**32, size=(P, B, L // P, H, d), dtype=np.uint32)
    y = oracle.seq_to_head(x, B, L, H, d, P)
    np.testing.assert_array_equal(oracle.head_to_seq(y, B, L, H, d, P), x)
    z = rng.integers(0, 2**32, size=(P, B, L, H // P, d), dtype=np.uint32)
    np.testing.assert_array_equal(oracle.seq_to_head(oracle.head_to_seq(z, B, L, H, d, P), B, L, H, d, P), z)
    rows = oracle.seq_to_head_source_rows(B, L, H, P)
    assert np.array_equal(np.sort(rows), np.arange(B * L * H))  # every source row used exactly once
    rows2 = oracle.head_to_seq_source_rows(B, L, H, P)
    assert np.array_equal(rows2[rows], np.arange(B * L * H))   # the two maps are inverse
    for p in range(P):  # per-rank blocks agree with the whole tensors
        np.testing.assert_array_equal(oracle.seq_to_head_part(x, B, L, H, d, P, p), y[p])
        np.testing.assert_array_equal(oracle.head_to_seq_part(z, B, L, H, d, P, p),
                                      oracle.head_to_seq(z, B, L, H, d, P)[p])


def test_one_rank_is_identity():
    x = np.arange(1 * 2 * 16 * 4 * 8, dtype=np.uint32).reshape(1, 2, 16, 4, 8)
    np.testing.assert_array_equal(oracle.seq_to_head(x, 2, 16, 4, 8, 1), x)
    np.testing.assert_array_equal(oracle.head_to_seq(x, 2, 16, 4, 8, 1), x)


def test_batch_one_seq_buffer_is_global_layout():
    # B = 1: rank-major [P, 1, L/P, H, d] is byte-identical to the global [1, L, H, d]
    B, L, H, d, P = 1, 16, 4, 2, 4
    g = np.arange(L * H * d, dtype=np.uint32).reshape(L, H, d)          # global [L, H, d]
    seq = np.stack([g[r * (L // P):(r + 1) * (L // P)] for r in range(P)])[:, None]
    assert np.array_equal(seq.reshape(-1), g.reshape(-1))
    y = oracle.seq_to_head(seq, B, L, H, d, P)
    for p in range(P):  # rank p holds all tokens of heads p*Hp..
        np.testing.assert_array_equal(y[p, 0], g[:, p * (H // P):(p + 1) * (H // P)])


def _read_grid(name):
    grids, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = line.strip("[]")
                grids[cur] = []
            else:
                grids[cur].append([int(v) for v in line.split()])
    return {k: np.array(v) for k, v in grids.items()}


def test_ownership_grid_golden():
    grids = _read_grid("ownership_L8_H4_P2.txt")
    L, H, P, B, d = 8, 4, 2, 1, 1
    # each cell carries its own (token, head) code; the seq buffer is laid out
    # by the token cut of the grid
    code = lambda t, h: 100 * t + h  # noqa: E731
    seq = np.zeros((P, B, L // P, H, d), dtype=np.int64)
    for t in range(L):
        for h in range(H):
            r = grids["token_cut"][t, h]
            seq[r, 0, t - r * (L // P), h, 0] = code(t, h)
    head = oracle.seq_to_head(seq, B, L, H, d, P)
    for t in range(L):
        for h in range(H):
            p = grids["head_cut"][t, h]
            j = h - p * (H // P)
            assert head[p, 0, t, j, 0] == code(t, h)
    np.testing.assert_array_equal(oracle.head_to_seq(head, B, L, H, d, P), seq)


def test_permutation_moves_bits_not_values():
    # NaN payloads, infinities, -0, subnormals: every bit pattern must survive
    specials = np.array([0x7FC1, 0xFFC3, 0x7F81, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x807F, 0x3F80],
                        dtype=np.uint16)
    B, L, H, d, P = 1, 8, 4, 8, 2
    x = np.resize(specials, (P, B, L // P, H, d)).astype(np.uint16)
    y = oracle.seq_to_head(x, B, L, H, d, P)
    assert sorted(y.ravel().tolist()) == sorted(x.ravel().tolist())
    np.testing.assert_array_equal(oracle.head_to_seq(y, B, L, H, d, P), x)


def test_divisibility_is_enforced():
    with pytest.raises(ValueError):
        oracle.seq_to_head_source_rows(1, 16, 6, 4)   # H % P != 0
    with pytest.raises(ValueError):
        oracle.seq_to_head_source_rows(1, 10, 4, 4)   # L % P != 0


# ---------------------------------------------------------------------------
# the bf16 encoding of inputs
# ---------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    got = oracle.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0x8000, 0x4049], np.uint16))
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 2.0 ** -133
    assert math.isinf(got[3]) and got[4] == 0.0 and math.copysign(1, got[4]) < 0
    assert got[5] == 3.140625


def test_bf16_round_to_nearest_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -1.0 - 2.0 ** -8], np.float32)
    got = oracle.bf16_bits_to_f64(f32_to_bf16_bits(x))
    np.testing.assert_array_equal(got, [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -1.0])
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    y = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-30, 30, 100000)).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(y), ref)


# ---------------------------------------------------------------------------
# attention forward
# ---------------------------------------------------------------------------

def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("causal", [True, False])
def test_zero_queries_or_keys_give_uniform_attention(causal):
    B, L, Hh, d = 2, 37, 2, 8
    v = _rand((B, L, Hh, d), 4)
    nvis = np.arange(1, L + 1) if causal else np.full(L, L)
    want = (np.cumsum(v, axis=1) / nvis[None, :, None, None]) if causal else np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
    for zero in ("q", "k"):
        q = np.zeros((B, L, Hh, d)) if zero == "q" else _rand((B, L, Hh, d), 5)
        k = np.zeros((B, L, Hh, d)) if zero == "k" else _rand((B, L, Hh, d), 6)
        o, lse = oracle.attn_fwd(q, k, v, causal, row_block=16)
        np.testing.assert_allclose(o, want, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, np.broadcast_to(np.log(nvis), lse.shape), rtol=0, atol=1e-13)


def test_causal_row_zero_is_v0():
    q, k, v = (_rand((1, 50, 3, 16), s) for s in (7, 8, 9))
    o, lse = oracle.attn_fwd(q, k, v, True)
    np.testing.assert_array_equal(o[:, 0], v[:, 0])
    np.testing.assert_allclose(lse[:, :, 0], np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]) / 4.0, rtol=1e-14)


def test_two_token_closed_form():
    # row 1 of a causal 2-token head: weights 1/(1+e^a), e^a/(1+e^a), a = (s11 - s10)
    d = 4
    q = np.array([[0.3, -0.2, 0.5, 0.1], [1.0, 2.0, -1.0, 0.5]])
    k = np.array([[0.7, 0.1, -0.4, 0.2], [-0.3, 0.9, 0.8, -1.1]])
    v = np.array([[1.0, 2.0, 3.0, 4.0], [-5.0, 6.0, -7.0, 8.0]])
    s10 = sum(q[1, e] * k[0, e] for e in range(d)) / 2.0
    s11 = sum(q[1, e] * k[1, e] for e in range(d)) / 2.0
    a = math.exp(s11 - s10)
    want = (v[0] + a * v[1]) / (1.0 + a)
    o, lse = oracle.attn_fwd_head(q, k, v, True)
    np.testing.assert_allclose(o[1], want, rtol=1e-14)
    np.testing.assert_allclose(lse[1], s10 + math.log(1.0 + a), rtol=1e-14)


def _brute_force_attention(q, k, v, causal):
    """Pure-Python loops with math.exp: softmax of scaled dot products, then the weighted sum."""
    L, d = len(q), len(q[0])
    out, lses = [], []
    for i in range(L):
        js = range(i + 1) if causal else range(len(k))
        s = [sum(q[i][e] * k[j][e] for e in range(d)) / math.sqrt(d) for j in js]
        w = [math.exp(x) for x in s]
        z = sum(w)
        out.append([sum(w[n] * v[j][e] for n, j in enumerate(js)) / z for e in range(d)])
        lses.append(math.log(z))
    return np.array(out), np.array(lses)


@pytest.mark.parametrize("causal", [True, False])
def test_forward_brute_force(causal):
    q, k, v = (_rand((13, 5), s) for s in (10, 11, 12))
    o, lse = oracle.attn_fwd_head(q, k, v, causal, row_block=4)
    bo, blse = _brute_force_attention(q.tolist(), k.tolist(), v.tolist(), causal)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, blse, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_forward_matches_torch_sdpa_fp64(causal):
    torch = pytest.importorskip("torch")
    B, L, Hh, d = 2, 300, 2, 64
    q, k, v = (_rand((B, L, Hh, d), s, 2.0) for s in (13, 14, 15))
    o, lse = oracle.attn_fwd(q, k, v, causal, row_block=64)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))  # noqa: E731
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal)
    np.testing.assert_allclose(o, ref.numpy().transpose(0, 2, 1, 3), rtol=0, atol=1e-12)
    s = torch.einsum("bhid,bhjd->bhij", t(q), t(k)) / math.sqrt(d)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-11)


def test_softmax_invariants():
    B, L, Hh, d = 1, 96, 2, 16
    q, k, v = (_rand((B, L, Hh, d), s) for s in (16, 17, 18))
    o, lse = oracle.attn_fwd(q, k, v, True, row_block=32)
    # rows sum to one: V == 1 gives O == 1
    o1, _ = oracle.attn_fwd(q, k, np.ones_like(v), True)
    np.testing.assert_allclose(o1, 1.0, rtol=0, atol=1e-14)
    # affine in V
    oa, _ = oracle.attn_fwd(q, k, 3.0 * v - 2.0, True)
    np.testing.assert_allclose(oa, 3.0 * o - 2.0, rtol=0, atol=1e-12)
    # adding one vector c to every key shifts each row's scores by a constant
    c = _rand((1, 1, Hh, d), 19)
    ok, lsek = oracle.attn_fwd(q, k + c, v, True)
    np.testing.assert_allclose(ok, o, rtol=0, atol=1e-12)
    shift = np.einsum("blhd,bhd->bhl", q, c[:, 0]) / math.sqrt(d)
    np.testing.assert_allclose(lsek, lse + shift, rtol=0, atol=1e-12)
    # causal prefix: the first L' rows do not depend on later tokens
    op, lsep = oracle.attn_fwd(q[:, :40], k[:, :40], v[:, :40], True)
    np.testing.assert_allclose(op, o[:, :40], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lsep, lse[:, :, :40], rtol=0, atol=1e-14)


def test_large_logits_stay_finite():
    # rows scaled by 8 (the stress rows of the 30B-shaped workload) give logits in the hundreds
    q = _rand((64, 128), 20, 0.5 * 8)
    k = _rand((64, 128), 21, 0.5 * 8)
    v = _rand((64, 128), 22)
    o, lse = oracle.attn_fwd_head(q, k, v, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    bo, blse = _brute_force_attention((q / 4).tolist(), (k * 4).tolist(), v.tolist(), True)
    np.testing.assert_allclose(o, bo, rtol=1e-9, atol=1e-12)


def test_pipeline_equals_monolithic():
    # "numerically identical to monolithic attention" (aifetchly blog, simulator section)
    B, L, H, d, P = 2, 64, 8, 16, 4
    q, k, v = (_rand((P, B, L // P, H, d), s) for s in (23, 24, 25))
    o_u, lse_u = oracle.ulysses_attention_fwd(q, k, v, B, L, H, d, P, True)
    o_m = oracle.monolithic_attention_fwd(q, k, v, B, L, H, d, P, True)
    np.testing.assert_array_equal(o_u, o_m)


# ---------------------------------------------------------------------------
# attention backward
# ---------------------------------------------------------------------------

def _objective(q, k, v, do, causal):
    o, _ = oracle.attn_fwd(q, k, v, causal)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [True, False])
def test_backward_finite_differences(causal):
    B, L, Hh, d = 1, 12, 1, 6
    q, k, v, do = (_rand((B, L, Hh, d), s) for s in (26, 27, 28, 29))
    dq, dk, dv, o, lse, D = oracle.attn_bwd(q, k, v, do, causal, row_block=5)
    h = 1e-5
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(grad.shape):
            args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            args[name][idx] += h
            fp = _objective(args["q"], args["k"], args["v"], do, causal)
            args[name][idx] -= 2 * h
            fm = _objective(args["q"], args["k"], args["v"], do, causal)
            num[idx] = (fp - fm) / (2 * h)
        err = np.max(np.abs(num - grad)) / np.max(np.abs(grad))
        assert err < 1e-8, (name, err)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_torch_autograd_fp64(causal):
    torch = pytest.importorskip("torch")
    B, L, Hh, d = 1, 200, 2, 32
    q, k, v, do = (_rand((B, L, Hh, d), s) for s in (30, 31, 32, 33))
    dq, dk, dv, o, lse, D = oracle.attn_bwd(q, k, v, do, causal, row_block=48)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3))).requires_grad_(True)  # noqa: E731
    tq, tk, tv = t(q), t(k), t(v)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    out.backward(torch.from_numpy(np.ascontiguousarray(do.transpose(0, 2, 1, 3))))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy().transpose(0, 2, 1, 3), rtol=0, atol=1e-11)
    np.testing.assert_allclose(o, out.detach().numpy().transpose(0, 2, 1, 3), rtol=0, atol=1e-12)


def test_backward_invariants_and_closed_forms():
    B, L, Hh, d = 1, 70, 2, 8
    q, k, v, do = (_rand((B, L, Hh, d), s) for s in (34, 35, 36, 37))
    dq, dk, dv, o, lse, D = oracle.attn_bwd(q, k, v, do, True, row_block=32)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)           # rows of dS sum to zero
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), atol=1e-12)  # rows of P sum to one
    np.testing.assert_allclose(dq[:, 0], 0.0, atol=1e-14)                   # one visible key at row 0
    np.testing.assert_allclose(D, np.einsum("blhd,blhd->bhl", do, o), atol=1e-13)
    # Q = 0: uniform weights 1/(i+1); dK = 0; dV_j = sum_{i >= j} dO_i / (i+1)
    z = np.zeros_like(q)
    dq0, dk0, dv0, *_ = oracle.attn_bwd(z, k, v, do, True)
    np.testing.assert_allclose(dk0, 0.0, atol=1e-14)
    w = do / np.arange(1, L + 1)[None, :, None, None]
    want = np.flip(np.cumsum(np.flip(w, axis=1), axis=1), axis=1)
    np.testing.assert_allclose(dv0, want, atol=1e-13)
    # linear in dO; dO = 0 gives zero gradients
    dq2, dk2, dv2, *_ = oracle.attn_bwd(q, k, v, -2.5 * do, True)
    np.testing.assert_allclose(dq2, -2.5 * dq, atol=1e-12)
    np.testing.assert_allclose(dk2, -2.5 * dk, atol=1e-12)
    np.testing.assert_allclose(dv2, -2.5 * dv, atol=1e-12)
    dqz, dkz, dvz, *_ = oracle.attn_bwd(q, k, v, np.zeros_like(do), True)
    assert not dqz.any() and not dkz.any() and not dvz.any()


@pytest.mark.parametrize("Lq,Lk,causal", [(300, 300, True), (70, 70, False), (45, 300, False)])
def test_zero_query_closed_forms(Lq, Lk, causal):
    """With Q = 0 the oracle's O, LSE, dQ, dK and dV equal the closed forms of
    tests/closed_forms.py, derived from uniform weights 1/n_i (dQ through the
    running sums of v_j k_j^T and k_j, a route the oracle never takes)."""
    from closed_forms import zero_query_attention
    Hh, d = 2, 16
    k, v = (_rand((1, Lk, Hh, d), s) for s in (41, 42))
    do = _rand((1, Lq, Hh, d), 43)
    for h in range(Hh):
        dq, dk, dv, o, lse, _ = oracle.attn_bwd_head(np.zeros((Lq, d)), k[0, :, h], v[0, :, h], do[0, :, h],
                                                     causal, row_block=64)
        r = zero_query_attention(k[0, :, h], v[0, :, h], do[0, :, h], causal, Lq, block=128)
        np.testing.assert_allclose(dk, 0.0, atol=1e-14)
        np.testing.assert_allclose(o, r["o"], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, r["lse"], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(dq, r["dq"], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv, r["dv"], rtol=1e-12, atol=1e-13)


def _round_bf16(x):
    return oracle.to_f64(f32_to_bf16_bits(np.asarray(x, np.float32)), "bf16")


@pytest.mark.parametrize("causal", [True, False])
def test_abs_sums_bound_operand_rounding(causal):
    """attn_abs_sums_head bounds the effect of rounding P (for O, dV) and dS
    (for dQ, dK) to bf16: recomputing each output with that factor rounded,
    in fp64 otherwise, moves it by at most 2^-8 * A (bf16's unit roundoff
    times the absolute sum), and A dominates the output itself."""
    L, d = 70, 16
    q, k, v, do = (_rand((L, d), s, 1.5) for s in (51, 52, 53, 54))
    dq, dk, dv, o, lse, D = oracle.attn_bwd_head(q, k, v, do, causal, row_block=32)
    a_dq, a_dk, a_dv, a_o = oracle.attn_abs_sums_head(q, k, v, do, causal, row_block=32)
    scale = 1.0 / np.sqrt(d)
    s = (q @ k.T) * scale
    if causal:
        s[np.triu_indices(L, 1)] = -np.inf
    p = np.exp(s - lse[:, None])
    ds = p * (do @ v.T - D[:, None])
    pr, dsr = _round_bf16(p), _round_bf16(ds)
    u = 2.0 ** -8
    for name, exact, emul, a in (("O", o, pr @ v, a_o), ("dV", dv, pr.T @ do, a_dv),
                                 ("dQ", dq, (dsr @ k) * scale, a_dq), ("dK", dk, (dsr.T @ q) * scale, a_dk)):
        assert np.all(np.abs(emul - exact) <= u * a + 1e-12), name
        assert np.all(np.abs(exact) <= a + 1e-12), name
        # the bound is not vacuous: rounding moves some element by a tenth of it or more
        assert np.max(np.abs(emul - exact) / (u * a + 1e-300)) > 0.1, name


def test_block_sparse_abs_sums_bound_operand_rounding():
    """The block-layout absolute sums bound the same rounding under a sparse
    layout (visibility from the layout expanded to tokens, causal inside)."""
    L, d, block = 300, 16, 128
    q, k, v, do = (_rand((L, d), s, 1.5) for s in (71, 72, 73, 74))
    lay = np.array([[1, 0, 0], [0, 1, 0], [1, 1, 1]], np.uint8)
    dq, dk, dv, o, lse, D = oracle.attn_bwd_block_sparse_head(q, k, v, do, lay, block, True)
    a_dq, a_dk, a_dv, a_o = oracle.attn_abs_sums_block_sparse_head(q, k, v, do, lay, block, True)
    vis = np.kron(lay, np.ones((block, block), np.uint8))[:L, :L].astype(bool) & np.tri(L, dtype=bool)
    s = np.where(vis, (q @ k.T) / np.sqrt(d), -np.inf)
    p = np.exp(s - lse[:, None])
    ds = p * (do @ v.T - D[:, None])
    pr, dsr = _round_bf16(p), _round_bf16(ds)
    u = 2.0 ** -8
    for name, exact, emul, a in (("O", o, pr @ v, a_o), ("dV", dv, pr.T @ do, a_dv),
                                 ("dQ", dq, (dsr @ k) / np.sqrt(d), a_dq), ("dK", dk, (dsr.T @ q) / np.sqrt(d), a_dk)):
        assert np.all(np.abs(emul - exact) <= u * a + 1e-12), name
        assert np.all(np.abs(exact) <= a + 1e-12), name


def test_abs_sums_under_a_full_layout_equal_the_dense_ones():
    """With every block of the layout set, the block-sparse absolute sums are
    the dense ones (the layout only removes pairs)."""
    L, d, block = 300, 16, 128
    q, k, v, do = (_rand((L, d), s) for s in (61, 62, 63, 64))
    nb = -(-L // block)
    full = np.ones((nb, nb), np.uint8)
    for causal in (True, False):
        dense = oracle.attn_abs_sums_head(q, k, v, do, causal)
        sparse = oracle.attn_abs_sums_block_sparse_head(q, k, v, do, full, block, causal)
        for a, b in zip(dense, sparse):
            np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# sampled evaluation agrees with the full oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [True, False])
def test_sampled_rows_and_columns(causal):
    L, d = 150, 16
    q, k, v, do = (_rand((L, d), s) for s in (38, 39, 40, 41))
    dq, dk, dv, o, lse, D = oracle.attn_bwd_head(q, k, v, do, causal, row_block=32)
    rows = [0, 1, 63, 64, 149]
    r = oracle.attn_rows(q, k, v, rows, causal, do=do)
    np.testing.assert_allclose(r["o"], o[rows], atol=1e-13)
    np.testing.assert_allclose(r["lse"], lse[rows], atol=1e-13)
    np.testing.assert_allclose(r["dq"], dq[rows], atol=1e-12)
    np.testing.assert_allclose(r["D"], D[rows], atol=1e-12)
    cols, dkc, dvc = oracle.attn_dkv_cols(q, k, v, do, [149, 0, 77, 140, 31], causal, row_block=32)
    np.testing.assert_allclose(dkc, dk[cols], atol=1e-12)
    np.testing.assert_allclose(dvc, dv[cols], atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_column_sums_split_over_row_ranges(causal):
    # the rows= restriction: a partition of the query rows sums to the whole,
    # and one row's part is that row's term P_ij (dP_ij - D_i) q_i / sqrt(d)
    # (dK) and P_ij dO_i (dV), formed here from the full oracle's LSE and D
    L, d = 150, 16
    q, k, v, do = (_rand((L, d), s) for s in (42, 43, 44, 45))
    cols = [0, 5, 63, 64, 149]
    c, dk_all, dv_all = oracle.attn_dkv_cols(q, k, v, do, cols, causal, row_block=32)
    parts = [oracle.attn_dkv_cols(q, k, v, do, cols, causal, row_block=32, rows=r)
             for r in ((0, 7), (7, 64), (64, 65), (65, 150))]
    np.testing.assert_allclose(sum(p[1] for p in parts), dk_all, atol=1e-12)
    np.testing.assert_allclose(sum(p[2] for p in parts), dv_all, atol=1e-12)
    _, _, _, _, lse, D = oracle.attn_bwd_head(q, k, v, do, causal)
    i = 64
    _, dk_i, dv_i = parts[2]
    for n, j in enumerate(c):
        if causal and j > i:
            assert not dk_i[n].any() and not dv_i[n].any()
            continue
        p_ij = math.exp(q[i] @ k[j] / math.sqrt(d) - lse[i])
        np.testing.assert_allclose(dk_i[n], p_ij * (do[i] @ v[j] - D[i]) * q[i] / math.sqrt(d), atol=1e-13)
        np.testing.assert_allclose(dv_i[n], p_ij * do[i], atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_split_over_row_ranges(causal):
    # attn_bwd_head's rows= restriction: each range fills its own rows of dq,
    # o, lse and D, and the ranges' dk, dv add up to the whole
    L, d = 150, 16
    q, k, v, do = (_rand((L, d), s) for s in (46, 47, 48, 49))
    whole = oracle.attn_bwd_head(q, k, v, do, causal, row_block=32)
    ranges = ((0, 40), (40, 41), (41, 150))
    parts = [oracle.attn_bwd_head(q, k, v, do, causal, row_block=32, rows=r) for r in ranges]
    for (r0, r1), p in zip(ranges, parts):
        for i in (0, 3, 4, 5):      # dq, o, lse, D: the range's rows only
            np.testing.assert_allclose(p[i][r0:r1], whole[i][r0:r1], atol=1e-13)
            assert not np.any(p[i][:r0]) and not np.any(p[i][r1:])
    for i in (1, 2):                # dk, dv
        np.testing.assert_allclose(sum(p[i] for p in parts), whole[i], atol=1e-12)


def test_host_parallel_matches_sequential_bit_for_bit():
    # the GPU tests form oracle parts in host threads, one BLAS thread each
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from gpu_common import causal_row_ranges, host_parallel
    L, d = 2048, 64
    heads = [[_rand((L, d), 50 + 4 * h + j) for j in range(4)] for h in range(3)]
    tasks = [(h, r) for h in range(3) for r in causal_row_ranges(L, 4)]
    assert [r for h, r in tasks if h == 0][0][0] == 0 and [r for h, r in tasks if h == 0][-1][1] == L
    res = host_parallel(lambda t: oracle.attn_bwd_head(*heads[t[0]], True, rows=t[1]), tasks)
    seq = [oracle.attn_bwd_head(*heads[h], True, rows=r) for h, r in tasks]
    for a, b in zip(res, seq):
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("Lq,Lk", [(70, 150), (150, 33)])
def test_sampled_rows_and_columns_cross_attention(Lq, Lk):
    # the sampled forms with queries and keys of different lengths (bidirectional)
    d = 16
    q, do = _rand((Lq, d), 60), _rand((Lq, d), 61)
    k, v = _rand((Lk, d), 62), _rand((Lk, d), 63)
    dq, dk, dv, o, lse, D = oracle.attn_bwd_head(q, k, v, do, False, row_block=32)
    rows = [0, 1, Lq // 2, Lq - 1]
    r = oracle.attn_rows(q, k, v, rows, False, do=do)
    np.testing.assert_allclose(r["o"], o[rows], atol=1e-13)
    np.testing.assert_allclose(r["dq"], dq[rows], atol=1e-12)
    cols, dkc, dvc = oracle.attn_dkv_cols(q, k, v, do, [0, Lk - 1, Lk // 3], False, row_block=32)
    np.testing.assert_allclose(dkc, dk[cols], atol=1e-12)
    np.testing.assert_allclose(dvc, dv[cols], atol=1e-12)


# ---------------------------------------------------------------------------
# the seeded inputs
# ---------------------------------------------------------------------------

def test_host_inputs_are_seeded_and_shaped():
    wl = WORKLOADS["tiny-fp32-L256"]
    a = host_tensor(wl, "q")
    assert a.shape == (4, 1, 64, 8, 64) and a.dtype == np.float32
    np.testing.assert_array_equal(a, host_tensor(wl, "q"))
    assert not np.array_equal(a, host_tensor(wl, "k"))
    assert abs(float(a.std()) - 1.0) < 0.02
    wl2 = custom(1, 64, 4, 16, 2, dtype="bf16", stress_rows=True)
    b = host_tensor(wl2, "q")
    assert b.dtype == np.uint16 and b.shape == (2, 1, 32, 4, 16)
    from workloads import stress_positions
    pos = stress_positions(wl2, "q")
    vals = oracle.bf16_bits_to_f64(b)
    for h in range(4):
        t = int(pos[0, h])
        row = np.abs(vals[t // 32, 0, t % 32, h]).mean()
        assert row > 4 * 0.5 * 0.5  # scaled by 8 from 0.5*N(0,1)


# ---------------------------------------------------------------------------
# grouped-query attention and cross-attention
# ---------------------------------------------------------------------------

def _bhld(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))


@pytest.mark.parametrize("Hq,Hkv,causal", [(8, 2, True), (8, 1, False), (6, 3, True), (4, 4, False)])
def test_gqa_matches_torch_sdpa_and_autograd_fp64(Hq, Hkv, causal):
    # torch's enable_gqa shares KV head h // (Hq/Hkv) with query head h, the
    # grouping of the pages' GQA/MQA (pinyu.ai, "Head-count constraints")
    torch = pytest.importorskip("torch")
    B, L, d = 2, 90, 16
    q, do = _rand((B, L, Hq, d), 40), _rand((B, L, Hq, d), 41)
    k, v = _rand((B, L, Hkv, d), 42), _rand((B, L, Hkv, d), 43)
    o, lse = oracle.attn_fwd_gqa(q, k, v, causal, row_block=32)
    dq, dk, dv = oracle.attn_bwd_gqa(q, k, v, do, causal, row_block=32)
    tq, tk, tv = (_bhld(a).requires_grad_(True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, enable_gqa=True)
    out.backward(_bhld(do))
    back = lambda t: t.detach().numpy().transpose(0, 2, 1, 3)  # noqa: E731
    np.testing.assert_allclose(o, back(out), rtol=0, atol=1e-12)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, back(ref), rtol=0, atol=1e-11)
    # the textbook reduction: GQA is MHA on K/V heads repeated G times
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
    om, lsem = oracle.attn_fwd(q, kr, vr, causal)
    np.testing.assert_allclose(o, om, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lsem, rtol=0, atol=1e-14)


@pytest.mark.parametrize("Lq,Lkv", [(37, 100), (130, 21), (1, 64)])
def test_cross_attention_matches_torch_fp64(Lq, Lkv):
    # queries and keys of different lengths (cross-attention, papers.chlience.com
    # note, section 5.4): bidirectional, every query sees every key
    torch = pytest.importorskip("torch")
    d = 24
    q, do = _rand((Lq, d), 44), _rand((Lq, d), 45)
    k, v = _rand((Lkv, d), 46), _rand((Lkv, d), 47)
    o, lse = oracle.attn_fwd_head(q, k, v, False, row_block=16)
    dq, dk, dv, o2, lse2, D = oracle.attn_bwd_head(q, k, v, do, False, row_block=16)
    tq, tk, tv = (torch.from_numpy(a).requires_grad_(True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None])[0]
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(o, out.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, torch.logsumexp(tq @ tk.T / math.sqrt(d), -1).detach().numpy(),
                               rtol=0, atol=1e-12)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=0, atol=1e-11)
    bo, blse = _brute_force_attention(q[:5].tolist(), k.tolist(), v.tolist(), False)
    np.testing.assert_allclose(o[:5], bo, rtol=1e-12, atol=1e-13)


def test_cross_attention_rejects_causal_mask():
    q, k = _rand((8, 4), 48), _rand((9, 4), 49)
    with pytest.raises(ValueError):
        oracle.attn_fwd_head(q, k, k, True)
    with pytest.raises(ValueError):
        oracle.attn_bwd_head(q, k, k, q, True)


def test_kv_replication_factor():
    assert oracle.kv_replication(8, 8) == 1        # LLaMA-3-style 8 KV heads at P = 8
    assert oracle.kv_replication(8, 4) == 1
    assert oracle.kv_replication(2, 8) == 4
    assert oracle.kv_replication(1, 4) == 4        # MQA: every rank holds the one KV head
    for Hkv, P in ((3, 2), (4, 6)):
        with pytest.raises(ValueError):
            oracle.kv_replication(Hkv, P)
    with pytest.raises(ValueError):
        oracle.check_gqa(8, 3)


@pytest.mark.parametrize("B,L,Hkv,d,P", [(2, 12, 1, 3, 4), (1, 16, 2, 2, 8), (2, 8, 4, 2, 2), (1, 6, 2, 1, 6)])
def test_kv_layout_change_by_procedure_and_adjoint(B, L, Hkv, d, P):
    rng = np.random.default_rng(50)
    x = rng.integers(0, 2**16, size=(P, B, L // P, Hkv, d), dtype=np.uint16)
    y = oracle.seq_to_head_kv(x, B, L, Hkv, d, P)
    R = oracle.kv_replication(Hkv, P)
    if R == 1:
        np.testing.assert_array_equal(y, oracle.seq_to_head(x, B, L, Hkv, d, P))
    else:
        # every rank gathers one KV head over all tokens: the head shared by
        # its query-head group, which R consecutive ranks hold alike
        full = np.concatenate([x[r] for r in range(P)], axis=1)        # [B, L, Hkv, d]
        assert y.shape == (P, B, L, 1, d)
        for p in range(P):
            np.testing.assert_array_equal(y[p, :, :, 0], full[:, :, p // R])
    # the gradient map is the adjoint of the gather: <S x, g> == <x, S^T g>
    xf = rng.standard_normal((P, B, L // P, Hkv, d))
    g = rng.standard_normal(y.shape)
    lhs = float(np.sum(oracle.seq_to_head_kv(xf, B, L, Hkv, d, P) * g))
    rhs = float(np.sum(xf * oracle.head_to_seq_kv_grad(g, B, L, Hkv, d, P)))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    # the row maps restate both directions as index arithmetic
    rows = oracle.seq_to_head_kv_source_rows(B, L, Hkv, P)
    np.testing.assert_array_equal(x.reshape(-1, d)[rows].reshape(y.shape), y)
    grows = oracle.head_to_seq_kv_grad_source_rows(B, L, Hkv, P)
    assert grows.shape[0] == R
    summed = sum(g.reshape(-1, d)[grows[j]] for j in range(R)).reshape(P, B, L // P, Hkv, d)
    np.testing.assert_allclose(summed, oracle.head_to_seq_kv_grad(g, B, L, Hkv, d, P), rtol=0, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv,P", [(8, 2, 2), (8, 2, 4), (4, 1, 4), (8, 2, 8)])
def test_gqa_pipeline_equals_monolithic(Hq, Hkv, P):
    # each rank runs GQA on its query heads and the KV heads they share; the
    # result and the gradients equal single-device GQA attention
    B, L, d = 1, 32, 8
    q, do = _rand((P, B, L // P, Hq, d), 51), _rand((P, B, L // P, Hq, d), 52)
    k, v = _rand((P, B, L // P, Hkv, d), 53), _rand((P, B, L // P, Hkv, d), 54)
    qh = oracle.seq_to_head(q, B, L, Hq, d, P)
    doh = oracle.seq_to_head(do, B, L, Hq, d, P)
    kh = oracle.seq_to_head_kv(k, B, L, Hkv, d, P)
    vh = oracle.seq_to_head_kv(v, B, L, Hkv, d, P)
    outs = [oracle.attn_fwd_gqa(qh[p], kh[p], vh[p], True)[0] for p in range(P)]
    grads = [oracle.attn_bwd_gqa(qh[p], kh[p], vh[p], doh[p], True) for p in range(P)]
    o = oracle.head_to_seq(np.stack(outs), B, L, Hq, d, P)
    dq = oracle.head_to_seq(np.stack([g[0] for g in grads]), B, L, Hq, d, P)
    dk = oracle.head_to_seq_kv_grad(np.stack([g[1] for g in grads]), B, L, Hkv, d, P)
    dv = oracle.head_to_seq_kv_grad(np.stack([g[2] for g in grads]), B, L, Hkv, d, P)
    glob = lambda a: np.concatenate(list(a), axis=1)  # noqa: E731  [P,B,L/P,..] -> [B,L,..]
    om, _ = oracle.attn_fwd_gqa(glob(q), glob(k), glob(v), True)
    dqm, dkm, dvm = oracle.attn_bwd_gqa(glob(q), glob(k), glob(v), glob(do), True)
    for mine, ref in ((o, om), (dq, dqm), (dk, dkm), (dv, dvm)):
        np.testing.assert_allclose(glob(mine), ref, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# block-sparse attention
# ---------------------------------------------------------------------------

def _layout(nb, kind, seed=0):
    if kind == "ones":
        return np.ones((nb, nb), np.uint8)
    if kind == "lower":
        return np.tril(np.ones((nb, nb), np.uint8))
    if kind == "diag":
        return np.eye(nb, dtype=np.uint8)
    rng = np.random.default_rng(seed)
    lay = (rng.random((nb, nb)) < 0.4).astype(np.uint8)
    np.fill_diagonal(lay, 1)
    return lay


@pytest.mark.parametrize("causal", [True, False])
def test_block_sparse_reduces_to_dense(causal):
    L, d, block = 100, 8, 16
    q, k, v, do = (_rand((L, d), s) for s in (70, 71, 72, 73))
    nb = -(-L // block)
    for kind in ("ones",) + (("lower",) if causal else ()):
        o, lse = oracle.attn_fwd_block_sparse_head(q, k, v, _layout(nb, kind), block, causal)
        od, lsed = oracle.attn_fwd_head(q, k, v, causal)
        np.testing.assert_allclose(o, od, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lsed, rtol=0, atol=1e-13)
        g = oracle.attn_bwd_block_sparse_head(q, k, v, do, _layout(nb, kind), block, causal)
        gd = oracle.attn_bwd_head(q, k, v, do, causal)
        for a, b_ in zip(g[:3], gd[:3]):
            np.testing.assert_allclose(a, b_, rtol=0, atol=1e-12)


def test_block_diagonal_layout_is_independent_blocks():
    # a diagonal layout cuts the sequence into independent causal blocks
    L, d, block = 70, 6, 16
    q, k, v, do = (_rand((L, d), s) for s in (74, 75, 76, 77))
    nb = -(-L // block)
    o, lse = oracle.attn_fwd_block_sparse_head(q, k, v, _layout(nb, "diag"), block, True)
    g = oracle.attn_bwd_block_sparse_head(q, k, v, do, _layout(nb, "diag"), block, True)
    for i0 in range(0, L, block):
        sl = slice(i0, min(L, i0 + block))
        ob, lseb = oracle.attn_fwd_head(q[sl], k[sl], v[sl], True)
        np.testing.assert_allclose(o[sl], ob, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[sl], lseb, rtol=0, atol=1e-13)
        gb = oracle.attn_bwd_head(q[sl], k[sl], v[sl], do[sl], True)
        for a, b_ in zip(g[:3], gb[:3]):
            np.testing.assert_allclose(a[sl], b_, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_block_sparse_matches_torch_masked_sdpa_and_autograd(causal):
    torch = pytest.importorskip("torch")
    L, d, block = 96, 16, 16
    q, k, v, do = (_rand((L, d), s) for s in (78, 79, 80, 81))
    nb = L // block
    lay = _layout(nb, "random", seed=3)
    o, lse = oracle.attn_fwd_block_sparse_head(q, k, v, lay, block, causal)
    dq, dk, dv, *_ = oracle.attn_bwd_block_sparse_head(q, k, v, do, lay, block, causal)
    vis = np.kron(lay, np.ones((block, block), np.uint8)).astype(bool)
    if causal:
        vis &= np.tril(np.ones((L, L), bool))
    tq, tk, tv = (torch.from_numpy(a).requires_grad_(True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                                           attn_mask=torch.from_numpy(vis)[None])[0]
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(o, out.detach().numpy(), rtol=0, atol=1e-12)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=0, atol=1e-11)
    s = (q @ k.T) / math.sqrt(d)
    np.testing.assert_allclose(lse, np.log(np.sum(np.where(vis, np.exp(s), 0.0), axis=1)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_batched_block_sparse_uses_each_heads_layout(causal):
    """The batched entry points take head h's layout for every batch entry:
    against torch's fp64 masked attention and autograd on [B, H, L, L] masks
    built from a different layout per head (a ragged last block included)."""
    torch = pytest.importorskip("torch")
    B, L, H, d, block = 2, 88, 3, 8, 16
    nb = -(-L // block)
    q, k, v, do = (_rand((B, L, H, d), s) for s in (91, 92, 93, 94))
    layout = np.stack([_layout(nb, "random", seed=10 + h) for h in range(H)])
    o, lse = oracle.attn_fwd_block_sparse(q, k, v, layout, block, causal)
    dq, dk, dv = oracle.attn_bwd_block_sparse(q, k, v, do, layout, block, causal)
    vis = np.stack([np.kron(layout[h], np.ones((block, block), np.uint8))[:L, :L].astype(bool) for h in range(H)])
    if causal:
        vis &= np.tril(np.ones((L, L), bool))[None]
    mask = torch.from_numpy(np.broadcast_to(vis, (B, H, L, L)).copy())
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3))).requires_grad_(True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    out.backward(torch.from_numpy(np.ascontiguousarray(do.transpose(0, 2, 1, 3))))
    np.testing.assert_allclose(o, out.detach().numpy().transpose(0, 2, 1, 3), rtol=0, atol=1e-12)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy().transpose(0, 2, 1, 3), rtol=0, atol=1e-11)
    s = np.einsum("bihe,bjhe->bhij", q, k) / math.sqrt(d)
    np.testing.assert_allclose(lse, np.log(np.sum(np.where(vis[None], np.exp(s), 0.0), axis=-1)), rtol=0, atol=1e-12)


def test_block_sparse_brute_force_and_sampled_rows():
    L, d, block = 40, 5, 8
    q, k, v, do = (_rand((L, d), s) for s in (82, 83, 84, 85))
    nb = L // block
    lay = _layout(nb, "random", seed=7)
    o, lse = oracle.attn_fwd_block_sparse_head(q, k, v, lay, block, True)
    for i in range(L):
        js = [j for j in range(i + 1) if lay[i // block, j // block]]
        w = [math.exp(sum(q[i, e] * k[j, e] for e in range(d)) / math.sqrt(d)) for j in js]
        z = sum(w)
        want = [sum(wj * v[j, e] for wj, j in zip(w, js)) / z for e in range(d)]
        np.testing.assert_allclose(o[i], want, rtol=1e-12, atol=1e-13)
        assert abs(lse[i] - math.log(z)) < 1e-12
    dq, dk, dv, *_ = oracle.attn_bwd_block_sparse_head(q, k, v, do, lay, block, True)
    c, dkc, dvc = oracle.attn_dkv_cols_block_sparse(q, k, v, do, [39, 31, 30, 9, 0], lay, block, True)
    np.testing.assert_allclose(dkc, dk[c], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dvc, dv[c], rtol=0, atol=1e-12)
    rows = [0, 7, 8, 23, 39]
    r = oracle.attn_rows_block_sparse(q, k, v, rows, lay, block, True, do=do)
    np.testing.assert_allclose(r["o"], o[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["lse"], lse[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["dq"], dq[rows], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_block_sparse_sampled_functions_cover_every_row_and_column(causal):
    # the sampled forms (formed over the active blocks' keys) against the full
    # masked head on a ragged length, a random layout and an emptied block row
    L, d, block = 45, 6, 8
    q, k, v, do = (_rand((L, d), s) for s in (90, 91, 92, 93))
    nb = -(-L // block)
    lay = _layout(nb, "random", seed=11)
    lay[3] = 0
    dq, dk, dv, o, lse, _ = oracle.attn_bwd_block_sparse_head(q, k, v, do, lay, block, causal)
    r = oracle.attn_rows_block_sparse(q, k, v, range(L), lay, block, causal, do=do)
    np.testing.assert_allclose(r["o"], o, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(np.isinf(r["lse"]), np.isinf(lse))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(r["lse"][fin], lse[fin], rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["dq"], dq, rtol=0, atol=1e-12)
    c, dkc, dvc = oracle.attn_dkv_cols_block_sparse(q, k, v, do, range(L), lay, block, causal)
    np.testing.assert_allclose(dkc, dk[c], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dvc, dv[c], rtol=0, atol=1e-12)
    # over a partition of the query blocks the parts add up to the whole
    parts = [oracle.attn_dkv_cols_block_sparse(q, k, v, do, range(L), lay, block, causal, row_blocks=rb)
             for rb in ((0, 2), (2, 3), (3, nb))]
    np.testing.assert_allclose(sum(p[1] for p in parts), dk[c], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sum(p[2] for p in parts), dv[c], rtol=0, atol=1e-12)
    # the absolute sums of the columns' products, as the full head's
    _, _, _, a_dkc, a_dvc = oracle.attn_dkv_cols_block_sparse(q, k, v, do, range(L), lay, block, causal,
                                                              abs_sums=True)
    _, a_dk, a_dv, _ = oracle.attn_abs_sums_block_sparse_head(q, k, v, do, lay, block, causal)
    np.testing.assert_allclose(a_dkc, a_dk[c], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a_dvc, a_dv[c], rtol=0, atol=1e-12)
    assert np.all(a_dkc >= np.abs(dkc) - 1e-12) and np.all(a_dvc >= np.abs(dvc) - 1e-12)


def test_block_sparse_row_without_keys():
    # a block row the layout leaves empty: zero output, LSE -inf, no gradient flow
    L, d, block = 32, 4, 8
    q, k, v, do = (_rand((L, d), s) for s in (86, 87, 88, 89))
    lay = np.tril(np.ones((4, 4), np.uint8))
    lay[2] = 0
    o, lse = oracle.attn_fwd_block_sparse_head(q, k, v, lay, block, True)
    assert np.all(o[16:24] == 0) and np.all(np.isneginf(lse[16:24]))
    assert np.all(np.isfinite(lse[:16])) and np.all(np.isfinite(lse[24:]))
    dq, dk, dv, *_ = oracle.attn_bwd_block_sparse_head(q, k, v, do, lay, block, True)
    assert np.all(dq[16:24] == 0)
    # dO of the empty rows does not reach dV
    do2 = do.copy()
    do2[16:24] = 123.0
    _, _, dv2, *_ = oracle.attn_bwd_block_sparse_head(q, k, v, do2, lay, block, True)
    np.testing.assert_allclose(dv2, dv, rtol=0, atol=1e-12)


def test_block_layout_generator_structure():
    from workloads import block_layout, custom
    wl = custom(1, 1000, 4, 64, 2, block=64, window=3, n_global=1, n_random=2, index=321)
    lay = block_layout(wl)
    nb = 16
    assert lay.shape == (4, nb, nb) and lay.dtype == np.uint8
    for h in range(4):
        assert np.all(np.triu(lay[h], 1) == 0)                   # causal: nothing above the diagonal
        for i in range(nb):
            row = lay[h, i]
            assert all(row[j] for j in range(max(0, i - 2), i + 1))   # window of 3
            assert row[0] == 1                                     # the global block
            extra = row[:i + 1].sum() - len(set(range(max(0, i - 2), i + 1)) | {0})
            assert extra == min(2, i + 1 - len(set(range(max(0, i - 2), i + 1)) | {0}))
    assert not np.array_equal(lay[0], lay[1])                      # random blocks differ per head
    np.testing.assert_array_equal(block_layout(wl), lay)          # seeded


# ---------------------------------------------------------------------------
# the comparison helper every bf16 bar uses: max |x - ref| and the relative
# Frobenius norm over the whole array, pinned on hand-computed values
# ---------------------------------------------------------------------------

def test_error_stats_hand_computed():
    # one element off by -1: max 1, ||diff|| = 1, ||ref|| = sqrt(1 + 4 + 16)
    st = oracle.error_stats(np.array([1.0, 2.0, 3.0]), np.array([1.0, 2.0, 4.0]))
    assert st["max_abs"] == 1.0
    assert st["rel_fro"] == pytest.approx(1.0 / math.sqrt(21.0), rel=1e-15)
    # the norm runs over every element of a matrix (not a per-row or spectral
    # norm): diff [[3, 0], [0, -4]] has Frobenius norm 5 (spectral 4), the
    # reference [[0, 0], [0, 4]] has 4, so the ratio is 1.25 (spectral: 1.0)
    st = oracle.error_stats(np.array([[3.0, 0.0], [0.0, 0.0]]), np.array([[0.0, 0.0], [0.0, 4.0]]))
    assert st["max_abs"] == 4.0
    assert st["rel_fro"] == pytest.approx(1.25, rel=1e-15)
    # the sign of the difference does not matter; a larger error below the
    # largest reference entry is still the maximum
    st = oracle.error_stats(np.array([-5.0, 10.0]), np.array([0.0, 10.5]))
    assert st["max_abs"] == 5.0
    assert st["rel_fro"] == pytest.approx(math.sqrt(25.25) / 10.5, rel=1e-15)
    # an exact match, and a zero reference (then the plain norm of the difference)
    assert oracle.error_stats(np.arange(6.0), np.arange(6.0)) == {"max_abs": 0.0, "rel_fro": 0.0}
    st = oracle.error_stats(np.array([0.0, 3.0, -4.0]), np.zeros(3))
    assert st == {"max_abs": 4.0, "rel_fro": 5.0}
    # integer-coded bf16 inputs are compared as float64, not in their own type
    st = oracle.error_stats(np.array([65535], dtype=np.uint16), np.array([0.0]))
    assert st["max_abs"] == 65535.0
    # empty arrays have no error
    assert oracle.error_stats(np.zeros(0), np.zeros(0))["max_abs"] == 0.0
