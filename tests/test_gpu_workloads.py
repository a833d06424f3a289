"""GPU parity on the named workloads at their full sizes, launched as bench.py launches them.

For each workload: Q, K, V (and dO) are drawn on the device in the
token-sharded layout, seq_to_head runs on the full tensors, attention runs on
rank 0's head group, head_to_seq runs on the full head buffers. Checked
against the fp64 oracle, which reads the generator's bits (never a kernel's
output):
  * permutations: bit-exact on whole destination-rank blocks and on head_to_seq;
  * forward: O and LSE of sampled rows -- hand-picked ones (both ends, tile
    edges, stressed rows) against the elementwise bar, uniformly drawn ones
    also against the relative Frobenius bar -- and every row of a causal prefix: the kernel's rows below
    L' do not depend on later tokens, so a run on the first L' tokens must
    equal the first L' rows of the full run bit for bit, and is checked
    in full against the oracle;
  * backward: dQ of the sampled rows (also prefix-checked), dK/dV of sampled
    key columns near the end, and over the full outputs the identities
    sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i.
"""
import gc

import numpy as np
import pytest

import exact_attention_ulysses_amd as U
import oracle
from workloads import WORKLOADS, device_tensor, stress_positions

from gpu_common import check_close, to_f64, to_host_bits, torch_mod

pytestmark = pytest.mark.gpu

NAMES = ["gpt1.2b-L32k-fwd", "gpt7b-L131k", "gpt30b-L262k", "L1m"]
PREFIX = 8192


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    U.lib()


class Run:
    """Device state of one workload after one pass of the hot path."""

    def __init__(self, key):
        torch = torch_mod()
        self.wl = wl = WORKLOADS[key]
        B, L, H, d, P, Hh = wl.B, wl.L, wl.H, wl.d, wl.P, wl.Hp
        self.ins = ["q", "k", "v"] + (["do"] if wl.backward else [])
        self.outs = ["o"] + (["dq", "dk", "dv"] if wl.backward else [])
        print(f"[{key}] drawing inputs", flush=True)
        self.seq = {n: device_tensor(wl, n) for n in self.ins}
        self.head = {}
        for n in self.ins:
            self.head[n] = torch.empty(wl.head_shape, dtype=torch.bfloat16, device="cuda")
            U.ulysses_seq_to_head(self.seq[n], self.head[n], B, L, H, d, P)
        self.ohead = {n: device_tensor(wl, "fill_" + n) for n in self.outs}
        r0 = {n: self.head[n][0] for n in self.ins}
        o0 = {n: self.ohead[n][0] for n in self.outs}
        self.lse = torch.empty((B, Hh, L), dtype=torch.float32, device="cuda")
        print(f"[{key}] attention", flush=True)
        U.ulysses_attn_fwd(r0["q"], r0["k"], r0["v"], o0["o"], self.lse, B, L, H, d, P, wl.causal)
        if wl.backward:
            ws = torch.empty(U.ulysses_attn_bwd_workspace_bytes(B, L, H, d, P, wl.causal), dtype=torch.uint8,
                             device="cuda")
            U.ulysses_attn_bwd(r0["q"], r0["k"], r0["v"], o0["o"], r0["do"], self.lse, o0["dq"], o0["dk"],
                               o0["dv"], ws, B, L, H, d, P, wl.causal)
        self.oseq = {}
        for n in self.outs:
            self.oseq[n] = torch.empty(wl.seq_shape, dtype=torch.bfloat16, device="cuda")
            U.ulysses_head_to_seq(self.ohead[n], self.oseq[n], B, L, H, d, P)
        torch.cuda.synchronize()
        print(f"[{key}] device pass done", flush=True)
        self._f64 = {}
        self._host = {}

    def host_seq(self, n):
        """Raw bits of input n as drawn (seq layout), cached on the host."""
        if n not in self._host:
            self._host[n] = to_host_bits(self.seq[n])
        return self._host[n]

    def oracle_head(self, n):
        """Rank 0's head block of input n, [B, L, Hh, d] float64, via the oracle's own layout change."""
        if n not in self._f64:
            wl = self.wl
            bits = oracle.seq_to_head_part(self.host_seq(n), wl.B, wl.L, wl.H, wl.d, wl.P, 0)
            self._f64[n] = oracle.bf16_bits_to_f64(bits)
            gc.collect()
        return self._f64[n]


_runs = {}


def get_run(key):
    if key not in _runs:
        for k in list(_runs):   # one workload resident at a time
            del _runs[k]
        gc.collect()
        torch_mod().cuda.empty_cache()
        _runs[key] = Run(key)
    return _runs[key]


def edge_rows(wl, head):
    """Hand-picked rows: both ends, tile edges, the stressed rows of the head."""
    L = wl.L
    rows = {0, 1, 2, 63, 64, 127, 128, 129, 255, 256, L // 2, L - 129, L - 128, L - 65, L - 64, L - 1}
    for name in ("q", "k"):
        pos = stress_positions(wl, name)
        if pos is not None:
            rows.add(int(pos[0, head]))   # rank 0 holds global heads 0 .. Hh-1
    return sorted(r for r in rows if 0 <= r < L)


def uniform_rows(wl, head, n=24):
    """Rows drawn uniformly: their relative Frobenius error estimates the whole tensor's."""
    rng = np.random.default_rng(1000 + 10 * wl.index + head)
    return sorted(set(int(r) for r in rng.integers(0, wl.L, size=n)))


@pytest.mark.parametrize("key", NAMES)
def test_seq_to_head_and_back_bit_exact(key):
    run = get_run(key)
    wl = run.wl
    B, L, H, d, P = wl.B, wl.L, wl.H, wl.d, wl.P
    rng = np.random.default_rng(5)
    ranks = sorted({0, P - 1, int(rng.integers(1, P))})
    for n in run.ins:
        host = run.host_seq(n)
        for p in ranks:
            np.testing.assert_array_equal(to_host_bits(run.head[n][p]),
                                          oracle.seq_to_head_part(host, B, L, H, d, P, p))
    # head_to_seq of the outputs (rank 0's head block from attention, the other blocks filler)
    for n in run.outs[:2]:
        y = to_host_bits(run.ohead[n])
        for r in ranks:
            np.testing.assert_array_equal(to_host_bits(run.oseq[n][r]), oracle.head_to_seq_part(y, B, L, H, d, P, r))
        del y
        gc.collect()


@pytest.mark.parametrize("key", NAMES)
def test_forward_sampled_rows(key):
    run = get_run(key)
    wl = run.wl
    q, k, v = (run.oracle_head(n) for n in "qkv")
    o = to_f64(run.ohead["o"][0], "bf16")
    lse = run.lse.cpu().numpy()
    for h in range(wl.Hp):
        for kind, rows in (("edge", edge_rows(wl, h)), ("uniform", uniform_rows(wl, h))):
            ref = oracle.attn_rows(q[0, :, h], k[0, :, h], v[0, :, h], rows, wl.causal)
            check_close(f"O {kind} rows head {h}", o[0, rows, h], ref["o"], "bf16", fro=(kind == "uniform"))
            assert np.max(np.abs(lse[0, h, rows] - ref["lse"])) <= 1e-3


@pytest.mark.parametrize("key", NAMES)
def test_causal_prefix_matches_full_run_and_oracle(key):
    torch = torch_mod()
    run = get_run(key)
    wl = run.wl
    B, H, d, P, Hh = wl.B, wl.H, wl.d, wl.P, wl.Hp
    Lp = PREFIX
    r0 = {n: run.head[n][0][:, :Lp] for n in run.ins}   # B = 1: the first Lp rows are contiguous
    assert B == 1 and all(t.is_contiguous() for t in r0.values())
    o = torch.empty((B, Lp, Hh, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hh, Lp), dtype=torch.float32, device="cuda")
    U.ulysses_attn_fwd(r0["q"], r0["k"], r0["v"], o, lse, B, Lp, H, d, P, True)
    full_o = run.ohead["o"][0][:, :Lp]
    assert torch.equal(o.view(torch.int16), full_o.view(torch.int16)), "prefix rows differ from the full run"
    assert torch.equal(lse, run.lse[:, :, :Lp].contiguous())
    q, k, v = (run.oracle_head(n)[:, :Lp] for n in "qkv")
    if wl.backward:
        do = run.oracle_head("do")[:, :Lp]
        dq, dk, dv = (torch.empty_like(o) for _ in range(3))
        ws = torch.empty(U.ulysses_attn_bwd_workspace_bytes(B, Lp, H, d, P), dtype=torch.uint8, device="cuda")
        U.ulysses_attn_bwd(r0["q"], r0["k"], r0["v"], o, r0["do"], lse, dq, dk, dv, ws, B, Lp, H, d, P, True)
        # dQ rows depend only on earlier keys: equal to the full run's
        assert torch.equal(dq.view(torch.int16), run.ohead["dq"][0][:, :Lp].view(torch.int16))
        dq_r, dk_r, dv_r, o_r, lse_r, _ = oracle.attn_bwd(q, k, v, do, True)
        check_close("dQ prefix", to_f64(dq, "bf16"), dq_r, "bf16")
        check_close("dK prefix problem", to_f64(dk, "bf16"), dk_r, "bf16")
        check_close("dV prefix problem", to_f64(dv, "bf16"), dv_r, "bf16")
    else:
        o_r, lse_r = oracle.attn_fwd(q, k, v, True)
    check_close("O prefix", to_f64(o, "bf16"), o_r, "bf16")
    assert np.max(np.abs(lse.cpu().numpy() - lse_r)) <= 1e-3


@pytest.mark.parametrize("key", [n for n in NAMES if WORKLOADS[n].backward])
def test_backward_sampled_rows_and_columns(key):
    run = get_run(key)
    wl = run.wl
    L = wl.L
    q, k, v, do = (run.oracle_head(n) for n in ("q", "k", "v", "do"))
    dq, dk, dv = (to_f64(run.ohead[n][0], "bf16") for n in ("dq", "dk", "dv"))
    rng = np.random.default_rng(77)
    cols = sorted({L - 1, L - 2, L - 63, L - 64, L - 65, L - 128, L - 129, L - 200, L - 256}
                  | set(int(c) for c in rng.integers(L - 384, L, size=4)))
    for h in range(wl.Hp):
        for kind, rows in (("edge", edge_rows(wl, h)), ("uniform", uniform_rows(wl, h))):
            ref = oracle.attn_rows(q[0, :, h], k[0, :, h], v[0, :, h], rows, wl.causal, do=do[0, :, h])
            check_close(f"dQ {kind} rows head {h}", dq[0, rows, h], ref["dq"], "bf16", fro=(kind == "uniform"))
        c, dk_r, dv_r = oracle.attn_dkv_cols(q[0, :, h], k[0, :, h], v[0, :, h], do[0, :, h], cols, wl.causal,
                                             row_block=64)
        check_close(f"dK cols head {h}", dk[0, c, h], dk_r, "bf16")
        check_close(f"dV cols head {h}", dv[0, c, h], dv_r, "bf16")


@pytest.mark.parametrize("key", [n for n in NAMES if WORKLOADS[n].backward])
def test_backward_identities_over_full_outputs(key):
    run = get_run(key)
    wl = run.wl
    do = run.oracle_head("do")
    dk, dv = (to_f64(run.ohead[n][0], "bf16") for n in ("dk", "dv"))
    # Rows of P sum to one, so sum_j dV_j = sum_i dO_i; rows of dS sum to zero, so
    # sum_j dK_j = 0. These are gross-error checks over every output row (a wrong
    # sign, scale or a large missing part); the bounds allow for bf16 rounding of
    # P, dS and the outputs (2^-9 relative each) accumulated with any sign.
    for h in range(wl.Hp):
        sv = dv[0, :, h].sum(axis=0)
        want = do[0, :, h].sum(axis=0)
        bound_v = 2.0 ** -7 * (np.abs(dv[0, :, h]).sum(axis=0) + np.abs(do[0, :, h]).sum(axis=0))
        assert np.all(np.abs(sv - want) <= bound_v), (h, np.max(np.abs(sv - want) / bound_v))
        sk = dk[0, :, h].sum(axis=0)
        bound_k = 2.0 ** -6 * np.abs(dk[0, :, h]).sum(axis=0) + 1e-6
        assert np.all(np.abs(sk) <= bound_k), (h, np.max(np.abs(sk) / bound_k))
