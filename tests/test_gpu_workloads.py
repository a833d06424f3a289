"""GPU parity on the named workloads at their full sizes, launched as bench.py launches them.

For each workload: Q, K, V (and dO) are drawn on the device in the
token-sharded layout, seq_to_head runs on the full tensors, attention runs on
rank 0's head group, head_to_seq runs on the full head buffers. Checked
against the fp64 oracle, which reads the generator's bits (never a kernel's
output):
  * permutations: bit-exact on whole destination-rank blocks and on head_to_seq;
  * forward: O and LSE of sampled rows -- hand-picked ones (both ends, tile
    edges, stressed rows) against the elementwise bar, uniformly drawn ones
    also against the relative Frobenius bar -- and every row of a causal
    prefix: rows below L' do not depend on later tokens, so a run on the
    first L' tokens equals the first L' rows of the full run bit for bit
    (for an L' whose launch takes the full run's path), and a run on the
    first 8192 tokens is checked in full against the oracle;
  * backward: dQ of the sampled rows (also prefix-checked), dK/dV of sampled
    key columns near the end, every element of the early key columns (the
    longest sums) of the 262K workload's first head, and over the full
    outputs the identities sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i;
  * every element of rank 0's outputs against the full oracle on the 32K
    forward, the 8K forward and backward and the 131K forward and backward,
    and of the first head of the 262K forward and backward.
Grouped-query workloads run K and V through the K/V layout change (and dK,
dV through its gradient form); a K/V head's dK/dV columns are checked
against the sum of its query heads' oracle columns. The cross-attention
workload (queries and keys of different lengths) is bidirectional, so it has
no causal prefix; its dK/dV columns are checked on its first head. The
block-sparse workload runs the block-sparse entry points with rank 0's seeded
block layout, and every oracle value is formed under the same layout.
"""
import gc
import time

import numpy as np
import pytest

import exact_attention_ulysses_amd as U
import oracle
from workloads import WORKLOADS, block_layout, device_tensor, stress_positions

from gpu_common import (bf16_ulp, causal_row_ranges, check_close, host_parallel, shared_head_allowed, to_f64,
                        to_host_bits, torch_mod)

pytestmark = pytest.mark.gpu

NAMES = ["gpt1.2b-L32k-fwd", "gpt7b-L131k", "gpt30b-L262k", "L1m", "gqa8-L131k", "gqa2-L131k",
         "cross-L16k-L131k", "bsparse-L131k", "gpt7b-L8k"]


def _kv(n):
    return n in ("k", "v", "dk", "dv")
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
        B, L, H, d, P, Hh, Lk, Hk = wl.B, wl.L, wl.H, wl.d, wl.P, wl.Hp, wl.Lk, wl.Hk
        self.G = Hh // wl.Hkp      # local query heads per local K/V head
        self.ins = ["q", "k", "v"] + (["do"] if wl.backward else [])
        self.outs = ["o"] + (["dq", "dk", "dv"] if wl.backward else [])
        print(f"[{key}] drawing inputs", flush=True)
        self.seq = {n: device_tensor(wl, n) for n in self.ins}
        self.head = {}
        for n in self.ins:
            self.head[n] = torch.empty(wl.shape_of("fill_d" + n if _kv(n) else "fill_o"), dtype=torch.bfloat16,
                                       device="cuda")
            if _kv(n):
                U.ulysses_seq_to_head_kv(self.seq[n], self.head[n], B, Lk, Hk, d, P)
            else:
                U.ulysses_seq_to_head(self.seq[n], self.head[n], B, L, H, d, P)
        self.ohead = {n: device_tensor(wl, "fill_" + n) for n in self.outs}
        r0 = {n: self.head[n][0] for n in self.ins}
        o0 = {n: self.ohead[n][0] for n in self.outs}
        self.lse = torch.empty((B, Hh, L), dtype=torch.float32, device="cuda")
        # block layout of rank 0's heads (block-sparse workloads)
        self.layout = block_layout(wl, heads=range(Hh)) if wl.block else None
        lay = torch.from_numpy(self.layout).to("cuda") if wl.block else None
        print(f"[{key}] attention", flush=True)
        if wl.block:
            U.ulysses_attn_fwd_block_sparse(r0["q"], r0["k"], r0["v"], o0["o"], self.lse, lay, B, L, H, Hk, d, P,
                                            wl.causal)
        else:
            U.ulysses_attn_fwd_gqa(r0["q"], r0["k"], r0["v"], o0["o"], self.lse, B, L, Lk, H, Hk, d, P, wl.causal)
        if wl.backward:
            ws_bytes = (U.ulysses_attn_bwd_block_sparse_workspace_bytes(B, L, H, Hk, d, P, wl.causal) if wl.block
                        else U.ulysses_attn_bwd_gqa_workspace_bytes(B, L, Lk, H, Hk, d, P, wl.causal))
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
            if wl.block:
                U.ulysses_attn_bwd_block_sparse(r0["q"], r0["k"], r0["v"], o0["o"], r0["do"], self.lse, o0["dq"],
                                                o0["dk"], o0["dv"], lay, ws, B, L, H, Hk, d, P, wl.causal)
            else:
                U.ulysses_attn_bwd_gqa(r0["q"], r0["k"], r0["v"], o0["o"], r0["do"], self.lse, o0["dq"], o0["dk"],
                                       o0["dv"], ws, B, L, Lk, H, Hk, d, P, wl.causal)
        self.oseq = {}
        for n in self.outs:
            self.oseq[n] = torch.empty(wl.shape_of(n[1:] if _kv(n) else "q"), dtype=torch.bfloat16,
                                       device="cuda")
            if _kv(n):
                U.ulysses_head_to_seq_kv_grad(self.ohead[n], self.oseq[n], B, Lk, Hk, d, P)
            else:
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
        """Rank 0's head block of input n, [B, L, heads, d] float64, via the oracle's own layout change."""
        if n not in self._f64:
            wl = self.wl
            if _kv(n):
                bits = oracle.seq_to_head_kv(self.host_seq(n), wl.B, wl.Lk, wl.Hk, wl.d, wl.P)[0]
            else:
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
    B, L, H, d, P, Lk, Hk = wl.B, wl.L, wl.H, wl.d, wl.P, wl.Lk, wl.Hk
    rng = np.random.default_rng(5)
    ranks = sorted({0, P - 1, int(rng.integers(1, P))})
    for n in run.ins:
        host = run.host_seq(n)
        if _kv(n):
            want = oracle.seq_to_head_kv(host, B, Lk, Hk, d, P)
            for p in ranks:
                np.testing.assert_array_equal(to_host_bits(run.head[n][p]), want[p])
            del want
        else:
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
    # the gradient form of the K/V layout change (bits copied, or replicas summed)
    if wl.backward:
        y = to_host_bits(run.ohead["dk"])
        R = P * wl.Hkp // Hk
        if R == 1:
            for r in ranks:
                np.testing.assert_array_equal(to_host_bits(run.oseq["dk"][r]),
                                              oracle.head_to_seq_part(y, B, Lk, Hk, d, P, r))
        else:
            yf = oracle.bf16_bits_to_f64(y)
            want = oracle.head_to_seq_kv_grad(yf, B, Lk, Hk, d, P)
            mag = oracle.head_to_seq_kv_grad(np.abs(yf), B, Lk, Hk, d, P)
            del yf
            acc = (R - 1) * 2.0 ** -24 * mag
            got = to_f64(run.oseq["dk"], "bf16")
            assert np.all(np.abs(got - want) <= 0.5 * bf16_ulp(np.abs(want) + acc) + acc)
            del want, mag, got
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
        j = h // run.G
        for kind, rows in (("edge", edge_rows(wl, h)), ("uniform", uniform_rows(wl, h))):
            if wl.block:
                ref = oracle.attn_rows_block_sparse(q[0, :, h], k[0, :, j], v[0, :, j], rows, run.layout[h], wl.block,
                                                    wl.causal)
            else:
                ref = oracle.attn_rows(q[0, :, h], k[0, :, j], v[0, :, j], rows, wl.causal)
            check_close(f"O {kind} rows head {h}", o[0, rows, h], ref["o"], "bf16", fro=(kind == "uniform"))
            assert np.max(np.abs(lse[0, h, rows] - ref["lse"])) <= 1e-3


# Dense causal launches split each query block's key walk below these block
# counts (over all batch entries and heads): the forward between two wave
# groups below 384 blocks of 256 rows and between four below 192; dQ, below
# 1024 blocks of 128 rows, between two wave groups or into chunks whose
# partial sums are added. A split rounds differently, so a prefix run is
# compared bit for bit with the full run only when its launches take the
# same paths.
FWD_SPLIT_BELOW_256 = 384
FWD_SPLIT4_BELOW_256 = 192
DQ_SPLIT_BELOW_128 = 1024


def _prefix_run(run, Lp):
    """Attention (and backward) of rank 0's heads on the first Lp tokens."""
    torch = torch_mod()
    wl = run.wl
    B, H, d, P, Hh, Hk = wl.B, wl.H, wl.d, wl.P, wl.Hp, wl.Hk
    r0 = {n: run.head[n][0][:, :Lp] for n in run.ins}   # B = 1: the first Lp rows are contiguous
    assert B == 1 and all(t.is_contiguous() for t in r0.values())
    out = {"o": torch.empty((B, Lp, Hh, d), dtype=torch.bfloat16, device="cuda"),
           "lse": torch.empty((B, Hh, Lp), dtype=torch.float32, device="cuda")}
    lay_dev = None
    if wl.block:   # the prefix's blocks keep their layout entries
        nbp = Lp // wl.block
        out["layout"] = np.ascontiguousarray(run.layout[:, :nbp, :nbp])
        lay_dev = torch.from_numpy(out["layout"]).to("cuda")
        U.ulysses_attn_fwd_block_sparse(r0["q"], r0["k"], r0["v"], out["o"], out["lse"], lay_dev, B, Lp, H, Hk, d,
                                        P, True)
    else:
        U.ulysses_attn_fwd_gqa(r0["q"], r0["k"], r0["v"], out["o"], out["lse"], B, Lp, Lp, H, Hk, d, P, True)
    if wl.backward:
        out["dq"] = torch.empty_like(out["o"])
        out["dk"], out["dv"] = torch.empty_like(r0["k"]), torch.empty_like(r0["v"])
        ws_bytes = (U.ulysses_attn_bwd_block_sparse_workspace_bytes(B, Lp, H, Hk, d, P) if wl.block
                    else U.ulysses_attn_bwd_gqa_workspace_bytes(B, Lp, Lp, H, Hk, d, P))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        if wl.block:
            U.ulysses_attn_bwd_block_sparse(r0["q"], r0["k"], r0["v"], out["o"], r0["do"], out["lse"], out["dq"],
                                            out["dk"], out["dv"], lay_dev, ws, B, Lp, H, Hk, d, P, True)
        else:
            U.ulysses_attn_bwd_gqa(r0["q"], r0["k"], r0["v"], out["o"], r0["do"], out["lse"], out["dq"], out["dk"],
                                   out["dv"], ws, B, Lp, Lp, H, Hk, d, P, True)
    return out


def _same_path_prefix(wl):
    """Shortest prefix length >= PREFIX whose dense launches take the full run's paths
    (each path covers a range of launch sizes: at least the lower end of the full
    run's range keeps the prefix on it)."""
    if wl.block:
        return PREFIX
    nhb = wl.B * wl.Hp
    Lb = PREFIX
    w256 = -(-wl.L // 256) * nhb
    if w256 >= FWD_SPLIT_BELOW_256:
        Lb = max(Lb, -(-FWD_SPLIT_BELOW_256 // nhb) * 256)
    elif w256 >= FWD_SPLIT4_BELOW_256:
        Lb = max(Lb, -(-FWD_SPLIT4_BELOW_256 // nhb) * 256)
    if wl.backward and -(-wl.L // 128) * nhb >= DQ_SPLIT_BELOW_128:
        Lb = max(Lb, -(-DQ_SPLIT_BELOW_128 // nhb) * 128)
    return min(wl.L, -(-Lb // 256) * 256)


@pytest.mark.parametrize("key", [n for n in NAMES if WORKLOADS[n].causal])
def test_causal_prefix_matches_full_run_and_oracle(key):
    torch = torch_mod()
    run = get_run(key)
    wl = run.wl
    Hh = wl.Hp
    # rows below Lb depend only on the first Lb tokens: a run on them equals
    # the full run's rows bit for bit (O, LSE and, from the same O, dQ)
    Lb = _same_path_prefix(wl)
    same = _prefix_run(run, Lb)
    full_o = run.ohead["o"][0][:, :Lb]
    assert torch.equal(same["o"].view(torch.int16), full_o.view(torch.int16)), "prefix rows differ from the full run"
    assert torch.equal(same["lse"], run.lse[:, :, :Lb].contiguous())
    if wl.backward:
        assert torch.equal(same["dq"].view(torch.int16), run.ohead["dq"][0][:, :Lb].view(torch.int16))
    # the first PREFIX tokens as a problem of their own, in full against the oracle
    Lp = PREFIX
    pre = same if Lb == Lp else _prefix_run(run, Lp)
    del same
    o, lse = pre["o"], pre["lse"]
    q, k, v = (run.oracle_head(n)[:, :Lp] for n in "qkv")
    if wl.backward:
        do = run.oracle_head("do")[:, :Lp]
        dq, dk, dv = pre["dq"], pre["dk"], pre["dv"]
        if wl.block:
            dq_r, dk_r, dv_r = oracle.attn_bwd_block_sparse(q, k, v, do, pre["layout"], wl.block, True)
            o_r, lse_r = oracle.attn_fwd_block_sparse(q, k, v, pre["layout"], wl.block, True)
        else:
            dq_r, dk_r, dv_r = oracle.attn_bwd_gqa(q, k, v, do, True)
            o_r, lse_r = oracle.attn_fwd_gqa(q, k, v, True)
        check_close("dQ prefix", to_f64(dq, "bf16"), dq_r, "bf16")
        G = run.G
        if G == 1:
            allowed = {"dK": None, "dV": None}
        else:   # a shared K/V head sums its G query heads' gradients
            parts = {"dK": np.zeros((G,) + dk_r.shape), "dV": np.zeros((G,) + dv_r.shape)}
            for h in range(Hh):
                r = oracle.attn_bwd_head(q[0, :, h], k[0, :, h // G], v[0, :, h // G], do[0, :, h], True)
                parts["dK"][h % G, 0, :, h // G] = r[1]
                parts["dV"][h % G, 0, :, h // G] = r[2]
            allowed = {nm: shared_head_allowed(parts[nm], want, "bf16") for nm, want in (("dK", dk_r), ("dV", dv_r))}
        check_close("dK prefix problem", to_f64(dk, "bf16"), dk_r, "bf16", allowed=allowed["dK"])
        check_close("dV prefix problem", to_f64(dv, "bf16"), dv_r, "bf16", allowed=allowed["dV"])
    elif wl.block:
        o_r, lse_r = oracle.attn_fwd_block_sparse(q, k, v, pre["layout"], wl.block, True)
    else:
        o_r, lse_r = oracle.attn_fwd_gqa(q, k, v, True)
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
    Lk, G = wl.Lk, run.G
    cols = sorted({Lk - 1, Lk - 2, Lk - 63, Lk - 64, Lk - 65, Lk - 128, Lk - 129, Lk - 200, Lk - 256}
                  | set(int(c) for c in rng.integers(Lk - 384, Lk, size=4)))
    for h in range(wl.Hp):
        j = h // G
        for kind, rows in (("edge", edge_rows(wl, h)), ("uniform", uniform_rows(wl, h))):
            if wl.block:
                ref = oracle.attn_rows_block_sparse(q[0, :, h], k[0, :, j], v[0, :, j], rows, run.layout[h], wl.block,
                                                    wl.causal, do=do[0, :, h])
            else:
                ref = oracle.attn_rows(q[0, :, h], k[0, :, j], v[0, :, j], rows, wl.causal, do=do[0, :, h])
            check_close(f"dQ {kind} rows head {h}", dq[0, rows, h], ref["dq"], "bf16", fro=(kind == "uniform"))
    # bidirectional attention: every query row sees every column, so a column
    # costs a full pass over the rows; check the first K/V head there
    kv_heads = range(wl.Hkp) if wl.causal else range(1)
    for j in kv_heads:
        parts_k, parts_v = [], []
        for h in range(j * G, (j + 1) * G):
            if wl.block:
                c, dk_r, dv_r = oracle.attn_dkv_cols_block_sparse(q[0, :, h], k[0, :, j], v[0, :, j], do[0, :, h],
                                                                  cols, run.layout[h], wl.block, wl.causal)
            else:
                c, dk_r, dv_r = oracle.attn_dkv_cols(q[0, :, h], k[0, :, j], v[0, :, j], do[0, :, h], cols,
                                                     wl.causal, row_block=64)
            parts_k.append(dk_r)
            parts_v.append(dv_r)
        if G == 1:
            check_close(f"dK cols K/V head {j}", dk[0, c, j], parts_k[0], "bf16")
            check_close(f"dV cols K/V head {j}", dv[0, c, j], parts_v[0], "bf16")
        else:
            wk, wv = np.sum(parts_k, axis=0), np.sum(parts_v, axis=0)
            check_close(f"dK cols K/V head {j}", dk[0, c, j], wk, "bf16", allowed=shared_head_allowed(parts_k, wk, "bf16"))
            check_close(f"dV cols K/V head {j}", dv[0, c, j], wv, "bf16", allowed=shared_head_allowed(parts_v, wv, "bf16"))


@pytest.mark.parametrize("key", [n for n in NAMES if WORKLOADS[n].backward])
def test_backward_identities_over_full_outputs(key):
    run = get_run(key)
    wl = run.wl
    do = run.oracle_head("do")
    dk, dv = (to_f64(run.ohead[n][0], "bf16") for n in ("dk", "dv"))
    G = run.G
    # Rows of P sum to one, so sum_j dV_j = sum_i dO_i (summed over the query
    # heads that share the K/V head); rows of dS sum to zero, so sum_j dK_j = 0.
    # These are gross-error checks over every output row (a wrong sign, scale
    # or a large missing part); the bounds allow for bf16 rounding of P, dS and
    # the outputs (2^-9 relative each) accumulated with any sign.
    for j in range(wl.Hkp):
        sv = dv[0, :, j].sum(axis=0)
        dog = do[0, :, j * G:(j + 1) * G]
        want = dog.sum(axis=(0, 1))
        bound_v = 2.0 ** -7 * (np.abs(dv[0, :, j]).sum(axis=0) + np.abs(dog).sum(axis=(0, 1)))
        assert np.all(np.abs(sv - want) <= bound_v), (j, np.max(np.abs(sv - want) / bound_v))
        sk = dk[0, :, j].sum(axis=0)
        bound_k = 2.0 ** -6 * np.abs(dk[0, :, j]).sum(axis=0) + 1e-6
        assert np.all(np.abs(sk) <= bound_k), (j, np.max(np.abs(sk) / bound_k))


@pytest.mark.parametrize("key", ["gpt30b-L262k"])
def test_backward_early_key_columns(key):
    """dK and dV of the early key columns at full size, every element of them:
    key 0 is seen by every query row, so these are the longest sums of the
    backward and the first work items of the dK/dV launch, plus the tile
    edges 63/64 and 127/128, the middle key, and the stressed K row of the
    head. Each column needs every later row's LSE and D, so the oracle forms
    the whole forward of the head (about one 262K-token forward of fp64 work)."""
    run = get_run(key)
    wl = run.wl
    L = wl.Lk
    h = 0
    q, k, v, do = (run.oracle_head(n) for n in ("q", "k", "v", "do"))
    dk, dv = (to_f64(run.ohead[n][0], "bf16") for n in ("dk", "dv"))
    cols = {0, 1, 2, 63, 64, 127, 128, 129, 255, 256, L // 2 - 1, L // 2}
    pos = stress_positions(wl, "k")
    if pos is not None:
        cols.add(int(pos[0, h]))
    cols = sorted(c for c in cols if 0 <= c < L)
    t0 = time.perf_counter()
    # every query row sees key 0: split the rows' sum into ranges formed side by side
    parts = host_parallel(lambda r: oracle.attn_dkv_cols(q[0, :, h], k[0, :, h], v[0, :, h], do[0, :, h], cols,
                                                         wl.causal, rows=r), causal_row_ranges(wl.L, 16))
    c = parts[0][0]
    dk_r, dv_r = sum(p[1] for p in parts), sum(p[2] for p in parts)
    print(f"[{key}] early columns {cols}: oracle {time.perf_counter() - t0:.0f} s", flush=True)
    check_close(f"dK early cols head {h} {key}", dk[0, c, h], dk_r, "bf16", fro=False)
    check_close(f"dV early cols head {h} {key}", dv[0, c, h], dv_r, "bf16", fro=False)


# heads compared in full (all of rank 0's unless listed): the 262K workload's
# full backward costs four times a 131K head, so one head (with its stressed
# Q and K rows) is compared
FULL_HEADS = {"gpt30b-L262k": (0,)}


@pytest.mark.parametrize("key", ["gpt1.2b-L32k-fwd", "gpt7b-L8k", "gpt7b-L131k", "gpt30b-L262k"])
def test_full_oracle_every_element(key):
    """A workload as the benchmark would run it, every element of rank 0's
    O and LSE (and dQ, dK, dV) against the full fp64 oracle: seconds for the
    32K forward and the 8K forward and backward (whose launches split every
    walk: two-group forward, dK/dV halves, dQ chunks), about a minute of 16
    host cores per head for the 131K forward and backward (its early key
    columns, the longest dK/dV sums, included), whose four heads the oracle
    forms side by side, and about a minute for one 262K head (its stressed
    Q and K rows included) cut into 16 row ranges."""
    run = get_run(key)
    wl = run.wl
    assert run.G == 1
    q, k, v = (run.oracle_head(n) for n in ("q", "k", "v"))
    do = run.oracle_head("do") if wl.backward else None
    got = {n: to_f64(run.ohead[n][0], "bf16") for n in run.outs}
    lse = run.lse.cpu().numpy()

    # the heads, each cut into row ranges of equal work, side by side; the
    # ranges' dK, dV terms add up to the whole
    heads = FULL_HEADS.get(key, tuple(range(wl.Hp)))
    parts = max(1, 16 // len(heads)) if wl.backward else 1
    tasks = [(h, r) for h in heads for r in causal_row_ranges(wl.L, parts)]

    def task(hr):
        h, r = hr
        if wl.backward:
            return oracle.attn_bwd_head(q[0, :, h], k[0, :, h], v[0, :, h], do[0, :, h], wl.causal, rows=r)
        return oracle.attn_fwd_head(q[0, :, h], k[0, :, h], v[0, :, h], wl.causal)

    t0 = time.perf_counter()
    res = host_parallel(task, tasks)
    print(f"[{key}] oracle of {len(heads)} heads in {len(tasks)} parts: {time.perf_counter() - t0:.0f} s", flush=True)
    refs = []
    for h in heads:
        mine = [x for (hh, _), x in zip(tasks, res) if hh == h]
        if wl.backward:
            dq_r, dk_r, dv_r, o_r, lse_r = (sum(x[i] for x in mine) for i in range(5))
            refs.append(((("o", o_r), ("dq", dq_r), ("dk", dk_r), ("dv", dv_r)), lse_r))
        else:
            refs.append(((("o", mine[0][0]),), mine[0][1]))
    del res
    for h, (want_all, lse_r) in zip(heads, refs):
        for name, want in want_all:
            st = check_close(f"{name} head {h} {key} (every element)", got[name][0, :, h], want, "bf16")
            print(f"  {name}: max_abs {st['max_abs']:.3e} rel_fro {st['rel_fro']:.3e} "
                  f"max_err_over_allowed {st['max_err_over_allowed']:.3f} n_over_1e-2 {st['n_over_flat']}",
                  flush=True)
        err = float(np.max(np.abs(lse[0, h] - lse_r)))
        print(f"  lse: max_abs {err:.3e}", flush=True)
        assert err <= 1e-3
