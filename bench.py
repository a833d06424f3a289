"""Benchmark of the Ulysses per-rank hot path on one MI355X.

One step = the whole path over one batch of seeded synthetic input, inputs
already resident in HBM:
    seq_to_head on Q, K, V (and dO)          -- full [P][B][L/P][H][d_h] tensors
                                                (K, V: the K/V form, replicating
                                                 K/V heads when P > H_kv)
    attention forward on rank 0's head group  -- [B][L][H/P][d_h], causal
    attention backward (workloads with a backward pass)
    head_to_seq on O (and dQ, dK, dV)         -- full head buffers (dK, dV: the
                                                gradient form, summing replicas)
Prints ONE JSON line. `value` is attention fwd(+bwd) algorithmic TFLOP/s over
the whole step time (transposes included); per-op figures come from HIP
events recorded on the launch stream around every call in the timed steps,
and `detail.sclk` is the graphics clock the host read (amdsmi) meanwhile.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Warm-up: W untimed steps when --warmup is given; by default as many steps as
fill --warmup-seconds (1 s, at least 3 steps), so that short steps are timed
at the clocks the GPU holds under sustained load rather than while it ramps
up from idle (measured on the 32K forward-only workload: 0.67 ms per forward
after 3 warm-up steps, 0.58 ms after 600). The line's "warmup" is the count
run.
    python bench.py --gemm-ceiling      # vendor bf16 GEMM rate, for context

HBM traffic of the dominant op (roofline "traffic"): two rocprofv3 counter
runs of this script with --calibration-copy, one collecting FETCH_SIZE and
one WRITE_SIZE, are reduced with --summarize-traffic into
profiles/hbm_traffic_<workload>.json; the counters are scaled by what they
read for a device copy of known size. The summary carries a hash of the
kernel sources and is used only while the sources still match it.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attn fwd+bwd TFLOP/s (% MFMA peak) + seq<->head transpose GB/s, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X dense fp32 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E


CALIB_BYTES = 1 << 30   # device copy of known size for counter calibration


def kernel_sources_hash() -> str:
    """sha256 over the HIP sources and build script (the counters belong to one build)."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "exact_attention_ulysses_amd")
    for f in sorted(glob.glob(os.path.join(pkg, "csrc", "*"))) + [os.path.join(pkg, "build.py")]:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")


OP_KERNELS = {"attn_fwd": ("attn_fwd_bf16_kernel",),
              "attn_bwd": ("bwd_delta_kernel", "bwd_dkdv_bf16_kernel", "bwd_dq_bf16_kernel"),
              "perm": ("perm_kernel",)}


def summarize_traffic(workload: str, fetch_dir: str, write_dir: str, cmd_fetch: str, cmd_write: str) -> None:
    """Reduce two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) to per-op bytes."""
    import csv

    def per_kernel(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return vals

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy_f = [v for k, vs in fetch.items() if "copyBuffer" in k for v in vs]
    copy_w = [v for k, vs in write.items() if "copyBuffer" in k for v in vs]
    if not copy_f or not copy_w:
        raise SystemExit("no calibration copy found in the counter runs (use --calibration-copy)")
    fscale, wscale = CALIB_BYTES / max(copy_f), CALIB_BYTES / max(copy_w)

    def avg(vals, names):
        out = 0.0
        for n in names:
            hits = [sum(v) / len(v) for k, v in vals.items() if n in k]
            out += hits[0] if hits else 0.0
        return out

    ops = {op: {"read_bytes": avg(fetch, ks) * fscale, "write_bytes": avg(write, ks) * wscale}
           for op, ks in OP_KERNELS.items()}
    res = {"workload": workload, "kernel_sources_sha256": kernel_sources_hash(),
           "fetch_scale": fscale, "write_scale": wscale, "per_launch": ops,
           "commands": [cmd_fetch, cmd_write]}
    with open(traffic_path(workload), "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


def load_traffic(workload: str, op: str):
    """HBM bytes per launch of `op` from the committed summary, or None if absent or stale."""
    try:
        with open(traffic_path(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sources_sha256") != kernel_sources_hash():
        return None
    b = t["per_launch"][op]
    return b["read_bytes"] + b["write_bytes"]


class ClockSampler:
    """Samples the graphics clock of one GPU from the host (amdsmi) while the timed
    steps run: the clock the chip holds under the load sets the MFMA rate, and it
    differs from box to box. Failure to sample is reported, never fatal."""

    def __init__(self, props, period_s: float = 0.02):
        import threading
        self.samples, self.error, self.period = [], None, period_s
        self._stop = threading.Event()
        self._thread = None
        self._h = None
        self._smi = None
        try:
            import amdsmi
            amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
            self._smi = amdsmi
            want = (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
            for h in amdsmi.amdsmi_get_processor_handles():
                dom, bus, rest = amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self._h = h
            if self._h is None:
                self.error = f"no amdsmi device at PCI {want}"
        except Exception as e:  # noqa: BLE001  (reported in the JSON line)
            self.error = repr(e)

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(float(self._smi.amdsmi_get_clock_info(self._h, self._smi.AmdSmiClkType.SYS)["clk"]))
            except Exception as e:  # noqa: BLE001
                self.error = repr(e)
                return
            self._stop.wait(self.period)

    def start(self):
        import threading
        if self._h is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self) -> dict:
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        if self._smi is not None:
            try:
                self._smi.amdsmi_shut_down()
            except Exception:  # noqa: BLE001  (the samples are already taken)
                pass
            self._smi = None
        if not self.samples:
            return {"error": self.error or "no samples"}
        n = len(self.samples)
        return {"mean_MHz": sum(self.samples) / n, "min_MHz": min(self.samples), "max_MHz": max(self.samples),
                "samples": n,
                "source": f"amdsmi graphics clock, sampled every {self.period * 1e3:.0f} ms by the host during the timed steps"}


def npairs(L: int, causal: bool, Lk: int = 0) -> int:
    """Visible (query, key) pairs of one head: causal self-attention or all L x Lk."""
    return L * (L + 1) // 2 if causal else L * (Lk or L)


def npairs_layout(layout, block: int, L: int, causal: bool) -> int:
    """Visible (query, key) pairs summed over the heads of a block layout [H][nb][nb]."""
    import numpy as np
    nb = layout.shape[1]
    size = np.minimum(block, L - block * np.arange(nb))          # tokens per block
    full = np.outer(size, size)
    if causal:
        w = np.tril(full, -1) + np.diag(size * (size + 1) // 2)
    else:
        w = full
    return int(sum(int((w * (lay != 0)).sum()) for lay in layout))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: as many as fill --warmup-seconds, at least 3)")
    ap.add_argument("--warmup-seconds", type=float, default=1.0)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=65536,
                    help="prefix length of one head that the fp64 oracle runs fwd+bwd on")
    ap.add_argument("--cold-reps", type=int, default=3,
                    help="repetitions of each layout change timed after a cache-evicting write")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration for rocprofv3 runs)")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="time the vendor bf16 GEMM (torch.matmul) on random and constant operands instead")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CMD_FETCH", "CMD_WRITE"),
                    help="reduce two rocprofv3 counter runs to profiles/hbm_traffic_<workload>.json")
    return ap.parse_args()


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, prefix_host, layout=None):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload.

    prefix_host holds the raw bits of the first T tokens of each input (B = 1:
    the first T token rows of the global [L][H][d_h] tensor are the seq
    buffer of the same problem at length T). The oracle runs its own
    seq_to_head over all P ranks of that T-token problem, then attention
    forward (and backward) of head 0 of rank 0 over the T tokens. Its rates
    also give an extrapolated time for the whole step at full size: attention
    work grows as the visible pairs, the layout changes as the bytes.
    """
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = None
    cores = len(os.sched_getaffinity(0))
    B, d, P = wl.B, wl.d, wl.P
    assert B == 1
    T = prefix_host["q"].size // (wl.H * d)
    Tk = prefix_host["k"].size // (wl.Hk * d)
    t0 = time.perf_counter()
    heads, perm_bytes = {}, 0
    for n, x in prefix_host.items():
        if n in ("k", "v"):
            xh = oracle.seq_to_head_kv(x, B, Tk, wl.Hk, d, P)
        else:
            xh = oracle.seq_to_head(x, B, T, wl.H, d, P)
        perm_bytes += x.nbytes + xh.nbytes      # read once, written once
        heads[n] = xh[0]
    t_perm = time.perf_counter() - t0
    f = {n: oracle.to_f64(heads[n][0, :, 0], wl.dtype) for n in heads}
    t0 = time.perf_counter()
    gemms = 6 if wl.backward else 2          # the oracle's products: S, PV (+ dP, dV, dQ, dK), no recompute
    if layout is not None:    # block-sparse: the layout of head 0 over the sampled prefix
        nbs = -(-T // wl.block)
        lay = layout[0, :nbs, :nbs]
        if wl.backward:
            oracle.attn_bwd_block_sparse_head(f["q"], f["k"], f["v"], f["do"], lay, wl.block, wl.causal)
        else:
            oracle.attn_fwd_block_sparse_head(f["q"], f["k"], f["v"], lay, wl.block, wl.causal)
        pairs = npairs_layout(lay[None], wl.block, T, wl.causal)
        full_pairs = None
    else:
        if wl.backward:
            oracle.attn_bwd_head(f["q"], f["k"], f["v"], f["do"], wl.causal)
        else:
            oracle.attn_fwd_head(f["q"], f["k"], f["v"], wl.causal)
        pairs = npairs(T, wl.causal, Tk)
        full_pairs = wl.B * wl.Hp * npairs(wl.L, wl.causal, wl.Lk)
    t_attn = time.perf_counter() - t0
    flops = 2 * gemms * d * pairs
    rate = flops / t_attn
    perm_rate = perm_bytes / t_perm
    out = {"value": rate / 1e12, "unit": "TFLOP/s", "cores": threads if threads else cores,
           "host_cores_visible": cores, "cpu_model": _cpu_model(), "kind": "oracle",
           "sample": (f"fp64 numpy oracle: seq_to_head over all {P} ranks of the first {T} tokens of "
                      f"{len(prefix_host)} inputs ({t_perm:.1f} s), then attention "
                      f"{'fwd+bwd' if wl.backward else 'fwd'} of head 0 of rank 0 over those {T} tokens "
                      f"({t_attn:.1f} s)"),
           "flops_counted": f"{2 * gemms}*d_h*Npairs (the oracle's {gemms} products, no recompute)",
           "attn_s": t_attn, "perm_s": t_perm, "perm_GBps": perm_rate / 1e9}
    if full_pairs is not None:
        n_perm = 2 * len(prefix_host)       # every input in, every output back
        full_perm_bytes = n_perm * 2 * wl.tensor_bytes
        est = 2 * gemms * d * full_pairs / rate + full_perm_bytes / perm_rate
        out["extrapolated_full_s"] = est
        out["extrapolated_full_note"] = (f"extrapolated, not run: one step at full size ({wl.L} tokens, "
                                         f"{wl.B * wl.Hp} heads, {n_perm} layout changes of "
                                         f"{wl.tensor_bytes / 1e9:.2f} GB) at the sampled rates")
    return out


def gemm_ceiling() -> None:
    """bf16 GEMM rate of the vendor library (torch.matmul -> hipBLASLt) on seeded
    N(0,1) operands and on all-ones operands: a practical MFMA ceiling for this
    chip under its power limit (random bits toggle more and lower the clock),
    printed as one JSON line beside the published dense peak."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    res = []
    for n in (8192, 16384):
        for kind in ("randn", "ones"):
            if kind == "randn":
                a = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
                b = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
            else:
                a = torch.ones((n, n), device=dev, dtype=torch.bfloat16)
                b = torch.ones((n, n), device=dev, dtype=torch.bfloat16)
            c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
            for _ in range(3):
                torch.matmul(a, b, out=c)
            torch.cuda.synchronize()
            reps = 20 if n == 8192 else 5
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                torch.matmul(a, b, out=c)
            e1.record()
            e1.synchronize()
            ms = e0.elapsed_time(e1) / reps
            res.append({"m_n_k": n, "operands": kind, "ms": ms, "TFLOPs": 2 * n ** 3 / ms / 1e9,
                        "frac_peak": 2 * n ** 3 / ms / 1e9 / PEAK_BF16_TFLOPS})
            del a, b, c
    print(json.dumps({"gemm_ceiling": res, "peak_TFLOPs": PEAK_BF16_TFLOPS, "dtype": "bf16"}))


def main():
    args = parse()
    if args.gemm_ceiling:
        gemm_ceiling()
        return
    if args.summarize_traffic:
        from workloads import HEADLINE
        summarize_traffic(args.workload or HEADLINE, *args.summarize_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the exchange between GPUs is not "
              "implemented", file=sys.stderr)
        sys.exit(2)
    import torch

    import exact_attention_ulysses_amd as U
    from workloads import HEADLINE, WORKLOADS, block_layout, device_tensor

    wl = WORKLOADS[args.workload or HEADLINE]
    B, L, H, d, P, Hh, causal = wl.B, wl.L, wl.H, wl.d, wl.P, wl.Hp, wl.causal
    Lk, Hk = wl.Lk, wl.Hk
    rep = P * wl.Hkp // Hk      # ranks holding each K/V head
    assert wl.dtype == "bf16", "bench.py measures the bf16 path"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    U.lib()

    ins = ["q", "k", "v"] + (["do"] if wl.backward else [])
    outs = ["o"] + (["dq", "dk", "dv"] if wl.backward else [])
    kv = lambda n: n in ("k", "v", "dk", "dv")  # noqa: E731  (K/V-side tensors)
    seq = {n: device_tensor(wl, n, dev) for n in ins}
    head = {n: torch.empty(wl.shape_of("fill_d" + n if kv(n) else "fill_o"), dtype=torch.bfloat16, device=dev)
            for n in ins}
    # output head buffers: rank 0's block is written by attention, the other blocks hold seeded filler
    ohead = {n: device_tensor(wl, "fill_" + n, dev) for n in outs}
    oseq = {n: torch.empty(wl.shape_of(n[1:] if kv(n) else "q"), dtype=torch.bfloat16, device=dev) for n in outs}
    lse = torch.empty((B, Hh, L), dtype=torch.float32, device=dev)
    ws_bytes = (U.ulysses_attn_bwd_block_sparse_workspace_bytes(B, L, H, Hk, d, P, causal) if wl.block
                else U.ulysses_attn_bwd_gqa_workspace_bytes(B, L, Lk, H, Hk, d, P, causal))
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    # block-sparse workloads: rank 0's seeded block layout
    layout_host = block_layout(wl, heads=range(Hh)) if wl.block else None
    layout = torch.from_numpy(layout_host).to(dev) if wl.block else None
    r0 = {n: head[n][0] for n in ins}
    o0 = {n: ohead[n][0] for n in outs}
    stream = torch.cuda.current_stream()

    ops = []  # (name, callable, HBM bytes read + written)
    tq, tk = B * L * H * d * 2, B * Lk * Hk * d * 2     # seq-layout tensor bytes, query side and K/V side
    for n in ins:
        if kv(n):
            ops.append(("seq_to_head", lambda n=n: U.ulysses_seq_to_head_kv(seq[n], head[n], B, Lk, Hk, d, P),
                        tk * (1 + rep)))
        else:
            ops.append(("seq_to_head", lambda n=n: U.ulysses_seq_to_head(seq[n], head[n], B, L, H, d, P), 2 * tq))
    if wl.block:
        ops.append(("attn_fwd", lambda: U.ulysses_attn_fwd_block_sparse(r0["q"], r0["k"], r0["v"], o0["o"], lse,
                                                                        layout, B, L, H, Hk, d, P, causal), 0))
    else:
        ops.append(("attn_fwd", lambda: U.ulysses_attn_fwd_gqa(r0["q"], r0["k"], r0["v"], o0["o"], lse, B, L, Lk,
                                                               H, Hk, d, P, causal), 0))
    if wl.backward and wl.block:
        ops.append(("attn_bwd", lambda: U.ulysses_attn_bwd_block_sparse(
            r0["q"], r0["k"], r0["v"], o0["o"], r0["do"], lse, o0["dq"], o0["dk"], o0["dv"], layout, ws, B, L, H, Hk,
            d, P, causal), 0))
    elif wl.backward:
        ops.append(("attn_bwd", lambda: U.ulysses_attn_bwd_gqa(r0["q"], r0["k"], r0["v"], o0["o"], r0["do"], lse,
                                                               o0["dq"], o0["dk"], o0["dv"], ws, B, L, Lk, H, Hk,
                                                               d, P, causal), 0))
    for n in outs:
        if kv(n):
            ops.append(("head_to_seq", lambda n=n: U.ulysses_head_to_seq_kv_grad(ohead[n], oseq[n], B, Lk, Hk, d,
                                                                                  P), tk * (1 + rep)))
        else:
            ops.append(("head_to_seq", lambda n=n: U.ulysses_head_to_seq(ohead[n], oseq[n], B, L, H, d, P), 2 * tq))

    def step(events=None):
        for i, (_, fn, _) in enumerate(ops):
            if events is not None:
                events[i][0].record(stream)
            fn()
            if events is not None:
                events[i][1].record(stream)

    if args.warmup is not None:
        for _ in range(args.warmup):
            step()
        warmup_steps = args.warmup
    else:
        # whole steps until --warmup-seconds of them have run (at least 3),
        # the host waiting for the GPU every 4 steps to read the clock
        warmup_steps = 0
        w0 = time.perf_counter()
        while True:
            step()
            warmup_steps += 1
            if warmup_steps % 4 == 3:
                torch.cuda.synchronize()
                if time.perf_counter() - w0 >= args.warmup_seconds or warmup_steps >= 100000:
                    break
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ops]
           for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    clocks = ClockSampler(torch.cuda.get_device_properties(dev))
    torch.cuda.synchronize()
    clocks.start()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        step(evs[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    sclk = clocks.stop()
    ms_step = t_start.elapsed_time(t_end) / args.steps

    per_op = {}
    for s in range(args.steps):
        for i, (name, _, _) in enumerate(ops):
            per_op.setdefault(name, []).append(evs[s][i][0].elapsed_time(evs[s][i][1]))
    avg = {k: sum(v) / len(v) for k, v in per_op.items()}       # ms per launch of that op

    # visible (query, key) pairs over the rank's heads
    npr_heads = (B * npairs_layout(layout_host, wl.block, L, causal) if wl.block
                 else B * Hh * npairs(L, causal, Lk))
    fwd_flops = 4 * d * npr_heads
    bwd_flops = 10 * d * npr_heads
    attn_flops = fwd_flops + (bwd_flops if wl.backward else 0)
    perm_ms = sum(v for k, vs in per_op.items() if k in ("seq_to_head", "head_to_seq") for v in vs) / args.steps
    perm_bytes = sum(b for name, _, b in ops if name in ("seq_to_head", "head_to_seq"))
    attn_ms = avg["attn_fwd"] + (avg.get("attn_bwd", 0.0))
    value = attn_flops / (ms_step * 1e-3) / 1e12

    # dominant op: largest share of the step
    dom = max(("attn_fwd", "attn_bwd") if wl.backward else ("attn_fwd",), key=lambda k: avg[k])
    dom_flops = bwd_flops if dom == "attn_bwd" else fwd_flops
    achieved = dom_flops / (avg[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": ("ulysses_attn_bwd (delta, dK/dV and dQ launches)" if dom == "attn_bwd"
                                            else "ulysses_attn_fwd"),
                "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": load_traffic(wl.key, dom),
                "per_launch": {"flops": dom_flops, "ms": avg[dom]}}

    detail = {
        "attn_fwd_ms": avg["attn_fwd"], "attn_fwd_TFLOPs": fwd_flops / (avg["attn_fwd"] * 1e-3) / 1e12,
        "attn_fwd_bwd_TFLOPs": attn_flops / (attn_ms * 1e-3) / 1e12,
        "attn_fwd_bwd_frac_peak": attn_flops / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "attn_12dN_TFLOPs": (12 if wl.backward else 4) * d * npr_heads / (attn_ms * 1e-3) / 1e12,
        "seq_to_head_ms": avg["seq_to_head"], "head_to_seq_ms": avg["head_to_seq"],
        "transpose_GBps": perm_bytes / (perm_ms * 1e-3) / 1e9,
        "transpose_frac_peak": perm_bytes / (perm_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "wall_s_timed_region": wall,
        "sclk": sclk,
    }
    if wl.backward:
        detail.update({"attn_bwd_ms": avg["attn_bwd"],
                       "attn_bwd_TFLOPs": bwd_flops / (avg["attn_bwd"] * 1e-3) / 1e12})

    # Layout changes timed cold: a 1 GiB write before every repetition evicts
    # the 256 MB last-level cache (and the L2) so no tensor is timed from
    # cache; the write is outside the events.
    evict = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = {}
    for name, fn, nbytes in ops:
        if name not in ("seq_to_head", "head_to_seq"):
            continue
        for _ in range(args.cold_reps):
            evict.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            cold.setdefault(name, []).append((e0.elapsed_time(e1), nbytes))
    del evict
    cold_ms = {k: sum(t for t, _ in v) / len(v) for k, v in cold.items()}
    cold_gbps = {k: sum(b for _, b in v) / (sum(t for t, _ in v) * 1e-3) / 1e9 for k, v in cold.items()}
    all_cold = [x for v in cold.values() for x in v]
    detail.update({"seq_to_head_ms_cold": cold_ms.get("seq_to_head"), "head_to_seq_ms_cold": cold_ms.get("head_to_seq"),
                   "seq_to_head_GBps_cold": cold_gbps.get("seq_to_head"),
                   "head_to_seq_GBps_cold": cold_gbps.get("head_to_seq"),
                   "transpose_GBps_cold": sum(b for _, b in all_cold) / (sum(t for t, _ in all_cold) * 1e-3) / 1e9,
                   "transpose_cold_note": f"{args.cold_reps} reps of every layout change, each after a 1 GiB "
                                          "cache-evicting write outside the events"})
    detail["transpose_frac_peak_cold"] = detail["transpose_GBps_cold"] / PEAK_HBM_GBPS
    for nm in ("seq_to_head", "head_to_seq"):     # in the timed steps: bytes per step over time per step
        detail[nm + "_GBps"] = (sum(b for n_, _, b in ops if n_ == nm) / 1e9
                                / (sum(per_op[nm]) / args.steps * 1e-3)) if nm in per_op else None

    if args.calibration_copy:
        src = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        # only the sampled prefix crosses to the host: the first T tokens (a
        # multiple of P) of every input
        T = max(P, min(args.cpu_sample_tokens, L) // P * P)
        Tk = max(P, min(args.cpu_sample_tokens, Lk) // P * P)
        host = {n: seq[n].view(-1)[:(Tk * Hk if kv(n) else T * H) * d].view(torch.int16).cpu().numpy().view("uint16")
                for n in ins}
        cpu = cpu_baseline(wl, host, layout_host)

    metric = METRIC if wl.key == HEADLINE else METRIC.replace(
        "causal attn", ("causal" if causal else "bidirectional") + (" block-sparse" if wl.block else "")
        + (" grouped-query" if Hk != H else "") + (" cross-" if Lk != L else " ") + "attn")
    line = {
        "metric": metric, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": warmup_steps, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded, device-generated)",
        "config": {"workload": wl.key, "B": B, "L": L, "H": H, "d_h": d, "P": P, "local_heads": Hh,
                   "causal": causal, "backward": wl.backward, "parallelism": "1 GPU, P virtual ranks",
                   **({"L_kv": Lk} if Lk != L else {}), **({"H_kv": Hk, "local_kv_heads": wl.Hkp}
                                                          if Hk != H else {}),
                   **({"block": wl.block, "window": wl.window, "global_blocks": wl.n_global,
                       "random_blocks": wl.n_random, "visible_pairs": npr_heads} if wl.block else {})},
        "roofline": roofline, "cpu_baseline": cpu, "detail": detail,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
