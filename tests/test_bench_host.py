"""Host-side logic of bench.py (no GPU needed): the flop counts behind the
reported TFLOP/s, the guard that drops stale HBM traffic figures, the
refusal of multi-GPU runs and the clock sampler's fallback."""
import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("L,Lk,causal", [(1, 0, True), (7, 0, True), (300, 0, True), (300, 0, False),
                                          (17, 40, False)])
def test_pair_counts_by_brute_force(bench, L, Lk, causal):
    keys = Lk or L
    mask = np.tril(np.ones((L, keys), bool)) if causal else np.ones((L, keys), bool)
    assert bench.npairs(L, causal, Lk) == int(mask.sum())


@pytest.mark.parametrize("L,causal", [(1000, True), (1000, False), (128, True), (129, True)])
def test_layout_pair_counts_by_brute_force(bench, L, causal):
    block = 128
    nb = -(-L // block)
    rng = np.random.default_rng(L)
    layout = (rng.random((3, nb, nb)) < 0.5).astype(np.uint8)
    want = 0
    for lay in layout:
        vis = np.kron(lay, np.ones((block, block), np.uint8))[:L, :L].astype(bool)
        if causal:
            vis &= np.tri(L, dtype=bool)
        want += int(vis.sum())
    assert bench.npairs_layout(layout, block, L, causal) == want


def test_traffic_figures_need_matching_sources(bench, tmp_path, monkeypatch):
    """A committed traffic summary counts only while its source hash matches."""
    monkeypatch.setattr(bench, "traffic_path", lambda w: str(tmp_path / f"t_{w}.json"))
    rec = {"kernel_sources_sha256": bench.kernel_sources_hash(),
           "per_launch": {"attn_bwd": {"read_bytes": 3.0, "write_bytes": 4.0}}}
    (tmp_path / "t_w.json").write_text(json.dumps(rec))
    assert bench.load_traffic("w", "attn_bwd") == 7.0
    rec["kernel_sources_sha256"] = "0" * 64
    (tmp_path / "t_w.json").write_text(json.dumps(rec))
    assert bench.load_traffic("w", "attn_bwd") is None
    assert bench.load_traffic("absent", "attn_bwd") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


@pytest.mark.parametrize("backward", [True, False])
def test_cpu_baseline_on_a_prefix(bench, backward):
    """The oracle leg runs on the first T tokens only; it counts the oracle's own
    products (6 with a backward pass, 2 without) and extrapolates a full step."""
    from workloads import custom, host_tensor
    wl = custom(1, 512, 8, 64, 4, dtype="bf16", backward=backward, index=950)
    T = 128
    names = ["q", "k", "v"] + (["do"] if backward else [])
    prefix = {n: host_tensor(wl, n).reshape(-1)[:T * wl.H * wl.d] for n in names}
    r = bench.cpu_baseline(wl, prefix)
    gemms = 6 if backward else 2
    flops = 2 * gemms * wl.d * T * (T + 1) // 2
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] == pytest.approx(flops / r["attn_s"] / 1e12)
    assert f"first {T} tokens" in r["sample"]
    perm_bytes = 2 * len(names) * T * wl.H * wl.d * 2
    assert r["perm_GBps"] == pytest.approx(perm_bytes / r["perm_s"] / 1e9)
    full = 2 * gemms * wl.d * wl.Hp * wl.L * (wl.L + 1) // 2 / (flops / r["attn_s"]) \
        + 2 * len(names) * 2 * wl.tensor_bytes / (perm_bytes / r["perm_s"])
    assert r["extrapolated_full_s"] == pytest.approx(full)
    assert "extrapolated" in r["extrapolated_full_note"]


def test_clock_sampler_reports_instead_of_failing(bench):
    """Where amdsmi cannot reach the GPU (no device, or no device at that PCI
    address) the clock sampler reports why in the JSON line; the bench goes on."""
    import types
    props = types.SimpleNamespace(pci_domain_id=0xFFFF, pci_bus_id=0xFF, pci_device_id=0x1F)
    c = bench.ClockSampler(props)
    c.start()
    out = c.stop()
    assert set(out) == {"error"} and out["error"]
