"""The kernels' work decomposition, checked on the host (no GPU).

tests/job_maps.cpp includes the library's own index helpers (the header the
kernels use) and runs them over whole launches: the XCD-run job map covers
every (block, head pair) job exactly once for 19,362 launch shapes, the
chunked causal walks number every part of every block exactly once (longest
blocks first) and the reduce kernels' slot formula finds each part where its
work item wrote it, and the multiply-shift division agrees with `/` on 1.6 M
quotients (every divisor up to 4096, random ones up to 2^32 - 1, powers of
two and their neighbours; multiples of each divisor and their neighbours).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="needs hipcc (host-only build)")
def test_job_maps(tmp_path):
    exe = tmp_path / "job_maps"
    cmd = [HIPCC, "-x", "hip", "--offload-host-only", "-std=c++17", "-O2",
           "-I", os.path.join(ROOT, "exact_attention_ulysses_amd", "csrc"),
           os.path.join(ROOT, "tests", "job_maps.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
