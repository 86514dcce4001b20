"""bench.py without a GPU: the one-GPU guard, the algorithmic counts it
divides by, and the link between the committed HBM-traffic profile and the
kernel sources it was measured on."""
import os
import subprocess
import sys

import pytest

import bench
from synth.workloads import BY_NAME

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_counts_of_the_12M_workload():
    # per token-head: Q, K, V, dO in and O, dQ, dK, dV out at 128 bytes each;
    # forward 4dLP + 2U and backward 8dLP + 4U FLOPs with U = 2 L R (d + 1)
    # (L16, P4: 82,944 + 165,888)
    layer, kernels = bench.per_token_head_counts(BY_NAME["causal_long_n12M"])
    assert layer["bytes"] == 1408
    assert layer["flops"] == 82944 + 165888
    U = 2 * 16 * 16 * 65
    assert U == 33280
    assert kernels["pass_bwd_q"] == (512, 2 * 64 * 16 * 4 + 2 * U)
    assert kernels["pass_bwd_v"] == (256, 2 * U)


def test_committed_traffic_profile_matches_the_sources():
    # the summary's sources sha256 is the digest of the current kernel sources,
    # so bench.py reports its measured bytes for the dominant kernel
    path = os.path.join(ROOT, "profiles", "hbm_traffic_causal_long_n12M.md")
    text = open(path).read()
    digest = [ln.split(":", 1)[1].strip() for ln in text.splitlines() if ln.startswith("sources sha256:")]
    assert len(digest) == 1
    if digest[0] != bench.source_digest():
        pytest.skip("the committed traffic profile predates the current kernel sources (bench.py then "
                    "reports traffic = null)")
    traffic = bench.measured_traffic("causal_long_n12M", "pass_bwd_q")
    assert isinstance(traffic, int) and traffic > 24.58e9   # at least the algorithmic bytes
