"""Host-side logic of bench.py, without a GPU: the algorithmic bytes the
roofline divides by, the rotating-copy rule, the staleness check on the
committed HBM-traffic summaries, and the refusal of more than one GPU."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import bit_weight_amd as bw  # noqa: E402
from bit_weight_amd import synth  # noqa: E402


def test_algorithmic_bytes_of_the_step():
    """Workload 2a (M=1, K=N=4096): packed codes N*K*5/32, alpha 4N, the
    activations (int8 x + s_x, or fp32 x for the fused form) and fp32 y."""
    w = synth.WORKLOADS["2a"]
    assert w.packed_bytes == 4096 * 4096 * 5 // 32 == 2_621_440
    assert bench.algorithmic_bytes(w) == 2_621_440 + 4 * 4096 + (4096 + 4) + 4 * 4096 == 2_658_308
    assert bench.algorithmic_bytes(w, fp32_x=True) == 2_621_440 + 4 * 4096 + 4 * 4096 + 4 * 4096 == 2_670_592
    w5 = synth.WORKLOADS["5"]
    assert w5.packed_bytes == 14336 * 4096 * 5 // 32 == 9_175_040


def test_rotating_copies_exceed_twice_the_last_level_cache():
    assert bench.copies_for(10_240, 0) == 2            # under 1 MiB: not rotated
    assert bench.copies_for(5_000_000, 7) == 7          # an explicit count is kept
    for nb in (2_621_440, 7_045_120, 9_175_040, 36_700_160, 1 << 30):
        R = bench.copies_for(nb, 0)
        assert R >= 2 and R * nb > 2 * bench.MALL_BYTES


def _write_profile(root, kernel, workload, sha, plan, value):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", f"traffic_{kernel}_{workload}.txt"), "w") as f:
        f.write(f"# test summary\nkernel_sources_sha: {sha}\nplan: {bench.plan_tag(plan)}\n"
                f"hbm_bytes_per_launch: {value}\n")


def test_traffic_summary_is_used_only_while_sources_and_plan_match(tmp_path, monkeypatch):
    os.symlink(os.path.join(ROOT, "bit_weight_amd"), tmp_path / "bit_weight_amd")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    plan = bw.plan(1, 4096, 4096)
    sha = bench.kernel_sources_sha("mfma_gemv")
    assert sha == bench.kernel_sources_sha("mfma_gemv") and len(sha) == 16
    assert bench.traffic_from_profile("mfma_gemv", "2a", plan) is None          # no summary
    _write_profile(str(tmp_path), "mfma_gemv", "2a", sha, plan, 3_000_000.0)
    assert bench.traffic_from_profile("mfma_gemv", "2a", plan) == 3_000_000.0
    other = dict(plan, splits=plan["splits"] + 1)
    assert bench.traffic_from_profile("mfma_gemv", "2a", other) is None         # plan changed
    _write_profile(str(tmp_path), "mfma_gemv", "2a", "0" * 16, plan, 3_000_000.0)
    assert bench.traffic_from_profile("mfma_gemv", "2a", plan) is None         # sources changed
    # the hash covers the kernel's own source, not another kernel's
    assert bench.kernel_sources_sha("mfma_gemm") != sha


def test_committed_traffic_summaries_name_their_plan():
    """Every committed summary records the sources' hash, the launch plan and
    a positive byte count (whether it is current is decided at run time)."""
    names = [n for n in os.listdir(os.path.join(ROOT, "profiles")) if n.startswith("traffic_")]
    assert names
    for n in names:
        vals = {}
        for line in open(os.path.join(ROOT, "profiles", n)):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
        assert len(vals.get("kernel_sources_sha", "")) == 16, n
        assert vals.get("plan", "").startswith("grid="), n
        assert float(vals["hbm_bytes_per_launch"]) > 0, n


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_default_workload_is_the_hbm_bound_decode_shape():
    """The headline is the batched decode GEMV at the 70B-class MLP shape
    (M=8, K=8192, N=28672), the HBM-bound decode configuration."""
    assert bench.parse.__code__ is not None
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        args = bench.parse()
    finally:
        sys.argv = old
    assert args.workload == "4"
    w = synth.WORKLOADS[args.workload]
    assert (w.M, w.K, w.N) == (8, 8192, 28672)
    assert w.packed_bytes == 36_700_160
    assert bench.algorithmic_bytes(w) == 36_700_160 + 4 * 28672 + (8 * 8192 + 4 * 8) + 4 * 8 * 28672
    assert set(bench.WORKLOAD_NAMES) == set(synth.WORKLOADS)


def test_host_identity_names_the_cpu():
    h = bench.host_identity()
    assert h["cpu_model"] and h["nproc"] >= 1 and 1 <= h["usable_cpus"] <= h["nproc"]
