"""Host-side logic of bench.py (CPU): which kernels make up a step in the committed profile
summaries, and the single-GPU contract."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("key,workload,want", [
    # Large, fp32 storage: step 1, the schedule, the shared-row aggregate without the envelope
    ("e2f::k_eaas<2, 4, float, true>", "large", True),
    ("e2f::k_sched_count", "large", True),
    ("e2f::k_aggregate_mt<2, 4, 1, 2, false>", "large", True),
    ("e2f::k_aggregate_mt<2, 3, 2, 2, false>", "large", True),
    ("e2f::k_aggregate_mt<2, 3, 2, 2, true>", "large", False),      # envelope variant
    ("e2f::k_bwd_q_mt<2, 3, 2, 2, false>", "large", False),
    ("e2f::k_proj_eaas<2, float, 128>", "large", False),
    # Scale-out, bf16 storage: the bf16 kernels only, not the backward's fp32 recompute
    ("e2f::k_eaas<2, 8, unsigned short, true>", "scaleout", True),
    ("e2f::k_aggregate<2, 8, unsigned short, 1, 1, true, false, true>", "scaleout", True),
    ("e2f::k_aggregate<2, 8, unsigned short, 1, 1, true, true, true>", "scaleout", False),
    ("e2f::k_eaas<2, 4, float, true>", "scaleout", False),
    ("e2f::k_aggregate_mt<2, 3, 2, 2, false>", "scaleout", False),
    ("e2f::k_aggregate_mt<2, 4, 1, 2, false>", "scaleout", False),
    ("e2f::k_sched_scatter", "scaleout", True),
    # the EAAS workload: the product alone, without the workspace's query rows
    ("e2f::k_eaas<2, 4, float, false>", "eaas", True),
    ("e2f::k_eaas<2, 4, float, true>", "eaas", False),
])
def test_step_kernels(key, workload, want):
    assert bench.step_kernel(key, workload) is want


@pytest.mark.parametrize("workload", ["large", "scaleout", "eaas"])
def test_committed_summaries_parse(workload):
    """Each committed summary lists per-kernel counters, and its step kernels are one storage
    type (when the summary is current)."""
    cc = bench.committed_counters(workload)
    if cc is None:
        pytest.skip("summary older than the kernel sources")
    step = [k for k in cc if bench.step_kernel(k, workload)]
    assert step and all(cc[k]["traffic"] > 0 and cc[k]["avg_ns"] > 0 for k in step)
    if workload == "scaleout":
        assert not any("float" in k for k in step)
    assert bench.committed_step_traffic(workload) == pytest.approx(
        sum(cc[k]["traffic"] for k in step))


def test_more_than_one_gpu_is_refused():
    """One GPU only: --gpus 2 ends with a message before anything touches a device."""
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT,
                         env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert res.returncode != 0
    assert "one GPU" in res.stderr or "--gpus 1" in res.stderr
