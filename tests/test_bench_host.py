"""Host logic of bench.py that needs no GPU: the one-GPU refusal, the roofline arithmetic per workload, and the rule
that a committed counter measurement is used only for the kernel source and plan it was taken on."""

import json
import os
import subprocess
import sys

import pytest

import bench
from deterministic_fp32_gemm_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


# Per step: x read once, d_dv read once, d_u read and written once (4 * P * (C^2 + 3*C*hd) bytes), and 2 flops per
# fma of the chain plus the final add (P * (2*C^2*hd + C*hd)); the values written out per workload.
EXPECTED = {2: (524288, 4227072), 3: (3670016, 33816576), 4: (33554432, 538968064), 5: (109051904, 1082130432)}


@pytest.mark.parametrize("key", sorted(EXPECTED))
def test_algorithmic_bytes_and_flops(key):
    w = inputs.WORKLOADS[key]
    assert (w.bytes_per_step, w.flops_per_step) == EXPECTED[key]


def test_every_workload_is_hbm_bound():
    """Arithmetic intensity below the ridge of 157.3 TFLOP/s over 8 TB/s for every timed workload."""
    for key in EXPECTED:
        w = inputs.WORKLOADS[key]
        assert w.flops_per_step / w.bytes_per_step < 157.3e12 / 8.0e12


def test_traffic_is_used_only_for_the_kernel_and_plan_it_was_taken_on(tmp_path, monkeypatch):
    path = os.path.join(ROOT, "profiles", "traffic_gx_mfma_dma_kernel_workload5_fused.json")
    d = json.load(open(path))
    plan = dict(d["plan"])
    got = bench.measured_traffic(5, "fused", plan)
    if d.get("kernel_sha256_16") == bench.kernel_hash():
        assert got == d["hbm_bytes_per_launch"]
    else:
        assert got is None
    other = dict(plan, mf_stages=plan["mf_stages"] + 1)
    assert bench.measured_traffic(5, "fused", other) is None               # another plan
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.measured_traffic(5, "fused", plan) is None                # another kernel source
    assert bench.measured_traffic(4, "per-step", plan) is None             # no measurement for that driver


def test_kernel_hash_ignores_comments_only():
    h = bench.kernel_hash()
    assert len(h) == 16 and h == bench.kernel_hash()


def test_host_cpus():
    cpus, aff, quota, model = bench.host_cpus()
    assert 1 <= cpus <= aff and (quota is None or cpus <= quota)
    assert model is None or isinstance(model, str)
