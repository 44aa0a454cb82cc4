"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
algorithmic work per launch that the roofline figures divide by."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_moe_layer_rmsnorm_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_replica_work_per_launch_closed_forms():
    s = wl.workload("replica")
    T, d, l, E, k, f, fs, B = s.T, s.d, s.l, s.E, s.k, s.f, s.f_s, s.B
    w = bench.kernel_work(s, T)
    # GEMM FLOPs: two per multiply-add over each product's M x N x K
    assert w["flops"]["gemm_h"] == 2 * T * d * (E + 2 * fs + l) == 77_309_411_328
    assert w["flops"]["gemm_out"] == 2 * T * d * (fs + l)
    assert w["flops"]["expert_up"] == 2 * (T * k) * l * (2 * f)
    assert w["flops"]["expert_down"] == 2 * (T * k) * f * l
    # bytes of the memory-bound steps, as the layer's own data (bf16 activations)
    assert w["bytes"]["rmsnorm"] == 2 * T * d * 2 + 4 * d
    assert w["bytes"]["topk"] == 4 * T * E + 8 * T * k + 4 * E * B
    assert w["bytes"]["combine"] == T * k * l * 2 + 8 * T * k + T * l * 2
    assert w["bytes"]["scan"] + w["bytes"]["scatter"] == 16 * T * k


@pytest.mark.parametrize("name,parts", [("replica", 16), ("decode", 32), ("k3", 8)])
def test_histogram_parts_in_the_implementation_extra(name, parts):
    """The histogram's atomic adds counted apart from the layer's bytes: one
    E x B read-modify-write per token part, with the part count the top-k
    launch uses for that shape."""
    s = wl.workload(name)
    w = bench.kernel_work(s, s.T)
    nchunks = (s.T + 31) // 32
    nsuper = (nchunks + 15) // 16
    assert w["impl_extra"]["topk"] == 8 * parts * s.E * s.B + 4 * nchunks * s.E + 8 * nsuper * s.E
