"""Host-side checks of bench.py (no GPU): the one-GPU contract, the
algorithmic byte counts behind the GB/s figures, and the CPU-baseline
object's fields."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from workloads import WORKLOADS, make_inputs, small_workload  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                       env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_memory_kernel_bytes_follow_the_per_token_formulas():
    T, d, k, s = 32768, 2048, 8, 2
    assert bench.mem_bytes("permute", T, d, k, s) == T * ((1 + k) * d * s + 4 * k)
    assert bench.mem_bytes("combine", T, d, k, s) == T * ((k + 1) * d * s + 8 * k)
    assert bench.mem_bytes("combine_bwd", T, d, k, s) == T * ((1 + 2 * k) * d * s + 12 * k)
    assert bench.mem_bytes("permute_bwd", T, d, k, s) == T * ((k + 1) * d * s + 4 * k)
    # the router's fp32 dx joins the un-permute backward's reads
    assert bench.mem_bytes("permute_bwd", T, d, k, s, router=True) == T * ((k + 1) * d * s + 4 * k + 4 * d)
    # the 32k EP-share step moves 5.91 GB through the four kernels
    total = sum(bench.mem_bytes(n, T, d, k, s) for n in bench.MEM_KERNELS)
    assert abs(total - 5.91e9) < 0.01e9


def test_gemm_flop_units_sum_to_the_layer_count():
    fwd = bench.GEMM_KERNELS["gg_gateup_fwd"] + bench.GEMM_KERNELS["gg_down_fwd"]
    bwd = sum(bench.GEMM_KERNELS[n] for n in ("gg_down_dgrad", "gg_down_wgrad", "gg_gateup_dgrad",
                                              "gg_gateup_wgrad"))
    assert fwd == 6 and fwd + bwd == 18   # 6 R d F forward, 18 R d F forward+backward
    w = WORKLOADS["ep_share_32k"]
    assert w.flops_fwd_bwd() == 18.0 * w.T * w.k * w.d * w.F
    assert w.flops_fwd() == 6.0 * w.T * w.k * w.d * w.F


def test_measured_traffic_is_tied_to_its_workload():
    assert bench.measured_traffic("gg_gateup_fwd", "large_share_zipf") is None
    assert bench.measured_traffic("no_such_kernel", "ep_share_32k") is None


def test_cpu_baseline_object():
    w = small_workload(96, 64, 4, 2, 64, "bf16", "zipf", seed=81, n_empty=1)
    cb = bench.cpu_baseline(w, make_inputs(w), target_s=0.05)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert "oracle" in cb["sample"] and "96" in cb["sample"]
    cbf = bench.cpu_baseline(w, make_inputs(w), target_s=0.05, fwd_only=True)
    assert "forward of" in cbf["sample"]


def test_route_bytes():
    T, E, k = 32768, 32, 8
    nblk = T // bench.ROUTE_TOKENS
    assert bench.route_bytes("route_topk", T, E, k, nblk) == T * (4 * E + 12 * k) + 4 * nblk * E
    assert bench.route_bytes("route_bwd", T, E, k, nblk) == T * (8 * E + 12 * k)
    assert bench.route_bytes("route_bwd", T, E, k, nblk, renorm=True) == T * (4 * E + 12 * k)
    assert bench.route_bytes("route_rows", T, E, k, nblk) == 16 * T * k + 4 * nblk * E + 8 * E
    assert bench.route_bytes("gg_gateup_fwd", T, E, k, nblk) is None
