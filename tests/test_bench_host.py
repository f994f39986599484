"""CPU checks of bench.py's host logic: the one-GPU guard, the work models
behind the roofline figures (against their definitions written out here on
small shapes), and the JSON contract's static fields."""
import os
import subprocess
import sys

import pytest

import bench
from post_weight_quantization_hessian_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


class _WL:
    bits = (4, 3)
    group_size = 128


def test_chmc_flops_match_their_definition():
    # lazy update of block b (at j0): rows x j0 x bw multiply-adds; in-block
    # propagation rows x bw (bw - 1) / 2; per bit width
    plan = [bench.HPlan("x", 300, 100, 37), bench.HPlan("y", 128, 100, 5)]
    upd = sum(2.0 * h.rows * j0 * min(128, h.dim - j0) for h in plan
              for j0 in range(0, h.dim, 128)) * 2
    inb = sum(2.0 * h.rows * min(128, h.dim - j0) * (min(128, h.dim - j0) - 1) / 2
              for h in plan for j0 in range(0, h.dim, 128)) * 2
    assert bench.kernel_work("chmc_update", _WL, plan)[:2] == (upd, "flop")
    assert bench.kernel_work("chmc_sweep", _WL, plan)[:2] == (inb, "flop")
    assert bench.kernel_work("chmc_sweep", _WL, plan)[2] == "f64_vec"


def test_hessian_work_is_the_symmetric_half():
    plan = [bench.HPlan("x", 896, 2048, 10, split8=False),
            bench.HPlan("y", 4864, 2048, 10, split8=True)]
    assert bench.kernel_work("hessian_tile", _WL, plan)[0] == 2048 * 896 * 897
    assert bench.kernel_work("hessian_split8", _WL, plan)[0] == 13 * 2048 * 4864 * 4865
    assert bench.kernel_work("fill", _WL, plan)[0] is None


def test_default_workload_and_peaks():
    wl = W.WORKLOADS[bench.DEFAULT_WORKLOAD] if hasattr(W, "WORKLOADS") else None
    # the largest single-GPU workload: the 70B-shape down projection
    assert bench.DEFAULT_WORKLOAD == "llama70b_down"
    assert bench.PEAK["hbm_gbs"] == 8000.0
    assert bench.PEAK["f64_mfma"] == 78.6 and bench.PEAK["f32_mfma"] == 157.3
    assert bench.PEAK["i8_mfma"] == 5000.0 and bench.PEAK["bf16_mfma"] == 2500.0
    if wl is not None:
        assert wl.weights_per_step() == 8192 * 28672 * 2  # 2-bit and 4-bit
        sizes = {n: sum(l.rows * w.input(l.hessian).dim for l in w.layers)
                 for n, w in W.WORKLOADS.items()}
        assert max(sizes, key=sizes.get) == bench.DEFAULT_WORKLOAD
