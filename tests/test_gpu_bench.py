"""bench.py on the GPU, cut short (fixed tile config, 3 steps): one JSON line with
the fields the benchmark contract names, a roofline object for the timed kernel
and numbers that agree with each other."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import ensure_built, say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    ensure_built()
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1", "--no-cpu-baseline",
           *args]
    say("bench", " ".join(args))
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.parametrize("workload,cfg", [("causal_bf16", "256,128,8,2"), ("dense_bf16", "256,128,8,2"),
                                          ("tiny_f32", "64,64,2,1")])
def test_bench_line(workload, cfg):
    res = _bench("--workload", workload, "--config", cfg)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in res, key
    assert res["n_gpus"] == 1 and res["steps"] == 3 and res["warmup"] == 1
    assert res["config"]["workload"] == workload
    assert res["config"]["tile_config"] == [int(x) for x in cfg.split(",")]
    assert res["value"] > 0 and res["ms_per_step"] > 0
    # value is the step's FLOPs over its time
    flops = res["config"]["flops_per_step"]
    assert abs(res["value"] - flops / (res["ms_per_step"] * 1e-3) / 1e12) <= 1e-6 * res["value"]
    rf = res["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    assert abs(rf["achieved"] - flops / (rf["kernel_ms"] * 1e-3) / 1e12) <= 1e-6 * rf["achieved"]
    assert 0 < rf["frac"] < 1
    # the kernel runs inside the (cold) step; warm figures beside the headline
    assert rf["kernel_ms"] <= res["ms_per_step"] * (1 + 1e-6)
    assert res["warm"]["ms_per_step"] > 0 and res["warm"]["kernel_ms"] > 0
    assert "rocminfo" in rf["peak_source"] or "published" in rf["peak_source"]
    # spread of the timed steps: min <= mean, std >= 0
    assert 0 < res["ms_per_step_min"] <= res["ms_per_step"] * (1 + 1e-9) and res["ms_per_step_std"] >= 0
    assert 0 < rf["kernel_ms_min"] <= rf["kernel_ms"] * (1 + 1e-9) and rf["kernel_ms_std"] >= 0


def test_bench_default_workload_is_causal():
    res = _bench("--config", "256,128,8,2")
    assert res["config"]["workload"] == "causal_bf16"
    assert res["config"]["active_blocks"] == 133120


@pytest.mark.parametrize("args,dtype", [(("--workload", "dense_bf16", "--backward"), "bf16"),
                                        (("--workload", "dense_bf16", "--fp8"), "fp8_e4m3"),
                                        (("--workload", "causal_elem_bf16",), "bf16"),
                                        (("--workload", "ragged_bf16",), "bf16")])
def test_bench_other_modes(args, dtype):
    """The backward, fp8, element-mask and ragged-dot lines keep the same contract:
    one JSON line, the contract's fields, a roofline object whose frac is achieved
    over peak, and the traffic figure of the committed counter summary (taken on
    the current sources)."""
    res = _bench(*args)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in res, key
    assert res["n_gpus"] == 1 and res["steps"] == 3 and res["value"] > 0 and res["dtype"] == dtype
    assert res["config"]["workload"].startswith(args[1])
    rf = res["roofline"]
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9 and 0 < rf["frac"] < 1
    assert rf["traffic"] is not None and rf["traffic"] > 0
    assert rf["kernel_ms"] > 0
