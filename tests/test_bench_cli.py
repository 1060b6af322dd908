"""bench.py's command line without a GPU: more than one GPU is refused with a
message (the path runs on one GPU), before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


SAMPLE_ROCMINFO = """
*******
Agent 1
*******
  Name:                    Intel(R) Xeon(R) Platinum
  Marketing Name:          Intel(R) Xeon(R) Platinum
  Device Type:             CPU
  Max Clock Freq. (MHz):   3800
  Compute Unit:            96
*******
Agent 2
*******
  Name:                    gfx950
  Marketing Name:          AMD Instinct MI355X
  Device Type:             GPU
  Cache Info:
    L2:                      4096(0x1000) KB
  Max Clock Freq. (MHz):   2400
  Compute Unit:            256
  SIMDs per CU:            4
  ISA Info:
    ISA 1
      Name:                    amdgcn-amd-amdhsa--gfx950:sramecc+:xnack-
"""


def test_peak_from_rocminfo():
    """The bf16 peak is CUs x max engine clock x 4096 FLOP/clk/CU of the GPU
    agent (the CPU agent and the nested ISA name are skipped)."""
    sys.path.insert(0, ROOT)
    import bench
    assert bench.parse_rocminfo(SAMPLE_ROCMINFO) == (256, 2400, "gfx950")
    assert bench.parse_rocminfo("no agents here") is None
    cu, mhz, _ = bench.parse_rocminfo(SAMPLE_ROCMINFO)
    assert abs(cu * mhz * 1e6 * bench.FLOP_PER_CLK_CU["bf16"] / 1e12 - 2516.58) < 0.01


def test_cpu_baseline_fields():
    """The oracle timed beside the bench line (tiny workload, short budget): its
    rate, the threads it used, the host, and the one-thread per-core figure; the
    one-thread run leaves the oracle's default thread count as it was."""
    sys.path.insert(0, ROOT)
    import bench
    import oracle
    import workloads as W
    w = W.WORKLOADS["tiny_f32"]
    q, k, v, mask = W.make_inputs(w)
    n0 = oracle.max_threads()
    cb = bench.cpu_baseline(w, q, k, v, mask, 0.2)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0
    assert cb["cores"] == n0 == oracle.max_threads()
    assert cb["nproc"] >= 1 and "query rows" in cb["sample"]
    assert cb["one_thread"]["value"] > 0 and cb["one_thread"]["unit"] == "TFLOP/s"


def test_traffic_summaries_match_the_current_sources():
    """Each committed counter summary (profiles/attn_traffic_*.json) was taken on the
    current sources of its kernel family, so bench.py reports its traffic figure;
    a kernel edit without new counters fails here instead of turning the figure
    into null."""
    import glob
    import json
    sys.path.insert(0, ROOT)
    import bench
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "attn_traffic_*.json")))
    assert paths
    for p in paths:
        name = os.path.basename(p)[len("attn_traffic_"):-len(".json")]
        family = ("bwd" if name.endswith("_bwd") else "fp8" if name.endswith("_fp8")
                  else "ragged" if name.startswith("ragged") else "fwd")
        rec = json.load(open(p))
        assert rec["kernel_source_hash"] == bench.kernel_source_hash(family), (name, family)
        assert rec["by_config"], name
