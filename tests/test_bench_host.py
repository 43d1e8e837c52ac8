"""bench.py's host logic (no GPU): the algorithmic bytes behind roofline.achieved,
the HBM-traffic figure's source check, and the one-GPU guard."""
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_single_workload():
    cfg = workloads.config("single")
    ctx = 8192
    b = bench.algorithmic_bytes(cfg, ctx)
    # context K and V once: 2 tensors x 8192 keys x 8 KV heads x 128 dims x 2 bytes
    kv = 2 * 8192 * 8 * 128 * 2
    # tree q and out (8 query heads) and tree k, v (8 KV heads): 33 nodes x 128 dims x 2 bytes
    tree = 33 * 128 * 2 * (8 + 8 + 8 + 8)
    assert b["attention"] == kv + tree == 33_824_768
    # every node's target row once: 33 x 163840 bf16 logits
    assert b["vocab"] == 33 * 163840 * 2 == 10_813_440
    assert b["residual"] == 0                      # greedy: no residual row
    assert b["total"] == b["attention"] + b["vocab"]


def test_algorithmic_bytes_sampling_adds_one_residual_row_per_request():
    cfg = workloads.config("batched")
    b = bench.algorithmic_bytes(cfg, 16 * 4096)
    assert b["residual"] == 16 * 163840 * 2
    assert b["vocab"] == 16 * 33 * 163840 * 2
    assert b["attention"] == 2 * 16 * 4096 * 8 * 128 * 2 + 16 * 33 * 128 * 2 * 32


def test_traffic_figure_only_for_the_profiled_source():
    # each committed profile names its workload and the attention source it was measured on
    for name in ("tiny", "single", "batched", "long", "ragged"):
        path = bench.traffic_profile(name)
        if not os.path.exists(path):
            assert bench.measured_traffic(name) is None
            continue
        prof = open(path).read()
        digest = [l.split(":", 1)[1].strip() for l in prof.splitlines()
                  if l.startswith("source_digest:")][0]
        assert ("workload: " + name) in prof
        t = bench.measured_traffic(name)
        if bench.attention_source_digest() == digest:
            assert isinstance(t, int) and t > 0
        else:
            assert t is None
    # no summary file at all: no figure
    assert not os.path.exists(bench.traffic_profile("no_such_workload"))
    assert bench.measured_traffic("no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_cpu_baseline_legs_and_sample_scaling():
    """The CPU baseline: a single-core leg and an all-core leg, the CPU model, and
    a sample whose stage times are scaled to the whole step."""
    cfg = workloads.config("tiny")
    r = bench.run_cpu_baseline(cfg, 0.05)
    assert r["kind"] == "oracle" and r["unit"] == "steps/s" and r["value"] > 0
    assert r["cores"] == len(os.sched_getaffinity(0))
    assert r["single_core"]["cores"] == 1 and r["single_core"]["value"] > 0
    assert isinstance(r["cpu_model"], str) and r["cpu_model"]
    assert "full oracle step" in r["sample"]
    st = r["stage_seconds_per_step"]
    assert abs(sum(st.values()) - 1.0 / r["value"]) <= 1e-4 + 0.01 / r["value"]


def test_subset_inputs_repack_the_contexts():
    import numpy as np
    cfg = workloads.config("ragged", B=5, ctx=(3, 40), V=64, Hq=2, Hkv=2, Dh=64)
    inp = workloads.make_inputs(cfg)
    scfg, sub = bench._subset_inputs(cfg, inp, [0, 1, 2])
    assert scfg.B == 3
    offs = inp["ctx_offsets"]
    assert list(sub["ctx_offsets"]) == [int(x) for x in offs[:4]]
    assert np.array_equal(sub["k_ctx"], inp["k_ctx"][:offs[3]])
    scfg, sub = bench._subset_inputs(cfg, inp, [3])
    assert np.array_equal(sub["v_ctx"], inp["v_ctx"][offs[3]:offs[4]])
    assert np.array_equal(sub["q"], inp["q"][3:4])
