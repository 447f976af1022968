"""bench.py contract checks that need no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baselines_report_the_contract_fields():
    """The oracle-timing legs (selector + sparse layers, and the first-generation layout)
    on small workloads: value > 0, unit, the threads used, the kind and the sample."""
    sys.path.insert(0, ROOT)
    import bench
    from workloads.configs import BlockSpec, make_block_inputs
    from workloads.v1 import make_v1_inputs, v1_config

    import numpy as np

    inp = make_block_inputs(BlockSpec("cpu-bl", [3000], [[2999, 2000]], dtype="bf16", n_sparse=1,
                                      needles_per_query=0, seed=31))
    pre = BlockSpec("cpu-prefill", [2000], [list(range(2000))], dtype="bf16", n_sparse=0, needles_per_query=0, seed=32)
    pin = make_block_inputs(pre)
    grid = np.array([1999, 0, 1000, 500])
    for r in (bench.cpu_baseline(inp, 0.2), bench.cpu_baseline_v1(make_v1_inputs(v1_config(10), with_kv=False), 0.2),
              bench.cpu_baseline_prefill(pre, pin.k, pin.v, grid, pin.q_sel[grid], 0.2)):
        assert r["value"] > 0 and r["unit"] == "tokens/s" and r["kind"] == "oracle"
        assert r["cores"] >= 1 and ("queries" in r["sample"] or "positions" in r["sample"])
        assert r["host_cpus"] >= 1 and r["cpus_in_affinity"] >= 1 and isinstance(r["cpu_model"], str)


def test_counter_summary_matches_the_pass1_source():
    """The committed HBM-traffic summary of selector pass 1 was taken on the current kernel
    source (the benchmark reports traffic only when the digests agree)."""
    import json
    sys.path.insert(0, ROOT)
    import bench

    with open(bench.COUNTERS) as f:
        c = json.load(f)
    assert c["source_digest"] == bench.source_digest()
    assert 0.99 < c["hbm_bytes_per_launch"] / (c["keys_per_launch"] * 512) < 1.05
