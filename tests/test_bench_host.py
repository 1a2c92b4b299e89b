"""Host-side logic of bench.py: the single-GPU contract, the algorithmic byte and
flop counts the roofline divides by, and the counter summaries it may quote."""
import os
import subprocess
import sys
import types

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from draft_token_verification_flattened_amd import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_algorithmic_bytes():
    # verify reads 2V bytes per bf16 row: N + R target rows, plus N draft rows when sampling
    w = types.SimpleNamespace(V=151936, dtype="bf16")
    assert bench.algorithmic_bytes(w, "sample", 1280, 256) == 2 * 151936 * (2 * 1280 + 256)   # 855.7 MB
    assert bench.algorithmic_bytes(w, "greedy", 1280, 256) == 2 * 151936 * (1280 + 256)       # 466.7 MB
    assert abs(bench.algorithmic_bytes(w, "sample", 1280, 256) / 1e6 - 855.7) < 0.1
    w32 = types.SimpleNamespace(V=32, dtype="f32")
    assert bench.algorithmic_bytes(w32, "sample", 3, 4) == 4 * 32 * (2 * 3 + 4)


def test_markov_bytes_and_flops_per_position():
    # P once (2 d_m V), the gathered operand rows (2 R d_m), backbone read and logits written (2 R V each)
    w = types.SimpleNamespace(V=151936, R=512, dtype="bf16", emb=np.zeros((1, 256), np.uint16))
    nb, fl = bench.markov_bytes_flops(w)
    assert nb == 2 * (256 * 151936 + 512 * 256 + 2 * 512 * 151936)
    assert abs(nb / 1e6 - 389.2) < 0.1
    assert fl == 2.0 * 512 * 256 * 151936
    assert abs(fl / 1e9 - 39.83) < 0.01


def test_counter_summaries_parse_and_are_keyed_by_workload():
    for (kernel, cfg), (path, _files) in bench.TRAFFIC.items():
        assert os.path.exists(path), path
        vals = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
        for key in ("fetch_scale", "write_scale", "hbm_bytes_per_launch", "source_hash", "workload"):
            assert key in vals, (path, key)
        assert float(vals["hbm_bytes_per_launch"]) > 0
        assert vals["workload"].split()[0] == cfg, path
        # never quoted for another workload: another mode of the same configuration,
        # or the same mode of another one
        other = types.SimpleNamespace(config=cfg, mode="greedy", head="markov")
        assert bench.committed_traffic(kernel, bench.workload_key(other, 5))[0] is None
        wk = vals["workload"].split()
        other = types.SimpleNamespace(config="c0", mode=wk[1], head=wk[3].split("=")[1])
        assert bench.committed_traffic(kernel, bench.workload_key(other, int(wk[2].split("=")[1])))[0] is None


def test_workload_configs_match_the_recipes():
    c2 = workloads.CONFIGS["c2"]
    assert (c2["R"], c2["k"], c2["V"]) == (256, 5, 151936)
    c4 = workloads.CONFIGS["c4"]
    assert (c4["R"], c4["k"], c4["V"], c4["d_m"]) == (512, 5, 151936, 256)


def test_verify_kernel_bytes_split():
    # spec_step: one streaming launch reads every row, the rows (r, 0) included
    w = types.SimpleNamespace(V=151936, dtype="bf16")
    per = bench.verify_kernel_bytes(w, "sample", 512, 256, True, True)
    assert per == {"verify_step_stream": 2 * 151936 * (2 * 512 + 256)}
    assert per["verify_step_stream"] == bench.algorithmic_bytes(w, "sample", 512, 256)
    assert bench.verify_kernel_bytes(w, "greedy", 512, 256, True, False) == {
        "verify_stream": 2 * 151936 * (512 + 256)}
    # the draft head's statistics: no draft rows
    assert bench.algorithmic_bytes(w, "sample", 512, 256, draft_rows=False) == 2 * 151936 * (512 + 256)
