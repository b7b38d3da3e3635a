"""CPU checks of bench.py's contract: the headline workload prints the metric the
benchmark is quoted on, the other workloads name their own shape and bit widths,
and a request for more than one GPU exits with a message."""
import json
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_metric_strings():
    headline = json.load(open(os.path.join(ROOT, "BASELINE.json")))["metric"]
    assert bench.metric_of(synth.BLOCK_CFG4) == headline
    names = {k: bench.metric_of(c) for k, c in bench.workloads().items()}
    assert len(set(names.values())) == len(names)
    assert "70B" in names["llama70b_block_w4a16"] and "W4A16" in names["llama70b_block_w4a16"]
    assert "FFN" in names["llama7b_ffn_w3a16"] and "W3A16" in names["llama7b_ffn_w3a16"]
    assert "W2A16g128" in names["llama7b_block_w2a16g128"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
