"""bench.py host logic: the algorithmic byte count against the lecture's bs=1
roofline figures for Llama-3.2-1B (tests/golden/page_examples.json), and the
one-GPU contract."""
import json
import os
import subprocess
import sys

import bench
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))


def test_llama1b_bytes_match_the_lecture_roofline():
    inp_cfg = synth.config("llama1b")
    g = GOLD["llama1b_step_bytes"]
    total = bench.algorithmic_bytes(inp_cfg, [1024])
    assert total == 2505733120
    # the page counts the step at about 2.48 GB and 313 us at 8 TB/s
    assert abs(total / 1e9 - g["bytes_per_step_GB"]) / g["bytes_per_step_GB"] < 0.015
    assert abs(total / 8e12 * 1e6 - g["ideal_us_at_8TBps"]) < 1.0


def test_kv_and_logit_terms():
    cfg = dict(synth.config("tiny"))
    base = bench.algorithmic_bytes(cfg, [0])
    L, nkv, hd = cfg["n_layers"], cfg["n_kv_heads"], cfg["head_dim"]
    assert bench.algorithmic_bytes(cfg, [10]) - base == 10 * L * nkv * hd * 2 * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
