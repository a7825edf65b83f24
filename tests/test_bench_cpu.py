"""bench.py host logic: the algorithmic byte count against the lecture's bs=1
roofline figures for Llama-3.2-1B (tests/golden/page_examples.json), the
one-GPU contract, and the trace decoder on a hand-built trace."""
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


def test_trace_report_on_a_hand_built_trace():
    """The trace decoder on two CUs with two instructions each (ticks at 10 per
    us): busy intervals [1.0, 3.0] + [5.2, 8.0] and [1.2, 4.0] + [5.0, 7.0] us over
    a span of 8.2 us give an active-CU fraction of 9.6 / 16.4 and bubbles of 2.2
    and 1.0 us; the QKV -> attention event's producers signal at 3.2 and 4.4 us
    (tail 0.6 us) and its consumers start at 5.0 and 4.8 us (detection 0.5 us)."""
    import numpy as np
    q = np.zeros((2, 3, 32), dtype=np.int32)
    tr = np.zeros((2, 3, 16), dtype=np.uint64)
    # (op, waits on event 0, signals event e) per instruction; slot 2 is a NoOp
    for c in range(2):
        q[c, 0, 0], q[c, 0, 6], q[c, 0, 7] = 1, 1, 0          # QKV, signals event 0
        q[c, 1, 0], q[c, 1, 3], q[c, 1, 4] = 2, 1, 0          # attention, waits on event 0
        q[c, 1, 6], q[c, 1, 7] = 1, 1                         # ... and signals event 1
    tr[0, 0, :4] = (0, 10, 30, 32)
    tr[0, 1, :4] = (50, 52, 80, 82)
    tr[1, 0, :4] = (0, 12, 40, 44)
    tr[1, 1, :4] = (48, 50, 70, 71)
    r = bench.trace_report(tr, 10.0, q)
    assert r["traced_step_us"] == 8.2
    assert r["active_cu_frac"] == round(9.6 / 16.4, 4)
    assert r["bubble_median_us"] == 1.6 and r["bubble_share"] == round(3.2 / 16.4, 4)
    assert r["events"] == 1 and r["hop_tail_median_us"] == 0.6 and r["hop_detect_median_us"] == 0.5
    assert r["per_op"]["qkv"] == dict(tasks=2, median_task_us=2.4, median_span_us=3.4)
    assert r["per_op"]["attn"] == dict(tasks=2, median_task_us=2.4, median_span_us=3.2)
