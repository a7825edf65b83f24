"""O3: the decode plan's queues replayed on the CPU with per-tile fp64
semantics (oracle/replay.py, DecodeTiles) reproduce the monolithic oracle step
(oracle.decode_step), serially and under random interleavings of the workers,
and a plan with one dependency edge dropped is caught -- the CMU 15-779 lecture
7 notes, section 6.5 and exercise 5: the static happens-before check flags it,
some random interleaving reads unwritten (NaN) data, and a single worker never
does.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import planner as P
from oracle.replay import DecodeTiles, replay
from tests.test_planner_pins import _check_happens_before

OPTS = dict(num_cus=16, gemv_rows=16, gateup_outs=8, down_rows=16, lm_rows=16, attn_splits=3)


def _run(inp, pl, order, seed=0, workers=None):
    ex = DecodeTiles(inp, pl)
    ctr, done = replay(pl.queue, pl.num_events, ex, order=order, seed=seed, workers=workers)
    return ex, ctr, done


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("name,overrides,opts", [
    ("tiny", {}, OPTS),
    ("tiny", dict(batch=3, kv_len=(0, 200), seed=11), dict(OPTS, attn_splits=5, num_cus=7)),
    ("tiny", dict(arch="qwen3", qk_norm=1, tied=0, head_dim=128, ffn=720, vocab=4100, seed=8),
     dict(OPTS, down_rows=6, gateup_outs=5, lm_rows=12)),
    # the pairing-strategy plan (two waits on O and down) and longest-first attention
    ("tiny", {}, dict(OPTS, pairing=1)),
    ("tiny", dict(batch=3, kv_len=(0, 200), seed=11), dict(OPTS, attn_splits=5, num_cus=7, pairing=1, attn_order=1)),
    ("tiny", dict(batch=4, kv_len=(10, 300), seed=5), dict(OPTS, attn_splits=4, num_cus=9, attn_order=1)),
])
def test_replay_of_the_decode_plan_matches_the_oracle(name, overrides, opts):
    inp = synth.make_inputs(name, norm_sigma=0.1, **overrides)
    cfg = inp["cfg"]
    ref = oracle.decode_step(inp)
    pl = P.plan_model(cfg, cfg["batch"], synth.kv_lengths(cfg), opts)
    ex, ctr, done = _run(inp, pl, "serial")
    assert list(ctr) == list(pl.event_target)  # every counter at its target
    assert sorted(done) == list(range(pl.num_tasks))  # every task exactly once
    assert np.isfinite(ex.logits).all()
    assert _rel(ex.logits, ref["logits"]) < 1e-12
    assert np.array_equal(ex.next, ref["next"])
    assert np.array_equal(ex.kv, ref["kv_cache"])  # the new rows, and nothing else
    for seed in range(20 if name == "tiny" and not overrides and len(opts) == len(OPTS) else 4):
        ex2, ctr2, done2 = _run(inp, pl, "random", seed)
        assert list(ctr2) == list(pl.event_target)
        assert sorted(done2) == list(range(pl.num_tasks))
        # fixed-order reductions inside every tile: bitwise the same in any order
        assert np.array_equal(ex2.logits, ex.logits), seed
        assert np.array_equal(ex2.kv, ex.kv)


def test_dropped_edge_in_the_decode_plan_is_caught():
    """Layer 0's combine -> O-projection edge dropped: the O tiles no longer
    wait for the attention output."""
    inp = synth.make_inputs("tiny", norm_sigma=0.1)
    cfg = inp["cfg"]
    kv = synth.kv_lengths(cfg)
    ops, edges, info = P.model_graph(cfg, 1, kv, OPTS)
    good = P.plan_graph(ops, edges, OPTS["num_cus"])
    good.info = info
    cut = [e for e in edges if not (e.name == "ao" and ops[e.cons].layer == 0)]
    assert len(cut) == len(edges) - 1
    bad = P.plan_graph(ops, cut, OPTS["num_cus"])
    bad.info = info
    _check_happens_before(good, ops, edges)
    with pytest.raises(AssertionError):
        _check_happens_before(bad, ops, edges)
    ref = oracle.decode_step(inp)
    wrong = 0
    for seed in range(12):
        ex, _, _ = _run(inp, bad, "random", seed)
        wrong += not np.isfinite(ex.logits).all()
    assert wrong > 0
    ex, _, _ = _run(inp, bad, "serial", workers=1)  # one worker runs tasks in id order
    assert np.isfinite(ex.logits).all() and _rel(ex.logits, ref["logits"]) < 1e-12
