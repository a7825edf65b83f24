"""Pins of the reference planner (oracle/planner.py) to the pages' worked
examples and to brute-force region overlap.

* MPK notes (dpshk.com), "handling fork producer": F(4) -> A(4), B(2) gives 2
  events per edge and event 0 releases A tasks 0-1 and B task 0.
* MPK notes, "handling join consumer": A(4), B(2) -> G(4) gives 2 join events
  with 3 triggers each, releasing G tasks 0-1 and 2-3.
* MPK notes, gcd examples: 128/128 -> 128 events, 128/64 -> 64, 128/1 -> 1,
  128/127 -> 1.
* CMU 15-779 lecture 7 notes, section 6.2: the GEMV -> tanh -> GEMV -> split-K
  GEMV demo has 28 tasks, 52 pairwise edges and 9 events (the per-op task
  counts 12/4/8/4 are our reconstruction from those totals); the Llama-1B layer
  has 1,984 tasks, 15 events and 3,968 task-event edges, and about 380K
  pairwise edges (the partition QKV 192 / attention 128 / O 128 / gate-up 1024
  / down 4x128 follows sections 3.1 and 5.1; the exact 379,904 is computed here
  by brute force).
* MegaRTP article, section 4 "KernelPlan": 732 tasks round-robin over 148
  queues give [148, 5, 32] with 140 queues of 5 and 8 of 4.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import planner as P

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))


def test_fork_then_join_worked_example():
    ops = [P.Op("F", 1, (4,)), P.Op("A", 2, (4,)), P.Op("B", 3, (2,)), P.Op("G", 4, (4,))]
    edges = [P.Edge(0, 1, (0,), (0,)), P.Edge(0, 2, (0,), (0,)), P.Edge(1, 3, (0,), (0,)), P.Edge(2, 3, (0,), (0,))]
    pl = P.plan_graph(ops, edges, num_cus=8)
    fk, jn = GOLD["fork_example"], GOLD["join_example"]
    assert [pl.evd[i][0] for i in range(4)] == [fk["events_per_edge"]] * 2 + [jn["events"]] * 2
    assert pl.num_events == 4 and pl.num_tasks == 14
    names = [(ops[o].name, x) for (o, x, y, z) in pl.tasks]
    # fork event 0 releases A0, A1, B0; event 1 releases A2, A3, B1
    assert names[pl.event_first[0]:pl.event_last[0]] == [tuple(v) for v in fk["event0_releases"]]
    assert names[pl.event_first[1]:pl.event_last[1]] == [tuple(v) for v in fk["event1_releases"]]
    assert pl.event_target[0] == 2 and pl.event_target[1] == 2  # F tasks {0,1} and {2,3}
    # join events: 2 (A) + 1 (B) triggers, releasing G0-1 and G2-3
    assert pl.event_target[2:] == [jn["triggers_per_event"]] * jn["events"]
    for e, rel in enumerate(jn["event_releases"]):
        assert names[pl.event_first[2 + e]:pl.event_last[2 + e]] == [("G", g) for g in rel]
    trig = {names[t]: pl.trigger[t] for t in range(pl.num_tasks)}
    assert trig[("F", 0)] == trig[("F", 1)] == 0 and trig[("F", 2)] == trig[("F", 3)] == 1
    assert trig[("A", 0)] == trig[("A", 1)] == trig[("B", 0)] == 2
    assert trig[("A", 2)] == trig[("A", 3)] == trig[("B", 1)] == 3


@pytest.mark.parametrize("prod,cons,events", [tuple(r) for r in GOLD["gcd_table"]["rows"]])
def test_gcd_examples(prod, cons, events):
    triggers = prod // events
    ops = [P.Op("P", 1, (prod,)), P.Op("C", 2, (cons,))]
    pl = P.plan_graph(ops, [P.Edge(0, 1, (0,), (0,))], num_cus=256)
    assert pl.num_events == events
    assert set(pl.event_target) == {triggers}
    assert all(pl.event_last[e] - pl.event_first[e] == cons // events for e in range(events))


def _tile_regions(op, amap, extent, tile):
    """element region (per tensor dim, [lo, hi)) that each task of ``op`` touches"""
    out = {}
    for x, y, z in itertools.product(*(range(g) for g in op.grid)):
        c = (x, y, z)
        reg = []
        for d in range(len(extent)):
            axes = [a for a in range(3) if amap[a] == d]
            if axes:
                i = c[axes[0]]
                reg.append((min(i * tile[d], extent[d]), min((i + 1) * tile[d], extent[d])))
            else:
                reg.append((0, extent[d]))
        out[c] = reg
    return out


def _overlap_pairs(ops, e):
    pr = _tile_regions(ops[e.prod], e.out_map, e.extent, e.ptile)
    cr = _tile_regions(ops[e.cons], e.in_map, e.extent, e.ctile)
    pairs = []
    for pc, preg in pr.items():
        for cc, creg in cr.items():
            if all(max(a[0], b[0]) < min(a[1], b[1]) for a, b in zip(preg, creg)):
                pairs.append((pc, cc))
    return pairs


def _waits_on(pl):
    """for each task, the set of tasks it transitively waits for"""
    trig_of_event = {}
    for t, e in enumerate(pl.trigger):
        if e >= 0:
            trig_of_event.setdefault(e, []).append(t)
    dep = [None] * pl.num_tasks
    for t in range(pl.num_tasks):  # task ids are topological
        s = set()
        e = pl.wait[t]
        if e >= 0:
            for p in trig_of_event.get(e, []):
                assert p < t
                s.add(p)
                s |= dep[p]
        dep[t] = s
    return dep


def _check_happens_before(pl, ops, edges):
    idx = {(o, x, y, z): t for t, (o, x, y, z) in enumerate(pl.tasks)}
    dep = _waits_on(pl)
    n = 0
    for e in edges:
        for pc, cc in _overlap_pairs(ops, e):
            n += 1
            assert idx[(e.prod,) + pc] in dep[idx[(e.cons,) + cc]], (e.name, pc, cc)
    return n


def demo_graph():
    """GEMV(96 out, 12 tasks of 8) -> tanh (4 tasks of 24) -> GEMV (64 out, 8 tasks of 8,
    full input) -> split-K GEMV (4 K-segments of 16)"""
    ops = [P.Op("gemv1", 1, (12,)), P.Op("tanh", 2, (4,)), P.Op("gemv3", 3, (8,)), P.Op("gemv4", 4, (4,))]
    edges = [P.Edge(0, 1, (0,), (0,), [96], [8], [24], "y1"),
             P.Edge(1, 2, (0,), (), [96], [24], [96], "y2"),
             P.Edge(2, 3, (0,), (0,), [64], [8], [16], "y3")]
    return ops, edges


def test_lecture_demo_graph():
    ops, edges = demo_graph()
    pl = P.plan_graph(ops, edges, num_cus=6)
    g = GOLD["lecture_demo"]
    assert pl.num_tasks == g["tasks"]
    assert pl.num_events == g["events"]
    assert sum(len(_overlap_pairs(ops, e)) for e in edges) == g["pairwise_edges"]
    assert _check_happens_before(pl, ops, edges) == g["pairwise_edges"]
    # tanh task i waits for exactly the 3 GEMV tasks of its 24 elements
    for t, (o, x, y, z) in enumerate(pl.tasks):
        if o == 1:
            assert pl.event_target[pl.wait[t]] == 3
        if o == 3:
            assert pl.event_target[pl.wait[t]] == 2


def megasim_layers(n_layers=3):
    """Llama-3.2-1B layers with the lecture's task partition: QKV 3072 rows in 16-row
    tiles over 8 kv groups (24 each), attention per kv head x 16, O 2048 rows in 16s,
    gate/up 8192 outputs in 8s, down 2048 rows in 16s x 4 K-chunks of 2048."""
    ops, edges = [], []
    prev = None
    for l in range(n_layers):
        q = len(ops)
        ops += [P.Op("qkv", 1, (8, 24), l), P.Op("attn", 2, (8, 16), l), P.Op("o", 3, (128,), l),
                P.Op("gu", 4, (1024,), l), P.Op("down", 5, (128, 4), l)]
        a, o, g, d = q + 1, q + 2, q + 3, q + 4
        if prev is not None:
            edges.append(P.Edge(prev, q, (1, -1), (), [1, 2048], [1, 16], [1, 2048], "x"))
        edges.append(P.Edge(q, a, (0, 1), (0,), [8, 384], [1, 16], [1, 384], "qkv"))
        edges.append(P.Edge(a, o, (0,), (), [8, 1], [1, 1], [8, 1], "attn"))
        if prev is not None:
            edges.append(P.Edge(prev, o, (1, -1), (), [1, 2048], [1, 16], [1, 2048], "x_res"))
        edges.append(P.Edge(o, g, (1,), (), [1, 2048], [1, 16], [1, 2048], "h"))
        edges.append(P.Edge(o, d, (1,), (), [1, 2048], [1, 16], [1, 2048], "h_res"))
        edges.append(P.Edge(g, d, (1,), (-1, 1), [1, 8192], [1, 8], [1, 2048], "act"))
        prev = d
    return ops, edges


def test_lecture_llama1b_layer_counts():
    ops, edges = megasim_layers(3)
    pl = P.plan_graph(ops, edges, num_cus=132)
    mid = {i for i, op in enumerate(ops) if op.layer == 1}
    tasks = [t for t, (o, x, y, z) in enumerate(pl.tasks) if o in mid]
    g = GOLD["lecture_llama1b_layer"]
    assert len(tasks) == g["tasks"]
    events = {pl.wait[t] for t in tasks}
    assert len(events) == g["events"]
    edges_te = sum((pl.wait[t] >= 0) + (pl.trigger[t] >= 0) for t in tasks)
    assert edges_te == g["task_event_edges"]
    # ~380K pairwise edges (the page gives the rounded figure), counted here by
    # brute-force region overlap of layer 1's inputs
    pairwise = sum(len(_overlap_pairs(ops, e)) for e in edges if e.cons in mid and not e.name.endswith("_res"))
    assert pairwise == 379904
    assert abs(pairwise - g["pairwise_edges_approx"]) / g["pairwise_edges_approx"] < 0.01
    assert not any(pl.kept[i] for i, e in enumerate(edges) if e.name.endswith("_res"))


def test_round_robin_queue_shape():
    g = GOLD["megartp_queue"]
    pl = P.plan_graph([P.Op("t", 1, (g["tasks"],))], [], num_cus=g["num_cus"])
    q = np.array(pl.queue)
    assert q.shape == tuple(g["queue_shape"])
    valid = (q[:, :, P.W_OPCODE] != 0).sum(axis=1)
    assert list(valid[:140]) == [5] * 140 and list(valid[140:]) == [4] * 8
    assert (q[140:, 4] == 0).all()  # NoOp rows are all zero


TINY = dict(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=688, vocab=4096)


@pytest.mark.parametrize("batch,kv", [(1, [128]), (3, [0, 7, 300])])
def test_model_plan_invariants_and_happens_before(batch, kv):
    pl = P.plan_model(TINY, batch, kv, dict(num_cus=37, gemv_rows=16, gateup_outs=8, down_rows=16, lm_rows=16,
                                            attn_splits=3))
    q = np.array(pl.queue)
    C, L = q.shape[:2]
    T = pl.num_tasks
    ids = q[:, :, P.W_TASK][q[:, :, P.W_OPCODE] != 0]
    assert sorted(ids.tolist()) == list(range(T))  # every task in exactly one slot
    assert (q[:, :, P.W_OPCODE] == 0).sum() == C * L - T
    assert sum(pl.event_target) == sum(1 for t in pl.trigger if t >= 0)
    for e in range(pl.num_events):
        assert all(pl.wait[t] == e for t in range(pl.event_first[e], pl.event_last[e]))
    _check_happens_before(pl, pl.ops, pl.edges)
    # per-kv-group attention events with 24/ (RPG/16) triggers; one event per whole edge
    T_qkv = pl.info["T_qkv"]
    attn_events = {pl.wait[t] for t, (o, *_) in enumerate(pl.tasks) if pl.ops[o].opcode == P.ATTN}
    assert len(attn_events) == TINY["n_layers"] * TINY["n_kv_heads"]
    assert {pl.event_target[e] for e in attn_events} == {T_qkv}


# ---------------------------------------------------------------------------
# Replay: the lecture's interpreter experiment (section 6.5 and exercise 5)
# ---------------------------------------------------------------------------
def _demo_semantics(seed=0):
    rng = np.random.default_rng(seed)
    W1, W3, W4 = rng.standard_normal((96, 32)), rng.standard_normal((64, 96)), rng.standard_normal((8, 64))
    xin = rng.standard_normal(32)
    ref = W4 @ (W3 @ np.tanh(W1 @ xin))

    def run(pl, order, seed, workers=None):
        from oracle.replay import replay
        mem = dict(y1=np.full(96, np.nan), y2=np.full(96, np.nan), y3=np.full(64, np.nan), p4=np.full((4, 8), np.nan))

        def execute(r):
            op, x = r[P.W_OPROW], r[P.W_GX]
            if op == 0:
                mem["y1"][8 * x:8 * x + 8] = W1[8 * x:8 * x + 8] @ xin
            elif op == 1:
                mem["y2"][24 * x:24 * x + 24] = np.tanh(mem["y1"][24 * x:24 * x + 24])
            elif op == 2:
                mem["y3"][8 * x:8 * x + 8] = W3[8 * x:8 * x + 8] @ mem["y2"]
            else:
                mem["p4"][x] = W4[:, 16 * x:16 * x + 16] @ mem["y3"][16 * x:16 * x + 16]
        ctr, done = replay(pl.queue, pl.num_events, execute, order=order, seed=seed, workers=workers)
        return mem["p4"].sum(axis=0), ctr, done
    return ref, run


def test_replay_random_interleavings_agree():
    ops, edges = demo_graph()
    pl = P.plan_graph(ops, edges, num_cus=6)
    ref, run = _demo_semantics()
    for s in range(20):
        out, ctr, done = run(pl, "random", s)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
        assert ctr == pl.event_target  # every counter reaches its target
        assert sorted(done) == list(range(pl.num_tasks))  # every task exactly once


def test_dropped_edge_is_caught():
    """Drop GEMV3[7] -> GEMV4[3]: the happens-before check flags it statically and
    some random interleavings read unwritten (NaN) data; one worker never does."""
    import copy
    ops, edges = demo_graph()
    pl = P.plan_graph(ops, edges, num_cus=6)
    bad = copy.deepcopy(pl)
    t7 = bad.tasks.index((2, 7, 0, 0))
    e = bad.trigger[t7]
    bad.trigger[t7] = -1
    bad.event_target[e] -= 1
    for q in bad.queue:
        for r in q:
            if r[P.W_OPCODE] and r[P.W_TASK] == t7:
                r[P.W_SIG_CNT] = r[P.W_SIG_EV] = r[P.W_SIG_INC] = 0
            if r[P.W_OPCODE] and r[P.W_WAIT_CNT] and r[P.W_WAIT_EV] == e:
                r[P.W_WAIT_TGT] -= 1
    with pytest.raises(AssertionError):
        _check_happens_before(bad, ops, edges)
    ref, run = _demo_semantics()
    wrong = sum(not np.allclose(run(bad, "random", s)[0], ref) for s in range(40))
    assert 0 < wrong < 40
    assert np.allclose(run(bad, "serial", 0, workers=1)[0], ref)


def test_replay_reports_deadlock():
    from oracle.replay import replay, Deadlock
    ops, edges = demo_graph()
    pl = P.plan_graph(ops, edges, num_cus=6)
    import copy
    bad = copy.deepcopy(pl)
    for q in bad.queue:
        for r in q:
            if r[P.W_OPCODE] and r[P.W_WAIT_CNT] and r[P.W_WAIT_EV] == 4:
                r[P.W_WAIT_TGT] += 1  # a target that can never be reached
    with pytest.raises(Deadlock):
        replay(bad.queue, bad.num_events, lambda r: None)


# ---------------------------------------------------------------------------
# MegaRTP article, section 4: the plan of the GLM pre-attention subgraph at
# M=16, KV=8192 under the pairing strategies.  Graph only (no arithmetic): the
# op grids are the page's tile counts; the publications and edges are our
# reading of its event list -- A0 publishes the hidden fp8/scale rows and the
# norm rows; B0 and D1 finish split-K tiles in their last split, and only B0's
# first 16 N tiles (the Q/scale tiles that make up D0's K=2048 input) are read
# downstream; B1 signals once, from the tile that completes the cache write;
# D0 publishes one region per head (its two N tiles), which D2's four tiles of
# that head read.
def megartp_graph():
    G = GOLD["megartp_plan"]
    names = G["ops_in_page_order"]
    ops = [P.Op(n, 100 + i, tuple(G["tiles"][n])) for i, n in enumerate(names)]
    ix = {n: i for i, n in enumerate(names)}
    pubs = [
        P.Pub(ix["A0"], name="hidden"), P.Pub(ix["A0"], name="norm"),
        P.Pub(ix["B0"], map=(1,), div=(16,), sel=(-1, -1, 3), name="q"),
        P.Pub(ix["C0"], name="gate_partial"),
        P.Pub(ix["B1"], sel=(-1, 7), name="kcache"),
        P.Pub(ix["D1"], sel=(-1, -1, 3), name="idx_q"),
        P.Pub(ix["D0"], map=(1,), name="q_b"),
    ]
    pix = {p.name: k for k, p in enumerate(pubs)}
    E = P.PairEdge
    edges = [
        E(pix["hidden"], ix["B0"], P.TILE_COVER), E(pix["norm"], ix["C0"], P.TILE_COVER),
        E(pix["hidden"], ix["B1"], P.TILE_COVER),
        E(pix["q"], ix["D1"], P.TILE_COVER), E(pix["gate_partial"], ix["D1"], P.TILE_REDUCE),
        E(pix["q"], ix["D0"], P.TILE_COVER),
        E(pix["q_b"], ix["D2"], P.TILE_COVER, map=(1,)),
        E(pix["idx_q"], ix["E1"], P.TILE_COVER), E(pix["kcache"], ix["E1"], P.TILE),
    ]
    return ops, pubs, edges, ix


def test_megartp_page_plan():
    G = GOLD["megartp_plan"]
    ops, pubs, edges, ix = megartp_graph()
    pl = P.pair_plan(ops, pubs, edges, num_cus=G["queue_shape"][0])
    assert pl.num_tasks == G["tasks"] and pl.num_events == G["events"]
    th = G["thresholds"]
    want = [th["event0"], th["event1"], th["event2"], th["event3"]] + [th["events4_67"]] * 64 + \
        [th["event68"], th["event69"]]
    assert pl.event_target == want
    assert list(pl.queue.shape) == G["queue_shape"]
    live = (pl.queue[:, :, P.W_OPCODE] != 0).sum(axis=1)
    assert (live == 5).sum() == G["queues_with_5"] and (live == 4).sum() == G["queues_with_4"]
    rows = pl.queue.reshape(-1, P.WORDS)
    rows = rows[rows[:, P.W_OPCODE] != 0]
    by_op = {n: rows[rows[:, P.W_OPROW] == i] for n, i in ix.items()}

    def waits(r):
        w = [(r[P.W_WAIT_EV], r[P.W_WAIT_TGT])] if r[P.W_WAIT_CNT] >= 1 else []
        if r[P.W_WAIT_CNT] == 2:
            w.append((r[P.W_WAIT2_EV], r[P.W_WAIT2_TGT]))
        return [tuple(map(int, v)) for v in w]

    for n, wl in G["waits"].items():
        for r in by_op[n]:
            assert waits(r) == [tuple(v) for v in wl], n
    d0 = G["d0_head_events"]
    for r in by_op["D2"]:
        assert waits(r) == [(d0["first"] + int(r[P.W_GY]), d0["threshold"])]
    assert (by_op["A0"][:, P.W_WAIT_CNT] == 0).all()
    # signals: A0 publishes two outputs; split-K ops from their final split
    for r in by_op["A0"]:
        assert r[P.W_SIG_CNT] == 2 and [r[P.W_SIG_EV], r[P.W_SIG2_EV]] == G["a0_signals"]
        assert [r[P.W_SIG_PUB], r[P.W_SIG2_PUB]] == [0, 1]
    sig = lambda n: by_op[n][by_op[n][:, P.W_SIG_CNT] > 0]
    assert len(sig("B0")) == th["event2"] and set(sig("B0")[:, P.W_GZ]) == {3}
    assert len(sig("C0")) == th["event3"] and len(sig("D1")) == th["event68"] and len(sig("B1")) == th["event69"]
    assert len(sig("D0")) == 128 and len(sig("D2")) == 0 and len(sig("E1")) == 0
    for r in sig("D0"):
        assert r[P.W_SIG_EV] == d0["first"] + r[P.W_GY]
    assert set(by_op["E1"][:, P.W_OPROW]) == {G["e1_operand_row"]}
    # every wait's threshold equals the number of signals to its event
    n_sig = np.zeros(pl.num_events, dtype=int)
    for r in rows:
        for k in range(r[P.W_SIG_CNT]):
            n_sig[r[(P.W_SIG_EV, P.W_SIG2_EV)[k]]] += 1
    assert list(n_sig) == want


def test_pairing_strategies_are_checked():
    ops = [P.Op("P", 1, (4,)), P.Op("C", 2, (2,))]
    # 'tile' needs one producer tile per region
    with pytest.raises(ValueError, match="tile"):
        P.pair_plan(ops, [P.Pub(0)], [P.PairEdge(0, 1, P.TILE)], 8)
    # 'whole' needs one region published by every tile
    with pytest.raises(ValueError, match="whole"):
        P.pair_plan(ops, [P.Pub(0, map=(0,), div=(2,))], [P.PairEdge(0, 1, P.WHOLE)], 8)
    with pytest.raises(ValueError, match="whole"):
        P.pair_plan(ops, [P.Pub(0, sel=(3,))], [P.PairEdge(0, 1, P.WHOLE)], 8)
    # regions of a tile_reduce edge hold equal partial counts
    ops3 = [P.Op("P", 1, (3,)), P.Op("C", 2, (2,))]
    with pytest.raises(ValueError, match="tile_reduce"):
        P.pair_plan(ops3, [P.Pub(0, map=(0,), div=(2,))], [P.PairEdge(0, 1, P.TILE_REDUCE, map=(0,))], 8)
    pl = P.pair_plan(ops3, [P.Pub(0, map=(0,), div=(2,))], [P.PairEdge(0, 1, P.TILE_COVER, map=(0,))], 8)
    assert pl.event_target == [2, 1]
    # a consumer region outside the publication, and three waits
    with pytest.raises(ValueError, match="outside"):
        P.pair_plan(ops, [P.Pub(0, map=(0,), div=(4,))], [P.PairEdge(0, 1, P.TILE_COVER, map=(0,))], 8)
    ops4 = [P.Op("A", 1, (1,)), P.Op("B", 2, (1,)), P.Op("C", 3, (1,)), P.Op("D", 4, (1,))]
    with pytest.raises(ValueError, match="more than two"):
        P.pair_plan(ops4, [P.Pub(0), P.Pub(1), P.Pub(2)], [P.PairEdge(k, 3, P.TILE) for k in range(3)], 8)
    # an op publishing three read outputs signals three events
    with pytest.raises(ValueError, match="more than two"):
        P.pair_plan(ops4, [P.Pub(0), P.Pub(0), P.Pub(0)], [P.PairEdge(k, 1 + k, P.TILE) for k in range(3)], 8)


def test_megartp_page_plan_replays_under_random_interleavings():
    """The page plan executed by the CPU replay (two waits, two signals): no
    deadlock in 20 random worker interleavings, every consumer starts only
    after all producer tiles of its regions finished."""
    from oracle.replay import replay
    ops, pubs, edges, ix = megartp_graph()
    pl = P.pair_plan(ops, pubs, edges, num_cus=148)
    pos = {}
    for seed in range(20):
        ctr, done = replay(pl.queue, pl.num_events, lambda r: None, order="random", seed=seed)
        assert ctr == pl.event_target and sorted(done) == list(range(pl.num_tasks))
        at = {t: i for i, t in enumerate(done)}
        for t in range(pl.num_tasks):
            for ev in (pl.wait[t], pl.wait2[t]):
                if ev >= 0:
                    prods = [u for u in range(pl.num_tasks) if ev in (pl.trigger[u], pl.trigger2[u])]
                    assert max(at[u] for u in prods) < at[t]
