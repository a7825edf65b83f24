"""CPU tests of the HIP library (no GPU): it loads, exports every symbol the
header declares, rejects bad arguments, and its C++ planner reproduces the
reference planner (oracle/planner.py) bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import planner as P
from tests.lib_defaults import documented_choices, documented_defaults

mk = pytest.importorskip("persistent_megakernel_decode_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "mk.h")).read()
    declared = set(re.findall(r"\b(mk_[a-z_]+)\s*\(", hdr))
    assert {"mk_plan_build", "mk_run", "mk_run_layerwise"} <= declared
    L = mk.lib()
    for name in sorted(declared):
        assert hasattr(L, name), name
    assert set(mk.EXPORTED) == declared
    assert L.mk_abi_version() == mk.MK_ABI_VERSION


def _compare(lib_plan, ref):
    ex = lib_plan.export()
    assert ex["num_cus"] == ref.num_cus and ex["max_len"] == ref.max_len
    assert ex["num_tasks"] == ref.num_tasks and ex["num_events"] == ref.num_events
    assert np.array_equal(ex["queue"], np.asarray(ref.queue, dtype=np.int32))
    assert ex["event_target"].tolist() == list(ref.event_target)
    assert ex["event_first"].tolist() == list(ref.event_first)
    assert ex["event_last"].tolist() == list(ref.event_last)
    assert ex["task_trigger"].tolist() == list(ref.trigger)
    assert ex["task_wait"].tolist() == list(ref.wait)
    assert ex["task_trigger2"].tolist() == list(ref.trigger2)
    assert ex["task_wait2"].tolist() == list(ref.wait2)
    assert ex["edge_kept"].astype(bool).tolist() == list(ref.kept)
    assert ex["op_table"].tolist() == P.op_table(ref)
    return ex


@pytest.mark.parametrize("name,overrides,num_cus,opts", [
    ("tiny", {}, 256, {}),
    ("tiny", {}, 37, dict(attn_splits=5)),
    ("tiny", dict(kv_len=0), 64, {}),
    ("tiny", dict(ffn=688 + 32, vocab=4100, kv_len=999), 100, {}),  # ragged FFN and vocab tails
    ("tiny", dict(arch="qwen3", qk_norm=1, tied=0, head_dim=128), 256, {}),
    ("llama1b", {}, 256, {}),
    ("tiny", dict(batch=3, kv_len=(0, 200), seed=11), 37, {}),
    ("llama1b_b16", {}, 256, {}),
    ("llama1b", {}, 148, dict(gemv_rows=8, down_rows=2)),
    ("qwen3_8b", {}, 256, {}),
    ("qwen3_8b", dict(batch=4, kv_len=(100, 3000), seed=3), 256, {}),  # batched default down tiles, F 12288
    ("tiny", dict(batch=6, kv_len=(1, 120), seed=15), 64, dict(down_rows=6, gateup_outs=3)),
])
def test_cpp_planner_matches_reference(name, overrides, num_cus, opts):
    """Both planners get the same explicit tile options (every field given)."""
    cfg = synth.config(name, **overrides)
    kv = synth.kv_lengths(cfg)
    cap = synth.kv_capacity(kv)
    o = documented_defaults(cfg, cfg["batch"], kv, num_cus, **opts)
    ref = P.plan_model(cfg, cfg["batch"], kv, dict(o, **documented_choices(cfg["batch"])))
    plan = mk.Plan.build(cfg, cfg["batch"], kv, cap, **o)
    try:
        ex = _compare(plan, ref)
        assert ex["tile_opts"] == o
    finally:
        plan.free()


@pytest.mark.parametrize("name,overrides,num_cus,opts", [
    ("tiny", {}, 256, {}),
    ("tiny", dict(kv_len=0), 64, {}),
    ("tiny", dict(ffn=688 + 32, vocab=4100, kv_len=999), 100, {}),
    ("llama1b", {}, 256, {}),
    ("llama1b", {}, 148, dict(gemv_rows=8, down_rows=2)),
    ("llama1b_b16", {}, 256, {}),
    ("qwen3_8b", {}, 256, {}),
    ("qwen3_8b", {}, 200, {}),
    ("qwen3_8b", dict(batch=4, kv_len=(100, 3000), seed=3), 256, {}),
    ("tiny", dict(batch=3, kv_len=(0, 200), seed=11), 37, {}),
])
def test_library_defaults_follow_the_documented_rule(name, overrides, num_cus, opts):
    """With fields left at 0 the library resolves each by the rule its header
    documents (tested here against that documentation, not the oracle)."""
    cfg = synth.config(name, **overrides)
    kv = synth.kv_lengths(cfg)
    plan = mk.Plan.build(cfg, cfg["batch"], kv, synth.kv_capacity(kv), num_cus=num_cus, **opts)
    try:
        assert plan.export()["tile_opts"] == documented_defaults(cfg, cfg["batch"], kv, num_cus, **opts)
    finally:
        plan.free()


@pytest.mark.parametrize("name,num_cus", [("glm_preattn", 256), ("glm_preattn", 148), ("glm_tiny", 37),
                                           ("glm_tiny", 7)])
def test_cpp_planner_matches_reference_glm(name, num_cus):
    cfg = synth.config(name)
    pos, _ = synth.glm_positions(cfg)
    ref = P.plan_model(cfg, len(pos), pos, dict(num_cus=num_cus))
    plan = mk.Plan.build(cfg, len(pos), pos, synth.glm_capacity(cfg), num_cus=num_cus)
    try:
        _compare(plan, ref)
    finally:
        plan.free()


def test_glm_plan_structure():
    """A0 (16 rows) forks to QKV-A / gate / indexer-K through one event of 16
    triggers; the gate's 4 row tiles x 12 K-splits (4 blocks of 128 columns
    each) reach the gate reduce through one event per row tile (tile_reduce, 12
    triggers); QKV-A's 132 tiles join into the q-path norm (one event, 132
    triggers); the norm forks to QKV-B (64 heads x 12 tiles) and indexer-Q (256
    tiles) through one event of 16 triggers: 1248 tasks in all."""
    cfg = synth.config("glm_preattn")
    pos, _ = synth.glm_positions(cfg)
    ref = P.plan_model(cfg, len(pos), pos, dict(num_cus=256))
    assert ref.num_tasks == 16 + 132 + 4 * 12 + 8 + 4 + 16 + 64 * 12 + 256 == 1248
    assert list(ref.event_target) == [16, 12, 12, 12, 12, 132, 16] and ref.max_len == 5
    q = np.asarray(ref.queue).reshape(-1, 32)
    gate = q[q[:, 0] == P.G_GATE]
    # split y covers blocks 4y .. 4y + 3 of the 48
    assert sorted({(r[12], r[17], r[18]) for r in gate}) == [(y, 4 * y, 4) for y in range(12)]
    # QKV-B payloads: plain tiles of 16 rows, then RoPE-pair tiles (8 rows + 8 rows 32 further on)
    q = np.asarray(ref.queue).reshape(-1, 32)
    qb = q[q[:, 0] == P.G_QKVB]
    pays = sorted(tuple(r[14:17]) for r in qb if r[11] == 1)
    assert pays[:8] == [(192 + 16 * y, 16, -1) for y in range(8)]
    assert pays[8:] == [(192 + 128 + 8 * j, 8, 192 + 160 + 8 * j) for j in range(4)]


def _graph_via_lib(ops, edges, num_cus):
    lops = [(op.opcode, op.grid, op.spec, op.layer) for op in ops]
    ledges = [(e.prod, e.cons, e.out_map, e.in_map, e.extent, e.ptile, e.ctile) for e in edges]
    return mk.Plan.graph(lops, ledges, num_cus)


def test_cpp_planner_matches_reference_on_page_examples():
    from tests.test_planner_pins import demo_graph, megasim_layers
    cases = [
        ([P.Op("F", 1, (4,)), P.Op("A", 2, (4,)), P.Op("B", 3, (2,)), P.Op("G", 4, (4,))],
         [P.Edge(0, 1, (0,), (0,)), P.Edge(0, 2, (0,), (0,)), P.Edge(1, 3, (0,), (0,)), P.Edge(2, 3, (0,), (0,))], 8),
        demo_graph() + (6,),
        megasim_layers(3) + (132,),
        ([P.Op("t", 1, (732,))], [], 148),
        # a mixed fork/join component (falls back to one event)
        ([P.Op("A", 1, (4,)), P.Op("B", 2, (8,)), P.Op("C", 3, (2,)), P.Op("D", 4, (8,)), P.Op("E", 5, (4,))],
         [P.Edge(0, 1, (0,), (0,)), P.Edge(0, 2, (0,), (0,)), P.Edge(1, 3, (0,), (0,)), P.Edge(1, 4, (0,), (0,)),
          P.Edge(2, 4, (0,), (0,))], 16),
    ]
    for prod in (128,):
        for cons in (128, 64, 1, 127):
            cases.append(([P.Op("P", 1, (prod,)), P.Op("C", 2, (cons,))], [P.Edge(0, 1, (0,), (0,))], 256))
    for ops, edges, C in cases:
        ref = P.plan_graph(ops, edges, C)
        plan = _graph_via_lib(ops, edges, C)
        try:
            _compare(plan, ref)
        finally:
            plan.free()


def test_plan_build_rejects_bad_arguments():
    cfg = synth.config("tiny")
    with pytest.raises(mk.MKError) as e:
        mk.Plan.build(cfg, 1, [200], 100, num_cus=8)  # kv_len + 1 > capacity
    assert e.value.status == mk.MK_E_UNSUPPORTED
    with pytest.raises(mk.MKError) as e:
        mk.Plan.build(dict(cfg, head_dim=96), 1, [10], 100, num_cus=8)
    assert e.value.status == mk.MK_E_UNSUPPORTED
    # more GEMV rows than the tile shape for K allows (K = 8192: at most 4)
    with pytest.raises(mk.MKError) as e:
        mk.Plan.build(synth.config("llama1b"), 1, [10], 100, num_cus=8, down_rows=8)
    assert e.value.status == mk.MK_E_UNSUPPORTED and b"rows" in mk.lib().mk_last_error()
    d = mk.model_desc(cfg, 100)
    d.struct_size = 4
    h = ctypes.c_void_p()
    kv = np.array([10], np.int32)
    assert mk.lib().mk_plan_build(ctypes.byref(d), 1, kv.ctypes.data, None, ctypes.byref(h)) == mk.MK_E_INVALID
    assert mk.lib().mk_plan_build(None, 1, kv.ctypes.data, None, ctypes.byref(h)) == mk.MK_E_INVALID
    assert b"null" in mk.lib().mk_last_error()
    # GLM: bf16 weights, two rows of one request at one position, positions past the cache
    g = synth.config("glm_tiny")
    pos, _ = synth.glm_positions(g)
    cap = synth.glm_capacity(g)
    gd = mk.model_desc(g, cap)
    gd.weight_dtype = mk.MK_BF16
    assert mk.lib().mk_plan_build(ctypes.byref(gd), len(pos), pos.ctypes.data, None, ctypes.byref(h)) == mk.MK_E_UNSUPPORTED
    dup = pos.copy()
    dup[1] = dup[0]
    with pytest.raises(mk.MKError) as e:
        mk.Plan.build(g, len(pos), dup, cap, num_cus=8)
    assert e.value.status == mk.MK_E_INVALID
    with pytest.raises(mk.MKError) as e:
        mk.Plan.build(g, len(pos), pos + cap, cap, num_cus=8)
    assert e.value.status == mk.MK_E_UNSUPPORTED
    with pytest.raises(mk.MKError) as e:
        mk.Plan.build(dict(g, rope_dim=40), len(pos), pos, cap, num_cus=8)
    assert e.value.status == mk.MK_E_UNSUPPORTED
    # planner choices: out of range, or on the GLM path
    for bad in (dict(pairing=2), dict(pairing=-1), dict(attn_order=2), dict(attn_order=-2)):
        with pytest.raises(mk.MKError) as e:
            mk.Plan.build(cfg, 1, [10], 100, num_cus=8, **bad)
        assert e.value.status == mk.MK_E_INVALID, bad
    for bad in (dict(pairing=1), dict(attn_order=1)):
        with pytest.raises(mk.MKError) as e:
            mk.Plan.build(g, len(pos), pos, cap, num_cus=8, **bad)
        assert e.value.status == mk.MK_E_UNSUPPORTED, bad
    # a graph-only plan cannot run
    g = mk.Plan.graph([(1, (4,))], [], 4)
    w = mk.Weights()
    assert mk.lib().mk_run(g._h, ctypes.byref(w), None, None, None) == mk.MK_E_STATE
    g.free()
    # an edge that goes backwards is rejected
    with pytest.raises(mk.MKError):
        mk.Plan.graph([(1, (4,)), (2, (4,))], [(1, 0, (0,), (0,), None, None, None)], 4)


@pytest.mark.parametrize("name,num_cus,splits,shift", [("tiny", 37, 5, 3), ("llama1b_b16", 256, 4, 7),
                                                        ("tiny", 256, 0, 9)])
def test_set_kv_len_patches_match_a_fresh_plan(name, num_cus, splits, shift):
    """Moving a plan to new sequence lengths (no device needed before its first
    run) gives exactly the queue the planner builds for those lengths with the
    same attention split count: only the attention payloads change."""
    cfg = synth.config(name)
    kv0 = synth.kv_lengths(cfg)
    kv1 = kv0 + shift
    cap = synth.kv_capacity(kv1)
    for order in (-1, 0):
        plan = mk.Plan.build(cfg, cfg["batch"], kv0, cap, num_cus=num_cus, attn_splits=splits, attn_order=order)
        try:
            ex = plan.export()
            o = ex["tile_opts"]
            # the reference: the plan for kv0 (its placement) with kv1's payloads
            ref1 = P.plan_model(cfg, cfg["batch"], kv0, dict(o, attn_order=ex["attn_order"]))
            ref1.ops = P.model_graph(cfg, cfg["batch"], kv1, o)[0]
            P.encode(ref1)
            if ex["attn_order"] == 0:  # plan order does not depend on the lengths
                fresh = P.plan_model(cfg, cfg["batch"], kv1, o)
                assert np.array_equal(fresh.queue, ref1.queue)
            before = ex["queue"].copy()
            plan.set_kv_len(kv1)
            after = plan.export()["queue"]
            assert np.array_equal(after, np.asarray(ref1.queue, dtype=np.int32))
            changed = np.nonzero((before != after).any(axis=2))
            assert set(before[changed][:, 0]) <= {P.ATTN}
        finally:
            plan.free()


def test_set_kv_len_rejections():
    cfg = synth.config("tiny")
    kv = synth.kv_lengths(cfg)
    cap = synth.kv_capacity(kv)
    plan = mk.Plan.build(cfg, 1, kv, cap, num_cus=8)
    try:
        with pytest.raises(mk.MKError) as e:
            plan.set_kv_len(np.array([cap], np.int32))  # kv_len + 1 > capacity
        assert e.value.status == mk.MK_E_UNSUPPORTED
        with pytest.raises(mk.MKError) as e:  # a split past the ring: replan
            small = mk.Plan.build(cfg, 1, [10], 100000, num_cus=8, attn_splits=1)
            try:
                small.set_kv_len(np.array([99000], np.int32))
            finally:
                small.free()
        assert e.value.status == mk.MK_E_UNSUPPORTED and b"ring" in mk.lib().mk_last_error()
        assert mk.lib().mk_plan_set_kv_len(plan._h, None, None) == mk.MK_E_INVALID
    finally:
        plan.free()
    g = synth.config("glm_tiny")
    pos, _ = synth.glm_positions(g)
    gp = mk.Plan.build(g, len(pos), pos, synth.glm_capacity(g), num_cus=8)
    try:
        with pytest.raises(mk.MKError) as e:
            gp.set_kv_len(pos + 1)
        assert e.value.status == mk.MK_E_UNSUPPORTED
    finally:
        gp.free()


def test_set_kv_len_random_lengths_match_fresh_plans():
    """Property check over random mixed lengths (batch 5, fixed split count):
    moving one plan through a sequence of lengths always leaves exactly the
    queue a fresh plan for those lengths has."""
    rng = np.random.default_rng(2024)
    cfg = synth.config("tiny", batch=5, kv_len=(0, 300), seed=21)
    kv0 = synth.kv_lengths(cfg)
    cap = 400
    plan = mk.Plan.build(cfg, 5, kv0, cap, num_cus=29, attn_splits=6, attn_order=-1)
    try:
        for _ in range(6):
            kv = rng.integers(0, cap - 1, size=5).astype(np.int32)
            plan.set_kv_len(kv)
            ref = P.plan_model(cfg, 5, kv, documented_defaults(cfg, 5, kv0, 29, attn_splits=6))
            assert np.array_equal(plan.export()["queue"], np.asarray(ref.queue, dtype=np.int32))
    finally:
        plan.free()


def test_default_down_tiles_by_batch():
    """Batch 1 keeps a down tile within the compute waves' registers (64 KiB of
    weights); batched plans fill up to the 128 KiB page ring."""
    for name, overrides, want in (("llama1b", {}, 4), ("llama1b_b16", {}, 8), ("qwen3_8b", {}, 2),
                                  ("qwen3_8b", dict(batch=4, kv_len=(100, 3000), seed=3), 5)):
        cfg = synth.config(name, **overrides)
        kv = synth.kv_lengths(cfg)
        plan = mk.Plan.build(cfg, cfg["batch"], kv, synth.kv_capacity(kv), num_cus=256)
        try:
            assert plan.export()["tile_opts"]["down_rows"] == want
        finally:
            plan.free()


def test_split_rule_one_task_per_cu():
    """While the attention tasks fit on the compute units at one each, the
    split count is lowered until they fit on 7/8 of them and the per-split byte
    cap is the page ring less 64 KiB; 64 KiB otherwise.  Qwen3-8B at KV 4096
    (8 kv heads, 4097 positions, 512 bytes per position) takes 28 splits of 147
    positions (75,264 bytes) on 256 CUs, and 33 on 200 CUs, where 32 splits
    would already need 256 tasks."""
    cfg = synth.config("qwen3_8b")
    kv = synth.kv_lengths(cfg)
    for cus, want in ((256, 28), (200, 33)):
        plan = mk.Plan.build(cfg, 1, kv, synth.kv_capacity(kv), num_cus=cus)
        try:
            assert plan.export()["tile_opts"]["attn_splits"] == want
        finally:
            plan.free()


def test_streamed_attention_tasks_may_exceed_the_ring():
    """Batched head_dim-64 attention tasks stream their K/V rows through the
    page ring, so a split may be longer than the 128 KiB ring (one split of
    2041 rows = 510 KiB here); the head_dim-128 path reads its split whole and
    still rejects it, as batch 1 does."""
    cfg = synth.config("tiny")
    kv = [2040, 1100]
    plan = mk.Plan.build(dict(cfg, batch=2), 2, kv, 2080, num_cus=16, attn_splits=1)
    plan.free()
    for c, b, k in ((dict(cfg, head_dim=128, batch=2), 2, kv), (cfg, 1, [2040])):
        with pytest.raises(mk.MKError) as e:
            mk.Plan.build(c, b, k, 2080, num_cus=16, attn_splits=1)
        assert e.value.status == mk.MK_E_UNSUPPORTED and b"ring" in mk.lib().mk_last_error()
    # moving a plan to longer lengths follows the same rule
    plan = mk.Plan.build(dict(cfg, batch=2), 2, [100, 50], 2080, num_cus=16, attn_splits=1)
    try:
        plan.set_kv_len(np.array(kv, dtype=np.int32))
    finally:
        plan.free()
    plan = mk.Plan.build(dict(cfg, head_dim=128, batch=2), 2, [100, 50], 2080, num_cus=16, attn_splits=1)
    try:
        with pytest.raises(mk.MKError) as e:
            plan.set_kv_len(np.array(kv, dtype=np.int32))
        assert e.value.status == mk.MK_E_UNSUPPORTED and b"ring" in mk.lib().mk_last_error()
    finally:
        plan.free()


def test_split_rule_streamed_attention():
    """Batched head_dim-64 attention streams its K/V rows through the page
    ring, so no byte cap raises the split count: Llama-1B at batch 16 (16 x 8
    (sequence, kv head) pairs, longest KV 2016) keeps ceil(2 * 256 / 128) = 4
    splits of up to 505 positions (129,280 bytes, more than the 128 KiB ring),
    while head_dim 128 at batch 16 is still raised until a split fits 64 KiB."""
    cfg = synth.config("llama1b_b16")
    kv = synth.kv_lengths(cfg)
    assert int(kv.max()) == 2016
    plan = mk.Plan.build(cfg, 16, kv, synth.kv_capacity(kv), num_cus=256)
    try:
        assert plan.export()["tile_opts"]["attn_splits"] == 4
    finally:
        plan.free()
    q = dict(cfg, head_dim=128)
    n = int(kv.max()) + 1
    want = 4
    while -(-n // want) * 128 * 4 > 65536:
        want += 1
    plan = mk.Plan.build(q, 16, kv, synth.kv_capacity(kv), num_cus=256)
    try:
        assert plan.export()["tile_opts"]["attn_splits"] == want
    finally:
        plan.free()


def test_operand_table_layout():
    """The operand table has one row of 16 slots per op, shared by all of its
    tile instructions; the exported layout names the tensor kind of each slot
    (0 for unused ones), so it compares exactly: MegaRTP article, section 4
    ("OperandPtrTable")."""
    S = mk
    want = {
        P.QKV: [S.MK_SLOT_WQ, S.MK_SLOT_WK, S.MK_SLOT_WV, S.MK_SLOT_ATTN_NORM, "x", S.MK_SLOT_EMBED, S.MK_SLOT_TOKENS,
                S.MK_SLOT_QKV],
        P.ATTN: [S.MK_SLOT_QKV, S.MK_SLOT_K_CACHE, S.MK_SLOT_V_CACHE, S.MK_SLOT_ROPE, S.MK_SLOT_ATTN_PART],
        P.COMBINE: [S.MK_SLOT_ATTN_PART, S.MK_SLOT_ATTN_OUT],
        P.OPROJ: [S.MK_SLOT_WO, S.MK_SLOT_ATTN_OUT, "x", S.MK_SLOT_EMBED, S.MK_SLOT_TOKENS, S.MK_SLOT_HIDDEN_ATTN],
        P.GATEUP: [S.MK_SLOT_W_GATE, S.MK_SLOT_W_UP, S.MK_SLOT_FFN_NORM, S.MK_SLOT_HIDDEN_ATTN, S.MK_SLOT_FFN_ACT],
        P.DOWN: [S.MK_SLOT_W_DOWN, S.MK_SLOT_FFN_ACT, S.MK_SLOT_HIDDEN_ATTN, S.MK_SLOT_HIDDEN_FFN],
        P.LMHEAD: [S.MK_SLOT_EMBED, S.MK_SLOT_FINAL_NORM, S.MK_SLOT_HIDDEN_FFN, S.MK_SLOT_LOGITS, S.MK_SLOT_LM_MAX],
        P.ARGMAX: [S.MK_SLOT_LM_MAX, S.MK_SLOT_NEXT_TOKEN],
    }
    cfg = synth.config("tiny")
    kv = synth.kv_lengths(cfg)
    plan = mk.Plan.build(cfg, 1, kv, synth.kv_capacity(kv), num_cus=64)
    try:
        ex = plan.export()
        slots = ex["op_slots"]
        assert slots.shape == (len(ex["op_table"]), 16)
        for o, row in enumerate(ex["op_table"]):
            opcode, layer = int(row[0]), int(row[2])
            w = [(S.MK_SLOT_HIDDEN_FFN if layer else 0) if k == "x" else k for k in want[opcode]]
            assert slots[o].tolist() == w + [0] * (16 - len(w)), (o, opcode)
    finally:
        plan.free()
    # Qwen3-style: the attention row also holds the q/k norm weights; untied LM head
    cfg = synth.config("tiny", arch="qwen3", qk_norm=1, tied=0, head_dim=128)
    plan = mk.Plan.build(cfg, 1, kv, synth.kv_capacity(kv), num_cus=64)
    try:
        ex = plan.export()
        for o, row in enumerate(ex["op_table"]):
            if row[0] == P.ATTN:
                assert ex["op_slots"][o, 5:7].tolist() == [S.MK_SLOT_Q_NORM, S.MK_SLOT_K_NORM]
            if row[0] == P.LMHEAD:
                assert ex["op_slots"][o, 0] == S.MK_SLOT_LM_HEAD
    finally:
        plan.free()
    # GLM path: every op's weight slots are (codes, block scales); caches and row info
    g = synth.config("glm_tiny")
    pos, _ = synth.glm_positions(g)
    plan = mk.Plan.build(g, len(pos), pos, synth.glm_capacity(g), num_cus=8)
    try:
        ex = plan.export()
        kinds = {int(r[0]): ex["op_slots"][o].tolist() for o, r in enumerate(ex["op_table"])}
        assert kinds[P.G_A0][:7] == [S.MK_SLOT_G_X, S.MK_SLOT_G_R, S.MK_SLOT_G_ATTN_NORM, S.MK_SLOT_G_R_OUT,
                                     S.MK_SLOT_G_NORM, S.MK_SLOT_G_ACT, S.MK_SLOT_G_ACT_SCALE]
        for op in (P.G_QKVA, P.G_GATE, P.G_IDXK, P.G_QKVB, P.G_IDXQ):
            assert kinds[op][:2] == [S.MK_SLOT_G_W, S.MK_SLOT_G_W_SCALE]
        assert kinds[P.G_GATE][4] == S.MK_SLOT_G_NORM and kinds[P.G_GATE][2:4] == [0, 0]
        assert S.MK_SLOT_G_KV_CACHE in kinds[P.G_QANORM] and S.MK_SLOT_G_IDX_CACHE in kinds[P.G_IDXK]
    finally:
        plan.free()


@pytest.mark.parametrize("name,overrides,num_cus,extra", [
    ("tiny", {}, 37, dict(pairing=1)),
    ("tiny", dict(batch=3, kv_len=(0, 200), seed=11), 37, dict(pairing=1, attn_order=1)),
    ("tiny", dict(batch=6, kv_len=(1, 120), seed=15), 64, dict(attn_order=1)),
    ("tiny", dict(batch=6, kv_len=(1, 120), seed=15), 64, dict(attn_order=-1)),
    ("llama1b", {}, 256, dict(pairing=1)),
    ("llama1b", {}, 256, dict(attn_order=1)),
    ("llama1b_b16", {}, 256, dict(attn_order=1)),
    ("llama1b_b16", {}, 256, dict(pairing=1, attn_order=1)),
    ("qwen3_8b", dict(batch=4, kv_len=(100, 3000), seed=3), 256, dict(pairing=1, attn_order=1)),
])
def test_cpp_pairing_and_longest_first_match_reference(name, overrides, num_cus, extra):
    """The pairing-strategy plan (two waits on O and down) and the
    longest-first attention placement: bit-exact with the reference planner."""
    cfg = synth.config(name, **overrides)
    kv = synth.kv_lengths(cfg)
    o = documented_defaults(cfg, cfg["batch"], kv, num_cus)
    ref = P.plan_model(cfg, cfg["batch"], kv, dict(o, **documented_choices(cfg["batch"], **extra)))
    plan = mk.Plan.build(cfg, cfg["batch"], kv, synth.kv_capacity(kv), **o, **extra)
    try:
        ex = _compare(plan, ref)
        assert ex["pairing"] == extra.get("pairing", 0)
        assert ex["attn_order"] == documented_choices(cfg["batch"], **extra)["attn_order"]
        if extra.get("pairing"):
            assert (ex["queue"][:, :, P.W_WAIT_CNT] == 2).any()
    finally:
        plan.free()


def test_longest_first_lowers_the_attention_load_per_queue():
    """Variable sequence lengths at batch 16: the largest per-queue attention
    work (KV rows) of a layer drops with longest-first placement, the plan's
    events and thresholds stay the same, and tasks move only within runs of
    identical waits."""
    cfg = synth.config("llama1b_b16")
    kv = synth.kv_lengths(cfg)
    o = documented_defaults(cfg, cfg["batch"], kv, 256)
    base = P.plan_model(cfg, cfg["batch"], kv, o)
    lf = P.plan_model(cfg, cfg["batch"], kv, dict(o, attn_order=1))
    assert lf.event_target == base.event_target and lf.event_first == base.event_first
    assert lf.wait == base.wait and lf.wait2 == base.wait2

    def max_load(pl):
        ld = np.zeros(pl.num_cus, dtype=np.int64)
        for t, (op, x, y, z) in enumerate(pl.tasks):
            if pl.ops[op].opcode == P.ATTN and pl.ops[op].layer == 0:
                lo, hi = P.split_range(int(kv[x]), o["attn_splits"], z)
                ld[t % pl.num_cus] += hi - lo
        return ld.max(), ld.sum()

    (mb, sb), (ml, sl) = max_load(base), max_load(lf)
    assert sb == sl and ml < mb
    print("  max KV rows per queue, layer 0: %d -> %d (mean %.1f)" % (mb, ml, sl / base.num_cus))
    assert sorted(base.tasks) == sorted(lf.tasks)


def test_cpp_pair_plan_matches_reference_on_the_megartp_graph():
    from tests.test_planner_pins import megartp_graph
    ops, pubs, edges, _ = megartp_graph()
    ref = P.pair_plan(ops, pubs, edges, num_cus=148)
    plan = mk.Plan.pairs([(op.opcode, op.grid) for op in ops], [(p.op, p.map, p.div, p.sel) for p in pubs],
                         [(e.pub, e.cons, e.strategy, e.map, e.div) for e in edges], 148)
    try:
        ex = _compare(plan, ref)
        assert ex["pairing"] == 1 and list(ex["queue"].shape) == [148, 5, 32]
    finally:
        plan.free()
    # the host checks of the strategies, through the library
    bad = [((1, (4,)), (2, (2,))), [(0, (), (), ())], [(0, 1, mk.MK_PAIR_TILE, (), ())]]
    with pytest.raises(mk.MKError, match="tile") as e:
        mk.Plan.pairs(*bad, 8)
    assert e.value.status == mk.MK_E_INVALID
    with pytest.raises(mk.MKError, match="more than two"):
        mk.Plan.pairs([(1, (1,)), (2, (1,)), (3, (1,)), (4, (1,))], [(k, (), (), ()) for k in range(3)],
                      [(k, 3, mk.MK_PAIR_TILE, (), ()) for k in range(3)], 8)


@pytest.mark.parametrize("name,overrides", [
    ("tiny", {}), ("tiny", dict(batch=3, kv_len=(0, 200), seed=11)), ("tiny", dict(ffn=720, vocab=4100, kv_len=999)),
    ("tiny", dict(arch="qwen3", qk_norm=1, tied=0, head_dim=128)), ("llama1b_b16", {}), ("glm_tiny", {}),
])
def test_plans_satisfy_the_cached_read_layout(name, overrides):
    """Every plan's workspace passes the library's check of the cached-read
    layout (each buffer read through the caches starts its per-event slices on
    256-byte boundaries; a plan that broke it would fail to build)."""
    cfg = synth.config(name, **overrides)
    if cfg.get("arch") == "glm":
        pos, _ = synth.glm_positions(cfg)
        plan = mk.Plan.build(cfg, len(pos), pos, synth.glm_capacity(cfg), num_cus=37)
    else:
        kv = synth.kv_lengths(cfg)
        plan = mk.Plan.build(cfg, cfg["batch"], kv, synth.kv_capacity(kv), num_cus=37)
    plan.free()
    assert mk.lib().mk_last_error() == b""
