"""Reference tile planner (test infrastructure; part of the oracle).

Turns an operator DAG into the static per-CU instruction queues that the HIP
library's planner must reproduce bit for bit.  Written from the pages, not
from the library:

* Tiles and events.  Each operator is cut into tasks over a grid of up to
  three axes; an edge producer -> consumer over a tensor carries, per tensor
  dimension d, ``event_dim[d] = gcd(prod_part[d], cons_part[d])`` where a part
  is the grid extent of the axis that the operator's map sends to d (1 if none)
  -- MPK notes (dpshk.com), section "fine-grained pipeline" (build_partition /
  event_dim).  Counters count completions only; a consumer waits until its
  event has seen all of its producers -- MegaRTP article, section 4 "TaskGraph"
  (pairing strategies whole / tile / tile_cover / tile_reduce).
* Fork producers: the producer-side spans of all out-edges are brought to
  their lcm so one event set serves every branch; join consumers: the
  consumer-side spans of all in-edges are brought to their lcm and a join event
  counts the producers of every edge in its slice -- MPK notes, "handling fork
  producer" / "handling join consumer" worked examples.
* Linearization: operators in topological order; for each event (lexicographic,
  last axis fastest) the event is created, its successor tasks are appended
  contiguously, and the producer tasks of its slice are given it as their
  trigger -- MPK notes, "building the SM-level DAG".
* Placement: task t goes to queue t mod C at slot t div C; short queues are
  padded with NoOp rows, giving int32[C, max_len, 32] -- MegaRTP article,
  section 4 "KernelPlan" and section 3 (Stanford megakernels).

Readings where the pages are silent (each listed in the design notes):
  - residual edges: an edge P -> C is dropped when another kept in-edge X -> C
    already makes every task of C wait for every task of P (transitively);
  - a component of edges that is neither a chain, a pure fork nor a pure join
    falls back to one event for the whole component (the "whole" strategy);
  - gcd slices must cut the tensor at the same element boundaries on both
    sides (ragged last tiles); otherwise that dimension falls back to 1 event;
  - a chain or join enumerates events over the consumer's grid axes, a fork
    over the producer's, lexicographically with the last axis fastest.
"""
from math import gcd
from itertools import product

import numpy as np

WORDS = 32
MAX_DIMS = 4

# instruction word layout
W_OPCODE, W_SPEC, W_OPROW, W_WAIT_CNT, W_WAIT_EV, W_WAIT_TGT = 0, 1, 2, 3, 4, 5
W_SIG_CNT, W_SIG_EV, W_SIG_INC, W_TASK, W_LAYER, W_GX, W_GY, W_GZ, W_PAY = 6, 7, 8, 9, 10, 11, 12, 13, 14
N_PAY = 10

# opcodes of the Llama-family decode step
NOOP, QKV, ATTN, COMBINE, OPROJ, GATEUP, DOWN, LMHEAD, ARGMAX = range(9)
# opcodes of the GLM-style pre-attention path
G_A0, G_QKVA, G_GATE, G_IDXK, G_QANORM, G_QKVB, G_IDXQ, G_GATE_RED = range(9, 17)
GLM_ROWS = 16  # weight rows per fp8 GEMM tile (the matrix-core M dimension)
GATE_BLOCKS = 4  # 128-column blocks per head-gate K-split tile


def lcm(a, b):
    return a * b // gcd(a, b)


def ceil_div(a, b):
    return -(-a // b)


class Op:
    def __init__(self, name, opcode, grid, layer=0, spec=0, payload=None):
        g = tuple(grid) + (1,) * (3 - len(grid))
        assert all(v >= 1 for v in g)
        self.name, self.opcode, self.grid, self.layer, self.spec = name, opcode, g, layer, spec
        self.payload = payload or (lambda x, y, z: ())


class Edge:
    """producer/consumer op indices; maps give, per grid axis (x, y, z), the tensor
    dimension that axis partitions (-1 for none).  ``extent`` is the tensor's size
    per dimension and ``ptile`` / ``ctile`` the elements one producer / consumer
    tile covers along each dimension (used only to check ragged alignment)."""

    def __init__(self, prod, cons, out_map, in_map, extent=None, ptile=None, ctile=None, name=""):
        self.prod, self.cons, self.name = prod, cons, name
        self.out_map = tuple(out_map) + (-1,) * (3 - len(out_map))
        self.in_map = tuple(in_map) + (-1,) * (3 - len(in_map))
        self.extent, self.ptile, self.ctile = extent, ptile, ctile


def build_partition(grid, amap):
    part = [1] * MAX_DIMS
    for a in range(3):
        if amap[a] >= 0:
            part[amap[a]] *= grid[a]
    return part


class Plan:
    pass


def plan_graph(ops, edges, num_cus):
    n_ops = len(ops)
    # --- 1. per-edge gcd partition (+ ragged alignment check) ---------------
    evd = []
    for e in edges:
        P, C = ops[e.prod], ops[e.cons]
        pp = build_partition(P.grid, e.out_map)
        cp = build_partition(C.grid, e.in_map)
        ed = [gcd(pp[d], cp[d]) for d in range(MAX_DIMS)]
        if e.extent is not None:
            for d in range(MAX_DIMS):
                g = ed[d]
                if g <= 1:
                    continue
                ext = e.extent[d]
                for i in range(1, g):
                    bp = min(i * (pp[d] // g) * e.ptile[d], ext)
                    bc = min(i * (cp[d] // g) * e.ctile[d], ext)
                    if bp != bc:
                        ed[d] = 1
                        break
        evd.append(ed)

    def is_whole(i):
        return all(v == 1 for v in evd[i])

    # --- 2. residual stripping (full-dependency sets) ------------------------
    in_edges = [[] for _ in range(n_ops)]
    for i, e in enumerate(edges):
        assert e.prod < e.cons, "ops must be listed in topological order"
        in_edges[e.cons].append(i)
    fd = [set() for _ in range(n_ops)]
    kept = [True] * len(edges)
    for c in range(n_ops):
        for i in in_edges[c]:
            p = edges[i].prod
            for j in in_edges[c]:
                if j != i and edges[j].prod != p and p in fd[edges[j].prod]:
                    kept[i] = False
                    break
        for i in in_edges[c]:
            if kept[i]:
                x = edges[i].prod
                fd[c] |= fd[x]
                if is_whole(i):
                    fd[c].add(x)
    kedges = [i for i in range(len(edges)) if kept[i]]

    # --- 3. components of kept edges (shared producer or shared consumer) -----
    parent = {i: i for i in kedges}

    def find(i):
        while parent[i] != i:
            parent[i] = parent[parent[i]]
            i = parent[i]
        return i

    by_prod, by_cons = {}, {}
    for i in kedges:
        by_prod.setdefault(edges[i].prod, []).append(i)
        by_cons.setdefault(edges[i].cons, []).append(i)
    for grp in list(by_prod.values()) + list(by_cons.values()):
        for i in grp[1:]:
            a, b = find(grp[0]), find(i)
            if a != b:
                parent[max(a, b)] = min(a, b)
    comps = {}
    for i in kedges:
        comps.setdefault(find(i), []).append(i)
    comp_of_cons = {}
    kind = {}
    for root, es in comps.items():
        prods = sorted({edges[i].prod for i in es})
        conss = sorted({edges[i].cons for i in es})
        pairs = {(edges[i].prod, edges[i].cons) for i in es}
        if len(es) == 1:
            k = "chain"
        elif len(pairs) != len(es):
            k = "mixed"
        elif len(prods) == 1 and all(len(by_cons[c]) == 1 for c in conss):
            k = "fork"
        elif len(conss) == 1 and all(len(by_prod[p]) == 1 for p in prods):
            k = "join"
        else:
            k = "mixed"
        kind[root] = k
        if k == "mixed":
            for i in es:
                evd[i] = [1] * MAX_DIMS
        for c in conss:
            comp_of_cons[c] = root
        # components emit when their first consumer is visited: every producer must precede it
        assert max(prods) < min(conss), "component producers must precede its consumers"

    # --- 4. fork / join lcm normalization ------------------------------------
    for root, es in comps.items():
        if kind[root] == "fork":
            P = ops[edges[es[0]].prod]
            for a in range(3):
                spans = []
                for i in es:
                    d = edges[i].out_map[a]
                    ev = evd[i][d] if d >= 0 else 1
                    spans.append(P.grid[a] // ev)
                Lx = 1
                for s in spans:
                    Lx = lcm(Lx, s)
                for i in es:
                    d = edges[i].out_map[a]
                    if d >= 0:
                        evd[i][d] = P.grid[a] // Lx if P.grid[a] % Lx == 0 else 1
        elif kind[root] == "join":
            C = ops[edges[es[0]].cons]
            for a in range(3):
                spans = []
                for i in es:
                    d = edges[i].in_map[a]
                    ev = evd[i][d] if d >= 0 else 1
                    spans.append(C.grid[a] // ev)
                Lx = 1
                for s in spans:
                    Lx = lcm(Lx, s)
                for i in es:
                    d = edges[i].in_map[a]
                    if d >= 0:
                        evd[i][d] = C.grid[a] // Lx if C.grid[a] % Lx == 0 else 1

    # --- 5. linearization -----------------------------------------------------
    tasks = []  # (op, x, y, z)
    task_of = {}
    trig, wait = [], []
    ev_first, ev_last, ev_ntrig = [], [], []
    emitted = [False] * n_ops

    def new_task(o, x, y, z):
        task_of[(o, x, y, z)] = len(tasks)
        tasks.append((o, x, y, z))
        trig.append(-1)
        wait.append(-1)

    def axis_ranges(grid, amap, ed, idx_of_dim):
        """per grid axis: range of task coordinates in the slice whose per-tensor-dim
        event index is idx_of_dim[d]"""
        rs = []
        for a in range(3):
            d = amap[a]
            if d >= 0 and ed[d] > 1:
                span = grid[a] // ed[d]
                i = idx_of_dim[d]
                rs.append(range(i * span, (i + 1) * span))
            else:
                rs.append(range(grid[a]))
        return rs

    def emit_event(cons_slices, prod_slices):
        eid = len(ev_first)
        ev_first.append(len(tasks))
        for o, rs in cons_slices:
            for x, y, z in product(*rs):
                new_task(o, x, y, z)
                wait[-1] = eid
        ev_last.append(len(tasks))
        n = 0
        for o, rs in prod_slices:
            for x, y, z in product(*rs):
                t = task_of[(o, x, y, z)]
                assert trig[t] == -1, "a task triggers at most one event"
                trig[t] = eid
                n += 1
        ev_ntrig.append(n)

    for c in range(n_ops):
        if emitted[c]:
            continue
        C = ops[c]
        if c not in comp_of_cons:
            for x, y, z in product(range(C.grid[0]), range(C.grid[1]), range(C.grid[2])):
                new_task(c, x, y, z)
            emitted[c] = True
            continue
        root = comp_of_cons[c]
        es = comps[root]
        k = kind[root]
        if k in ("chain", "join"):
            i0 = es[0]
            # consumer-axis event grid
            nev = []
            for a in range(3):
                d = edges[i0].in_map[a]
                nev.append(evd[i0][d] if d >= 0 else 1)
            for ix, iy, iz in product(range(nev[0]), range(nev[1]), range(nev[2])):
                cidx = (ix, iy, iz)
                cons_rs = []
                for a in range(3):
                    span = C.grid[a] // nev[a]
                    cons_rs.append(range(cidx[a] * span, (cidx[a] + 1) * span))
                prod_slices = []
                for i in es:
                    e = edges[i]
                    idx_of_dim = [0] * MAX_DIMS
                    for a in range(3):
                        if e.in_map[a] >= 0:
                            idx_of_dim[e.in_map[a]] = cidx[a]
                    prod_slices.append((e.prod, axis_ranges(ops[e.prod].grid, e.out_map, evd[i], idx_of_dim)))
                emit_event([(c, cons_rs)], prod_slices)
            emitted[c] = True
        elif k == "fork":
            p = edges[es[0]].prod
            P = ops[p]
            nev = []
            for a in range(3):
                d = edges[es[0]].out_map[a]
                nev.append(evd[es[0]][d] if d >= 0 else 1)
            order = sorted(es, key=lambda i: edges[i].cons)
            for ix, iy, iz in product(range(nev[0]), range(nev[1]), range(nev[2])):
                pidx = (ix, iy, iz)
                prod_rs = []
                for a in range(3):
                    span = P.grid[a] // nev[a]
                    prod_rs.append(range(pidx[a] * span, (pidx[a] + 1) * span))
                cons_slices = []
                for i in order:
                    e = edges[i]
                    idx_of_dim = [0] * MAX_DIMS
                    for a in range(3):
                        if e.out_map[a] >= 0:
                            idx_of_dim[e.out_map[a]] = pidx[a]
                    cons_slices.append((e.cons, axis_ranges(ops[e.cons].grid, e.in_map, evd[i], idx_of_dim)))
                emit_event(cons_slices, [(p, prod_rs)])
            for i in es:
                emitted[edges[i].cons] = True
        else:  # mixed: one event for the whole component
            conss = sorted({edges[i].cons for i in es})
            prods = sorted({edges[i].prod for i in es})
            full = lambda o: [range(ops[o].grid[a]) for a in range(3)]
            emit_event([(o, full(o)) for o in conss], [(o, full(o)) for o in prods])
            for o in conss:
                emitted[o] = True

    # --- 6. placement and encoding -------------------------------------------
    T = len(tasks)
    max_len = max(1, ceil_div(T, num_cus))
    queue = np.zeros((num_cus, max_len, WORDS), dtype=np.int32)
    for t, (o, x, y, z) in enumerate(tasks):
        op = ops[o]
        w = queue[t % num_cus, t // num_cus]
        w[W_OPCODE] = op.opcode
        w[W_SPEC] = op.spec
        w[W_OPROW] = o
        if wait[t] >= 0:
            w[W_WAIT_CNT], w[W_WAIT_EV], w[W_WAIT_TGT] = 1, wait[t], ev_ntrig[wait[t]]
        if trig[t] >= 0:
            w[W_SIG_CNT], w[W_SIG_EV], w[W_SIG_INC] = 1, trig[t], 1
        w[W_TASK] = t
        w[W_LAYER] = op.layer
        w[W_GX], w[W_GY], w[W_GZ] = x, y, z
        pay = tuple(op.payload(x, y, z))
        assert len(pay) <= N_PAY
        for j, v in enumerate(pay):
            w[W_PAY + j] = int(v)

    pl = Plan()
    pl.num_cus, pl.max_len, pl.num_tasks, pl.num_events = num_cus, max_len, T, len(ev_first)
    pl.queue = queue
    pl.tasks, pl.trigger, pl.wait = tasks, trig, wait
    pl.event_first, pl.event_last, pl.event_target = ev_first, ev_last, ev_ntrig
    pl.kept = kept
    pl.evd = evd
    pl.kind = {tuple(sorted(es)): kind[r] for r, es in comps.items()}
    pl.ops = ops
    pl.edges = edges
    return pl


# ---------------------------------------------------------------------------
# Llama-family decode step as an operator DAG
# ---------------------------------------------------------------------------
# The pages fix no tile size and no split count (the CMU 15-779 lecture 7 notes,
# section 5.1, use 16-row tiles and 16 KV splits as one example), so the
# reference planner takes all of them as inputs; the library chooses its own
# and both are fed the same values.
MODEL_OPTS = ("num_cus", "gemv_rows", "gateup_outs", "down_rows", "lm_rows", "attn_splits")


def check_opts(opts):
    """Every entry of MODEL_OPTS must be given, as a positive int."""
    missing = [k for k in MODEL_OPTS if not (opts or {}).get(k)]
    if missing:
        raise ValueError("the reference planner needs every tile option given explicitly; missing %s" % missing)
    return {k: int(opts[k]) for k in MODEL_OPTS}


def split_range(pos, S, s):
    """positions [lo, hi) of split s when pos + 1 positions are cut into S splits"""
    n = pos + 1
    sz = ceil_div(n, S)
    lo = min(s * sz, n)
    hi = min(lo + sz, n)
    return lo, hi


def glm_graph(desc, M):
    """GLM-style pre-attention path (MegaRTP article, section 4, "OpGraph"/"TaskGraph":
    A0 works one token row per tile; GEMMs are cut into output-row tiles; the
    QKV-A, head-gate and indexer-K branches hang off A0 independently; the q path
    (RMSNorm + requant of QKV-A's q columns, one row per tile) feeds QKV-B and
    indexer-Q).  QKV-B tiles: per head, nope/16 plain 16-row tiles, then rope/16
    tiles that pair 8 rows of the first half of the rope dims with the 8 rows
    rope/2 further on, so one tile holds both members of its RoPE pairs.
    Payload: A0 / q-norm (row); GEMMs (row0, nrows, second-segment row0 or -1)."""
    H, QL, KL, RD = desc["hidden"], desc["q_lora"], desc["kv_lora"], desc["rope_dim"]
    nh, hd = desc["n_q_heads"], desc["head_dim"]
    NOPE, R = hd - RD, GLM_ROWS
    Na = QL + KL + RD
    Ng, Nk, Niq = desc["n_gate"], desc["idx_head_dim"], desc["n_idx_heads"] * desc["idx_head_dim"]
    assert NOPE % R == 0 and RD % R == 0
    ops, edges = [], []

    def add(op):
        ops.append(op)
        return len(ops) - 1

    def rows(N):
        return lambda x, y, z: (x * R, min(R, N - x * R), -1)

    def qb_rows(x, y, z):
        if y < NOPE // R:
            return (x * hd + y * R, R, -1)
        j = y - NOPE // R
        return (x * hd + NOPE + j * (R // 2), R // 2, x * hd + NOPE + RD // 2 + j * (R // 2))

    # the head gate is cut along K too (GATE_BLOCKS blocks of 128 columns per
    # task) and a reduce op adds each row tile's partials: the tile_reduce
    # pairing of the MegaRTP article, section 4 ("TaskGraph")
    nkb = H // 128
    GS, Tg = ceil_div(nkb, GATE_BLOCKS), ceil_div(Ng, R)
    a0 = add(Op("a0", G_A0, (M,), 0, 0, lambda x, y, z: (x,)))
    qa = add(Op("qkva", G_QKVA, (ceil_div(Na, R),), 0, 0, rows(Na)))
    ga = add(Op("gate", G_GATE, (Tg, GS), 0, 0,
                lambda x, y, z: (x * R, min(R, Ng - x * R), -1, y * GATE_BLOCKS, min(GATE_BLOCKS, nkb - y * GATE_BLOCKS))))
    ik = add(Op("idxk", G_IDXK, (ceil_div(Nk, R),), 0, 0, rows(Nk)))
    gr = add(Op("gate_red", G_GATE_RED, (Tg,), 0, 0, lambda x, y, z: (x * R, min(R, Ng - x * R), GS)))
    qn = add(Op("qanorm", G_QANORM, (M,), 0, 0, lambda x, y, z: (x,)))
    qb = add(Op("qkvb", G_QKVB, (nh, (NOPE + RD) // R), 0, 0, qb_rows))
    iq = add(Op("idxq", G_IDXQ, (ceil_div(Niq, R),), 0, 0, rows(Niq)))
    for c in (qa, ga, ik):
        edges.append(Edge(a0, c, (0,), (), [M, H, 1, 1], [1, H, 1, 1], [M, H, 1, 1], "act"))
    edges.append(Edge(ga, gr, (1,), (1,), [M, Ng, 1, 1], [M, R, 1, 1], [M, R, 1, 1], "gate_part"))
    edges.append(Edge(qa, qn, (1,), (0,), [M, Na, 1, 1], [M, R, 1, 1], [1, Na, 1, 1], "qkva"))
    for c in (qb, iq):
        edges.append(Edge(qn, c, (0,), (), [M, QL, 1, 1], [1, QL, 1, 1], [M, QL, 1, 1], "qa"))
    return ops, edges, dict(opts=dict(num_cus=0))


def model_graph(desc, batch, kv_len, opts):
    """The decode step's operators per layer -- QKV (RMSNorm fused), attention
    (RoPE, KV write, split-KV partials), combine, O projection (+ residual),
    gate/up (RMSNorm and SiLU fused), down (+ residual) -- then the LM head
    (final RMSNorm fused) and argmax: the chain of the CMU 15-779 lecture 7
    notes, sections 2 and 5.1.  opts: MODEL_OPTS, all explicit."""
    if desc.get("arch") == "glm":
        ops, edges, info = glm_graph(desc, batch)
        return ops, edges, info
    o = check_opts(opts)
    H, nq, nkv, hd = desc["hidden"], desc["n_q_heads"], desc["n_kv_heads"], desc["head_dim"]
    F, V, L = desc["ffn"], desc["vocab"], desc["n_layers"]
    B = batch
    hpg = nq // nkv
    RPG = (hpg + 2) * hd
    R, GU, DR, LR = o["gemv_rows"], o["gateup_outs"], o["down_rows"], o["lm_rows"]
    assert RPG % R == 0 and hd % R == 0
    T_qkv, T_o, T_f, T_d, T_v = RPG // R, ceil_div(H, R), ceil_div(F, GU), ceil_div(H, DR), ceil_div(V, LR)
    S = o["attn_splits"]
    spec = 1 if B > 4 else 0
    ops, edges = [], []

    def add(op):
        ops.append(op)
        return len(ops) - 1

    prev_down = None
    for l in range(L):
        q = add(Op("qkv%d" % l, QKV, (nkv, T_qkv), l, spec, lambda x, y, z: (y * R, R)))
        a = add(Op("attn%d" % l, ATTN, (B, nkv, S), l, 0,
                   lambda x, y, z: split_range(int(kv_len[x]), S, z) + (int(kv_len[x]),)))
        c = add(Op("combine%d" % l, COMBINE, (B, nkv), l, 0, lambda x, y, z: (S,)))
        op_ = add(Op("oproj%d" % l, OPROJ, (T_o,), l, spec, lambda x, y, z: (x * R, min(R, H - x * R))))
        g = add(Op("gateup%d" % l, GATEUP, (T_f,), l, spec, lambda x, y, z: (x * GU, min(GU, F - x * GU))))
        d = add(Op("down%d" % l, DOWN, (T_d,), l, spec, lambda x, y, z: (x * DR, min(DR, H - x * DR), 0, F)))
        if prev_down is not None:
            edges.append(Edge(prev_down, q, (1,), (), [B, H, 1, 1], [1, DR, 1, 1], [1, H, 1, 1], "xb"))
        edges.append(Edge(q, a, (1, 2), (0, 1), [B, nkv, RPG, 1], [B, 1, R, 1], [1, 1, RPG, 1], "qkv"))
        edges.append(Edge(a, c, (0, 1, 2), (0, 1), [B, nkv, S, 1], [1, 1, 1, 1], [1, 1, S, 1], "part"))
        edges.append(Edge(c, op_, (0, 1), (), [B, nkv, 1, 1], [1, 1, 1, 1], [B, nkv, 1, 1], "ao"))
        if prev_down is not None:
            edges.append(Edge(prev_down, op_, (1,), (), [B, H, 1, 1], [1, DR, 1, 1], [1, H, 1, 1], "xb_res"))
        edges.append(Edge(op_, g, (1,), (), [B, H, 1, 1], [1, R, 1, 1], [1, H, 1, 1], "xa"))
        edges.append(Edge(op_, d, (1,), (), [B, H, 1, 1], [1, R, 1, 1], [1, H, 1, 1], "xa_res"))
        edges.append(Edge(g, d, (1,), (), [B, F, 1, 1], [1, GU, 1, 1], [1, F, 1, 1], "act"))
        prev_down = d
    lm = add(Op("lmhead", LMHEAD, (T_v,), L, spec, lambda x, y, z: (x * LR, min(LR, V - x * LR))))
    am = add(Op("argmax", ARGMAX, (B,), L, 0, lambda x, y, z: (T_v,)))
    edges.append(Edge(prev_down, lm, (1,), (), [B, H, 1, 1], [1, DR, 1, 1], [1, H, 1, 1], "xb"))
    edges.append(Edge(lm, am, (1,), (0,), [B, T_v, 1, 1], [B, 1, 1, 1], [1, T_v, 1, 1], "lmmax"))
    return ops, edges, dict(S=S, T_qkv=T_qkv, T_o=T_o, T_f=T_f, T_d=T_d, T_v=T_v, spec=spec, opts=o)


def plan_model(desc, batch, kv_len, opts):
    """opts: num_cus (GLM path), or every entry of MODEL_OPTS (Llama family)."""
    if desc.get("arch") == "glm":
        if not (opts or {}).get("num_cus"):
            raise ValueError("num_cus must be given")
        o = dict(num_cus=int(opts["num_cus"]))
    else:
        o = check_opts(opts)
    ops, edges, info = model_graph(desc, batch, kv_len, o)
    pl = plan_graph(ops, edges, o["num_cus"])
    pl.info = info
    return pl


def op_table(pl):
    """[num_ops][8] int32 rows: opcode, spec, layer, gx, gy, gz, ntasks, 0"""
    rows = []
    for op in pl.ops:
        rows.append([op.opcode, op.spec, op.layer, op.grid[0], op.grid[1], op.grid[2],
                     op.grid[0] * op.grid[1] * op.grid[2], 0])
    return rows
