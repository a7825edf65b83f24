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
# second wait and second signal, and the publication of each signal (pairing plans)
W_WAIT2_EV, W_WAIT2_TGT, W_SIG2_EV, W_SIG2_INC, W_SIG_PUB, W_SIG2_PUB = 24, 25, 26, 27, 28, 29

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
    pl = Plan()
    pl.num_cus, pl.num_tasks, pl.num_events = num_cus, T, len(ev_first)
    pl.tasks, pl.trigger, pl.wait = tasks, trig, wait
    pl.trigger2, pl.wait2 = [-1] * T, [-1] * T
    pl.event_first, pl.event_last, pl.event_target = ev_first, ev_last, ev_ntrig
    pl.kept = kept
    pl.evd = evd
    pl.kind = {tuple(sorted(es)): kind[r] for r, es in comps.items()}
    pl.ops = ops
    pl.edges = edges
    encode(pl)
    return pl


# ---------------------------------------------------------------------------
# Pairing strategies (MegaRTP article, section 4, "TaskGraph")
# ---------------------------------------------------------------------------
# An op publishes one or more outputs ("publications"); an edge reads one
# publication of an earlier op under one of four pairing strategies.  A
# publication's output is cut into regions: the region of a producer tile is
# its grid coordinates mapped and divided per region dimension, and only the
# tiles a publication selects publish (a split-K op whose last split writes the
# final tile publishes from that split only).  Each region that some consumer
# reads becomes one counter event; every publishing tile adds one; the event's
# threshold is the number of its publishing tiles.  The strategies differ only
# in what the host checks (the device sees counters and thresholds alone):
#   whole       -- one region, every producer tile publishes: the consumer
#                  waits for the whole producer;
#   tile        -- one producer tile per region (threshold 1);
#   tile_cover  -- several disjoint producer tiles make up the region;
#   tile_reduce -- several partials of one region (the same count for every
#                  region the edge reads).
# An instruction waits on up to two events (the page's D1 waits on two, a
# join) and signals up to two (its A0 publishes two outputs).  Tasks are
# listed op by op, each op's grid in row-major order (last axis fastest), and
# events are numbered in the order consumers first wait on them; placement is
# round-robin as in ``plan_graph``.  Readings (where the page leaves a step
# open): the region map (divide the mapped coordinate), the publisher selection
# (a fixed index per axis) and the numbering orders above.
WHOLE, TILE, TILE_COVER, TILE_REDUCE = range(4)
PAIR_NAMES = ("whole", "tile", "tile_cover", "tile_reduce")


def _pad3(v, fill):
    v = tuple(v)
    return v + (fill,) * (3 - len(v))


class Pub:
    """Publication of op ``op``.  Region dim r of producer tile c is
    c[map[r]] // div[r] (0 where map[r] is -1); tile c publishes only if
    c[a] == sel[a] for every axis a with sel[a] >= 0."""

    def __init__(self, op, map=(), div=(), sel=(), name=""):
        self.op, self.name = op, name
        self.map, self.div, self.sel = _pad3(map, -1), _pad3(div, 1), _pad3(sel, -1)


class PairEdge:
    """Consumer ``cons`` reads publication ``pub``; the region a consumer tile c
    waits on has dim r = c[map[r]] // div[r] (0 where map[r] is -1)."""

    def __init__(self, pub, cons, strategy, map=(), div=(), name=""):
        self.pub, self.cons, self.strategy, self.name = pub, cons, strategy, name
        self.map, self.div = _pad3(map, -1), _pad3(div, 1)


def _region(coord, amap, div):
    return tuple(coord[amap[r]] // div[r] if amap[r] >= 0 else 0 for r in range(3))


def pair_plan(ops, pubs, edges, num_cus):
    """Plan an op graph whose edges carry pairing strategies (see above)."""
    n_ops = len(ops)
    for p in pubs:
        if not 0 <= p.op < n_ops:
            raise ValueError("publication of an unknown op")
        for r in range(3):
            if p.map[r] >= 3 or p.div[r] < 1 or (p.sel[r] >= 0 and p.sel[r] >= ops[p.op].grid[r]):
                raise ValueError("publication map/div/sel out of range")
    for e in edges:
        if not 0 <= e.pub < len(pubs) or not pubs[e.pub].op < e.cons < n_ops:
            raise ValueError("an edge must read a publication of an earlier op")
        if e.strategy not in (WHOLE, TILE, TILE_COVER, TILE_REDUCE):
            raise ValueError("unknown pairing strategy")
        if any(e.map[r] >= 3 or e.div[r] < 1 for r in range(3)):
            raise ValueError("edge map/div out of range")

    def nregions(p):
        g = ops[p.op].grid
        return tuple(ceil_div(g[p.map[r]], p.div[r]) if p.map[r] >= 0 else 1 for r in range(3))

    def pub_region(p, c):
        if any(p.sel[a] >= 0 and c[a] != p.sel[a] for a in range(3)):
            return None
        return _region(c, p.map, p.div)

    # publishing tiles per (publication, region)
    count = [{} for _ in pubs]
    for k, p in enumerate(pubs):
        for c in product(*(range(v) for v in ops[p.op].grid)):
            r = pub_region(p, c)
            if r is not None:
                count[k][r] = count[k].get(r, 0) + 1

    tasks = [(o,) + c for o in range(n_ops) for c in product(*(range(v) for v in ops[o].grid))]
    in_edges = [[] for _ in range(n_ops)]
    for i, e in enumerate(edges):
        in_edges[e.cons].append(i)
    ev_of, ev_target, ev_pub, ev_tasks = {}, [], [], []
    reduce_n = {}
    waits = []
    for t, (o, x, y, z) in enumerate(tasks):
        w = []
        for i in in_edges[o]:
            e = edges[i]
            p = pubs[e.pub]
            r = _region((x, y, z), e.map, e.div)
            if any(r[d] >= nregions(p)[d] for d in range(3)):
                raise ValueError("edge %d: consumer tile %s reads region %s outside the publication" % (i, (x, y, z), r))
            n = count[e.pub].get(r, 0)
            if n == 0:
                raise ValueError("edge %d: region %s has no publishing tile" % (i, r))
            if e.strategy == WHOLE and (nregions(p) != (1, 1, 1) or any(s >= 0 for s in p.sel)):
                raise ValueError("edge %d: 'whole' needs one region that every producer tile publishes" % i)
            if e.strategy == TILE and n != 1:
                raise ValueError("edge %d: 'tile' needs one producer tile per region" % i)
            if e.strategy == TILE_REDUCE and reduce_n.setdefault(i, n) != n:
                raise ValueError("edge %d: 'tile_reduce' regions must have equal partial counts" % i)
            key = (e.pub, r)
            if key not in ev_of:
                ev_of[key] = len(ev_target)
                ev_target.append(n)
                ev_pub.append(e.pub)
                ev_tasks.append([])
            ev = ev_of[key]
            if ev not in w:
                w.append(ev)
                ev_tasks[ev].append(t)
        if len(w) > 2:
            raise ValueError("task %s waits on more than two events" % ((o, x, y, z),))
        waits.append(w)
    pubs_of = [[k for k, p in enumerate(pubs) if p.op == o] for o in range(n_ops)]
    sigs = []
    for (o, x, y, z) in tasks:
        s = []
        for k in pubs_of[o]:
            r = pub_region(pubs[k], (x, y, z))
            if r is not None and (k, r) in ev_of:
                s.append((ev_of[(k, r)], k))
        if len(s) > 2:
            raise ValueError("task %s signals more than two events" % ((o, x, y, z),))
        sigs.append(s)

    pl = Plan()
    T = len(tasks)
    pl.num_cus, pl.num_tasks, pl.num_events = num_cus, T, len(ev_target)
    pl.tasks = tasks
    pl.wait = [w[0] if w else -1 for w in waits]
    pl.wait2 = [w[1] if len(w) > 1 else -1 for w in waits]
    pl.trigger = [s[0][0] if s else -1 for s in sigs]
    pl.trigger2 = [s[1][0] if len(s) > 1 else -1 for s in sigs]
    pl.sig_pub = [[k for _, k in s] for s in sigs]
    pl.event_target, pl.event_pub = ev_target, ev_pub
    # successors of a pairing event need not be contiguous: [first, last) spans them
    pl.event_first = [ts[0] for ts in ev_tasks]
    pl.event_last = [ts[-1] + 1 for ts in ev_tasks]
    pl.ops, pl.pubs, pl.edges = ops, pubs, edges
    pl.kept = [True] * len(edges)
    encode(pl)
    return pl


def encode(pl):
    """Place task t in queue t mod C at slot t div C and write its 32 words."""
    T, C = pl.num_tasks, pl.num_cus
    pl.max_len = max(1, ceil_div(T, C))
    queue = np.zeros((C, pl.max_len, WORDS), dtype=np.int32)
    sig_pub = getattr(pl, "sig_pub", None)
    for t, (o, x, y, z) in enumerate(pl.tasks):
        op = pl.ops[o]
        w = queue[t % C, t // C]
        w[W_OPCODE], w[W_SPEC], w[W_OPROW] = op.opcode, op.spec, o
        if pl.wait[t] >= 0:
            w[W_WAIT_CNT], w[W_WAIT_EV], w[W_WAIT_TGT] = 1, pl.wait[t], pl.event_target[pl.wait[t]]
            if pl.wait2[t] >= 0:
                w[W_WAIT_CNT], w[W_WAIT2_EV], w[W_WAIT2_TGT] = 2, pl.wait2[t], pl.event_target[pl.wait2[t]]
        if pl.trigger[t] >= 0:
            w[W_SIG_CNT], w[W_SIG_EV], w[W_SIG_INC] = 1, pl.trigger[t], 1
            if sig_pub is not None:
                w[W_SIG_PUB] = sig_pub[t][0]
            if pl.trigger2[t] >= 0:
                w[W_SIG_CNT], w[W_SIG2_EV], w[W_SIG2_INC], w[W_SIG2_PUB] = 2, pl.trigger2[t], 1, sig_pub[t][1]
        w[W_TASK], w[W_LAYER] = t, op.layer
        w[W_GX], w[W_GY], w[W_GZ] = x, y, z
        pay = tuple(op.payload(x, y, z))
        assert len(pay) <= N_PAY
        for j, v in enumerate(pay):
            w[W_PAY + j] = int(v)
    pl.queue = queue
    return queue


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


def model_pairs(ops):
    """Publications and pairing edges of the Llama-family decode step over the
    ops of ``model_graph`` (six per layer -- QKV, attention, combine, O, gate/up,
    down -- then LM head and argmax).  QKV tiles cover their kv head's q/k/v
    rows (one region per kv head); attention splits are partials of their
    (sequence, kv head) region, reduced by combine; every other input is read
    whole.  The residual inputs stay explicit: O waits on combine and on the
    previous layer's down, down on gate/up and on O (two waits each)."""
    L = (len(ops) - 2) // 6
    pubs, edges = [], []

    def pub(op, **kw):
        pubs.append(Pub(op, **kw))
        return len(pubs) - 1

    prev_d = None
    for l in range(L):
        q, a, c, o, g, d = range(6 * l, 6 * l + 6)
        pq = pub(q, map=(0,), name="qkv%d" % l)
        pa = pub(a, map=(0, 1), name="part%d" % l)
        pc = pub(c, name="ao%d" % l)
        po = pub(o, name="xa%d" % l)
        pg = pub(g, name="act%d" % l)
        if prev_d is not None:
            edges.append(PairEdge(prev_d, q, WHOLE, name="xb"))
        edges.append(PairEdge(pq, a, TILE_COVER, map=(1,), name="qkv"))
        edges.append(PairEdge(pa, c, TILE_REDUCE, map=(0, 1), name="part"))
        edges.append(PairEdge(pc, o, WHOLE, name="ao"))
        if prev_d is not None:
            edges.append(PairEdge(prev_d, o, WHOLE, name="xb_res"))
        edges.append(PairEdge(po, g, WHOLE, name="xa"))
        edges.append(PairEdge(pg, d, WHOLE, name="act"))
        edges.append(PairEdge(po, d, WHOLE, name="xa_res"))
        prev_d = pub(d, name="xb%d" % l)
    lm, am = 6 * L, 6 * L + 1
    edges.append(PairEdge(prev_d, lm, WHOLE, name="xb"))
    edges.append(PairEdge(pub(lm, name="lmmax"), am, WHOLE, name="lmmax"))
    return pubs, edges


def balance_attention(pl, kv_len, S):
    """Longest-first placement of the attention tasks (CMU 15-779 lecture 7
    notes, section 6.4: variable-length tasks placed longest first).  Within
    each run of consecutive attention tasks with identical waits (one event's
    consumers: any order within the run keeps every dependency), the tasks are
    taken longest first (KV rows of their split; ties in task order) and each
    is put on the free position of the run whose compute unit holds the least
    attention work of that op so far (ties: the lowest position).  Positions
    keep their compute unit (t mod C), so only which task lands where changes."""
    C, T = pl.num_cus, pl.num_tasks
    ops = pl.ops
    rows = lambda t: (lambda lo_hi: lo_hi[1] - lo_hi[0])(split_range(int(kv_len[pl.tasks[t][1]]), S, pl.tasks[t][3]))
    load = {}
    t = 0
    while t < T:
        o = pl.tasks[t][0]
        if ops[o].opcode != ATTN:
            t += 1
            continue
        e = t + 1
        while e < T and pl.tasks[e][0] == o and (pl.wait[e], pl.wait2[e]) == (pl.wait[t], pl.wait2[t]):
            e += 1
        ld = load.setdefault(o, [0] * C)
        run = list(range(t, e))
        order = sorted(run, key=lambda u: (-rows(u), u))
        free = list(run)
        new_at = {}
        for u in order:
            pos = min(free, key=lambda v: (ld[v % C], v))
            free.remove(pos)
            new_at[pos] = u
            ld[pos % C] += rows(u)
        old = [(pl.tasks[u], pl.trigger[u], pl.trigger2[u]) for u in run]
        for pos in run:
            pl.tasks[pos], pl.trigger[pos], pl.trigger2[pos] = old[new_at[pos] - t]
        if getattr(pl, "sig_pub", None) is not None:
            sp = [pl.sig_pub[u] for u in run]
            for pos in run:
                pl.sig_pub[pos] = sp[new_at[pos] - t]
        t = e


def plan_model(desc, batch, kv_len, opts):
    """opts: num_cus (GLM path), or every entry of MODEL_OPTS (Llama family);
    optionally ``pairing`` (1: plan with the pairing strategies of
    ``model_pairs`` instead of the gcd/lcm rules) and ``attn_order`` (1:
    longest-first attention placement, ``balance_attention``)."""
    if desc.get("arch") == "glm":
        if not (opts or {}).get("num_cus"):
            raise ValueError("num_cus must be given")
        o = dict(num_cus=int(opts["num_cus"]))
    else:
        o = check_opts(opts)
    pairing, attn_order = int((opts or {}).get("pairing", 0)), int((opts or {}).get("attn_order", 0))
    ops, edges, info = model_graph(desc, batch, kv_len, o)
    if pairing and desc.get("arch") != "glm":
        pubs, pedges = model_pairs(ops)
        pl = pair_plan(ops, pubs, pedges, o["num_cus"])
    else:
        pl = plan_graph(ops, edges, o["num_cus"])
    if attn_order and desc.get("arch") != "glm":
        balance_attention(pl, kv_len, o["attn_splits"])
        encode(pl)
    pl.info = info
    return pl


def op_table(pl):
    """[num_ops][8] int32 rows: opcode, spec, layer, gx, gy, gz, ntasks, 0"""
    rows = []
    for op in pl.ops:
        rows.append([op.opcode, op.spec, op.layer, op.grid[0], op.grid[1], op.grid[2],
                     op.grid[0] * op.grid[1] * op.grid[2], 0])
    return rows
