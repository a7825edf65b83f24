"""CPU replay of a plan's queues (test infrastructure; part of the oracle: only
tests, the smoke check and the benchmark's CPU leg use it).

Models the persistent interpreter the way the CMU 15-779 lecture 7 notes do in
section 6.5: each worker walks its own queue in order; a task may start only
when the counters of the events it waits on (one or two) have reached their
targets; finishing a task adds its increments to the events it signals.  ``order="random"``
picks a random runnable worker at each step (uneven worker speeds);
``order="serial"`` always takes the smallest runnable task id.  A state where
unfinished work remains but no worker can start raises ``Deadlock`` with the
stuck heads, the analogue of the interpreter's watchdog record.
"""
import random

import numpy as np

from .planner import W_OPCODE, W_TASK, W_WAIT_CNT, W_WAIT_EV, W_WAIT_TGT, W_SIG_CNT, W_SIG_EV, W_SIG_INC
from .planner import W_WAIT2_EV, W_WAIT2_TGT, W_SIG2_EV, W_SIG2_INC


class Deadlock(RuntimeError):
    pass


# (event, target) and (event, increment) word pairs of an instruction's up to
# two waits and two signals
WAITS = ((W_WAIT_EV, W_WAIT_TGT), (W_WAIT2_EV, W_WAIT2_TGT))
SIGNALS = ((W_SIG_EV, W_SIG_INC), (W_SIG2_EV, W_SIG2_INC))


def replay(queue, num_events, execute, order="serial", seed=0, workers=None):
    """queue: [C][L][32] nested lists or array.  execute(word_row) runs one task.
    Returns (counters, executed task ids in execution order)."""
    C = len(queue)
    use = range(C) if workers is None else range(min(workers, C))
    if workers is not None and workers < C:
        # fold the queues onto fewer workers while keeping each queue's order:
        # a single worker then runs all tasks in task-id order
        rows = [r for q in queue for r in q if r[W_OPCODE] != 0]
        rows.sort(key=lambda r: r[W_TASK])
        queues = [[] for _ in range(workers)]
        for i, r in enumerate(rows):
            queues[i % workers].append(r)
    else:
        queues = [[r for r in queue[c] if r[W_OPCODE] != 0] for c in use]
    head = [0] * len(queues)
    ctr = [0] * num_events
    rng = random.Random(seed)
    done = []
    remaining = sum(len(q) for q in queues)
    while remaining:
        runnable = []
        for w, q in enumerate(queues):
            if head[w] < len(q):
                r = q[head[w]]
                if all(ctr[r[ev]] >= r[tg] for ev, tg in WAITS[:r[W_WAIT_CNT]]):
                    runnable.append(w)
        if not runnable:
            stuck = [(w, queues[w][head[w]][W_TASK], queues[w][head[w]][W_WAIT_EV]) for w in range(len(queues))
                     if head[w] < len(queues[w])]
            raise Deadlock("no runnable worker; heads (worker, task, event): %s" % stuck[:8])
        if order == "random":
            w = rng.choice(runnable)
        else:
            w = min(runnable, key=lambda i: queues[i][head[i]][W_TASK])
        r = queues[w][head[w]]
        execute(r)
        for ev, inc in SIGNALS[:r[W_SIG_CNT]]:
            ctr[r[ev]] += r[inc]
        head[w] += 1
        done.append(r[W_TASK])
        remaining -= 1
    return ctr, done


# ---------------------------------------------------------------------------
# Per-tile semantics of the decode plan (O3)
# ---------------------------------------------------------------------------
def _bf16(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _to_bf16(v):
    """fp64 -> bf16 bits: one rounding, to nearest with ties to even."""
    f = np.asarray(v, dtype=np.float64)
    out = np.empty(f.shape, dtype=np.uint16)
    flat, o = f.ravel(), out.ravel()
    for i, x in enumerate(flat):
        o[i] = _round_bf16(float(x))
    return out


def _round_bf16(x):
    import math
    if math.isnan(x):
        return 0x7FC0
    s = 0x8000 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    if a == 0.0:
        return s
    if a < 2.0 ** -126:
        return s | int(round(a * 2.0 ** 133))  # round() is half-to-even
    m, e = math.frexp(a)  # a = m 2^e, m in [0.5, 1)
    q = round(m * 256.0)
    r = math.ldexp(q, e - 8)
    if r >= 2.0 ** 128:
        return s | 0x7F80
    e2 = math.frexp(r)[1] - 1  # r = 1.f * 2^e2
    return s | ((e2 + 127) << 7) | (int(math.ldexp(r, -e2) * 128) & 0x7F)


class DecodeTiles:
    """Executes the decode plan's tasks one tile at a time, in fp64, on a
    NaN-poisoned workspace: each task reads only the data of its tile's inputs
    and writes only its tile's outputs, following the payload words the
    planner encodes (CMU 15-779 lecture 7 notes, sections 5.1 and 6: QKV row
    tiles with the RMSNorm recomputed per tile, attention per (sequence, kv
    head, KV split) with RoPE and the KV-cache write, the log-sum-exp combine,
    O-projection / gate-up / down row tiles with their residual or SiLU, LM-head
    row tiles with per-tile maxima, and the argmax over the tiles in order).
    A task that runs before its inputs are written reads NaN."""

    def __init__(self, inputs, plan):
        cfg, w = inputs["cfg"], inputs["weights"]
        self.cfg, self.w = cfg, w
        self.kv_len = [int(v) for v in inputs["kv_len"]]
        self.tokens = [int(v) for v in inputs["tokens"]]
        self.kv = inputs["kv_cache"].copy()
        o = plan.info["opts"]
        self.R, self.GU, self.DR, self.LR, self.S = o["gemv_rows"], o["gateup_outs"], o["down_rows"], o["lm_rows"], \
            o["attn_splits"]
        L, B, H, F, V = cfg["n_layers"], cfg["batch"], cfg["hidden"], cfg["ffn"], cfg["vocab"]
        nq, nkv, hd = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
        self.hpg = nq // nkv
        self.RPG = (self.hpg + 2) * hd
        self.T_v = plan.info["T_v"]
        nan = lambda *shp: np.full(shp, np.nan)
        self.qkv = nan(L, B, nkv, self.RPG)
        self.part = nan(L, B, nkv, self.S, self.hpg, hd + 2)
        self.ao = nan(L, B, nq * hd)
        self.xa = nan(L, B, H)
        self.act = nan(L, B, F)
        self.xb = nan(L, B, H)
        self.logits = nan(B, V)
        self.lmmax = nan(B, self.T_v, 2)
        self.next = np.full(B, -1, dtype=np.int64)
        self.Wf = {}  # widened weights, cached

    def W(self, l, name):
        key = (l, name)
        if key not in self.Wf:
            src = self.w[name] if l is None else self.w["layers"][l][name]
            self.Wf[key] = _bf16(src)
        return self.Wf[key]

    def rms(self, x, wname, l):
        c = self.cfg
        return x / np.sqrt(np.mean(x * x) + c["rms_eps"]) * self.W(l, wname)

    def x_in(self, l, b):
        """input of layer l for sequence b: the embedding row (layer 0) or the
        previous layer's FFN output"""
        if l == 0:
            return self.W(None, "embed")[self.tokens[b]]
        return self.xb[l - 1, b]

    def rope(self, v, pos):
        c = self.cfg
        d = v.size
        half = d // 2
        i = np.arange(half)
        ang = pos * np.power(float(c["rope_theta"]), -2.0 * i / d)
        cs, sn = np.cos(ang), np.sin(ang)
        a, b = v[:half].copy(), v[half:].copy()
        return np.concatenate([a * cs - b * sn, b * cs + a * sn])

    def __call__(self, r):
        from .planner import (W_OPCODE, W_LAYER, W_GX, W_GY, W_GZ, W_PAY, QKV, ATTN, COMBINE, OPROJ, GATEUP, DOWN,
                              LMHEAD, ARGMAX)
        op, l, gx, gy, gz = r[W_OPCODE], r[W_LAYER], r[W_GX], r[W_GY], r[W_GZ]
        pay = r[W_PAY:W_PAY + 10]
        c = self.cfg
        B, H, hd, hpg = c["batch"], c["hidden"], c["head_dim"], self.hpg
        if op == QKV:
            g, row0, n = gx, pay[0], pay[1]
            qr = hpg * hd
            for b in range(B):
                y = self.rms(self.x_in(l, b), "attn_norm", l)
                for rr in range(row0, row0 + n):
                    if rr < qr:
                        w = self.W(l, "wq")[g * qr + rr]
                    elif rr < qr + hd:
                        w = self.W(l, "wk")[g * hd + rr - qr]
                    else:
                        w = self.W(l, "wv")[g * hd + rr - qr - hd]
                    self.qkv[l, b, g, rr] = w @ y
        elif op == ATTN:
            b, g, s = gx, gy, gz
            lo, hi, pos = pay[0], pay[1], pay[2]
            blk = self.qkv[l, b, g]
            knew = blk[hpg * hd:(hpg + 1) * hd].copy()
            vnew = blk[(hpg + 1) * hd:(hpg + 2) * hd].copy()
            if c["qk_norm"]:
                knew = self.rms(knew, "k_norm", l)
            knew = self.rope(knew, pos)
            kb, vb = _to_bf16(knew), _to_bf16(vnew)
            if lo <= pos < hi:  # the split that holds the new row writes it
                self.kv[l, 0, b, g, pos] = kb
                self.kv[l, 1, b, g, pos] = vb
            end = min(hi, pos + 1)
            Kp = _bf16(self.kv[l, 0, b, g, lo:min(end, pos)])
            Vp = _bf16(self.kv[l, 1, b, g, lo:min(end, pos)])
            if lo <= pos < end:
                Kp = np.vstack([Kp, _bf16(kb)[None]])
                Vp = np.vstack([Vp, _bf16(vb)[None]])
            for h in range(hpg):
                q = blk[h * hd:(h + 1) * hd].copy()
                if c["qk_norm"]:
                    q = self.rms(q, "q_norm", l)
                q = self.rope(q, pos)
                out = self.part[l, b, g, s, h]
                if Kp.shape[0] == 0:
                    out[0], out[1], out[2:] = -np.inf, 0.0, 0.0
                    continue
                sc = Kp @ q / np.sqrt(hd)
                m = sc.max()
                p = np.exp(sc - m)
                out[0], out[1], out[2:] = m, p.sum(), p @ Vp
        elif op == COMBINE:
            b, g = gx, gy
            for h in range(hpg):
                P = self.part[l, b, g, :, h]
                hq = g * hpg + h
                if np.isnan(P).any():  # a split not written yet
                    self.ao[l, b, hq * hd:(hq + 1) * hd] = np.nan
                    continue
                live = P[:, 1] > 0
                M = P[live, 0].max()
                wgt = np.where(live, np.exp(np.where(live, P[:, 0], M) - M), 0.0)
                Lsum = wgt @ np.where(live, P[:, 1], 0.0)
                o = wgt @ np.where(live[:, None], P[:, 2:], 0.0)
                self.ao[l, b, hq * hd:(hq + 1) * hd] = o / Lsum
        elif op == OPROJ:
            row0, n = pay[0], pay[1]
            for b in range(B):
                res = self.x_in(l, b)[row0:row0 + n]
                self.xa[l, b, row0:row0 + n] = res + self.W(l, "wo")[row0:row0 + n] @ self.ao[l, b]
        elif op == GATEUP:
            row0, n = pay[0], pay[1]
            for b in range(B):
                y = self.rms(self.xa[l, b], "ffn_norm", l)
                gt = self.W(l, "w_gate")[row0:row0 + n] @ y
                up = self.W(l, "w_up")[row0:row0 + n] @ y
                self.act[l, b, row0:row0 + n] = gt / (1.0 + np.exp(-gt)) * up
        elif op == DOWN:
            row0, n = pay[0], pay[1]
            for b in range(B):
                self.xb[l, b, row0:row0 + n] = self.xa[l, b, row0:row0 + n] + \
                    self.W(l, "w_down")[row0:row0 + n] @ self.act[l, b]
        elif op == LMHEAD:
            x, row0, n = gx, pay[0], pay[1]
            lm = "embed" if c["tied"] else "lm_head"
            for b in range(B):
                y = self.rms(self.xb[c["n_layers"] - 1, b], "final_norm", None)
                v = self.W(None, lm)[row0:row0 + n] @ y
                self.logits[b, row0:row0 + n] = v
                k = int(np.argmax(v))  # first maximum: the lowest index on ties
                self.lmmax[b, x] = (v[k], row0 + k) if not np.isnan(v).any() else (np.nan, -1)
        elif op == ARGMAX:
            b = gx
            best, bi = -np.inf, -1
            for t in range(self.T_v):  # tiles in order, lowest index on ties
                v, i = self.lmmax[b, t]
                if np.isnan(v):
                    best, bi = np.nan, -1
                    break
                if v > best:
                    best, bi = v, int(i)
            self.next[b] = bi
        else:
            raise ValueError("unknown opcode %d" % op)
