"""CPU replay of a plan's queues (test infrastructure; part of the oracle).

Models the persistent interpreter the way the CMU 15-779 lecture 7 notes do in
section 6.5: each worker walks its own queue in order; a task may start only
when the counter of the event it waits on has reached its target; finishing a
task adds one to the counter of the event it triggers.  ``order="random"``
picks a random runnable worker at each step (uneven worker speeds);
``order="serial"`` always takes the smallest runnable task id.  A state where
unfinished work remains but no worker can start raises ``Deadlock`` with the
stuck heads, the analogue of the interpreter's watchdog record.
"""
import random

from .planner import W_OPCODE, W_TASK, W_WAIT_CNT, W_WAIT_EV, W_WAIT_TGT, W_SIG_CNT, W_SIG_EV, W_SIG_INC


class Deadlock(RuntimeError):
    pass


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
                if not r[W_WAIT_CNT] or ctr[r[W_WAIT_EV]] >= r[W_WAIT_TGT]:
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
        if r[W_SIG_CNT]:
            ctr[r[W_SIG_EV]] += r[W_SIG_INC]
        head[w] += 1
        done.append(r[W_TASK])
        remaining -= 1
    return ctr, done
