"""2-D Greedy Overlapping Optimization (GOO) step planner, written from the pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[Mesh] section 3.4.  A GPU's Q partitions are cut into k_Q chunks and its KV
partitions into k_KV chunks.  The collectives become chunk tasks AG-Q-i,
RS-Q-i (i < k_Q) and AG-KV-j (j < k_KV); the attention tile becomes compute
tasks C-i-j.  C-i-j is ready once AG-Q-i and AG-KV-j are done; RS-Q-i is ready
once every C-i-j (j < k_KV) is done.  The planner builds steps; a step runs one
communication task and zero or more compute tasks that were ready when the step
began, and everything in a step ends before the next one starts.

Choice of the communication task: among the candidates, the largest
profit(c) = T_unlock(c) / T_comm(c), where T_unlock(c) is the compute time that
becomes ready when c completes.  Compute tasks of the step: ready ones, added
until their summed time reaches T_target(c) = gamma * T_comm(c).  When no
communication task can run but computation is ready, a compute-only step runs one
ready compute task.

Readings where the text leaves a choice open (each checked against the worked
example of Figure 4, which they reproduce step by step):
  * candidates are the lowest-index unscheduled chunk of each collective type
    (RS-Q only once ready);
  * ties in profit go to AG-KV, then AG-Q, then RS-Q;
  * ready compute tasks are taken in (i, j) order, and one is added while the
    running sum is below T_target (the last one may pass it);
  * T_unlock sums the newly ready tasks' times in (i, j) order.

Tasks are written ("AG-Q", i), ("AG-KV", j), ("RS-Q", i) and ("C", i, j).
"""
from __future__ import annotations


def plan(kq, kkv, t_agq, t_agkv, t_rsq, t_c, gamma):
    """Steps of the greedy schedule: a list of (comm task or None, [compute tasks]).

    t_c: compute time of C-i-j, either one number or a kq x kkv nested list."""
    def tc(i, j):
        return t_c[i][j] if isinstance(t_c, (list, tuple)) else t_c

    t_comm = {"AG-Q": t_agq, "AG-KV": t_agkv, "RS-Q": t_rsq}
    done = set()           # finished tasks
    ran = set()            # compute tasks already placed in a step
    steps = []
    n_comm = {"AG-Q": kq, "AG-KV": kkv, "RS-Q": kq}

    def c_ready(i, j, finished):
        return ("AG-Q", i) in finished and ("AG-KV", j) in finished

    def rs_ready(i, finished):
        return all(("C", i, j) in finished for j in range(kkv))

    while True:
        # candidates: the lowest-index unscheduled chunk of each type, in tie-break order
        cands = []
        for kind in ("AG-KV", "AG-Q", "RS-Q"):
            idx = next((x for x in range(n_comm[kind]) if (kind, x) not in done), None)
            if idx is None:
                continue
            if kind == "RS-Q" and not rs_ready(idx, done):
                continue
            cands.append((kind, idx))
        ready = [("C", i, j) for i in range(kq) for j in range(kkv)
                 if ("C", i, j) not in ran and c_ready(i, j, done)]
        if not cands:
            if not ready:
                break
            # compute-only step: one ready compute task
            steps.append((None, [ready[0]]))
            ran.add(ready[0])
            done.add(ready[0])
            continue
        best, best_profit = None, None
        for c in cands:
            after = done | {c}
            unlock = 0.0
            for i in range(kq):
                for j in range(kkv):
                    t = ("C", i, j)
                    if t not in ran and not c_ready(i, j, done) and c_ready(i, j, after):
                        unlock += tc(i, j)
            profit = unlock / t_comm[c[0]]
            if best is None or profit > best_profit:
                best, best_profit = c, profit
        target = gamma * t_comm[best[0]]
        chosen, total = [], 0.0
        for t in ready:
            if total >= target:
                break
            chosen.append(t)
            total += tc(t[1], t[2])
        steps.append((best, chosen))
        done.add(best)
        for t in chosen:
            ran.add(t)
            done.add(t)
    return steps
