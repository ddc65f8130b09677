"""A CPU model of the persistent executor's dependency protocol, run on the
planner's real task graph (mk_inspect_plan): one thread per worker runs its
queue in list order, step after step, with random delays.

Counter edges: a task reports its completions (sig_count of them) by adding
to the event's counter; a waiter of step e needs counter >= (e + 1) *
threshold (counters are never reset between steps).  Split attention: the
split that arrives last for its (layer, slot, KV head), counted on an arrival
counter, merges the group and reports its one completion.  Data edges: every
producer unit writes its outputs with the step's tag; a reader accepts them
only when all of them carry the current step's tag.  Every wait has a budget;
an exceeded budget records the first error (task, event) and every worker
stops at its next wait (the Mirage MPK summary, "Part 2. Runtime": workers
run their task queues and bump event counters; the Cohere article, "Egyetlen
tartós kernelre épül a kiszolgálás": counters in global memory instead of
barriers).

Checked: with random delays every task runs exactly once per step and starts
after every producer of its inputs finished; one withheld counter increment,
or one producer that never tags its outputs, ends in a reported timeout of
the waiting task on that event, and every worker thread exits.
"""
import random
import threading
import time

import pytest

from persistent_runtime_amd import mk
from synth.configs import TINY

ATTN = mk.OP_ID["ATTN"]


class Sim:
    def __init__(self, tasks, thr, S, budget=2.0, seed=0, withhold=None, untagged=None):
        self.tasks, self.thr, self.S = tasks, thr, S
        self.budget, self.withhold, self.untagged = budget, withhold, untagged
        self.rng_seed = seed
        self.lock = threading.Lock()
        self.count = [0] * len(thr)
        self.arrive = {}
        self.tags = {}          # (event, producer unit) -> tag
        self.units = {}         # event -> set of producer units (data edges)
        for i, t in enumerate(tasks):
            for k in range(t.n_sig):
                if t.data_edges >> (3 + k) & 1:
                    self.units.setdefault(t.sig_ev[k], set()).add(self._unit(i))
        self.error = None
        self.clock = 0
        self.start, self.finish, self.runs = {}, {}, {}

    def _unit(self, i):
        t = self.tasks[i]
        if t.op == ATTN and self.S > 1:
            return ("group", t.layer, t.a0, t.a1)
        return ("task", i)

    def _tick(self):
        with self.lock:
            self.clock += 1
            return self.clock

    def _fail(self, task, ev):
        with self.lock:
            if self.error is None:
                self.error = (task, ev)

    def _wait(self, i, epoch, tag, rng):
        t = self.tasks[i]
        for k in range(t.n_wait):
            e = t.wait_ev[k]
            data = t.data_edges >> k & 1
            t0 = time.monotonic()
            while True:
                with self.lock:
                    if data:
                        ok = all(self.tags.get((e, u)) == tag for u in self.units[e])
                    else:
                        ok = self.count[e] >= (epoch + 1) * self.thr[e]
                    err = self.error is not None
                if ok:
                    break
                if err:
                    return False
                if time.monotonic() - t0 > self.budget:
                    self._fail(i, e)
                    return False
                time.sleep(rng.random() * 1e-4)
        return True

    def _signal(self, i, epoch, tag):
        t = self.tasks[i]
        report = t.sig_count
        if t.op == ATTN and self.S > 1:
            key = (t.layer, t.a0, t.a1)
            with self.lock:
                self.arrive[key] = self.arrive.get(key, 0) + 1
                report = 1 if self.arrive[key] == (epoch + 1) * self.S else 0
        for k in range(t.n_sig):
            e = t.sig_ev[k]
            if t.data_edges >> (3 + k) & 1:
                if report or not (t.op == ATTN and self.S > 1):
                    if (e, i) != self.untagged:
                        with self.lock:
                            self.tags[(e, self._unit(i))] = tag
            elif report and i != self.withhold:
                with self.lock:
                    self.count[e] += report

    def worker(self, queue, steps, wid):
        rng = random.Random(self.rng_seed * 1000 + wid)
        for epoch in range(steps):
            tag = epoch + 1
            for i in queue:
                if not self._wait(i, epoch, tag, rng):
                    return
                self.start[(epoch, i)] = self._tick()
                time.sleep(rng.random() * 2e-4)
                self.runs[(epoch, i)] = self.runs.get((epoch, i), 0) + 1
                self.finish[(epoch, i)] = self._tick()
                self._signal(i, epoch, tag)

    def run(self, steps, n_workers):
        queues = [[] for _ in range(n_workers)]
        for i, t in enumerate(self.tasks):
            queues[t.worker].append(i)
        th = [threading.Thread(target=self.worker, args=(q, steps, w), daemon=True)
              for w, q in enumerate(queues)]
        for x in th:
            x.start()
        for x in th:
            x.join(timeout=60)
        return all(not x.is_alive() for x in th)


def _plan(**kw):
    cfg = mk.make_config(TINY, max_batch=2, max_pages_per_seq=8)
    opts = mk.default_options(n_cus=8, attn_splits=2, attn_pool=-1, **kw)
    tasks, thr = mk.inspect_plan(cfg, opts)
    S = sum(1 for t in tasks if t.op == ATTN and t.layer == 0 and t.a0 == 0 and t.a1 == 0)
    return tasks, thr, S


def _producers(tasks):
    sig = {}
    for i, t in enumerate(tasks):
        for k in range(t.n_sig):
            sig.setdefault(t.sig_ev[k], []).append(i)
    return sig


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_protocol_runs_every_task_once_in_dependency_order(seed):
    tasks, thr, S = _plan()
    assert S == 2 and any(t.data_edges for t in tasks) and any(
        t.n_sig and not (t.data_edges >> 3 & 1) for t in tasks)
    sim = Sim(tasks, thr, S, seed=seed)
    assert sim.run(steps=3, n_workers=8)
    assert sim.error is None
    sig = _producers(tasks)
    for epoch in range(3):
        for c, t in enumerate(tasks):
            assert sim.runs[(epoch, c)] == 1
            for k in range(t.n_wait):
                for p in sig[t.wait_ev[k]]:
                    assert sim.finish[(epoch, p)] < sim.start[(epoch, c)], (epoch, p, c)


def _first_counter_signal(tasks, op):
    for i, t in enumerate(tasks):
        if mk.OPS[t.op] == op and t.sig_count > 0 and t.n_sig and not (t.data_edges >> 3 & 1):
            return i, t.sig_ev[0]
    raise AssertionError(f"no counter-signalling {op} task")


def test_dropped_counter_increment_ends_in_timeout():
    """One LM-head task never reports: the argmax task's wait on the LM-head
    event exceeds its budget in the step where the increment is missing,
    the error names that task and event, and every worker exits."""
    tasks, thr, S = _plan()
    lm, ev = _first_counter_signal(tasks, "LMHEAD")
    sim = Sim(tasks, thr, S, budget=0.3, withhold=lm)
    assert sim.run(steps=2, n_workers=8), "a worker did not exit"
    args = [i for i, t in enumerate(tasks) if mk.OPS[t.op] == "ARGMAX" and ev in
            list(t.wait_ev)[:t.n_wait]]  # one per slot
    task, e = sim.error
    assert task in args and e == ev, sim.error
    assert (0, task) not in sim.start  # it never ran: its wait gave up


def test_untagged_data_edge_ends_in_timeout():
    """One projection tile never tags its outputs (a data edge): the
    consumer that reads the whole vector waits past its budget and reports
    that event; every worker exits."""
    tasks, thr, S = _plan()
    i, e = next((i, t.sig_ev[0]) for i, t in enumerate(tasks)
                if mk.OPS[t.op] == "DOWN" and t.layer == 0 and t.data_edges >> 3 & 1)
    sim = Sim(tasks, thr, S, budget=0.3, untagged=(e, i))
    assert sim.run(steps=1, n_workers=8), "a worker did not exit"
    assert sim.error is not None and sim.error[1] == e
    assert e in list(tasks[sim.error[0]].wait_ev)[:tasks[sim.error[0]].n_wait]
