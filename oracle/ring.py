"""Event schedule of the N-stage circular buffer (oracle).

Source: "Add TMA support for circular buffering pass" (nvFuser PR #2833),
sections "Description", "Loop Structure" and "Detailed Pseudo-Code":

* pre-prologue: allocate the stages (and, on that hardware, one completion
  barrier per stage);
* prologue: issue the loads of the first ``stages - 1`` iterations;
* main loop, for ``i`` in ``[0, N - (stages - 1))``: issue the load of
  iteration ``i + stages - 1`` into stage ``(i + stages - 1) % stages``, wait
  for the current stage ``i % stages``, compute;
* epilogue, for ``i`` in ``[N - (stages - 1), N)``: wait for stage
  ``i % stages``, compute (no loads);
* post-epilogue: release the per-stage barriers.

Readings: when ``N < stages - 1`` the prologue issues only ``N`` loads and
the epilogue starts at 0 (the page's bounds assume ``N >= stages - 1``).
The same formulas with one stage give load, wait, compute per iteration
(no overlap); the one-tile-per-workgroup copy and elementwise calls use it.  The
load of iteration ``j`` always goes to stage ``j % stages`` (for
``j = i + stages - 1`` this is the page's ``load_stage`` formula).

Per-wait counter.  On the target the completion of a stage is tracked by the
in-order count of a wave's outstanding memory operations: the wait for
iteration ``i`` may leave outstanding exactly the operations issued after
the last load of iteration ``i``.  ``schedule`` simulates the issued
operation stream (``loads`` memory ops per load step, ``stores`` per compute
step) and counts them; it does not use any closed form.
"""
from __future__ import annotations

from dataclasses import dataclass

LOAD, WAIT, CONSUME = 0, 1, 2


@dataclass(frozen=True)
class Event:
    kind: int
    iteration: int
    stage: int
    count: int = 0   # for WAIT: operations allowed to stay outstanding


def schedule(n_iters: int, stages: int, loads: int = 1, stores: int = 0):
    if stages < 1:
        raise ValueError("a ring needs at least 1 stage")
    events = []
    issued = []          # the memory-op stream: iteration tag per op ("L", j) or ("S", i)

    def load(j):
        events.append(Event(LOAD, j, j % stages))
        issued.extend([("L", j)] * loads)

    def wait_and_consume(i):
        last = max(k for k, op in enumerate(issued) if op == ("L", i))
        events.append(Event(WAIT, i, i % stages, len(issued) - 1 - last))
        events.append(Event(CONSUME, i, i % stages))
        issued.extend([("S", i)] * stores)

    prologue = min(stages - 1, n_iters)
    for j in range(prologue):
        load(j)
    main = max(0, n_iters - (stages - 1))
    for i in range(main):
        load(i + stages - 1)
        wait_and_consume(i)
    for i in range(main, n_iters):
        wait_and_consume(i)
    return events

