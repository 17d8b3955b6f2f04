"""Iteration-level batching of a swarm of sequences (pure bookkeeping, fp64
times).  Test infrastructure; see package docstring.

Follows [static] ("Why Static Batching Wastes an RX 9070 XT Agent Swarm and
Continuous Batching Wins It Back"), sections "The whole point of batching is
a shared weight stream" (a step over B sequences costs t(B) = t0 + t1 B),
"What a draining batch actually costs" (a frozen batch keeps finished lanes
as padding until its longest member stops; a shrinking one drops them) and
"Continuous batching refills the slot instead of freezing it" (membership
is decided every step: a finished sequence leaves and a waiting one takes
its slot on the very next step).

Requests are served in submission order.  A request of n tokens is done once
it has emitted n tokens (a step may emit several, e.g. a verify pass's
accepted drafts plus one; tokens past n are not counted as useful).

Policies, with `slots` lanes:
  static      a batch takes the next `slots` waiting requests when every lane
              is free and keeps all of its lanes (finished ones as padding)
              until every member is done; a step costs t(slots taken);
  shrink      the same batches, but a finished member leaves at once: a step
              costs t(members still running);
  continuous  at every step each free lane takes the next waiting request; a
              step costs t(lanes in use).
"""
from __future__ import annotations

import dataclasses

__all__ = ["STATIC", "SHRINK", "CONTINUOUS", "Step", "schedule", "throughput"]

STATIC, SHRINK, CONTINUOUS = "static", "shrink", "continuous"


@dataclasses.dataclass
class Step:
    slot_request: list   # per lane: request id, or -1 for an empty lane
    live: list           # per lane: 1 if that request still needs tokens
    width: int           # sequences the step carries (padding lanes included)


def schedule(policy: str, slots: int, lengths, emitted_fn=None, max_steps: int = 10 ** 7):
    """The step-by-step membership of a run over the requests `lengths`
    (request r needs lengths[r] tokens).  emitted_fn(step, slot, request)
    gives the tokens a live lane emits at that step (default 1).  Returns
    (steps, useful tokens per step)."""
    lane = [-1] * slots       # request held by each lane
    left = [0] * slots        # tokens still needed by that request
    nxt = 0                   # next waiting request
    steps, useful = [], []
    n = len(lengths)
    while len(steps) < max_steps:
        # membership for this step
        if policy == CONTINUOUS:
            for s in range(slots):
                if (lane[s] < 0 or left[s] == 0) and nxt < n:
                    lane[s], left[s] = nxt, int(lengths[nxt])
                    nxt += 1
                elif lane[s] >= 0 and left[s] == 0:
                    lane[s] = -1
        else:
            if all(l < 0 or left[s] == 0 for s, l in enumerate(lane)):
                lane = [-1] * slots
                left = [0] * slots
                for s in range(slots):
                    if nxt < n:
                        lane[s], left[s] = nxt, int(lengths[nxt])
                        nxt += 1
            if policy == SHRINK:
                for s in range(slots):
                    if lane[s] >= 0 and left[s] == 0:
                        lane[s] = -1
        live = [1 if lane[s] >= 0 and left[s] > 0 else 0 for s in range(slots)]
        if not any(live):
            break
        width = sum(1 for s in range(slots) if lane[s] >= 0)
        steps.append(Step(list(lane), live, width))
        got = 0
        for s in range(slots):
            if live[s]:
                e = 1 if emitted_fn is None else int(emitted_fn(len(steps) - 1, s, lane[s]))
                take = min(e, left[s])
                left[s] -= take
                got += take
        useful.append(got)
    return steps, useful


def throughput(policy: str, slots: int, lengths, t0: float, t1: float, emitted_fn=None):
    """(useful tokens, seconds, tokens per second, utilization) of a run
    under the step-time model t(B) = t0 + t1 B milliseconds; utilization is
    useful tokens over the token slots of the steps' widths."""
    steps, useful = schedule(policy, slots, lengths, emitted_fn)
    ms = sum(t0 + t1 * st.width for st in steps)
    tok = sum(useful)
    slots_paid = sum(st.width for st in steps)
    return tok, ms / 1e3, tok / (ms / 1e3), tok / slots_paid
