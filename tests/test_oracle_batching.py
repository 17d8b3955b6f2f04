"""Batching-policy oracle pinned to the static-batching page's worked example
(tests/golden/pages_batching.json: each value with its section)."""
import json
import os

import pytest

from oracle import batching as OB


@pytest.fixture(scope="module")
def G(golden_dir):
    with open(os.path.join(golden_dir, "pages_batching.json")) as fh:
        return json.load(fh)


def test_static_batch_of_the_swarm(G):
    t0, t1, L, W = G["floor_ms"], G["per_seq_ms"], G["lengths"], G["slots"]
    s = G["static"]
    steps, useful = OB.schedule(OB.STATIC, W, L)
    assert sum(L) == s["useful_tokens"] == sum(useful)
    assert len(steps) == s["steps"] and all(st.width == W for st in steps)
    assert t0 + t1 * W == pytest.approx(s["step_ms"])
    tok, sec, tps, util = OB.throughput(OB.STATIC, W, L, t0, t1)
    assert sec == pytest.approx(s["seconds"], abs=0.05)
    assert len(steps) * W == s["slots_filled"]
    assert util == pytest.approx(s["utilization"], abs=0.005)
    assert tps == pytest.approx(s["tok_s"], abs=0.5)


def test_shrinking_batch_of_the_swarm(G):
    t0, t1, L, W = G["floor_ms"], G["per_seq_ms"], G["lengths"], G["slots"]
    s = G["shrink"]
    tok, sec, tps, util = OB.throughput(OB.SHRINK, W, L, t0, t1)
    assert tps == pytest.approx(s["tok_s"], abs=0.5)
    # the tail: the last agent alone for its final 250 tokens at B = 1
    steps, _ = OB.schedule(OB.SHRINK, W, L)
    alone = [st for st in steps if st.width == 1]
    assert len(alone) == s["tail_tokens"]
    assert 1e3 / (t0 + t1) == pytest.approx(s["tail_tok_s"], abs=0.5)


def test_continuous_batching_holds_the_ceiling(G):
    t0, t1, L, W = G["floor_ms"], G["per_seq_ms"], G["lengths"], G["slots"]
    ceiling = W / ((t0 + t1 * W) / 1e3)
    assert ceiling == pytest.approx(G["continuous"]["tok_s"], abs=0.5)
    # with a queue that keeps the lanes busy (the swarm resubmitting its 8
    # requests 200 times), every step but the final drain runs full
    queue = L * 200
    tok, sec, tps, util = OB.throughput(OB.CONTINUOUS, W, queue, t0, t1)
    assert tok == sum(queue)
    assert 0.99 * ceiling < tps <= ceiling
    steps, _ = OB.schedule(OB.CONTINUOUS, W, queue)
    full = sum(1 for st in steps if st.width == W)
    assert full / len(steps) > 0.98
    # the three policies in the page's order
    t_static = OB.throughput(OB.STATIC, W, queue, t0, t1)[2]
    t_shrink = OB.throughput(OB.SHRINK, W, queue, t0, t1)[2]
    assert t_static < t_shrink < tps


def test_refill_is_next_step_and_emitted_counts():
    # a lane whose request finishes is refilled on the very next step
    steps, useful = OB.schedule(OB.CONTINUOUS, 2, [1, 3, 2])
    assert [st.slot_request for st in steps] == [[0, 1], [2, 1], [2, 1]]
    assert useful == [2, 2, 2]
    # several tokens per step (accepted drafts plus one), capped at the need
    steps, useful = OB.schedule(OB.SHRINK, 2, [5, 2], emitted_fn=lambda st, s, r: 3)
    assert [st.width for st in steps] == [2, 1] and useful == [5, 2]
    # static keeps the finished lane as padding
    steps, _ = OB.schedule(OB.STATIC, 2, [1, 3])
    assert [st.width for st in steps] == [2, 2, 2] and [st.live for st in steps] == [[1, 1], [0, 1], [0, 1]]
