"""Planner and closed forms of the oracle, pinned to the values the pages print
(tests/golden/pages_planner.json holds each value with its source)."""
import json
import math
import os

import pytest

from oracle import plan


@pytest.fixture(scope="module")
def G(golden_dir):
    with open(os.path.join(golden_dir, "pages_planner.json")) as f:
        return json.load(f)


def _model(G):
    m = G["model_tax"]
    return m["t_w_ms"], m["k_ms"], m["c_ms"], m["draft_frac"]


def _e_decay(g):
    return plan.expected_tokens_cond(plan.decaying_alphas(g), g)


def test_expected_tokens_independent(G):
    for e in G["expected_tokens"]:
        v = plan.expected_tokens_indep(e["alpha"], e["gamma"])
        assert v == pytest.approx(e["value"], rel=e["rel"])


def test_expected_tokens_limits():
    # alpha = 0: only the model's own token; alpha = 1: every draft plus one
    assert plan.expected_tokens_indep(0.0, 7) == 1.0
    assert plan.expected_tokens_indep(1.0, 7) == 8.0
    # the conditional form with a constant rate is the independent form
    for a in (0.3, 0.8, 0.97):
        for g in range(0, 9):
            assert plan.expected_tokens_cond([a] * g, g) == pytest.approx(
                plan.expected_tokens_indep(a, g), rel=1e-13)


def test_expected_tokens_decaying(G):
    e, d = G["expected_tokens_decaying"]
    assert _e_decay(e["gamma"]) == pytest.approx(e["value"], rel=e["rel"])
    gain = _e_decay(d["gamma_to"]) - _e_decay(d["gamma_from"])
    assert gain == pytest.approx(d["delta"], abs=d["abs"])


def test_crossover(G):
    tw, k, c, _ = _model(G)
    for e in G["crossover"]:
        assert plan.crossover_batch(e["gamma"], tw, k, c) == pytest.approx(e["value"], abs=e["abs"])
    # a KV term larger than the extra compute never turns compute-bound
    assert plan.crossover_batch(0, tw, 0.2, 0.1) == math.inf


def test_crossover_is_where_step_turns_compute_bound(G):
    tw, k, c, _ = _model(G)
    for g in (3, 7):
        bs = plan.crossover_batch(g, tw, k, c)
        lo, hi = math.floor(bs), math.ceil(bs)
        t = lambda b: plan.StepModel(tw, k, c).pass_time(b, g + 1)  # noqa: E731
        assert t(lo) == pytest.approx(tw + lo * k)           # memory side
        assert t(hi) == pytest.approx(hi * (g + 1) * c)      # compute side


def test_speedup_batch1(G):
    tw, k, c, f = _model(G)
    s = G["speedup_b1"]
    assert plan.speedup(s["batch"], s["gamma"], _e_decay(s["gamma"]), tw, k, c, f) == \
        pytest.approx(s["value"], abs=s["abs"])


def test_optimal_gamma(G):
    tw, k, c, f = _model(G)
    o = G["optimal_gamma"]
    for b, g in o["by_batch"].items():
        best, _ = plan.best_gamma(int(b), o["gamma_max"], _e_decay, tw, k, c, f)
        assert best == g, (b, best, g)


def test_curves_cross(G):
    tw, k, c, f = _model(G)
    cc = G["curves_cross"]
    s = lambda b, g: plan.speedup(b, g, _e_decay(g), tw, k, c, f)  # noqa: E731
    for b in range(1, cc["wins_through"] + 1):
        assert s(b, 7) > s(b, 3), b
    assert s(cc["loses_at"], 7) < s(cc["loses_at"], 3)


def test_break_even(G):
    tw, k, c, f = _model(G)
    for e in G["break_even"]:
        if e["acceptance"] == "decaying":
            eg = _e_decay(e["gamma"])
        else:
            eg = plan.expected_tokens_indep(e["acceptance"], e["gamma"])
        first = next(b for b in range(1, 5000)
                     if plan.speedup(b, e["gamma"], eg, tw, k, c, f) < 1.0)
        assert first == e["batch"], (e, first)


def test_budget(G):
    bd = G["budget"]
    n = plan.budget_tokens_from_rates(bd["decode_tok_s"], bd["compute_tok_s"])
    assert n == bd["budget_tokens"]
    for b, per in bd["per_agent"].items():
        g = plan.plan_budget(int(b), n, gamma_max=64)
        assert sum(g) / len(g) == pytest.approx(per)
        assert sum(x + 1 for x in g) <= n
    for b, free in G["budget_table"]["free_total"].items():
        g = plan.plan_budget(int(b), n, gamma_max=64)
        assert sum(g) == free


def test_budget_edges():
    assert plan.plan_budget(0, 24, 8) == []
    assert plan.plan_budget(24, 24, 8) == [0] * 24
    assert plan.plan_budget(30, 24, 8) == [0] * 30
    assert plan.plan_budget(1, 24, 8) == [8]                  # capped
    assert plan.plan_budget(16, 24, 8, fill_remainder=False) == [0] * 16
    g = plan.plan_budget(5, 24, 64)                          # 19 free over 5 agents
    assert g == [4, 4, 4, 4, 3] and sum(g) + 5 == 24


def test_plan_speedup_independent_and_decaying(G):
    tw, k, c, f = _model(G)
    gam, s, bstar = plan.plan_speedup(4, 8, [0.8], tw, k, c, f)
    assert gam == [8] * 4 and s > 1
    assert bstar == pytest.approx(plan.crossover_batch(8, tw, k, c))
    gam, _, _ = plan.plan_speedup(128, 8, plan.decaying_alphas(8), tw, k, c, f)
    assert gam == [3] * 128
