"""Acceptance oracle pins.

* Exhaustive: over every draft sequence, every acceptance outcome and every
  sampling-uniform interval of the 2^-24 grid (tiny V, gamma <= 3, rows that
  do not depend on context), the k-th emitted token must be distributed as the
  target row p_k -- the lossless property of rejection sampling.
* The primer's worked example (3 of 4 accepted -> 4 tokens, none -> 1).
* Mean tokens per pass against E(alpha, gamma) under the one-hot construction.
* A chi-square test of accept_commit's emitted tokens.
* Edge cases: bonus, residual support, zero-mass fallbacks, bad tokens, greedy.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import accept as A
from oracle import plan

GRID = 1 << 24


def _first_true(lo, hi, pred):
    """Least m in [lo, hi] with pred(m) (pred monotone false->true); hi if none."""
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


def _pass_threshold(qd, pd):
    """Number of grid uniforms that pass the draft test (pass set is a prefix)."""
    return _first_true(0, GRID, lambda m: not A.passes(np.float32(m / GRID), qd, pd))


def _draw_intervals(R):
    """For each token x, (first grid index drawing x, count of grid indices)."""
    V = len(R)
    starts = [_first_true(0, GRID, lambda m, x=x: A.draw_integer_cdf(R, np.float32(m / GRID)) >= x)
              for x in range(V + 1)]
    starts[V] = GRID
    return [(starts[x], starts[x + 1] - starts[x]) for x in range(V)]


def _dyadic_rows(rng, n, V, bits=6, zero_frac=0.25):
    rows = []
    for _ in range(n):
        w = rng.integers(1, 8, size=V).astype(np.float64)
        w[rng.random(V) < zero_frac] = 0
        if w.sum() == 0:
            w[rng.integers(V)] = 1
        c = np.floor(w / w.sum() * (1 << bits))
        c[np.argmax(c)] += (1 << bits) - c.sum()
        rows.append((c / (1 << bits)).astype(np.float32))
    return np.array(rows)


@pytest.mark.parametrize("gamma,V,seed", [(1, 4, 0), (2, 4, 1), (2, 3, 2), (3, 3, 3), (3, 4, 4)])
def test_lossless_exhaustive(gamma, V, seed):
    rng = np.random.default_rng(seed)
    P = _dyadic_rows(rng, gamma + 1, V)          # target rows p_1..p_{gamma+1}
    Q = _dyadic_rows(rng, gamma, V, zero_frac=0.1)
    # one sequence: p rows stacked [gamma+1, V], q rows [gamma, V]
    marg = np.zeros((gamma + 1, V))              # P(emitted_k = x, a+1 >= k)
    reach = np.zeros(gamma + 1)                  # P(a+1 >= k)
    thr = {(j, x): _pass_threshold(Q[j, x], P[j, x]) for j in range(gamma) for x in range(V)}
    draws = {}
    for d in itertools.product(range(V), repeat=gamma):
        pd = np.prod([Q[j, d[j]] for j in range(gamma)])
        if pd == 0:
            continue
        # acceptance outcome a: drafts 1..a pass, draft a+1 fails (or a == gamma)
        for a in range(gamma + 1):
            pa, u_acc = 1.0, np.zeros(gamma, np.float32)
            for j in range(a):
                pa *= thr[(j, d[j])] / GRID
                u_acc[j] = 0.0
            if a < gamma:
                t = thr[(a, d[a])]
                pa *= 1.0 - t / GRID
                u_acc[a] = np.float32(t / GRID) if t < GRID else np.float32(0)
            if pa == 0:
                continue
            key = a if a == gamma else (a, a)
            if key not in draws:
                R = A.resample_weights(P[a], Q[a] if a < gamma else None)
                draws[key] = _draw_intervals(R)
            for x, (start, cnt) in enumerate(draws[key]):
                if cnt == 0:
                    continue
                u_s = np.float32(start / GRID)
                acc, nxt, kv, err = A.accept_commit([gamma], np.array(d, np.int32), P, Q,
                                                    u_acc, [u_s], [10])
                assert err[0] == 0 and acc[0] == a and nxt[0] == x and kv[0] == 10 + a + 1
                w = pd * pa * cnt / GRID
                emitted = list(d[:a]) + [x]
                for k, tok in enumerate(emitted):
                    marg[k, tok] += w
                    reach[k] += w
    for k in range(gamma + 1):
        assert reach[k] > 0
        cond = marg[k] / reach[k]
        np.testing.assert_allclose(cond, P[k], atol=2e-6, err_msg=f"position {k + 1}")


def test_primer_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "primer_worked_example.json")) as f:
        ex = json.load(f)
    g, V = ex["gamma"], 16
    p = np.full((g + 1, V), 1.0 / V, np.float32)
    q = np.full((g, V), 1.0 / V, np.float32)
    draft = np.arange(1, g + 1, dtype=np.int32)
    for case in ex["cases"]:
        a_want = case["accepted"]
        # p(d) = q(d) for all drafts; u < 1 passes, so force a rejection at
        # position a_want + 1 by giving that draft zero target mass
        pp = p.copy()
        if a_want < g:
            pp[a_want, draft[a_want]] = 0.0
        u = np.full(g, 0.5, np.float32)
        acc, nxt, kv, err = A.accept_commit([g], draft, pp, q, u, [0.3], [100])
        assert acc[0] == a_want
        assert acc[0] + 1 == case["tokens_emitted"]
        assert kv[0] == 100 + case["tokens_emitted"]
        assert nxt[0] != draft[a_want] if a_want < g else True


def _alpha_batch(rng, B, gamma, V, alpha):
    """One-hot drafts with target mass alpha on the draft (every test passes
    with probability alpha exactly, up to fp32 rounding of alpha)."""
    draft = rng.integers(0, V, size=B * gamma).astype(np.int32)
    q = np.zeros((B * gamma, V), np.float32)
    q[np.arange(B * gamma), draft] = 1
    base = rng.random((B * (gamma + 1), V)).astype(np.float32)
    base /= base.sum(1, keepdims=True)
    p = base.copy()
    for i in range(B):
        for j in range(gamma):
            r, dr = i * (gamma + 1) + j, i * gamma + j
            row = base[r].astype(np.float64)
            row = (1 - alpha) * row / (1 - row[draft[dr]])
            row[draft[dr]] = alpha
            p[r] = row
    u_acc = (rng.integers(0, GRID, size=B * gamma) / GRID).astype(np.float32)
    u_s = (rng.integers(0, GRID, size=B) / GRID).astype(np.float32)
    return draft, p, q, u_acc, u_s


@pytest.mark.parametrize("alpha,gamma", [(0.8, 4), (0.5, 2), (0.97, 3)])
def test_mean_tokens_matches_expected(alpha, gamma):
    rng = np.random.default_rng(7)
    B, V = 20000, 16
    draft, p, q, u_acc, u_s = _alpha_batch(rng, B, gamma, V, alpha)
    acc, nxt, kv, err = A.accept_commit(np.full(B, gamma), draft, p, q, u_acc, u_s,
                                        np.zeros(B, np.int64))
    tokens = acc + 1
    e = plan.expected_tokens_indep(alpha, gamma)
    assert abs(tokens.mean() - e) < 4 * tokens.std() / np.sqrt(B)
    # the accepted count is truncated-geometric: P(a >= k) = alpha^k
    for k in range(1, gamma + 1):
        assert abs((acc >= k).mean() - alpha ** k) < 4 * np.sqrt(alpha ** k / B)


def test_chi_square_emitted_tokens():
    from scipy import stats
    rng = np.random.default_rng(11)
    B, V, g = 60000, 8, 2
    p1 = rng.dirichlet(np.ones(V)).astype(np.float32)
    p2 = rng.dirichlet(np.ones(V)).astype(np.float32)
    p3 = rng.dirichlet(np.ones(V)).astype(np.float32)
    q1 = rng.dirichlet(np.ones(V)).astype(np.float32)
    q2 = rng.dirichlet(np.ones(V)).astype(np.float32)
    P = np.tile(np.stack([p1, p2, p3]), (B, 1))
    Q = np.tile(np.stack([q1, q2]), (B, 1))
    d1 = rng.choice(V, size=B, p=q1 / q1.sum())
    d2 = rng.choice(V, size=B, p=q2 / q2.sum())
    draft = np.stack([d1, d2], 1).reshape(-1).astype(np.int32)
    u_acc = (rng.integers(0, GRID, size=B * g) / GRID).astype(np.float32)
    u_s = (rng.integers(0, GRID, size=B) / GRID).astype(np.float32)
    acc, nxt, _, _ = A.accept_commit(np.full(B, g), draft, P, Q, u_acc, u_s, np.zeros(B))
    first = np.where(acc >= 1, d1, nxt)
    second_mask = acc >= 1
    second = np.where(acc >= 2, d2, nxt)[second_mask]
    for obs, pr in ((first, p1), (second, p2)):
        counts = np.bincount(obs, minlength=V).astype(np.float64)
        pr = pr.astype(np.float64)
        assert np.all(counts[pr == 0] == 0)
        keep = pr > 0
        exp = pr[keep] / pr[keep].sum() * counts[keep].sum()
        chi = stats.chisquare(counts[keep], exp)
        assert chi.pvalue > 1e-4, chi


def test_bonus_token_from_last_row():
    V, g = 10, 3
    p = np.full((g + 1, V), 0.1, np.float32)
    p[g] = 0
    p[g, 7] = 1.0
    q = np.full((g, V), 0.1, np.float32)
    acc, nxt, kv, _ = A.accept_commit([g], [1, 2, 3], p, q, [0.0, 0.5, 0.9], [0.99], [5])
    assert acc[0] == 3 and nxt[0] == 7 and kv[0] == 9


def test_residual_support_only():
    V = 6
    p = np.array([[0.5, 0.5, 0, 0, 0, 0], [1 / 6] * 6], np.float32)
    q = np.array([[0.0, 0.5, 0.5, 0, 0, 0]], np.float32)
    for u in np.linspace(0, 0.999, 50, dtype=np.float32):
        acc, nxt, _, _ = A.accept_commit([1], [2], p, q, [0.1], [u], [0])
        assert acc[0] == 0 and nxt[0] == 0   # only token 0 has p > q


def test_zero_mass_fallbacks():
    V = 5
    q = np.array([[0.2, 0.2, 0.2, 0.2, 0.2]], np.float32)
    p = (q / 2).astype(np.float32)
    p = np.concatenate([p, np.full((1, V), 0.2, np.float32)])
    # u = 0.75 fails (0.75*0.2 >= 0.1); residual is all zero -> draw from p row
    acc, nxt, _, _ = A.accept_commit([1], [3], p, q, [0.75], [0.5], [0])
    assert acc[0] == 0 and nxt[0] == 2
    # a zero target row on the bonus path -> argmax, lowest index
    p2 = np.zeros((1, V), np.float32)
    acc, nxt, kv, _ = A.accept_commit([0], np.zeros(0, np.int32), p2, np.zeros((0, V), np.float32),
                                      np.zeros(0, np.float32), [0.5], [4])
    assert acc[0] == 0 and nxt[0] == 0 and kv[0] == 5


def test_bad_token_leaves_sequence_uncommitted():
    V, g = 4, 2
    p = np.full((2 * (g + 1), V), 0.25, np.float32)
    q = np.full((2 * g, V), 0.25, np.float32)
    acc, nxt, kv, err = A.accept_commit([g, g], [0, 9, 1, 1], p, q, np.zeros(4), [0.1, 0.1],
                                        [7, 8])
    assert (acc[0], nxt[0], kv[0], err[0]) == (-1, -1, 7, A.ERR_BAD_TOKEN)
    assert acc[1] == 2 and kv[1] == 11 and err[1] == 0


def test_greedy_prefix_and_ties():
    V = 5
    p = np.array([[0.1, 0.4, 0.4, 0.1, 0.0],     # argmax 1 (lowest of tie)
                  [0.0, 0.0, 0.0, 0.9, 0.1],     # argmax 3
                  [0.3, 0.3, 0.4, 0.0, 0.0]], np.float32)
    q = np.zeros((2, V), np.float32)
    acc, nxt, kv, _ = A.accept_commit([2], [1, 3], p, q, [0, 0], [0], [0], greedy=True)
    assert acc[0] == 2 and nxt[0] == 2 and kv[0] == 3
    acc, nxt, _, _ = A.accept_commit([2], [2, 3], p, q, [0, 0], [0], [0], greedy=True)
    assert acc[0] == 0 and nxt[0] == 1


def test_integer_cdf_is_exact_quantised_inverse_cdf():
    R = np.array([0, 3, 0, 5, 2], np.uint64)     # S = 10
    for k in range(10):
        u = np.float32(k / 10 + 0.01)
        t = int(np.floor(np.float64(u) * 10))
        want = [1, 1, 1, 3, 3, 3, 3, 3, 4, 4][t]
        assert A.draw_integer_cdf(R, u) == want
    # weights: exact scale by 2^32, truncation, negatives clipped
    w = A.integer_weights(np.array([1.0, 0.5, 2 ** -32, 2 ** -33, -0.25], np.float32))
    assert list(w) == [2 ** 32, 2 ** 31, 1, 0, 0]


def test_position_counts_hand_example():
    # gamma, accepted -> drafts tested / accepted at positions 1..4
    gamma = [3, 2, 0, 4, 3]
    acc = [1, 2, 0, 4, -1]            # the last sequence was left uncommitted
    c = A.position_counts(gamma, acc, 4)
    np.testing.assert_array_equal(c[0], [3, 3, 1, 1])   # reached
    np.testing.assert_array_equal(c[1], [3, 2, 1, 1])   # accepted
    assert c[1].sum() == sum(a for a in acc if a > 0)
    assert A.conditional_rates(c) == [1.0, 2 / 3, 1.0, 1.0]
    assert A.conditional_rates(A.position_counts([0, 0], [0, 0], 2)) == [0.0, 0.0]


@pytest.mark.parametrize("alphas", [(0.8,) * 5, (0.94, 0.87, 0.80, 0.73, 0.66)])
def test_position_counts_recover_conditional_acceptance(alphas):
    """With acceptance alpha_k at position k given the earlier drafts passed
    (independent: all equal; the decaying reading: 94 % falling 7 points per
    position), the counters' conditional rates estimate alpha_k, not the
    unconditional P(a >= k) = prod alpha_j."""
    rng = np.random.default_rng(11)
    B, V, gamma = 30000, 16, len(alphas)
    draft, p, q, u_acc, u_s = _alpha_batch(rng, B, gamma, V, 0.5)
    # re-weight each target row so draft j is accepted with probability alpha_j
    base = p.copy()
    for i in range(B):
        for j in range(gamma):
            r, dr = i * (gamma + 1) + j, i * gamma + j
            row = base[r].astype(np.float64)
            row = (1 - alphas[j]) * row / (1 - row[draft[dr]])
            row[draft[dr]] = alphas[j]
            p[r] = row
    acc, _, _, _ = A.accept_commit(np.full(B, gamma), draft, p, q, u_acc, u_s, np.zeros(B, np.int64))
    c = A.position_counts(np.full(B, gamma), acc, gamma)
    rates = A.conditional_rates(c)
    for k in range(gamma):
        n = c[0, k]
        assert n == (acc >= k).sum()
        assert abs(rates[k] - alphas[k]) < 4 * np.sqrt(alphas[k] * (1 - alphas[k]) / n), (k, rates[k])
    # the expected tokens of the estimated rates match the measured mean
    e = plan.expected_tokens_cond(rates, gamma)
    assert abs((acc + 1).mean() - e) < 0.02 * e
