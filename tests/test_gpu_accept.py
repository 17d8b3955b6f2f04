"""GPU acceptance/commit parity: bit-exact against the oracle given the same
probabilities and uniforms, at the workloads' batch shapes and full vocabulary,
plus the statistical pins (E(alpha, gamma), chi-square) on the GPU kernel."""
import numpy as np
import pytest

from gpu_helpers import accept_inputs, oracle_accept, run_accept, say, sv
from workloads import custom_workload, workload, SHAPES

pytestmark = pytest.mark.gpu


def _exact(wl, inp, V, kv=None, greedy=False):
    kv = wl.ctx if kv is None else kv
    mode = sv.SV_ACCEPT_GREEDY if greedy else sv.SV_ACCEPT_STOCHASTIC
    a, y, k, err = run_accept(wl.gamma, V, inp, kv, mode)
    ra, ry, rk, rerr = oracle_accept(wl.gamma, inp, kv, greedy=greedy)
    np.testing.assert_array_equal(a, ra)
    np.testing.assert_array_equal(y, ry)
    np.testing.assert_array_equal(k, rk)
    assert (err != 0) == bool(rerr.any())
    return a, y


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_accept_bit_exact_workload_shapes(cid):
    wl = workload(cid)
    V = wl.shape.vocab
    say(f"accept parity workload {cid}: B={wl.B} T={wl.T} V={V}")
    alphas = wl.alphas or (None,)
    for a in alphas:
        inp = accept_inputs(wl, V, alpha=a)
        acc, _ = _exact(wl, inp, V)
        say(f"  alpha={a} mean accepted {acc.mean():.3f}")


@pytest.mark.parametrize("greedy", [False, True])
def test_accept_bit_exact_large_batch(greedy):
    """Batches above the size whose token map travels with the launch: the
    kernel builds each sequence's row offsets on the device."""
    sh = SHAPES["tiny"]
    rng = np.random.default_rng(77)
    gam = rng.integers(0, 5, size=300)
    ctx = rng.integers(0, 1000, size=300)
    wl = custom_workload(sh, "f32", gam, ctx, draft="noise", seed=77)
    V = 3001
    inp = accept_inputs(wl, V, target_logits=rng.standard_normal((wl.T, V)).astype(np.float32) * 2)
    a, _ = _exact(wl, inp, V, greedy=greedy)
    say(f"accept B=300 greedy={greedy}: mean accepted {a.mean():.3f}")


@pytest.mark.parametrize("greedy", [False, True])
def test_accept_ragged_small_vocab(greedy):
    sh = SHAPES["tiny"]
    for seed in range(6):
        rng = np.random.default_rng(seed)
        gam = rng.integers(0, 9, size=rng.integers(1, 40))
        ctx = rng.integers(0, 500, size=len(gam))
        wl = custom_workload(sh, "f32", gam, ctx, draft="noise", seed=seed)
        V = int(rng.integers(2, 20000))
        inp = accept_inputs(wl, V, target_logits=rng.standard_normal((wl.T, V)).astype(np.float32) * 3)
        _exact(wl, inp, V, greedy=greedy)


def test_accept_edge_cases():
    sh = SHAPES["tiny"]
    # all gamma 0 (plain decode: only the bonus draw)
    wl = custom_workload(sh, "f32", [0] * 5, [3] * 5, draft="noise", seed=1)
    inp = accept_inputs(wl, 64, target_logits=np.random.default_rng(1).standard_normal((5, 64)).astype(np.float32))
    a, _ = _exact(wl, inp, 64)
    assert (a == 0).all()
    # bad draft ids leave their sequence uncommitted, others commit
    wl = custom_workload(sh, "f32", [2, 3, 1], [4, 5, 6], draft="noise", seed=2)
    inp = accept_inputs(wl, 50, target_logits=np.random.default_rng(2).standard_normal((wl.T, 50)).astype(np.float32))
    inp["draft"] = inp["draft"].copy()
    inp["draft"][3] = 50       # second sequence, first draft out of range
    a, y = _exact(wl, inp, 50)
    assert a[1] == -1 and y[1] == -1
    # zero-mass residual and zero target row fallbacks
    V = 16
    wl = custom_workload(sh, "f32", [1, 0], [0, 0], draft="noise", seed=3)
    inp = {"draft": np.array([3], np.int32), "q": np.full((1, V), 1 / V, np.float32),
           "u_acc": np.array([0.75], np.float32), "u_samp": np.array([0.5, 0.5], np.float32)}
    p = np.zeros((3, V), np.float32)
    p[0] = 0.5 / V      # p = q / 2: rejected at u = 0.75, residual all zero -> draw from p
    inp["p"] = p        # rows 1 (bonus of seq 0) and 2 (seq 1) are all zero -> argmax
    _exact(wl, inp, V)


def test_accept_mean_tokens_gpu():
    """Mean (a + 1) against E(alpha, gamma) under the one-hot construction."""
    from oracle.plan import expected_tokens_indep
    sh = SHAPES["tiny"]
    B, g, V, alpha = 4096, 4, 512, 0.8
    wl = custom_workload(sh, "f32", [g] * B, [0] * B, draft="alpha", alphas=(alpha,), seed=5)
    inp = accept_inputs(wl, V, alpha=alpha)
    a, _, _, _ = run_accept(wl.gamma, V, inp, wl.ctx)
    tok = a + 1
    e = expected_tokens_indep(alpha, g)
    say(f"mean tokens {tok.mean():.4f} vs E={e:.4f}")
    assert abs(tok.mean() - e) < 4 * tok.std() / np.sqrt(B)


def test_accept_chi_square_gpu():
    from scipy import stats
    sh = SHAPES["tiny"]
    rng = np.random.default_rng(9)
    Bc, calls, V = 4096, 50, 8       # 204800 sequences in calls of 4096
    p1, p2 = rng.dirichlet(np.ones(V)).astype(np.float32), rng.dirichlet(np.ones(V)).astype(np.float32)
    q1 = rng.dirichlet(np.ones(V)).astype(np.float32)
    wl = custom_workload(sh, "f32", [1] * Bc, [0] * Bc, seed=9)
    firsts = []
    for _ in range(calls):
        d = rng.choice(V, size=Bc, p=q1 / q1.sum()).astype(np.int32)
        inp = {"draft": d, "q": np.tile(q1, (Bc, 1)), "p": np.tile(np.stack([p1, p2]), (Bc, 1)),
               "u_acc": (rng.integers(0, 1 << 24, Bc) / 2 ** 24).astype(np.float32),
               "u_samp": (rng.integers(0, 1 << 24, Bc) / 2 ** 24).astype(np.float32)}
        a, y, _, _ = run_accept(wl.gamma, V, inp, wl.ctx)
        firsts.append(np.where(a >= 1, d, y))
    first = np.concatenate(firsts)
    B = len(first)
    counts = np.bincount(first, minlength=V).astype(np.float64)
    exp = p1.astype(np.float64) / p1.sum() * B
    chi = stats.chisquare(counts, exp)
    say(f"chi-square p={chi.pvalue:.3g}")
    assert chi.pvalue > 1e-4
