"""Token-tree oracle pins.

1. Structure: depths and ancestor masks of a hand-drawn tree.
2. Verify: a chain tree is exactly the linear verify pass (also over int8
   caches); every node of a branching tree equals the linear pass over its
   own root path (a node sees only its ancestors, also over int8 caches), so
   siblings do not affect each other.
3. Accept: on a chain the tree rule is the linear rule bit for bit (both
   modes); with several children drawn i.i.d. from the parent's draft
   distribution the first emitted token is distributed as the target row,
   checked by exact enumeration over the whole 2^-24 uniform grid.
4. Commit: the accepted path's rows move to ctx + depth.
"""
import numpy as np
import pytest

from oracle import accept as OA
from oracle import tree as OT
from oracle import verify as OV
from workloads import Shape, hidden_states, kv_cache, kv_cache_int8, layer_weights

SMALL = Shape(d=128, n_q=4, n_kv=2, hd=32, ffn=192, vocab=300)
GRID = 1 << 24


def test_depths_and_masks_hand_example():
    #        0
    #      / | \
    #     1  2  3
    #    / \     \
    #   4   5     6
    #   |
    #   7
    par = [-1, 0, 0, 0, 1, 1, 3, 4]
    np.testing.assert_array_equal(OT.depths(par), [0, 1, 1, 1, 2, 2, 2, 3])
    m = OT.ancestor_masks(par)
    want = [0b1, 0b11, 0b101, 0b1001, 0b10011, 0b100011, 0b1001001, 0b10010011]
    np.testing.assert_array_equal(m, np.array(want, np.uint64))
    assert OT.children(par, 0) == [1, 2, 3] and OT.children(par, 1) == [4, 5]
    assert OT.children(par, 7) == []


def _layer_inputs(parents, ctx, seed):
    T = sum(len(p) for p in parents)
    W = layer_weights(SMALL, "f32", seed)
    cap = (max(c + len(p) for c, p in zip(ctx, parents)) + 31) // 32 * 32
    kc, vc = kv_cache(SMALL, np.asarray(ctx), cap, seed)
    x = hidden_states(T, SMALL.d, seed)
    return W, kc, vc, x


def test_chain_tree_is_the_linear_pass():
    gamma, ctx = [3, 0, 5], [17, 4, 40]
    parents = [[-1] + list(range(g)) for g in gamma]
    W, kc, vc, x = _layer_inputs(parents, ctx, 3)
    lin = OV.decoder_layer(SMALL, W, x, gamma, ctx, kc, vc)
    tre = OT.tree_decoder_layer(SMALL, W, x, parents, ctx, kc, vc)
    np.testing.assert_array_equal(tre.y, lin.y)
    for i in range(len(gamma)):
        np.testing.assert_array_equal(tre.k_new[i], lin.k_new[i])
        np.testing.assert_array_equal(tre.v_new[i], lin.v_new[i])


def test_chain_tree_over_int8_caches_is_the_linear_pass():
    gamma, ctx = [3, 0, 5], [17, 4, 40]
    parents = [[-1] + list(range(g)) for g in gamma]
    W, _, _, x = _layer_inputs(parents, ctx, 4)
    cap = (max(c + g + 1 for c, g in zip(ctx, gamma)) + 31) // 32 * 32
    k8, ks, v8, vs = kv_cache_int8(SMALL, np.asarray(ctx), cap, 4)
    lin = OV.decoder_layer(SMALL, W, x, gamma, ctx, k8, v8, kscale=ks, vscale=vs)
    tre = OT.tree_decoder_layer(SMALL, W, x, parents, ctx, k8, v8, kscale=ks, vscale=vs)
    np.testing.assert_array_equal(tre.y, lin.y)
    for i in range(len(gamma)):
        np.testing.assert_array_equal(tre.k_new[i], lin.k_new[i])
        np.testing.assert_array_equal(tre.v_new[i], lin.v_new[i])
    # and the int8 caches change the result
    plain = OT.tree_decoder_layer(SMALL, W, x, parents, ctx, *_layer_inputs(parents, ctx, 4)[1:3])
    assert np.abs(plain.y - tre.y).max() > 0


def test_every_node_over_int8_caches_equals_the_linear_pass_over_its_root_path():
    par = [-1, 0, 0, 1, 1, 2, 4, 6, 0]
    ctx = [23]
    W, _, _, x = _layer_inputs([par], ctx, 6)
    k8, ks, v8, vs = kv_cache_int8(SMALL, np.asarray(ctx), 64, 6)
    tre = OT.tree_decoder_layer(SMALL, W, x, [par], ctx, k8, v8, kscale=ks, vscale=vs)
    for j in range(len(par)):
        path, v = [], j
        while v >= 0:
            path.append(v)
            v = par[v] if v > 0 else -1
        path = path[::-1]
        lin = OV.decoder_layer(SMALL, W, x[path], [len(path) - 1], ctx, k8, v8, kscale=ks, vscale=vs)
        np.testing.assert_allclose(tre.y[j], lin.y[-1], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(tre.k_new[0][:, j], lin.k_new[0][:, -1], rtol=0, atol=0)


def test_every_node_equals_the_linear_pass_over_its_root_path():
    par = [-1, 0, 0, 1, 1, 2, 4, 6, 0]
    ctx = [23]
    W, kc, vc, x = _layer_inputs([par], ctx, 5)
    tre = OT.tree_decoder_layer(SMALL, W, x, [par], ctx, kc, vc)
    dep = OT.depths(par)
    for j in range(len(par)):
        path, v = [], j
        while v >= 0:
            path.append(v)
            v = par[v] if v > 0 else -1
        path = path[::-1]
        lin = OV.decoder_layer(SMALL, W, x[path], [len(path) - 1], ctx, kc, vc)
        np.testing.assert_allclose(tre.y[j], lin.y[-1], rtol=1e-12, atol=1e-12)
        # its key went to row ctx + j at position ctx + depth
        np.testing.assert_allclose(tre.k_new[0][:, j], lin.k_new[0][:, -1], rtol=0, atol=0)
        assert dep[j] == len(path) - 1


def _rand_rows(rng, n, V, scale=2.0):
    z = rng.standard_normal((n, V)) * scale
    e = np.exp(z - z.max(1, keepdims=True))
    return (e / e.sum(1, keepdims=True)).astype(np.float32)


@pytest.mark.parametrize("greedy", [False, True])
def test_chain_accept_is_the_linear_rule(greedy):
    rng = np.random.default_rng(9)
    for trial in range(40):
        gamma = rng.integers(0, 6, size=rng.integers(1, 6))
        V = int(rng.integers(2, 12))
        T = int(np.sum(gamma + 1))
        p = _rand_rows(rng, T, V)
        qn = _rand_rows(rng, T, V, 1.0)          # node rows: draft dist. of the node's child
        tokens = rng.integers(0, V, size=T)
        if trial % 3 == 0:                        # some drafts equal to the target's argmax
            tokens = np.argmax(p, 1)[np.maximum(np.arange(T) - 1, 0)]
        u_node = (rng.integers(0, GRID, size=T) / GRID).astype(np.float32)
        u_samp = (rng.integers(0, GRID, size=len(gamma)) / GRID).astype(np.float32)
        ctx = rng.integers(0, 50, size=len(gamma))
        parents = [[-1] + list(range(g)) for g in gamma]
        # the linear pass's arrays: draft j of sequence i is node j; its draft row is
        # node j-1's q row, its uniform node j's
        qs = np.concatenate([[0], np.cumsum(gamma + 1)])
        drafts, qrows, ua = [], [], []
        for i, g in enumerate(gamma):
            for j in range(1, g + 1):
                drafts.append(tokens[qs[i] + j])
                qrows.append(qn[qs[i] + j - 1])
                ua.append(u_node[qs[i] + j])
        drafts = np.asarray(drafts, np.int32)
        qrows = np.asarray(qrows, np.float32).reshape(-1, V)
        ua = np.asarray(ua, np.float32)
        a1, y1, k1, _ = OA.accept_commit(gamma, drafts, p, qrows, ua, u_samp, ctx, greedy=greedy)
        a2, y2, k2, paths = OT.tree_accept(parents, tokens, p, qn, u_node, u_samp, ctx, greedy=greedy)
        np.testing.assert_array_equal(a1, a2)
        np.testing.assert_array_equal(y1, y2)
        np.testing.assert_array_equal(k1, k2)
        for i in range(len(gamma)):
            assert paths[i] == list(range(a2[i] + 1))


def _u_grid():
    return (np.arange(GRID, dtype=np.float64) / GRID).astype(np.float32)


def _first_token_distribution(p0, q0, m, V):
    """Exact law of the first emitted token when the root has m children drawn
    i.i.d. from q0 (every child a leaf): enumeration of the children's tokens
    and counting over the full uniform grid of every test and of the draw."""
    ug = _u_grid()
    Ug = np.arange(GRID, dtype=object)
    Q = OA.integer_weights(q0)
    SQ = int(Q.sum(dtype=np.uint64))
    dist = np.zeros(V)

    def draw_law(R):
        R = np.asarray(R, dtype=np.uint64)
        S = int(R.sum(dtype=np.uint64))
        if S == 0:
            out = np.zeros(V)
            out[int(np.argmax(p0))] = 1.0
            return out
        t = np.minimum(np.floor(ug.astype(np.float64) * np.float64(S)), S - 1)
        cs = np.cumsum(R.astype(np.float64))
        y = np.searchsorted(cs, t, side="right")
        return np.bincount(y, minlength=V)[:V] / GRID

    def walk(kids, prob, R, S, k):
        # kids: the children's tokens; k: index of the child under test
        if k == len(kids):
            law = draw_law(R if R is not None else OA.integer_weights(p0))
            return prob * law
        d = kids[k]
        out = np.zeros(V)
        if R is None:
            npass = int(np.count_nonzero(ug * np.float32(q0[d]) < np.float32(p0[d])))
        else:
            # U * Q(d) * S < R(d) * SQ * 2^24, counted exactly
            lhs_per_u = int(Q[d]) * S
            rhs = int(R[d]) * SQ * GRID
            npass = GRID if lhs_per_u == 0 and rhs > 0 else (
                0 if lhs_per_u == 0 else min(GRID, max(0, -(-rhs // lhs_per_u))))
        pa = npass / GRID
        out[d] += prob * pa
        if pa < 1.0:
            if R is None:
                res = np.maximum(np.float32(0), (p0 - q0).astype(np.float32))
                R2 = [int(t) for t in OA.integer_weights(res)]
                S2 = sum(R2)
            else:
                R2, S2 = OT._residual_after(R, S, Q, SQ)
            if S2 == 0:
                R2 = [int(t) for t in OA.integer_weights(p0)]
                S2 = sum(R2)
            out += walk(kids, prob * (1 - pa), R2, S2, k + 1)
        return out

    for kids in np.ndindex(*([V] * m)):
        w = float(np.prod([q0[d] for d in kids]))
        if w == 0:
            continue
        dist += walk(list(kids), w, None, 0, 0)
    return dist


@pytest.mark.parametrize("m,seed", [(2, 0), (3, 1), (2, 2)])
def test_multi_child_root_keeps_the_target_distribution(m, seed):
    rng = np.random.default_rng(seed)
    V = 3
    p0 = _rand_rows(rng, 1, V)[0]
    q0 = _rand_rows(rng, 1, V)[0]
    dist = _first_token_distribution(p0.astype(np.float64).astype(np.float32), q0, m, V)
    np.testing.assert_allclose(dist.sum(), 1.0, atol=1e-9)
    np.testing.assert_allclose(dist, p0, atol=2e-6)


def test_multi_child_tree_accept_matches_enumeration_frequencies():
    """The tree_accept implementation itself (not the enumeration's copy of
    the rule) over many uniform draws: first-token frequencies approach p0."""
    rng = np.random.default_rng(4)
    V, m, N = 4, 3, 40000
    p0 = _rand_rows(rng, 1, V)[0]
    q0 = _rand_rows(rng, 1, V)[0]
    par = [-1] + [0] * m
    p = np.repeat(p0[None], m + 1, 0)
    q = np.repeat(q0[None], m + 1, 0)
    counts = np.zeros(V)
    qd = q0.astype(np.float64)
    qd /= qd.sum()
    for _ in range(N):
        toks = np.concatenate([[0], rng.choice(V, size=m, p=qd)])
        u = (rng.integers(0, GRID, size=m + 1) / GRID).astype(np.float32)
        us = np.asarray([rng.integers(0, GRID) / GRID], np.float32)
        a, y, _, path = OT.tree_accept([par], toks, p, q, u, us, [0])
        first = toks[path[0][1]] if a[0] >= 1 else y[0]
        counts[first] += 1
    freq = counts / N
    assert np.all(np.abs(freq - p0) < 4 * np.sqrt(p0 * (1 - p0) / N) + 1e-4), (freq, p0)


def test_greedy_tree_follows_the_argmax_branch():
    V = 5
    par = [-1, 0, 0, 1, 2, 2]
    p = np.full((6, V), 0.1, np.float32)
    p[0, 3] = 0.6          # root: argmax 3 -> child 2 (token 3), not child 1 (token 1)
    p[2, 4] = 0.6          # node 2: argmax 4 -> child 5 (token 4)
    p[5, 0] = 0.6          # node 5: leaf, bonus argmax 0
    tokens = np.array([0, 1, 3, 2, 2, 4])
    a, y, k, paths = OT.tree_accept([par], tokens, p, p, np.zeros(6, np.float32),
                                    np.zeros(1, np.float32), [10], greedy=True)
    assert a[0] == 2 and y[0] == 0 and k[0] == 13 and paths[0] == [0, 2, 5]


def test_compact_rows_moves_the_path():
    cache = np.arange(1 * 12 * 2).reshape(1, 12, 2)
    out = OT.compact_rows(cache, 4, [0, 2, 5])
    np.testing.assert_array_equal(out[0, :4], cache[0, :4])
    np.testing.assert_array_equal(out[0, 4], cache[0, 4])
    np.testing.assert_array_equal(out[0, 5], cache[0, 6])
    np.testing.assert_array_equal(out[0, 6], cache[0, 9])
    np.testing.assert_array_equal(out[0, 7:], cache[0, 7:])
