"""GPU parity of token-tree verification against the oracle: the decoder
layer over stacked trees (ancestor masks derived on the device from the
parent arrays, positions at ctx + depth, rows at ctx + node), more than 64
query rows per KV head, tree acceptance bit for bit (both modes, full and
small vocabularies), and the commit's cache-row moves; then one round end to
end (tree verify -> head -> tree accept -> commit) against the oracle."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, GpuDecoder, GpuHead, OF, OV, dev_bf16_to_f64, rel_rows, say, sv, tg
from oracle import tree as OT
from workloads import Shape, custom_workload, hidden_states, kv_cache, kv_cache_int8, layer_weights

pytestmark = pytest.mark.gpu
GRID = 1 << 24


def random_tree(rng, n, width=3):
    """Parent array of an n-node tree: each node hangs under one of the last
    `width` nodes (deep and bushy enough)."""
    par = [-1]
    for j in range(1, n):
        par.append(int(rng.integers(max(0, j - width), j)))
    return par


def spine_tree(depth, width=2):
    """A chain of `depth` drafts with width - 1 extra candidates beside it at
    each of the first depth - 1 levels (the chain goes on through the first)."""
    par, chain = [-1], 0
    for lvl in range(depth):
        first = len(par)
        par.append(chain)
        if lvl < depth - 1:
            par += [chain] * (width - 1)
        chain = first
    return par


def _tree_layer(shape, wtype, parents, ctx, seed, packed=False):
    gamma = [len(p) - 1 for p in parents]
    wl = custom_workload(shape, wtype, gamma, ctx, seed=seed)
    W = layer_weights(shape, wtype, wl.seed)
    mats = {k: tg.upload_matrix(v, packed=packed) for k, v in W.items()}
    L = tg.decoder_struct(shape, wtype, mats, packed=packed)
    kc, vc = kv_cache(shape, wl.ctx, wl.cap, wl.seed)
    batch = tg.DeviceBatch(gamma, ctx, wl.cap, kcache=kc, vcache=vc, tree_parents=parents)
    bs = batch.struct()
    n = sv.sv_verify_layer_workspace_bytes(L, bs)
    ws = tg.workspace(n)
    xh = hidden_states(wl.T, shape.d, wl.seed)
    x = tg.to_dev(xh)
    y = torch.empty_like(x)
    assert sv.sv_verify_layer(L, bs, x, y, 0, ws, n, tg.stream_handle()) == sv.SV_OK
    torch.cuda.synchronize()
    assert batch.err.item() == 0
    ref = OT.tree_decoder_layer(shape, W, xh, parents, ctx, kc, vc)
    return wl, batch, y, ref


CASES = [
    # (name, shape, wtype, tree sizes, ctx)
    ("gqa4-rows96-and-small", Shape(512, 8, 2, 128, 1024, 3000), "bf16", [24, 5, 1, 9], [700, 33, 0, 257]),
    ("gqa5-rows120", Shape(640, 10, 2, 128, 1280, 2000), "bf16", [24, 2], [300, 1100]),
    ("gqa4-keysplit-rows16", Shape(512, 8, 2, 128, 1024, 3000), "bf16", [4, 3, 2], [100, 513, 5]),
    ("hd64-gqa2-int4", Shape(512, 8, 4, 64, 1024, 3000), "int4", [17, 6], [64, 2000]),
    # fp32 weights (the small model's precision: hi + lo bf16 halves), no GQA
    ("tiny-f32", Shape(256, 4, 4, 64, 1024, 1024), "f32", [9, 5, 1], [128, 3, 40]),
]


@pytest.mark.parametrize("name,shape,wtype,sizes,ctx", CASES, ids=[c[0] for c in CASES])
def test_tree_verify_parity(name, shape, wtype, sizes, ctx):
    rng = np.random.default_rng(len(name))
    parents = [random_tree(rng, n) for n in sizes]
    wl, batch, y, ref = _tree_layer(shape, wtype, parents, ctx, seed=31, packed=(wtype == "int4"))
    err = rel_rows(dev_bf16_to_f64(y), ref.y)
    say(f"{name}: depths {[int(OT.depths(p).max()) for p in parents]}, y rel err {err:.2e}")
    assert err < TOL[wtype]
    hd = shape.hd
    for i, par in enumerate(parents):
        c, n = ctx[i], len(par)
        kg = OF.bf16_to_f64(batch.k_logical(i)[:, c:c + n])
        vg = OF.bf16_to_f64(batch.v_logical(i)[:, c:c + n])
        assert rel_rows(kg.reshape(-1, hd), ref.k_new[i].reshape(-1, hd)) < TOL[wtype]
        assert rel_rows(vg.reshape(-1, hd), ref.v_new[i].reshape(-1, hd)) < TOL[wtype]


INT8_CASES = [
    # (name, shape, tree sizes, ctx): up to 16 query rows per KV head (the
    # key-split kernel) and up to 96 (the query-tiled kernel)
    ("gqa4-rows16", Shape(512, 8, 2, 128, 1024, 3000), [4, 3, 1], [300, 17, 0]),
    ("gqa4-rows96", Shape(512, 8, 2, 128, 1024, 3000), [24, 9, 2], [700, 33, 257]),
]


@pytest.mark.parametrize("name,shape,sizes,ctx", INT8_CASES, ids=[c[0] for c in INT8_CASES])
def test_tree_verify_over_int8_caches(name, shape, sizes, ctx):
    """Tree verify (ancestor masks, positions ctx + depth) over int8 caches:
    layer outputs and the appended keys and values (code times scale)
    against the oracle's int8 form."""
    rng = np.random.default_rng(len(name))
    parents = [random_tree(rng, n) for n in sizes]
    gamma = [n - 1 for n in sizes]
    wl = custom_workload(shape, "bf16", gamma, ctx, seed=77)
    W = layer_weights(shape, "bf16", wl.seed)
    mats = {k: tg.upload_matrix(v, packed=True) for k, v in W.items()}
    L = tg.decoder_struct(shape, "bf16", mats, packed=True)
    k8, ks, v8, vs = kv_cache_int8(shape, wl.ctx, wl.cap, wl.seed)
    batch = tg.DeviceBatch(gamma, ctx, wl.cap, kcache=k8, vcache=v8, kscale=ks, vscale=vs,
                           tree_parents=parents)
    bs = batch.struct()
    n = sv.sv_verify_layer_workspace_bytes(L, bs)
    ws = tg.workspace(n)
    xh = hidden_states(wl.T, shape.d, wl.seed)
    y = torch.empty_like(tg.to_dev(xh))
    assert sv.sv_verify_layer(L, bs, tg.to_dev(xh), y, 0, ws, n, tg.stream_handle()) == sv.SV_OK
    torch.cuda.synchronize()
    assert batch.err.item() == 0
    ref = OT.tree_decoder_layer(shape, W, xh, parents, ctx, k8, v8, kscale=ks, vscale=vs)
    err = rel_rows(dev_bf16_to_f64(y), ref.y)
    say(f"tree verify {name} over int8 caches: y rel err {err:.2e}")
    assert err < TOL["bf16"]
    hd = shape.hd
    for i, c in enumerate(ctx):
        m = sizes[i]
        kd = batch.k_logical(i)[:, c:c + m].astype(np.float64) * \
            batch.ks[i].cpu().numpy()[:, c:c + m].astype(np.float64)[..., None]
        vd = batch.v_logical(i)[:, c:c + m].astype(np.float64) * \
            batch.vs[i].cpu().numpy()[:, c:c + m].astype(np.float64)[..., None]
        assert rel_rows(kd.reshape(-1, hd), ref.k_new[i].reshape(-1, hd)) < TOL["bf16"]
        assert rel_rows(vd.reshape(-1, hd), ref.v_new[i].reshape(-1, hd)) < TOL["bf16"]


def test_tree_verify_at_the_size_limits():
    """A 64-node tree and a 64-node chain (the ancestor masks' limit) at a
    GQA group of 2: 128 query rows per KV head, the attention kernels'
    limit; one tree starts from an empty cache."""
    shape = Shape(256, 4, 2, 64, 512, 1000)
    rng = np.random.default_rng(111)
    parents = [random_tree(rng, 64), [-1] + list(range(63))]
    ctx = [100, 0]
    wl, batch, y, ref = _tree_layer(shape, "bf16", parents, ctx, seed=112, packed=True)
    err = rel_rows(dev_bf16_to_f64(y), ref.y)
    say(f"tree verify at 64 nodes, 128 rows per KV head: y rel err {err:.2e}")
    assert err < TOL["bf16"]


@pytest.mark.parametrize("greedy", [False, True])
def test_tree_accept_full_depth_chain(greedy):
    """A 64-node chain whose every draft passes (drafts from q = p, or the
    argmax in greedy mode): accepted depth 63, every path slot filled, the
    bonus token drawn at the last node; bit for bit against the oracle."""
    rng = np.random.default_rng(113 + greedy)
    V = 5003
    par = [-1] + list(range(63))
    p = _rows(rng, 64, V)
    tokens = np.zeros(64, np.int64)
    for j in range(1, 64):
        row = p[j - 1].astype(np.float64)
        tokens[j] = int(np.argmax(row)) if greedy else int(rng.choice(V, p=row / row.sum()))
    ua = (rng.integers(0, GRID, size=64) / GRID).astype(np.float32)
    us = np.array([0.61], np.float32)
    got = _run_tree_accept([par], tokens, p, p.copy(), ua, us, [9], greedy)
    want = OT.tree_accept([par], tokens, p, p.copy(), ua, us, [9], greedy=greedy)
    assert int(want[0][0]) == 63 and len(want[3][0]) == 64
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])
    np.testing.assert_array_equal(got[2], want[2])
    np.testing.assert_array_equal(got[3][0], want[3][0])
    assert got[4] == 0


def test_chain_beyond_64_rows_per_kv_head():
    """Linear drafts with 96 query rows per KV head (the eight-wave kernel)."""
    shape = Shape(512, 8, 2, 128, 1024, 3000)
    wl = custom_workload(shape, "bf16", [23, 3, 0], [400, 17, 1000], seed=8)
    dec = GpuDecoder(wl)
    xh = hidden_states(wl.T, shape.d, wl.seed)
    y = dec.run(tg.to_dev(xh))
    torch.cuda.synchronize()
    ref = dec.oracle(xh)
    err = rel_rows(dev_bf16_to_f64(y), ref.y)
    say(f"chain 96 rows: y rel err {err:.2e}")
    assert err < TOL["bf16"] and dec.batch.err.item() == 0


def test_bad_parent_is_flagged():
    shape = Shape(512, 8, 2, 128, 1024, 3000)
    parents = [[-1, 0, 5, 1]]           # node 2 names a later node
    wl = custom_workload(shape, "bf16", [3], [50], seed=9)
    W = layer_weights(shape, "bf16", wl.seed)
    mats = {k: tg.upload_matrix(v) for k, v in W.items()}
    L = tg.decoder_struct(shape, "bf16", mats)
    kc, vc = kv_cache(shape, wl.ctx, wl.cap, wl.seed)
    batch = tg.DeviceBatch([3], [50], wl.cap, kcache=kc, vcache=vc, tree_parents=parents)
    bs = batch.struct()
    n = sv.sv_verify_layer_workspace_bytes(L, bs)
    ws = tg.workspace(n)
    x = tg.to_dev(hidden_states(wl.T, shape.d, wl.seed))
    assert sv.sv_verify_layer(L, bs, x, torch.empty_like(x), 0, ws, n, tg.stream_handle()) == 0
    torch.cuda.synchronize()
    assert batch.err.item() & sv.SV_DEV_ERR_BAD_TREE


def _rows(rng, n, V, scale=3.0):
    z = rng.standard_normal((n, V)).astype(np.float32) * scale
    z -= z.max(1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(1, keepdims=True)).astype(np.float32)


def _run_tree_accept(parents, tokens, p, q, ua, us, ctx, greedy, from_logits=False):
    """p: host probabilities [T][V], or (from_logits) the head's device output
    of logits and row statistics."""
    B, V = len(parents), q.shape[1]
    gam = [len(x) - 1 for x in parents]
    dev = lambda a, dt: torch.as_tensor(np.ascontiguousarray(a), dtype=dt, device="cuda")  # noqa: E731
    par = dev(np.concatenate([np.asarray(x) for x in parents]), torch.int32)
    tok = dev(tokens, torch.int32)
    kv = dev(np.asarray(ctx), torch.int32)
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    path = torch.full((B, 64), -7, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    n = sv.sv_accept_tree_workspace_bytes(B, V, gam)
    ws = tg.workspace(n)
    mode = sv.SV_ACCEPT_GREEDY if greedy else sv.SV_ACCEPT_STOCHASTIC
    if from_logits:
        mode |= sv.SV_ACCEPT_FROM_LOGITS
    pd = p if from_logits else dev(p, torch.float32)
    st = sv.sv_accept_tree(B, V, mode, gam, par, tok, pd, dev(q, torch.float32),
                           dev(ua, torch.float32), dev(us, torch.float32), kv, acc, nxt, path, err, ws,
                           n, tg.stream_handle())
    assert st == sv.SV_OK
    torch.cuda.synchronize()
    return (acc.cpu().numpy(), nxt.cpu().numpy(), kv.cpu().numpy(), path.cpu().numpy(),
            int(err.item()))


def _tree_accept_case(rng, sizes, V, greedy, draft_from_q=True, q_equals_p=False, mix=0.0, parents=None):
    if parents is None:
        parents = [random_tree(rng, n) for n in sizes]
    sizes = [len(par) for par in parents]
    T = sum(sizes)
    p = _rows(rng, T, V)
    q = p.copy() if q_equals_p else _rows(rng, T, V, 2.0)
    if mix > 0:  # drafts close to the target: deep acceptance, several siblings tested
        q = (mix * p + (1 - mix) * q).astype(np.float32)
        q /= q.sum(1, keepdims=True)
    tokens = np.zeros(T, np.int64)
    r0 = 0
    for par in parents:
        for j in range(1, len(par)):
            row = q[r0 + par[j]].astype(np.float64)
            if greedy and rng.random() < 0.6:
                tokens[r0 + j] = int(np.argmax(p[r0 + par[j]]))
            elif draft_from_q:
                tokens[r0 + j] = int(rng.choice(V, p=row / row.sum()))
            else:
                tokens[r0 + j] = int(rng.integers(0, V))
        r0 += len(par)
    ua = (rng.integers(0, GRID, size=T) / GRID).astype(np.float32)
    us = (rng.integers(0, GRID, size=len(sizes)) / GRID).astype(np.float32)
    ctx = rng.integers(0, 3000, size=len(sizes))
    got = _run_tree_accept(parents, tokens, p, q, ua, us, ctx, greedy)
    want = OT.tree_accept(parents, tokens, p, q, ua, us, ctx, greedy=greedy)
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])
    np.testing.assert_array_equal(got[2], want[2])
    for i, path in enumerate(want[3]):
        np.testing.assert_array_equal(got[3][i, :len(path)], path)
        assert (got[3][i, len(path):] == -1).all()
    assert got[4] == 0
    return got


@pytest.mark.parametrize("greedy", [False, True])
def test_tree_accept_bit_exact_small_vocab(greedy):
    rng = np.random.default_rng(40 + greedy)
    depth_seen = []
    for trial in range(6):
        sizes = [int(v) for v in rng.integers(1, 25, size=int(rng.integers(1, 6)))]
        got = _tree_accept_case(rng, sizes, int(rng.integers(3, 400)), greedy, q_equals_p=(trial == 5))
        depth_seen += got[0].tolist()
    say(f"tree accept small vocab greedy={greedy}: accepted depths {depth_seen}")
    assert max(depth_seen) >= 2


def test_tree_accept_bit_exact_close_drafts():
    rng = np.random.default_rng(45)
    depths = []
    for trial in range(8):
        sizes = [int(v) for v in rng.integers(8, 25, size=int(rng.integers(1, 4)))]
        got = _tree_accept_case(rng, sizes, int(rng.integers(3, 60)), False, mix=0.85)
        depths += got[0].tolist()
    say(f"tree accept, drafts close to the target: accepted depths {depths}")
    assert max(depths) >= 3


@pytest.mark.parametrize("greedy", [False, True])
def test_tree_accept_bit_exact_full_vocab(greedy):
    rng = np.random.default_rng(50 + greedy)
    got = _tree_accept_case(rng, [16, 9], 151936, greedy)
    say(f"tree accept V=151936 greedy={greedy}: accepted {got[0].tolist()} next {got[1].tolist()}")


@pytest.mark.parametrize("V", [20003, 151936])
def test_tree_accept_bit_exact_spines(V):
    """Spines of two and of four candidates per level over several vocabulary
    chunks (V = 20003: the scalar path, V = 151936: 16-byte loads).  Walks end
    on the bonus row (a leaf), on the first residual (one child rejected), on
    the second (both of two rejected) and at a node of four whose first two
    are rejected, finished by one workgroup alone; all bit for bit."""
    rng = np.random.default_rng(61 + V % 2)
    assert spine_tree(8) == [-1, 0, 0, 1, 1, 3, 3, 5, 5, 7, 7, 9, 9, 11, 11, 13]
    ends = {}
    for mix in (0.0, 0.5, 0.9):
        parents = [spine_tree(8), spine_tree(4, 4), spine_tree(3), [-1, 0], [-1]]
        got = _tree_accept_case(rng, None, V, False, mix=mix, parents=parents)
        for i, par in enumerate(parents):
            last = int(got[3][i, got[0][i]])
            kids = min(3, sum(1 for x in par[1:] if x == last))
            ends[kids] = ends.get(kids, 0) + 1
    say(f"tree accept spines V={V}: walks ending at nodes of 0/1/2/3+ children: {ends}")
    assert ends.get(0, 0) > 0 and ends.get(2, 0) > 0


def test_tree_accept_bit_exact_sixteen_trees():
    """Sixteen trees at V = 151936 (304 chunk workgroups per grid, more than
    one round of CUs): spines, a bushy spine and a small binary tree, in both
    modes, bit for bit against the oracle."""
    V, B = 151936, 16
    rng = np.random.default_rng(106)
    shapes = [spine_tree(8), spine_tree(4, 4), spine_tree(3), [-1, 0, 0, 1, 1, 2, 2]]
    parents = [shapes[k % len(shapes)] for k in range(B)]
    for greedy in (False, True):
        got = _tree_accept_case(rng, None, V, greedy, mix=0.5, parents=parents)
        say(f"tree accept B={B} V={V} greedy={greedy}: accepted {got[0].tolist()}")


@pytest.mark.parametrize("greedy", [False, True])
def test_tree_accept_bit_exact_256_trees(greedy):
    """The largest batch (256 trees of 1 to 8 nodes, small vocabulary): every
    sequence's row range comes from the launch's start table at its full
    size, bit for bit against the oracle."""
    rng = np.random.default_rng(120 + greedy)
    sizes = [int(v) for v in rng.integers(1, 9, size=256)]
    got = _tree_accept_case(rng, sizes, 301, greedy, mix=0.6)
    say(f"tree accept B=256 greedy={greedy}: mean accepted depth {got[0].mean():.2f}")


@pytest.mark.parametrize("V", [20003, 151936])
def test_tree_accept_bit_exact_many_rejections(V):
    """Candidates drawn uniformly over the vocabulary, so most tests reject:
    nodes of four to seven children run the residual through further updates
    (the workgroup-alone path: 128-bit products and shifts) before a later
    candidate passes or the draw; bit for bit against the oracle."""
    rng = np.random.default_rng(80 + V % 2)
    parents = [spine_tree(3, 6), spine_tree(2, 4), [-1, 0, 0, 0, 0, 0, 0, 0], spine_tree(4)]
    past_second = 0  # nodes settled by a third or later candidate, or after rejecting three or more
    for _ in range(2):
        got = _tree_accept_case(rng, None, V, False, draft_from_q=False, parents=parents)
        for i, par in enumerate(parents):
            path = got[3][i, :got[0][i] + 1].tolist()
            for k, v in enumerate(path):
                kids = OT.children(par, v)
                if k + 1 < len(path):
                    past_second += kids.index(path[k + 1]) >= 2
                else:
                    past_second += len(kids) >= 3
    say(f"tree accept, uniform drafts V={V}: {past_second} nodes settled past their second candidate")
    assert past_second >= 3


@pytest.mark.parametrize("vocab", [20011, 151936])
@pytest.mark.parametrize("greedy", [False, True])
def test_tree_accept_from_logits(vocab, greedy):
    """Acceptance from the head's logits and row statistics
    (SV_ACCEPT_FROM_LOGITS, no probability rows materialised) decides exactly
    as from the head's probabilities, which match the oracle; spines, a
    random tree and a lone root, over several vocabulary chunks (20011: the
    scalar path, 151936: 16-byte loads)."""
    shape = Shape(512, 8, 2, 128, 1024, vocab)
    rng = np.random.default_rng(70 + greedy)
    parents = [spine_tree(8), random_tree(rng, 20), spine_tree(4, 4), [-1]]
    sizes = [len(par) for par in parents]
    wl = custom_workload(shape, "bf16", [n - 1 for n in sizes], [5] * len(sizes), seed=71)
    head = GpuHead(wl, packed=True)
    y = tg.to_dev(hidden_states(wl.T, shape.d, 72))
    pr = head.run(y)
    lgs = head.run(y, flags=sv.SV_HEAD_LOGITS_STATS)
    torch.cuda.synchronize()
    p = pr.cpu().numpy()
    q = (0.6 * p + 0.4 * _rows(rng, wl.T, vocab, 2.0)).astype(np.float32)
    q /= q.sum(1, keepdims=True)
    tokens = np.zeros(wl.T, np.int64)
    r0 = 0
    for par in parents:
        for j in range(1, len(par)):
            row = q[r0 + par[j]].astype(np.float64)
            tokens[r0 + j] = int(rng.choice(vocab, p=row / row.sum()))
        r0 += len(par)
    ua = (rng.integers(0, GRID, size=wl.T) / GRID).astype(np.float32)
    us = (rng.integers(0, GRID, size=len(sizes)) / GRID).astype(np.float32)
    ctx = [5] * len(sizes)
    got_p = _run_tree_accept(parents, tokens, p, q, ua, us, ctx, greedy)
    got_l = _run_tree_accept(parents, tokens, lgs, q, ua, us, ctx, greedy, from_logits=True)
    want = OT.tree_accept(parents, tokens, p, q, ua, us, ctx, greedy=greedy)
    for k in range(4):
        np.testing.assert_array_equal(got_l[k], got_p[k])
    np.testing.assert_array_equal(got_p[0], want[0])
    np.testing.assert_array_equal(got_p[1], want[1])
    assert got_l[4] == 0
    say(f"tree accept from logits V={vocab} greedy={greedy}: accepted {got_l[0].tolist()} next {got_l[1].tolist()}")


def test_tree_commit_moves_accepted_rows():
    shape = Shape(512, 8, 2, 128, 1024, 3000)
    B, cap = 3, 96
    ctx = np.array([10, 40, 3])
    acc = np.array([3, 0, 2])
    paths = [[0, 2, 5, 9], [0], [0, 1, 4]]
    kc, vc = kv_cache(shape, ctx + 20, cap, 77)
    batch = tg.DeviceBatch([0] * B, list(ctx), cap, kcache=kc, vcache=vc)
    kv_after = torch.tensor(ctx + acc + 1, dtype=torch.int32, device="cuda")
    a_dev = torch.tensor(acc, dtype=torch.int32, device="cuda")
    pm = np.full((B, 64), -1, np.int32)
    for i, pth in enumerate(paths):
        pm[i, :len(pth)] = pth
    assert sv.sv_tree_commit_kv(B, shape.n_kv, shape.hd, cap, kv_after, a_dev,
                                torch.tensor(pm, device="cuda"), batch.kptr, batch.vptr,
                                tg.stream_handle()) == sv.SV_OK
    torch.cuda.synchronize()
    for i in range(B):
        np.testing.assert_array_equal(batch.k_logical(i), OT.compact_rows(kc[i], int(ctx[i]), paths[i]))
        np.testing.assert_array_equal(batch.v_logical(i), OT.compact_rows(vc[i], int(ctx[i]), paths[i]))


def test_tree_commit_moves_int8_rows_and_scales():
    """The commit's moves on int8 caches: each accepted node's key and value
    codes and their scales move to ctx + depth (hd 64 and 128)."""
    for shape in (Shape(512, 8, 2, 128, 1024, 3000), Shape(256, 4, 2, 64, 512, 1000)):
        B, cap = 3, 96
        ctx = np.array([10, 40, 3])
        acc = np.array([3, 0, 2])
        paths = [[0, 2, 5, 9], [0], [0, 1, 4]]
        k8, ks, v8, vs = kv_cache_int8(shape, ctx + 20, cap, 78)
        batch = tg.DeviceBatch([0] * B, list(ctx), cap, kcache=k8, vcache=v8, kscale=ks, vscale=vs)
        kv_after = torch.tensor(ctx + acc + 1, dtype=torch.int32, device="cuda")
        pm = np.full((B, 64), -1, np.int32)
        for i, pth in enumerate(paths):
            pm[i, :len(pth)] = pth
        assert sv.sv_tree_commit_kv_int8(B, shape.n_kv, shape.hd, cap, kv_after,
                                         torch.tensor(acc, dtype=torch.int32, device="cuda"),
                                         torch.tensor(pm, device="cuda"), batch.kptr, batch.vptr, batch.ksptr,
                                         batch.vsptr, tg.stream_handle()) == sv.SV_OK
        torch.cuda.synchronize()
        for i in range(B):
            c = int(ctx[i])
            np.testing.assert_array_equal(batch.k_logical(i), OT.compact_rows(k8[i], c, paths[i]))
            np.testing.assert_array_equal(batch.v_logical(i), OT.compact_rows(v8[i], c, paths[i]))
            np.testing.assert_array_equal(batch.ks[i].cpu().numpy(), OT.compact_rows(ks[i][..., None], c, paths[i])[..., 0])
            np.testing.assert_array_equal(batch.vs[i].cpu().numpy(), OT.compact_rows(vs[i][..., None], c, paths[i])[..., 0])


def test_tree_round_end_to_end():
    """Tree verify of a lone sequence (a 20-node tree, 80 query rows per KV
    head), the LM head over its nodes, tree acceptance on the GPU's
    probabilities against the oracle, and the commit's row moves."""
    shape = Shape(512, 8, 2, 128, 1024, 3000)
    rng = np.random.default_rng(61)
    parents = [random_tree(rng, 20, width=2)]
    ctx = [333]
    wl, batch, y, ref = _tree_layer(shape, "bf16", parents, ctx, seed=62, packed=True)
    assert rel_rows(dev_bf16_to_f64(y), ref.y) < TOL["bf16"]
    head = GpuHead(wl, packed=True)
    pr = head.run(y)
    torch.cuda.synchronize()
    lg = OV.head_logits(head.Wlm, dev_bf16_to_f64(y))
    p = pr.cpu().numpy()
    np.testing.assert_allclose(p, OV.softmax(head.run(y, logits=True).cpu().numpy()), rtol=2e-5, atol=1e-9)
    assert rel_rows(head.run(y, logits=True).cpu().numpy(), lg) < TOL["bf16"]
    V = shape.vocab
    # drafts: each node's children from a draft distribution close to the target
    q = _rows(rng, len(parents[0]), V, 1.0)
    q = (0.7 * p + 0.3 * q).astype(np.float32)
    q /= q.sum(1, keepdims=True)
    tokens = np.zeros(len(parents[0]), np.int64)
    for j in range(1, len(parents[0])):
        row = q[parents[0][j]].astype(np.float64)
        tokens[j] = int(rng.choice(V, p=row / row.sum()))
    ua = (rng.integers(0, GRID, size=len(tokens)) / GRID).astype(np.float32)
    us = np.array([0.37], np.float32)
    got = _run_tree_accept(parents, tokens, p, q, ua, us, ctx, False)
    want = OT.tree_accept(parents, tokens, p, q, ua, us, ctx)
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])
    a = int(got[0][0])
    say(f"tree round: accepted depth {a}, path {want[3][0]}, next {int(got[1][0])}")
    # commit: the accepted path's rows move to ctx + depth
    k_before = batch.k_logical(0).copy()
    v_before = batch.v_logical(0).copy()
    kv_after = torch.tensor(got[2], dtype=torch.int32, device="cuda")
    assert sv.sv_tree_commit_kv(1, shape.n_kv, shape.hd, wl.cap, kv_after,
                                torch.tensor(got[0], dtype=torch.int32, device="cuda"),
                                torch.tensor(got[3], dtype=torch.int32, device="cuda"), batch.kptr,
                                batch.vptr, tg.stream_handle()) == sv.SV_OK
    torch.cuda.synchronize()
    np.testing.assert_array_equal(batch.k_logical(0), OT.compact_rows(k_before, ctx[0], want[3][0]))
    np.testing.assert_array_equal(batch.v_logical(0), OT.compact_rows(v_before, ctx[0], want[3][0]))
