"""Token-tree verification (fp64 layer, integer acceptance).  Test
infrastructure; see package docstring.

[slack], "What the budget says to build" (Table 1) plans, for a lone agent,
"a small tree, ~8 to 16 deep" of candidate tokens under one verify pass, and
the opening of the same page has the tree ride along under the weight stream.
The pages name the structure and nothing of its mechanics; the plainest
reading, kept as close to the linear pass as it can be:

Tree of one sequence: nodes 0..n-1 in topological order (parent[j] < j);
node 0 is the last committed token (the root), node j >= 1 a drafted token.
depth(0) = 0, depth(j) = depth(parent[j]) + 1.  The children of a node were
drafted independently from that node's draft distribution q_v.

Verify: node j sits at position ctx + depth(j) (its RoPE angle), its key and
value go to cache row ctx + j, and it attends to the cached keys 0..ctx-1
and to the new keys of its ancestors and itself (a parent-pointer mask).
A chain (parent[j] = j - 1) is exactly the linear verify pass.

Accept (stochastic), walking down from the root; at node v with target row
p_v, draft row q_v and children c_1..c_m in index order:
  1. the first child is tested as in the linear rule: fl32(u * q_v(d)) < p_v(d);
  2. after a rejection the target becomes the residual of the rejected
     candidate's draft distribution.  The first residual is the linear
     rule's: R(x) = trunc(fl32(max(0, fl32(p_v(x) - q_v(x))) * 2^32)) with
     S = sum R.  Child k >= 2 (token d) then passes iff
     U * Q(d) * S < R(d) * SQ * 2^24, with U = u * 2^24 (u on the 2^-24 grid),
     Q(x) = trunc(fl32(q_v(x) * 2^32)), SQ = sum Q -- i.e. u < r(d) / q(d)
     for the normalised r = R / S, q = Q / SQ -- and on rejection
     R(x) <- max(0, R(x) * SQ - Q(x) * S), shifted right until the sum fits
     32 bits (all exact integer arithmetic);
  3. the first child that passes becomes v and the walk goes on;
  4. when no child passes (or v is a leaf), the token is drawn from the
     current weights: R of the residual after rejections, or
     trunc(fl32(p_v * 2^32)) when v's children all passed nothing / v is a
     leaf reached by acceptance (the bonus token), with the integer
     inverse-CDF draw of the linear rule (t = floor(fl64(u_samp * S)), the
     least x whose running sum exceeds t); an empty residual falls back to
     p_v, an empty p_v to its argmax.
With one child per node every step is the linear rule's, so a chain accepts
exactly as the linear pass does.  With several children drawn i.i.d. from q_v
this is multi-candidate speculative sampling, which keeps the target's
distribution (up to the 2^-32 weight quantisation).
Greedy mode: from the root, follow the child (lowest index) whose token is
argmax p_v; stop when none is; emit argmax p_v of the last node.

Commit: accepted = depth of the last accepted node a; kv_len += a + 1; the
accepted nodes' cached rows move to ctx + depth (the path's nodes keep their
keys and values; rows of rejected branches are dropped).
"""
from __future__ import annotations

import numpy as np

from .accept import draw_integer_cdf, integer_weights, passes
from .formats import bf16_to_f64, matrix_f64, round_bf16
from .verify import LayerOut, attend, dequantize_int8, quantize_int8_row, rms_norm, rope, silu

__all__ = ["depths", "ancestor_masks", "children", "tree_decoder_layer", "tree_accept",
           "compact_rows"]

_GRID = 1 << 24


def depths(parent) -> np.ndarray:
    """Depth of every node (parent[0] = -1, parent[j] < j)."""
    parent = np.asarray(parent, np.int64)
    d = np.zeros(len(parent), np.int64)
    for j in range(1, len(parent)):
        assert 0 <= parent[j] < j, "nodes must be in topological order"
        d[j] = d[parent[j]] + 1
    return d


def ancestor_masks(parent) -> np.ndarray:
    """Bit m of mask[j] set iff node m is node j or one of its ancestors."""
    parent = np.asarray(parent, np.int64)
    n = len(parent)
    assert n <= 64
    out = np.zeros(n, np.uint64)
    for j in range(n):
        m, v = 0, j
        while v >= 0:
            m |= 1 << int(v)
            v = int(parent[v]) if v > 0 else -1
        out[j] = np.uint64(m)
    return out


def children(parent, v: int) -> list:
    return [j for j in range(1, len(parent)) if parent[j] == v]


def tree_decoder_layer(shape, w, x, parents, ctx, kcache, vcache, *, eps=1e-6,
                       theta=10000.0, kscale=None, vscale=None) -> LayerOut:
    """One decoder layer over the stacked tree nodes of every sequence
    (sequence i owns stacked rows q_start[i] .. q_start[i] + n_i - 1, node j of
    its tree at row q_start[i] + j).  Inputs as verify.decoder_layer; the
    appended keys and values are returned in node order (cache rows
    ctx_i + j), bf16-rounded as the cache stores them.  kscale / vscale
    given: int8 caches, read and appended as verify.decoder_layer does
    (a cached vector is code * scale; an appended one is rounded to bf16,
    then stored as its int8 code and scale)."""
    W = {n: (m if isinstance(m, np.ndarray) else matrix_f64(m)) for n, m in w.items()}
    x = np.asarray(x)
    x = bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
    hd, hq, hk = shape.hd, shape.n_q, shape.n_kv
    grp = hq // hk
    h = rms_norm(x, eps)
    T = x.shape[0]
    q = (h @ W["wq"].T).reshape(T, hq, hd)
    k = (h @ W["wk"].T).reshape(T, hk, hd)
    v = (h @ W["wv"].T).reshape(T, hk, hd)
    o = np.zeros((T, hq, hd))
    int8 = kscale is not None
    if int8:
        def store(a):
            codes, sc = quantize_int8_row(round_bf16(a))
            return dequantize_int8(codes, sc)
    else:
        store = round_bf16
    k_new, v_new = {}, {}
    r0 = 0
    for i, par in enumerate(parents):
        n = len(par)
        c = int(ctx[i])
        dep = depths(par)
        anc = ancestor_masks(par)
        kk = np.empty((hk, c + n, hd))
        vv = np.empty((hk, c + n, hd))
        if int8:
            kk[:, :c] = np.asarray(kcache[i, :, :c], np.float64) * \
                np.asarray(kscale[i, :, :c], np.float32).astype(np.float64)[..., None]
            vv[:, :c] = np.asarray(vcache[i, :, :c], np.float64) * \
                np.asarray(vscale[i, :, :c], np.float32).astype(np.float64)[..., None]
        else:
            kk[:, :c] = bf16_to_f64(kcache[i, :, :c])
            vv[:, :c] = bf16_to_f64(vcache[i, :, :c])
        for j in range(n):
            pos = c + int(dep[j])
            for g in range(hk):
                kk[g, c + j] = store(rope(k[r0 + j, g], pos, theta))
                vv[g, c + j] = store(v[r0 + j, g])
        k_new[i], v_new[i] = kk[:, c:].copy(), vv[:, c:].copy()
        for j in range(n):
            pos = c + int(dep[j])
            vis = list(range(c)) + [c + m for m in range(n) if (int(anc[j]) >> m) & 1]
            for hh in range(hq):
                g = hh // grp
                qr = rope(q[r0 + j, hh], pos, theta)
                o[r0 + j, hh] = attend(qr, kk[g, vis], vv[g, vis])
        r0 += n
    assert r0 == T
    x1 = x + o.reshape(T, hq * hd) @ W["wo"].T
    h2 = rms_norm(x1, eps)
    a = silu(h2 @ W["w_gate"].T) * (h2 @ W["w_up"].T)
    y = x1 + a @ W["w_down"].T
    return LayerOut(y, np.arange(T), k_new, v_new)


def _sibling_passes(U: int, Qd: int, S: int, Rd: int, SQ: int) -> bool:
    """u < r(d) / q(d) for r = R / S, q = Q / SQ, in exact integers."""
    return U * Qd * S < Rd * SQ * _GRID


def _residual_after(R, S: int, Q, SQ: int):
    """max(0, R * SQ - Q * S) rescaled by a power of two until its sum fits 32
    bits; returns (weights as Python ints, their sum)."""
    raw = [max(0, int(r) * SQ - int(q) * S) for r, q in zip(R, Q)]
    tot = sum(raw)
    sh = max(0, tot.bit_length() - 32)
    out = [r >> sh for r in raw]
    return out, sum(out)


def tree_accept(parents, tokens, p, q, u_acc, u_samp, kv_len, *, greedy=False):
    """Acceptance over the trees of a batch.

    parents: per sequence, its parent array (n_i nodes); tokens [T]: the token
    of every stacked node (the root's is ignored); p [T, V]: target row of each
    node; q [T, V]: draft distribution of each node's children; u_acc [T]: one
    uniform per node (its own test; the root's unused); u_samp [B].
    Returns (accepted, next_token, kv_len_new, paths) -- paths[i] the accepted
    nodes by depth (starting with the root)."""
    B = len(parents)
    acc = np.zeros(B, np.int64)
    nxt = np.zeros(B, np.int64)
    kv = np.asarray(kv_len, np.int64).copy()
    paths = []
    r0 = 0
    for i, par in enumerate(parents):
        n = len(par)
        v = 0
        path = [0]
        while True:
            prow = np.asarray(p[r0 + v], np.float32)
            kids = children(par, v)
            if greedy:
                y = int(np.argmax(prow))
                nxt_v = next((c for c in kids if int(tokens[r0 + c]) == y), None)
                if nxt_v is None:
                    nxt[i] = y
                    break
                v = nxt_v
                path.append(v)
                continue
            qrow = np.asarray(q[r0 + v], np.float32)
            R = None          # integer weights after the first rejection
            S = 0
            moved = False
            for kk, c in enumerate(kids):
                d = int(tokens[r0 + c])
                u = np.float32(u_acc[r0 + c])
                if R is None:
                    ok = passes(u, qrow[d], prow[d])
                else:
                    Q = integer_weights(qrow)
                    SQ = int(Q.sum(dtype=np.uint64))
                    U = int(np.float64(u) * _GRID)
                    ok = _sibling_passes(U, int(Q[d]), S, int(R[d]), SQ)
                if ok:
                    v = c
                    path.append(v)
                    moved = True
                    break
                # rejected: the residual becomes the target
                if R is None:
                    res = np.maximum(np.float32(0), (prow - qrow).astype(np.float32))
                    R = [int(t) for t in integer_weights(res)]
                    S = sum(R)
                else:
                    R, S = _residual_after(R, S, Q, SQ)
                if S == 0:
                    R = [int(t) for t in integer_weights(prow)]
                    S = sum(R)
            if moved:
                continue
            # draw: from the residual after rejections, else (leaf, or no
            # children) the bonus row p_v
            if R is None:
                R = [int(t) for t in integer_weights(prow)]
                S = sum(R)
            if S == 0:
                nxt[i] = int(np.argmax(prow))
            else:
                nxt[i] = draw_integer_cdf(np.asarray(R, dtype=np.uint64), np.float32(u_samp[i]))
            break
        acc[i] = len(path) - 1
        kv[i] += acc[i] + 1
        paths.append(path)
        r0 += n
    return acc, nxt, kv, paths


def compact_rows(cache_seq, ctx: int, path) -> np.ndarray:
    """The commit's row moves on one sequence's cache [n_kv, cap, hd]: the node
    at depth k of the accepted path moves from row ctx + node to ctx + k."""
    out = cache_seq.copy()
    for k, node in enumerate(path):
        out[:, ctx + k] = cache_seq[:, ctx + node]
    return out
