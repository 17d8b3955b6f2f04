"""The verification forward pass (fp64).  Test infrastructure; see package docstring.

What the pass computes follows [primer] section "The idea" (the large model
checks every drafted token in one pass, reading its weights once as for a
batch) and [slack] FAQ "What is the ragged tensor problem ..." and section
"The batch also goes ragged" (each sequence carries its own position ids,
mask and KV length; no padding to a common length).  The pages name no layer
internals; the plainest reading of "one target-model forward pass" is a
standard pre-norm decoder layer:

  h  = RMSNorm(x)                       (eps 1e-6, unit gain)
  q, k, v = h Wq^T, h Wk^T, h Wv^T      (weights stored [out, in])
  q, k <- RoPE at the token's position  (rotate-half pairs (i, i + hd/2),
                                          angle pos * theta^(-2i/hd))
  k, v appended to the sequence's cache at that position (cache storage is bf16)
  o  = softmax(q K^T / sqrt(hd)) V      (query j of sequence i sees keys
                                          0 .. ctx_i + j; q-head h reads
                                          kv-head floor(h / group))
  x1 = x + o Wo^T
  y  = x1 + (silu(RMSNorm(x1) Wg^T) * (RMSNorm(x1) Wu^T)) Wd^T
  head: logits = RMSNorm(y) Wlm^T, p = softmax(logits)
  embedding: x = E[token]

Quantized KV cache (optional): [static], section "The catch is prefill, and
it points back at admission", has the swarm quantize its KV to keep the
per-sequence read from sinking the ceiling as context grows ([tax], "What
does this model leave out?", names longer context as the term the model
misses).  The pages fix no format; the plainest reading is symmetric int8
per cached vector (one position of one KV head): scale = fl32(absmax / 127),
code = clamp(rne(fl32(x / scale)), -127, 127), value = code * scale, with
the appended keys and values rounded to bf16 first and stored the same way.

Token map: sequence i owns stacked rows q_start[i] .. q_start[i] + gamma_i,
q_start = exclusive prefix sum of (gamma_i + 1); row j of sequence i is the
token at position ctx_i + j (ctx_i = tokens already cached).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .formats import bf16_to_f64, matrix_f64, round_bf16

__all__ = ["token_map", "rms_norm", "rope", "attend", "LayerOut", "decoder_layer",
           "head_logits", "softmax", "embed", "quantize_int8_row", "dequantize_int8"]


def token_map(gamma, ctx):
    """(q_start[B+1], seq_of[T], j_of[T], pos_of[T]) for ragged draft chunks."""
    gamma = np.asarray(gamma, dtype=np.int64)
    ctx = np.asarray(ctx, dtype=np.int64)
    b = len(gamma)
    q_start = np.zeros(b + 1, dtype=np.int64)
    for i in range(b):
        q_start[i + 1] = q_start[i] + gamma[i] + 1
    t = int(q_start[-1])
    seq_of = np.zeros(t, dtype=np.int64)
    j_of = np.zeros(t, dtype=np.int64)
    pos_of = np.zeros(t, dtype=np.int64)
    for i in range(b):
        for j in range(int(gamma[i]) + 1):
            r = q_start[i] + j
            seq_of[r], j_of[r], pos_of[r] = i, j, ctx[i] + j
    return q_start, seq_of, j_of, pos_of


def rms_norm(x, eps: float = 1e-6):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope(x, pos: int, theta: float = 10000.0):
    """Rotate pairs (i, i + hd/2) of x[..., hd] by pos * theta^(-2i/hd)."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * theta ** (-2.0 * i / hd)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def softmax(z, axis=-1):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=axis, keepdims=True))
    return e / e.sum(axis=axis, keepdims=True)


def attend(q, keys, vals):
    """Softmax attention of one query over the visible keys [L, hd]."""
    s = keys @ q / np.sqrt(q.shape[-1])
    w = softmax(s)
    return w @ vals


def silu(z):
    return z / (1.0 + np.exp(-z))


@dataclasses.dataclass
class LayerOut:
    y: np.ndarray          # [T_sel, d] fp64, rows of the selected sequences in order
    rows: np.ndarray       # stacked-row index of each output row
    k_new: dict            # seq -> [n_kv, gamma+1, hd] bf16-valued fp64 (rotated keys)
    v_new: dict            # seq -> [n_kv, gamma+1, hd]


def quantize_int8_row(v):
    """Symmetric int8 code of one cached key or value vector (one position,
    one KV head): scale = fl32(absmax / 127), code = clamp(rne(fl32(x / scale)),
    -127, 127) with fp32 division; an all-zero vector has scale 0 and codes 0.
    v holds the vector's values (bf16-representable).  Returns (codes int8,
    scale fp32)."""
    x = np.asarray(v, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if amax == 0:
        return np.zeros(x.shape, np.int8), np.float32(0)
    scale = np.float32(amax / np.float32(127.0))
    codes = np.clip(np.rint(x / scale), -127, 127).astype(np.int8)
    return codes, scale


def dequantize_int8(codes, scale):
    """code * scale, exact in fp64."""
    return np.asarray(codes, np.float64) * np.float64(np.float32(scale))


def decoder_layer(shape, w, x, gamma, ctx, kcache, vcache, *, eps=1e-6, theta=10000.0,
                  seqs=None, store_bf16=True, kscale=None, vscale=None) -> LayerOut:
    """One decoder layer over the stacked verify tokens.

    shape: object with d, n_q, n_kv, hd, ffn.  w: dict of decoded fp64
    matrices wq, wk, wv, wo, w_gate, w_up, w_down in [out, in] layout (or
    workloads.Weights, decoded here).  x: [T, d] hidden states (fp64 or bf16
    bits).  kcache / vcache: bf16 bits [B, n_kv, cap, hd] (logical layout,
    position-major).  seqs: subset of sequences to evaluate (default all).
    store_bf16: round appended keys/values to the cache's bf16 storage (the
    default; False keeps them exact, for comparisons with formulations that
    have no bf16 cache).
    kscale / vscale (fp32 [B, n_kv, cap]) given: an int8 cache -- kcache and
    vcache hold int8 codes, a cached vector is code * scale, and every appended
    key or value is rounded to bf16 and then stored as its int8 code and
    scale (quantize_int8_row): attention reads the stored values."""
    W = {n: (m if isinstance(m, np.ndarray) else matrix_f64(m)) for n, m in w.items()}
    gamma = np.asarray(gamma, dtype=np.int64)
    ctx = np.asarray(ctx, dtype=np.int64)
    q_start, _, _, _ = token_map(gamma, ctx)
    x = np.asarray(x)
    x = bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
    seqs = list(range(len(gamma))) if seqs is None else list(seqs)
    rows = np.concatenate([np.arange(q_start[i], q_start[i + 1]) for i in seqs]).astype(np.int64)
    hd, hq, hk = shape.hd, shape.n_q, shape.n_kv
    grp = hq // hk
    int8 = kscale is not None
    if int8:
        def store(a):
            codes, sc = quantize_int8_row(round_bf16(a))
            return dequantize_int8(codes, sc)
    else:
        store = round_bf16 if store_bf16 else (lambda a: a)

    xs = x[rows]
    h = rms_norm(xs, eps)
    q = (h @ W["wq"].T).reshape(len(rows), hq, hd)
    k = (h @ W["wk"].T).reshape(len(rows), hk, hd)
    v = (h @ W["wv"].T).reshape(len(rows), hk, hd)

    o = np.zeros((len(rows), hq, hd))
    k_new, v_new = {}, {}
    r0 = 0
    for i in seqs:
        n = int(gamma[i]) + 1
        c = int(ctx[i])
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
            pos = c + j
            for g in range(hk):
                kk[g, pos] = store(rope(k[r0 + j, g], pos, theta))
                vv[g, pos] = store(v[r0 + j, g])
        k_new[i], v_new[i] = kk[:, c:].copy(), vv[:, c:].copy()
        for j in range(n):
            pos = c + j
            for hh in range(hq):
                g = hh // grp
                qr = rope(q[r0 + j, hh], pos, theta)
                o[r0 + j, hh] = attend(qr, kk[g, :pos + 1], vv[g, :pos + 1])
        r0 += n

    x1 = xs + o.reshape(len(rows), hq * hd) @ W["wo"].T
    h2 = rms_norm(x1, eps)
    a = silu(h2 @ W["w_gate"].T) * (h2 @ W["w_up"].T)
    y = x1 + a @ W["w_down"].T
    return LayerOut(y, rows, k_new, v_new)


def head_logits(w_lm, y, *, eps=1e-6, chunk_rows: int = 16384):
    """logits = RMSNorm(y) Wlm^T, streaming the head matrix in row chunks.

    w_lm: workloads.Weights or fp64 [V, d]; y: [T, d] fp64 (or bf16 bits)."""
    y = np.asarray(y)
    y = bf16_to_f64(y) if y.dtype == np.uint16 else y.astype(np.float64)
    h = rms_norm(y, eps)
    if isinstance(w_lm, np.ndarray):
        return h @ np.asarray(w_lm, dtype=np.float64).T
    out = np.empty((h.shape[0], w_lm.n))
    for r0 in range(0, w_lm.n, chunk_rows):
        r1 = min(w_lm.n, r0 + chunk_rows)
        out[:, r0:r1] = h @ matrix_f64(w_lm, slice(r0, r1)).T
    return out


def embed(table, tokens):
    """x[t] = E[token[t]] (table fp32 [V, d] or bf16 bits)."""
    table = np.asarray(table)
    rows = table[np.asarray(tokens, dtype=np.int64)]
    return bf16_to_f64(rows) if table.dtype == np.uint16 else rows.astype(np.float64)
