"""Acceptance, resampling and KV-length commit.  Test infrastructure; see
package docstring.

The rule is rejection sampling in the sense of Leviathan, Kalman and Matias,
which [tax] cites by name (sections "Why do the headline speedups all come
from batch 1?" and "Sources") for keeping the output distribution identical to
plain decoding; [primer] section "The idea" gives its shape: keep the drafts up
to the first one the large model rejects, then add one token of the large
model's own (3 of 4 accepted -> 4 tokens, none accepted -> 1 token).  The pages
do not print the sampling steps; this is the plainest reading, fixed so that
two implementations agree bit for bit:

Stochastic mode, per sequence i (draft j = 1..gamma_i, 1-based):
  1. Draft j passes iff fl32(u_acc_j * q_j(d_j)) < p_j(d_j): one IEEE fp32
     multiply, strict compare (equivalent to u < p/q, accepting with
     probability min(1, p/q)).  a = number of leading passes.
  2. Resampling weights: r = max(0, fl32(p_{a+1} - q_{a+1})) if a < gamma_i
     (residual after a rejection); r = p_{gamma_i+1} if every draft passed
     (bonus token).
  3. Integer weights R(x) = trunc(fl32(r(x) * 2^32)) (the scale is exact),
     S = sum R as an exact integer.  If S = 0 after a rejection, use
     R = trunc(p_{a+1} * 2^32) instead; if still 0, y = argmax p_{a+1}
     (lowest index).
  4. t = floor(fl64(u_samp * S)) (clamped to S - 1); y = the least x whose
     running sum of R exceeds t.  Integer sums make the draw independent of
     summation order.
  5. accepted = a, next_token = y, kv_len = ctx_i + a + 1.

Greedy mode: a = number of leading drafts equal to argmax p_j (lowest index
on ties); y = argmax p_{a+1}.

A draft token outside [0, V) is a data error: that sequence is left
uncommitted (accepted = next_token = -1, kv_len unchanged) and the error is
reported.
"""
from __future__ import annotations

import numpy as np

__all__ = ["accept_commit", "passes", "resample_weights", "integer_weights",
           "position_counts", "conditional_rates",
           "draw_integer_cdf", "ERR_BAD_TOKEN"]

ERR_BAD_TOKEN = 1
_TWO32 = np.float32(2.0 ** 32)


def passes(u, q_d, p_d) -> bool:
    """Draft test: fl32(u * q(d)) < p(d), strict."""
    return bool(np.float32(u) * np.float32(q_d) < np.float32(p_d))


def resample_weights(p_row, q_row):
    """Integer weights for the token drawn after a rejection (q_row given) or
    as the bonus (q_row None), with the zero-mass fallback to p_row."""
    p_row = np.asarray(p_row, dtype=np.float32)
    if q_row is not None:
        R = integer_weights(p_row - np.asarray(q_row, dtype=np.float32))
        if int(R.sum(dtype=np.uint64)) > 0:
            return R
    return integer_weights(p_row)


def integer_weights(r) -> np.ndarray:
    """trunc(fl32(max(0, r) * 2^32)) as uint64 (r fp32)."""
    r = np.maximum(np.asarray(r, dtype=np.float32), np.float32(0.0))
    return np.floor(r * _TWO32).astype(np.uint64)


def draw_integer_cdf(R: np.ndarray, u: np.float32) -> int:
    """Least x with sum_{x' <= x} R(x') > floor(fl64(u * S)); requires S > 0."""
    S = int(R.sum(dtype=np.uint64))
    t = int(np.floor(np.float64(u) * np.float64(S)))
    t = min(t, S - 1)
    csum = np.cumsum(R, dtype=np.uint64)
    # side='right' gives the first index whose running sum exceeds t
    return int(np.searchsorted(csum, np.uint64(t), side="right"))


def accept_commit(gamma, draft, p, q, u_acc, u_samp, kv_len, *, greedy=False):
    """Returns (accepted[B], next_token[B], new_kv_len[B], err_flags[B]).

    p: fp32 [T, V] target rows; q: fp32 [sum gamma, V] draft rows; rows follow
    the token map (target row q_start[i] + j, draft row q_start[i] - i + j)."""
    gamma = np.asarray(gamma, dtype=np.int64)
    draft = np.asarray(draft, dtype=np.int64)
    p = np.asarray(p, dtype=np.float32)
    q = np.asarray(q, dtype=np.float32)
    u_acc = np.asarray(u_acc, dtype=np.float32)
    u_samp = np.asarray(u_samp, dtype=np.float32)
    kv_len = np.asarray(kv_len, dtype=np.int64)
    b = len(gamma)
    V = p.shape[1]
    acc = np.zeros(b, np.int64)
    nxt = np.zeros(b, np.int64)
    new_len = kv_len.copy()
    err = np.zeros(b, np.int64)
    qs = 0
    for i in range(b):
        g = int(gamma[i])
        ds = qs - i
        toks = draft[ds:ds + g]
        if np.any((toks < 0) | (toks >= V)):
            acc[i], nxt[i], err[i] = -1, -1, ERR_BAD_TOKEN
            qs += g + 1
            continue
        a = 0
        for j in range(g):
            dj = int(toks[j])
            if greedy:
                ok = dj == int(np.argmax(p[qs + j]))
            else:
                ok = passes(u_acc[ds + j], q[ds + j, dj], p[qs + j, dj])
            if not ok:
                break
            a = j + 1
        prow = p[qs + a]
        if greedy:
            y = int(np.argmax(prow))
        else:
            R = resample_weights(prow, q[ds + a] if a < g else None)
            if int(R.sum(dtype=np.uint64)) == 0:
                y = int(np.argmax(prow))
            else:
                y = draw_integer_cdf(R, u_samp[i])
        acc[i], nxt[i] = a, y
        new_len[i] = kv_len[i] + a + 1
        qs += g + 1
    return acc, nxt, new_len, err


def position_counts(gamma, accepted, n_pos: int) -> np.ndarray:
    """Per-position acceptance counters of one verify pass, for positions
    k = 1..n_pos (draft k of a sequence):

      reached[k-1]  = sequences that tested draft k: gamma_i >= k and the
                      drafts before it were all accepted (a_i >= k - 1);
      accepted[k-1] = sequences that accepted draft k (a_i >= k).

    accepted / reached is the conditional acceptance rate at position k
    (draft k accepted given drafts 1..k-1 were), the measure [tax] section
    "How do you measure this on your own server?" asks for.  Uncommitted
    sequences (a_i < 0) are not counted.  Returns int64 [2, n_pos]:
    row 0 reached, row 1 accepted."""
    out = np.zeros((2, n_pos), dtype=np.int64)
    for g, a in zip(np.asarray(gamma, np.int64), np.asarray(accepted, np.int64)):
        if a < 0:
            continue
        for k in range(1, n_pos + 1):
            if g >= k and a >= k - 1:
                out[0, k - 1] += 1
            if a >= k:
                out[1, k - 1] += 1
    return out


def conditional_rates(counts) -> list:
    """accepted / reached per position (0 where nothing reached it)."""
    counts = np.asarray(counts, np.int64)
    return [float(counts[1, k]) / float(counts[0, k]) if counts[0, k] else 0.0
            for k in range(counts.shape[1])]
