"""Planner and closed forms (fp64).  Test infrastructure; see package docstring.

Sources:
* [tax] section "What does one speculative iteration actually cost?": expected
  tokens per verify pass under independent acceptance, and the speedup ratio
  of an iteration (expected tokens x plain step time over verify + draft time).
* [tax] section "How does the roofline model work?": the step-time model
  (memory time of weights x fraction plus per-sequence KV, against compute time
  proportional to batch x tokens per sequence x fraction) and the closed-form
  crossover batch B* = t_w / ((gamma + 1) c - k).
* [tax] section "Why should you not trust an independent-acceptance model for
  long drafts?": acceptance that falls 7 points per position from 94 %,
  treated as conditional acceptances.
* [slack] sections "The budget is fixed, and the batch is inside it" and "What
  the budget says to build": the compute-slack budget (decode floor divided by
  per-token compute time) and splitting what the batch leaves over its agents.
"""
from __future__ import annotations

import dataclasses
import math

__all__ = [
    "expected_tokens_indep", "expected_tokens_cond", "decaying_alphas",
    "StepModel", "speedup", "crossover_batch", "budget_tokens_from_rates",
    "plan_budget", "plan_speedup", "best_gamma",
]


def expected_tokens_indep(alpha: float, gamma: int) -> float:
    """Tokens produced per verify pass when each of gamma drafts is accepted
    independently with probability alpha: (1 - alpha^(gamma+1)) / (1 - alpha).

    At alpha = 1 every draft is accepted and the pass yields gamma + 1."""
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def expected_tokens_cond(alphas, gamma: int) -> float:
    """Expected tokens with conditional acceptance alphas[k-1] at position k.

    Draft k is emitted only if drafts 1..k are all accepted, so
    E = 1 + sum_{k=1..gamma} prod_{j<=k} alphas[j-1] (the 1 is the token the
    target always adds)."""
    e, run = 1.0, 1.0
    for k in range(gamma):
        run *= alphas[k]
        e += run
    return e


def decaying_alphas(n: int, first: float = 0.94, step: float = 0.07) -> list:
    """Linear decay of conditional acceptance per position, clipped at 0."""
    return [max(0.0, first - step * k) for k in range(n)]


@dataclasses.dataclass(frozen=True)
class StepModel:
    """The roofline step model of [tax], "How does the roofline model work?".

    A pass over b sequences that each carry n tokens, through a model whose
    size is `size` times the target's, takes the larger of two times: reading
    its weights (size * t_w) plus every sequence's KV cache (b * k -- a
    drafter reads its own KV per sequence, so this term is not scaled by
    size), and its arithmetic (size * c per token, b * n tokens).

    t_w: weight-read time of the target, k: KV-read time per sequence,
    c: compute time per token (2 * params / peak flops)."""
    t_w: float
    k: float
    c: float

    def pass_time(self, b: float, n: float, size: float = 1.0) -> float:
        reads = size * self.t_w + b * self.k
        arithmetic = size * self.c * b * n
        return reads if reads >= arithmetic else arithmetic

    def iteration_time(self, b: float, gamma: int, draft_frac: float) -> float:
        """One speculative iteration: the target verifies gamma + 1 tokens per
        sequence, a drafter of draft_frac the target's size proposes gamma."""
        return self.pass_time(b, gamma + 1) + self.pass_time(b, gamma, draft_frac)

    def speedup(self, b: float, gamma: int, e_tokens: float, draft_frac: float = 0.04) -> float:
        """[tax], "What does one speculative iteration actually cost?": tokens
        per iteration times the plain decode step, over the iteration's time
        (throughput relative to plain decoding at the same batch).  gamma = 0
        is plain decoding itself, exactly 1."""
        if gamma == 0:
            return 1.0
        return e_tokens * self.pass_time(b, 1) / self.iteration_time(b, gamma, draft_frac)


def speedup(b: float, gamma: int, e_tokens: float, t_w: float, k: float, c: float,
            draft_frac: float = 0.04) -> float:
    """StepModel(t_w, k, c).speedup(...)."""
    return StepModel(t_w, k, c).speedup(b, gamma, e_tokens, draft_frac)


def crossover_batch(gamma: int, t_w: float, k: float, c: float) -> float:
    """B* = t_w / ((gamma + 1) c - k); infinite when the denominator is <= 0
    (the per-sequence KV time never falls behind the extra compute)."""
    den = (gamma + 1) * c - k
    return math.inf if den <= 0 else t_w / den


def budget_tokens_from_rates(decode_tok_s: float, compute_tok_s: float) -> int:
    """Compute-slack budget: decode step time divided by per-token compute time,
    floored to whole tokens (39.6 tok/s and 962 tok/s give 24)."""
    return int(math.floor((1.0 / decode_tok_s) / (1.0 / compute_tok_s)))


def plan_budget(b_live: int, budget: int, gamma_max: int, fill_remainder: bool = True) -> list:
    """Per-agent draft lengths that keep sum(gamma_i + 1) within the budget.

    Each live agent commits one token per step, so b_live of the budget is
    spent before drafting; the rest, budget - b_live, is split evenly (floor)
    and, if fill_remainder, the first (budget - b_live) mod b_live agents get
    one more.  A batch at or above the budget drafts nothing."""
    if b_live <= 0:
        return []
    if b_live >= budget:
        return [0] * b_live
    free = budget - b_live
    base, rem = divmod(free, b_live)
    out = []
    for i in range(b_live):
        g = base + (1 if (fill_remainder and i < rem) else 0)
        out.append(min(gamma_max, g))
    return out


def best_gamma(b: float, gamma_max: int, e_of_gamma, t_w: float, k: float, c: float,
               draft_frac: float = 0.04):
    """argmax over gamma in 0..gamma_max of speedup (ties -> smaller gamma).

    e_of_gamma(g) gives the expected tokens per pass for draft length g."""
    best_g, best_s = 0, 1.0
    for g in range(1, gamma_max + 1):
        s = speedup(b, g, e_of_gamma(g), t_w, k, c, draft_frac)
        if s > best_s:
            best_g, best_s = g, s
    return best_g, best_s


def plan_speedup(b_live: int, gamma_max: int, alphas, t_w: float, k: float, c: float,
                 draft_frac: float = 0.04):
    """One draft length for every live sequence, chosen to maximise the page's
    speedup model.  alphas of length 1 means independent acceptance at that
    rate; longer lists are conditional acceptances per position (the last
    value repeats beyond the list)."""
    if len(alphas) == 1:
        e_of = lambda g: expected_tokens_indep(alphas[0], g)  # noqa: E731
    else:
        ext = lambda g: [alphas[min(i, len(alphas) - 1)] for i in range(g)]  # noqa: E731
        e_of = lambda g: expected_tokens_cond(ext(g), g)  # noqa: E731
    g, s = best_gamma(b_live, gamma_max, e_of, t_w, k, c, draft_frac)
    return [g] * b_live, s, crossover_batch(g, t_w, k, c)
