"""The five verification workloads, plus the draft/target constructions they use.

Workload index (sizes as stated by the workloads themselves):

1. tiny two-layer decoder (d 256, 4 heads of 64, FFN 1024, vocab 1024), fp32
   N(0, 1/d) weights, B=1, gamma=4, 128 cached tokens; draft rows are
   softmax(N(0,1) logits / 0.7).
2. one 9B-class bf16 layer, B=8, gamma=2 each, 2048 cached bf16 tokens, a
   151936-entry LM head; acceptance rate 0.8.
3. one 27B-class bf16 layer, B=32, gamma=7 each (256 verify tokens), 2048
   cached tokens; draft logits = target logits + N(0, 0.5) noise.
4. ragged batch on the 9B-class layer: B=16, gamma_i = max(0, floor(24/B) - 1
   + delta_i) with delta_i uniform on {-1, 0, 1}, context uniform in
   [256, 4096]; acceptance rates 0.5 / 0.8 / 0.97.
5. the 9B-class layer with int4 group-32 weights (and LM head), B=128,
   gamma=3, 1024 cached tokens; full-vocabulary residual and bonus sampling.

Readings of the workload text (listed with reasons in the design notes):
* N(mu, s) names a variance s, so N(0, 0.5) noise has std sqrt(0.5).
* "acceptance rate a" is realised with a one-hot draft row q_j = e_{d_j} and a
  target row p_j that puts mass a on d_j and spreads 1 - a over the other
  tokens in proportion to a synthetic model row; then every draft test passes
  with probability exactly a.
* synthetic target logits are N(0, 1): RMS-normalised hidden states times
  N(0, 1/d) head weights have exactly that law.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .gen import (SHAPES, Shape, rng_for, sample_from_probs, stable_softmax_f32,
                  uniforms_2m24)

__all__ = ["Workload", "workload", "custom_workload", "accept_inputs",
           "SEED_BASE", "WORKLOAD_IDS"]

SEED_BASE = 20260
WORKLOAD_IDS = (1, 2, 3, 4, 5)


@dataclasses.dataclass
class Workload:
    cid: int
    name: str
    shape: Shape
    wtype: str           # 'f32' | 'bf16' | 'int4'
    n_layers: int
    gamma: np.ndarray    # int32 [B]
    ctx: np.ndarray      # int32 [B] cached tokens before the pass
    cap: int             # KV capacity per sequence (multiple of 32)
    head: bool           # an LM head is part of the pass
    embed: bool          # token embedding is part of the pass
    draft: str           # 'temp' | 'alpha' | 'noise'
    alphas: tuple = ()
    temp: float = 1.0
    noise_var: float = 0.0
    seed: int = SEED_BASE

    @property
    def B(self) -> int:
        return int(len(self.gamma))

    @property
    def T(self) -> int:
        return int(np.sum(self.gamma + 1))

    @property
    def n_draft(self) -> int:
        return int(np.sum(self.gamma))

    @property
    def q_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.gamma + 1)]).astype(np.int32)


def _cap_for(ctx, gamma) -> int:
    need = int(np.max(np.asarray(ctx) + np.asarray(gamma) + 1)) if len(ctx) else 32
    return max(32, (need + 31) // 32 * 32)


def workload(cid: int) -> Workload:
    seed = SEED_BASE + cid
    if cid == 1:
        g = np.array([4], np.int32)
        c = np.array([128], np.int32)
        return Workload(1, "tiny-2L-d256-B1-g4-ctx128", SHAPES["tiny"], "f32", 2, g, c,
                        _cap_for(c, g), True, True, "temp", temp=0.7, seed=seed)
    if cid == 2:
        g = np.full(8, 2, np.int32)
        c = np.full(8, 2048, np.int32)
        return Workload(2, "9B-layer-bf16-B8-g2-ctx2048", SHAPES["9b"], "bf16", 1, g, c,
                        _cap_for(c, g), True, False, "alpha", alphas=(0.8,), seed=seed)
    if cid == 3:
        g = np.full(32, 7, np.int32)
        c = np.full(32, 2048, np.int32)
        return Workload(3, "27B-layer-bf16-B32-g7-ctx2048", SHAPES["27b"], "bf16", 1, g, c,
                        _cap_for(c, g), True, False, "noise", noise_var=0.5, seed=seed)
    if cid == 4:
        rng = rng_for(seed, "geometry")
        b = 16
        delta = rng.integers(-1, 2, size=b)
        g = np.maximum(0, 24 // b - 1 + delta).astype(np.int32)
        c = rng.integers(256, 4097, size=b).astype(np.int32)
        return Workload(4, "9B-layer-bf16-ragged-B16-ctx256-4096", SHAPES["9b"], "bf16", 1,
                        g, c, _cap_for(c, g), False, False, "alpha",
                        alphas=(0.5, 0.8, 0.97), seed=seed)
    if cid == 5:
        g = np.full(128, 3, np.int32)
        c = np.full(128, 1024, np.int32)
        return Workload(5, "9B-layer-int4g32-B128-g3-ctx1024", SHAPES["9b"], "int4", 1, g, c,
                        _cap_for(c, g), True, False, "noise", noise_var=0.5, seed=seed)
    raise ValueError(f"unknown workload {cid}")


def custom_workload(shape: Shape, wtype: str, gamma, ctx, *, head=True, embed=False,
                    n_layers=1, draft="noise", alphas=(), temp=1.0, noise_var=0.5,
                    seed=12345, cap=None, name="custom") -> Workload:
    g = np.asarray(gamma, np.int32)
    c = np.asarray(ctx, np.int32)
    return Workload(0, name, shape, wtype, n_layers, g, c,
                    cap if cap is not None else _cap_for(c, g), head, embed, draft,
                    alphas=tuple(alphas), temp=temp, noise_var=noise_var, seed=seed)


def accept_inputs(wl: Workload, vocab: int | None = None, *, alpha: float | None = None,
                  target_logits: np.ndarray | None = None,
                  target_probs: np.ndarray | None = None, seed: int | None = None,
                  tag: str = "accept") -> dict:
    """Drafts, draft rows q, target rows p and uniforms for one pass.

    Row conventions: target row q_start[i] + j (j = 0..gamma_i) is the target
    distribution of the (j+1)-th new token of sequence i; draft row
    q_start[i] - i + j (j = 0..gamma_i - 1) is the draft distribution of draft
    token j+1.  One acceptance uniform per draft and one sampling uniform per
    sequence.

    With target_logits / target_probs given (e.g. from a model), those rows
    are used for p (or as the model rows of the acceptance-rate construction);
    otherwise N(0, 1) synthetic logits are drawn."""
    seed = wl.seed if seed is None else seed
    V = vocab if vocab is not None else wl.shape.vocab
    T, ND = wl.T, wl.n_draft
    qs = wl.q_start
    r = lambda name: rng_for(seed, f"{tag}/{name}")  # noqa: E731
    out = {}
    if target_probs is None:
        if target_logits is None:
            target_logits = r("target_logits").standard_normal((T, V), dtype=np.float32)
        base = stable_softmax_f32(target_logits)
    else:
        base = np.asarray(target_probs, np.float32)
    draft_rows = np.concatenate([np.arange(qs[i], qs[i] + wl.gamma[i]) for i in range(wl.B)]
                                ).astype(np.int64) if ND else np.zeros(0, np.int64)
    if wl.draft == "alpha":
        a = float(alpha if alpha is not None else wl.alphas[0])
        d = r("draft_tokens").integers(0, V, size=ND).astype(np.int32)
        q = np.zeros((ND, V), np.float32)
        q[np.arange(ND), d] = 1.0
        p = base.copy()
        for n in range(ND):
            row = base[draft_rows[n]].astype(np.float64)
            rest = 1.0 - row[d[n]]
            mixed = (1.0 - a) * row / rest
            mixed[d[n]] = a
            p[draft_rows[n]] = mixed.astype(np.float32)
    elif wl.draft == "noise":
        if target_logits is None:
            raise ValueError("noise drafts need target logits")
        eps = r("draft_noise").standard_normal((ND, V), dtype=np.float32) * np.float32(
            np.sqrt(wl.noise_var))
        q = stable_softmax_f32(np.asarray(target_logits, np.float32)[draft_rows] + eps)
        d = sample_from_probs(r("draft_draw"), q)
        p = base
    elif wl.draft == "temp":
        z = r("draft_logits").standard_normal((ND, V), dtype=np.float32)
        q = stable_softmax_f32(z / np.float32(wl.temp))
        d = sample_from_probs(r("draft_draw"), q)
        p = base
    else:
        raise ValueError(wl.draft)
    out["draft"] = d.astype(np.int32)
    out["q"] = np.ascontiguousarray(q, np.float32)
    out["p"] = np.ascontiguousarray(p, np.float32)
    out["u_acc"] = uniforms_2m24(r("u_acc"), ND)
    out["u_samp"] = uniforms_2m24(r("u_samp"), wl.B)
    return out
