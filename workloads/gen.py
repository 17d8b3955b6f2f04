"""Random draws and storage encodings.

Every array is produced from a named, seeded PCG64 stream so that the GPU path
and the oracle see bit-identical inputs.  Encodings:

* bf16: round-to-nearest-even of the fp32 value, kept as uint16 bit patterns.
* int4 groups of 32 along the reduction axis (symmetric, codes -7..7, code -8
  never produced): scale = bf16(absmax / 7), code = clamp(rne(w / scale), -7, 7).
  Codes are stored offset by +8 as nibbles, 8 per uint32, nibble i of word m
  holding reduction index 8*m + i; scales are bf16 bit patterns [N, K/32].
* uniforms on the 2^-24 grid in [0, 1): (k >> 8) * 2^-24 for a uint32 k.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
import zlib

import numpy as np

__all__ = [
    "Shape", "SHAPES", "rng_for", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "normal_f32", "normal_bf16", "quantize_int4_g32", "uniforms_2m24",
    "stable_softmax_f32", "sample_from_probs", "Weights", "layer_weights",
    "head_weights", "embed_weights", "kv_cache", "kv_cache_int8", "hidden_states",
]

_CHUNK = 1 << 24
_GEN_CHUNK = 1 << 22  # elements per independent child stream of a large draw
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        n = min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 8)
        _POOL = _cf.ThreadPoolExecutor(max_workers=max(1, n))
    return _POOL


def _parallel_chunks(rng: np.random.Generator, total: int, step: int, fn):
    """fn(child_rng, start, count) for consecutive chunks of `step` elements,
    each with its own child stream spawned from rng (deterministic for a given
    rng state and size), run on a thread pool."""
    n = (total + step - 1) // step
    kids = rng.spawn(n) if n else []
    futs = [_pool().submit(fn, kids[c], c * step, min(step, total - c * step)) for c in range(n)]
    for f in futs:
        f.result()


@dataclasses.dataclass(frozen=True)
class Shape:
    """Decoder layer geometry: model width, query/key-value heads, head size,
    FFN width and vocabulary size."""
    d: int
    n_q: int
    n_kv: int
    hd: int
    ffn: int
    vocab: int

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv

    @property
    def layer_params(self) -> int:
        d, hq, hk, hd, f = self.d, self.n_q, self.n_kv, self.hd, self.ffn
        return d * (hq + 2 * hk) * hd + hq * hd * d + 3 * d * f


SHAPES = {
    # two-layer toy decoder used end to end (embedding -> 2 layers -> head)
    "tiny": Shape(d=256, n_q=4, n_kv=4, hd=64, ffn=1024, vocab=1024),
    # 9B-class dense layer: d 4096, 32 query / 8 KV heads of 128, SwiGLU 12288
    "9b": Shape(d=4096, n_q=32, n_kv=8, hd=128, ffn=12288, vocab=151936),
    # 27B-class dense layer: d 5120, 40 query / 8 KV heads of 128, SwiGLU 17408
    "27b": Shape(d=5120, n_q=40, n_kv=8, hd=128, ffn=17408, vocab=151936),
}


def rng_for(seed: int, tag: str) -> np.random.Generator:
    """Independent PCG64 stream for (seed, tag)."""
    ss = np.random.SeedSequence([int(seed) & 0xFFFFFFFF, zlib.crc32(tag.encode())])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    fa, fo = a.reshape(-1), out.reshape(-1)
    for s in range(0, fa.size, _CHUNK):
        u = fa[s:s + _CHUNK].view(np.uint32)
        r = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
        fo[s:s + _CHUNK] = ((u + r) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(u) -> np.ndarray:
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def normal_f32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """N(0, std^2) in fp32; chunks of the draw come from child streams of rng."""
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)

    def fill(r, s, n):
        flat[s:s + n] = r.standard_normal(n, dtype=np.float32) * np.float32(std)
    _parallel_chunks(rng, flat.size, _GEN_CHUNK, fill)
    return out


def normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """N(0, std^2) drawn in fp32, stored as bf16 bit patterns."""
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)

    def fill(r, s, n):
        flat[s:s + n] = f32_to_bf16_bits(r.standard_normal(n, dtype=np.float32) * np.float32(std))
    _parallel_chunks(rng, flat.size, _GEN_CHUNK, fill)
    return out


def quantize_int4_g32(w: np.ndarray):
    """Symmetric int4, groups of 32 consecutive reduction elements.

    Returns (packed uint32 [N, K/8], scales as bf16 bits [N, K/32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    if k % 32:
        raise ValueError("reduction size must be a multiple of 32")
    packed = np.empty((n, k // 8), dtype=np.uint32)
    scales = np.empty((n, k // 32), dtype=np.uint16)
    rows = max(1, _CHUNK // k)
    for r0 in range(0, n, rows):
        g = w[r0:r0 + rows].reshape(-1, k // 32, 32)
        amax = np.abs(g).max(axis=2)
        s_bits = f32_to_bf16_bits(amax / np.float32(7.0))
        s = bf16_bits_to_f32(s_bits)
        safe = np.where(s > 0, s, np.float32(1.0))[..., None]
        qf = np.where(s[..., None] > 0, g / safe, np.float32(0.0))
        q = np.clip(np.rint(qf), -7, 7).astype(np.int64) + 8
        nib = q.reshape(q.shape[0], k // 8, 8).astype(np.uint32)
        word = np.zeros(nib.shape[:2], dtype=np.uint32)
        for i in range(8):
            word |= nib[..., i] << np.uint32(4 * i)
        packed[r0:r0 + rows] = word
        scales[r0:r0 + rows] = s_bits
    return packed, scales


def uniforms_2m24(rng: np.random.Generator, n: int) -> np.ndarray:
    """n uniforms on the 2^-24 grid of [0, 1), exact in fp32."""
    k = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    return ((k >> np.uint32(8)).astype(np.float32) * np.float32(2.0 ** -24)).astype(np.float32)


def stable_softmax_f32(z: np.ndarray) -> np.ndarray:
    """Synthetic probability rows from synthetic logits (rows sum to ~1 in fp32).

    Used only to build the draft/target distributions a workload names."""
    z = np.asarray(z, dtype=np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def sample_from_probs(rng: np.random.Generator, probs: np.ndarray) -> np.ndarray:
    """One categorical draw per row of a [n, V] probability matrix."""
    probs = np.asarray(probs, dtype=np.float64)
    cdf = np.cumsum(probs, axis=1)
    u = rng.random(probs.shape[0]) * cdf[:, -1]
    idx = (cdf < u[:, None]).sum(axis=1)
    return np.minimum(idx, probs.shape[1] - 1).astype(np.int32)


@dataclasses.dataclass
class Weights:
    """One matrix in [N, K] (output features x reduction) layout.

    wtype 'f32': data float32 [N, K]; 'bf16': uint16 bits [N, K];
    'int4': data uint32 [N, K/8] packed codes, scale uint16 bits [N, K/32]."""
    wtype: str
    n: int
    k: int
    data: np.ndarray
    scale: np.ndarray | None = None

    @property
    def nbytes(self) -> int:
        return int(self.data.nbytes + (0 if self.scale is None else self.scale.nbytes))


def _matrix(rng, n, k, std, wtype) -> Weights:
    if wtype == "f32":
        return Weights("f32", n, k, normal_f32(rng, (n, k), std))
    if wtype == "bf16":
        return Weights("bf16", n, k, normal_bf16(rng, (n, k), std))
    if wtype == "int4":
        packed = np.empty((n, k // 8), dtype=np.uint32)
        scales = np.empty((n, k // 32), dtype=np.uint16)
        rows = max(1, (1 << 22) // k)

        def block(r, r0, m):
            w = r.standard_normal((m, k), dtype=np.float32) * np.float32(std)
            packed[r0:r0 + m], scales[r0:r0 + m] = quantize_int4_g32(w)
        _parallel_chunks(rng, n, rows, block)
        return Weights("int4", n, k, packed, scales)
    raise ValueError(wtype)


def layer_weights(shape: Shape, wtype: str, seed: int, tag: str = "layer0") -> dict:
    """Decoder-layer matrices, all N(0, 1/d) as the workloads state."""
    d, hq, hk, hd, f = shape.d, shape.n_q, shape.n_kv, shape.hd, shape.ffn
    std = d ** -0.5
    out = {}
    for name, n, k in (("wq", hq * hd, d), ("wk", hk * hd, d), ("wv", hk * hd, d),
                       ("wo", d, hq * hd), ("w_gate", f, d), ("w_up", f, d),
                       ("w_down", d, f)):
        out[name] = _matrix(rng_for(seed, f"{tag}/{name}"), n, k, std, wtype)
    return out


def head_weights(shape: Shape, wtype: str, seed: int) -> Weights:
    return _matrix(rng_for(seed, "lm_head"), shape.vocab, shape.d, shape.d ** -0.5, wtype)


def embed_weights(shape: Shape, seed: int) -> np.ndarray:
    return normal_f32(rng_for(seed, "embed"), (shape.vocab, shape.d), shape.d ** -0.5)


def kv_cache(shape: Shape, ctx: np.ndarray, cap: int, seed: int, tag: str = "layer0"):
    """Logical K and V caches [B, n_kv, cap, hd] as bf16 bits.

    Rows < ctx_i hold N(0,1) entries (already-rotated keys); rows >= ctx_i hold
    a finite sentinel (bf16 of 3.0e38) that must never influence a result."""
    b = len(ctx)
    k = np.full((b, shape.n_kv, cap, shape.hd), 0x7F61, dtype=np.uint16)
    v = np.full((b, shape.n_kv, cap, shape.hd), 0x7F61, dtype=np.uint16)
    ctx = [int(c) for c in np.asarray(ctx)]
    rk, rv = rng_for(seed, f"{tag}/kcache"), rng_for(seed, f"{tag}/vcache")
    kk, vk = (rk.spawn(b), rv.spawn(b)) if b else ([], [])

    def seq(i):  # sequence i from its own child streams (no nested pool use)
        c = ctx[i]
        if c:
            shp = (shape.n_kv, c, shape.hd)
            k[i, :, :c] = f32_to_bf16_bits(kk[i].standard_normal(shp, dtype=np.float32))
            v[i, :, :c] = f32_to_bf16_bits(vk[i].standard_normal(shp, dtype=np.float32))
    for f in [_pool().submit(seq, i) for i in range(b)]:
        f.result()
    return k, v


def kv_cache_int8(shape: Shape, ctx: np.ndarray, cap: int, seed: int, tag: str = "layer0"):
    """Synthetic int8 K and V caches: codes [B, n_kv, cap, hd] int8 and fp32
    scales [B, n_kv, cap] per cached vector, shaped like quantised N(0,1)
    vectors (codes from a rounded N(0, 40^2) clipped to +-127, scales around
    3/127).  Rows >= ctx_i hold code 127 with scale 3e38 (never to be read)."""
    b = len(ctx)
    out = []
    for which in ("k", "v"):
        codes = np.full((b, shape.n_kv, cap, shape.hd), 127, dtype=np.int8)
        scales = np.full((b, shape.n_kv, cap), 3.0e38, dtype=np.float32)
        rng = rng_for(seed, f"{tag}/{which}cache_int8")
        for i in range(b):
            c = int(np.asarray(ctx)[i])
            if c:
                codes[i, :, :c] = np.clip(np.rint(rng.standard_normal((shape.n_kv, c, shape.hd)) * 40.0),
                                          -127, 127).astype(np.int8)
                scales[i, :, :c] = (3.0 / 127.0 * np.exp(0.1 * rng.standard_normal((shape.n_kv, c)))
                                    ).astype(np.float32)
        out += [codes, scales]
    return tuple(out)  # kcodes, kscales, vcodes, vscales


def hidden_states(t: int, d: int, seed: int, tag: str = "x") -> np.ndarray:
    return normal_bf16(rng_for(seed, tag), (t, d), 1.0)
