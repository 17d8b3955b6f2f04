"""Verify-pass oracle pins (no page prints logits, so these pin it to
mathematics and to independent library formulations):

1. Equality with a formulation built from torch's own routines in fp64:
   rms_norm, linear, scaled_dot_product_attention with an explicit causal
   mask, silu, and RoPE written as multiplication by a unit complex number.
2. Verifying gamma+1 tokens equals gamma+1 sequential single-token decodes
   (each committing its key/value row before the next).
3. gamma = 0 is plain decoding, and a sequence's result does not depend on
   the rest of the batch.
4. RoPE: identity at position 0, pairwise norm preserved, scores invariant to
   a common position shift.
5. Attention: one visible key returns its value; identical keys return the
   mean of the values.
6. Storage formats: int4 decode order/values and bf16 rounding against torch.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import formats as OF
from oracle import verify as OV
from workloads import (Shape, custom_workload, f32_to_bf16_bits, hidden_states,
                       kv_cache, layer_weights, quantize_int4_g32)

SMALL = Shape(d=128, n_q=4, n_kv=2, hd=32, ffn=192, vocab=300)


def _torch_int8_store(t):
    """Per (position, head) symmetric int8 storage of appended keys/values,
    written with torch routines: bf16 rounding, fp32 absmax / 127 scale,
    round-half-even codes clipped to +-127, then code * scale."""
    b = t.to(torch.bfloat16).to(torch.float32)
    scale = (b.abs().amax(dim=-1, keepdim=True) / 127.0).to(torch.float32)
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    codes = torch.clamp(torch.round(b / safe), -127, 127)
    codes = torch.where(scale > 0, codes, torch.zeros_like(codes))
    return codes.to(torch.float64) * scale.to(torch.float64)


def _torch_layer(shape, W, x, gamma, ctx, kc, vc, eps=1e-6, theta=10000.0, ks=None, vs=None):
    """Independent formulation from torch library routines (fp64).  With
    ks / vs (fp32 scales) the caches hold int8 codes and the appended rows are
    stored as int8 (_torch_int8_store)."""
    Wt = {k: torch.from_numpy(v) for k, v in W.items()}
    hd, hq, hk = shape.hd, shape.n_q, shape.n_kv
    half = hd // 2
    freqs = theta ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ys, r0 = [], 0
    for i in range(len(gamma)):
        n, c = int(gamma[i]) + 1, int(ctx[i])
        xs = torch.from_numpy(x[r0:r0 + n])
        h = F.rms_norm(xs, (shape.d,), eps=eps)
        q = F.linear(h, Wt["wq"]).view(n, hq, hd)
        k = F.linear(h, Wt["wk"]).view(n, hk, hd)
        v = F.linear(h, Wt["wv"]).view(n, hk, hd)
        pos = torch.arange(c, c + n, dtype=torch.float64)
        rot = torch.polar(torch.ones(n, half, dtype=torch.float64), pos[:, None] * freqs[None])

        def rope(t):
            z = torch.complex(t[..., :half], t[..., half:]) * rot[:, None, :]
            return torch.cat([z.real, z.imag], dim=-1)
        q, k = rope(q), rope(k)
        if ks is None:
            Kc = torch.from_numpy(OF.bf16_to_f64(kc[i, :, :c]))
            Vc = torch.from_numpy(OF.bf16_to_f64(vc[i, :, :c]))
        else:
            Kc = torch.from_numpy(kc[i, :, :c].astype(np.float64)) * \
                torch.from_numpy(ks[i, :, :c].astype(np.float64))[..., None]
            Vc = torch.from_numpy(vc[i, :, :c].astype(np.float64)) * \
                torch.from_numpy(vs[i, :, :c].astype(np.float64))[..., None]
            k, v = _torch_int8_store(k), _torch_int8_store(v)
        K = torch.cat([Kc, k.transpose(0, 1)], dim=1)
        V = torch.cat([Vc, v.transpose(0, 1)], dim=1)
        G = hq // hk
        K = K.repeat_interleave(G, dim=0)
        V = V.repeat_interleave(G, dim=0)
        mask = torch.arange(c + n)[None, :] <= (c + torch.arange(n))[:, None]
        o = F.scaled_dot_product_attention(q.transpose(0, 1), K, V, attn_mask=mask)
        x1 = xs + F.linear(o.transpose(0, 1).reshape(n, hq * hd), Wt["wo"])
        h2 = F.rms_norm(x1, (shape.d,), eps=eps)
        y = x1 + F.linear(F.silu(F.linear(h2, Wt["w_gate"])) * F.linear(h2, Wt["w_up"]),
                          Wt["w_down"])
        ys.append(y.numpy())
        r0 += n
    return np.concatenate(ys)


def _case(gamma, ctx, seed=3, wtype="bf16", shape=SMALL):
    wl = custom_workload(shape, wtype, gamma, ctx, seed=seed)
    W = {k: OF.matrix_f64(v) for k, v in layer_weights(shape, wtype, seed).items()}
    kc, vc = kv_cache(shape, wl.ctx, wl.cap, seed)
    x = OF.bf16_to_f64(hidden_states(wl.T, shape.d, seed))
    return wl, W, kc, vc, x


@pytest.mark.parametrize("wtype", ["bf16", "int4", "f32"])
def test_layer_matches_library_formulation(wtype):
    wl, W, kc, vc, x = _case([2, 0, 3, 1], [5, 0, 17, 40], wtype=wtype)
    out = OV.decoder_layer(SMALL, W, x, wl.gamma, wl.ctx, kc, vc, store_bf16=False)
    ref = _torch_layer(SMALL, W, x, wl.gamma, wl.ctx, kc, vc)
    np.testing.assert_allclose(out.y, ref, rtol=0, atol=1e-11 * np.abs(ref).max())


def test_layer_tiny_shape_matches_library_formulation():
    from workloads import SHAPES
    sh = SHAPES["tiny"]
    wl, W, kc, vc, x = _case([4], [128], wtype="f32", shape=sh)
    out = OV.decoder_layer(sh, W, x, wl.gamma, wl.ctx, kc, vc, store_bf16=False)
    ref = _torch_layer(sh, W, x, wl.gamma, wl.ctx, kc, vc)
    np.testing.assert_allclose(out.y, ref, rtol=0, atol=1e-11 * np.abs(ref).max())


def test_verify_equals_sequential_decodes():
    wl, W, kc, vc, x = _case([4, 2, 0], [9, 0, 30], seed=5)
    full = OV.decoder_layer(SMALL, W, x, wl.gamma, wl.ctx, kc, vc)
    kc2, vc2 = kc.copy(), vc.copy()
    for i in range(wl.B):
        for j in range(int(wl.gamma[i]) + 1):
            row = int(wl.q_start[i]) + j
            pos = int(wl.ctx[i]) + j
            ctx_now = wl.ctx.copy()
            ctx_now[i] = pos
            gam = np.zeros(wl.B, np.int32)
            # single-token decode of this row: place it as sequence i's only token
            xs = np.zeros((wl.B, SMALL.d))
            xs[i] = x[row]
            one = OV.decoder_layer(SMALL, W, xs, gam, ctx_now, kc2, vc2, seqs=[i])
            np.testing.assert_allclose(one.y[0], full.y[row], rtol=0,
                                       atol=1e-12 * np.abs(full.y).max())
            np.testing.assert_array_equal(one.k_new[i][:, 0], full.k_new[i][:, j])
            kc2[i, :, pos] = f32_to_bf16_bits(one.k_new[i][:, 0].astype(np.float32))
            vc2[i, :, pos] = f32_to_bf16_bits(one.v_new[i][:, 0].astype(np.float32))


def test_sequence_independent_of_batch():
    wl, W, kc, vc, x = _case([1, 3, 0, 2], [7, 11, 0, 64], seed=9)
    full = OV.decoder_layer(SMALL, W, x, wl.gamma, wl.ctx, kc, vc)
    for i in range(wl.B):
        part = OV.decoder_layer(SMALL, W, x, wl.gamma, wl.ctx, kc, vc, seqs=[i])
        rows = np.arange(wl.q_start[i], wl.q_start[i + 1])
        np.testing.assert_allclose(part.y, full.y[rows], rtol=0, atol=1e-12 * np.abs(full.y).max())


def test_token_map():
    qs, seq, j, pos = OV.token_map([2, 0, 3], [10, 0, 5])
    assert list(qs) == [0, 3, 4, 8]
    assert list(seq) == [0, 0, 0, 1, 2, 2, 2, 2]
    assert list(j) == [0, 1, 2, 0, 0, 1, 2, 3]
    assert list(pos) == [10, 11, 12, 0, 5, 6, 7, 8]


def test_rope_properties():
    rng = np.random.default_rng(0)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    np.testing.assert_array_equal(OV.rope(q, 0), q)
    r = OV.rope(q, 1234)
    pair_norm = lambda a: a[:32] ** 2 + a[32:] ** 2  # noqa: E731
    np.testing.assert_allclose(pair_norm(r), pair_norm(q), rtol=1e-12)
    for m, n, dlt in ((5, 3, 100), (0, 77, 4000), (1000, 2, 17)):
        s0 = OV.rope(q, m) @ OV.rope(k, n)
        s1 = OV.rope(q, m + dlt) @ OV.rope(k, n + dlt)
        assert s0 == pytest.approx(s1, rel=1e-9, abs=1e-9)
    # first pair turns by exactly pos radians (theta^0 = 1)
    e = np.zeros(64)
    e[0] = 1.0
    r = OV.rope(e, 3)
    assert r[0] == pytest.approx(np.cos(3.0)) and r[32] == pytest.approx(np.sin(3.0))


def test_attention_special_cases():
    rng = np.random.default_rng(1)
    q = rng.standard_normal(16)
    keys, vals = rng.standard_normal((1, 16)), rng.standard_normal((1, 16))
    np.testing.assert_allclose(OV.attend(q, keys, vals), vals[0], rtol=1e-15)
    keys = np.tile(rng.standard_normal(16), (7, 1))
    vals = rng.standard_normal((7, 16))
    np.testing.assert_allclose(OV.attend(q, keys, vals), vals.mean(0), rtol=1e-13)


def test_empty_context_first_token_sees_itself():
    # ctx = 0, gamma = 0: attention output is the token's own value row
    wl, W, kc, vc, x = _case([0], [0], seed=2)
    out = OV.decoder_layer(SMALL, W, x, wl.gamma, wl.ctx, kc, vc, store_bf16=False)
    h = OV.rms_norm(x)
    v = (h @ W["wv"].T).reshape(SMALL.n_kv, SMALL.hd)
    o = np.repeat(v, SMALL.n_q // SMALL.n_kv, axis=0).reshape(-1)
    x1 = x + o @ W["wo"].T
    np.testing.assert_allclose(out.y - x1, _torch_layer(SMALL, W, x, [0], [0], kc, vc) - x1,
                               atol=1e-12)


def test_head_matches_library_formulation():
    rng = np.random.default_rng(4)
    y = rng.standard_normal((5, 64))
    w = rng.standard_normal((300, 64)) / 8
    lg = OV.head_logits(w, y)
    ref = F.linear(F.rms_norm(torch.from_numpy(y), (64,), eps=1e-6), torch.from_numpy(w)).numpy()
    np.testing.assert_allclose(lg, ref, rtol=1e-13, atol=1e-13)
    p = OV.softmax(lg)
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(p, torch.softmax(torch.from_numpy(lg), -1).numpy(), rtol=1e-12)


def test_int4_decode_layout_and_values():
    # hand-packed word: nibble i of word m is reduction index 8m + i, value code + 8
    codes = np.array([-7, -3, 0, 1, 7, 2, -1, 5] * 4, dtype=np.int64)   # one group of 32
    word = np.zeros(4, np.uint32)
    for kk, c in enumerate(codes):
        word[kk // 8] |= np.uint32((c + 8) << (4 * (kk % 8)))
    scale = f32_to_bf16_bits(np.array([[0.375]], np.float32))
    w = OF.int4_to_f64(word[None, :], scale)
    np.testing.assert_array_equal(w[0], codes * 0.375)
    # quantizer round trip: error at most half a step, exact for on-grid values
    rng = np.random.default_rng(0)
    m = rng.standard_normal((6, 64)).astype(np.float32)
    packed, sc = quantize_int4_g32(m)
    dq = OF.int4_to_f64(packed, sc)
    s = np.repeat(OF.bf16_to_f64(sc), 32, axis=1)
    assert np.all(np.abs(dq - m) <= 0.5 * s + 1e-7 + np.abs(m) * 0.01)
    p2, s2 = quantize_int4_g32(dq.astype(np.float32))
    np.testing.assert_array_equal(OF.int4_to_f64(p2, s2), dq)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(OF.round_bf16(a.astype(np.float64)), ref)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0])
    np.testing.assert_array_equal(OF.round_bf16(ties), [1.0, 1 + 2 ** -6, -1.0, 0.0])
    np.testing.assert_array_equal(OF.bf16_to_f64(f32_to_bf16_bits(a)), ref)


def test_embed_selects_rows_by_token():
    # a hand-written table: row r holds r + 0.25 c, so each gathered value names
    # its row and column; bf16 storage decodes to the same values
    table = np.array([[r + 0.25 * c for c in range(4)] for r in range(5)], np.float32)
    got = OV.embed(table, [3, 0, 3, 4])
    np.testing.assert_array_equal(got, [[3, 3.25, 3.5, 3.75], [0, 0.25, 0.5, 0.75],
                                        [3, 3.25, 3.5, 3.75], [4, 4.25, 4.5, 4.75]])
    got_bf = OV.embed(f32_to_bf16_bits(table), np.array([1, 2], np.int32))
    np.testing.assert_array_equal(got_bf, [[1, 1.25, 1.5, 1.75], [2, 2.25, 2.5, 2.75]])
    assert OV.embed(table, []).shape == (0, 4)


def test_int8_kv_quantizer_hand_example_and_bounds():
    codes, sc = OV.quantize_int8_row([0.75, -1.0, 0.3, 0.0])
    assert sc == np.float32(np.float32(1.0) / np.float32(127.0))
    np.testing.assert_array_equal(codes, [95, -127, 38, 0])
    codes, sc = OV.quantize_int8_row(np.zeros(8))
    assert sc == 0 and not codes.any()
    rng = np.random.default_rng(3)
    for _ in range(50):
        v = OF.round_bf16(rng.standard_normal(128) * np.exp(rng.uniform(-6, 6)))
        codes, sc = OV.quantize_int8_row(v)
        dq = OV.dequantize_int8(codes, sc)
        assert np.abs(codes).max() == 127
        # half a step, plus the fp32 rounding of the division (|x / s| <= 127)
        assert np.all(np.abs(dq - v) <= (0.5 + 127 * 2.0 ** -23) * float(sc))


def _int8_cache(kc, vc):
    """Synthetic int8 caches from the bf16 ones: one code vector and scale per
    (sequence, head, position)."""
    B, H, cap, hd = kc.shape
    out = []
    for c in (kc, vc):
        codes = np.zeros(c.shape, np.int8)
        scales = np.zeros((B, H, cap), np.float32)
        vals = OF.bf16_to_f64(c)
        for b in range(B):
            for h in range(H):
                for pos in range(cap):
                    codes[b, h, pos], scales[b, h, pos] = OV.quantize_int8_row(vals[b, h, pos])
        out += [codes, scales]
    return out


def test_int8_kv_layer_matches_library_formulation():
    wl, W, kc, vc, x = _case([2, 0, 3], [5, 0, 17], wtype="bf16")
    k8, ks, v8, vs = _int8_cache(kc, vc)
    out = OV.decoder_layer(SMALL, W, x, wl.gamma, wl.ctx, k8, v8, kscale=ks, vscale=vs)
    ref = _torch_layer(SMALL, W, x, wl.gamma, wl.ctx, k8, v8, ks=ks, vs=vs)
    np.testing.assert_allclose(out.y, ref, rtol=0, atol=1e-11 * np.abs(ref).max())
    # and it is a different layer from the bf16 cache's
    out16 = OV.decoder_layer(SMALL, W, x, wl.gamma, wl.ctx, kc, vc)
    assert np.abs(out16.y - out.y).max() > 1e-4 * np.abs(out.y).max()
