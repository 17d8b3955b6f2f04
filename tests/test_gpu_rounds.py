"""Several rounds of draft -> verify -> accept/commit -> re-plan on one batch.

A small model (embedding, two bf16 decoder layers on packed weights, LM
head) keeps its KV caches on the device from round to round; each round the
planner (budget mode) sets the draft lengths for the sequences still live,
drafts are drawn from random draft distributions, the stacked tokens
(last committed token + drafts) go through the model, and the acceptance
kernel commits.  The oracle replays every round with its own caches: hidden
states and logits within the bf16 tolerance, acceptance, next tokens and
committed lengths bit-exact on the GPU's probabilities (the acceptance rule
is exact arithmetic on given probabilities), and the device caches equal to
the oracle's at every committed position within bf16 rounding.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (TOL, OF, OV, dev_bf16_to_f64, oracle_accept, rel_rows, run_accept, say, sv,
                         tg)
from workloads import (Shape, accept_inputs, custom_workload, embed_weights, f32_to_bf16_bits,
                       head_weights, kv_cache, layer_weights)

pytestmark = pytest.mark.gpu


def _layer_out(L, bs, x, ws_cache):
    y = torch.empty_like(x)
    n = sv.sv_verify_layer_workspace_bytes(L, bs)
    if ws_cache.get("n", 0) < n:
        ws_cache["ws"], ws_cache["n"] = tg.workspace(n), n
    assert sv.sv_verify_layer(L, bs, x, y, 0, ws_cache["ws"], ws_cache["n"], tg.stream_handle()) == 0
    return y


def test_rounds_plan_verify_accept_commit():
    shape = Shape(d=512, n_q=8, n_kv=2, hd=128, ffn=1024, vocab=4099)
    seed, cap, n_layers, budget = 2024, 128, 2, 14
    ctx = [5, 40, 0, 17, 23]
    stop_at = [11, 49, 4, 29, 30]               # a sequence leaves once its length reaches this
    B0 = len(ctx)
    ctx0 = list(ctx)
    E = embed_weights(shape, seed)
    table = tg.to_dev(E)
    Ws = [layer_weights(shape, "bf16", seed, f"layer{k}") for k in range(n_layers)]
    devs = [{k: tg.upload_matrix(v, packed=True) for k, v in W.items()} for W in Ws]
    Ls = [tg.decoder_struct(shape, "bf16", d, packed=True) for d in devs]
    Wlm = head_weights(shape, "bf16", seed)
    lm = tg.upload_matrix(Wlm, packed=True)
    Lh = tg.head_struct(shape, "bf16", lm, packed=True)
    # per layer: host oracle caches (bf16 bits [B][n_kv][cap][hd]) and the device caches
    kc_o, vc_o, kdev, vdev = [], [], [], []
    for k in range(n_layers):
        kc, vc = kv_cache(shape, np.asarray(ctx), cap, seed, f"layer{k}")
        kc_o.append(kc.copy())
        vc_o.append(vc.copy())
        kdev.append([tg.to_dev(kc[i]) for i in range(B0)])
        vdev.append([tg.to_dev(tg.v_blocked(vc[i])) for i in range(B0)])
    last = list(np.random.default_rng(seed).integers(0, shape.vocab, B0).astype(np.int32))
    live = list(range(B0))
    ws_cache = {}
    plan = sv.make_plan_params(sv.SV_PLAN_BUDGET, 4, budget_tokens=budget, fill_remainder=True)
    total_acc, rounds = 0, 0
    seen_gammas = set()
    while live and rounds < 16:
        st, gl, _ = sv.sv_plan_gamma(plan, len(live))
        assert st == sv.SV_OK
        gamma = [int(g) for g in gl]
        seen_gammas.add(tuple(gamma))
        lctx = [ctx[i] for i in live]
        assert all(c + g + 1 <= cap for c, g in zip(lctx, gamma))
        wl = custom_workload(shape, "bf16", gamma, lctx, draft="temp", temp=0.7, seed=seed + rounds,
                             cap=cap)
        acc_in = accept_inputs(wl, shape.vocab, seed=seed + 101 * rounds)
        # stacked tokens: each live sequence's last committed token, then its drafts
        tokens, o = [], 0
        for i, g in zip(live, gamma):
            tokens += [last[i]] + list(acc_in["draft"][o:o + g])
            o += g
        tokens = np.asarray(tokens, np.int32)
        T = len(tokens)
        # device: embedding, layers (caches shared across rounds), head
        b_emb = tg.DeviceBatch(gamma, lctx, cap)
        x = torch.empty(T, shape.d, dtype=torch.bfloat16, device="cuda")
        assert sv.sv_verify_layer(tg.embed_struct(shape, table), b_emb.struct(),
                                  torch.tensor(tokens, device="cuda"), x, 0, None, 0,
                                  tg.stream_handle()) == 0
        h = x
        xo = OV.embed(E, tokens)
        for k in range(n_layers):
            bk = tg.DeviceBatch(gamma, lctx, cap, caches=([kdev[k][i] for i in live],
                                                          [vdev[k][i] for i in live]))
            h = _layer_out(Ls[k], bk.struct(), h, ws_cache)
            ref = OV.decoder_layer(shape, Ws[k], xo, gamma, lctx, kc_o[k][live], vc_o[k][live])
            err = rel_rows(dev_bf16_to_f64(h), ref.y)
            assert err < TOL["bf16"], (rounds, k, err)
            # the oracle appends its own rows (rounded to bf16) at ctx_i .. ctx_i + gamma_i
            for n_i, i in enumerate(live):
                c, g = ctx[i], gamma[n_i]
                kc_o[k][i, :, c:c + g + 1] = f32_to_bf16_bits(ref.k_new[n_i].astype(np.float32))
                vc_o[k][i, :, c:c + g + 1] = f32_to_bf16_bits(ref.v_new[n_i].astype(np.float32))
            xo = ref.y
        bh = tg.DeviceBatch(gamma, lctx, cap)
        nh = {f: sv.sv_verify_layer_workspace_bytes(Lh, bh.struct(), f) for f in (0, sv.SV_HEAD_LOGITS)}
        wsh = tg.workspace(max(nh.values()))
        lg = torch.empty(T, shape.vocab, dtype=torch.float32, device="cuda")
        pr = torch.empty_like(lg)
        assert sv.sv_verify_layer(Lh, bh.struct(), h, lg, sv.SV_HEAD_LOGITS, wsh, nh[sv.SV_HEAD_LOGITS],
                                  tg.stream_handle()) == 0
        assert sv.sv_verify_layer(Lh, bh.struct(), h, pr, 0, wsh, nh[0], tg.stream_handle()) == 0
        errh = rel_rows(lg.cpu().numpy(), OV.head_logits(Wlm, xo))
        assert errh < TOL["bf16"], (rounds, errh)
        # accept + commit on the GPU's probabilities, against the oracle on the same rows
        inp = dict(acc_in, p=pr.cpu().numpy())
        ga, gy, gk, gerr = run_accept(gamma, shape.vocab, inp, lctx)
        ra, ry, rk, _ = oracle_accept(gamma, inp, lctx)
        assert gerr == 0
        np.testing.assert_array_equal(ga, ra)
        np.testing.assert_array_equal(gy, ry)
        np.testing.assert_array_equal(gk, rk)
        say(f"round {rounds}: live {live} gamma {gamma} accepted {ga.tolist()} next {gy.tolist()} "
            f"lengths {gk.tolist()} (layer err {err:.1e}, logits err {errh:.1e})")
        total_acc += int(ga.sum())
        for n_i, i in enumerate(live):
            ctx[i] = int(gk[n_i])
            last[i] = int(gy[n_i])
        live = [i for i in live if ctx[i] < stop_at[i]]
        rounds += 1
    assert not live, "every sequence reaches its stop length"
    assert len(seen_gammas) > 1                 # the plan changed as the batch shrank
    assert total_acc > 0
    # the device caches: the starting rows untouched, every row committed since
    # equal to the oracle's (bf16 rounding of the two computations apart)
    for k in range(n_layers):
        for i in range(B0):
            kd = tg.DeviceBatch([0], [ctx[i]], cap, caches=([kdev[k][i]], [vdev[k][i]]))
            c0, c = ctx0[i], ctx[i]
            gk_bits, gv_bits = kd.k_logical(0), kd.v_logical(0)
            np.testing.assert_array_equal(gk_bits[:, :c0], kc_o[k][i, :, :c0])
            np.testing.assert_array_equal(gv_bits[:, :c0], vc_o[k][i, :, :c0])
            for got, want in ((gk_bits, kc_o[k][i]), (gv_bits, vc_o[k][i])):
                e = rel_rows(OF.bf16_to_f64(got[:, c0:c]).reshape(-1, shape.hd),
                             OF.bf16_to_f64(want[:, c0:c]).reshape(-1, shape.hd))
                assert e < TOL["bf16"], (k, i, e)
