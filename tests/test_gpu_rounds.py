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

from gpu_helpers import (TOL, OA, OF, OV, dev_bf16_to_f64, oracle_accept, rel_rows, run_accept, say,
                         sv, tg)
from oracle import plan as OP
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


class _Model:
    """The small model, its device caches and the oracle's caches, with one
    round of verify -> accept/commit on both sides."""

    def __init__(self, ctx, seed=2024, cap=128, n_layers=2):
        self.shape = shape = Shape(d=512, n_q=8, n_kv=2, hd=128, ffn=1024, vocab=4099)
        self.seed, self.cap, self.n_layers = seed, cap, n_layers
        self.ctx = list(ctx)
        self.ctx0 = list(ctx)
        B0 = len(ctx)
        self.E = embed_weights(shape, seed)
        self.table = tg.to_dev(self.E)
        self.Ws = [layer_weights(shape, "bf16", seed, f"layer{k}") for k in range(n_layers)]
        devs = [{k: tg.upload_matrix(v, packed=True) for k, v in W.items()} for W in self.Ws]
        self.devs = devs
        self.Ls = [tg.decoder_struct(shape, "bf16", d, packed=True) for d in devs]
        self.Wlm = head_weights(shape, "bf16", seed)
        self.lm = tg.upload_matrix(self.Wlm, packed=True)
        self.Lh = tg.head_struct(shape, "bf16", self.lm, packed=True)
        # per layer: host oracle caches (bf16 bits [B][n_kv][cap][hd]) and the device caches
        self.kc_o, self.vc_o, self.kdev, self.vdev = [], [], [], []
        for k in range(n_layers):
            kc, vc = kv_cache(shape, np.asarray(ctx), cap, seed, f"layer{k}")
            self.kc_o.append(kc.copy())
            self.vc_o.append(vc.copy())
            self.kdev.append([tg.to_dev(kc[i]) for i in range(B0)])
            self.vdev.append([tg.to_dev(tg.v_blocked(vc[i])) for i in range(B0)])
        self.last = list(np.random.default_rng(seed).integers(0, shape.vocab, B0).astype(np.int32))
        self.ws_cache = {}

    def round(self, live, gamma, r):
        """One round for the live sequences with these draft lengths; returns
        the GPU's (accepted, next, lengths) after checking them against the
        oracle, and commits them to both sides' state."""
        shape, cap, seed = self.shape, self.cap, self.seed
        lctx = [self.ctx[i] for i in live]
        assert all(c + g + 1 <= cap for c, g in zip(lctx, gamma))
        wl = custom_workload(shape, "bf16", gamma, lctx, draft="temp", temp=0.7, seed=seed + r, cap=cap)
        acc_in = accept_inputs(wl, shape.vocab, seed=seed + 101 * r)
        # stacked tokens: each live sequence's last committed token, then its drafts
        tokens, o = [], 0
        for i, g in zip(live, gamma):
            tokens += [self.last[i]] + list(acc_in["draft"][o:o + g])
            o += g
        tokens = np.asarray(tokens, np.int32)
        T = len(tokens)
        # device: embedding, layers (caches shared across rounds), head
        b_emb = tg.DeviceBatch(gamma, lctx, cap)
        x = torch.empty(T, shape.d, dtype=torch.bfloat16, device="cuda")
        assert sv.sv_verify_layer(tg.embed_struct(shape, self.table), b_emb.struct(),
                                  torch.tensor(tokens, device="cuda"), x, 0, None, 0,
                                  tg.stream_handle()) == 0
        h = x
        xo = OV.embed(self.E, tokens)
        for k in range(self.n_layers):
            bk = tg.DeviceBatch(gamma, lctx, cap, caches=([self.kdev[k][i] for i in live],
                                                          [self.vdev[k][i] for i in live]))
            h = _layer_out(self.Ls[k], bk.struct(), h, self.ws_cache)
            ref = OV.decoder_layer(shape, self.Ws[k], xo, gamma, lctx, self.kc_o[k][live],
                                   self.vc_o[k][live])
            err = rel_rows(dev_bf16_to_f64(h), ref.y)
            assert err < TOL["bf16"], (r, k, err)
            # the oracle appends its own rows (rounded to bf16) at ctx_i .. ctx_i + gamma_i
            for n_i, i in enumerate(live):
                c, g = self.ctx[i], gamma[n_i]
                self.kc_o[k][i, :, c:c + g + 1] = f32_to_bf16_bits(ref.k_new[n_i].astype(np.float32))
                self.vc_o[k][i, :, c:c + g + 1] = f32_to_bf16_bits(ref.v_new[n_i].astype(np.float32))
            xo = ref.y
        bh = tg.DeviceBatch(gamma, lctx, cap)
        nh = {f: sv.sv_verify_layer_workspace_bytes(self.Lh, bh.struct(), f) for f in (0, sv.SV_HEAD_LOGITS)}
        wsh = tg.workspace(max(nh.values()))
        lg = torch.empty(T, shape.vocab, dtype=torch.float32, device="cuda")
        pr = torch.empty_like(lg)
        assert sv.sv_verify_layer(self.Lh, bh.struct(), h, lg, sv.SV_HEAD_LOGITS, wsh,
                                  nh[sv.SV_HEAD_LOGITS], tg.stream_handle()) == 0
        assert sv.sv_verify_layer(self.Lh, bh.struct(), h, pr, 0, wsh, nh[0], tg.stream_handle()) == 0
        errh = rel_rows(lg.cpu().numpy(), OV.head_logits(self.Wlm, xo))
        assert errh < TOL["bf16"], (r, errh)
        # accept + commit on the GPU's probabilities, against the oracle on the same rows
        inp = dict(acc_in, p=pr.cpu().numpy())
        ga, gy, gk, gerr = run_accept(gamma, shape.vocab, inp, lctx)
        ra, ry, rk, _ = oracle_accept(gamma, inp, lctx)
        assert gerr == 0
        np.testing.assert_array_equal(ga, ra)
        np.testing.assert_array_equal(gy, ry)
        np.testing.assert_array_equal(gk, rk)
        say(f"round {r}: live {live} gamma {gamma} accepted {ga.tolist()} next {gy.tolist()} "
            f"lengths {gk.tolist()} (layer err {err:.1e}, logits err {errh:.1e})")
        for n_i, i in enumerate(live):
            self.ctx[i] = int(gk[n_i])
            self.last[i] = int(gy[n_i])
        return ga, gy, gk

    def check_caches(self):
        """The device caches: the starting rows untouched, every row committed
        since equal to the oracle's (bf16 rounding of the two computations apart)."""
        hd = self.shape.hd
        for k in range(self.n_layers):
            for i in range(len(self.ctx)):
                kd = tg.DeviceBatch([0], [self.ctx[i]], self.cap,
                                    caches=([self.kdev[k][i]], [self.vdev[k][i]]))
                c0, c = self.ctx0[i], self.ctx[i]
                gk_bits, gv_bits = kd.k_logical(0), kd.v_logical(0)
                np.testing.assert_array_equal(gk_bits[:, :c0], self.kc_o[k][i, :, :c0])
                np.testing.assert_array_equal(gv_bits[:, :c0], self.vc_o[k][i, :, :c0])
                for got, want in ((gk_bits, self.kc_o[k][i]), (gv_bits, self.vc_o[k][i])):
                    e = rel_rows(OF.bf16_to_f64(got[:, c0:c]).reshape(-1, hd),
                                 OF.bf16_to_f64(want[:, c0:c]).reshape(-1, hd))
                    assert e < TOL["bf16"], (k, i, e)


def test_rounds_plan_verify_accept_commit():
    ctx = [5, 40, 0, 17, 23]
    stop_at = [11, 49, 4, 29, 30]               # a sequence leaves once its length reaches this
    m = _Model(ctx)
    live = list(range(len(ctx)))
    plan = sv.make_plan_params(sv.SV_PLAN_BUDGET, 4, budget_tokens=14, fill_remainder=True)
    total_acc, rounds = 0, 0
    seen_gammas = set()
    while live and rounds < 16:
        st, gl, _ = sv.sv_plan_gamma(plan, len(live))
        assert st == sv.SV_OK
        gamma = [int(g) for g in gl]
        seen_gammas.add(tuple(gamma))
        ga, _, _ = m.round(live, gamma, rounds)
        total_acc += int(ga.sum())
        live = [i for i in live if m.ctx[i] < stop_at[i]]
        rounds += 1
    assert not live, "every sequence reaches its stop length"
    assert len(seen_gammas) > 1                 # the plan changed as the batch shrank
    assert total_acc > 0
    m.check_caches()


# Step-model constants fitted on MI355X (9B-class bf16 layer, its 151936-entry
# head and acceptance at 2048 cached tokens; the gamma = 1 fit of the (B, gamma)
# sweep): weight-read time, KV time per sequence, compute time per token, ms.
MI355X_FIT = {"t_w_ms": 0.3112, "k_ms": 0.0054, "c_ms": 0.0031}
PRIOR = [0.94 - 0.07 * k for k in range(8)]   # decaying acceptance until measured


def _alphas_from_counts(counts, min_reached=3):
    rates = OA.conditional_rates(counts)
    return [rates[k] if counts[0, k] >= min_reached else PRIOR[k] for k in range(counts.shape[1])]


def test_rounds_speedup_replan_from_position_counters():
    """Every round re-plans one draft length for the live batch in SPEEDUP
    mode, with the MI355X-fitted step model and per-position acceptance
    measured so far by the library's counters (accumulated on the device over
    the rounds; positions not yet measured take a decaying prior).  The
    oracle derives the same counters from its own acceptance results (bit
    for bit) and the oracle planner picks the same draft length."""
    ctx = [5, 40, 0, 17, 23, 9]
    stop_at = [c + n for c, n in zip(ctx, [14, 9, 20, 12, 16, 11])]
    m = _Model(ctx, seed=2025)
    live = list(range(len(ctx)))
    npos = 8
    counts_dev = torch.zeros(2, npos, dtype=torch.int64, device="cuda")
    counts_ref = np.zeros((2, npos), np.int64)
    rounds, gammas = 0, []
    while live and rounds < 40:
        alphas = _alphas_from_counts(counts_ref)
        pp = sv.make_plan_params(sv.SV_PLAN_SPEEDUP, npos, alpha=tuple(alphas), **MI355X_FIT)
        st, gl, bstar = sv.sv_plan_gamma(pp, len(live))
        assert st == sv.SV_OK
        want, _, want_bstar = OP.plan_speedup(len(live), npos, alphas, MI355X_FIT["t_w_ms"],
                                              MI355X_FIT["k_ms"], MI355X_FIT["c_ms"])
        assert gl == want and bstar == pytest.approx(want_bstar)
        # keep every draft within the cache
        gamma = [min(g, m.cap - 1 - m.ctx[i]) for g, i in zip(gl, live)]
        ga, _, _ = m.round(live, gamma, rounds)
        g_dev = torch.tensor(gamma, dtype=torch.int32, device="cuda")
        a_dev = torch.tensor(ga, dtype=torch.int32, device="cuda")
        assert sv.sv_accept_position_counts(len(live), npos, g_dev, a_dev, counts_dev,
                                            tg.stream_handle()) == sv.SV_OK
        counts_ref += OA.position_counts(gamma, ga, npos)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(counts_dev.cpu().numpy(), counts_ref)
        gammas.append(gl[0] if gl else 0)
        live = [i for i in live if m.ctx[i] < stop_at[i]]
        rounds += 1
    assert not live, "every sequence reaches its stop length"
    say(f"planned gammas per round {gammas}; conditional rates {OA.conditional_rates(counts_ref)}")
    assert counts_ref[0, 0] > 0
    # the same measured rates at larger live batches: the plan follows the batch
    alphas = _alphas_from_counts(counts_ref)
    pp = sv.make_plan_params(sv.SV_PLAN_SPEEDUP, npos, alpha=tuple(alphas), **MI355X_FIT)
    picks = []
    for b in (1, 8, 64, 256, 1024, 4096):
        st, gl, _ = sv.sv_plan_gamma(pp, b)
        want, _, _ = OP.plan_speedup(b, npos, alphas, MI355X_FIT["t_w_ms"], MI355X_FIT["k_ms"],
                                     MI355X_FIT["c_ms"])
        assert st == sv.SV_OK and gl == want
        picks.append(gl[0])
    say(f"planned gamma at B = 1, 8, 64, 256, 1024, 4096: {picks}")
    assert picks[0] >= picks[-1] and len(set(picks)) > 1
    m.check_caches()


def test_continuous_batching_refills_lanes():
    """Iteration-level batching through the verify path: the library's
    scheduler (continuous policy, 4 lanes) serves 7 requests of different
    lengths; each step the budget planner splits 12 tokens over the lanes in
    use, the lanes' sequences go through verify -> accept/commit (checked
    against the oracle inside each round), a lane whose request is done is
    refilled from the queue on the next step with a fresh context, and the
    oracle's batching model, fed the same emitted counts, makes the same
    membership decisions."""
    from oracle import batching as OB
    slots, ctx0 = 4, 10
    need = [5, 12, 3, 9, 7, 4, 10]
    m = _Model([ctx0] * slots, seed=2026)
    sch = sv.Scheduler(slots, sv.SV_SCHED_CONTINUOUS)
    for n in need:
        sch.submit(n)
    plan = sv.make_plan_params(sv.SV_PLAN_BUDGET, 6, budget_tokens=12, fill_remainder=True)
    owner = [-1] * slots
    history, emitted_log = [], {}
    r = useful = 0
    while True:
        req, live, width = sch.next()
        if width == 0:
            break
        history.append((req, live, width))
        lanes = [k for k in range(slots) if req[k] >= 0]
        for k in lanes:
            if owner[k] != req[k]:           # refilled: the new request's own context
                owner[k] = req[k]
                m.ctx[k] = ctx0
        st, gl, _ = sv.sv_plan_gamma(plan, len(lanes))
        assert st == sv.SV_OK
        ga, _, _ = m.round(lanes, [int(g) for g in gl], r)
        emitted = [0] * slots
        for n_i, k in enumerate(lanes):
            emitted[k] = int(ga[n_i]) + 1
        emitted_log[r] = emitted
        useful += sch.commit(emitted)
        r += 1
        assert r < 60
    assert useful == sum(need)
    refills = sum(1 for (req, _, _), (req2, _, _) in zip(history, history[1:])
                  for k in range(slots) if req2[k] >= 0 and req2[k] != req[k])
    say(f"continuous batching: {r} steps, {refills} refills, widths {[h[2] for h in history]}")
    assert refills >= len(need) - slots
    want, _ = OB.schedule(OB.CONTINUOUS, slots, need, emitted_fn=lambda st, s, q: emitted_log[st][s])
    assert [(w.slot_request, w.live, w.width) for w in want] == history
