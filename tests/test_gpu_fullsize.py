"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (default launch policy, packed weights).

The oracle evaluates every sequence of the batch: every layer output row and
every appended K/V row, then the LM-head logits of every stacked row computed
from the kernel's own layer output (so every row group and token block of the
full-size launches is compared).  Acceptance runs on the kernel's own
probabilities for every sequence and is compared bit for bit.  Properties
that hold at any size (commit arithmetic, 0 <= a <= gamma, probabilities
summing to 1, no device error flags) are checked on every sequence."""
import numpy as np
import pytest
import torch

from gpu_helpers import (TOL, GpuDecoder, GpuHead, OF, OV, accept_inputs, dev_bf16_to_f64,
                         hidden_states, oracle_accept, rel_rows, run_accept, say, sv, tg)
from workloads import workload

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def _sampled(wl):
    return list(range(wl.B))


def _decoder_parity(wl, dec, xh):
    y = dec.run(tg.to_dev(xh))
    torch.cuda.synchronize()
    assert dec.batch.err.item() == 0
    seqs = _sampled(wl)
    ref = dec.oracle(xh, seqs=seqs)
    yh = dev_bf16_to_f64(y)
    err = rel_rows(yh[ref.rows], ref.y)
    say(f"  decoder: {len(seqs)} sequences ({len(ref.rows)} rows) y rel err {err:.2e}")
    assert err < TOL[wl.wtype]
    hd = wl.shape.hd
    for i in seqs:
        c, n = int(wl.ctx[i]), int(wl.gamma[i]) + 1
        kg = OF.bf16_to_f64(dec.batch.k_logical(i)[:, c:c + n])
        vg = OF.bf16_to_f64(dec.batch.v_logical(i)[:, c:c + n])
        assert rel_rows(kg.reshape(-1, hd), ref.k_new[i].reshape(-1, hd)) < TOL[wl.wtype]
        assert rel_rows(vg.reshape(-1, hd), ref.v_new[i].reshape(-1, hd)) < TOL[wl.wtype]
    return y, yh


def _head_parity(wl, head, y, yh):
    lg = head.run(y, logits=True)
    pr = head.run(y)
    torch.cuda.synchronize()
    lg_all = lg.cpu().numpy()
    # every stacked row, in blocks of rows (keeps the fp64 oracle's memory small)
    err = 0.0
    for r0 in range(0, wl.T, 64):
        rows = list(range(r0, min(wl.T, r0 + 64)))
        ref = OV.head_logits(head.Wlm, yh[rows])
        err = max(err, rel_rows(lg_all[rows], ref))
    say(f"  head: all {wl.T} rows logits rel err {err:.2e}")
    assert err < TOL[wl.wtype]
    rows = sorted({0, wl.T // 2, wl.T - 1})
    p_rows = pr[rows].cpu().numpy()
    np.testing.assert_allclose(p_rows, OV.softmax(lg_all[rows]), rtol=2e-5, atol=1e-9)
    sums = pr.sum(dim=1).cpu().numpy()
    np.testing.assert_allclose(sums, 1.0, rtol=1e-4)
    return pr


def _accept_parity(wl, inp, V):
    a, y, k, err = run_accept(wl.gamma, V, inp, wl.ctx)
    ra, ry, rk, rerr = oracle_accept(wl.gamma, inp, wl.ctx)
    np.testing.assert_array_equal(a, ra)
    np.testing.assert_array_equal(y, ry)
    np.testing.assert_array_equal(k, rk)
    assert err == 0 and not rerr.any()
    assert ((a >= 0) & (a <= wl.gamma)).all()
    np.testing.assert_array_equal(k, wl.ctx + a + 1)
    assert ((y >= 0) & (y < V)).all()
    return a


@pytest.mark.parametrize("cid", [2, 3, 5])
def test_fullsize_layer_head_accept(cid):
    wl = workload(cid)
    V = wl.shape.vocab
    say(f"workload {cid} {wl.name}: B={wl.B} T={wl.T} wtype={wl.wtype}")
    dec = GpuDecoder(wl, packed=True)
    xh = hidden_states(wl.T, wl.shape.d, wl.seed)
    y, yh = _decoder_parity(wl, dec, xh)
    del dec
    head = GpuHead(wl, packed=True)
    pr = _head_parity(wl, head, y, yh)
    p_gpu = pr.cpu().numpy()
    del pr, head
    torch.cuda.empty_cache()
    if wl.draft == "alpha":
        inp = accept_inputs(wl, V, alpha=wl.alphas[0], target_probs=p_gpu)
    else:
        inp = accept_inputs(wl, V, target_logits=np.log(np.maximum(p_gpu, 1e-30)))
        inp = dict(inp, p=p_gpu)
    a = _accept_parity(wl, inp, V)
    say(f"  accept: mean accepted {a.mean():.3f} (gamma {wl.gamma.mean():.2f})")


def test_fullsize_ragged_layer_and_accept():
    wl = workload(4)
    V = wl.shape.vocab
    say(f"workload 4 {wl.name}: B={wl.B} T={wl.T} gamma={wl.gamma.tolist()} ctx {wl.ctx.min()}..{wl.ctx.max()}")
    dec = GpuDecoder(wl, packed=True)
    xh = hidden_states(wl.T, wl.shape.d, wl.seed)
    _decoder_parity(wl, dec, xh)
    for alpha in wl.alphas:
        inp = accept_inputs(wl, V, alpha=alpha)
        a = _accept_parity(wl, inp, V)
        say(f"  alpha {alpha}: mean accepted {a.mean():.3f}")
