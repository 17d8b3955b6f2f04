"""GPU parity of verification over int8 KV caches (one fp32 scale per cached
vector) against the oracle: layer outputs and the pass's own appended keys
and values (dequantised) on ragged batches with up to 16 query rows per KV
head (the key-split attention kernel) and beyond (the query-tiled kernel),
and at the int4 and 27B-class workloads' full size."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, OF, OV, dev_bf16_to_f64, rel_rows, say, sv, tg
from workloads import (Shape, custom_workload, hidden_states, kv_cache_int8, layer_weights,
                       workload)

pytestmark = pytest.mark.gpu


def _run(wl, packed, seqs=None, max_ctx=None):
    sh = wl.shape
    W = layer_weights(sh, wl.wtype, wl.seed)
    mats = {k: tg.upload_matrix(v, packed=packed) for k, v in W.items()}
    L = tg.decoder_struct(sh, wl.wtype, mats, packed=packed)
    k8, ks, v8, vs = kv_cache_int8(sh, wl.ctx, wl.cap, wl.seed)
    batch = tg.DeviceBatch(wl.gamma, wl.ctx, wl.cap, max_ctx=max_ctx, kcache=k8, vcache=v8,
                           kscale=ks, vscale=vs)
    bs = batch.struct()
    n = sv.sv_verify_layer_workspace_bytes(L, bs)
    ws = tg.workspace(n)
    xh = hidden_states(wl.T, sh.d, wl.seed)
    x = tg.to_dev(xh)
    y = torch.empty_like(x)
    assert sv.sv_verify_layer(L, bs, x, y, 0, ws, n, tg.stream_handle()) == sv.SV_OK
    torch.cuda.synchronize()
    assert batch.err.item() == 0
    ref = OV.decoder_layer(sh, W, xh, wl.gamma, wl.ctx, k8, v8, kscale=ks, vscale=vs, seqs=seqs)
    return batch, y, ref, (k8, ks, v8, vs)


def _check_appended(wl, batch, ref, seqs, wtype):
    hd = wl.shape.hd
    for n_i, i in enumerate(seqs):
        c, n = int(wl.ctx[i]), int(wl.gamma[i]) + 1
        kc = batch.k_logical(i)[:, c:c + n].astype(np.float64)
        vc = batch.v_logical(i)[:, c:c + n].astype(np.float64)
        ksc = batch.ks[i].cpu().numpy()[:, c:c + n].astype(np.float64)
        vsc = batch.vs[i].cpu().numpy()[:, c:c + n].astype(np.float64)
        kd = kc * ksc[..., None]
        vd = vc * vsc[..., None]
        assert rel_rows(kd.reshape(-1, hd), ref.k_new[i].reshape(-1, hd)) < TOL[wtype]
        assert rel_rows(vd.reshape(-1, hd), ref.v_new[i].reshape(-1, hd)) < TOL[wtype]
        assert np.abs(kc).max() == 127 and np.abs(vc).max() == 127


CASES = [
    ("hd128-gqa4-bf16", Shape(512, 8, 2, 128, 1024, 3000), "bf16", [2, 0, 3, 1], [300, 0, 777, 64]),
    ("hd64-gqa2-bf16", Shape(256, 4, 2, 64, 512, 1000), "bf16", [7, 0, 3, 5, 1], [10, 513, 260, 1, 2000]),
    ("hd128-gqa4-int4", Shape(512, 8, 2, 128, 1024, 3000), "int4", [3, 3, 0], [1000, 17, 513]),
    # more than 16 query rows per KV head: the query-tiled kernel (four waves,
    # 40 rows; eight waves, 128 rows), ragged chunks and an empty context
    ("hd128-gqa5-rows40-bf16", Shape(640, 10, 2, 128, 1280, 2000), "bf16", [7, 7, 3, 0], [300, 1000, 64, 0]),
    ("hd64-gqa8-rows128-bf16", Shape(256, 16, 2, 64, 512, 1000), "bf16", [15, 3, 0, 9], [100, 31, 250, 777]),
]


@pytest.mark.parametrize("name,shape,wtype,gamma,ctx", CASES, ids=[c[0] for c in CASES])
def test_int8_kv_decoder_parity(name, shape, wtype, gamma, ctx):
    wl = custom_workload(shape, wtype, gamma, ctx, seed=71)
    batch, y, ref, _ = _run(wl, packed=(wtype == "int4"))
    err = rel_rows(dev_bf16_to_f64(y), ref.y)
    say(f"{name}: int8 KV, y rel err {err:.2e}")
    assert err < TOL[wtype]
    _check_appended(wl, batch, ref, range(wl.B), wtype)


def test_int8_kv_fullsize_int4_workload():
    """The 9B-class int4 workload (B=128, gamma=3, 1024 cached tokens) over
    int8 caches, every row against the oracle."""
    wl = workload(5)
    batch, y, ref, _ = _run(wl, packed=True)
    err = rel_rows(dev_bf16_to_f64(y), ref.y)
    say(f"int4 workload, int8 KV: all {wl.T} rows, y rel err {err:.2e}")
    assert err < TOL["int4"]
    _check_appended(wl, batch, ref, [0, 63, 127], "int4")


def test_int8_kv_fullsize_27b_workload():
    """The 27B-class workload (B=32, gamma=7, 2048 cached tokens: 40 query rows
    per KV head, the query-tiled kernel) over int8 caches, every row against
    the oracle."""
    wl = workload(3)
    batch, y, ref, _ = _run(wl, packed=True)
    err = rel_rows(dev_bf16_to_f64(y), ref.y)
    say(f"27B workload, int8 KV: all {wl.T} rows, y rel err {err:.2e}")
    assert err < TOL["bf16"]
    _check_appended(wl, batch, ref, [0, 15, 31], "bf16")
