"""GPU parity of the verify pass against the fp64 oracle on sizes that span
several GEMM tiles, K splits and attention chunks with ragged tails, plus the
tiny two-layer model end to end (embedding -> 2 layers -> head -> accept)."""
import numpy as np
import pytest
import torch

from gpu_helpers import (TOL, GpuDecoder, GpuHead, OF, OV, accept_inputs, dev_bf16_to_f64,
                         embed_weights, hidden_states, oracle_accept, rel_rows, run_accept, say,
                         sv, tg)
from workloads import SHAPES, Shape, custom_workload, f32_to_bf16_bits, workload

pytestmark = pytest.mark.gpu

CASES = [
    # (name, shape, wtype, gamma, ctx)
    ("hd128-gqa4-bf16", Shape(512, 8, 2, 128, 1024, 3000), "bf16", [2, 0, 5, 1], [300, 0, 777, 64]),
    ("hd64-gqa1-f32", SHAPES["tiny"], "f32", [4, 0, 2], [128, 5, 260]),
    ("hd128-gqa4-int4", Shape(512, 8, 2, 128, 1024, 3000), "int4", [3, 3, 0], [1000, 17, 513]),
    ("hd128-gqa5-bf16-rows48", Shape(640, 10, 2, 128, 1280, 2000), "bf16", [7, 1], [400, 2]),
    ("hd64-gqa2-bf16-tok>64", Shape(256, 4, 2, 64, 512, 1000), "bf16",
     [6, 0, 3, 9, 2, 4, 1, 8, 5, 7, 3, 0, 6, 2], list(range(10, 150, 10))),
    # 8 query heads per KV head x 8 tokens: 64 query rows (four row tiles)
    ("hd64-gqa8-bf16-rows64", Shape(256, 16, 2, 64, 512, 1000), "bf16", [7, 3, 0], [100, 31, 250]),
]


PACKED_CASES = [(c[0] + "-packed",) + c[1:] for c in CASES if c[2] != "f32"]


@pytest.mark.parametrize("name,shape,wtype,gamma,ctx", CASES + PACKED_CASES,
                         ids=[c[0] for c in CASES + PACKED_CASES])
def test_decoder_parity(name, shape, wtype, gamma, ctx):
    wl = custom_workload(shape, wtype, gamma, ctx, seed=31)
    say(f"decoder {name}: T={wl.T} B={wl.B}")
    dec = GpuDecoder(wl, packed=name.endswith("-packed"))
    xh = hidden_states(wl.T, shape.d, wl.seed)
    y = dec.run(tg.to_dev(xh))
    torch.cuda.synchronize()
    ref = dec.oracle(xh)
    err = rel_rows(dev_bf16_to_f64(y), ref.y)
    say(f"  y rel err {err:.2e}")
    assert err < TOL[wtype]
    assert dec.batch.err.item() == 0
    # appended cache rows (rotated keys, values) at positions ctx_i .. ctx_i + gamma_i
    for i in range(wl.B):
        c, n = int(wl.ctx[i]), int(wl.gamma[i]) + 1
        kg = OF.bf16_to_f64(dec.batch.k_logical(i)[:, c:c + n])
        vg = OF.bf16_to_f64(dec.batch.v_logical(i)[:, c:c + n])
        assert rel_rows(kg.reshape(-1, shape.hd), ref.k_new[i].reshape(-1, shape.hd)) < TOL[wtype]
        assert rel_rows(vg.reshape(-1, shape.hd), ref.v_new[i].reshape(-1, shape.hd)) < TOL[wtype]
        # the cached prefix is untouched
        np.testing.assert_array_equal(dec.batch.k_logical(i)[:, :c], dec.kc[i][:, :c])
        np.testing.assert_array_equal(dec.batch.v_logical(i)[:, :c], dec.vc[i][:, :c])


def test_decoder_deterministic_and_repeatable():
    shape = Shape(512, 8, 2, 128, 1024, 3000)
    wl = custom_workload(shape, "bf16", [3, 1, 0], [500, 20, 0], seed=4)
    dec = GpuDecoder(wl)
    x = tg.to_dev(hidden_states(wl.T, shape.d, wl.seed))
    y1 = dec.run(x).clone()
    y2 = dec.run(x).clone()   # same lengths: rewrites the same cache rows
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_verify_equals_sequential_decodes_gpu():
    """gamma+1 tokens in one pass == gamma+1 single-token passes that commit
    one row each (spec property 1), and gamma = 0 is plain decoding."""
    shape = Shape(256, 4, 2, 64, 512, 1000)
    gam, ctx = [3, 5], [40, 300]
    wl = custom_workload(shape, "bf16", gam, ctx, seed=8)
    xh = hidden_states(wl.T, shape.d, wl.seed)
    full = GpuDecoder(wl)
    yf = dev_bf16_to_f64(full.run(tg.to_dev(xh)))
    seqd = GpuDecoder(wl)     # fresh caches, same contents
    rows = []
    for j in range(max(gam) + 1):
        live = [i for i in range(wl.B) if j <= gam[i]]
        # one token per live sequence, at position ctx_i + j
        b = tg.DeviceBatch([0] * len(live), [ctx[i] + j for i in live], wl.cap)
        b.k = [seqd.batch.k[i] for i in live]
        b.v = [seqd.batch.v[i] for i in live]
        b.kptr = torch.tensor([t.data_ptr() for t in b.k], dtype=torch.int64, device="cuda")
        b.vptr = torch.tensor([t.data_ptr() for t in b.v], dtype=torch.int64, device="cuda")
        b.max_ctx = max(ctx) + max(gam)
        bs = b.struct()
        n = sv.sv_verify_layer_workspace_bytes(seqd.L, bs)
        ws = tg.workspace(n)
        xs = np.stack([xh[int(wl.q_start[i]) + j] for i in live])
        y = torch.empty(len(live), shape.d, dtype=torch.bfloat16, device="cuda")
        assert sv.sv_verify_layer(seqd.L, bs, tg.to_dev(xs), y, 0, ws, n, tg.stream_handle()) == 0
        yh = dev_bf16_to_f64(y)
        for k, i in enumerate(live):
            rows.append((int(wl.q_start[i]) + j, yh[k]))
    for r, v in rows:
        assert rel_rows(v[None], yf[r][None]) < 1e-2, r


@pytest.mark.parametrize("packed", [False, True])
def test_head_parity(packed):
    shape = Shape(512, 8, 2, 128, 1024, 5003)
    for wtype in ("bf16", "int4"):
        wl = custom_workload(shape, wtype, [2, 0, 4], [1, 1, 1], seed=12)
        head = GpuHead(wl, packed=packed)
        yh = hidden_states(wl.T, shape.d, 77)
        yd = tg.to_dev(yh)
        lg = head.run(yd, logits=True).cpu().numpy()
        pr = head.run(yd).cpu().numpy()
        ref = OV.head_logits(head.Wlm, yh)
        err = rel_rows(lg, ref)
        say(f"head {wtype}: logits rel err {err:.2e}")
        assert err < TOL[wtype]
        np.testing.assert_allclose(pr.sum(1), 1.0, rtol=1e-4)
        np.testing.assert_allclose(pr, OV.softmax(lg), rtol=2e-5, atol=1e-9)


@pytest.mark.parametrize("vocab", [5003, 12288])
def test_head_logits_stats_feed_accept(vocab):
    """The head's logits plus per-row (max, sum of exp) fed to acceptance give
    the same accepted counts, next tokens and KV lengths, bit for bit, as the
    head's probabilities; the statistics are the rows' max and sum of exp.
    Vocabularies: odd (scalar loads, two chunks) and a multiple of 4 (vector
    loads, three chunks)."""
    shape = Shape(512, 8, 2, 128, 1024, vocab)
    gamma = [3, 0, 5, 1, 2, 4]
    wl = custom_workload(shape, "bf16", gamma, [1] * len(gamma), seed=21)
    head = GpuHead(wl)
    yh = hidden_states(wl.T, shape.d, 5)
    yd = tg.to_dev(yh)
    T, V = wl.T, vocab
    pr = head.run(yd).cpu().numpy()
    lg = head.run(yd, logits=True).cpu().numpy()
    fused = head.run(yd, flags=sv.SV_HEAD_LOGITS_STATS).cpu().numpy()
    np.testing.assert_array_equal(fused[:T * V].reshape(T, V), lg)
    ms = fused[T * V:].reshape(T, 2)
    np.testing.assert_array_equal(ms[:, 0], lg.max(1))
    ref_s = np.exp(lg.astype(np.float64) - lg.max(1, keepdims=True).astype(np.float64)).sum(1)
    np.testing.assert_allclose(ms[:, 1], ref_s, rtol=1e-5)
    kv = np.full(wl.B, 40, np.int32)
    drows = np.concatenate([np.arange(wl.q_start[i], wl.q_start[i] + gamma[i]) for i in range(wl.B)])
    lens = set()
    for seed in (1, 2, 3):
        for greedy in (False, True):
            inp = accept_inputs(wl, V, target_logits=lg, target_probs=pr, seed=seed)
            if greedy:  # agree with the target's argmax on a seed-dependent prefix
                d = inp["draft"].copy()
                for n, r in enumerate(drows):
                    if (n + seed) % 3:
                        d[n] = int(np.argmax(pr[r]))
                inp["draft"] = d
            mode = sv.SV_ACCEPT_GREEDY if greedy else sv.SV_ACCEPT_STOCHASTIC
            a1, y1, k1, e1 = run_accept(gamma, V, inp, kv, mode)
            a2, y2, k2, e2 = run_accept(gamma, V, dict(inp, p=fused), kv,
                                        mode | sv.SV_ACCEPT_FROM_LOGITS)
            ra, ry, rk, _ = oracle_accept(gamma, inp, kv, greedy=greedy)
            say(f"V={V} seed={seed} greedy={greedy}: accepted {a1.tolist()}")
            for u, w in ((a1, a2), (y1, y2), (k1, k2), (a1, ra), (y1, ry), (k1, rk)):
                np.testing.assert_array_equal(u, w)
            assert e1 == e2 == 0
            lens.update(a1.tolist())
    assert len(lens) >= 3  # the cases reach several accepted lengths


def test_decoder_then_head_shared_workspace():
    """The chain a verify step runs: decoder layer then LM head on one stream,
    sharing one workspace, against the oracle chain."""
    shape = Shape(512, 8, 2, 128, 1024, 4099)
    wl = custom_workload(shape, "bf16", [2, 0, 3], [300, 7, 64], seed=7)
    dec = GpuDecoder(wl)
    head = GpuHead(wl)
    n = max(dec.ws_bytes, head.ws_bytes[sv.SV_HEAD_LOGITS])
    ws = tg.workspace(n)
    xh = hidden_states(wl.T, shape.d, wl.seed)
    x = tg.to_dev(xh)
    y = torch.empty_like(x)
    lg = torch.empty(wl.T, shape.vocab, dtype=torch.float32, device="cuda")
    st = tg.stream_handle()
    assert sv.sv_verify_layer(dec.L, dec.bs, x, y, 0, ws, n, st) == 0
    assert sv.sv_verify_layer(head.L, dec.bs, y, lg, sv.SV_HEAD_LOGITS, ws, n, st) == 0
    torch.cuda.synchronize()
    ref = dec.oracle(xh)
    ey = rel_rows(dev_bf16_to_f64(y), ref.y)
    el = rel_rows(lg.cpu().numpy(), OV.head_logits(head.Wlm, ref.y))
    el_own = rel_rows(lg.cpu().numpy(), OV.head_logits(head.Wlm, dev_bf16_to_f64(y)))
    say(f"chain: y {ey:.2e}  logits {el:.2e}  logits-on-gpu-y {el_own:.2e}")
    assert ey < TOL["bf16"] and el_own < TOL["bf16"] and el < TOL["bf16"]


def _pack_reference(m):
    """Expected packed bytes, by an independent numpy re-layout of [N][K]."""
    n, k = m.n, m.k
    ng = (n + 31) // 32
    if m.wtype == "bf16":
        w = np.zeros((ng * 32, k), np.uint16)
        w[:n] = m.data
        ks = k // 64   # row 32g+16a+l, k = 64s + 32m + 8q + e  ->  [s][g][a][m][q*16+l][e]
        a = w.reshape(ng, 2, 16, ks, 2, 4, 8).transpose(3, 0, 1, 4, 5, 2, 6)
        return a.reshape(-1).view(np.uint8), None
    w = np.zeros((ng * 32, k // 8), np.uint32)
    w[:n] = m.data
    s = np.zeros((ng * 32, k // 32), np.uint16)
    s[:n] = m.scale
    ks = k // 128  # word 16s + 4q + j of row 32g+16a+l -> [s][g][a][q*16+l][j]
    a = w.reshape(ng, 2, 16, ks, 4, 4).transpose(3, 0, 1, 4, 2, 5)
    b = s.reshape(ng, 2, 16, ks, 4).transpose(3, 0, 1, 4, 2)
    return a.reshape(-1).view(np.uint8), b.reshape(-1).view(np.uint8)


@pytest.mark.parametrize("wtype,n,k", [("bf16", 100, 256), ("bf16", 4096, 512), ("int4", 77, 384),
                                       ("int4", 1024, 1024)])
def test_pack_matrix_bit_exact(wtype, n, k):
    from workloads.gen import _matrix, rng_for
    m = _matrix(rng_for(5, f"pack/{wtype}/{n}"), n, k, 0.05, wtype)
    dm = tg.upload_matrix(m, packed=True)
    want_w, want_s = _pack_reference(m)
    np.testing.assert_array_equal(dm.w.cpu().numpy(), want_w)
    if want_s is not None:
        np.testing.assert_array_equal(dm.scale.cpu().numpy()[:want_s.size], want_s)


def test_embed_and_bad_token():
    sh = SHAPES["tiny"]
    E = embed_weights(sh, 3)
    table = tg.to_dev(E)
    L = tg.embed_struct(sh, table)
    b = tg.DeviceBatch([2, 0], [0, 0], 16)
    toks = torch.tensor([5, 1023, 0, 77], dtype=torch.int32, device="cuda")
    out = torch.empty(4, sh.d, dtype=torch.bfloat16, device="cuda")
    assert sv.sv_verify_layer(L, b.struct(), toks, out, 0, None, 0, tg.stream_handle()) == 0
    want = f32_to_bf16_bits(E[[5, 1023, 0, 77]])
    np.testing.assert_array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), want)
    assert b.err.item() == 0
    toks = torch.tensor([5, 1024, 0, -1], dtype=torch.int32, device="cuda")
    assert sv.sv_verify_layer(L, b.struct(), toks, out, 0, None, 0, tg.stream_handle()) == 0
    torch.cuda.synchronize()
    assert b.err.item() & sv.SV_DEV_ERR_BAD_TOKEN
    assert (out[1].float() == 0).all() and (out[3].float() == 0).all()


def test_tiny_model_end_to_end():
    """Workload 1: embedding -> 2 fp32 layers -> head -> accept, against the
    oracle; acceptance is bit-exact when both sides get the GPU's p."""
    wl = workload(1)
    sh = wl.shape
    rng = np.random.default_rng(wl.seed)
    acc_in = accept_inputs(wl, sh.vocab)           # drafts d_j ~ q_j (temperature 0.7)
    x_last = int(rng.integers(0, sh.vocab))
    tokens = np.concatenate([[x_last], acc_in["draft"]]).astype(np.int32)
    E = embed_weights(sh, wl.seed)
    table = tg.to_dev(E)
    b = tg.DeviceBatch(wl.gamma, wl.ctx, wl.cap)
    x = torch.empty(wl.T, sh.d, dtype=torch.bfloat16, device="cuda")
    assert sv.sv_verify_layer(tg.embed_struct(sh, table), b.struct(),
                              torch.tensor(tokens, device="cuda"), x, 0, None, 0,
                              tg.stream_handle()) == 0
    layers = [GpuDecoder(wl, tag=f"layer{k}") for k in range(2)]
    h = x
    for ly in layers:
        h = ly.run(h)
    head = GpuHead(wl)
    lg = head.run(h, logits=True).cpu().numpy()
    p_gpu = head.run(h).cpu().numpy()
    # oracle chain in fp64
    xo = OV.embed(E, tokens)
    for ly in layers:
        xo = ly.oracle(xo).y
    ref = OV.head_logits(head.Wlm, xo)
    err = rel_rows(lg, ref)
    say(f"tiny model logits rel err {err:.2e}")
    assert err < TOL["f32"]
    # acceptance on the GPU's probabilities: bit-exact
    inp = dict(acc_in, p=p_gpu)
    ga, gy, gk, _ = run_accept(wl.gamma, sh.vocab, inp, wl.ctx)
    ra, ry, rk, _ = oracle_accept(wl.gamma, inp, wl.ctx)
    np.testing.assert_array_equal(ga, ra)
    np.testing.assert_array_equal(gy, ry)
    np.testing.assert_array_equal(gk, rk)
    # against the oracle's own probabilities a flip is possible only where
    # u * q(d) sits within the logits tolerance of p(d); report it
    inp_o = dict(acc_in, p=OV.softmax(ref).astype(np.float32))
    oa, oy, _, _ = oracle_accept(wl.gamma, inp_o, wl.ctx)
    say(f"tiny model: accepted gpu={ga.tolist()} oracle-p={oa.tolist()} next {gy.tolist()}/{oy.tolist()}")
    for ly in layers:
        assert ly.batch.err.item() == 0


# Launch settings (splits:depth:waves per unit) covering every GEMM variant:
# waves per unit 1/4/8/16, depth 2/4/8, K splits across units alone and on
# top of in-workgroup splits, uneven split sizes; settings beyond a kernel's
# register budget fall back to smaller ones, which the same comparison covers.
LAUNCH_SETTINGS = [
    None,
    "qkv:1:8:4,o:1:8:4,gu:1:8:4,down:1:8:4",
    "qkv:1:4:8,o:1:8:8,gu:1:8:8,down:2:8:8",
    "qkv:2:4:16,o:1:4:16,gu:1:4:16,down:4:4:16",
    "qkv:4:2:1,o:2:4:1,gu:3:8:1,down:5:2:1",
    "qkv:1:2:0,o:1:2:0,gu:1:2:0,down:1:2:0",   # LDS-tiled kernel (bf16 packed)
    "qkv:1:2:2,o:2:2:2,gu:1:2:2,down:3:2:2",   # wide streaming kernel (bf16 / int4 packed)
    "qkv:1:2:3,o:1:2:3,gu:1:2:3,down:1:2:3",   # square-tiled kernel (bf16 packed)
]


@pytest.mark.parametrize("wtype", ["bf16", "int4", "f32"])
@pytest.mark.parametrize("gamma", [[2, 0, 5, 1, 3, 1, 0, 4], [7, 7, 7, 7, 7, 7, 3, 2]],
                         ids=["T24", "T55"])
def test_decoder_launch_settings(wtype, gamma):
    shape = Shape(2048, 16, 4, 128, 8192, 1000)
    ctx = [300, 0, 777, 64, 1500, 5, 256, 900]
    wl = custom_workload(shape, wtype, gamma, ctx, seed=5)
    dec = GpuDecoder(wl, packed=wtype != "f32")
    xh = hidden_states(wl.T, shape.d, wl.seed)
    x = tg.to_dev(xh)
    ref = dec.oracle(xh)
    try:
        for spec in LAUNCH_SETTINGS:
            assert sv.sv_set_gemm_tuning(spec) == 0
            dec.ws_bytes = sv.sv_verify_layer_workspace_bytes(dec.L, dec.bs)
            dec.ws = tg.workspace(dec.ws_bytes)
            y = dec.run(x)
            torch.cuda.synchronize()
            err = rel_rows(dev_bf16_to_f64(y), ref.y)
            say(f"decoder {wtype} T={wl.T} [{spec}]: y rel err {err:.2e}")
            assert err < TOL[wtype], spec
            assert dec.batch.err.item() == 0
    finally:
        sv.sv_set_gemm_tuning(None)


@pytest.mark.parametrize("wtype", ["bf16", "int4"])
def test_head_launch_settings(wtype):
    shape = Shape(1024, 8, 2, 128, 1024, 20011)
    wl = custom_workload(shape, wtype, [2, 0, 4, 3, 9], [1, 1, 1, 1, 1], seed=13)
    head = GpuHead(wl, packed=True)
    yh = hidden_states(wl.T, shape.d, 78)
    yd = tg.to_dev(yh)
    ref = OV.head_logits(head.Wlm, yh)
    try:
        for spec in (None, "head:1:4:1", "head:1:8:1", "head:1:8:4", "head:2:4:8", "head:3:8:1",
                     "head:1:2:0", "head:3:2:2"):
            assert sv.sv_set_gemm_tuning(spec) == 0
            n = sv.sv_verify_layer_workspace_bytes(head.L, head.bs, sv.SV_HEAD_LOGITS)
            head.ws = tg.workspace(n)
            head.ws_bytes[sv.SV_HEAD_LOGITS] = n
            lg = head.run(yd, logits=True).cpu().numpy()
            err = rel_rows(lg, ref)
            say(f"head {wtype} [{spec}]: logits rel err {err:.2e}")
            assert err < TOL[wtype], spec
    finally:
        sv.sv_set_gemm_tuning(None)


@pytest.mark.parametrize("gamma", [[3, 3, 0, 1], [0, 2, 1], [7, 7, 7, 7, 7, 3, 2], [9, 0, 4, 7, 5, 3]],
                         ids=["T13", "T6", "T45", "T34"])
def test_int4_wide_token_blocks(gamma):
    """The int4 wide kernel at every token-block size (16, 32 and 64 tokens,
    ragged) and with K splits, forced on every GEMM of the decoder layer and
    the head, against the oracle."""
    shape = Shape(2048, 16, 4, 128, 8192, 20011)
    ctx = [int(c) for c in np.linspace(3, 700, len(gamma)).astype(int)]
    wl = custom_workload(shape, "int4", gamma, ctx, seed=23)
    dec = GpuDecoder(wl, packed=True)
    xh = hidden_states(wl.T, shape.d, wl.seed)
    ref = dec.oracle(xh)
    head = GpuHead(wl, packed=True)
    try:
        for spec in ("qkv:1:2:2,o:1:2:2,gu:1:2:2,down:1:2:2,head:1:2:2",
                     "qkv:3:2:2,o:2:2:2,gu:5:2:2,down:7:2:2,head:2:2:2"):
            assert sv.sv_set_gemm_tuning(spec) == 0
            dec.ws_bytes = sv.sv_verify_layer_workspace_bytes(dec.L, dec.bs)
            dec.ws = tg.workspace(dec.ws_bytes)
            y = dec.run(tg.to_dev(xh))
            torch.cuda.synchronize()
            assert dec.batch.err.item() == 0
            err = rel_rows(dev_bf16_to_f64(y), ref.y)
            n = sv.sv_verify_layer_workspace_bytes(head.L, head.bs, sv.SV_HEAD_LOGITS)
            head.ws = tg.workspace(n)
            head.ws_bytes[sv.SV_HEAD_LOGITS] = n
            yh = dev_bf16_to_f64(y)
            lg = head.run(y, logits=True).cpu().numpy()
            errh = rel_rows(lg, OV.head_logits(head.Wlm, yh))
            say(f"int4 wide T={wl.T} [{spec}]: y rel err {err:.2e}, logits {errh:.2e}")
            assert err < TOL["int4"] and errh < TOL["int4"], spec
    finally:
        sv.sv_set_gemm_tuning(None)


@pytest.mark.parametrize("gamma", [[9] * 10, [14] * 10, [15] * 16, [19] * 15], ids=["T100", "T150", "T256", "T300"])
def test_int4_head_default_policy(gamma):
    """The int4 LM head with the default launch policy across its kernel
    changes: the wide kernel with one and with three 128-token blocks, and
    the square-tiled one for 129 to 256 tokens (one 256-token block)."""
    shape = Shape(2048, 16, 4, 128, 8192, 20011)
    wl = custom_workload(shape, "int4", gamma, [5] * len(gamma), seed=29)
    head = GpuHead(wl, packed=True)
    yh = hidden_states(wl.T, shape.d, 81)
    lg = head.run(tg.to_dev(yh), logits=True).cpu().numpy()
    err = rel_rows(lg, OV.head_logits(head.Wlm, yh))
    say(f"int4 head T={wl.T}: logits rel err {err:.2e}")
    assert err < TOL["int4"]


def test_kv_overflow_flagged_and_contained():
    """A sequence whose chunk would run past its cache capacity is flagged on
    the device (SV_DEV_ERR_KV_OVERFLOW): no row at or past the capacity is
    written and the other sequences' results and caches are unaffected."""
    shape = Shape(512, 8, 2, 128, 1024, 3000)
    gamma, ctx, cap = [2, 3, 1], [100, 222, 50], 224   # sequence 1 needs rows 222..225
    wl = custom_workload(shape, "bf16", gamma, ctx, seed=21, cap=cap)
    dec = GpuDecoder(wl)
    sentinel_before = [dec.batch.k_logical(i).copy() for i in range(wl.B)]
    xh = hidden_states(wl.T, shape.d, wl.seed)
    y = dec.run(tg.to_dev(xh))
    torch.cuda.synchronize()
    assert dec.batch.err.item() & sv.SV_DEV_ERR_KV_OVERFLOW
    ref = dec.oracle(xh, seqs=[0, 2])
    yh = dev_bf16_to_f64(y)
    assert rel_rows(yh[ref.rows], ref.y) < TOL["bf16"]
    for i in (0, 2):
        c = int(ctx[i])
        np.testing.assert_array_equal(dec.batch.k_logical(i)[:, :c], sentinel_before[i][:, :c])
        np.testing.assert_array_equal(dec.batch.k_logical(i)[:, c + gamma[i] + 1:],
                                      sentinel_before[i][:, c + gamma[i] + 1:])
    # the overflowing sequence keeps its cached prefix
    np.testing.assert_array_equal(dec.batch.k_logical(1)[:, :222], sentinel_before[1][:, :222])


def test_ctx_bound_flagged_and_contained():
    """A sequence longer than the batch's max_ctx (here by enough that its keys
    would span more than the attention merge's 32 chunks) gets no attention
    work and sets SV_DEV_ERR_CTX_BOUND; every other sequence's rows, and its
    appended K/V, still match the oracle."""
    shape = Shape(512, 8, 2, 128, 1024, 3000)
    B = 40
    gamma = [1] * B
    gamma[1] = 15                       # 64 query rows per KV head: the query-tiled kernel
    gamma[7] = 15
    ctx = [10 + 3 * i for i in range(B)]
    ctx[1] = 13000                      # 51 chunks of 256 keys
    cap = 13024
    wl = custom_workload(shape, "bf16", gamma, ctx, seed=23, cap=cap)
    dec = GpuDecoder(wl, max_ctx=1000)
    xh = hidden_states(wl.T, shape.d, wl.seed)
    y = dec.run(tg.to_dev(xh))
    torch.cuda.synchronize()
    assert dec.batch.err.item() == sv.SV_DEV_ERR_CTX_BOUND
    others = [i for i in range(B) if i != 1]
    ref = dec.oracle(xh, seqs=others)
    yh = dev_bf16_to_f64(y)
    err = rel_rows(yh[ref.rows], ref.y)
    say(f"ctx bound: {len(others)} other sequences, y rel err {err:.2e}")
    assert err < TOL["bf16"]
    for i in (0, 7, B - 1):
        c, n = int(ctx[i]), gamma[i] + 1
        kg = OF.bf16_to_f64(dec.batch.k_logical(i)[:, c:c + n])
        assert rel_rows(kg.reshape(-1, 128), ref.k_new[i].reshape(-1, 128)) < TOL["bf16"]


@pytest.mark.parametrize("tiling", [None, "qkv:1:2:0,o:1:2:0,gu:1:2:0,down:1:2:0,head:1:2:0",
                                    "qkv:2:2:1,o:1:4:1,gu:1:2:1,down:3:4:1,head:1:2:1",
                                    "qkv:1:2:2,o:3:2:2,gu:1:2:2,down:2:2:2,head:2:2:2",
                                    "qkv:1:2:3,o:1:2:3,gu:1:2:3,down:1:2:3,head:1:2:3",
                                    "qkv:3:2:3,o:2:2:3,gu:5:2:3,down:7:2:3,head:2:2:3"])
@pytest.mark.parametrize("wtype", ["bf16", "int4"])
def test_many_tokens_layer_and_head(tiling, wtype):
    """300 stacked tokens (three 128-token blocks of the tiled kernel with a
    ragged tail): decoder layer and head against the oracle, with the default
    policy, with every GEMM tiled,
    with every GEMM streamed one wave per unit (five token blocks, K splits,
    workgroups sharing the token operand), with every GEMM on the wide
    streaming kernel (three 128-token blocks, K splits), and with every GEMM
    on the square-tiled kernel (two 256-token blocks, the second ragged),
    without and with uneven K splits (partial tiles per 128-token block, the
    third block ragged and the fourth empty).  With int4 weights the default
    and wide settings (and the tiled one: the tiled kernel has no int4 form)
    run the int4 wide kernel (codes converted in registers, three 128-token
    blocks, even and uneven K splits), the square launches convert the int4
    codes in LDS, and the one-wave setting keeps the int4 streaming kernel."""
    shape = Shape(2048, 16, 4, 128, 8192, 20011)
    gamma = [14] * 18 + [11, 12, 4]                  # 18*15 + 12 + 13 + 5 = 300 tokens
    ctx = [int(c) for c in np.linspace(0, 300, len(gamma)).astype(int)]
    wl = custom_workload(shape, wtype, gamma, ctx, seed=17)
    assert wl.T == 300
    try:
        assert sv.sv_set_gemm_tuning(tiling) == 0
        dec = GpuDecoder(wl, packed=True)
        xh = hidden_states(wl.T, shape.d, wl.seed)
        y = dec.run(tg.to_dev(xh))
        torch.cuda.synchronize()
        assert dec.batch.err.item() == 0
        seqs = [0, 7, len(gamma) - 2, len(gamma) - 1]
        ref = dec.oracle(xh, seqs=seqs)
        yh = dev_bf16_to_f64(y)
        err = rel_rows(yh[ref.rows], ref.y)
        say(f"many tokens {wtype} [{tiling}]: y rel err {err:.2e}")
        assert err < TOL[wtype]
        head = GpuHead(wl, packed=True)
        lg = head.run(y, logits=True).cpu().numpy()
        rows = [0, 127, 128, 255, 256, 299]
        errh = rel_rows(lg[rows], OV.head_logits(head.Wlm, yh[rows]))
        say(f"  head logits rel err {errh:.2e}")
        assert errh < TOL[wtype]
    finally:
        sv.sv_set_gemm_tuning(None)
