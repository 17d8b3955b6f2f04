"""C-ABI checks that need no GPU: the library loads, exports every function
include/sv.h declares, rejects bad arguments on the host before enqueuing
anything, and its host-only planner agrees with the oracle's."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import verify_pass_amd as sv
from oracle import plan as OP

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "sv.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    decl = _declared()
    assert "sv_verify_layer" in decl and "sv_accept_commit" in decl and "sv_plan_gamma" in decl
    lib = C.CDLL(sv.LIB_PATH)
    for name in decl:
        assert hasattr(lib, name), name
    assert sorted(sv.exported_symbols()) == decl


def test_version_and_status_strings():
    assert sv.sv_version() >= 100
    for st in (sv.SV_OK, sv.SV_ERR_INVALID_ARG, sv.SV_ERR_UNSUPPORTED, sv.SV_ERR_WORKSPACE,
               sv.SV_ERR_HIP):
        assert sv.sv_status_string(st) != "unknown status"
    assert sv.sv_status_string(123) == "unknown status"


def _layer(kind=sv.SV_LAYER_DECODER, wtype=sv.SV_W_BF16, d=256, hq=4, hk=2, hd=64, ffn=512, V=1000):
    L = sv.sv_layer()
    L.kind, L.wtype, L.d, L.n_q_heads, L.n_kv_heads = kind, wtype, d, hq, hk
    L.head_dim, L.ffn, L.vocab, L.eps, L.rope_theta = hd, ffn, V, 1e-6, 1e4
    fake = sv.sv_matrix(0x1000, 0x2000)
    for n in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "embed", "lm_head"):
        setattr(L, n, fake)
    return L


def _batch(gamma, T=None, max_ctx=100, cap=128):
    b = sv.sv_batch()
    b.B = len(gamma)
    b.T = sum(g + 1 for g in gamma) if T is None else T
    b.max_ctx, b.kv_cap = max_ctx, cap
    arr = (C.c_int32 * max(1, len(gamma)))(*gamma)
    b.gamma_host = C.cast(arr, C.POINTER(C.c_int32))
    b._keep = arr
    b.gamma = b.kv_len = b.k_cache = b.v_cache = 0x3000
    b.err_flag = None
    return b


def _ws(L, b, flags=0):
    n = C.c_size_t(0)
    return sv._lib.sv_verify_layer_workspace_bytes(C.byref(L), C.byref(b), flags, C.byref(n)), n.value


def test_workspace_query_valid():
    st, n = _ws(_layer(), _batch([2, 0, 3]))
    assert st == sv.SV_OK and n > 0
    st, n2 = _ws(_layer(kind=sv.SV_LAYER_HEAD), _batch([2, 0, 3]))
    assert st == sv.SV_OK and n2 > 0
    st, n3 = _ws(_layer(kind=sv.SV_LAYER_EMBED, wtype=sv.SV_W_F32), _batch([1]))
    assert st == sv.SV_OK and n3 == 0


@pytest.mark.parametrize("mut,want", [
    (lambda L, b: setattr(b, "T", b.T + 1), sv.SV_ERR_INVALID_ARG),        # T != sum(gamma+1)
    (lambda L, b: setattr(L, "kind", 7), sv.SV_ERR_INVALID_ARG),
    (lambda L, b: setattr(L, "wtype", 9), sv.SV_ERR_UNSUPPORTED),
    (lambda L, b: setattr(L, "head_dim", 96), sv.SV_ERR_UNSUPPORTED),
    (lambda L, b: setattr(L, "n_kv_heads", 3), sv.SV_ERR_UNSUPPORTED),     # 4 % 3
    (lambda L, b: setattr(L, "d", 200), sv.SV_ERR_UNSUPPORTED),            # not a multiple of 64
    (lambda L, b: setattr(b, "kv_cap", 112), sv.SV_ERR_INVALID_ARG),       # not a multiple of 32
    (lambda L, b: setattr(b, "max_ctx", -1), sv.SV_ERR_INVALID_ARG),
    (lambda L, b: setattr(L, "wq", sv.sv_matrix(None, None)), sv.SV_ERR_INVALID_ARG),
    (lambda L, b: setattr(b, "gamma", None), sv.SV_ERR_INVALID_ARG),
])
def test_host_validation(mut, want):
    L, b = _layer(), _batch([2, 0, 3])
    mut(L, b)
    st = sv._lib.sv_verify_layer(C.byref(L), C.byref(b), 0x10, 0x20, 0, 0x30, 1 << 30, None)
    assert st == want


def test_negative_gamma_and_flags_rejected():
    L = _layer()
    st = sv._lib.sv_verify_layer(C.byref(L), C.byref(_batch([1, -1], T=1)), 0x10, 0x20, 0, 0x30,
                                 1 << 30, None)
    assert st == sv.SV_ERR_INVALID_ARG
    st = sv._lib.sv_verify_layer(C.byref(L), C.byref(_batch([1])), 0x10, 0x20, 8, 0x30, 1 << 30, None)
    assert st == sv.SV_ERR_INVALID_ARG
    # the two head output flags exclude each other; each alone is a valid query
    H = _layer(kind=sv.SV_LAYER_HEAD)
    for f in (sv.SV_HEAD_LOGITS, sv.SV_HEAD_LOGITS_STATS):
        assert _ws(H, _batch([2, 0, 3]), f)[0] == sv.SV_OK
    assert _ws(H, _batch([2, 0, 3]), sv.SV_HEAD_LOGITS | sv.SV_HEAD_LOGITS_STATS)[0] == \
        sv.SV_ERR_INVALID_ARG


def test_int4_needs_scales_and_128_multiples():
    L = _layer(wtype=sv.SV_W_INT4_G32, d=192)
    st, _ = _ws(L, _batch([1]))
    assert st == sv.SV_ERR_UNSUPPORTED
    L = _layer(wtype=sv.SV_W_INT4_G32, d=256, ffn=512)
    L.wk = sv.sv_matrix(0x1000, None)
    st, _ = _ws(L, _batch([1]))
    assert st == sv.SV_ERR_INVALID_ARG


def test_gqa_rows_limit():
    # group 2 x (gamma + 1) query rows per KV head must fit 128
    st, _ = _ws(_layer(), _batch([63], max_ctx=10, cap=128))
    assert st == sv.SV_OK
    st, _ = _ws(_layer(), _batch([64], max_ctx=10, cap=128))
    assert st == sv.SV_ERR_UNSUPPORTED


def test_tree_fields_validated():
    b = _batch([3, 5])
    b.tree_parent = 0x4000
    st, _ = _ws(_layer(), b)
    assert st == sv.SV_OK
    b = _batch([63], max_ctx=10, cap=128)    # 64 nodes: the largest tree a mask describes
    b.tree_parent = 0x4000
    assert _ws(_layer(), b)[0] == sv.SV_OK
    b = _batch([64], max_ctx=10, cap=128)
    b.tree_parent = 0x4000
    assert _ws(_layer(hq=2, hk=2), b)[0] == sv.SV_ERR_UNSUPPORTED


def test_workspace_too_small_and_empty_batch():
    L, b = _layer(), _batch([2, 1])
    st, n = _ws(L, b)
    assert st == sv.SV_OK
    st = sv._lib.sv_verify_layer(C.byref(L), C.byref(b), 0x10, 0x20, 0, 0x30, n - 1, None)
    assert st == sv.SV_ERR_WORKSPACE
    st = sv._lib.sv_verify_layer(C.byref(L), C.byref(b), 0x10, 0x20, 0, None, n, None)
    assert st == sv.SV_ERR_WORKSPACE
    # empty batch: nothing to do, nothing enqueued
    st = sv._lib.sv_verify_layer(C.byref(L), C.byref(_batch([])), None, None, 0, None, 0, None)
    assert st == sv.SV_OK


def test_accept_validation():
    g = [2, 0]
    n = sv.sv_accept_commit_workspace_bytes(2, 100, sv.SV_ACCEPT_STOCHASTIC, g)
    assert n > 0
    ga = (C.c_int32 * 2)(*g)
    f = sv._lib.sv_accept_commit
    ok_ptrs = [0x10] * 10
    # bad mode, negative V, negative gamma, missing uniforms, small workspace
    assert f(2, 100, 5, ga, *ok_ptrs, 0x20, n, None) == sv.SV_ERR_INVALID_ARG
    assert f(2, 0, 0, ga, *ok_ptrs, 0x20, n, None) == sv.SV_ERR_INVALID_ARG
    gb = (C.c_int32 * 2)(2, -1)
    assert f(2, 100, 0, gb, *ok_ptrs, 0x20, n, None) == sv.SV_ERR_INVALID_ARG
    ptrs = list(ok_ptrs)
    ptrs[6] = None  # u_samp
    assert f(2, 100, 0, ga, *ptrs, 0x20, n, None) == sv.SV_ERR_INVALID_ARG
    assert f(2, 100, 0, ga, *ok_ptrs, 0x20, n - 1, None) == sv.SV_ERR_WORKSPACE
    assert f(0, 100, 0, ga, *([None] * 10), None, 0, None) == sv.SV_OK
    # greedy needs no q / uniforms
    ng = sv.sv_accept_commit_workspace_bytes(2, 100, sv.SV_ACCEPT_GREEDY, g)
    assert ng > 0
    # the logits flag combines with either mode and changes no workspace size;
    # other high bits are rejected
    for m, size in ((sv.SV_ACCEPT_STOCHASTIC, n), (sv.SV_ACCEPT_GREEDY, ng)):
        assert sv.sv_accept_commit_workspace_bytes(2, 100, m | sv.SV_ACCEPT_FROM_LOGITS, g) == size
    assert f(2, 100, 0x200, ga, *ok_ptrs, 0x20, n, None) == sv.SV_ERR_INVALID_ARG
    assert f(2, 100, sv.SV_ACCEPT_FROM_LOGITS | 2, ga, *ok_ptrs, 0x20, n, None) == sv.SV_ERR_INVALID_ARG


# ---- planner: host logic, against the oracle -------------------------------

def test_plan_budget_matches_oracle():
    for b in range(0, 40):
        for gmax in (0, 3, 8, 64):
            for fill in (True, False):
                p = sv.make_plan_params(sv.SV_PLAN_BUDGET, gmax, budget_tokens=24,
                                        fill_remainder=fill)
                st, g, _ = sv.sv_plan_gamma(p, b)
                assert st == sv.SV_OK
                assert g == OP.plan_budget(b, 24, gmax, fill), (b, gmax, fill)
    # budget derived from the decode floor and per-token compute time
    p = sv.make_plan_params(sv.SV_PLAN_BUDGET, 64, t_floor_ms=1000 / 39.6, c_ms=1000 / 962)
    st, g, _ = sv.sv_plan_gamma(p, 8)
    assert st == sv.SV_OK and g == [2] * 8


def test_plan_speedup_matches_oracle():
    tw, k, c = 20.1, 0.2, 0.109
    dec = OP.decaying_alphas(8)
    for alphas in ([0.8], [0.6], dec):
        for b in (1, 4, 8, 16, 32, 48, 64, 100, 128, 256, 600):
            p = sv.make_plan_params(sv.SV_PLAN_SPEEDUP, 8, t_w_ms=tw, k_ms=k, c_ms=c,
                                    draft_frac=0.04, alpha=alphas)
            st, g, bstar = sv.sv_plan_gamma(p, b)
            want, _, wb = OP.plan_speedup(b, 8, alphas, tw, k, c, 0.04)
            assert st == sv.SV_OK and g == want, (alphas, b)
            assert (bstar == wb) or (np.isinf(bstar) and np.isinf(wb)) or bstar == pytest.approx(wb)


def test_plan_rejects_bad_params():
    p = sv.make_plan_params(sv.SV_PLAN_SPEEDUP, 8, t_w_ms=0.0, c_ms=0.1, alpha=[0.8])
    assert sv.sv_plan_gamma(p, 4)[0] == sv.SV_ERR_INVALID_ARG
    p = sv.make_plan_params(sv.SV_PLAN_SPEEDUP, 8, t_w_ms=1.0, c_ms=0.1, alpha=[1.5])
    assert sv.sv_plan_gamma(p, 4)[0] == sv.SV_ERR_INVALID_ARG
    p = sv.make_plan_params(7, 8)
    assert sv.sv_plan_gamma(p, 4)[0] == sv.SV_ERR_INVALID_ARG
    p = sv.make_plan_params(sv.SV_PLAN_BUDGET, 8)  # no budget and no rates
    assert sv.sv_plan_gamma(p, 4)[0] == sv.SV_ERR_INVALID_ARG


def test_packed_sizes_and_validation():
    assert sv.sv_packed_matrix_bytes(sv.SV_W_BF16, 100, 256) == (128 * 256 * 2, 0)
    assert sv.sv_packed_matrix_bytes(sv.SV_W_INT4_G32, 77, 384) == (96 * 384 // 2, 96 * 12 * 2)
    with pytest.raises(sv.SvError):
        sv.sv_packed_matrix_bytes(sv.SV_W_F32, 16, 64)
    with pytest.raises(sv.SvError):
        sv.sv_packed_matrix_bytes(sv.SV_W_INT4_G32, 16, 64)    # K not a multiple of 128
    assert sv.sv_pack_matrix(sv.SV_W_BF16, 16, 64, None, None, 0x10, None, None) == sv.SV_ERR_INVALID_ARG
    assert sv.sv_pack_matrix(sv.SV_W_INT4_G32, 16, 128, 0x10, None, 0x20, 0x30, None) == \
        sv.SV_ERR_INVALID_ARG
    # an fp32 layer cannot use the packed layout; an unknown layout is rejected
    L = _layer(wtype=sv.SV_W_F32)
    L.layout = sv.SV_LAYOUT_PACKED
    assert _ws(L, _batch([1]))[0] == sv.SV_ERR_UNSUPPORTED
    L = _layer()
    L.layout = 5
    assert _ws(L, _batch([1]))[0] == sv.SV_ERR_INVALID_ARG


def test_gemm_tuning_setter():
    """The launch-policy override parses, changes the plan (workspace size with
    K splits across workgroups) and restores the defaults."""
    L, b = _layer(d=1024, hq=8, hk=2, hd=128, ffn=4096), _batch([2, 0, 3])
    try:
        assert sv.sv_set_gemm_tuning(None) == sv.SV_OK
        st, base = _ws(L, b)
        assert st == sv.SV_OK
        assert sv.sv_set_gemm_tuning("qkv:1:4:1,o:1:4:1,gu:1:4:1,down:1:4:1") == sv.SV_OK
        st, single = _ws(L, b)
        assert st == sv.SV_OK
        assert sv.sv_set_gemm_tuning("down:8:4:1,gu:4:8") == sv.SV_OK
        st, split = _ws(L, b)
        assert st == sv.SV_OK and split > single
        for bad in ("gu:x", "down:-1:4", "qkv:2"):
            assert sv.sv_set_gemm_tuning(bad) == sv.SV_ERR_INVALID_ARG
        assert _ws(L, b)[1] == split          # a rejected spec leaves the setting alone
        assert sv.sv_set_gemm_tuning(None) == sv.SV_OK
        assert _ws(L, b)[1] == base
    finally:
        sv.sv_set_gemm_tuning(None)


def test_trace_arguments():
    """The timing trace rejects a bad class, capacity or stride, and an end
    with no active trace."""
    assert sv.sv_trace_begin(-1, 4) == sv.SV_ERR_INVALID_ARG
    assert sv.sv_trace_begin(sv.SV_K_COUNT, 4) == sv.SV_ERR_INVALID_ARG
    assert sv.sv_trace_begin(sv.SV_K_SOFTMAX, 0) == sv.SV_ERR_INVALID_ARG
    assert sv.sv_trace_begin(sv.SV_K_SOFTMAX, 4, 0) == sv.SV_ERR_INVALID_ARG
    assert sv.sv_trace_end(4)[0] == sv.SV_ERR_INVALID_ARG        # none active


def _oracle_sched_run(policy_name, slots, lengths, emitted_fn):
    from oracle import batching as OB
    return OB.schedule(policy_name, slots, lengths, emitted_fn)


@pytest.mark.parametrize("policy,name", [(sv.SV_SCHED_STATIC, "static"), (sv.SV_SCHED_SHRINK, "shrink"),
                                         (sv.SV_SCHED_CONTINUOUS, "continuous")])
def test_scheduler_matches_oracle(policy, name):
    import numpy as np
    rng = np.random.default_rng(policy + 3)
    for trial in range(5):
        slots = int(rng.integers(1, 9))
        lengths = [int(v) for v in rng.integers(1, 60, size=int(rng.integers(1, 25)))]
        em_table = rng.integers(1, 5, size=(5000, slots))   # tokens a lane emits per step
        emit = (lambda st, s, r: 1) if trial % 2 == 0 else (lambda st, s, r: int(em_table[st, s]))
        want_steps, want_useful = _oracle_sched_run(name, slots, lengths, emit)
        sch = sv.Scheduler(slots, policy)
        assert [sch.submit(n) for n in lengths] == list(range(len(lengths)))
        k = 0
        while True:
            req, live, width = sch.next()
            if width == 0:
                break
            w = want_steps[k]
            assert req == w.slot_request and live == w.live and width == w.width, (trial, k)
            useful = sch.commit([emit(k, s, req[s]) for s in range(slots)])
            assert useful == want_useful[k]
            k += 1
        assert k == len(want_steps)


def test_scheduler_validation():
    with pytest.raises(sv.SvError):
        sv.Scheduler(0, sv.SV_SCHED_STATIC)
    with pytest.raises(sv.SvError):
        sv.Scheduler(4, 7)
    sch = sv.Scheduler(2, sv.SV_SCHED_CONTINUOUS)
    with pytest.raises(sv.SvError):
        sch.submit(0)
    with pytest.raises(sv.SvError):
        sch.commit([1, 1])                   # no step taken
    assert sch.next() == ([-1, -1], [0, 0], 0)


def test_int8_kv_validation():
    b = _batch([3, 1])                       # G = 2: 8 rows per KV head
    b.kv_dtype = sv.SV_KV_INT8
    assert _ws(_layer(), b)[0] == sv.SV_ERR_INVALID_ARG   # scales missing
    b.k_scale = b.v_scale = 0x6000
    assert _ws(_layer(), b)[0] == sv.SV_OK
    b = _batch([8], max_ctx=10)              # 18 rows per KV head: the query-tiled int8 kernel
    b.kv_dtype, b.k_scale, b.v_scale = sv.SV_KV_INT8, 0x6000, 0x6000
    assert _ws(_layer(), b)[0] == sv.SV_OK
    b.kv_dtype = 5
    assert _ws(_layer(), b)[0] == sv.SV_ERR_INVALID_ARG
    b = _batch([64], max_ctx=10)             # 130 rows per KV head: past every attention kernel's 128
    b.kv_dtype, b.k_scale, b.v_scale = sv.SV_KV_INT8, 0x6000, 0x6000
    assert _ws(_layer(), b)[0] == sv.SV_ERR_UNSUPPORTED
