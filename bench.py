#!/usr/bin/env python3
"""Benchmark of one batched speculative-verification step on one MI355X.

A step is the whole hot path over one batch: plan the draft lengths (host),
the decoder layer over the stacked verify tokens (QKV + RoPE + KV append,
ragged attention, O, SwiGLU FFN), the LM head (logits + row statistics), and
acceptance / resampling / KV-length commit reading the head's logits.  The
headline workload is the largest single-GPU one: a 27B-class bf16 layer,
B=32 sequences with gamma=7 drafts each (256 verify tokens), 2048 cached
tokens, a 151936-entry head, drafts from noisy target logits.  The 9B-class
bf16 layer (B=8, gamma=2) and the 9B-class int4 layer (B=128, gamma=3, 1024
cached tokens) are reported beside it under "workloads".  Inputs are seeded
synthetic data resident in HBM before timing starts.

Prints one JSON line (stdout); progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload N] [--extra 2,5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify tokens/s & accepted tokens/s vs (B,γ); % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_algorithmic(wl, which: str):
    """(bytes, flops) that one launch of a weight GEMM must move / compute:
    weights once, activations in, outputs out."""
    sh = wl.shape
    d, hq, hk, hd, F, V, T = sh.d, sh.n_q, sh.n_kv, sh.hd, sh.ffn, sh.vocab, wl.T
    wbytes = (lambda n, k: n * k * 2) if wl.wtype == "bf16" else (
        (lambda n, k: n * k // 2 + n * (k // 32) * 2) if wl.wtype == "int4" else (lambda n, k: n * k * 4))
    if which == "lm_head":
        n, k, extra = V, d, T * d * 2 + T * V * 4
    elif which == "qkv":
        n, k, extra = (hq + 2 * hk) * hd, d, T * d * 2 + T * (hq + 2 * hk) * hd * 2
    elif which == "o":
        n, k, extra = d, hq * hd, T * hq * hd * 2 + 2 * T * d * 2
    elif which == "gate_up":
        n, k, extra = 2 * F, d, T * d * 2 + T * F * 2
    else:  # down
        n, k, extra = d, F, T * F * 2 + 2 * T * d * 2
    return wbytes(n, k) + extra, 2.0 * T * n * k


def attention_algorithmic(wl, kv8=False):
    """Bytes and flops of the attention: every key and value of every
    sequence once (int8 caches: one byte per value plus an fp32 scale per
    vector), the queries in and the outputs out."""
    sh = wl.shape
    keys = int(sum(int(c) + int(g) + 1 for c, g in zip(wl.ctx, wl.gamma)))
    kv = keys * sh.n_kv * (sh.hd + 4) * 2 if kv8 else keys * sh.n_kv * sh.hd * 2 * 2
    qo = wl.T * sh.n_q * sh.hd * 2 * 2
    pairs = sum((int(g) + 1) * int(c) + (int(g) + 1) * (int(g) + 2) // 2
                for c, g in zip(wl.ctx, wl.gamma))
    return kv + qo, 4.0 * sh.hd * sh.n_q * pairs


def roofline_of(bytes_, flops, ms):
    t = ms * 1e-3
    gbs = bytes_ / t / 1e9
    tfs = flops / t / 1e12
    if bytes_ / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFS * 1e12):
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFS,
            "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}


# Sources of the dominant GEMM kernel: traffic counters taken on another
# version of them no longer describe the kernel that runs.
GEMM_SOURCES = ("verify_pass_amd/csrc/sv_gemm_kernel.h", "verify_pass_amd/csrc/sv_gemm_bf16.hip",
                "verify_pass_amd/csrc/sv_common.h")


def gemm_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(wl, dom_name):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (profiles/<kernel>_traffic_<workload>.md), or None when there is
    none for this workload or the kernel sources changed since."""
    import re
    path = os.path.join(ROOT, "profiles", f"gemm_{dom_name}_traffic_{wl.name}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    fields = dict(re.findall(r"^(source_sha256|fetch_bytes_per_launch|write_bytes_per_launch):\s*(\S+)",
                             txt, flags=re.M))
    if fields.get("source_sha256") != gemm_source_digest():
        return None
    try:
        return int(fields["fetch_bytes_per_launch"]) + int(fields["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, W, Wlm, kc, vc, xh, acc_in, seqs_per_rep, min_seconds=10.0, max_reps=6):
    """The oracle, as it stands, on a bounded sample of the same workload:
    whole verify steps of the first seqs_per_rep sequences (decoder layer,
    LM head + softmax, acceptance), repeated until min_seconds have passed or
    max_reps steps are done."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import accept as OA
    from oracle import verify as OV
    cores = len(os.sched_getaffinity(0))
    S = max(1, min(wl.B, int(seqs_per_rep)))
    seqs = list(range(S))
    qs = wl.q_start
    g = wl.gamma[:S]
    drows = int(np.sum(g))
    with threadpool_limits(limits=cores):
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t0 = time.perf_counter()
        reps = n_tok = 0
        while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_seconds):
            out = OV.decoder_layer(wl.shape, W, xh, wl.gamma, wl.ctx, kc, vc, seqs=seqs)
            if Wlm is not None:
                p = OV.softmax(OV.head_logits(Wlm, out.y)).astype(np.float32)
            else:
                p = acc_in["p"][:qs[S]]
            OA.accept_commit(g, acc_in["draft"][:drows], p, acc_in["q"][:drows],
                             acc_in["u_acc"][:drows], acc_in["u_samp"][:S], wl.ctx[:S])
            n_tok += len(out.rows)
            reps += 1
        dt = time.perf_counter() - t0
    return {"value": round(n_tok / dt, 4), "unit": "verify tokens/s", "cores": int(blas),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{reps} verify step(s) of the first {S} of the workload's {wl.B} sequences "
                      f"({n_tok} verify tokens in all): decoder layer, "
                      f"{'LM head + softmax, ' if Wlm is not None else ''}acceptance; {dt:.1f} s on "
                      f"{blas} BLAS threads ({cores} cores visible)"}


def expected_tokens(alpha: float, gamma: int) -> float:
    """Tokens per verify pass at independent per-draft acceptance alpha
    (accepted drafts plus the bonus token)."""
    return float(gamma + 1) if alpha >= 1.0 else (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def fit_step_model(bs, ts, n):
    """Least-squares fit of t(B) = max(t_w + k B, c B n) (n = gamma + 1 tokens
    per sequence) to measured step times; returns (t_w, k, c)."""
    import numpy as np
    from scipy.optimize import least_squares
    b = np.asarray(bs, float)
    t = np.asarray(ts, float)

    def resid(v):
        tw, k, c = v
        return (np.maximum(tw + k * b, c * b * n) - t) / t
    x0 = [t[0], max(1e-6, (t[min(2, len(t) - 1)] - t[0]) / max(1.0, b[min(2, len(b) - 1)] - b[0])),
          t[-1] / (b[-1] * n)]
    r = least_squares(resid, x0, bounds=([0, 0, 0], [np.inf, np.inf, np.inf]))
    return tuple(float(v) for v in r.x)


def head_modes(args, sv):
    """Head flags and acceptance mode of a step: by default the head writes
    logits plus each row's (max, sum of exp) and acceptance forms the
    probabilities it reads from them (bit-identical to reading materialized
    probabilities); --head-probs materializes the probabilities."""
    if args.head_probs:
        return 0, sv.SV_ACCEPT_STOCHASTIC
    return sv.SV_HEAD_LOGITS_STATS, sv.SV_ACCEPT_STOCHASTIC | sv.SV_ACCEPT_FROM_LOGITS


def sweep(args):
    """Step time over a (B, gamma) grid: one layer of the chosen shape, the
    151936-entry head and acceptance, all on device-generated synthetic data
    (N(0,1) hidden states and KV entries, one-hot drafts); weights as in the
    workloads (N(0, 1/d), packed)."""
    import numpy as np
    import torch

    import verify_pass_amd as sv
    hflags, amode = head_modes(args, sv)
    from verify_pass_amd import torch_glue as tg
    from workloads import SHAPES, head_weights, layer_weights

    torch.cuda.set_device(0)
    sh = SHAPES[args.sweep_shape]
    wt, ctx = args.sweep_wtype, args.sweep_ctx
    blist = [int(v) for v in args.sweep_b.split(",")]
    glist = [int(v) for v in args.sweep_gamma.split(",")]
    seed = 20260
    log(f"sweep: {args.sweep_shape} {wt} ctx {ctx}, B {blist}, gamma {glist}")
    mats = {k: tg.upload_matrix(v, packed=True) for k, v in layer_weights(sh, wt, seed).items()}
    lm = tg.upload_matrix(head_weights(sh, wt, seed), packed=True)
    Ld = tg.decoder_struct(sh, wt, mats, packed=True)
    Lh = tg.head_struct(sh, wt, lm, packed=True)
    V = sh.vocab
    stream = tg.stream_handle()
    gen = torch.Generator(device="cuda").manual_seed(seed)
    rows = []
    for B in blist:
        cap = (ctx + max(glist) + 1 + 31) // 32 * 32
        kcs = [torch.randn(sh.n_kv, cap, sh.hd, device="cuda", generator=gen).to(torch.bfloat16)
               for _ in range(B)]
        vcs = [torch.randn(sh.n_kv, cap // 32, sh.hd, 32, device="cuda", generator=gen).to(torch.bfloat16)
               for _ in range(B)]
        for g in glist:
            T = B * (g + 1)
            batch = tg.DeviceBatch([g] * B, [ctx] * B, cap)
            batch.k, batch.v = kcs, vcs
            batch.kptr = torch.tensor([t.data_ptr() for t in kcs], dtype=torch.int64, device="cuda")
            batch.vptr = torch.tensor([t.data_ptr() for t in vcs], dtype=torch.int64, device="cuda")
            bs = batch.struct()
            nd = sv.sv_verify_layer_workspace_bytes(Ld, bs)
            nh = sv.sv_verify_layer_workspace_bytes(Lh, bs, hflags)
            na = sv.sv_accept_commit_workspace_bytes(B, V, amode, [g] * B)
            ws = tg.workspace(max(nd, nh, na))
            nws = ws.numel()
            x = torch.randn(T, sh.d, device="cuda", generator=gen).to(torch.bfloat16)
            y = torch.empty_like(x)
            probs = torch.empty(T * (V + 2), dtype=torch.float32, device="cuda")
            nd_ = max(1, B * g)
            draft = torch.randint(0, V, (nd_,), device="cuda", generator=gen, dtype=torch.int32)
            q = torch.zeros(nd_, V, device="cuda")
            q[torch.arange(nd_, device="cuda"), draft.long()] = 1.0
            ua = torch.rand(nd_, device="cuda", generator=gen)
            us = torch.rand(B, device="cuda", generator=gen)
            acc = torch.zeros(B, dtype=torch.int32, device="cuda")
            nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
            gl = [g] * B
            n_it = 10 if T <= 512 else 4
            # each step reads and commits its own copy of the starting lengths
            kv_all = batch.kv_len.clone().repeat(3 + n_it, 1).contiguous()
            bss = []
            for k in range(3 + n_it):
                b_ = batch.struct()
                b_.kv_len = kv_all[k].data_ptr()
                bss.append(b_)

            def step(k):
                assert sv.sv_verify_layer(Ld, bss[k], x, y, 0, ws, nws, stream) == 0
                assert sv.sv_verify_layer(Lh, bss[k], y, probs, hflags, ws, nws, stream) == 0
                assert sv.sv_accept_commit(B, V, amode, gl, batch.gamma, draft, probs, q, ua, us,
                                           kv_all[k], acc, nxt, batch.err, ws, nws, stream) == 0
            for k in range(3):
                step(k)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for k in range(n_it):
                step(3 + k)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / n_it
            assert batch.err.item() == 0
            row = {"B": B, "gamma": g, "T": T, "ms": round(ms, 5),
                   "verify_tok_s": round(T / ms * 1e3, 1),
                   "accepted_tok_s_alpha0.8": round(B * expected_tokens(0.8, g) / ms * 1e3, 1)}
            if args.sweep_kernels:
                kt = {}
                for cls, nm in kernel_names(sv, args.head_probs).items():
                    kv_all.copy_(batch.kv_len.expand_as(kv_all))
                    assert sv.sv_trace_begin(cls, n_it) == 0
                    for k in range(n_it):
                        step(3 + k)
                    torch.cuda.synchronize()
                    st_, t_ = sv.sv_trace_end(n_it)
                    if t_:
                        kt[nm] = round(float(sum(t_) / len(t_)), 5)
                row["kernels_ms"] = kt
            rows.append(row)
            log(json.dumps(row))
            del probs, q, ws, x, y
        del kcs, vcs
        torch.cuda.empty_cache()

    fits = {}
    for g in glist:
        pts = sorted((r["B"], r["ms"]) for r in rows if r["gamma"] == g)
        if len(pts) < 3:
            continue
        tw, k, c = fit_step_model([p[0] for p in pts], [p[1] for p in pts], g + 1)
        den = (g + 1) * c - k
        fits[g] = {"t_w_ms": tw, "k_ms": k, "c_ms": c, "bstar_fit": (tw / den) if den > 0 else None}
    base = {r["B"]: r["ms"] for r in rows if r["gamma"] == 0}
    for g in glist:
        first = next((r["B"] for r in sorted(rows, key=lambda r: r["B"])
                      if r["gamma"] == g and r["B"] in base and r["ms"] > 1.1 * base[r["B"]]), None)
        if g in fits:
            fits[g]["first_B_over_1.1x_gamma0"] = first
    # draft lengths the library's planner picks with the fitted model (gamma = 1 fit)
    plan = None
    if 1 in fits:
        f = fits[1]
        pp = sv.make_plan_params(sv.SV_PLAN_SPEEDUP, 8, t_w_ms=f["t_w_ms"], k_ms=f["k_ms"],
                                 c_ms=f["c_ms"], alpha=(0.8,))
        plan = {}
        for B in blist:
            st, gam, bstar = sv.sv_plan_gamma(pp, B)
            plan[B] = {"gamma": gam[0] if gam else None, "bstar": bstar}
    out = {"shape": args.sweep_shape, "wtype": wt, "ctx": ctx, "rows": rows,
           "fits": {str(g): v for g, v in fits.items()}, "planner_gamma_alpha0.8": plan}
    if args.sweep_out:
        with open(args.sweep_out, "w") as fh:
            json.dump(out, fh, indent=1)
    log(json.dumps(out["fits"]))
    print(json.dumps({"sweep": True, "points": len(rows), "fits": out["fits"]}), flush=True)


def kernel_names(sv, head_probs):
    return {sv.SV_K_GEMM_QKV: "gemm_qkv", sv.SV_K_ATTENTION: "attention", sv.SV_K_GEMM_O: "gemm_o",
            sv.SV_K_GEMM_GATE_UP: "gemm_gate_up", sv.SV_K_GEMM_DOWN: "gemm_down",
            sv.SV_K_GEMM_LM_HEAD: "gemm_lm_head",
            sv.SV_K_SOFTMAX: "softmax" if head_probs else "row_stats",
            sv.SV_K_ACCEPT: "accept", sv.SV_K_PREP: "prep"}


def run_workload(cid, args, K, Wm, headline, kv8=False):
    """Times K steps of workload cid after Wm warm-ups; returns the result
    dict (and, for the headline workload, the oracle baseline).  kv8: the
    same workload over int8 KV caches."""
    import numpy as np
    import torch

    import verify_pass_amd as sv
    from verify_pass_amd import torch_glue as tg
    from workloads import (accept_inputs, head_weights, hidden_states, kv_cache, kv_cache_int8,
                           layer_weights, rng_for, uniforms_2m24, workload)

    hflags, amode = head_modes(args, sv)
    wl = workload(cid)
    if kv8:
        wl.name = wl.name + "-kv8"
    sh = wl.shape
    log(f"workload {wl.cid} {wl.name}: B={wl.B} T={wl.T} wtype={wl.wtype}")

    t0 = time.perf_counter()
    W = layer_weights(sh, wl.wtype, wl.seed)
    Wlm = head_weights(sh, wl.wtype, wl.seed) if wl.head else None
    if kv8:
        k8, ks8, v8, vs8 = kv_cache_int8(sh, wl.ctx, wl.cap, wl.seed)
        kc, vc = k8, v8
    else:
        kc, vc = kv_cache(sh, wl.ctx, wl.cap, wl.seed)
    xh = hidden_states(wl.T, sh.d, wl.seed)
    log(f"generated inputs in {time.perf_counter() - t0:.1f} s")

    packed = wl.wtype != "f32"
    mats = {k: tg.upload_matrix(v, packed=packed) for k, v in W.items()}
    lm = tg.upload_matrix(Wlm, packed=packed) if Wlm is not None else None
    if kv8:
        batch = tg.DeviceBatch(wl.gamma, wl.ctx, wl.cap, kcache=kc, vcache=vc, kscale=ks8, vscale=vs8)
    else:
        batch = tg.DeviceBatch(wl.gamma, wl.ctx, wl.cap, kcache=kc, vcache=vc)
    bs = batch.struct()
    Ld = tg.decoder_struct(sh, wl.wtype, mats, packed=packed)
    nd = sv.sv_verify_layer_workspace_bytes(Ld, bs)
    ws_d = tg.workspace(nd)
    x = tg.to_dev(xh)
    y = torch.empty_like(x)
    V = sh.vocab
    stream = tg.stream_handle()
    if lm is not None:
        Lh = tg.head_struct(sh, wl.wtype, lm, packed=packed)
        nh = sv.sv_verify_layer_workspace_bytes(Lh, bs, hflags)
        nhl = sv.sv_verify_layer_workspace_bytes(Lh, bs, sv.SV_HEAD_LOGITS)
        ws_h = tg.workspace(max(nh, nhl))
        probs = torch.empty(wl.T * (V + 2), dtype=torch.float32, device="cuda")

    # draft rows / target rows for acceptance, built once from the model's own outputs
    if lm is not None:
        assert sv.sv_verify_layer(Ld, bs, x, y, 0, ws_d, nd, stream) == 0
        logits = torch.empty(wl.T, V, dtype=torch.float32, device="cuda")
        assert sv.sv_verify_layer(Lh, bs, y, logits, sv.SV_HEAD_LOGITS, ws_h, nhl, stream) == 0
        torch.cuda.synchronize()
        if wl.draft == "alpha":
            pm = torch.softmax(logits, 1).cpu().numpy()
            acc_in = accept_inputs(wl, V, alpha=wl.alphas[0], target_probs=pm)
        else:
            acc_in = accept_inputs(wl, V, target_logits=logits.cpu().numpy())
        del logits
    else:
        acc_in = accept_inputs(wl, V, alpha=wl.alphas[0] if wl.alphas else None)
    # the acceptance-rate construction fixes the target rows themselves (not
    # the head's output), so those workloads accept from staged probabilities
    p_alpha = tg.to_dev(acc_in["p"]) if (wl.draft == "alpha" or lm is None) else None
    draft = tg.to_dev(acc_in["draft"]) if wl.n_draft else torch.zeros(1, dtype=torch.int32, device="cuda")
    q = tg.to_dev(acc_in["q"]) if wl.n_draft else torch.zeros(1, V, device="cuda")
    nsteps = K + Wm
    ua = torch.stack([tg.to_dev(uniforms_2m24(rng_for(wl.seed, f"bench/ua{k}"), max(1, wl.n_draft)))
                      for k in range(nsteps)])
    us = torch.stack([tg.to_dev(uniforms_2m24(rng_for(wl.seed, f"bench/us{k}"), wl.B))
                      for k in range(nsteps)])
    acc_all = torch.zeros(nsteps, wl.B, dtype=torch.int32, device="cuda")
    nxt_all = torch.zeros(nsteps, wl.B, dtype=torch.int32, device="cuda")
    kv0 = batch.kv_len.clone()
    # every step verifies the same state: step k reads and commits its own
    # copy of the starting KV lengths (no restore inside the timed region)
    kv_all = kv0.repeat(nsteps, 1).contiguous()
    p_mode = sv.SV_ACCEPT_STOCHASTIC if p_alpha is not None else amode
    na = sv.sv_accept_commit_workspace_bytes(wl.B, V, p_mode, list(wl.gamma))
    ws_a = tg.workspace(na)

    # Draft lengths: the planner splits the step's verify-token budget (the
    # workload's T) over the live batch; each step's lengths go to the device
    # through their own pinned slot.  A workload whose lengths the split does
    # not reproduce (the ragged batch) keeps its own.
    plan = sv.make_plan_params(sv.SV_PLAN_BUDGET, 64, budget_tokens=wl.T)
    st, gplan, _ = sv.sv_plan_gamma(plan, wl.B)
    plan_drives = st == 0 and gplan == [int(g) for g in wl.gamma]
    g_pin = torch.tensor([int(g) for g in wl.gamma] * nsteps, dtype=torch.int32).reshape(
        nsteps, max(1, wl.B)).pin_memory()
    g_dev = torch.empty_like(g_pin, device="cuda")
    bss = []
    for k in range(nsteps):
        b_ = batch.struct()
        b_.kv_len = kv_all[k].data_ptr()
        if plan_drives:
            b_.gamma = g_dev[k].data_ptr()
        bss.append(b_)
    glist = [int(g) for g in wl.gamma]
    gh = [None] * nsteps  # host copies of each step's planned lengths (kept alive)

    def step(k):
        if plan_drives:
            st_, gam, _ = sv.sv_plan_gamma(plan, wl.B)     # host: lengths for the live batch
            assert st_ == 0 and len(gam) == wl.B
            g_pin[k] = torch.as_tensor(gam, dtype=torch.int32)
            g_dev[k].copy_(g_pin[k], non_blocking=True)
            gh[k] = (ctypes.c_int32 * wl.B)(*gam)
            bss[k].gamma_host = ctypes.cast(gh[k], ctypes.POINTER(ctypes.c_int32))
            gl = gam
        else:
            gl = glist
        assert sv.sv_verify_layer(Ld, bss[k], x, y, 0, ws_d, nd, stream) == 0
        if lm is not None:
            assert sv.sv_verify_layer(Lh, bss[k], y, probs, hflags, ws_h, nh, stream) == 0
        p_acc = p_alpha if p_alpha is not None else probs
        assert sv.sv_accept_commit(wl.B, V, p_mode, gl, bss[k].gamma, draft, p_acc, q, ua[k],
                                   us[k], kv_all[k], acc_all[k], nxt_all[k], batch.err, ws_a, na,
                                   stream) == 0

    if headline and args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
            torch.cuda.synchronize()
        log(f"copy probe: 3 x {n} bytes device to device")
        del src, dst

    for k in range(Wm):
        step(k)
    torch.cuda.synchronize()
    dominant = sv.SV_K_GEMM_LM_HEAD if lm is not None else sv.SV_K_GEMM_GATE_UP
    # every 4th launch of the dominant kernel in the timed region is bracketed
    # by HIP events (each record costs a few microseconds of stream time)
    stride = 4
    ntr = (K + stride - 1) // stride
    assert sv.sv_trace_begin(dominant, ntr, stride) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for k in range(Wm, Wm + K):
        step(k)
    e1.record()
    torch.cuda.synchronize()
    st, kms = sv.sv_trace_end(ntr)
    assert st == 0 and len(kms) == ntr, (st, len(kms))
    ms = e0.elapsed_time(e1) / K
    assert batch.err.item() == 0, f"device error flags {batch.err.item()}"
    acc_np = acc_all[Wm:].cpu().numpy()
    tokens_per_step = float((acc_np + 1).sum(axis=1).mean())
    verify_tok_s = wl.T / (ms * 1e-3)
    accepted_tok_s = tokens_per_step / (ms * 1e-3)
    log(f"step {ms:.4f} ms  verify {verify_tok_s:.1f} tok/s  accepted {accepted_tok_s:.1f} tok/s")

    dom_name = "lm_head" if lm is not None else "gate_up"
    dbytes, dflops = gemm_algorithmic(wl, dom_name)
    dms = float(np.mean(kms))
    roof = roofline_of(dbytes, dflops, dms)
    roof.update({"kernel": f"gemm_{dom_name}", "avg_ms": round(dms, 5),
                 "algorithmic_bytes": int(dbytes), "algorithmic_flops": dflops,
                 "traffic": measured_traffic(wl, dom_name)})

    # whole-step roofline: all algorithmic bytes / flops of the step
    tot_b, tot_f = 0, 0.0
    for w_ in ("qkv", "o", "gate_up", "down") + (("lm_head",) if lm is not None else ()):
        b_, f_ = gemm_algorithmic(wl, w_)
        tot_b += b_
        tot_f += f_
    ab, af = attention_algorithmic(wl, kv8)
    tot_b += ab
    tot_f += af
    step_roof = roofline_of(tot_b, tot_f, ms)
    step_roof.update({"algorithmic_bytes": int(tot_b), "algorithmic_flops": tot_f})

    kernels = {}
    if not args.no_kernel_table:
        for cls, nm in kernel_names(sv, args.head_probs).items():
            n = 10
            kv_all.copy_(kv0.expand_as(kv_all))   # the starting lengths again
            assert sv.sv_trace_begin(cls, n) == 0
            for k in range(n):
                step(k % nsteps)
            torch.cuda.synchronize()
            st, t = sv.sv_trace_end(n)
            if t:
                entry = {"avg_ms": round(float(np.mean(t)), 5)}
                gname = nm[5:] if nm.startswith("gemm_") else None
                if gname:
                    b_, f_ = gemm_algorithmic(wl, gname)
                    entry.update({k2: v for k2, v in roofline_of(b_, f_, entry["avg_ms"]).items()
                                  if k2 in ("bound", "achieved", "unit", "frac")})
                elif nm == "attention":
                    entry.update({k2: v for k2, v in roofline_of(ab, af, entry["avg_ms"]).items()
                                  if k2 in ("bound", "achieved", "unit", "frac")})
                kernels[nm] = entry
        log("kernels: " + json.dumps(kernels))

    has_head = lm is not None
    cpu = None
    if headline and not args.no_cpu_baseline:
        log("timing the oracle on the host (bounded sample)...")
        del mats, lm, ws_d, x, y
        torch.cuda.empty_cache()
        per_rep = max(1, args.cpu_tokens // max(1, int(wl.gamma[0]) + 1))
        cpu = cpu_baseline(wl, W, Wlm, kc, vc, xh, acc_in, per_rep)
        log(f"oracle: {cpu}")

    res = {
        "ms_per_step": round(ms, 5), "verify_tok_s": round(verify_tok_s, 2),
        "accepted_tok_s": round(accepted_tok_s, 2), "tokens_per_step": round(tokens_per_step, 3),
        "config": {"workload": wl.name, "B": wl.B,
                   "gamma": glist if wl.B <= 16 else int(wl.gamma[0]), "T": wl.T,
                   "ctx": int(wl.ctx[0]) if len(set(wl.ctx.tolist())) == 1 else "ragged",
                   "weights": wl.wtype + (" packed" if packed else ""), "d": sh.d,
                   "kv_cache": "int8 + fp32 scale per vector" if kv8 else "bf16",
                   "heads": f"{sh.n_q}q/{sh.n_kv}kv x {sh.hd}", "ffn": sh.ffn,
                   "vocab": V if has_head else None,
                   "acceptance": (wl.alphas[0] if wl.alphas else wl.draft),
                   "head_output": "probabilities" if args.head_probs else "logits+row stats",
                   "accept_reads": ("staged target probabilities (acceptance-rate construction)"
                                    if p_alpha is not None else
                                    ("the head's probabilities" if args.head_probs else
                                     "the head's logits + row stats")),
                   "gamma_source": "sv_plan_gamma (budget = T tokens), copied to the device each step"
                                   if plan_drives else "the workload's own draft lengths"},
        "roofline": roof, "step_roofline": step_roof, "kernels": kernels,
    }
    return res, cpu, wl


SWARM_LENGTHS = (40, 90, 150, 220, 300, 480, 650, 900)


def tree_shape(depth: int) -> list:
    """Parent array (topological order) of the measured token tree: a chain of
    `depth` drafts with one alternative child at each of its first depth - 1
    levels (2 * depth nodes with the root, e.g. 16 nodes 8 deep)."""
    par = [-1]
    for d in range(1, depth + 1):
        up = 0 if d == 1 else 2 * d - 3   # the chain node one level up
        par.append(up)                    # chain node at depth d: index 2d - 1
        if d < depth:
            par.append(up)                # its sibling: index 2d
    return par


def tree_bench(args):
    """Token-tree verification ([slack], "What the budget says to build": a
    small tree, about 8 to 16 deep) against linear drafts at the same depth
    and at the same number of verified rows: step time (decoder layer with
    ancestor masks, head logits and row statistics, tree acceptance from them
    and the commit's row moves, or linear acceptance and commit) and the tokens a step emits per
    sequence, on synthetic data: device-generated N(0,1) hidden states and
    KV entries, draft rows q = 0.7 p + 0.3 r (p the pass's own target row,
    r a random softmax row), each draft drawn from its parent's q row; every
    acceptance call gets fresh drafts and uniforms, and tokens per step are
    averaged over the timed calls and --tree-stat-calls untimed ones."""
    import numpy as np
    import torch

    import verify_pass_amd as sv
    from verify_pass_amd import torch_glue as tg
    from workloads import SHAPES, head_weights, layer_weights

    torch.cuda.set_device(0)
    sh = SHAPES[args.tree_shape_name]
    ctx, depth = args.tree_ctx, args.tree_depth
    blist = [int(v) for v in args.tree_b.split(",")]
    seed = 20261
    rng = np.random.default_rng(seed)
    mats = {k: tg.upload_matrix(v, packed=True) for k, v in layer_weights(sh, "bf16", seed).items()}
    lm = tg.upload_matrix(head_weights(sh, "bf16", seed), packed=True)
    Ld = tg.decoder_struct(sh, "bf16", mats, packed=True)
    Lh = tg.head_struct(sh, "bf16", lm, packed=True)
    V = sh.vocab
    stream = tg.stream_handle()
    gen = torch.Generator(device="cuda").manual_seed(seed)
    tpar = tree_shape(depth)
    variants = [("tree", len(tpar) - 1), ("chain-depth", depth), ("chain-rows", len(tpar) - 1)]
    amode = sv.SV_ACCEPT_STOCHASTIC | sv.SV_ACCEPT_FROM_LOGITS
    n_it, n_stat, rows = 10, args.tree_stat_calls, []
    log(f"tree: {args.tree_shape_name} bf16 ctx {ctx}, tree of {len(tpar)} nodes {depth} deep, B {blist}")

    def draw_rows(qrows, src, out, skip=None):
        """out[k, t] ~ qrows[src[t]] for every set k (independent draws by the
        inverse CDF of each row), t with skip[t] left alone."""
        for r in np.unique(src):
            ts = [t for t in np.nonzero(src == r)[0] if skip is None or not skip[t]]
            if not ts:
                continue
            c = np.cumsum(qrows[r].astype(np.float64))
            c /= c[-1]
            u = rng.random((out.shape[0], len(ts)))
            out[:, ts] = np.minimum(np.searchsorted(c, u, side="right"), V - 1)

    def rand_rows(n):
        z = rng.standard_normal((n, V)).astype(np.float32) * 3.0
        z -= z.max(1, keepdims=True)
        e = np.exp(z)
        return e / e.sum(1, keepdims=True)

    for B in blist:
        cap = (ctx + len(tpar) + 31) // 32 * 32
        kcs = [torch.randn(sh.n_kv, cap, sh.hd, device="cuda", generator=gen).to(torch.bfloat16)
               for _ in range(B)]
        vcs = [torch.randn(sh.n_kv, cap // 32, sh.hd, 32, device="cuda", generator=gen).to(torch.bfloat16)
               for _ in range(B)]
        for name, g in variants:
            tree = name == "tree"
            T = B * (g + 1)
            batch = tg.DeviceBatch([g] * B, [ctx] * B, cap, tree_parents=[tpar] * B if tree else None)
            batch.k, batch.v = kcs, vcs
            batch.kptr = torch.tensor([t.data_ptr() for t in kcs], dtype=torch.int64, device="cuda")
            batch.vptr = torch.tensor([t.data_ptr() for t in vcs], dtype=torch.int64, device="cuda")
            gl = [g] * B
            nd = sv.sv_verify_layer_workspace_bytes(Ld, batch.struct())
            nh = max(sv.sv_verify_layer_workspace_bytes(Lh, batch.struct(), f)
                     for f in (0, sv.SV_HEAD_LOGITS_STATS))
            na = (sv.sv_accept_tree_workspace_bytes(B, V, gl) if tree
                  else sv.sv_accept_commit_workspace_bytes(B, V, amode, gl))
            ws = tg.workspace(max(nd, nh, na))
            nws = ws.numel()
            x = torch.randn(T, sh.d, device="cuda", generator=gen).to(torch.bfloat16)
            y = torch.empty_like(x)
            # the head's logits and row statistics (acceptance forms the probabilities)
            logits = torch.empty(T * (V + 2), dtype=torch.float32, device="cuda")
            kv_all = batch.kv_len.clone().repeat(3 + n_it + n_stat, 1).contiguous()
            bss = []
            for k in range(3 + n_it):
                b_ = batch.struct()
                b_.kv_len = kv_all[k].data_ptr()
                bss.append(b_)
            # the pass's target rows, then drafts from q rows close to them
            probs = torch.empty(T, V, dtype=torch.float32, device="cuda")
            assert sv.sv_verify_layer(Ld, bss[0], x, y, 0, ws, nws, stream) == 0
            assert sv.sv_verify_layer(Lh, bss[0], y, probs, 0, ws, nws, stream) == 0
            torch.cuda.synchronize()
            assert batch.err.item() == 0
            p_h = probs.cpu().numpy()
            del probs
            # a fresh set of drafts for every call: warm-up, timed, then statistics only
            n_sets = 3 + n_it + n_stat
            if tree:
                q_h = (0.7 * p_h + 0.3 * rand_rows(T)).astype(np.float32)
                src = np.array([i * (g + 1) + (tpar[j] if j else 0) for i in range(B) for j in range(g + 1)])
                tok = np.zeros((n_sets, T), np.int32)
                draw_rows(q_h, src, tok, skip=np.arange(T) % (g + 1) == 0)
                q = torch.as_tensor(q_h, device="cuda")
                tokens = torch.as_tensor(tok, device="cuda")
                path = torch.zeros(B, 64, dtype=torch.int32, device="cuda")
                ua = torch.rand(n_sets, T, device="cuda", generator=gen)
            else:
                rows_q = np.concatenate([np.arange(i * (g + 1), i * (g + 1) + g) for i in range(B)])
                q_h = (0.7 * p_h[rows_q] + 0.3 * rand_rows(B * g)).astype(np.float32)
                drafts = np.zeros((n_sets, B * g), np.int32)
                draw_rows(q_h, np.arange(B * g), drafts)
                q = torch.as_tensor(q_h, device="cuda")
                draft = torch.as_tensor(drafts, device="cuda")
                ua = torch.rand(n_sets, max(1, B * g), device="cuda", generator=gen)
            us = torch.rand(n_sets, B, device="cuda", generator=gen)
            acc_all = torch.zeros(n_sets, B, dtype=torch.int32, device="cuda")
            nxt = torch.zeros(B, dtype=torch.int32, device="cuda")

            def accept(k):
                if tree:
                    assert sv.sv_accept_tree(B, V, amode, gl, batch.tree_parent, tokens[k], logits,
                                             q, ua[k], us[k], kv_all[k], acc_all[k], nxt, path, batch.err, ws,
                                             nws, stream) == 0
                    assert sv.sv_tree_commit_kv(B, sh.n_kv, sh.hd, cap, kv_all[k], acc_all[k], path,
                                                batch.kptr, batch.vptr, stream) == 0
                else:
                    assert sv.sv_accept_commit(B, V, amode, gl, batch.gamma, draft[k], logits, q,
                                               ua[k], us[k], kv_all[k], acc_all[k], nxt, batch.err, ws, nws,
                                               stream) == 0

            def step(k):
                assert sv.sv_verify_layer(Ld, bss[k], x, y, 0, ws, nws, stream) == 0
                assert sv.sv_verify_layer(Lh, bss[k], y, logits, sv.SV_HEAD_LOGITS_STATS, ws, nws, stream) == 0
                accept(k)

            kv_all.copy_(batch.kv_len.expand_as(kv_all))
            for k in range(3):
                step(k)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for k in range(n_it):
                step(3 + k)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / n_it
            assert batch.err.item() == 0
            # tokens per sequence-step over the timed calls and n_stat more, each
            # with its own drafts and uniforms
            for k in range(3 + n_it, n_sets):
                accept(k)
            torch.cuda.synchronize()
            assert batch.err.item() == 0
            emitted = float((acc_all[3:].float() + 1).mean().item())
            # acceptance (and commit) alone, on the same inputs
            kv_all.copy_(batch.kv_len.expand_as(kv_all))
            torch.cuda.synchronize()
            e0.record()
            for k in range(n_it):
                accept(3 + k)
            e1.record()
            torch.cuda.synchronize()
            acc_ms = e0.elapsed_time(e1) / n_it
            row = {"B": B, "variant": name, "rows_per_seq": g + 1, "T": T, "ms": round(ms, 5),
                   "accept_ms": round(acc_ms, 5), "tokens_per_seq_step": round(emitted, 3),
                   "verify_tok_s": round(T / ms * 1e3, 1), "emitted_tok_s": round(B * emitted / ms * 1e3, 1)}
            rows.append(row)
            log(json.dumps(row))
            del logits, q, ws, x, y
        del kcs, vcs
        torch.cuda.empty_cache()
    out = {"tree": True, "shape": args.tree_shape_name, "ctx": ctx, "depth": depth, "parents": tpar,
           "rows": rows}
    if args.tree_out:
        with open(args.tree_out, "w") as fh:
            json.dump(out, fh, indent=1)
    print(json.dumps({"tree": True, "points": len(rows)}), flush=True)


def swarm(args):
    """The static-batching page's eight-agent swarm (output lengths 40..900
    tokens, plain decoding: one token per live sequence per step) through the
    real verify path -- the 9B-class bf16 layer, the 151936-entry head and
    acceptance -- under each policy of the library's scheduler, with the
    requests resubmitted `--swarm-waves` times so that continuous batching
    has a queue to refill from.  Also measures the plain decode step t(B) at
    B = 1..8 and fits t(B) = t0 + t1 B, from which the oracle's batching
    model predicts each policy's throughput."""
    import numpy as np
    import torch

    import verify_pass_amd as sv
    from oracle import batching as OB
    from verify_pass_amd import torch_glue as tg
    from workloads import SHAPES, head_weights, layer_weights

    torch.cuda.set_device(0)
    sh = SHAPES["9b"]
    slots, ctx0 = 8, args.swarm_ctx
    lengths = list(SWARM_LENGTHS) * args.swarm_waves
    cap = (ctx0 + max(SWARM_LENGTHS) + 1 + 31) // 32 * 32
    seed = 20262
    mats = {k: tg.upload_matrix(v, packed=True) for k, v in layer_weights(sh, "bf16", seed).items()}
    lm = tg.upload_matrix(head_weights(sh, "bf16", seed), packed=True)
    Ld = tg.decoder_struct(sh, "bf16", mats, packed=True)
    Lh = tg.head_struct(sh, "bf16", lm, packed=True)
    gen = torch.Generator(device="cuda").manual_seed(seed)
    kcs = [torch.randn(sh.n_kv, cap, sh.hd, device="cuda", generator=gen).to(torch.bfloat16) for _ in range(slots)]
    vcs = [torch.randn(sh.n_kv, cap // 32, sh.hd, 32, device="cuda", generator=gen).to(torch.bfloat16)
           for _ in range(slots)]
    kp = [t.data_ptr() for t in kcs]
    vp = [t.data_ptr() for t in vcs]
    V = sh.vocab
    stream = tg.stream_handle()
    x_all = torch.randn(slots, sh.d, device="cuda", generator=gen).to(torch.bfloat16)
    y = torch.empty_like(x_all)
    probs = torch.empty(slots * (V + 2), dtype=torch.float32, device="cuda")
    us = torch.rand(slots, device="cuda", generator=gen)
    acc = torch.zeros(slots, dtype=torch.int32, device="cuda")
    nxt = torch.zeros(slots, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    zeros = torch.zeros(slots, dtype=torch.int32, device="cuda")
    amode = sv.SV_ACCEPT_STOCHASTIC | sv.SV_ACCEPT_FROM_LOGITS
    # per batch width: pointer tables and a workspace (built once)
    nmax = 0
    tables = {}
    for w in range(1, slots + 1):
        b = tg.DeviceBatch([0] * w, [ctx0] * w, cap, max_ctx=ctx0 + max(SWARM_LENGTHS))
        nmax = max(nmax, sv.sv_verify_layer_workspace_bytes(Ld, b.struct()),
                   sv.sv_verify_layer_workspace_bytes(Lh, b.struct(), sv.SV_HEAD_LOGITS_STATS),
                   sv.sv_accept_commit_workspace_bytes(w, V, amode, [0] * w))
        tables[w] = b
    ws = tg.workspace(nmax)
    # one pinned slot per step of the whole run (the host may run far ahead of
    # the device; a slot is never rewritten before its copy has executed)
    nring = 184 + 3 * len(lengths) * max(SWARM_LENGTHS) + 64
    kv_pin = torch.zeros(nring, slots, dtype=torch.int32).pin_memory()
    kv_dev = torch.zeros(nring, slots, dtype=torch.int32, device="cuda")
    ptr_pin = torch.zeros(nring, 2, slots, dtype=torch.int64).pin_memory()
    ptr_dev = torch.zeros(nring, 2, slots, dtype=torch.int64, device="cuda")

    def step(ring, lanes, kv_host):
        """One plain decode step over the given lanes (their caches and lengths)."""
        w = len(lanes)
        r = ring
        assert r < nring
        kv_pin[r, :w] = torch.as_tensor([kv_host[k] for k in lanes], dtype=torch.int32)
        ptr_pin[r, 0, :w] = torch.as_tensor([kp[k] for k in lanes], dtype=torch.int64)
        ptr_pin[r, 1, :w] = torch.as_tensor([vp[k] for k in lanes], dtype=torch.int64)
        kv_dev[r].copy_(kv_pin[r], non_blocking=True)
        ptr_dev[r].copy_(ptr_pin[r], non_blocking=True)
        b = tables[w].struct()
        b.kv_len = kv_dev[r].data_ptr()
        b.k_cache = ptr_dev[r, 0].data_ptr()
        b.v_cache = ptr_dev[r, 1].data_ptr()
        b.err_flag = err.data_ptr()
        x = x_all[:w]
        assert sv.sv_verify_layer(Ld, b, x, y[:w], 0, ws, nmax, stream) == 0
        assert sv.sv_verify_layer(Lh, b, y[:w], probs, sv.SV_HEAD_LOGITS_STATS, ws, nmax, stream) == 0
        assert sv.sv_accept_commit(w, V, amode, [0] * w, zeros, zeros, probs, None, None, us, kv_dev[r],
                                   acc, nxt, err, ws, nmax, stream) == 0

    # t(B): plain decode steps at fixed widths
    tb = {}
    kv_host = [ctx0] * slots
    ring = 0
    for w in range(1, slots + 1):
        for _ in range(3):
            step(ring, list(range(w)), kv_host)
            ring += 1
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            step(ring, list(range(w)), kv_host)
            ring += 1
        e1.record()
        torch.cuda.synchronize()
        tb[w] = e0.elapsed_time(e1) / 20
        log(f"t({w}) = {tb[w]:.4f} ms")
    ws_ = np.arange(1, slots + 1)
    t1, t0 = np.polyfit(ws_, np.array([tb[w] for w in ws_]), 1)
    log(f"fit t(B) = {t0:.4f} + {t1:.5f} B ms")

    res = {}
    for pname, pol in (("static", sv.SV_SCHED_STATIC), ("shrink", sv.SV_SCHED_SHRINK),
                       ("continuous", sv.SV_SCHED_CONTINUOUS)):
        sch = sv.Scheduler(slots, pol)
        for n in lengths:
            sch.submit(n)
        kv_host = [ctx0] * slots
        owner = [-1] * slots
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        t_host = time.perf_counter()
        nsteps = useful = widths = 0
        while True:
            req, live, width = sch.next()
            if width == 0:
                break
            lanes = [k for k in range(slots) if req[k] >= 0]
            for k in lanes:
                if owner[k] != req[k]:       # a new request took the lane: its own context
                    owner[k] = req[k]
                    kv_host[k] = ctx0
            step(ring, lanes, kv_host)
            ring += 1
            for k in lanes:
                kv_host[k] += 1               # plain decoding commits one token per step
            useful += sch.commit([1] * slots)
            nsteps += 1
            widths += width
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3
        host_s = time.perf_counter() - t_host
        _, msec, model_tps, util = OB.throughput(pname, slots, lengths, t0, t1)
        res[pname] = {"steps": nsteps, "useful_tokens": useful, "seconds": round(sec, 4),
                      "tok_s": round(useful / sec, 1), "utilization": round(useful / widths, 4),
                      "model_tok_s": round(model_tps, 1), "host_seconds": round(host_s, 4)}
        log(f"{pname}: {json.dumps(res[pname])}")
    ceiling = slots / (tb[slots] * 1e-3)
    out = {"swarm": True, "lengths": list(SWARM_LENGTHS), "waves": args.swarm_waves, "ctx": ctx0,
           "t_B_ms": {str(w): round(v, 5) for w, v in tb.items()},
           "fit_ms": {"t0": round(float(t0), 5), "t1": round(float(t1), 6)},
           "ceiling_tok_s": round(ceiling, 1), "policies": res,
           "ratio_to_ceiling": {k: round(v["tok_s"] / ceiling, 4) for k, v in res.items()}}
    if err.item() != 0:
        raise RuntimeError(f"device error flags {err.item()}")
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3,
                    help="headline workload (default 3: the 27B-class bf16 layer, B=32, gamma=7)")
    ap.add_argument("--extra", default="2,5,5k",
                    help="further workloads reported under 'workloads' (empty: none; a 'k' "
                         "suffix runs the workload over int8 KV caches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=64,
                    help="verify tokens per oracle step in the CPU baseline sample")
    ap.add_argument("--no-kernel-table", action="store_true")
    ap.add_argument("--head-probs", action="store_true",
                    help="head writes probabilities and acceptance reads them (default: logits "
                         "plus row (max, sum), acceptance forms the probabilities it reads)")
    ap.add_argument("--sweep", action="store_true",
                    help="time the step over a (B, gamma) grid on one layer shape instead, fit the "
                         "step model per gamma and report the crossover batch")
    ap.add_argument("--sweep-shape", default="9b", choices=("9b", "27b"))
    ap.add_argument("--sweep-wtype", default="bf16", choices=("bf16", "int4"))
    ap.add_argument("--sweep-ctx", type=int, default=2048)
    ap.add_argument("--sweep-b", default="1,2,4,8,16,32,64,128,256")
    ap.add_argument("--sweep-gamma", default="0,1,2,3,4,5,7")
    ap.add_argument("--sweep-out", default="")
    ap.add_argument("--sweep-kernels", action="store_true",
                    help="also time each kernel class at every sweep point")
    ap.add_argument("--swarm", action="store_true",
                    help="run the eight-agent swarm through the verify path under the static, "
                         "shrinking and continuous batching policies of the library's scheduler")
    ap.add_argument("--swarm-waves", type=int, default=16)
    ap.add_argument("--swarm-ctx", type=int, default=1024)
    ap.add_argument("--tree", action="store_true",
                    help="token-tree verification against linear drafts (step time, emitted tokens)")
    ap.add_argument("--tree-shape-name", default="27b", choices=("9b", "27b"))
    ap.add_argument("--tree-ctx", type=int, default=2048)
    ap.add_argument("--tree-depth", type=int, default=8)
    ap.add_argument("--tree-stat-calls", type=int, default=64,
                    help="untimed acceptance calls (fresh drafts each) added to the tokens-per-step statistic")
    ap.add_argument("--tree-b", default="1,2,4,8,16,32")
    ap.add_argument("--tree-out", default="")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the steps, copy a buffer of this many MiB device to device three "
                         "times (the known-size reference for HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the verify path runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding across GPUs is not implemented", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return
    if args.swarm:
        swarm(args)
        return
    if args.tree:
        tree_bench(args)
        return

    import torch
    torch.cuda.set_device(0)
    K, Wm = args.steps, args.warmup
    res, cpu, wl = run_workload(args.workload, args, K, Wm, headline=True)
    others = {}
    for tok in [v.strip() for v in args.extra.split(",") if v.strip()]:
        c, kv8 = int(tok.rstrip("k")), tok.endswith("k")
        if c == args.workload and not kv8:
            continue
        torch.cuda.empty_cache()
        r, _, w = run_workload(c, args, K, Wm, headline=False, kv8=kv8)
        others[w.name] = r
    out = {
        "metric": METRIC, "value": res["verify_tok_s"], "unit": "verify tokens/s",
        "n_gpus": 1, "steps": K, "warmup": Wm, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.wtype != "f32" else "f32", "data": "synthetic",
        "config": res["config"],
        "accepted_tok_s": res["accepted_tok_s"],
        "tokens_per_step": res["tokens_per_step"],
        "roofline": res["roofline"],
        "step_roofline": res["step_roofline"],
        "kernels": res["kernels"],
        "cpu_baseline": cpu,
        "workloads": others,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
