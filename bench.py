#!/usr/bin/env python3
"""Benchmark of one batched speculative-verification step on one MI355X.

A step is the whole hot path over one batch: plan the draft lengths (host),
the decoder layer over the stacked verify tokens (QKV + RoPE + KV append,
ragged attention, O, SwiGLU FFN), the LM head with softmax, and acceptance /
resampling / KV-length commit.  Default workload: one 9B-class bf16 layer,
B=8 sequences with gamma=2 drafts each, 2048 cached tokens, a 151936-entry
head, acceptance rate 0.8.  Inputs are seeded synthetic data resident in HBM
before timing starts.

Prints one JSON line (stdout); progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload N] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
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


def attention_algorithmic(wl):
    sh = wl.shape
    keys = int(sum(int(c) + int(g) + 1 for c, g in zip(wl.ctx, wl.gamma)))
    kv = keys * sh.n_kv * sh.hd * 2 * 2
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


def cpu_baseline(wl, W, Wlm, kc, vc, xh, acc_in):
    """The oracle, as it stands, on a bounded sample: sequence 0 of the batch
    through the layer, the head and acceptance."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import accept as OA
    from oracle import verify as OV
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t0 = time.perf_counter()
        out = OV.decoder_layer(wl.shape, W, xh, wl.gamma, wl.ctx, kc, vc, seqs=[0])
        n_tok = len(out.rows)
        if Wlm is not None:
            lg = OV.head_logits(Wlm, out.y)
            p = OV.softmax(lg).astype(np.float32)
        else:
            p = acc_in["p"][out.rows]
        g0 = int(wl.gamma[0])
        OA.accept_commit([g0], acc_in["draft"][:g0], p, acc_in["q"][:g0], acc_in["u_acc"][:g0],
                         acc_in["u_samp"][:1], wl.ctx[:1])
        dt = time.perf_counter() - t0
    return {"value": round(n_tok / dt, 4), "unit": "verify tokens/s", "cores": int(blas),
            "kind": "oracle",
            "sample": f"sequence 0 of the batch ({n_tok} verify tokens): decoder layer, "
                      f"{'LM head + softmax, ' if Wlm is not None else ''}acceptance; "
                      f"{dt:.1f} s on {blas} BLAS threads ({cores} cores visible)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-table", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the steps, copy a buffer of this many MiB device to device three "
                         "times (the known-size reference for HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the "
              "sharded design is described in DESIGN.md", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import verify_pass_amd as sv
    from verify_pass_amd import torch_glue as tg
    from workloads import (accept_inputs, head_weights, hidden_states, kv_cache, layer_weights,
                           rng_for, uniforms_2m24, workload)

    torch.cuda.set_device(0)
    wl = workload(args.workload)
    sh = wl.shape
    K, Wm = args.steps, args.warmup
    log(f"workload {wl.cid} {wl.name}: B={wl.B} T={wl.T} wtype={wl.wtype}")

    t0 = time.perf_counter()
    W = layer_weights(sh, wl.wtype, wl.seed)
    Wlm = head_weights(sh, wl.wtype, wl.seed) if wl.head else None
    kc, vc = kv_cache(sh, wl.ctx, wl.cap, wl.seed)
    xh = hidden_states(wl.T, sh.d, wl.seed)
    log(f"generated inputs in {time.perf_counter() - t0:.1f} s")

    packed = wl.wtype != "f32"
    mats = {k: tg.upload_matrix(v, packed=packed) for k, v in W.items()}
    lm = tg.upload_matrix(Wlm, packed=packed) if Wlm is not None else None
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
        nh = sv.sv_verify_layer_workspace_bytes(Lh, bs)
        nhl = sv.sv_verify_layer_workspace_bytes(Lh, bs, sv.SV_HEAD_LOGITS)
        ws_h = tg.workspace(max(nh, nhl))
        probs = torch.empty(wl.T, V, dtype=torch.float32, device="cuda")

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
    na = sv.sv_accept_commit_workspace_bytes(wl.B, V, 0, list(wl.gamma))
    ws_a = tg.workspace(na)
    glist = list(int(g) for g in wl.gamma)
    plan = sv.make_plan_params(sv.SV_PLAN_BUDGET, 64, budget_tokens=24)

    def step(k):
        st, _, _ = sv.sv_plan_gamma(plan, wl.B)          # host: draft lengths for the live batch
        assert st == 0
        batch.kv_len.copy_(kv0)                            # every step verifies the same state
        assert sv.sv_verify_layer(Ld, bs, x, y, 0, ws_d, nd, stream) == 0
        if lm is not None:
            assert sv.sv_verify_layer(Lh, bs, y, probs, 0, ws_h, nh, stream) == 0
        p_acc = p_alpha if p_alpha is not None else probs
        assert sv.sv_accept_commit(wl.B, V, 0, glist, batch.gamma, draft, p_acc, q, ua[k], us[k],
                                   batch.kv_len, acc_all[k], nxt_all[k], batch.err, ws_a, na,
                                   stream) == 0

    if args.copy_probe_mib > 0:
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
    ab, af = attention_algorithmic(wl)
    tot_b += ab
    tot_f += af
    step_roof = roofline_of(tot_b, tot_f, ms)
    step_roof.update({"algorithmic_bytes": int(tot_b), "algorithmic_flops": tot_f})

    kernels = {}
    if not args.no_kernel_table:
        names = {sv.SV_K_GEMM_QKV: "gemm_qkv", sv.SV_K_ATTENTION: "attention",
                 sv.SV_K_GEMM_O: "gemm_o",
                 sv.SV_K_GEMM_GATE_UP: "gemm_gate_up", sv.SV_K_GEMM_DOWN: "gemm_down",
                 sv.SV_K_GEMM_LM_HEAD: "gemm_lm_head", sv.SV_K_SOFTMAX: "softmax",
                 sv.SV_K_ACCEPT: "accept", sv.SV_K_PREP: "prep"}
        for cls, nm in names.items():
            n = 10
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

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (bounded sample)...")
        cpu = cpu_baseline(wl, W, Wlm, kc, vc, xh, acc_in)
        log(f"oracle: {cpu}")

    out = {
        "metric": METRIC, "value": round(verify_tok_s, 2), "unit": "verify tokens/s",
        "n_gpus": 1, "steps": K, "warmup": Wm, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.wtype != "f32" else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "gamma": glist if wl.B <= 16 else int(wl.gamma[0]),
                   "T": wl.T, "ctx": int(wl.ctx[0]) if len(set(wl.ctx.tolist())) == 1 else "ragged",
                   "weights": wl.wtype + (" packed" if packed else ""), "d": sh.d, "heads": f"{sh.n_q}q/{sh.n_kv}kv x {sh.hd}",
                   "ffn": sh.ffn, "vocab": V if lm is not None else None,
                   "acceptance": (wl.alphas[0] if wl.alphas else wl.draft)},
        "accepted_tok_s": round(accepted_tok_s, 2),
        "tokens_per_step": round(tokens_per_step, 3),
        "roofline": roof,
        "step_roofline": step_roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
