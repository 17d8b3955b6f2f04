"""Shared set-up for the GPU parity tests: uploads seeded workloads, runs the
library through its C-ABI binding and the oracle on the same inputs."""
from __future__ import annotations

import numpy as np
import torch

import verify_pass_amd as sv
from oracle import accept as OA
from oracle import formats as OF
from oracle import verify as OV
from verify_pass_amd import torch_glue as tg
from workloads import (accept_inputs, embed_weights, head_weights, hidden_states, kv_cache,
                       layer_weights)

TOL = {"bf16": 2e-2, "f32": 2e-2, "int4": 5e-2}


def say(*a):
    print(*a, flush=True)


def rel_rows(got, ref) -> float:
    """max over rows of max|got - ref| / max|ref| (the logits error measure)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((num / den).max())


def dev_bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return OF.bf16_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def check(st, what=""):
    if st != sv.SV_OK:
        raise sv.SvError(st, what)


class GpuDecoder:
    """One decoder layer of a workload on the device, with its caches."""

    def __init__(self, wl, tag="layer0", max_ctx=None, packed=False):
        self.wl = wl
        sh = wl.shape
        self.W = layer_weights(sh, wl.wtype, wl.seed, tag)
        self.dev = {k: tg.upload_matrix(v, packed=packed) for k, v in self.W.items()}
        self.L = tg.decoder_struct(sh, wl.wtype, self.dev, packed=packed)
        self.kc, self.vc = kv_cache(sh, wl.ctx, wl.cap, wl.seed, tag)
        self.batch = tg.DeviceBatch(wl.gamma, wl.ctx, wl.cap, max_ctx=max_ctx, kcache=self.kc,
                                    vcache=self.vc)
        self.bs = self.batch.struct()
        self.ws_bytes = sv.sv_verify_layer_workspace_bytes(self.L, self.bs)
        self.ws = tg.workspace(self.ws_bytes)

    def run(self, x: torch.Tensor) -> torch.Tensor:
        y = torch.empty_like(x)
        check(sv.sv_verify_layer(self.L, self.bs, x, y, 0, self.ws, self.ws_bytes,
                                 tg.stream_handle()), "decoder")
        return y

    def oracle(self, x_host, seqs=None):
        return OV.decoder_layer(self.wl.shape, self.W, x_host, self.wl.gamma, self.wl.ctx,
                                self.kc, self.vc, seqs=seqs)


class GpuHead:
    def __init__(self, wl, vocab=None, packed=False):
        self.wl = wl
        self.Wlm = head_weights(wl.shape, wl.wtype, wl.seed)
        self.dev = tg.upload_matrix(self.Wlm, packed=packed)
        self.L = tg.head_struct(wl.shape, wl.wtype, self.dev, packed=packed)
        self.batch = tg.DeviceBatch(wl.gamma, wl.ctx, wl.cap)
        self.bs = self.batch.struct()
        self.ws_bytes = {f: sv.sv_verify_layer_workspace_bytes(self.L, self.bs, f)
                         for f in (0, sv.SV_HEAD_LOGITS, sv.SV_HEAD_LOGITS_STATS)}
        self.ws = tg.workspace(max(self.ws_bytes.values()))

    def run(self, y: torch.Tensor, logits=False, flags=None) -> torch.Tensor:
        """Probabilities [T][V], logits [T][V] (logits=True), or with
        flags=SV_HEAD_LOGITS_STATS the flat T*V logits followed by T (max, sum)."""
        f = flags if flags is not None else (sv.SV_HEAD_LOGITS if logits else 0)
        T, V = y.shape[0], self.wl.shape.vocab
        if f == sv.SV_HEAD_LOGITS_STATS:
            out = torch.empty(T * (V + 2), dtype=torch.float32, device=y.device)
        else:
            out = torch.empty(T, V, dtype=torch.float32, device=y.device)
        check(sv.sv_verify_layer(self.L, self.bs, y, out, f, self.ws, self.ws_bytes[f],
                                 tg.stream_handle()), "head")
        return out


def run_accept(gamma, V, inp, kv_len, mode=sv.SV_ACCEPT_STOCHASTIC):
    """Run sv_accept_commit on host arrays; returns (accepted, next, kv, err)."""
    dev = "cuda"
    g = torch.tensor(list(gamma) or [0], dtype=torch.int32, device=dev)
    B = len(gamma)
    t = lambda a, dt: torch.as_tensor(np.ascontiguousarray(a), dtype=dt, device=dev)  # noqa: E731
    draft = t(inp["draft"] if len(inp["draft"]) else np.zeros(1, np.int32), torch.int32)
    p = t(inp["p"], torch.float32)
    q = t(inp["q"] if len(inp["q"]) else np.zeros((1, V), np.float32), torch.float32)
    ua = t(inp["u_acc"] if len(inp["u_acc"]) else np.zeros(1, np.float32), torch.float32)
    us = t(inp["u_samp"], torch.float32)
    kv = t(np.asarray(kv_len, np.int32), torch.int32)
    acc = torch.full((B,), -7, dtype=torch.int32, device=dev)
    nxt = torch.full((B,), -7, dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    n = sv.sv_accept_commit_workspace_bytes(B, V, mode, list(gamma))
    ws = tg.workspace(n)
    check(sv.sv_accept_commit(B, V, mode, list(gamma), g, draft, p, q, ua, us, kv, acc, nxt, err,
                              ws, n, tg.stream_handle()), "accept")
    torch.cuda.synchronize()
    return acc.cpu().numpy(), nxt.cpu().numpy(), kv.cpu().numpy(), int(err.item())


def oracle_accept(gamma, inp, kv_len, greedy=False):
    return OA.accept_commit(gamma, inp["draft"], inp["p"], inp["q"], inp["u_acc"], inp["u_samp"],
                            kv_len, greedy=greedy)


__all__ = ["TOL", "say", "rel_rows", "dev_bf16_to_f64", "check", "GpuDecoder", "GpuHead",
           "run_accept", "oracle_accept", "accept_inputs", "embed_weights", "hidden_states",
           "OV", "OF", "OA", "tg", "sv"]
