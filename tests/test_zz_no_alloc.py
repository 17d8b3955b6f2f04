"""sv_accept_commit_noalloc: the acceptance entry point for callers that cannot
allocate.  Its outputs must equal sv_accept_commit's bit for bit, also on a
second call in a row with a smaller input (the fixed scratch array keeps the
previous call's contents), and a call too large for the array is refused on
the host."""
import ctypes as C

import numpy as np
import pytest
import torch

import verify_pass_amd as sv
from verify_pass_amd import torch_glue as tg
from workloads import SHAPES, accept_inputs, custom_workload


def _dev(a, dt):
    return torch.as_tensor(np.ascontiguousarray(a), dtype=dt, device="cuda")


def _both(gamma, ctx, V, mode, seed):
    """Runs the same acceptance through the workspace entry point and the
    no-allocation one; returns both (accepted, next, kv, err)."""
    wl = custom_workload(SHAPES["tiny"], "f32", gamma, ctx, draft="noise", seed=seed)
    rng = np.random.default_rng(seed)
    inp = accept_inputs(wl, V, target_logits=rng.standard_normal((wl.T, V)).astype(np.float32) * 2)
    B = wl.B
    g = _dev(wl.gamma, torch.int32)
    draft = _dev(inp["draft"] if len(inp["draft"]) else np.zeros(1, np.int32), torch.int32)
    p = _dev(inp["p"], torch.float32)
    q = _dev(inp["q"] if len(inp["q"]) else np.zeros((1, V), np.float32), torch.float32)
    ua = _dev(inp["u_acc"] if len(inp["u_acc"]) else np.zeros(1, np.float32), torch.float32)
    us = _dev(inp["u_samp"], torch.float32)
    outs = []
    for which in ("workspace", "noalloc"):
        kv = _dev(np.asarray(ctx, np.int32), torch.int32)
        acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        if which == "workspace":
            n = sv.sv_accept_commit_workspace_bytes(B, V, mode, list(gamma))
            ws = tg.workspace(n)
            st = sv.sv_accept_commit(B, V, mode, list(gamma), g, draft, p, q, ua, us, kv, acc, nxt,
                                     err, ws, n, tg.stream_handle())
        else:
            st = sv.sv_accept_commit_noalloc(B, V, mode, list(gamma), g, draft, p, q, ua, us, kv,
                                             acc, nxt, err, tg.stream_handle())
        assert st == sv.SV_OK, (which, st)
        torch.cuda.synchronize()
        outs.append((acc.cpu().numpy(), nxt.cpu().numpy(), kv.cpu().numpy(), int(err.item())))
    return outs


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice():
    rng = np.random.default_rng(5)
    # first call: 64 sequences over the full 151936-entry vocabulary
    gam = rng.integers(0, 8, size=64)
    ctx = rng.integers(0, 2000, size=64)
    ref, got = _both(gam, ctx, 151936, sv.SV_ACCEPT_STOCHASTIC, seed=5)
    for a, b in zip(ref, got):
        np.testing.assert_array_equal(a, b)
    assert ref[3] == 0
    # second call in a row, smaller: 5 sequences, small vocabulary, greedy
    gam2 = [2, 0, 4, 1, 3]
    ref2, got2 = _both(gam2, [7, 0, 30, 5, 11], 3000, sv.SV_ACCEPT_GREEDY, seed=6)
    for a, b in zip(ref2, got2):
        np.testing.assert_array_equal(a, b)
    # and stochastic again at the small size
    ref3, got3 = _both(gam2, [7, 0, 30, 5, 11], 3000, sv.SV_ACCEPT_STOCHASTIC, seed=7)
    for a, b in zip(ref3, got3):
        np.testing.assert_array_equal(a, b)


def test_noalloc_refuses_calls_beyond_its_scratch():
    # greedy over 12000 stacked rows of a 151936-entry vocabulary needs more
    # than the fixed array: refused on the host, nothing enqueued
    B, V = 3000, 151936
    gam = [3] * B
    fake = 1 << 20  # never dereferenced: the size check comes first
    st = sv.sv_accept_commit_noalloc(B, V, sv.SV_ACCEPT_GREEDY, gam, fake, fake, fake, None, None,
                                     None, fake, fake, fake, None, None)
    assert st == sv.SV_ERR_TOO_LARGE
    assert "scratch" in sv.sv_status_string(st)
    # argument errors are still reported as such
    assert sv.sv_accept_commit_noalloc(-1, V, 0, [], None, None, None, None, None, None, None,
                                       None, None, None, None) == sv.SV_ERR_INVALID_ARG
