"""Host-side pieces of bench.py: the oracle baseline on a bounded sample and
the step-model fit (no GPU)."""
import numpy as np

import bench
from workloads import accept_inputs, head_weights, hidden_states, kv_cache, layer_weights, workload


def test_cpu_baseline_runs_whole_steps():
    wl = workload(1)
    sh = wl.shape
    W = layer_weights(sh, wl.wtype, wl.seed)
    Wlm = head_weights(sh, wl.wtype, wl.seed)
    kc, vc = kv_cache(sh, wl.ctx, wl.cap, wl.seed)
    xh = hidden_states(wl.T, sh.d, wl.seed)
    acc_in = accept_inputs(wl, sh.vocab)
    r = bench.cpu_baseline(wl, W, Wlm, kc, vc, xh, acc_in, seqs_per_rep=1, min_seconds=0.0,
                           max_reps=2)
    assert r["kind"] == "oracle" and r["unit"] == "verify tokens/s"
    assert r["value"] > 0 and r["cores"] >= 1 and r["cpu"]
    assert r["sample"].startswith(f"1 verify step(s) of the first 1 of the workload's {wl.B} "
                                  f"sequences ({wl.T} verify tokens in all)")


def test_cpu_baseline_sample_of_a_larger_batch():
    from workloads import SHAPES, custom_workload
    sh = SHAPES["tiny"]
    wl = custom_workload(sh, "f32", [2, 1, 3], [10, 20, 30], draft="noise", seed=5)
    W = layer_weights(sh, wl.wtype, wl.seed)
    Wlm = head_weights(sh, wl.wtype, wl.seed)
    kc, vc = kv_cache(sh, wl.ctx, wl.cap, wl.seed)
    xh = hidden_states(wl.T, sh.d, wl.seed)
    acc_in = accept_inputs(wl, sh.vocab)
    r = bench.cpu_baseline(wl, W, Wlm, kc, vc, xh, acc_in, seqs_per_rep=2, min_seconds=0.0,
                           max_reps=1)
    assert "first 2 of the workload's 3 sequences (5 verify tokens in all)" in r["sample"]


def test_step_model_fit_recovers_constants():
    tw, k, c, n = 100e-6, 0.5e-6, 4e-6, 3
    bs = np.array([1, 2, 4, 8, 16, 32, 64, 128, 256])
    ts = np.maximum(tw + k * bs, c * bs * n)
    ftw, fk, fc = bench.fit_step_model(bs, ts, n)
    assert abs(ftw - tw) / tw < 1e-3 and abs(fc - c) / c < 1e-3
    assert abs(fk - k) / k < 5e-2


def test_tree_shape_is_a_spine_with_one_extra_candidate_per_level():
    from oracle import tree as OT
    for depth in (1, 2, 5, 8, 16):
        par = bench.tree_shape(depth)
        assert len(par) == 2 * depth
        dep = OT.depths(par)          # also checks topological order
        assert dep.max() == depth
        kids = [OT.children(par, v) for v in range(len(par))]
        chain = [0] + [v for v in range(1, len(par)) if kids[v] or dep[v] == depth]
        assert [int(dep[v]) for v in chain] == list(range(depth + 1))
        for v in chain[:-1]:
            # two candidates at every level but the last, the chain going on through the first
            assert len(kids[v]) == (2 if dep[v] < depth - 1 else 1)
            assert kids[v][0] == chain[int(dep[v]) + 1]
            assert all(not kids[c] for c in kids[v][1:])
    assert bench.tree_shape(8) == [-1, 0, 0, 1, 1, 3, 3, 5, 5, 7, 7, 9, 9, 11, 11, 13]


def test_more_than_one_gpu_exits_with_a_message():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                       cwd=bench.os.path.dirname(bench.os.path.abspath(bench.__file__)), timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr and not r.stdout
