"""Python binding of libsv.so, the MI355X batched speculative-verification library.

The functions below carry the names of the C entry points declared in
include/sv.h and only marshal arguments: every step of the verification path
runs in the library's gfx950 kernels.  Importing this package loads the
in-tree libsv.so and fails loudly if it has not been built
(``python verify_pass_amd/csrc/build.py``).  torch is used by the helpers in
``verify_pass_amd.torch_glue`` for device memory and streams only.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsv.so")

SV_OK = 0
SV_ERR_INVALID_ARG = -1
SV_ERR_UNSUPPORTED = -2
SV_ERR_WORKSPACE = -3
SV_ERR_HIP = -4
SV_ERR_TOO_LARGE = -5
SV_ACCEPT_NOALLOC_SCRATCH_BYTES = 4 << 20

SV_DEV_ERR_BAD_TOKEN = 1
SV_DEV_ERR_KV_OVERFLOW = 2
SV_DEV_ERR_CTX_BOUND = 4
SV_DEV_ERR_BAD_TREE = 8

SV_LAYER_EMBED, SV_LAYER_DECODER, SV_LAYER_HEAD = 0, 1, 2
SV_W_F32, SV_W_BF16, SV_W_INT4_G32 = 0, 1, 2
SV_HEAD_LOGITS, SV_HEAD_LOGITS_STATS = 1, 2
SV_LAYOUT_ROWMAJOR, SV_LAYOUT_PACKED = 0, 1
SV_ACCEPT_STOCHASTIC, SV_ACCEPT_GREEDY = 0, 1
SV_ACCEPT_FROM_LOGITS = 0x100
SV_PLAN_BUDGET, SV_PLAN_SPEEDUP = 0, 1
SV_SCHED_STATIC, SV_SCHED_SHRINK, SV_SCHED_CONTINUOUS = 0, 1, 2
SV_KV_BF16, SV_KV_INT8 = 0, 1

SV_K_GEMM_QKV, SV_K_ATTENTION = 0, 1
(SV_K_GEMM_O, SV_K_GEMM_GATE_UP, SV_K_GEMM_DOWN, SV_K_GEMM_LM_HEAD, SV_K_SOFTMAX, SV_K_ACCEPT,
 SV_K_PREP, SV_K_EMBED, SV_K_COUNT) = range(3, 12)

WTYPES = {"f32": SV_W_F32, "bf16": SV_W_BF16, "int4": SV_W_INT4_G32}


class sv_matrix(C.Structure):
    _fields_ = [("w", C.c_void_p), ("scale", C.c_void_p)]


class sv_layer(C.Structure):
    _fields_ = [("kind", C.c_int32), ("wtype", C.c_int32), ("layout", C.c_int32), ("d", C.c_int32),
                ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("ffn", C.c_int32), ("vocab", C.c_int32), ("eps", C.c_float),
                ("rope_theta", C.c_float),
                ("wq", sv_matrix), ("wk", sv_matrix), ("wv", sv_matrix), ("wo", sv_matrix),
                ("w_gate", sv_matrix), ("w_up", sv_matrix), ("w_down", sv_matrix),
                ("embed", sv_matrix), ("lm_head", sv_matrix)]


class sv_batch(C.Structure):
    _fields_ = [("B", C.c_int32), ("T", C.c_int32), ("max_ctx", C.c_int32),
                ("kv_cap", C.c_int32), ("gamma_host", C.POINTER(C.c_int32)),
                ("gamma", C.c_void_p), ("kv_len", C.c_void_p), ("k_cache", C.c_void_p),
                ("v_cache", C.c_void_p), ("err_flag", C.c_void_p),
                ("tree_parent", C.c_void_p), ("kv_dtype", C.c_int32),
                ("k_scale", C.c_void_p), ("v_scale", C.c_void_p)]


class sv_plan_params(C.Structure):
    _fields_ = [("mode", C.c_int32), ("gamma_max", C.c_int32), ("budget_tokens", C.c_int32),
                ("fill_remainder", C.c_int32), ("t_floor_ms", C.c_double),
                ("t_w_ms", C.c_double), ("k_ms", C.c_double), ("c_ms", C.c_double),
                ("draft_frac", C.c_double), ("n_alpha", C.c_int32),
                ("alpha", C.POINTER(C.c_double))]


# (name, restype, argtypes) for every symbol declared in include/sv.h
_SIGNATURES = [
    ("sv_verify_layer_workspace_bytes", C.c_int32,
     [C.POINTER(sv_layer), C.POINTER(sv_batch), C.c_int32, C.POINTER(C.c_size_t)]),
    ("sv_verify_layer", C.c_int32,
     [C.POINTER(sv_layer), C.POINTER(sv_batch), C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
      C.c_size_t, C.c_void_p]),
    ("sv_accept_commit_workspace_bytes", C.c_int32,
     [C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_size_t)]),
    ("sv_accept_commit", C.c_int32,
     [C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_int32), C.c_void_p, C.c_void_p, C.c_void_p,
      C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
      C.c_void_p, C.c_size_t, C.c_void_p]),
    ("sv_accept_commit_noalloc", C.c_int32,
     [C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_int32), C.c_void_p, C.c_void_p, C.c_void_p,
      C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
      C.c_void_p]),
    ("sv_accept_tree_workspace_bytes", C.c_int32,
     [C.c_int32, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_size_t)]),
    ("sv_accept_tree", C.c_int32,
     [C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_int32)] + [C.c_void_p] * 14),
    ("sv_tree_commit_kv", C.c_int32,
     [C.c_int32, C.c_int32, C.c_int32, C.c_int32] + [C.c_void_p] * 6),
    ("sv_tree_commit_kv_int8", C.c_int32,
     [C.c_int32, C.c_int32, C.c_int32, C.c_int32] + [C.c_void_p] * 8),
    ("sv_accept_position_counts", C.c_int32,
     [C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    ("sv_packed_matrix_bytes", C.c_int32,
     [C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    ("sv_pack_matrix", C.c_int32,
     [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    ("sv_plan_gamma", C.c_int32,
     [C.POINTER(sv_plan_params), C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_double)]),
    ("sv_set_gemm_tuning", C.c_int32, [C.c_char_p]),
    ("sv_sched_create", C.c_int32, [C.c_int32, C.c_int32, C.POINTER(C.c_void_p)]),
    ("sv_sched_destroy", C.c_int32, [C.c_void_p]),
    ("sv_sched_submit", C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32)]),
    ("sv_sched_next", C.c_int32, [C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                  C.POINTER(C.c_int32)]),
    ("sv_sched_commit", C.c_int32, [C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    ("sv_trace_begin", C.c_int32, [C.c_int32, C.c_int32, C.c_int32]),
    ("sv_trace_end", C.c_int32, [C.POINTER(C.c_float), C.c_int32, C.POINTER(C.c_int32)]),
    ("sv_status_string", C.c_char_p, [C.c_int32]),
    ("sv_version", C.c_int32, []),
]


class SvError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {status} ({sv_status_string(status)})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python verify_pass_amd/csrc/build.py` "
                          "(the verification path has no fallback)")
    try:  # bind to the HIP runtime torch already loaded, if any
        import torch  # noqa: F401
    except Exception:  # pragma: no cover
        pass
    lib = C.CDLL(LIB_PATH)
    for name, res, args in _SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _ptr(x) -> int | None:
    """Device/host address of a tensor-like (anything with data_ptr) or int."""
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def sv_status_string(status: int) -> str:
    return _lib.sv_status_string(status).decode()


def sv_version() -> int:
    return _lib.sv_version()


def sv_verify_layer_workspace_bytes(layer: sv_layer, batch: sv_batch, flags: int = 0) -> int:
    n = C.c_size_t(0)
    st = _lib.sv_verify_layer_workspace_bytes(C.byref(layer), C.byref(batch), flags, C.byref(n))
    if st != SV_OK:
        raise SvError(st, "sv_verify_layer_workspace_bytes")
    return n.value


def sv_verify_layer(layer: sv_layer, batch: sv_batch, x_in, y_out, flags, workspace,
                    workspace_bytes, stream) -> int:
    return _lib.sv_verify_layer(C.byref(layer), C.byref(batch), _ptr(x_in), _ptr(y_out), flags,
                                _ptr(workspace), workspace_bytes, _ptr(stream))


def sv_accept_commit_workspace_bytes(B, V, mode, gamma_host) -> int:
    n = C.c_size_t(0)
    g = (C.c_int32 * max(1, len(gamma_host)))(*[int(x) for x in gamma_host])
    st = _lib.sv_accept_commit_workspace_bytes(B, V, mode, g, C.byref(n))
    if st != SV_OK:
        raise SvError(st, "sv_accept_commit_workspace_bytes")
    return n.value


def sv_accept_commit(B, V, mode, gamma_host, gamma, draft, p, q, u_acc, u_samp, kv_len, accepted,
                     next_token, err_flag, workspace, workspace_bytes, stream) -> int:
    g = (C.c_int32 * max(1, len(gamma_host)))(*[int(x) for x in gamma_host])
    return _lib.sv_accept_commit(B, V, mode, g, _ptr(gamma), _ptr(draft), _ptr(p), _ptr(q),
                                 _ptr(u_acc), _ptr(u_samp), _ptr(kv_len), _ptr(accepted),
                                 _ptr(next_token), _ptr(err_flag), _ptr(workspace),
                                 workspace_bytes, _ptr(stream))


def sv_accept_commit_noalloc(B, V, mode, gamma_host, gamma, draft, p, q, u_acc, u_samp, kv_len,
                             accepted, next_token, err_flag, stream) -> int:
    g = (C.c_int32 * max(1, len(gamma_host)))(*[int(x) for x in gamma_host])
    return _lib.sv_accept_commit_noalloc(B, V, mode, g, _ptr(gamma), _ptr(draft), _ptr(p), _ptr(q),
                                         _ptr(u_acc), _ptr(u_samp), _ptr(kv_len), _ptr(accepted),
                                         _ptr(next_token), _ptr(err_flag), _ptr(stream))


def sv_accept_tree_workspace_bytes(B, V, gamma_host) -> int:
    n = C.c_size_t(0)
    g = (C.c_int32 * max(1, len(gamma_host)))(*[int(x) for x in gamma_host])
    st = _lib.sv_accept_tree_workspace_bytes(B, V, g, C.byref(n))
    if st != SV_OK:
        raise SvError(st, "sv_accept_tree_workspace_bytes")
    return n.value


def sv_accept_tree(B, V, mode, gamma_host, parent, tokens, p, q, u_acc, u_samp, kv_len, accepted,
                   next_token, path, err_flag, workspace, workspace_bytes, stream) -> int:
    g = (C.c_int32 * max(1, len(gamma_host)))(*[int(x) for x in gamma_host])
    return _lib.sv_accept_tree(B, V, mode, g, _ptr(parent), _ptr(tokens), _ptr(p), _ptr(q),
                               _ptr(u_acc), _ptr(u_samp), _ptr(kv_len), _ptr(accepted),
                               _ptr(next_token), _ptr(path), _ptr(err_flag), _ptr(workspace),
                               workspace_bytes, _ptr(stream))


def sv_tree_commit_kv(B, n_kv_heads, head_dim, kv_cap, kv_len, accepted, path, k_cache, v_cache,
                      stream) -> int:
    return _lib.sv_tree_commit_kv(B, n_kv_heads, head_dim, kv_cap, _ptr(kv_len), _ptr(accepted),
                                  _ptr(path), _ptr(k_cache), _ptr(v_cache), _ptr(stream))


def sv_tree_commit_kv_int8(B, n_kv_heads, head_dim, kv_cap, kv_len, accepted, path, k_cache, v_cache,
                           k_scale, v_scale, stream) -> int:
    return _lib.sv_tree_commit_kv_int8(B, n_kv_heads, head_dim, kv_cap, _ptr(kv_len), _ptr(accepted),
                                       _ptr(path), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                       _ptr(v_scale), _ptr(stream))


def sv_accept_position_counts(B, n_pos, gamma, accepted, counts, stream) -> int:
    return _lib.sv_accept_position_counts(B, n_pos, _ptr(gamma), _ptr(accepted), _ptr(counts),
                                          _ptr(stream))


def sv_packed_matrix_bytes(wtype: int, N: int, K: int):
    """Returns (w_bytes, scale_bytes) of the packed layout."""
    w, s = C.c_size_t(0), C.c_size_t(0)
    st = _lib.sv_packed_matrix_bytes(wtype, N, K, C.byref(w), C.byref(s))
    if st != SV_OK:
        raise SvError(st, "sv_packed_matrix_bytes")
    return w.value, s.value


def sv_pack_matrix(wtype, N, K, w, scale, w_packed, scale_packed, stream) -> int:
    return _lib.sv_pack_matrix(wtype, N, K, _ptr(w), _ptr(scale), _ptr(w_packed),
                               _ptr(scale_packed), _ptr(stream))


def sv_plan_gamma(params: sv_plan_params, B_live: int):
    """Returns (status, gamma list, B*)."""
    out = (C.c_int32 * max(1, B_live))()
    bstar = C.c_double(0.0)
    st = _lib.sv_plan_gamma(C.byref(params), B_live, out, C.byref(bstar))
    return st, [int(out[i]) for i in range(B_live)], bstar.value


def sv_set_gemm_tuning(spec: str | None) -> int:
    return _lib.sv_set_gemm_tuning(None if spec is None else spec.encode())


def sv_trace_begin(kernel_class: int, capacity: int, stride: int = 1) -> int:
    return _lib.sv_trace_begin(kernel_class, capacity, stride)


def sv_trace_end(capacity: int):
    """Returns (status, list of per-launch milliseconds)."""
    buf = (C.c_float * max(1, capacity))()
    n = C.c_int32(0)
    st = _lib.sv_trace_end(buf, capacity, C.byref(n))
    return st, [float(buf[i]) for i in range(min(n.value, capacity))]


class Scheduler:
    """sv_sched_* handle: submit(tokens) -> request id; next() -> (slot
    requests, live flags, width); commit(emitted per lane) -> useful tokens."""

    def __init__(self, slots: int, policy: int):
        self.slots = slots
        self._h = C.c_void_p()
        st = _lib.sv_sched_create(slots, policy, C.byref(self._h))
        if st != SV_OK:
            raise SvError(st, "sv_sched_create")
        self._req = (C.c_int32 * slots)()
        self._live = (C.c_int32 * slots)()
        self._em = (C.c_int32 * slots)()

    def submit(self, tokens: int) -> int:
        r = C.c_int32(-1)
        st = _lib.sv_sched_submit(self._h, tokens, C.byref(r))
        if st != SV_OK:
            raise SvError(st, "sv_sched_submit")
        return r.value

    def next(self):
        w = C.c_int32(0)
        st = _lib.sv_sched_next(self._h, self._req, self._live, C.byref(w))
        if st != SV_OK:
            raise SvError(st, "sv_sched_next")
        return list(self._req), list(self._live), w.value

    def commit(self, emitted) -> int:
        for k in range(self.slots):
            self._em[k] = int(emitted[k])
        u = C.c_int32(0)
        st = _lib.sv_sched_commit(self._h, self._em, C.byref(u))
        if st != SV_OK:
            raise SvError(st, "sv_sched_commit")
        return u.value

    def __del__(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _lib.sv_sched_destroy(self._h)
            self._h = C.c_void_p()


def make_plan_params(mode, gamma_max, *, budget_tokens=0, fill_remainder=True, t_floor_ms=0.0,
                     t_w_ms=0.0, k_ms=0.0, c_ms=0.0, draft_frac=0.04, alpha=(1.0,)):
    arr = (C.c_double * len(alpha))(*alpha)
    p = sv_plan_params(mode, gamma_max, budget_tokens, 1 if fill_remainder else 0, t_floor_ms,
                       t_w_ms, k_ms, c_ms, draft_frac, len(alpha),
                       C.cast(arr, C.POINTER(C.c_double)))
    p._keep = arr  # keep the array alive with the struct
    return p


def exported_symbols():
    return [n for n, _, _ in _SIGNATURES]
