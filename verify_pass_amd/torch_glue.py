"""Marshalling between host arrays, torch device tensors and the C structs.

torch supplies device memory and the current HIP stream; nothing here computes
any part of the verification path.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import (SV_LAYER_DECODER, SV_LAYER_EMBED, SV_LAYER_HEAD, SV_LAYOUT_PACKED,
               SV_LAYOUT_ROWMAJOR, SV_OK, WTYPES, SvError, sv_batch, sv_layer, sv_matrix,
               sv_pack_matrix, sv_packed_matrix_bytes)

__all__ = ["to_dev", "stream_handle", "workspace", "DeviceMatrix", "upload_matrix",
           "decoder_struct", "head_struct", "embed_struct", "DeviceBatch", "v_blocked", "v_logical"]


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Copy a host array to the device keeping its bits (uint16 -> bf16,
    uint32 -> int32)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(device)
    return torch.from_numpy(a).to(device)


def stream_handle(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Zero-filled workspace (the library's counters must start at zero)."""
    return torch.zeros(max(1, int(nbytes)), dtype=torch.uint8, device=device)


class DeviceMatrix:
    def __init__(self, w: torch.Tensor, scale: torch.Tensor | None):
        self.w, self.scale = w, scale

    def struct(self) -> sv_matrix:
        return sv_matrix(self.w.data_ptr(), self.scale.data_ptr() if self.scale is not None else None)

    @property
    def nbytes(self) -> int:
        return self.w.numel() * self.w.element_size() + (
            0 if self.scale is None else self.scale.numel() * self.scale.element_size())


def upload_matrix(m, device="cuda", packed=False) -> DeviceMatrix:
    """workloads.Weights -> DeviceMatrix, optionally re-laid out by the
    library's packing kernel (sv_pack_matrix)."""
    w = to_dev(m.data, device)
    s = None if m.scale is None else to_dev(m.scale, device)
    if not packed:
        return DeviceMatrix(w, s)
    wt = WTYPES[m.wtype]
    wb, sb = sv_packed_matrix_bytes(wt, m.n, m.k)
    wp = torch.empty(wb, dtype=torch.uint8, device=device)
    sp = torch.empty(max(sb, 1), dtype=torch.uint8, device=device) if sb else None
    st = sv_pack_matrix(wt, m.n, m.k, w, s, wp, sp, stream_handle())
    if st != SV_OK:
        raise SvError(st, "sv_pack_matrix")
    torch.cuda.synchronize()
    return DeviceMatrix(wp, sp)


def decoder_struct(shape, wtype: str, mats: dict, eps=1e-6, theta=10000.0, packed=False) -> sv_layer:
    L = sv_layer()
    L.kind, L.wtype = SV_LAYER_DECODER, WTYPES[wtype]
    L.layout = SV_LAYOUT_PACKED if packed else SV_LAYOUT_ROWMAJOR
    L.d, L.n_q_heads, L.n_kv_heads = shape.d, shape.n_q, shape.n_kv
    L.head_dim, L.ffn, L.vocab = shape.hd, shape.ffn, shape.vocab
    L.eps, L.rope_theta = eps, theta
    for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
        setattr(L, name, mats[name].struct())
    return L


def head_struct(shape, wtype: str, lm: DeviceMatrix, eps=1e-6, packed=False) -> sv_layer:
    L = sv_layer()
    L.kind, L.wtype = SV_LAYER_HEAD, WTYPES[wtype]
    L.layout = SV_LAYOUT_PACKED if packed else SV_LAYOUT_ROWMAJOR
    L.d, L.vocab, L.eps = shape.d, shape.vocab, eps
    L.lm_head = lm.struct()
    return L


def embed_struct(shape, table: torch.Tensor) -> sv_layer:
    L = sv_layer()
    L.kind = SV_LAYER_EMBED
    L.wtype = WTYPES["bf16"] if table.dtype == torch.bfloat16 else WTYPES["f32"]
    L.d, L.vocab = shape.d, shape.vocab
    L.embed = sv_matrix(table.data_ptr(), None)
    return L


class DeviceBatch:
    """Per-sequence KV caches and the batch arrays on the device.

    K caches are [n_kv][cap][hd] per sequence; V caches are stored in blocks
    of 32 positions, [n_kv][cap/32][hd][32]."""

    def __init__(self, gamma, kv_len, cap: int, max_ctx: int | None = None, kcache=None,
                 vcache=None, shape=None, device="cuda", caches=None, tree_parents=None,
                 kscale=None, vscale=None):
        self.gamma_list = [int(g) for g in gamma]
        self.B = len(self.gamma_list)
        self.T = int(sum(g + 1 for g in self.gamma_list))
        self.cap = int(cap)
        self.max_ctx = int(max(kv_len) if max_ctx is None and len(kv_len) else (max_ctx or 0))
        self.gamma = torch.tensor(self.gamma_list or [0], dtype=torch.int32, device=device)
        self.kv_len = torch.tensor([int(x) for x in kv_len] or [0], dtype=torch.int32, device=device)
        self.err = torch.zeros(1, dtype=torch.int32, device=device)
        self._gh = (C.c_int32 * max(1, self.B))(*self.gamma_list)
        self.k, self.v = [], []
        if caches is not None:  # device caches of an earlier batch, shared (not copied)
            self.k, self.v = list(caches[0]), list(caches[1])
            assert len(self.k) == self.B and len(self.v) == self.B
        elif kcache is not None:
            for i in range(self.B):
                self.k.append(to_dev(kcache[i], device))
                self.v.append(to_dev(v_blocked(vcache[i]), device))
        elif shape is not None:
            for _ in range(self.B):
                self.k.append(torch.zeros(shape.n_kv, cap, shape.hd, dtype=torch.bfloat16, device=device))
                self.v.append(torch.zeros(shape.n_kv, cap // 32, shape.hd, 32, dtype=torch.bfloat16,
                                          device=device))
        # int8 caches (codes in the bf16 layouts, one byte per value) and their
        # per-vector fp32 scales [n_kv][cap]
        self.kv8 = kscale is not None
        self.ks, self.vs = [], []
        if self.kv8:
            self.ks = [to_dev(np.ascontiguousarray(kscale[i]), device) for i in range(self.B)]
            self.vs = [to_dev(np.ascontiguousarray(vscale[i]), device) for i in range(self.B)]
        self.ksptr = torch.tensor([t.data_ptr() for t in self.ks] or [0], dtype=torch.int64, device=device)
        self.vsptr = torch.tensor([t.data_ptr() for t in self.vs] or [0], dtype=torch.int64, device=device)
        # token trees: every sequence's parent array, stacked like the tokens
        self.tree_parent = None
        if tree_parents is not None:
            flat = [int(v) for par in tree_parents for v in par]
            assert len(tree_parents) == self.B and len(flat) == self.T
            self.tree_parent = torch.tensor(flat or [0], dtype=torch.int32, device=device)
        self.kptr = torch.tensor([t.data_ptr() for t in self.k] or [0], dtype=torch.int64, device=device)
        self.vptr = torch.tensor([t.data_ptr() for t in self.v] or [0], dtype=torch.int64, device=device)

    def struct(self) -> sv_batch:
        b = sv_batch()
        b.B, b.T, b.max_ctx, b.kv_cap = self.B, self.T, self.max_ctx, self.cap
        b.gamma_host = C.cast(self._gh, C.POINTER(C.c_int32))
        b.gamma = self.gamma.data_ptr()
        b.kv_len = self.kv_len.data_ptr()
        b.k_cache = self.kptr.data_ptr()
        b.v_cache = self.vptr.data_ptr()
        b.err_flag = self.err.data_ptr()
        b.tree_parent = self.tree_parent.data_ptr() if self.tree_parent is not None else None
        b.kv_dtype = 1 if self.kv8 else 0
        b.k_scale = self.ksptr.data_ptr() if self.kv8 else None
        b.v_scale = self.vsptr.data_ptr() if self.kv8 else None
        return b

    def k_logical(self, i: int) -> np.ndarray:
        """Sequence i's K cache as bf16 bits [n_kv][cap][hd] (int8 caches: the codes)."""
        if self.kv8:
            return self.k[i].cpu().numpy()
        return self.k[i].view(torch.int16).cpu().numpy().view(np.uint16)

    def v_logical(self, i: int) -> np.ndarray:
        """Sequence i's V cache as bf16 bits in position-major order [n_kv][cap][hd]
        (int8 caches: the codes)."""
        if self.kv8:
            return v_logical(self.v[i].cpu().numpy())
        return v_logical(self.v[i].view(torch.int16).cpu().numpy().view(np.uint16))


def v_blocked(v: np.ndarray) -> np.ndarray:
    """[n_kv][cap][hd] values -> the library's [n_kv][cap/32][hd][32] blocks."""
    n, cap, hd = v.shape
    return np.ascontiguousarray(v.reshape(n, cap // 32, 32, hd).transpose(0, 1, 3, 2))


def v_logical(vb: np.ndarray) -> np.ndarray:
    """Inverse of v_blocked."""
    n, nb, hd, _ = vb.shape
    return np.ascontiguousarray(vb.transpose(0, 1, 3, 2).reshape(n, nb * 32, hd))
