"""Thin Python binding of libhs2 (the C ABI in include/hs2.h).

Argument marshalling only: every step of the hot path runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream. The functions
raise if the built library cannot be loaded; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhs2.so")

HS2_OK, HS2_ERR_INVALID_ARG, HS2_ERR_UNSUPPORTED, HS2_ERR_WORKSPACE, HS2_ERR_HIP = 0, -1, -2, -3, -4
HS2_BF16, HS2_F32, HS2_FP8_E4M3 = 0, 1, 2
MAX_TOP_K = 4096

EXPORTED = [
    "hs2_version",
    "hs2_last_error",
    "hs2_bridge_kv_workspace_size",
    "hs2_bridge_kv",
    "hs2_bridge_kv_fp8kv",
    "hs2_full_attn_select_workspace_size",
    "hs2_full_attn_select",
    "hs2_sparse_attn_workspace_size",
    "hs2_sparse_attn",
    "hs2_sparse_attn_noalloc",
    "hs2_bridge_kv_append_workspace_size",
    "hs2_bridge_kv_append",
    "hs2_bridge_kv_append_fp8kv",
    "hs2_causal_attn_workspace_size",
    "hs2_causal_attn",
    "hs2_full_attn_select_fp8kv",
    "hs2_sparse_attn_fp8kv",
    "hs2_set_kernel_events",
    "hs2_v1_full_attn_select_workspace_size",
    "hs2_v1_full_attn_select",
    "hs2_v1_sparse_attn_workspace_size",
    "hs2_v1_sparse_attn",
]


class hs2_seqs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("kv_start", ctypes.c_void_p),
        ("kv_len", ctypes.c_void_p),
        ("q_start", ctypes.c_void_p),
        ("q_pos", ctypes.c_void_p),
        ("total_q", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32),
        ("total_kv_rows", ctypes.c_int64),
        ("max_q_per_seq", ctypes.c_int32),
        ("kv_len_host", ctypes.c_void_p),
    ]


class HS2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"hs2 status {status}: {msg}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libhs2.so (built in-tree by long_context_mqa_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m long_context_mqa_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    SP = ctypes.POINTER(hs2_seqs)
    lib.hs2_version.restype = I32
    lib.hs2_version.argtypes = []
    lib.hs2_last_error.restype = ctypes.c_char_p
    lib.hs2_last_error.argtypes = []
    lib.hs2_bridge_kv_workspace_size.restype = SZ
    lib.hs2_bridge_kv_workspace_size.argtypes = [I32, I32, I32]
    lib.hs2_bridge_kv.restype = I32
    lib.hs2_bridge_kv.argtypes = [P, I64, I32, I32, P, P, P, P, I32, P, SZ, I32, P]
    lib.hs2_bridge_kv_fp8kv.restype = I32
    lib.hs2_bridge_kv_fp8kv.argtypes = [P, I64, I32, I32, P, P, P, P, P, P, I32, P, SZ, P]
    lib.hs2_full_attn_select_workspace_size.restype = SZ
    lib.hs2_full_attn_select_workspace_size.argtypes = [SP, I32, I32, I32, I32, I32]
    lib.hs2_full_attn_select.restype = I32
    lib.hs2_full_attn_select.argtypes = [SP, P, P, P, I32, I32, I32, I32, F, P, P, P, P, P, SZ, I32, P]
    lib.hs2_sparse_attn_workspace_size.restype = SZ
    lib.hs2_sparse_attn_workspace_size.argtypes = [SP, I32, I32, I32, I32, I32]
    lib.hs2_sparse_attn.restype = I32
    lib.hs2_sparse_attn.argtypes = [SP, P, P, P, P, I32, I32, I32, I32, F, P, P, P, SZ, I32, P]
    lib.hs2_sparse_attn_noalloc.restype = I32
    lib.hs2_sparse_attn_noalloc.argtypes = [SP, P, P, P, P, I32, I32, I32, I32, F, P, P, I32, P]
    lib.hs2_bridge_kv_append_workspace_size.restype = SZ
    lib.hs2_bridge_kv_append_workspace_size.argtypes = [I32, I32, I32, I32]
    lib.hs2_bridge_kv_append.restype = I32
    lib.hs2_bridge_kv_append.argtypes = [P, I32, P, I64, I32, I32, P, P, P, P, I32, P, SZ, I32, P]
    lib.hs2_bridge_kv_append_fp8kv.restype = I32
    lib.hs2_bridge_kv_append_fp8kv.argtypes = [P, I32, P, I64, I32, I32, P, P, P, P, P, P, I32, P, SZ, P]
    lib.hs2_causal_attn_workspace_size.restype = SZ
    lib.hs2_causal_attn_workspace_size.argtypes = [SP, I32, I32, I32]
    lib.hs2_causal_attn.restype = I32
    lib.hs2_causal_attn.argtypes = [SP, P, P, P, I32, I32, F, P, P, P, SZ, I32, P]
    lib.hs2_full_attn_select_fp8kv.restype = I32
    lib.hs2_full_attn_select_fp8kv.argtypes = [SP, P, P, P, F, F, I32, I32, I32, I32, F, P, P, P, P, P, SZ, P]
    lib.hs2_sparse_attn_fp8kv.restype = I32
    lib.hs2_sparse_attn_fp8kv.argtypes = [SP, P, P, P, F, F, P, I32, I32, I32, I32, F, P, P, P, SZ, P]
    lib.hs2_set_kernel_events.restype = I32
    lib.hs2_set_kernel_events.argtypes = [P, I32]
    lib.hs2_v1_full_attn_select_workspace_size.restype = SZ
    lib.hs2_v1_full_attn_select_workspace_size.argtypes = [SP, I32, I32, I32, I32, I32]
    lib.hs2_v1_full_attn_select.restype = I32
    lib.hs2_v1_full_attn_select.argtypes = [SP, P, P, P, I32, I32, I32, I32, F, P, P, P, P, P, SZ, I32, P]
    lib.hs2_v1_sparse_attn_workspace_size.restype = SZ
    lib.hs2_v1_sparse_attn_workspace_size.argtypes = [SP, I32, I32, I32, I32, I32]
    lib.hs2_v1_sparse_attn.restype = I32
    lib.hs2_v1_sparse_attn.argtypes = [SP, P, P, P, P, I32, P, P, I32, I32, P, P, I32, I32, I32, F, P, P, SZ, I32, P]
    _lib = lib
    return lib


def _check(st: int) -> None:
    if st != HS2_OK:
        raise HS2Error(st, load().hs2_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HS2_BF16
    if t.dtype == torch.float32:
        return HS2_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _expect(name: str, t, dtypes, inner: tuple, min_rows: int, device=None) -> None:
    """Rejects a tensor that the library would read or write through its plain pointer with
    another element type, row length or row count than the entry point assumes (the C ABI
    sees no buffer sizes, so a mismatch would be an out-of-bounds access on the device)."""
    if t is None:
        return
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {', '.join(str(d) for d in dtypes)}")
    if tuple(t.shape[1:]) != tuple(inner) or t.dim() != 1 + len(inner):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected [rows, {', '.join(map(str, inner))}]")
    if t.shape[0] < min_rows:
        raise ValueError(f"{name}: {t.shape[0]} rows, the batch addresses {min_rows}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_attn_args(batch: "Batch", q, k, v, kv_dtypes, q_dtypes=(torch.bfloat16, torch.float32),
                     kv_inner=(128,), out=None, lse=None) -> None:
    """Q [total_q, 64, 128], K and V [total_kv_rows, *kv_inner], outputs like Q / [total_q, 64]."""
    _expect("q", q, q_dtypes, (64, 128), batch.total_q)
    _expect("k", k, kv_dtypes, kv_inner, batch.total_kv_rows, q.device)
    _expect("v", v, kv_dtypes, kv_inner, batch.total_kv_rows, q.device)
    _expect("out", out, (q.dtype,), (64, 128), batch.total_q, q.device)
    _expect("lse", lse, (torch.float32,), (64,), batch.total_q, q.device)


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


@dataclass
class Batch:
    """A ragged batch: device descriptor arrays plus the host sizes the library needs."""

    kv_start: torch.Tensor   # int64 [S]
    kv_len: torch.Tensor     # int32 [S]
    q_start: torch.Tensor    # int32 [S+1]
    q_pos: torch.Tensor      # int32 [total_q]
    total_q: int
    max_kv_len: int
    total_kv_rows: int
    max_q_per_seq: int
    kv_len_host: Optional[np.ndarray] = None   # int32 [S], contiguous: balances the key split

    def c(self) -> hs2_seqs:
        kh = None
        if self.kv_len_host is not None:
            assert self.kv_len_host.dtype == np.int32 and self.kv_len_host.flags["C_CONTIGUOUS"]
            assert self.kv_len_host.size == self.kv_start.numel()
            kh = self.kv_len_host.ctypes.data
        return hs2_seqs(int(self.kv_start.numel()), _ptr(self.kv_start), _ptr(self.kv_len), _ptr(self.q_start),
                        _ptr(self.q_pos), int(self.total_q), int(self.max_kv_len), int(self.total_kv_rows),
                        int(self.max_q_per_seq), kh)

    @staticmethod
    def from_host(kv_start, kv_len, q_start, q_pos, total_kv_rows: int, device="cuda") -> "Batch":
        """Builds the device descriptor from host sequences (numpy or lists)."""
        ks = torch.as_tensor(kv_start, dtype=torch.int64)
        kl = torch.as_tensor(kv_len, dtype=torch.int32)
        qs = torch.as_tensor(q_start, dtype=torch.int32)
        qp = torch.as_tensor(q_pos, dtype=torch.int32)
        per = (qs[1:] - qs[:-1]) if qs.numel() > 1 else torch.zeros(1, dtype=torch.int32)
        return Batch(ks.to(device), kl.to(device), qs.to(device), qp.to(device), int(qp.numel()),
                     max(1, int(kl.max().item()) if kl.numel() else 1), int(total_kv_rows),
                     int(per.max().item()) if per.numel() else 0,
                     np.ascontiguousarray(kl.numpy(), dtype=np.int32))


def _size_code(dtype) -> int:
    """dtype code of a workspace size query: torch.bfloat16, torch.float32 or "fp8" (FP8 K/V)."""
    if isinstance(dtype, str) and dtype == "fp8":
        return HS2_FP8_E4M3
    return HS2_BF16 if dtype == torch.bfloat16 else HS2_F32


def full_attn_select_workspace_size(batch: Batch, window: int, top_k: int, dtype=torch.bfloat16) -> int:
    b = batch.c()
    return int(load().hs2_full_attn_select_workspace_size(ctypes.byref(b), 64, 128, window, top_k,
                                                          _size_code(dtype)))


def sparse_attn_workspace_size(batch: Batch, window: int, top_k: int, dtype=torch.bfloat16) -> int:
    b = batch.c()
    return int(load().hs2_sparse_attn_workspace_size(ctypes.byref(b), 64, 128, window, top_k, _size_code(dtype)))


def bridge_kv_workspace_size(d_model: int, n_layers: int, head_dim: int = 128) -> int:
    return int(load().hs2_bridge_kv_workspace_size(d_model, n_layers, head_dim))


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def full_attn_select(batch: Batch, q, k, v, window: int = 128, top_k: int = 1024, scale: float | None = None,
                     out=None, lse=None, sel_idx=None, sel_count=None, workspace=None, stream=None,
                     want_lse: bool = True):
    """hs2_full_attn_select: exact causal MQA attention plus top-k selection per query.

    Returns (out [total_q, 64, 128], lse [total_q, 64] or None, sel_idx [total_q, top_k], sel_count [total_q]).
    """
    lib = load()
    dt = _dtype_code(q)
    _check_attn_args(batch, q, k, v, (q.dtype,), out=out, lse=lse)
    _expect("sel_idx", sel_idx, (torch.int32,), (max(top_k, 0),), batch.total_q, q.device)
    _expect("sel_count", sel_count, (torch.int32,), (), batch.total_q, q.device)
    scale = float(scale if scale is not None else q.shape[-1] ** -0.5)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(batch.total_q, 64, dtype=torch.float32, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty(batch.total_q, max(top_k, 0), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty(batch.total_q, dtype=torch.int32, device=dev)
    b = batch.c()
    need = lib.hs2_full_attn_select_workspace_size(ctypes.byref(b), 64, 128, window, top_k, dt)
    if workspace is None:
        workspace = _workspace(need, dev)
    _check(lib.hs2_full_attn_select(ctypes.byref(b), _ptr(q), _ptr(k), _ptr(v), q.shape[1], q.shape[2], window,
                                    top_k, scale, _ptr(out), _ptr(lse), _ptr(sel_idx) if top_k > 0 else None,
                                    _ptr(sel_count), _ptr(workspace), workspace.numel(), dt, _stream(stream)))
    return out, lse, sel_idx, sel_count


def sparse_attn(batch: Batch, q, k, v, sel_idx, window: int = 128, top_k: int | None = None,
                scale: float | None = None, out=None, lse=None, workspace=None, stream=None):
    """hs2_sparse_attn: attention over the window plus the selected rows. Returns (out, lse)."""
    lib = load()
    dt = _dtype_code(q)
    if top_k is None:
        top_k = sel_idx.shape[1] if sel_idx is not None else 0
    _check_attn_args(batch, q, k, v, (q.dtype,), out=out, lse=lse)
    _expect("sel_idx", sel_idx if top_k > 0 else None, (torch.int32,), (top_k,), batch.total_q, q.device)
    scale = float(scale if scale is not None else q.shape[-1] ** -0.5)
    if out is None:
        out = torch.empty_like(q)
    b = batch.c()
    need = lib.hs2_sparse_attn_workspace_size(ctypes.byref(b), 64, 128, window, top_k, dt)
    if workspace is None:
        workspace = _workspace(need, q.device)
    _check(lib.hs2_sparse_attn(ctypes.byref(b), _ptr(q), _ptr(k), _ptr(v), _ptr(sel_idx) if top_k > 0 else None,
                               q.shape[1], q.shape[2], window, top_k, scale, _ptr(out), _ptr(lse), _ptr(workspace),
                               workspace.numel(), dt, _stream(stream)))
    return out, lse


NOALLOC_SCRATCH_BYTES = 16 << 20


def sparse_attn_noalloc(batch: Batch, q, k, v, sel_idx, window: int = 128, top_k: int | None = None,
                        scale: float | None = None, out=None, lse=None, stream=None):
    """hs2_sparse_attn_noalloc: the sparse layer with its split partials in the library's
    fixed per-GPU scratch array (no workspace argument). Returns (out, lse)."""
    lib = load()
    dt = _dtype_code(q)
    if top_k is None:
        top_k = sel_idx.shape[1] if sel_idx is not None else 0
    _check_attn_args(batch, q, k, v, (q.dtype,), out=out, lse=lse)
    _expect("sel_idx", sel_idx if top_k > 0 else None, (torch.int32,), (top_k,), batch.total_q, q.device)
    scale = float(scale if scale is not None else q.shape[-1] ** -0.5)
    if out is None:
        out = torch.empty_like(q)
    b = batch.c()
    _check(lib.hs2_sparse_attn_noalloc(ctypes.byref(b), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(sel_idx) if top_k > 0 else None, q.shape[1], q.shape[2], window, top_k,
                                       scale, _ptr(out), _ptr(lse), dt, _stream(stream)))
    return out, lse


def bridge_kv(hidden, w_k: list, w_v: list, k_out: list | None = None, v_out: list | None = None,
              workspace=None, stream=None):
    """hs2_bridge_kv: K_l = H W_K^l, V_l = H W_V^l for every layer, one pass over H."""
    lib = load()
    n_rows, d_model = hidden.shape
    L = len(w_k)
    head_dim = w_k[0].shape[1]
    _expect("hidden", hidden, (torch.bfloat16,), (d_model,), n_rows)
    if len(w_v) != L or (k_out is not None and len(k_out) != L) or (v_out is not None and len(v_out) != L):
        raise ValueError("w_k, w_v, k_out and v_out must hold one tensor per layer")
    for name, ts in (("w_k", w_k), ("w_v", w_v)):
        for t in ts:
            _expect(name, t, (hidden.dtype,), (head_dim,), d_model, hidden.device)
    for name, ts in (("k_out", k_out or []), ("v_out", v_out or [])):
        for t in ts:
            _expect(name, t, (hidden.dtype,), (head_dim,), n_rows, hidden.device)
    if k_out is None:
        k_out = [torch.empty(n_rows, head_dim, dtype=hidden.dtype, device=hidden.device) for _ in range(L)]
    if v_out is None:
        v_out = [torch.empty(n_rows, head_dim, dtype=hidden.dtype, device=hidden.device) for _ in range(L)]
    arr = ctypes.c_void_p * L
    wk = arr(*[w.data_ptr() for w in w_k])
    wv = arr(*[w.data_ptr() for w in w_v])
    ko = arr(*[t.data_ptr() for t in k_out])
    vo = arr(*[t.data_ptr() for t in v_out])
    need = lib.hs2_bridge_kv_workspace_size(d_model, L, head_dim)
    if workspace is None:
        workspace = _workspace(need, hidden.device)
    _check(lib.hs2_bridge_kv(_ptr(hidden), n_rows, d_model, L, wk, wv, ko, vo, head_dim, _ptr(workspace),
                             workspace.numel(), _dtype_code(hidden), _stream(stream)))
    return k_out, v_out


def bridge_kv_fp8kv(hidden, w_k: list, w_v: list, k_scale, v_scale, k_out: list | None = None,
                    v_out: list | None = None, workspace=None, stream=None):
    """hs2_bridge_kv_fp8kv: the bridging projections written as FP8 E4M3 caches (uint8 codes
    [n_rows, 128] per layer) with one scale per tensor; k_scale and v_scale are one float
    for every layer or a list with one per layer."""
    lib = load()
    n_rows, d_model = hidden.shape
    L = len(w_k)
    head_dim = w_k[0].shape[1]
    ks = [float(k_scale)] * L if isinstance(k_scale, (int, float)) else [float(x) for x in k_scale]
    vs = [float(v_scale)] * L if isinstance(v_scale, (int, float)) else [float(x) for x in v_scale]
    _expect("hidden", hidden, (torch.bfloat16,), (d_model,), n_rows)
    if len(w_v) != L or len(ks) != L or len(vs) != L or (k_out is not None and len(k_out) != L) or \
            (v_out is not None and len(v_out) != L):
        raise ValueError("w_k, w_v, the scales, k_out and v_out must hold one entry per layer")
    for name, ts in (("w_k", w_k), ("w_v", w_v)):
        for t in ts:
            _expect(name, t, (torch.bfloat16,), (head_dim,), d_model, hidden.device)
    for name, ts in (("k_out", k_out or []), ("v_out", v_out or [])):
        for t in ts:
            _expect(name, t, (torch.uint8, torch.float8_e4m3fn), (head_dim,), n_rows, hidden.device)
    if k_out is None:
        k_out = [torch.empty(n_rows, head_dim, dtype=torch.uint8, device=hidden.device) for _ in range(L)]
    if v_out is None:
        v_out = [torch.empty(n_rows, head_dim, dtype=torch.uint8, device=hidden.device) for _ in range(L)]
    arr = ctypes.c_void_p * L
    farr = ctypes.c_float * L
    need = lib.hs2_bridge_kv_workspace_size(d_model, L, head_dim)
    if workspace is None:
        workspace = _workspace(need, hidden.device)
    _check(lib.hs2_bridge_kv_fp8kv(_ptr(hidden), n_rows, d_model, L, arr(*[w.data_ptr() for w in w_k]),
                                   arr(*[w.data_ptr() for w in w_v]), arr(*[t.data_ptr() for t in k_out]),
                                   arr(*[t.data_ptr() for t in v_out]), farr(*ks), farr(*vs), head_dim,
                                   _ptr(workspace), workspace.numel(), _stream(stream)))
    return k_out, v_out


def set_kernel_events(events: list | None) -> None:
    """hs2_set_kernel_events: bracket each kernel of later calls with HIP events.

    `events` is a flat list of hipEvent_t handles (ints), two per kernel, or None."""
    lib = load()
    if not events:
        _check(lib.hs2_set_kernel_events(None, 0))
        return
    arr = (ctypes.c_void_p * len(events))(*events)
    set_kernel_events._keep = arr
    _check(lib.hs2_set_kernel_events(arr, len(events) // 2))


def _fp8_codes(t: torch.Tensor) -> torch.Tensor:
    if t.element_size() != 1 or t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"FP8 K/V must be uint8 codes or torch.float8_e4m3fn (got {t.dtype})")
    return t


def full_attn_select_fp8kv(batch: Batch, q, k, v, k_scale: float, v_scale: float, window: int = 128,
                           top_k: int = 1024, scale: float | None = None, out=None, lse=None, sel_idx=None,
                           sel_count=None, workspace=None, stream=None, want_lse: bool = True):
    """hs2_full_attn_select_fp8kv: the selector on an OCP FP8 E4M3 K/V cache with per-tensor
    scales (q and out bf16). Returns (out, lse or None, sel_idx, sel_count)."""
    lib = load()
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16")
    k, v = _fp8_codes(k), _fp8_codes(v)
    _check_attn_args(batch, q, k, v, (k.dtype,), q_dtypes=(torch.bfloat16,), out=out, lse=lse)
    _expect("sel_idx", sel_idx, (torch.int32,), (max(top_k, 0),), batch.total_q, q.device)
    _expect("sel_count", sel_count, (torch.int32,), (), batch.total_q, q.device)
    scale = float(scale if scale is not None else q.shape[-1] ** -0.5)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(batch.total_q, 64, dtype=torch.float32, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty(batch.total_q, max(top_k, 0), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty(batch.total_q, dtype=torch.int32, device=dev)
    b = batch.c()
    need = lib.hs2_full_attn_select_workspace_size(ctypes.byref(b), 64, 128, window, top_k, HS2_FP8_E4M3)
    if workspace is None:
        workspace = _workspace(need, dev)
    _check(lib.hs2_full_attn_select_fp8kv(ctypes.byref(b), _ptr(q), _ptr(k), _ptr(v), float(k_scale), float(v_scale),
                                          q.shape[1], q.shape[2], window, top_k, scale, _ptr(out), _ptr(lse),
                                          _ptr(sel_idx) if top_k > 0 else None, _ptr(sel_count), _ptr(workspace),
                                          workspace.numel(), _stream(stream)))
    return out, lse, sel_idx, sel_count


def sparse_attn_fp8kv(batch: Batch, q, k, v, k_scale: float, v_scale: float, sel_idx, window: int = 128,
                      top_k: int | None = None, scale: float | None = None, out=None, lse=None, workspace=None,
                      stream=None):
    """hs2_sparse_attn_fp8kv: a sparse layer on the selector's FP8 E4M3 K/V cache. Returns (out, lse)."""
    lib = load()
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16")
    k, v = _fp8_codes(k), _fp8_codes(v)
    if top_k is None:
        top_k = sel_idx.shape[1] if sel_idx is not None else 0
    _check_attn_args(batch, q, k, v, (k.dtype,), q_dtypes=(torch.bfloat16,), out=out, lse=lse)
    _expect("sel_idx", sel_idx if top_k > 0 else None, (torch.int32,), (top_k,), batch.total_q, q.device)
    scale = float(scale if scale is not None else q.shape[-1] ** -0.5)
    if out is None:
        out = torch.empty_like(q)
    b = batch.c()
    need = lib.hs2_sparse_attn_workspace_size(ctypes.byref(b), 64, 128, window, top_k, HS2_FP8_E4M3)
    if workspace is None:
        workspace = _workspace(need, q.device)
    _check(lib.hs2_sparse_attn_fp8kv(ctypes.byref(b), _ptr(q), _ptr(k), _ptr(v), float(k_scale), float(v_scale),
                                     _ptr(sel_idx) if top_k > 0 else None, q.shape[1], q.shape[2], window, top_k,
                                     scale, _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                     _stream(stream)))
    return out, lse


def causal_attn_workspace_size(batch: Batch, dtype=torch.bfloat16) -> int:
    b = batch.c()
    return int(load().hs2_causal_attn_workspace_size(ctypes.byref(b), 64, 128, _size_code(dtype)))


def causal_attn(batch: Batch, q, k, v, scale: float | None = None, out=None, lse=None, workspace=None, stream=None,
                want_lse: bool = True):
    """hs2_causal_attn: exact causal attention of every query (prefill, no selection).
    Returns (out [total_q, 64, 128], lse [total_q, 64] or None)."""
    lib = load()
    dt = _dtype_code(q)
    _check_attn_args(batch, q, k, v, (q.dtype,), out=out, lse=lse)
    scale = float(scale if scale is not None else q.shape[-1] ** -0.5)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(batch.total_q, 64, dtype=torch.float32, device=q.device)
    b = batch.c()
    need = lib.hs2_causal_attn_workspace_size(ctypes.byref(b), 64, 128, dt)
    if workspace is None:
        workspace = _workspace(need, q.device)
    _check(lib.hs2_causal_attn(ctypes.byref(b), _ptr(q), _ptr(k), _ptr(v), q.shape[1], q.shape[2], scale, _ptr(out),
                               _ptr(lse), _ptr(workspace), workspace.numel(), dt, _stream(stream)))
    return out, lse


def bridge_kv_append_workspace_size(n_new: int, d_model: int, n_layers: int, head_dim: int = 128) -> int:
    return int(load().hs2_bridge_kv_append_workspace_size(n_new, d_model, n_layers, head_dim))


def bridge_kv_append(h, rows, w_k, w_v, k_cache, v_cache, workspace=None, stream=None):
    """hs2_bridge_kv_append: K_l[rows[i]] = h_i W_K^l and V_l[rows[i]] = h_i W_V^l, written in
    place into the caches (h [n_new, d_model] bf16, rows int64 [n_new] on the device)."""
    lib = load()
    n_layers = len(w_k)
    n_new, d_model = int(h.shape[0]), int(h.shape[1])
    assert rows.dtype == torch.int64 and rows.numel() == n_new
    cache_rows = int(k_cache[0].shape[0])
    assert all(int(c.shape[0]) == cache_rows for c in list(k_cache) + list(v_cache))
    _expect("h", h, (torch.bfloat16,), (d_model,), n_new)
    if len(w_v) != n_layers or len(k_cache) != n_layers or len(v_cache) != n_layers:
        raise ValueError("w_k, w_v, k_cache and v_cache must hold one tensor per layer")
    for name, ts in (("w_k", w_k), ("w_v", w_v)):
        for t in ts:
            _expect(name, t, (torch.bfloat16,), (128,), d_model, h.device)
    for name, ts in (("k_cache", k_cache), ("v_cache", v_cache)):
        for t in ts:
            _expect(name, t, (torch.bfloat16,), (128,), cache_rows, h.device)
    arr = ctypes.c_void_p * n_layers
    need = lib.hs2_bridge_kv_append_workspace_size(n_new, d_model, n_layers, 128)
    if workspace is None:
        workspace = _workspace(need, h.device)
    _check(lib.hs2_bridge_kv_append(_ptr(h), n_new, _ptr(rows), cache_rows, d_model, n_layers,
                                    arr(*[w.data_ptr() for w in w_k]), arr(*[w.data_ptr() for w in w_v]),
                                    arr(*[c.data_ptr() for c in k_cache]), arr(*[c.data_ptr() for c in v_cache]),
                                    128, _ptr(workspace), workspace.numel(), HS2_BF16, _stream(stream)))


def bridge_kv_append_fp8kv(h, rows, w_k, w_v, k_cache, v_cache, k_scale, v_scale, workspace=None, stream=None):
    """hs2_bridge_kv_append_fp8kv: the new tokens' K/V rows written as E4M3 codes into FP8
    caches (uint8 [cache_rows, 128]); k_scale and v_scale are one float for every layer or
    a list with one per layer."""
    lib = load()
    n_layers = len(w_k)
    n_new, d_model = int(h.shape[0]), int(h.shape[1])
    assert rows.dtype == torch.int64 and rows.numel() == n_new
    ks = [float(k_scale)] * n_layers if isinstance(k_scale, (int, float)) else [float(x) for x in k_scale]
    vs = [float(v_scale)] * n_layers if isinstance(v_scale, (int, float)) else [float(x) for x in v_scale]
    if len(w_v) != n_layers or len(k_cache) != n_layers or len(v_cache) != n_layers or len(ks) != n_layers or \
            len(vs) != n_layers:
        raise ValueError("w_k, w_v, k_cache, v_cache and the scales must hold one entry per layer")
    cache_rows = int(k_cache[0].shape[0])
    _expect("h", h, (torch.bfloat16,), (d_model,), n_new)
    for name, ts in (("w_k", w_k), ("w_v", w_v)):
        for t in ts:
            _expect(name, t, (torch.bfloat16,), (128,), d_model, h.device)
    for name, ts in (("k_cache", k_cache), ("v_cache", v_cache)):
        for t in ts:
            _expect(name, t, (torch.uint8, torch.float8_e4m3fn), (128,), cache_rows, h.device)
            if int(t.shape[0]) != cache_rows:
                raise ValueError("every cache must have the same number of rows")
    arr = ctypes.c_void_p * n_layers
    farr = ctypes.c_float * n_layers
    need = lib.hs2_bridge_kv_append_workspace_size(n_new, d_model, n_layers, 128)
    if workspace is None:
        workspace = _workspace(need, h.device)
    _check(lib.hs2_bridge_kv_append_fp8kv(_ptr(h), n_new, _ptr(rows), cache_rows, d_model, n_layers,
                                          arr(*[w.data_ptr() for w in w_k]), arr(*[w.data_ptr() for w in w_v]),
                                          arr(*[c.data_ptr() for c in k_cache]), arr(*[c.data_ptr() for c in v_cache]),
                                          farr(*ks), farr(*vs), 128, _ptr(workspace), workspace.numel(),
                                          _stream(stream)))


# ------------------------------------------------------------------------------------
# First-generation HySparse layout (the comparison variant): GQA 64:4, 64-token block
# selection per KV head, gated sliding-window branch.
# ------------------------------------------------------------------------------------
V1_KV_HEADS = 4


def v1_full_attn_select_workspace_size(batch: Batch, top_blocks: int = 16) -> int:
    b = batch.c()
    return int(load().hs2_v1_full_attn_select_workspace_size(ctypes.byref(b), 64, V1_KV_HEADS, 128, top_blocks,
                                                             HS2_BF16))


def v1_full_attn_select(batch: Batch, q, k, v, top_blocks: int = 16, scale: float | None = None, out=None,
                        lse=None, blk_idx=None, blk_count=None, workspace=None, stream=None, want_lse: bool = True):
    """hs2_v1_full_attn_select: exact causal GQA attention (k, v [rows, 4, 128]) plus the
    top_blocks 64-token blocks of each KV head.

    Returns (out [total_q, 64, 128], lse [total_q, 64] or None, blk_idx [total_q, 4, top_blocks],
    blk_count [total_q, 4]).
    """
    lib = load()
    _check_attn_args(batch, q, k, v, (q.dtype,), q_dtypes=(torch.bfloat16,), kv_inner=(V1_KV_HEADS, 128), out=out,
                     lse=lse)
    scale = float(scale if scale is not None else q.shape[-1] ** -0.5)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(batch.total_q, 64, dtype=torch.float32, device=dev)
    if blk_idx is None:
        blk_idx = torch.empty(batch.total_q, V1_KV_HEADS, top_blocks, dtype=torch.int32, device=dev)
    if blk_count is None:
        blk_count = torch.empty(batch.total_q, V1_KV_HEADS, dtype=torch.int32, device=dev)
    b = batch.c()
    need = lib.hs2_v1_full_attn_select_workspace_size(ctypes.byref(b), 64, V1_KV_HEADS, 128, top_blocks, HS2_BF16)
    if workspace is None:
        workspace = _workspace(need, dev)
    _check(lib.hs2_v1_full_attn_select(ctypes.byref(b), _ptr(q), _ptr(k), _ptr(v), q.shape[1],
                                       k.shape[1] if k.dim() == 3 else V1_KV_HEADS, q.shape[2], top_blocks, scale,
                                       _ptr(out), _ptr(lse), _ptr(blk_idx), _ptr(blk_count), _ptr(workspace),
                                       workspace.numel(), _dtype_code(q), _stream(stream)))
    return out, lse, blk_idx, blk_count


def v1_sparse_attn_workspace_size(batch: Batch, top_blocks: int = 16) -> int:
    b = batch.c()
    return int(load().hs2_v1_sparse_attn_workspace_size(ctypes.byref(b), 64, V1_KV_HEADS, 128, top_blocks,
                                                        HS2_BF16))


def v1_sparse_attn(batch: Batch, q, k, v, blk_idx, k_swa, v_swa, gate_sparse, gate_swa, window: int = 128,
                   scale: float | None = None, out=None, workspace=None, stream=None):
    """hs2_v1_sparse_attn: selected-block branch on the shared cache plus the window branch
    on the layer's own ring cache k_swa, v_swa [num_seqs, swa_slots, 4, 128], fused by the
    gates [total_q, 64]. Returns out [total_q, 64, 128]."""
    lib = load()
    top_blocks = blk_idx.shape[-1]
    _check_attn_args(batch, q, k, v, (q.dtype,), q_dtypes=(torch.bfloat16,), kv_inner=(V1_KV_HEADS, 128), out=out)
    _expect("blk_idx", blk_idx, (torch.int32,), (V1_KV_HEADS, top_blocks), batch.total_q, q.device)
    for name, t in (("gate_sparse", gate_sparse), ("gate_swa", gate_swa)):
        _expect(name, t, (torch.float32,), (64,), batch.total_q, q.device)
    scale = float(scale if scale is not None else q.shape[-1] ** -0.5)
    if out is None:
        out = torch.empty_like(q)
    b = batch.c()
    need = lib.hs2_v1_sparse_attn_workspace_size(ctypes.byref(b), 64, V1_KV_HEADS, 128, top_blocks, HS2_BF16)
    if workspace is None:
        workspace = _workspace(need, q.device)
    _check(lib.hs2_v1_sparse_attn(ctypes.byref(b), _ptr(q), _ptr(k), _ptr(v), _ptr(blk_idx), top_blocks,
                                  _ptr(k_swa), _ptr(v_swa), k_swa.shape[1], window, _ptr(gate_sparse),
                                  _ptr(gate_swa), q.shape[1], k.shape[1] if k.dim() == 3 else V1_KV_HEADS,
                                  q.shape[2], scale, _ptr(out), _ptr(workspace), workspace.numel(),
                                  _dtype_code(q), _stream(stream)))
    return out
