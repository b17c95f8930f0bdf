"""Python binding of libsas (SAS gated block-sparse attention on MI355X).

Thin ctypes layer over the C ABI declared in include/sas.h: it checks tensor
dtypes, shapes, contiguity and devices, allocates outputs and workspaces with
torch, and passes raw device pointers plus the current HIP stream.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback path.  Importing works without a GPU (so the CPU tests can check the
exported symbols); calling any compute function requires the built library
and a visible GPU and raises otherwise.
"""
from __future__ import annotations

import ctypes
import math
import os
import warnings

import torch

__all__ = [
    "Dims", "DecodeDims", "SasError", "load_library", "version", "workspace_size",
    "decode_workspace_size", "gate_score", "topk_blocks", "sparse_attn_fwd",
    "sparse_attn_bwd", "decode", "decode_paged", "decode_gate_key", "budget_to_topk",
    "EXPORTED_SYMBOLS",
    "set_timing_events",
    "take_device_fault", "gate_score_bwd", "decode_noalloc",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsas.so")

SAS_OK, SAS_ERR_INVALID, SAS_ERR_UNSUPPORTED, SAS_ERR_WORKSPACE, SAS_ERR_HIP = range(5)
FLAG_GATE_PER_QUERY_HEAD = 1
OP_GATE_SCORE, OP_TOPK, OP_FWD, OP_BWD, OP_GATE_BWD, OP_WALK_ORDER = range(6)

EXPORTED_SYMBOLS = (
    "sas_version", "sas_last_error", "sas_workspace_size", "sas_decode_workspace_size",
    "sas_gate_score", "sas_topk_blocks", "sas_sparse_attn_fwd", "sas_sparse_attn_bwd",
    "sas_decode", "sas_set_timing_events", "sas_take_device_fault", "sas_gate_score_bwd",
    "sas_decode_paged", "sas_decode_gate_key", "sas_decode_noalloc", "sas_walk_order",
)


class SasError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libsas status {status}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("dg", ctypes.c_int32),
                ("block", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("norm_eps", ctypes.c_float),
                ("flags", ctypes.c_int32)]


class DecodeDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("D", ctypes.c_int32), ("dg", ctypes.c_int32), ("block", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("Lmax", ctypes.c_int32), ("NBmax", ctypes.c_int32),
                ("apply_gate", ctypes.c_int32), ("kg_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsas.so (built by gated_block_sparse_gate_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libsas.so not found at {path}; build it with "
                           "`python -m gated_block_sparse_gate_amd.build`")
    lib = ctypes.CDLL(path)
    P, S, I32, F32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
    lib.sas_version.restype = I32
    lib.sas_last_error.restype = ctypes.c_char_p
    lib.sas_workspace_size.argtypes = [I32, ctypes.POINTER(Dims)]
    lib.sas_workspace_size.restype = S
    lib.sas_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeDims)]
    lib.sas_decode_workspace_size.restype = S
    lib.sas_gate_score.argtypes = [ctypes.POINTER(Dims)] + [P] * 8 + [P, S, P]
    lib.sas_topk_blocks.argtypes = [ctypes.POINTER(Dims)] + [P] * 6 + [P, S, P]
    lib.sas_gate_score_bwd.argtypes = [ctypes.POINTER(Dims)] + [P] * 16 + [P, S, P]
    lib.sas_sparse_attn_fwd.argtypes = [ctypes.POINTER(Dims)] + [P] * 5 + [F32] + [P] * 3 + [P, S, P]
    lib.sas_sparse_attn_bwd.argtypes = ([ctypes.POINTER(Dims)] + [P] * 9 + [F32] + [P] * 4
                                        + [P, S, P])
    lib.sas_decode.argtypes = ([ctypes.POINTER(DecodeDims)] + [P] * 6 + [F32] + [P] * 3
                               + [P, S, P])
    lib.sas_decode_noalloc.argtypes = ([ctypes.POINTER(DecodeDims)] + [P] * 6 + [F32] + [P] * 3
                                       + [P])
    lib.sas_decode_paged.argtypes = ([ctypes.POINTER(DecodeDims)] + [P] * 5 + [I32] + [P] * 2
                                     + [F32] + [P] * 3 + [P, S, P])
    lib.sas_decode_gate_key.argtypes = ([ctypes.POINTER(DecodeDims)] + [P, P, I32, P, P]
                                        + [ctypes.c_double, F32] + [P, P, P])
    lib.sas_walk_order.argtypes = [ctypes.POINTER(Dims), P, P, S, P]
    lib.sas_set_timing_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), I32]
    lib.sas_take_device_fault.argtypes = [ctypes.POINTER(ctypes.c_uint)]
    for fn in ("sas_gate_score", "sas_gate_score_bwd", "sas_topk_blocks", "sas_sparse_attn_fwd",
               "sas_sparse_attn_bwd", "sas_decode", "sas_decode_paged", "sas_decode_gate_key",
               "sas_decode_noalloc", "sas_walk_order",
               "sas_set_timing_events",
               "sas_take_device_fault"):
        getattr(lib, fn).restype = I32
    _lib = lib
    return lib


def version() -> int:
    return load_library().sas_version()


def _check(st: int):
    if st != SAS_OK:
        raise SasError(st, load_library().sas_last_error().decode())


def make_dims(B, T, Hq, Hkv, D, dg, topk, theta=1.0e6, eps=1.0e-6, block=64, flags=0) -> Dims:
    return Dims(B, T, Hq, Hkv, D, dg, block, topk, float(theta), float(eps), flags)


def _sel_flags(Hs, Hq, Hkv, what):
    """Gate mode from the number of selection heads of a gate-side tensor:
    Hkv (one gate per KV head) or Hq (one gate per query head)."""
    if Hs == Hkv:
        return 0
    if Hs == Hq:
        return FLAG_GATE_PER_QUERY_HEAD
    raise ValueError(f"{what}: {Hs} gate heads; expected Hkv = {Hkv} (one gate per KV head) "
                     f"or Hq = {Hq} (one gate per query head)")


def workspace_size(op: int, d: Dims) -> int:
    n = load_library().sas_workspace_size(op, ctypes.byref(d))
    if n == ctypes.c_size_t(-1).value:
        raise SasError(SAS_ERR_INVALID, load_library().sas_last_error().decode())
    return n


def decode_workspace_size(d: DecodeDims) -> int:
    n = load_library().sas_decode_workspace_size(ctypes.byref(d))
    if n == ctypes.c_size_t(-1).value:
        raise SasError(SAS_ERR_INVALID, load_library().sas_last_error().decode())
    return n


def set_timing_events(events=None):
    """Record the given torch.cuda.Event objects at the stage boundaries of the
    following sparse_attn_fwd / sparse_attn_bwd calls on this thread (see
    sas_set_timing_events in sas.h); None or [] switches the hook off."""
    lib = load_library()
    if not events:
        _check(lib.sas_set_timing_events(None, 0))
        return
    handles = []
    for e in events:
        if not e.cuda_event:          # torch creates the event on first record
            e.record()
        handles.append(e.cuda_event)
    arr = (ctypes.c_void_p * len(handles))(*handles)
    _check(lib.sas_set_timing_events(arr, len(handles)))


def take_device_fault() -> int:
    """Read and clear the attention kernels' fault flag (see
    sas_take_device_fault in sas.h); 0 means no fault.  Synchronises."""
    v = ctypes.c_uint(0)
    _check(load_library().sas_take_device_fault(ctypes.byref(v)))
    return v.value


def budget_to_topk(budget: int, block: int = 64) -> int:
    """Decode token budget (counts the current block) -> historical Top-K."""
    if budget < block or budget % block:
        raise ValueError("budget must be a positive multiple of the block size")
    return budget // block - 1


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _req(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ws(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _device_of(t):
    if t.device.type != "cuda":
        raise ValueError("libsas tensors must live on a GPU device")
    return t.device


def gate_score(q, k, wq, wk, w_qn, w_kn, topk: int, theta: float = 1.0e6, eps: float = 1.0e-6,
               q_gate=None, k_gate=None, workspace=None, per_query_head: bool = False):
    """Router: returns (q_gate [B,T,Hs,dg], k_gate [B,T,Hkv,dg]) fp32, with
    Hs = Hkv (wq [Hkv,G*D,dg]) or, per_query_head, Hs = Hq (wq [Hq,D,dg])."""
    lib = load_library()
    dev = _device_of(q)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    dg = wq.shape[2]
    G = Hq // Hkv
    Hs, Gs = (Hq, 1) if per_query_head else (Hkv, G)
    _req(q, "q", torch.bfloat16, (B, T, Hq, D), dev)
    _req(k, "k", torch.bfloat16, (B, T, Hkv, D), dev)
    _req(wq, "wq", torch.bfloat16, (Hs, Gs * D, dg), dev)
    _req(wk, "wk", torch.bfloat16, (Hkv, 3 * D, dg), dev)
    _req(w_qn, "w_qn", torch.float32, (dg,), dev)
    _req(w_kn, "w_kn", torch.float32, (dg,), dev)
    d = make_dims(B, T, Hq, Hkv, D, dg, topk, theta, eps,
                  flags=FLAG_GATE_PER_QUERY_HEAD if per_query_head else 0)
    if q_gate is None:
        q_gate = torch.empty((B, T, Hs, dg), dtype=torch.float32, device=dev)
    if k_gate is None:
        k_gate = torch.empty((B, T, Hkv, dg), dtype=torch.float32, device=dev)
    _req(q_gate, "q_gate", torch.float32, (B, T, Hs, dg), dev)
    _req(k_gate, "k_gate", torch.float32, (B, T, Hkv, dg), dev)
    nws = workspace_size(OP_GATE_SCORE, d)
    ws = workspace if workspace is not None else _ws(nws, dev)
    _check(lib.sas_gate_score(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(wq), _ptr(wk), _ptr(w_qn),
                              _ptr(w_kn), _ptr(q_gate), _ptr(k_gate), _ptr(ws),
                              ws.numel() if ws is not None else 0, _stream(dev)))
    return q_gate, k_gate


def gate_score_bwd(q, k, wq, wk, w_qn, w_kn, q_gate, k_gate, idx, dlogg, theta: float = 1.0e6,
                   eps: float = 1.0e-6, workspace=None, check_row_sums: bool = True,
                   row_sum_tol: float = 1e-3):
    """Router backward: returns dict of fp32 dq, dk, dwq, dwk, dw_qn, dw_kn from
    dlogg (as the attention backward gives it) with the selection idx fixed.
    With check_row_sums, warns when a row of dlogg does not sum to zero within
    row_sum_tol (the library then returns the gradient with each row's gate
    lse held constant; see sas_gate_score_bwd in sas.h).  The check reads
    dlogg back and synchronises; pass check_row_sums=False in timed loops."""
    lib = load_library()
    dev = _device_of(q)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    dg = wq.shape[2]
    G = Hq // Hkv
    S = idx.shape[-1]
    _req(q, "q", torch.bfloat16, (B, T, Hq, D), dev)
    _req(k, "k", torch.bfloat16, (B, T, Hkv, D), dev)
    _req(wq, "wq", torch.bfloat16, (Hkv, G * D, dg), dev)
    _req(wk, "wk", torch.bfloat16, (Hkv, 3 * D, dg), dev)
    _req(w_qn, "w_qn", torch.float32, (dg,), dev)
    _req(w_kn, "w_kn", torch.float32, (dg,), dev)
    _req(q_gate, "q_gate", torch.float32, (B, T, Hkv, dg), dev)
    _req(k_gate, "k_gate", torch.float32, (B, T, Hkv, dg), dev)
    _req(idx, "idx", torch.int32, (B, T, Hkv, S), dev)
    _req(dlogg, "dlogg", torch.float32, (B, T, Hkv, S), dev)
    d = make_dims(B, T, Hq, Hkv, D, dg, S - 1, theta, eps)
    if check_row_sums:
        # the library drops the -g * sum(dlogg) term of the gate-logit
        # gradient, which vanishes for the attention's dlogg (rows sum to 0)
        worst = float(torch.where(idx >= 0, dlogg, torch.zeros_like(dlogg)).sum(-1).abs().max())
        if worst > row_sum_tol:
            warnings.warn(f"dlogg rows do not sum to zero (max |row sum| {worst:.3g} > "
                          f"{row_sum_tol:g}); sas_gate_score_bwd holds each row's gate lse "
                          "constant, so the -g * sum(dlogg) term is not included",
                          UserWarning, stacklevel=2)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty((B, T, Hq, D), **f32), dk=torch.empty((B, T, Hkv, D), **f32),
               dwq=torch.empty((Hkv, G * D, dg), **f32), dwk=torch.empty((Hkv, 3 * D, dg), **f32),
               dw_qn=torch.empty((dg,), **f32), dw_kn=torch.empty((dg,), **f32))
    nws = workspace_size(OP_GATE_BWD, d)
    ws = workspace if workspace is not None else _ws(nws, dev)
    _check(lib.sas_gate_score_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(wq), _ptr(wk),
                                  _ptr(w_qn), _ptr(w_kn), _ptr(q_gate), _ptr(k_gate), _ptr(idx),
                                  _ptr(dlogg), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dwq"]),
                                  _ptr(out["dwk"]), _ptr(out["dw_qn"]), _ptr(out["dw_kn"]),
                                  _ptr(ws), ws.numel() if ws is not None else 0, _stream(dev)))
    return out


def topk_blocks(q_gate, k_gate, topk: int, Hq: int, D: int, want_probs: bool = False,
                out=None):
    """Candidate softmax + Top-K: returns (idx, logg, gate_lse, gate_probs or None),
    per selection head (q_gate [B,T,Hs,dg] with Hs = Hkv, or Hq for one gate
    per query head; k_gate [B,T,Hkv,dg])."""
    lib = load_library()
    dev = _device_of(q_gate)
    B, T, Hs, dg = q_gate.shape
    Hkv = k_gate.shape[2]
    S = topk + 1
    NB = -(-T // 64)
    flags = _sel_flags(Hs, Hq, Hkv, "q_gate")
    _req(q_gate, "q_gate", torch.float32, (B, T, Hs, dg), dev)
    _req(k_gate, "k_gate", torch.float32, (B, T, Hkv, dg), dev)
    d = make_dims(B, T, Hq, Hkv, D, dg, topk, flags=flags)
    if out is None:
        idx = torch.empty((B, T, Hs, S), dtype=torch.int32, device=dev)
        logg = torch.empty((B, T, Hs, S), dtype=torch.float32, device=dev)
        lse = torch.empty((B, T, Hs), dtype=torch.float32, device=dev)
    else:
        idx, logg, lse = out
    probs = torch.empty((B, T, Hs, NB), dtype=torch.float32, device=dev) if want_probs else None
    _check(lib.sas_topk_blocks(ctypes.byref(d), _ptr(q_gate), _ptr(k_gate), _ptr(idx), _ptr(logg),
                               _ptr(lse), _ptr(probs), None, 0, _stream(dev)))
    return idx, logg, lse, probs


def sparse_attn_fwd(q, k, v, idx, logg, scale: float | None = None, o=None, lse=None,
                    o_f32=None, want_f32: bool = False, workspace=None):
    """Gated sparse attention forward: returns (o bf16 [B,T,Hq,D], lse fp32 [B,T,Hq])
    or, with want_f32 / o_f32 given, (o, lse, o_f32) where o_f32 is the fp32
    result before rounding (pass it to sparse_attn_bwd for an exact Delta)."""
    lib = load_library()
    dev = _device_of(q)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    Hs, S = idx.shape[2], idx.shape[-1]
    flags = _sel_flags(Hs, Hq, Hkv, "idx")
    _req(q, "q", torch.bfloat16, (B, T, Hq, D), dev)
    _req(k, "k", torch.bfloat16, (B, T, Hkv, D), dev)
    _req(v, "v", torch.bfloat16, (B, T, Hkv, D), dev)
    _req(idx, "idx", torch.int32, (B, T, Hs, S), dev)
    _req(logg, "logg", torch.float32, (B, T, Hs, S), dev)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    d = make_dims(B, T, Hq, Hkv, D, 128, S - 1, flags=flags)
    if o is None:
        o = torch.empty((B, T, Hq, D), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=dev)
    if want_f32 and o_f32 is None:
        o_f32 = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    if o_f32 is not None:
        _req(o_f32, "o_f32", torch.float32, (B, T, Hq, D), dev)
    nws = workspace_size(OP_FWD, d)
    ws = workspace if workspace is not None else _ws(nws, dev)
    _check(lib.sas_sparse_attn_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                   _ptr(logg), ctypes.c_float(scale), _ptr(o), _ptr(lse),
                                   _ptr(o_f32), _ptr(ws), ws.numel() if ws is not None else 0,
                                   _stream(dev)))
    return (o, lse, o_f32) if o_f32 is not None else (o, lse)


def walk_order(idx, Hq: int, Hkv: int):
    """Staging order of the query-group walks for selection idx [B,T,Hs,S]
    (diagnostic): uint16 [groups, stride], row g = (b * Hs + sg) * ngrp + grp
    holding the union size nU and then the nU blocks in the order the forward
    and dQ kernels take them."""
    lib = load_library()
    dev = _device_of(idx)
    B, T, Hs, S = idx.shape
    flags = _sel_flags(Hs, Hq, Hkv, "idx")
    _req(idx, "idx", torch.int32, (B, T, Hs, S), dev)
    d = make_dims(B, T, Hq, Hkv, 128, 128, S - 1, flags=flags)
    nbytes = workspace_size(OP_WALK_ORDER, d)
    NB = -(-T // 64)
    stride = (NB + 8) & ~7
    out = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    _check(lib.sas_walk_order(ctypes.byref(d), _ptr(idx), _ptr(out), nbytes, _stream(dev)))
    return out.view(-1, stride)


def sparse_attn_bwd(q, k, v, o, dout, lse, idx, logg, scale: float | None = None,
                    workspace=None, out=None, o_f32=None):
    """Backward: returns (dq, dk, dv bf16, dlogg fp32 [B,T,Hkv,S]).  o_f32 (the
    forward's fp32 output, optional) makes Delta = rowsum(dout * o) exact."""
    lib = load_library()
    dev = _device_of(q)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    Hs, S = idx.shape[2], idx.shape[-1]
    flags = _sel_flags(Hs, Hq, Hkv, "idx")
    for t, n, dt, sh in ((q, "q", torch.bfloat16, (B, T, Hq, D)), (k, "k", torch.bfloat16, (B, T, Hkv, D)),
                         (v, "v", torch.bfloat16, (B, T, Hkv, D)), (o, "o", torch.bfloat16, (B, T, Hq, D)),
                         (dout, "dout", torch.bfloat16, (B, T, Hq, D)),
                         (lse, "lse", torch.float32, (B, T, Hq)),
                         (idx, "idx", torch.int32, (B, T, Hs, S)),
                         (logg, "logg", torch.float32, (B, T, Hs, S))):
        _req(t, n, dt, sh, dev)
    if o_f32 is not None:
        _req(o_f32, "o_f32", torch.float32, (B, T, Hq, D), dev)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    d = make_dims(B, T, Hq, Hkv, D, 128, S - 1, flags=flags)
    if out is None:
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        dlogg = torch.empty((B, T, Hs, S), dtype=torch.float32, device=dev)
    else:
        dq, dk, dv, dlogg = out
    nws = workspace_size(OP_BWD, d)
    ws = workspace if workspace is not None else _ws(nws, dev)
    _check(lib.sas_sparse_attn_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   _ptr(o_f32), _ptr(dout),
                                   _ptr(lse), _ptr(idx), _ptr(logg), ctypes.c_float(scale),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dlogg), _ptr(ws),
                                   ws.numel() if ws is not None else 0, _stream(dev)))
    return dq, dk, dv, dlogg


def decode(q, q_gate, k_cache, v_cache, kg_cache, ctx_len, topk: int, scale: float | None = None,
           apply_gate: bool = True, want_idx: bool = True, workspace=None, out=None):
    """Budgeted decode step: returns (o bf16 [B,Hq,D], idx [B,Hkv,K+1] or None,
    logg [B,Hkv,K+1] or None)."""
    lib = load_library()
    dev = _device_of(q)
    B, Hq, D = q.shape
    _, Hkv, Lmax, _ = k_cache.shape
    dg = q_gate.shape[-1]
    NBmax = -(-Lmax // 64)
    S = topk + 1
    _req(q, "q", torch.bfloat16, (B, Hq, D), dev)
    Hs = q_gate.shape[1]
    flags = _sel_flags(Hs, Hq, Hkv, "q_gate")
    _req(q_gate, "q_gate", torch.float32, (B, Hs, dg), dev)
    _req(k_cache, "k_cache", torch.bfloat16, (B, Hkv, Lmax, D), dev)
    _req(v_cache, "v_cache", torch.bfloat16, (B, Hkv, Lmax, D), dev)
    kg_bf16 = kg_cache.dtype == torch.bfloat16
    _req(kg_cache, "kg_cache", torch.bfloat16 if kg_bf16 else torch.float32, (B, Hkv, NBmax, dg),
         dev)
    _req(ctx_len, "ctx_len", torch.int32, (B,), dev)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    d = DecodeDims(B, Hq, Hkv, D, dg, 64, topk, Lmax, NBmax, 1 if apply_gate else 0,
                   1 if kg_bf16 else 0, flags)
    if out is None:
        o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
        idx = torch.empty((B, Hs, S), dtype=torch.int32, device=dev) if want_idx else None
        logg = torch.empty((B, Hs, S), dtype=torch.float32, device=dev) if want_idx else None
    else:
        o, idx, logg = out
    nws = decode_workspace_size(d)
    ws = workspace if workspace is not None else _ws(nws, dev)
    _check(lib.sas_decode(ctypes.byref(d), _ptr(q), _ptr(q_gate), _ptr(k_cache), _ptr(v_cache),
                          _ptr(kg_cache), _ptr(ctx_len), ctypes.c_float(scale), _ptr(o), _ptr(idx),
                          _ptr(logg), _ptr(ws), ws.numel() if ws is not None else 0, _stream(dev)))
    return o, idx, logg


def decode_noalloc(q, q_gate, k_cache, v_cache, kg_cache, ctx_len, topk: int,
                   scale: float | None = None, apply_gate: bool = True, out=None):
    """decode() without a workspace: the library's fixed per-device scratch
    (see sas_decode_noalloc in sas.h; calls on one GPU must not overlap).
    With out=(o, idx, logg) preallocated, nothing is allocated at all.
    Returns (o, idx, logg)."""
    lib = load_library()
    dev = _device_of(q)
    B, Hq, D = q.shape
    _, Hkv, Lmax, _ = k_cache.shape
    dg = q_gate.shape[-1]
    NBmax = -(-Lmax // 64)
    S = topk + 1
    _req(q, "q", torch.bfloat16, (B, Hq, D), dev)
    Hs = q_gate.shape[1]
    flags = _sel_flags(Hs, Hq, Hkv, "q_gate")
    _req(q_gate, "q_gate", torch.float32, (B, Hs, dg), dev)
    _req(k_cache, "k_cache", torch.bfloat16, (B, Hkv, Lmax, D), dev)
    _req(v_cache, "v_cache", torch.bfloat16, (B, Hkv, Lmax, D), dev)
    kg_bf16 = kg_cache.dtype == torch.bfloat16
    _req(kg_cache, "kg_cache", torch.bfloat16 if kg_bf16 else torch.float32, (B, Hkv, NBmax, dg),
         dev)
    _req(ctx_len, "ctx_len", torch.int32, (B,), dev)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    d = DecodeDims(B, Hq, Hkv, D, dg, 64, topk, Lmax, NBmax, 1 if apply_gate else 0,
                   1 if kg_bf16 else 0, flags)
    if out is None:
        o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
        idx = torch.empty((B, Hs, S), dtype=torch.int32, device=dev)
        logg = torch.empty((B, Hs, S), dtype=torch.float32, device=dev)
    else:
        o, idx, logg = out
    _check(lib.sas_decode_noalloc(ctypes.byref(d), _ptr(q), _ptr(q_gate), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(kg_cache), _ptr(ctx_len),
                                  ctypes.c_float(scale), _ptr(o), _ptr(idx), _ptr(logg),
                                  _stream(dev)))
    return o, idx, logg


def decode_paged(q, q_gate, k_pages, v_pages, kg_pages, block_table, ctx_len, topk: int,
                 scale: float | None = None, apply_gate: bool = True, want_idx: bool = True,
                 workspace=None, out=None):
    """decode() over a paged KV cache: k_pages, v_pages [P,Hkv,64,D] bf16,
    kg_pages [P,Hkv,dg] fp32, block_table [B,NBmax] int32 (page of each block).
    Returns (o, idx or None, logg or None) as decode()."""
    lib = load_library()
    dev = _device_of(q)
    B, Hq, D = q.shape
    P, Hkv, blk, _ = k_pages.shape
    if blk != 64:
        raise ValueError("pages hold 64-token blocks")
    dg = q_gate.shape[-1]
    NBmax = block_table.shape[1]
    Lmax = 64 * NBmax
    S = topk + 1
    _req(q, "q", torch.bfloat16, (B, Hq, D), dev)
    Hs = q_gate.shape[1]
    flags = _sel_flags(Hs, Hq, Hkv, "q_gate")
    _req(q_gate, "q_gate", torch.float32, (B, Hs, dg), dev)
    _req(k_pages, "k_pages", torch.bfloat16, (P, Hkv, 64, D), dev)
    _req(v_pages, "v_pages", torch.bfloat16, (P, Hkv, 64, D), dev)
    kg_bf16 = kg_pages.dtype == torch.bfloat16
    _req(kg_pages, "kg_pages", torch.bfloat16 if kg_bf16 else torch.float32, (P, Hkv, dg), dev)
    _req(block_table, "block_table", torch.int32, (B, NBmax), dev)
    _req(ctx_len, "ctx_len", torch.int32, (B,), dev)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    d = DecodeDims(B, Hq, Hkv, D, dg, 64, topk, Lmax, NBmax, 1 if apply_gate else 0,
                   1 if kg_bf16 else 0, flags)
    if out is None:
        o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
        idx = torch.empty((B, Hs, S), dtype=torch.int32, device=dev) if want_idx else None
        logg = torch.empty((B, Hs, S), dtype=torch.float32, device=dev) if want_idx else None
    else:
        o, idx, logg = out
    nws = decode_workspace_size(d)
    ws = workspace if workspace is not None else _ws(nws, dev)
    _check(lib.sas_decode_paged(ctypes.byref(d), _ptr(q), _ptr(q_gate), _ptr(k_pages),
                                _ptr(v_pages), _ptr(kg_pages), ctypes.c_int32(P),
                                _ptr(block_table), _ptr(ctx_len), ctypes.c_float(scale), _ptr(o),
                                _ptr(idx), _ptr(logg), _ptr(ws),
                                ws.numel() if ws is not None else 0, _stream(dev)))
    return o, idx, logg


def decode_gate_key(k_cache, wk, w_kn, ctx_len, kg_cache, theta: float, eps: float,
                    block_table=None):
    """Refresh the gate-key cache entry of each sequence's current block from
    the KV cache rows 64c .. L-1 (see sas_decode_gate_key).  k_cache
    [B,Hkv,Lmax,D] (block_table None) or pages [P,Hkv,64,D] with block_table
    [B,NBmax]; kg_cache [B,Hkv,NBmax,dg] or [P,Hkv,dg], fp32 or bf16, updated
    in place."""
    lib = load_library()
    dev = _device_of(k_cache)
    B = ctx_len.shape[0]
    Hkv, D = k_cache.shape[1], k_cache.shape[3]
    dg = kg_cache.shape[-1]
    if block_table is None:
        Lmax = k_cache.shape[2]
        NBmax = -(-Lmax // 64)
        npages = 0
        _req(kg_cache, "kg_cache", kg_cache.dtype, (B, Hkv, NBmax, dg), dev)
    else:
        NBmax = block_table.shape[1]
        Lmax = 64 * NBmax
        npages = k_cache.shape[0]
        _req(block_table, "block_table", torch.int32, (B, NBmax), dev)
        _req(kg_cache, "kg_cache", kg_cache.dtype, (npages, Hkv, dg), dev)
    if kg_cache.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("kg_cache must be float32 or bfloat16")
    _req(k_cache, "k_cache", torch.bfloat16, tuple(k_cache.shape), dev)
    _req(wk, "wk", torch.bfloat16, (Hkv, 3 * D, dg), dev)
    _req(w_kn, "w_kn", torch.float32, (dg,), dev)
    _req(ctx_len, "ctx_len", torch.int32, (B,), dev)
    d = DecodeDims(B, Hkv, Hkv, D, dg, 64, 0, Lmax, NBmax, 1,
                   1 if kg_cache.dtype == torch.bfloat16 else 0)
    _check(lib.sas_decode_gate_key(ctypes.byref(d), _ptr(k_cache), _ptr(block_table),
                                   ctypes.c_int32(npages), _ptr(wk), _ptr(w_kn),
                                   ctypes.c_double(theta), ctypes.c_float(eps), _ptr(ctx_len),
                                   _ptr(kg_cache), _stream(dev)))
    return kg_cache
