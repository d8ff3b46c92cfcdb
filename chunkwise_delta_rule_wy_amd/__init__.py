"""Chunkwise (gated) delta rule on AMD MI355X (gfx950).

The recurrence (Gated DeltaNet review thread, Table 1, rows "DeltaNet" and
"Gated DeltaNet"), per sequence and head:

    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t,   alpha_t = exp(g_t)

evaluated chunkwise in WY/UT form by hand-written HIP kernels in ``libdn.so``.
This module is a thin ctypes binding: it checks tensors, allocates outputs and
workspace with torch, and passes raw device pointers and the current HIP
stream to the C ABI declared in ``include/dn.h``.  Every step of the
computation runs in the library's kernels; there is no fallback.

States are stored transposed, ``h = S^T`` with shape ``[N, H, Dk, Dv]``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["chunk_fwd", "chunk_bwd", "chunk_bwd_noalloc", "bwd_workspace_bytes", "recurrent_step",
           "longhorn_eps", "longhorn_eps_bwd", "longhorn_fwd", "longhorn_bwd", "prologue", "prologue_bwd",
           "short_conv", "short_conv_bwd", "DeltaRule", "delta_rule", "ShortConv", "short_conv_fn",
           "load_library", "LIB_PATH", "DnError"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdn.so")

DN_F32, DN_BF16 = 0, 1
_DTYPES = {torch.float32: DN_F32, torch.bfloat16: DN_BF16}


class DnError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s: %s" % (fn, msg))
        self.status = status


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lib = None


def load_library():
    """Load libdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libdn.so is not built (%s); run __graft_entry__.build() or "
                           "python chunkwise_delta_rule_wy_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, S = ctypes.c_void_p, ctypes.POINTER(_Shape)
    lib.dn_status_str.argtypes = [ctypes.c_int]
    lib.dn_status_str.restype = ctypes.c_char_p
    lib.dn_chunk_fwd_workspace.argtypes = [S]
    lib.dn_chunk_fwd_workspace.restype = ctypes.c_size_t
    lib.dn_chunk_bwd_workspace.argtypes = [S]
    lib.dn_chunk_bwd_workspace.restype = ctypes.c_size_t
    lib.dn_chunk_fwd.argtypes = [S] + [P] * 9 + [P, ctypes.c_size_t, P]
    lib.dn_chunk_fwd.restype = ctypes.c_int
    lib.dn_chunk_bwd.argtypes = [S] + [P] * 7 + [P, P] + [P] * 6 + [P, ctypes.c_size_t, P]
    lib.dn_chunk_bwd.restype = ctypes.c_int
    lib.dn_chunk_bwd_events.argtypes = [S] + [P] * 7 + [P, P] + [P] * 6 + [P, ctypes.c_size_t, P, P]
    lib.dn_chunk_bwd_events.restype = ctypes.c_int
    lib.dn_chunk_fwd_save.argtypes = [S] + [P] * 9 + [P, ctypes.c_size_t, P]
    lib.dn_chunk_fwd_save.restype = ctypes.c_int
    lib.dn_chunk_bwd_saved.argtypes = [S] + [P] * 7 + [P, P] + [P] * 6 + [P, ctypes.c_size_t, P, P]
    lib.dn_chunk_bwd_saved.restype = ctypes.c_int
    lib.dn_chunk_bwd_prologue.argtypes = ([S] + [P] * 7 + [P, P] + [P, P, P, ctypes.c_float] + [P] * 6
                                          + [P, ctypes.c_size_t, P, P])
    lib.dn_chunk_bwd_prologue.restype = ctypes.c_int
    lib.dn_chunk_bwd_longhorn.argtypes = [S] + [P] * 7 + [P, P] + [P] + [P] * 6 + [P, ctypes.c_size_t, P, P]
    lib.dn_chunk_bwd_longhorn.restype = ctypes.c_int
    lib.dn_chunk_bwd_noalloc.argtypes = [S] + [P] * 7 + [P, P] + [P] * 6 + [P]
    lib.dn_chunk_bwd_noalloc.restype = ctypes.c_int
    lib.dn_recurrent_step.argtypes = [ctypes.c_int32] * 5 + [P] * 7 + [P]
    lib.dn_recurrent_step.restype = ctypes.c_int
    lib.dn_longhorn_eps.argtypes = [ctypes.c_int32] * 5 + [P] * 3 + [P]
    lib.dn_longhorn_eps.restype = ctypes.c_int
    lib.dn_longhorn_eps_bwd.argtypes = [ctypes.c_int32] * 5 + [P] * 5 + [P]
    lib.dn_longhorn_eps_bwd.restype = ctypes.c_int
    lib.dn_prologue.argtypes = [ctypes.c_int32] * 5 + [P] * 4 + [ctypes.c_float] + [P] * 4 + [P]
    lib.dn_prologue.restype = ctypes.c_int
    lib.dn_prologue_bwd.argtypes = [ctypes.c_int32] * 5 + [P] * 4 + [ctypes.c_float] + [P] * 8 + [P]
    lib.dn_prologue_bwd.restype = ctypes.c_int
    lib.dn_short_conv.argtypes = [ctypes.c_int32] * 7 + [P] * 4 + [P]
    lib.dn_short_conv.restype = ctypes.c_int
    lib.dn_short_conv_bwd.argtypes = [ctypes.c_int32] * 7 + [P] * 6 + [P]
    lib.dn_short_conv_bwd.restype = ctypes.c_int
    lib.dn_short_conv_l2.argtypes = [ctypes.c_int32] * 7 + [P] * 4 + [P]
    lib.dn_short_conv_l2.restype = ctypes.c_int
    lib.dn_short_conv_l2_bwd.argtypes = [ctypes.c_int32] * 7 + [P] * 6 + [P]
    lib.dn_short_conv_l2_bwd.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        msg = load_library().dn_status_str(status).decode()
        raise DnError(fn, status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dtype, shape, dev):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.device != dev:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _workspace(ws, dev, nbytes, name):
    """Check a caller's workspace: a contiguous uint8 tensor on the inputs'
    device holding at least nbytes."""
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise TypeError("%s must be a contiguous uint8 tensor" % name)
    if ws.device != dev:
        raise ValueError("%s is on %s, expected %s" % (name, ws.device, dev))
    if ws.numel() < nbytes:
        raise ValueError("%s holds %d bytes, %d needed" % (name, ws.numel(), nbytes))
    return ws


def _shape(q, v, cu_seqlens, chunk):
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, Dk]")
    if q.dtype not in _DTYPES:
        raise TypeError("q, k, v must be float32 or bfloat16")
    if q.device.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    return _Shape(B, T, H, Dk, Dv, N, chunk, _DTYPES[q.dtype]), N


def chunk_fwd(q, k, v, beta, g=None, h0=None, cu_seqlens=None, output_final_state=True,
              chunk: int = 64, save_workspace: Optional[torch.Tensor] = None):
    """Chunkwise forward pass.

    q, k ``[B,T,H,Dk]``, v ``[B,T,H,Dv]`` (float32 or bfloat16, one dtype);
    beta, g ``[B,T,H]`` float32 (g None: no gate); h0 ``[N,H,Dk,Dv]`` float32
    or None; cu_seqlens int32 ``[N+1]`` on the device for packed sequences
    (then B == 1).  Returns ``(o, hT)`` (hT None unless output_final_state).
    ``save_workspace`` (uint8, at least ``bwd_workspace_bytes``; bfloat16
    inputs only): also store the chunk-start states there for
    ``chunk_bwd(..., saved=True)`` (``dn_chunk_fwd_save``).
    """
    lib = load_library()
    s, N = _shape(q, v, cu_seqlens, chunk)
    dev = q.device
    B, T, H, Dk, Dv = s.B, s.T, s.H, s.Dk, s.Dv
    _need(q, "q", q.dtype, (B, T, H, Dk), dev)
    _need(k, "k", q.dtype, (B, T, H, Dk), dev)
    _need(v, "v", q.dtype, (B, T, H, Dv), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    _need(g, "g", torch.float32, (B, T, H), dev)
    _need(h0, "h0", torch.float32, (N, H, Dk, Dv), dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    o = torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev)
    hT = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev) if output_final_state else None
    if save_workspace is not None:
        _workspace(save_workspace, dev, lib.dn_chunk_bwd_workspace(ctypes.byref(s)), "save_workspace")
        _check("dn_chunk_fwd_save", lib.dn_chunk_fwd_save(
            ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(h0),
            _ptr(cu_seqlens), _ptr(o), _ptr(hT), _ptr(save_workspace), save_workspace.numel(),
            _stream(dev)))
        return o, hT
    wsb = lib.dn_chunk_fwd_workspace(ctypes.byref(s))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    _check("dn_chunk_fwd", lib.dn_chunk_fwd(
        ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(h0),
        _ptr(cu_seqlens), _ptr(o), _ptr(hT), _ptr(ws), wsb, _stream(dev)))
    return o, hT


def chunk_bwd(q, k, v, beta, g, h0, dO, dhT=None, cu_seqlens=None, chunk: int = 64,
              workspace: Optional[torch.Tensor] = None, events=None, saved: bool = False,
              prologue_inputs=None, longhorn_beta: Optional[torch.Tensor] = None):
    """Backward pass of ``<dO, o> + <dhT, hT>``.

    Returns a dict of float32 gradients dq, dk, dv, dbeta, dg (None without a
    gate) and dh0.  ``workspace`` (uint8, at least ``bwd_workspace_bytes``)
    may be passed to avoid an allocation per call.  ``events``: four
    ``torch.cuda.Event(enable_timing=True)`` that the library records before
    its first kernel and after the recompute, the state-gradient sweep and the
    chunk-gradient kernel (``dn_chunk_bwd_events``); a None entry is not
    recorded.  ``saved``: skip the
    recompute and read the states that ``chunk_fwd(..., save_workspace=
    workspace)`` stored for these inputs (``dn_chunk_bwd_saved``).
    ``prologue_inputs`` = (q_in, k_in, x_in, gate_scale), with ``saved``: q, k,
    beta, g are ``prologue``'s outputs for these raw inputs, and the dict holds
    the gradients of the raw inputs instead: dq_in, dk_in, db_in, dx_in, with
    dv and dh0 (``dn_chunk_bwd_prologue``: the prologue's backward folded into
    the chunk-gradient kernel).  ``longhorn_beta`` (with ``saved``): beta is
    the Longhorn step size ``longhorn_eps(k, longhorn_beta)``; dbeta is then the
    gradient of ``longhorn_beta`` and dk includes the step size's key term
    (``dn_chunk_bwd_longhorn``).
    """
    lib = load_library()
    s, N = _shape(q, v, cu_seqlens, chunk)
    dev = q.device
    B, T, H, Dk, Dv = s.B, s.T, s.H, s.Dk, s.Dv
    _need(q, "q", q.dtype, (B, T, H, Dk), dev)
    _need(k, "k", q.dtype, (B, T, H, Dk), dev)
    _need(v, "v", q.dtype, (B, T, H, Dv), dev)
    _need(dO, "dO", q.dtype, (B, T, H, Dv), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    _need(g, "g", torch.float32, (B, T, H), dev)
    _need(h0, "h0", torch.float32, (N, H, Dk, Dv), dev)
    _need(dhT, "dhT", torch.float32, (N, H, Dk, Dv), dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty((B, T, H, Dk), **f32)
    dk = torch.empty((B, T, H, Dk), **f32)
    dv = torch.empty((B, T, H, Dv), **f32)
    dbeta = torch.empty((B, T, H), **f32)
    dg = torch.empty((B, T, H), **f32) if g is not None else None
    dh0 = torch.empty((N, H, Dk, Dv), **f32)
    wsb = lib.dn_chunk_bwd_workspace(ctypes.byref(s))
    if saved and workspace is None:
        raise ValueError("saved=True needs the workspace that chunk_fwd filled")
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    else:
        _workspace(workspace, dev, wsb, "workspace")
    ev = None
    if events is not None:
        if len(events) != 4:
            raise ValueError("events: four torch.cuda.Event objects (or None) expected")
        for e in events:
            if e is not None and e.cuda_event == 0:  # torch creates the event on its first record
                e.record(torch.cuda.current_stream(dev))
        ev = (ctypes.c_void_p * 4)(*[None if e is None else e.cuda_event for e in events])
    if longhorn_beta is not None:
        if not saved or prologue_inputs is not None:
            raise ValueError("longhorn_beta needs saved=True and no prologue_inputs")
        _need(longhorn_beta, "longhorn_beta", torch.float32, (B, T, H), dev)
        _check("dn_chunk_bwd_longhorn", lib.dn_chunk_bwd_longhorn(
            ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(h0),
            _ptr(cu_seqlens), _ptr(dO), _ptr(dhT), _ptr(longhorn_beta), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(dbeta), _ptr(dg), _ptr(dh0), _ptr(workspace), workspace.numel(), _stream(dev), ev))
        return dict(dq=dq, dk=dk, dv=dv, dbeta=dbeta, dg=dg, dh0=dh0)
    if prologue_inputs is not None:
        if not saved:
            raise ValueError("prologue_inputs needs saved=True (the states dn_chunk_fwd_save kept)")
        q_in, k_in, x_in, gate_scale = prologue_inputs
        _need(q_in, "q_in", q.dtype, (B, T, H, Dk), dev)
        _need(k_in, "k_in", q.dtype, (B, T, H, Dk), dev)
        _need(x_in, "x_in", torch.float32, (B, T, H), dev)
        _check("dn_chunk_bwd_prologue", lib.dn_chunk_bwd_prologue(
            ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(h0),
            _ptr(cu_seqlens), _ptr(dO), _ptr(dhT), _ptr(q_in), _ptr(k_in), _ptr(x_in),
            float(gate_scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dg), _ptr(dh0),
            _ptr(workspace), workspace.numel(), _stream(dev), ev))
        return dict(dq_in=dq, dk_in=dk, dv=dv, db_in=dbeta, dx_in=dg, dh0=dh0)
    fn = lib.dn_chunk_bwd_saved if saved else lib.dn_chunk_bwd_events
    _check("dn_chunk_bwd_saved" if saved else "dn_chunk_bwd", fn(
        ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(h0),
        _ptr(cu_seqlens), _ptr(dO), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta),
        _ptr(dg), _ptr(dh0), _ptr(workspace), workspace.numel(), _stream(dev), ev))
    return dict(dq=dq, dk=dk, dv=dv, dbeta=dbeta, dg=dg, dh0=dh0)


def chunk_bwd_noalloc(q, k, v, beta, g, h0, dO, dhT=None, cu_seqlens=None, out=None, chunk: int = 64):
    """``chunk_bwd`` (recomputing) through ``dn_chunk_bwd_noalloc``: the
    library's static scratch buffer replaces the workspace, so the call
    allocates no device memory of its own.  ``out``: optional dict of
    preallocated float32 gradients (dq, dk, dv, dbeta, dg, dh0) to write into;
    missing ones are allocated here.  Returns that dict."""
    lib = load_library()
    s, N = _shape(q, v, cu_seqlens, chunk)
    dev = q.device
    B, T, H, Dk, Dv = s.B, s.T, s.H, s.Dk, s.Dv
    _need(q, "q", q.dtype, (B, T, H, Dk), dev)
    _need(k, "k", q.dtype, (B, T, H, Dk), dev)
    _need(v, "v", q.dtype, (B, T, H, Dv), dev)
    _need(dO, "dO", q.dtype, (B, T, H, Dv), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    _need(g, "g", torch.float32, (B, T, H), dev)
    _need(h0, "h0", torch.float32, (N, H, Dk, Dv), dev)
    _need(dhT, "dhT", torch.float32, (N, H, Dk, Dv), dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    shapes = dict(dq=(B, T, H, Dk), dk=(B, T, H, Dk), dv=(B, T, H, Dv), dbeta=(B, T, H), dg=(B, T, H),
                  dh0=(N, H, Dk, Dv))
    res = dict(out) if out is not None else {}
    for name, shp in shapes.items():
        if name == "dg" and g is None:
            res[name] = None
        elif res.get(name) is None:
            res[name] = torch.empty(shp, dtype=torch.float32, device=dev)
        else:
            _need(res[name], name, torch.float32, shp, dev)
    _check("dn_chunk_bwd_noalloc", lib.dn_chunk_bwd_noalloc(
        ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(h0), _ptr(cu_seqlens),
        _ptr(dO), _ptr(dhT), _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["dbeta"]),
        _ptr(res["dg"]), _ptr(res["dh0"]), _stream(dev)))
    return res


def bwd_workspace_bytes(B, T, H, Dk, Dv, n_seqs=None, dtype=torch.bfloat16, chunk=64) -> int:
    s = _Shape(B, T, H, Dk, Dv, B if n_seqs is None else n_seqs, chunk, _DTYPES[dtype])
    return int(load_library().dn_chunk_bwd_workspace(ctypes.byref(s)))


def recurrent_step(q, k, v, beta, g, state):
    """One decode step.  q, k ``[B,H,Dk]``, v ``[B,H,Dv]``, beta/g ``[B,H]``
    float32 (g may be None), state ``[B,H,Dk,Dv]`` float32 updated in place.
    Returns o ``[B,H,Dv]``."""
    lib = load_library()
    if q.dim() != 3 or q.dtype not in _DTYPES or q.device.type != "cuda":
        raise ValueError("q must be a [B, H, Dk] float32/bfloat16 GPU tensor")
    dev = q.device
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    _need(q, "q", q.dtype, (B, H, Dk), dev)
    _need(k, "k", q.dtype, (B, H, Dk), dev)
    _need(v, "v", q.dtype, (B, H, Dv), dev)
    _need(beta, "beta", torch.float32, (B, H), dev)
    _need(g, "g", torch.float32, (B, H), dev)
    _need(state, "state", torch.float32, (B, H, Dk, Dv), dev)
    o = torch.empty((B, H, Dv), dtype=q.dtype, device=dev)
    _check("dn_recurrent_step", lib.dn_recurrent_step(
        B, H, Dk, Dv, _DTYPES[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
        _ptr(state), _ptr(o), _stream(dev)))
    return o


def _key_rows(k, beta):
    """(B, T, H, Dk) of a key tensor [B,T,H,Dk] or a decode key [B,H,Dk]."""
    if k.dim() == 3:
        B, H, Dk = k.shape
        T = 1
    elif k.dim() == 4:
        B, T, H, Dk = k.shape
    else:
        raise ValueError("k must be [B,T,H,Dk] or [B,H,Dk]")
    if k.dtype not in _DTYPES or k.device.type != "cuda":
        raise ValueError("k must be a float32/bfloat16 GPU tensor")
    _need(k, "k", k.dtype, tuple(k.shape), k.device)
    _need(beta, "beta", torch.float32, tuple(k.shape[:-1]), k.device)
    return B, T, H, Dk


def longhorn_eps(k, beta):
    """Longhorn step size eps = beta / (1 + beta |k|^2) (``dn_longhorn_eps``),
    float32 with beta's shape; feed it to ``chunk_fwd`` / ``recurrent_step``
    as beta to run the Longhorn recurrence."""
    lib = load_library()
    B, T, H, Dk = _key_rows(k, beta)
    eps = torch.empty(beta.shape, dtype=torch.float32, device=k.device)
    _check("dn_longhorn_eps", lib.dn_longhorn_eps(
        B, T, H, Dk, _DTYPES[k.dtype], _ptr(k), _ptr(beta), _ptr(eps), _stream(k.device)))
    return eps


def longhorn_eps_bwd(k, beta, deps, dk):
    """Backward of ``longhorn_eps`` (``dn_longhorn_eps_bwd``): returns dbeta and
    adds the key term into ``dk`` (float32, updated in place)."""
    lib = load_library()
    B, T, H, Dk = _key_rows(k, beta)
    _need(deps, "deps", torch.float32, tuple(beta.shape), k.device)
    _need(dk, "dk", torch.float32, tuple(k.shape), k.device)
    dbeta = torch.empty(beta.shape, dtype=torch.float32, device=k.device)
    _check("dn_longhorn_eps_bwd", lib.dn_longhorn_eps_bwd(
        B, T, H, Dk, _DTYPES[k.dtype], _ptr(k), _ptr(beta), _ptr(deps), _ptr(dbeta), _ptr(dk),
        _stream(k.device)))
    return dbeta


def longhorn_fwd(q, k, v, beta, g=None, h0=None, cu_seqlens=None, output_final_state=True):
    """Forward pass of the Longhorn recurrence: ``longhorn_eps`` then
    ``chunk_fwd`` at beta := eps.  Returns (o, hT)."""
    return chunk_fwd(q, k, v, longhorn_eps(k, beta), g, h0, cu_seqlens, output_final_state)


def longhorn_bwd(q, k, v, beta, g, h0, dO, dhT=None, cu_seqlens=None, workspace=None):
    """Backward pass of the Longhorn recurrence: eps again (nothing is kept
    from the forward call), ``chunk_bwd`` at beta := eps, then
    ``longhorn_eps_bwd``.  Returns the gradient dict of ``chunk_bwd``."""
    eps = longhorn_eps(k, beta)
    gr = chunk_bwd(q, k, v, eps, g, h0, dO, dhT, cu_seqlens, workspace=workspace)
    gr["dbeta"] = longhorn_eps_bwd(k, beta, gr["dbeta"], gr["dk"])
    return gr


def prologue(q_in, k_in, b_in, x_in=None, gate_scale: float = 1.0):
    """Input prologue (``dn_prologue``): q, k L2-normalised per row (dtype of
    q_in), beta = sigmoid(b_in), g = -gate_scale * softplus(x_in) (None
    without x_in).  Returns (q, k, beta, g)."""
    lib = load_library()
    B, T, H, Dk = _key_rows(k_in, b_in)
    _need(q_in, "q_in", k_in.dtype, tuple(k_in.shape), k_in.device)
    _need(x_in, "x_in", torch.float32, tuple(b_in.shape), k_in.device)
    q = torch.empty_like(q_in)
    k = torch.empty_like(k_in)
    beta = torch.empty_like(b_in)
    g = torch.empty_like(x_in) if x_in is not None else None
    _check("dn_prologue", lib.dn_prologue(
        B, T, H, Dk, _DTYPES[k_in.dtype], _ptr(q_in), _ptr(k_in), _ptr(b_in), _ptr(x_in),
        float(gate_scale), _ptr(q), _ptr(k), _ptr(beta), _ptr(g), _stream(k_in.device)))
    return q, k, beta, g


def prologue_bwd(q_in, k_in, b_in, x_in, gate_scale, dq, dk, dbeta, dg=None):
    """Backward of ``prologue`` (``dn_prologue_bwd``): float32 gradients
    (dq_in, dk_in, db_in, dx_in) from those of q, k, beta, g."""
    lib = load_library()
    B, T, H, Dk = _key_rows(k_in, b_in)
    dev = k_in.device
    _need(q_in, "q_in", k_in.dtype, tuple(k_in.shape), dev)
    _need(x_in, "x_in", torch.float32, tuple(b_in.shape), dev)
    _need(dq, "dq", torch.float32, tuple(k_in.shape), dev)
    _need(dk, "dk", torch.float32, tuple(k_in.shape), dev)
    _need(dbeta, "dbeta", torch.float32, tuple(b_in.shape), dev)
    _need(dg, "dg", torch.float32, tuple(b_in.shape), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    dq_in = torch.empty(k_in.shape, **f32)
    dk_in = torch.empty(k_in.shape, **f32)
    db_in = torch.empty(b_in.shape, **f32)
    dx_in = torch.empty(b_in.shape, **f32) if x_in is not None else None
    _check("dn_prologue_bwd", lib.dn_prologue_bwd(
        B, T, H, Dk, _DTYPES[k_in.dtype], _ptr(q_in), _ptr(k_in), _ptr(b_in), _ptr(x_in),
        float(gate_scale), _ptr(dq), _ptr(dk), _ptr(dbeta), _ptr(dg), _ptr(dq_in), _ptr(dk_in),
        _ptr(db_in), _ptr(dx_in), _stream(dev)))
    return dq_in, dk_in, db_in, dx_in


def _conv_dims(x, w, cu_seqlens):
    if not isinstance(x, torch.Tensor) or x.dim() != 4:
        raise ValueError("x must be a [B, T, H, D] tensor")
    if x.dtype not in _DTYPES:
        raise TypeError("x must be float32 or bfloat16")
    B, T, H, D = x.shape
    if not isinstance(w, torch.Tensor) or w.dim() != 3 or tuple(w.shape[:2]) != (H, D):
        raise ValueError("w must be a [H, D, W] tensor")
    W = w.shape[2]
    _need(w, "w", torch.float32, (H, D, W), x.device)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    n_seqs = B
    if cu_seqlens is not None:
        n_seqs = cu_seqlens.numel() - 1
        _need(cu_seqlens, "cu_seqlens", torch.int32, (n_seqs + 1,), x.device)
    return B, T, H, D, W, n_seqs


def short_conv(x, w, cu_seqlens=None, l2norm: bool = False):
    """Depthwise causal short convolution (``dn_short_conv``): y[t] = sum_j
    w[:, :, j] x[t - (W - 1) + j] inside each sequence; x [B, T, H, D], w
    [H, D, W] float32.  With ``l2norm`` every (token, head) row of y is
    scaled to unit length in the same pass (``dn_short_conv_l2``).  Returns y
    (dtype of x)."""
    lib = load_library()
    B, T, H, D, W, n = _conv_dims(x, w, cu_seqlens)
    y = torch.empty_like(x)
    fn = "dn_short_conv_l2" if l2norm else "dn_short_conv"
    _check(fn, getattr(lib, fn)(
        B, T, H, D, W, n, _DTYPES[x.dtype], _ptr(x), _ptr(w), _ptr(cu_seqlens), _ptr(y), _stream(x.device)))
    return y


def short_conv_bwd(x, w, dy, cu_seqlens=None, l2norm: bool = False):
    """Backward of ``short_conv`` (``dn_short_conv_bwd``, or
    ``dn_short_conv_l2_bwd`` with ``l2norm``): float32 (dx, dw) from dy =
    dL/dy (float32, the shape of x)."""
    lib = load_library()
    B, T, H, D, W, n = _conv_dims(x, w, cu_seqlens)
    _need(dy, "dy", torch.float32, tuple(x.shape), x.device)
    dx = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    dw = torch.empty(w.shape, dtype=torch.float32, device=x.device)
    fn = "dn_short_conv_l2_bwd" if l2norm else "dn_short_conv_bwd"
    _check(fn, getattr(lib, fn)(
        B, T, H, D, W, n, _DTYPES[x.dtype], _ptr(x), _ptr(w), _ptr(cu_seqlens), _ptr(dy), _ptr(dx),
        _ptr(dw), _stream(x.device)))
    return dx, dw


class DeltaRule(torch.autograd.Function):
    """Autograd wrapper: forward by ``chunk_fwd``, backward by ``chunk_bwd``.
    Gradients are computed in float32 and cast to each input's dtype.  For
    bfloat16 inputs with ``save_states`` the forward pass keeps the bf16 chunk
    states (d_k d_v per chunk and head) and the backward pass skips their
    recompute; otherwise the backward pass recomputes them."""

    @staticmethod
    def forward(ctx, q, k, v, beta, g, h0, cu_seqlens, save_states=True):
        ws = None
        if save_states and q.dtype == torch.bfloat16:
            N = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
            ws = torch.empty(max(bwd_workspace_bytes(q.shape[0], q.shape[1], q.shape[2], q.shape[3],
                                                     v.shape[-1], N, q.dtype), 1),
                             dtype=torch.uint8, device=q.device)
        o, hT = chunk_fwd(q, k, v, beta, g, h0, cu_seqlens, output_final_state=True,
                          save_workspace=ws)
        ctx.save_for_backward(q, k, v, beta, g, h0, cu_seqlens)
        ctx.ws = ws
        return o, hT

    @staticmethod
    def backward(ctx, dO, dhT):
        q, k, v, beta, g, h0, cu = ctx.saved_tensors
        if dO is None:
            dO = torch.zeros(v.shape, dtype=q.dtype, device=q.device)
        ws, ctx.ws = ctx.ws, None
        gr = chunk_bwd(q, k, v, beta, g, h0, dO.to(q.dtype).contiguous(),
                       None if dhT is None else dhT.float().contiguous(), cu,
                       workspace=ws, saved=ws is not None)
        return (gr["dq"].to(q.dtype), gr["dk"].to(k.dtype), gr["dv"].to(v.dtype), gr["dbeta"],
                gr["dg"], None if h0 is None else gr["dh0"], None, None)


def delta_rule(q, k, v, beta, g=None, h0=None, cu_seqlens=None, save_states=True):
    """Differentiable chunkwise (gated) delta rule; returns (o, hT).
    ``save_states`` keeps the chunk states from the forward pass for the
    backward pass (bfloat16 inputs) instead of recomputing them."""
    return DeltaRule.apply(q, k, v, beta, g, h0, cu_seqlens, save_states)


class ShortConv(torch.autograd.Function):
    """Autograd wrapper of the depthwise causal short convolution: forward by
    ``short_conv``, backward by ``short_conv_bwd`` (dx cast to x's dtype, dw
    float32).  ``l2norm`` fuses the per-head L2 normalisation (q and k)."""

    @staticmethod
    def forward(ctx, x, w, cu_seqlens, l2norm=False):
        ctx.save_for_backward(x, w, cu_seqlens)
        ctx.l2norm = l2norm
        return short_conv(x, w, cu_seqlens, l2norm=l2norm)

    @staticmethod
    def backward(ctx, dy):
        x, w, cu = ctx.saved_tensors
        dx, dw = short_conv_bwd(x, w, dy.float().contiguous(), cu, l2norm=ctx.l2norm)
        return dx.to(x.dtype), dw, None, None


def short_conv_fn(x, w, cu_seqlens=None, l2norm=False):
    """Differentiable short convolution (optionally with the per-head L2
    normalisation fused in)."""
    return ShortConv.apply(x, w, cu_seqlens, l2norm)
