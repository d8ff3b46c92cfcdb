"""fp64 CPU oracle of the (gated) delta rule -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never touches it, and the two share no code: this wraps
``dn_oracle.c``, a plain token-by-token recurrence in double precision
(Gated DeltaNet review thread, Table 1, rows "DeltaNet" / "Gated DeltaNet":
S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t),
its sequential adjoint, and a single recurrent step; and the Longhorn row of
the same table (the delta rule at the step size beta / (1 + beta |k|^2)),
with its gradient by the chain rule through that step size; and the input
prologue of the workloads (L2-normalised q and k, sigmoid beta, negative
softplus log-gate) with its gradient, and the depthwise causal short
convolution with its adjoint, in numpy float64.

Inputs may be torch tensors (any float dtype, on any device) or numpy arrays;
they are upcast exactly to float64 on the host.  Results are float64 numpy.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dn_oracle.c")
_LIB = os.path.join(_HERE, "_dn_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the .so path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_fwd.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, I]
        lib.oracle_fwd.restype = I
        lib.oracle_bwd.argtypes = [I, I, I, I, I, I, P] + [P] * 8 + [P] * 6 + [I]
        lib.oracle_bwd.restype = I
        lib.oracle_step.argtypes = [I, I, I, I, P, P, P, P, P, P, P, I]
        lib.oracle_step.restype = I
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(q, v, cu):
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    N = (len(cu) - 1) if cu is not None else B
    return B, T, H, Dk, Dv, N


def fwd(q, k, v, beta, g=None, h0=None, cu_seqlens=None, nthreads=0):
    """Forward pass.  Returns (o [B,T,H,Dv], hT [N,H,Dk,Dv]) as float64."""
    q, k, v, beta, g, h0 = map(_f64, (q, k, v, beta, g, h0))
    cu = _i32(cu_seqlens)
    B, T, H, Dk, Dv, N = _dims(q, v, cu)
    o = np.zeros((B, T, H, Dv))
    hT = np.zeros((N, H, Dk, Dv))
    rc = _load().oracle_fwd(B, T, H, Dk, Dv, N, _ptr(cu), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(beta), _ptr(g), _ptr(h0), _ptr(o), _ptr(hT), int(nthreads))
    if rc:
        raise ValueError("oracle_fwd failed (%d)" % rc)
    return o, hT


def bwd(q, k, v, beta, g, h0, dO, dhT=None, cu_seqlens=None, nthreads=0):
    """Backward pass of L = <dO, o> + <dhT, hT>.  Returns a dict with
    dq, dk, dv, dbeta, dg (None if ungated) and dh0, all float64."""
    q, k, v, beta, g, h0, dO, dhT = map(_f64, (q, k, v, beta, g, h0, dO, dhT))
    cu = _i32(cu_seqlens)
    B, T, H, Dk, Dv, N = _dims(q, v, cu)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dbeta = np.zeros_like(beta)
    dg = np.zeros_like(beta) if g is not None else None
    dh0 = np.zeros((N, H, Dk, Dv))
    rc = _load().oracle_bwd(B, T, H, Dk, Dv, N, _ptr(cu), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(beta), _ptr(g), _ptr(h0), _ptr(dO), _ptr(dhT),
                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dg),
                            _ptr(dh0), int(nthreads))
    if rc:
        raise ValueError("oracle_bwd failed (%d)" % rc)
    return dict(dq=dq, dk=dk, dv=dv, dbeta=dbeta, dg=dg, dh0=dh0)


def step(q, k, v, beta, g, state, nthreads=0):
    """One recurrent step.  q, k [B,H,Dk], v [B,H,Dv], beta/g [B,H],
    state [B,H,Dk,Dv].  Returns (o [B,H,Dv], new_state) as float64."""
    q, k, v, beta, g = map(_f64, (q, k, v, beta, g))
    st = _f64(state).copy()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    o = np.zeros((B, H, Dv))
    rc = _load().oracle_step(B, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                             _ptr(g), _ptr(st), _ptr(o), int(nthreads))
    if rc:
        raise ValueError("oracle_step failed (%d)" % rc)
    return o, st


# ------------------------------------------------------------------ Longhorn
# Gated DeltaNet review thread, Table 1, row "Longhorn" (with the scalar beta
# of the table's caption): the delta-rule update with the step size
#     eps_t = beta_t / (1 + beta_t k_t^T k_t)
# in place of beta_t, S_t = S_{t-1}(I - eps_t k_t k_t^T) + eps_t v_t k_t^T.
# The row has no decay; g is passed through to the recurrence unchanged.

def longhorn_eps(k, beta):
    """eps = beta / (1 + beta |k|^2) per (token, head), float64 [..., H]."""
    k, beta = _f64(k), _f64(beta)
    return beta / (1.0 + beta * np.sum(k * k, axis=-1))


def longhorn_fwd(q, k, v, beta, g=None, h0=None, cu_seqlens=None, nthreads=0):
    """Forward pass of the Longhorn recurrence: (o, hT) as float64."""
    return fwd(q, k, v, longhorn_eps(k, beta), g, h0, cu_seqlens, nthreads)


def longhorn_eps_bwd(k, beta, deps):
    """Chain rule through eps = beta / (1 + beta s), s = |k|^2:
    dbeta = deps / (1 + beta s)^2 and the extra key gradient
    deps * (-beta^2 / (1 + beta s)^2) * 2 k.  Returns (dbeta, dk_extra)."""
    k, beta, deps = _f64(k), _f64(beta), _f64(deps)
    den = 1.0 + beta * np.sum(k * k, axis=-1)
    dbeta = deps / (den * den)
    dk = (deps * (-2.0 * beta * beta / (den * den)))[..., None] * k
    return dbeta, dk


def longhorn_bwd(q, k, v, beta, g, h0, dO, dhT=None, cu_seqlens=None, nthreads=0):
    """Backward pass of <dO, o> + <dhT, hT> for the Longhorn recurrence: the
    delta-rule adjoint at beta = eps, then the chain rule through eps."""
    eps = longhorn_eps(k, beta)
    gr = bwd(q, k, v, eps, g, h0, dO, dhT, cu_seqlens, nthreads)
    dbeta, dk_extra = longhorn_eps_bwd(k, beta, gr["dbeta"])
    gr["dbeta"] = dbeta
    gr["dk"] = gr["dk"] + dk_extra
    return gr


# ------------------------------------------------------------- input prologue
# The steps on either side of the recurrence in a (Gated) DeltaNet layer, as
# the workloads prepare their inputs: q and k are L2-normalised per token and
# head, beta = sigmoid(b), and the log-gate is g = -c * softplus(x).  A zero
# row normalises to zero with a zero gradient (the direction is undefined).

def prologue(q_in, k_in, b_in, g_in=None, gate_scale=1.0):
    """Returns (q, k, beta, g) in float64 (g None without a gate input)."""
    q_in, k_in, b_in, g_in = map(_f64, (q_in, k_in, b_in, g_in))

    def unit(x):
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)
    beta = 1.0 / (1.0 + np.exp(-b_in))
    g = None
    if g_in is not None:
        g = -float(gate_scale) * (np.maximum(g_in, 0.0) + np.log1p(np.exp(-np.abs(g_in))))
    return unit(q_in), unit(k_in), beta, g


def prologue_bwd(q_in, k_in, b_in, g_in, gate_scale, dq, dk, dbeta, dg=None):
    """Gradients of the prologue's inputs from those of its outputs:
    d x_in = (dx - u (u . dx)) / |x| with u = x / |x| (0 for a zero row),
    d b_in = dbeta * beta (1 - beta), d g_in = -c * sigmoid(x) * dg."""
    q_in, k_in, b_in, g_in, dq, dk, dbeta, dg = map(_f64, (q_in, k_in, b_in, g_in, dq, dk, dbeta, dg))

    def unit_bwd(x, dx):
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        safe = np.where(n > 0, n, 1.0)
        u = x / safe
        r = (dx - u * np.sum(u * dx, axis=-1, keepdims=True)) / safe
        return np.where(n > 0, r, 0.0)
    beta = 1.0 / (1.0 + np.exp(-b_in))
    db_in = dbeta * beta * (1.0 - beta)
    dg_in = None
    if g_in is not None:
        dg_in = -float(gate_scale) * dg / (1.0 + np.exp(-g_in))
    return unit_bwd(q_in, dq), unit_bwd(k_in, dk), db_in, dg_in


# ------------------------------------------------------------- short convolution
# The depthwise "short convolution" that the DeltaNet rebuttal (answer W2)
# names beside the token mixer: every channel of every head is filtered along
# time by its own W taps, causally, so a token sees itself and the W - 1
# tokens before it in its own sequence (zeros before the sequence start).
# The pages give neither the width nor an activation; the width is the
# caller's and no activation is applied.

def _seq_ranges(B, T, cu_seqlens):
    """(batch row, first token, end token) of every sequence."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(c) for c in _i32(cu_seqlens)]
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def short_conv(x, w, cu_seqlens=None):
    """y[t, h, c] = sum_{j < W} w[h, c, j] x[t - (W - 1) + j, h, c] inside each
    sequence (tap W - 1 is the current token).  x [B, T, H, D] (packed: B = 1
    with cu_seqlens [N + 1]), w [H, D, W].  Returns y in float64."""
    x, w = _f64(x), _f64(w)
    B, T = x.shape[:2]
    W = w.shape[-1]
    y = np.zeros_like(x)
    for b, t0, t1 in _seq_ranges(B, T, cu_seqlens):
        L = t1 - t0
        for j in range(W):
            s = W - 1 - j  # tap j reads the token s steps back
            if s < L:
                y[b, t0 + s:t1] += w[:, :, j] * x[b, t0:t1 - s]
    return y


def short_conv_bwd(x, w, dy, cu_seqlens=None):
    """Adjoint of short_conv: dx[t] = sum_j w[j] dy[t + (W - 1) - j] over the
    outputs of the same sequence, dw[h, c, j] = sum_t dy[t] x[t - (W - 1) + j].
    Returns (dx, dw) in float64."""
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    B, T = x.shape[:2]
    W = w.shape[-1]
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    for b, t0, t1 in _seq_ranges(B, T, cu_seqlens):
        L = t1 - t0
        for j in range(W):
            s = W - 1 - j
            if s < L:
                dx[b, t0:t1 - s] += w[:, :, j] * dy[b, t0 + s:t1]
                dw[:, :, j] += np.sum(dy[b, t0 + s:t1] * x[b, t0:t1 - s], axis=0)
    return dx, dw
