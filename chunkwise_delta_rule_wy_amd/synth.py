"""Seeded synthetic inputs for the chunkwise (gated) delta rule.

This module only draws random tensors and prepares them the way a DeltaNet /
Gated DeltaNet layer hands them to the token mixer: q and k are L2-normalised
per token and head, beta is a sigmoid, the log-gate g is a negative softplus.
It holds none of the recurrence's arithmetic, so both the fp64 oracle and the
HIP path can consume exactly the same bits.

Draw order is fixed (q, k, v, beta logits, gate noise, h0, dO, dhT) from a
CPU ``torch.Generator`` seeded with ``1000 + workload id``; every tensor is
drawn in fp32, then cast (round to nearest even) where the workload says bf16.

Workloads (the five problem settings of the delta-rule pages: an ungated fp32
parity case, a 1.3B-model DeltaNet layer, a gated layer with head dim 256, its
backward pass, and long-context varlen plus a decode step):

====  ==========================================================  ========
id    shape                                                        dtype
====  ==========================================================  ========
1     B=1  T=256   H=1  dk=dv=64, ungated, h0=0                    fp32
2     B=8  T=2048  H=16 dk=dv=128, ungated, h0=0                   bf16
3     B=4  T=4096  H=16 dk=128 dv=256, gated, h0                   bf16
4     workload 3 plus dO, dhT (forward + backward)                 bf16
5     varlen: 8 packed sequences, 65536 tokens, H=32, dk=dv=128    bf16
6     workload 5 plus dO, dhT (forward + backward, packed)         bf16
5dec  decode: batch 256, H=32, dk=dv=128, state fp32                bf16
====  ==========================================================  ========
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

# Lengths of the 8 packed sequences of the varlen workload.  They were drawn
# once as 7 distinct cut points uniformly from [1, 65535]
# (torch.randperm(65535, generator=manual_seed(1005))[:7] + 1, sorted) and are
# stored here so that runs do not depend on the RNG implementation.
VARLEN_LENGTHS = (13073, 3173, 21998, 5719, 7061, 6815, 3511, 4186)
assert sum(VARLEN_LENGTHS) == 65536


@dataclasses.dataclass(frozen=True)
class Shape:
    """One problem setting.  ``lengths`` is set for packed (varlen) inputs."""
    B: int
    T: int
    H: int
    Dk: int
    Dv: int
    dtype: torch.dtype
    gated: bool
    has_h0: bool
    backward: bool = False
    lengths: Optional[tuple] = None

    @property
    def n_seqs(self) -> int:
        return len(self.lengths) if self.lengths is not None else self.B

    @property
    def tokens(self) -> int:
        return self.B * self.T


WORKLOADS = {
    1: Shape(1, 256, 1, 64, 64, torch.float32, gated=False, has_h0=False),
    2: Shape(8, 2048, 16, 128, 128, torch.bfloat16, gated=False, has_h0=False),
    3: Shape(4, 4096, 16, 128, 256, torch.bfloat16, gated=True, has_h0=True),
    4: Shape(4, 4096, 16, 128, 256, torch.bfloat16, gated=True, has_h0=True,
             backward=True),
    5: Shape(1, 65536, 32, 128, 128, torch.bfloat16, gated=True, has_h0=True,
             lengths=VARLEN_LENGTHS),
    6: Shape(1, 65536, 32, 128, 128, torch.bfloat16, gated=True, has_h0=True,
             backward=True, lengths=VARLEN_LENGTHS),
}

WORKLOAD_NAMES = {
    1: "ungated-fp32-B1-T256-H1-d64",
    2: "deltanet-1.3B-layer-bf16-B8-T2048-H16-d128",
    3: "gated-bf16-B4-T4096-H16-dk128-dv256",
    4: "gated-fwd+bwd-bf16-B4-T4096-H16-dk128-dv256",
    5: "varlen-gated-bf16-8seqs-65536tok-H32-d128",
    6: "varlen-gated-fwd+bwd-bf16-8seqs-65536tok-H32-d128",
}


def cu_seqlens_of(lengths) -> torch.Tensor:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    """L2-normalise the last dimension (input preparation of q and k)."""
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


GATE_SCALE = 0.1  # g = -GATE_SCALE * softplus(noise)


def make_inputs(shape: Shape, seed: int, *, beta_override: Optional[float] = None,
                raw: bool = False) -> dict:
    """Draw one seeded input set on the CPU.

    Returns a dict with q, k, v (``shape.dtype``), beta, g (fp32 or None),
    h0 (fp32 or None), cu_seqlens (int32 or None) and, for backward settings,
    dO (``shape.dtype``) and dhT (fp32).  With ``raw`` it also holds the draws
    before preparation: q_in, k_in (``shape.dtype``), b_in (beta logits) and
    x_in (gate noise, None when ungated), with ``gate_scale``.  Tensors are contiguous, in the
    layouts q,k ``[B,T,H,Dk]``, v ``[B,T,H,Dv]``, beta/g ``[B,T,H]``,
    h0 ``[N,H,Dk,Dv]`` (the transposed state).
    """
    gen = torch.Generator("cpu").manual_seed(seed)
    B, T, H, Dk, Dv = shape.B, shape.T, shape.H, shape.Dk, shape.Dv
    N = shape.n_seqs
    q_raw = torch.randn(B, T, H, Dk, generator=gen)
    k_raw = torch.randn(B, T, H, Dk, generator=gen)
    q = _unit_rows(q_raw)
    k = _unit_rows(k_raw)
    v = torch.randn(B, T, H, Dv, generator=gen)
    b_raw = torch.randn(B, T, H, generator=gen)
    beta = torch.sigmoid(b_raw)
    if beta_override is not None:
        beta = torch.full_like(beta, float(beta_override))
    g = None
    noise = torch.randn(B, T, H, generator=gen)
    if shape.gated:
        g = -torch.nn.functional.softplus(noise) * GATE_SCALE
    h0 = None
    h0_draw = torch.randn(N, H, Dk, Dv, generator=gen) * 0.1
    if shape.has_h0:
        h0 = h0_draw
    out = dict(
        q=q.to(shape.dtype).contiguous(),
        k=k.to(shape.dtype).contiguous(),
        v=v.to(shape.dtype).contiguous(),
        beta=beta.float().contiguous(),
        g=None if g is None else g.float().contiguous(),
        h0=None if h0 is None else h0.contiguous(),
        cu_seqlens=None if shape.lengths is None else cu_seqlens_of(shape.lengths),
    )
    if shape.backward:
        out["dO"] = torch.randn(B, T, H, Dv, generator=gen).to(shape.dtype).contiguous()
        out["dhT"] = (torch.randn(N, H, Dk, Dv, generator=gen) * 0.1).contiguous()
    if raw:
        out["q_in"] = q_raw.to(shape.dtype).contiguous()
        out["k_in"] = k_raw.to(shape.dtype).contiguous()
        out["b_in"] = b_raw.contiguous()
        out["x_in"] = noise.contiguous() if shape.gated else None
        out["gate_scale"] = GATE_SCALE
    return out


def workload_inputs(wid: int, raw: bool = False) -> dict:
    """Inputs of a numbered workload, seeded with ``1000 + wid``."""
    return make_inputs(WORKLOADS[wid], 1000 + wid, raw=raw)


def decode_inputs(B: int = 256, H: int = 32, Dk: int = 128, Dv: int = 128,
                  dtype: torch.dtype = torch.bfloat16, gated: bool = True,
                  seed: int = 1105) -> dict:
    """One decode step's inputs: q, k, v ``[B,H,D]``, beta/g ``[B,H]`` and the
    fp32 state ``[B,H,Dk,Dv]`` (N(0, 0.01) entries)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    q = _unit_rows(torch.randn(B, H, Dk, generator=gen))
    k = _unit_rows(torch.randn(B, H, Dk, generator=gen))
    v = torch.randn(B, H, Dv, generator=gen)
    beta = torch.sigmoid(torch.randn(B, H, generator=gen))
    noise = torch.randn(B, H, generator=gen)
    g = (-torch.nn.functional.softplus(noise) * 0.1) if gated else None
    state = torch.randn(B, H, Dk, Dv, generator=gen) * 0.1
    return dict(q=q.to(dtype).contiguous(), k=k.to(dtype).contiguous(),
                v=v.to(dtype).contiguous(), beta=beta.contiguous(),
                g=None if g is None else g.contiguous(), state=state.contiguous())


def conv_inputs(B: int, T: int, H: int, D: int, W: int, dtype: torch.dtype = torch.bfloat16,
                seed: int = 1200, lengths=None) -> dict:
    """Inputs of the depthwise short convolution: a projection x ``[B,T,H,D]``
    (N(0, 1), cast to dtype), taps w ``[H,D,W]`` (uniform in +-1/sqrt(W)), the
    output gradient dy (N(0, 1), fp32) and, for packed sequences (B = 1, T =
    sum(lengths)), cu_seqlens.  Draw order x, w, dy."""
    gen = torch.Generator("cpu").manual_seed(seed)
    if lengths is not None:
        assert B == 1 and T == sum(lengths)
    x = torch.randn(B, T, H, D, generator=gen)
    w = (torch.rand(H, D, W, generator=gen) * 2 - 1) / W ** 0.5
    dy = torch.randn(B, T, H, D, generator=gen)
    return dict(x=x.to(dtype).contiguous(), w=w.contiguous(), dy=dy.contiguous(),
                cu_seqlens=None if lengths is None else cu_seqlens_of(lengths))


def rel_l2(x, y) -> float:
    """Relative L2 error ||x - y|| / ||y|| over a whole tensor, in fp64
    (absolute ||x|| when y is all zero)."""
    import numpy as np
    x = x.detach().double().cpu().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, np.float64)
    y = y.detach().double().cpu().numpy() if isinstance(y, torch.Tensor) else np.asarray(y, np.float64)
    den = float(np.linalg.norm(y.ravel()))
    num = float(np.linalg.norm((x - y).ravel()))
    return num / den if den > 0 else num
