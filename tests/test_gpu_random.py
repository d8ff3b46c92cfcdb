"""GPU parity on seeded random shapes: the forward pass, and the training pair
(the forward pass that keeps the chunk states, then the backward pass that
reads them), against the fp64 oracle, through the C ABI.

The shapes are drawn once from a fixed seed across the supported space (the
training pair with 64- and 32-token chunks):
batch, lengths uniform in [1, 320) (so mostly ragged tails), heads, d_k in
{64, 128}, d_v any multiple of 64 up to 512, every combination of gate and
initial state, and packed sequences of 2-6 members with lengths uniform in
[0, 200).  Tolerances as in the
other parity tests: relative L2 over each whole tensor and every (sequence,
head) pair, 2e-2 for bf16 inputs and 1e-4 for fp32 ones, 2.5 times that over
every 64-token chunk.
"""
import numpy as np
import pytest
import torch

import chunkwise_delta_rule_wy_amd as dn
import parity
from chunkwise_delta_rule_wy_amd.synth import Shape, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


def _draw_cases(n=12, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        Dk = int(rng.choice([64, 128]))
        Dv = 64 * int(rng.integers(1, 9))
        H = int(rng.choice([1, 2, 3, 5]))
        gated, h0 = i % 2 == 0, (i // 2) % 2 == 0  # every combination, three times
        if i % 3 == 2:  # packed sequences
            lens = tuple(int(x) for x in rng.integers(0, 200, size=int(rng.integers(2, 7))))
            if sum(lens) == 0:
                lens = lens[:-1] + (1,)
            cases.append((1, sum(lens), H, Dk, Dv, gated, h0, lens))
        else:
            B, T = int(rng.integers(1, 4)), int(rng.integers(1, 320))
            cases.append((B, T, H, Dk, Dv, gated, h0, None))
    return cases


CASES = _draw_cases()


def _id(c):
    B, T, H, Dk, Dv, gated, h0, lens = c
    return "B%dT%dH%dk%dv%d-g%d-h%d%s" % (B, T, H, Dk, Dv, gated, h0, "-packed%d" % len(lens) if lens else "")


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


@pytest.mark.parametrize("chunk", [64, 32])
@pytest.mark.parametrize("cfg", CASES, ids=_id)
def test_random_shape_training_pair(oracle_lib, cfg, chunk):
    B, T, H, Dk, Dv, gated, h0, lens = cfg
    sh = Shape(B, T, H, Dk, Dv, torch.bfloat16, gated, h0, backward=True, lengths=lens)
    x = make_inputs(sh, seed=7000 + T + Dv + H)
    d = to_dev(x)
    ws = torch.empty(dn.bwd_workspace_bytes(B, T, H, Dk, Dv, sh.n_seqs, chunk=chunk), dtype=torch.uint8, device=DEV)
    o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"], chunk=chunk,
                         save_workspace=ws)
    gr = dn.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["dO"], d["dhT"],
                      d["cu_seqlens"], chunk=chunk, workspace=ws, saved=True)
    torch.cuda.synchronize()
    oo, ho = oracle_lib.fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["cu_seqlens"])
    ref = oracle_lib.bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["dO"], x["dhT"],
                         cu_seqlens=x["cu_seqlens"])
    parity.check_fwd_outputs(o.cpu(), hT.cpu(), oo, ho, x["cu_seqlens"], TOL[torch.bfloat16], _id(cfg))
    gr = {k: (None if v is None else v.cpu()) for k, v in gr.items()}
    parity.check_grads(gr, ref, x["cu_seqlens"], TOL[torch.bfloat16], _id(cfg))


@pytest.mark.parametrize("cfg", [c for c in CASES if c[3] == 64][:4], ids=_id)
def test_random_shape_fp32_forward(oracle_lib, cfg):
    B, T, H, Dk, Dv, gated, h0, lens = cfg
    sh = Shape(B, T, H, Dk, Dv, torch.float32, gated, h0, lengths=lens)
    x = make_inputs(sh, seed=8000 + T + Dv + H)
    d = to_dev(x)
    o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"])
    torch.cuda.synchronize()
    oo, ho = oracle_lib.fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["cu_seqlens"])
    parity.check_fwd_outputs(o.cpu(), hT.cpu(), oo, ho, x["cu_seqlens"], TOL[torch.float32], _id(cfg) + " fp32")
