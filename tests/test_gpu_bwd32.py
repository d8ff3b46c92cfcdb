"""GPU parity of the training pair with 32-token chunks (the chunk-size
variant of the backward pass) against the fp64 oracle, through the C ABI.

The chunk length does not change the result (the chunk form is an exact
refactoring of the token recurrence), so the 32-token passes are held to the
same bounds as the 64-token ones: every gradient within relative L2 2e-2 of
the oracle over the whole tensor and every (sequence, head) pair, and within
2.5 times that over every 64-token block (tests/parity.py).
"""
import pytest
import torch

import chunkwise_delta_rule_wy_amd as dn
import parity
from chunkwise_delta_rule_wy_amd import synth
from chunkwise_delta_rule_wy_amd.synth import Shape, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 2e-2
NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def workspace(d):
    q, v = d["q"], d["v"]
    N = q.shape[0] if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
    return torch.empty(dn.bwd_workspace_bytes(q.shape[0], q.shape[1], q.shape[2], q.shape[3], v.shape[-1], N,
                                              chunk=32), dtype=torch.uint8, device=DEV)


def run32(x, saved):
    """(o, hT) of the 32-token forward pass (the saving one when `saved`) and
    the gradients of dn_chunk_bwd_saved / dn_chunk_bwd with chunk = 32."""
    d = to_dev(x)
    ws = workspace(d)
    o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"], chunk=32,
                         save_workspace=ws if saved else None)
    gr = dn.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["dO"], d["dhT"], d["cu_seqlens"],
                      chunk=32, workspace=ws, saved=saved)
    torch.cuda.synchronize()
    return o.cpu(), hT.cpu(), {k: (None if v is None else v.cpu()) for k, v in gr.items()}


def check32(x, oracle_lib, label, saved):
    o, hT, gr = run32(x, saved)
    oo, ho = oracle_lib.fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["cu_seqlens"])
    parity.check_fwd_outputs(o, hT, oo, ho, x["cu_seqlens"], TOL, label + " forward")
    ref = oracle_lib.bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["dO"], x["dhT"],
                         cu_seqlens=x["cu_seqlens"])
    parity.check_grads(gr, ref, x["cu_seqlens"], TOL, label)
    return gr


CASES = [
    # B, T, H, Dk, Dv, gated, h0: ragged tails around the 32-token boundary
    (2, 100, 2, 128, 128, True, True),
    (2, 64, 2, 128, 256, False, False),
    (1, 33, 3, 64, 192, True, True),
    (1, 31, 2, 128, 128, True, True),
    (1, 1, 2, 128, 128, True, True),
    (1, 130, 1, 128, 1024, True, True),   # the largest d_v
    (2, 70, 1, 64, 64, False, True),
    # N*H a multiple of 8: the XCD-aware workgroup placement
    (2, 200, 4, 128, 256, True, True),
    (2, 77, 8, 64, 192, True, False),
]


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "B%dT%dH%dk%dv%d-g%d-h%d" % c)
def test_bwd32_parity_small(oracle_lib, cfg, saved):
    B, T, H, Dk, Dv, gated, h0 = cfg
    sh = Shape(B, T, H, Dk, Dv, torch.bfloat16, gated, h0, backward=True)
    check32(make_inputs(sh, seed=300 + T + Dv), oracle_lib, "C=32 " + str(cfg), saved)


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
def test_bwd32_varlen_ragged(oracle_lib, saved):
    # empty, one-token, boundary and multi-chunk sequences; 7 x 2 pairs
    lens = (1, 31, 32, 33, 0, 130, 5)
    sh = Shape(1, sum(lens), 2, 128, 128, torch.bfloat16, True, True, backward=True, lengths=lens)
    x = make_inputs(sh, seed=331)
    gr = check32(x, oracle_lib, "C=32 varlen", saved)
    assert torch.equal(gr["dh0"][4], x["dhT"][4])  # the empty sequence passes dhT through


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
def test_bwd32_varlen_xcd_placement(oracle_lib, saved):
    lens = (200, 65, 1, 130)  # N*H = 16
    sh = Shape(1, sum(lens), 4, 128, 256, torch.bfloat16, True, True, backward=True, lengths=lens)
    check32(make_inputs(sh, seed=343), oracle_lib, "C=32 varlen N*H=16", saved)


def test_bwd32_strong_decay(oracle_lib):
    """g fifty times the workloads': the state scale restarts every chunk."""
    sh = Shape(2, 300, 2, 128, 128, torch.bfloat16, True, True, backward=True)
    x = make_inputs(sh, seed=377)
    x["g"] = (x["g"] * 50.0).contiguous()
    check32(x, oracle_lib, "C=32 strong decay", True)


def test_bwd32_saved_equals_recompute():
    """The saving 32-token forward pass writes the plain one's outputs bit for
    bit and the states the recompute writes, so both backward modes agree bit
    for bit."""
    sh = Shape(2, 150, 2, 128, 256, torch.bfloat16, True, True, backward=True)
    x = make_inputs(sh, seed=341)
    d = to_dev(x)
    o_ref, hT_ref = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], chunk=32)
    o, hT, gs = run32(x, True)
    _, _, gr = run32(x, False)
    assert torch.equal(o, o_ref.cpu()) and torch.equal(hT, hT_ref.cpu())
    for name in NAMES:
        assert torch.equal(gs[name], gr[name]), name


def test_bwd32_zero_length():
    sh = Shape(2, 0, 2, 128, 128, torch.bfloat16, True, True, backward=True)
    x = make_inputs(sh, seed=305)
    _, _, gr = run32(x, True)
    for name in ("dq", "dk", "dv", "dbeta", "dg"):
        assert gr[name].numel() == 0, name
    assert torch.equal(gr["dh0"], x["dhT"])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wid,saved", [(4, False), (4, True), (6, True)],
                         ids=["w4-recompute", "w4-saved", "w6-saved"])
def test_bwd32_full_size_every_pair(oracle_lib, wid, saved):
    """The training workloads at full size with 32-token chunks: the forward
    outputs and every gradient of every (sequence, head) pair and every chunk
    against the oracle (the same oracle run as the 64-token tests)."""
    x, (oo, ho), ref = parity.oracle_run(oracle_lib, wid)
    o, hT, gr = run32(x, saved)
    parity.check_fwd_outputs(o, hT, oo, ho, x["cu_seqlens"], TOL, "workload %d C=32 forward" % wid)
    parity.check_grads(gr, ref, x["cu_seqlens"], TOL, "workload %d C=32 %s" % (wid, "saved" if saved else "recompute"))


def test_bwd32_workspace_is_twice_the_states():
    sh = synth.WORKLOADS[4]
    w64 = dn.bwd_workspace_bytes(sh.B, sh.T, sh.H, sh.Dk, sh.Dv, sh.n_seqs)
    w32 = dn.bwd_workspace_bytes(sh.B, sh.T, sh.H, sh.Dk, sh.Dv, sh.n_seqs, chunk=32)
    assert w32 == 2 * w64
