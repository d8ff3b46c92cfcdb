"""GPU parity of the chunkwise backward pass against the fp64 oracle's
sequential adjoint, through the C ABI.

Every gradient (dq, dk, dv, dbeta, dg, dh0) must be within relative L2 2e-2
of the oracle (bf16 inputs, fp32 gradients), over the whole tensor and over
every (sequence, head) pair, and within 2.5 times that over every 64-token
chunk of every pair (tests/parity.py).  The full-size workloads are compared
on every pair, in both backward modes.
"""
import numpy as np
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


def gpu_bwd(x, saved=False):
    """Backward pass through dn_chunk_bwd, or (saved) through dn_chunk_fwd_save
    followed by dn_chunk_bwd_saved on one workspace."""
    d = to_dev(x)
    ws = None
    if saved:
        q, v = d["q"], d["v"]
        N = q.shape[0] if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
        ws = torch.empty(dn.bwd_workspace_bytes(q.shape[0], q.shape[1], q.shape[2], q.shape[3],
                                                v.shape[-1], N), dtype=torch.uint8, device=DEV)
        dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"],
                     save_workspace=ws)
    gr = dn.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["dO"], d["dhT"],
                      d["cu_seqlens"], workspace=ws, saved=saved)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu()) for k, v in gr.items()}


def check_bwd(x, oracle_lib, label, saved=False):
    gr = gpu_bwd(x, saved)
    ref = oracle_lib.bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["dO"], x["dhT"],
                         cu_seqlens=x["cu_seqlens"])
    parity.check_grads(gr, ref, x["cu_seqlens"], TOL, label)
    return gr


CASES = [
    # B, T, H, Dk, Dv, gated, h0
    (2, 150, 2, 128, 128, True, True),
    (2, 200, 2, 128, 128, False, False),
    (1, 300, 2, 128, 256, True, True),
    (2, 64, 3, 64, 192, True, True),
    (1, 1, 2, 128, 128, True, True),
    (1, 129, 9, 128, 64, True, False),
    (1, 130, 1, 128, 1024, True, True),   # the largest d_v, ragged tail
    (2, 70, 1, 64, 1024, False, True),
    # N*H a multiple of 8: the XCD-aware workgroup placement of the full-size shapes
    (2, 200, 4, 128, 256, True, True),
    (4, 130, 4, 128, 128, False, True),
    (2, 77, 8, 64, 192, True, False),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "B%dT%dH%dk%dv%d-g%d-h%d" % c)
def test_bwd_parity_small(oracle_lib, cfg):
    B, T, H, Dk, Dv, gated, h0 = cfg
    sh = Shape(B, T, H, Dk, Dv, torch.bfloat16, gated, h0, backward=True)
    check_bwd(make_inputs(sh, seed=100 + T + Dv), oracle_lib, str(cfg))


def test_bwd_varlen_ragged(oracle_lib):
    lens = (1, 63, 64, 65, 0, 130, 5)
    sh = Shape(1, sum(lens), 2, 128, 128, torch.bfloat16, True, True, backward=True, lengths=lens)
    x = make_inputs(sh, seed=31)
    gr = check_bwd(x, oracle_lib, "varlen")
    # an empty sequence passes its state gradient through
    assert torch.equal(gr["dh0"][4], x["dhT"][4])


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
def test_bwd_varlen_xcd_placement(oracle_lib, saved):
    # 4 packed sequences x 4 heads (N*H = 16, the XCD-aware placement), d_v 256
    lens = (200, 65, 1, 130)
    sh = Shape(1, sum(lens), 4, 128, 256, torch.bfloat16, True, True, backward=True, lengths=lens)
    check_bwd(make_inputs(sh, seed=43), oracle_lib, "varlen N*H=16", saved)


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
def test_bwd_varlen_many_sequences(oracle_lib, saved):
    """600 packed sequences of 0-90 tokens (more sequences than the chunk
    table's 256 threads, so each thread sums several), d_k = d_v = 64."""
    rng = np.random.default_rng(600)
    lens = tuple(int(x) for x in rng.integers(0, 91, size=600))
    sh = Shape(1, sum(lens), 2, 64, 64, torch.bfloat16, True, True, backward=True, lengths=lens)
    x = make_inputs(sh, seed=47)
    gr = check_bwd(x, oracle_lib, "600 sequences", saved)
    empty = [i for i, L in enumerate(lens) if L == 0]
    assert empty and all(torch.equal(gr["dh0"][i], x["dhT"][i]) for i in empty)


def test_bwd_no_final_state_gradient(oracle_lib):
    sh = Shape(2, 100, 2, 128, 128, torch.bfloat16, True, True, backward=True)
    x = make_inputs(sh, seed=33)
    x["dhT"] = None
    check_bwd(x, oracle_lib, "dhT=None")


def test_bwd_deterministic():
    sh = Shape(2, 260, 2, 128, 256, torch.bfloat16, True, True, backward=True)
    x = make_inputs(sh, seed=35)
    a = gpu_bwd(x)
    for _ in range(2):
        b = gpu_bwd(x)
        for name in NAMES:
            assert torch.equal(a[name], b[name]), name


def test_bwd_stage_events():
    """dn_chunk_bwd_events gives dn_chunk_bwd's gradients bit for bit and
    records its four events in stream order."""
    sh = Shape(1, 200, 2, 128, 256, torch.bfloat16, True, True, backward=True)
    x = make_inputs(sh, seed=39)
    a = gpu_bwd(x)
    d = to_dev(x)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    gr = dn.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["dO"], d["dhT"],
                      events=ev)
    ev[3].synchronize()
    for name in NAMES:
        assert torch.equal(a[name], gr[name].cpu()), name
    for i in range(3):
        assert ev[i].elapsed_time(ev[i + 1]) > 0.0


def test_autograd_wrapper_matches_entry_points():
    sh = Shape(1, 100, 2, 128, 128, torch.bfloat16, True, True, backward=True)
    x = to_dev(make_inputs(sh, seed=37))
    q, k, v = (x[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    beta = x["beta"].clone().requires_grad_(True)
    g = x["g"].clone().requires_grad_(True)
    h0 = x["h0"].clone().requires_grad_(True)
    o, hT = dn.delta_rule(q, k, v, beta, g, h0)
    loss = (o.float() * x["dO"].float()).sum() + (hT * x["dhT"]).sum()
    loss.backward()
    gr = dn.chunk_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["dO"], x["dhT"])
    assert torch.equal(beta.grad, gr["dbeta"]) and torch.equal(g.grad, gr["dg"])
    assert torch.equal(h0.grad, gr["dh0"])
    assert torch.equal(q.grad, gr["dq"].to(torch.bfloat16))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wid,saved", [(4, False), (4, True), (6, False), (6, True)],
                         ids=["w4-recompute", "w4-saved", "w6-recompute", "w6-saved"])
def test_bwd_full_size_every_pair(oracle_lib, wid, saved):
    """The training workloads at full size (workload 4; the packed workload 6,
    8 sequences of 65536 tokens with H=32, d=128, in one call), in the launch
    configuration the benchmark times: every gradient of every (sequence,
    head) pair and every chunk against the oracle, both backward modes."""
    x, (oo, ho), ref = parity.oracle_run(oracle_lib, wid)
    if saved:
        # the saved-state pair's forward outputs too
        d = to_dev(x)
        sh = synth.WORKLOADS[wid]
        ws = torch.empty(dn.bwd_workspace_bytes(sh.B, sh.T, sh.H, sh.Dk, sh.Dv, sh.n_seqs),
                         dtype=torch.uint8, device=DEV)
        o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"],
                             save_workspace=ws)
        gr = dn.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["dO"], d["dhT"],
                          d["cu_seqlens"], workspace=ws, saved=True)
        torch.cuda.synchronize()
        parity.check_fwd_outputs(o.cpu(), hT.cpu(), oo, ho, x["cu_seqlens"], TOL, "workload %d saving fwd" % wid)
        del d, ws, o, hT
        gr = {k: (None if v is None else v.cpu()) for k, v in gr.items()}
    else:
        gr = gpu_bwd(x, False)
    parity.check_grads(gr, ref, x["cu_seqlens"], TOL, "workload %d %s" % (wid, "saved" if saved else "recompute"))


SAVED_CASES = [
    # B, T, H, Dk, Dv, gated, h0, lengths
    (2, 150, 2, 128, 128, True, True, None),
    (2, 200, 2, 128, 256, False, False, None),
    (2, 64, 3, 64, 192, True, True, None),
    (1, 328, 2, 128, 128, True, True, (1, 63, 64, 65, 0, 130, 5)),
]


@pytest.mark.parametrize("cfg", SAVED_CASES, ids=lambda c: "B%dT%dH%dk%dv%d-g%d-h%d-%s" % (
    c[:7] + ("varlen" if c[7] else "fixed",)))
def test_saved_states_equal_recompute(oracle_lib, cfg):
    """dn_chunk_fwd_save writes dn_chunk_fwd's outputs bit for bit and the
    chunk states the backward's recompute would write, so dn_chunk_bwd_saved
    returns dn_chunk_bwd's gradients bit for bit; both are within the
    tolerance of the oracle."""
    B, T, H, Dk, Dv, gated, h0, lens = cfg
    sh = Shape(B, T, H, Dk, Dv, torch.bfloat16, gated, h0, backward=True, lengths=lens)
    x = make_inputs(sh, seed=41 + T)
    d = to_dev(x)
    o_ref, hT_ref = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"])
    N = sh.n_seqs
    ws = torch.empty(dn.bwd_workspace_bytes(B, T, H, Dk, Dv, N), dtype=torch.uint8, device=DEV)
    o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"],
                         save_workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(hT, hT_ref)
    gs = dn.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["dO"], d["dhT"],
                      d["cu_seqlens"], workspace=ws, saved=True)
    torch.cuda.synchronize()
    gs = {k: (None if v is None else v.cpu()) for k, v in gs.items()}
    gr = check_bwd(x, oracle_lib, "recompute " + str(cfg))
    for name in NAMES:
        if gr[name] is None:
            assert gs[name] is None
        else:
            assert torch.equal(gs[name], gr[name]), name


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
def test_bwd_zero_length(saved):
    """T = 0: nothing to differentiate but the initial state, whose gradient is
    dhT passed through; no token gradient has any element."""
    sh = Shape(2, 0, 2, 128, 128, torch.bfloat16, True, True, backward=True)
    x = make_inputs(sh, seed=5)
    gr = gpu_bwd(x, saved)
    for name in ("dq", "dk", "dv", "dbeta", "dg"):
        assert gr[name].numel() == 0, name
    assert torch.equal(gr["dh0"], x["dhT"])


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
def test_strong_decay_parity(oracle_lib, saved):
    """A gate fifty times the workloads' (g = -5 softplus(N(0, 1)), alpha down
    to e^-20 per token): the decay ratios underflow inside a chunk and the
    state scale restarts every chunk; forward and every gradient against the
    oracle."""
    sh = Shape(2, 300, 2, 128, 128, torch.bfloat16, True, True, backward=True)
    x = make_inputs(sh, seed=77)
    x["g"] = (x["g"] * 50.0).contiguous()
    d = to_dev(x)
    o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])
    torch.cuda.synchronize()
    oo, ho = oracle_lib.fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"])
    parity.check_fwd_outputs(o.cpu(), hT.cpu(), oo, ho, None, TOL, "strong decay forward")
    check_bwd(x, oracle_lib, "strong decay", saved)


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
def test_varlen_all_empty(saved):
    """Packed input whose sequences are all empty (T = 0, three sequences):
    hT = h0 and dh0 = dhT per sequence."""
    sh = Shape(1, 0, 2, 128, 128, torch.bfloat16, True, True, backward=True, lengths=(0, 0, 0))
    x = make_inputs(sh, seed=9)
    d = to_dev(x)
    o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"])
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(hT.cpu(), x["h0"])
    gr = gpu_bwd(x, saved)
    assert torch.equal(gr["dh0"], x["dhT"])


def test_partial_stage_events():
    # a None entry of the four stage events is not recorded; the others time their stages
    sh = Shape(2, 200, 2, 128, 128, torch.bfloat16, gated=True, has_h0=True, backward=True)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in make_inputs(sh, seed=1310).items()}
    ws = torch.empty(dn.bwd_workspace_bytes(sh.B, sh.T, sh.H, sh.Dk, sh.Dv), dtype=torch.uint8, device=DEV)
    dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], save_workspace=ws)
    args = (d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["dO"], d["dhT"])
    ref = dn.chunk_bwd(*args, workspace=ws, saved=True)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record()
    out = dn.chunk_bwd(*args, workspace=ws, saved=True, events=[None, None, e[1], e[2]])
    torch.cuda.synchronize()
    assert e[0].elapsed_time(e[1]) > 0 and e[1].elapsed_time(e[2]) > 0
    for k in ("dq", "dk", "dv", "dbeta", "dg", "dh0"):
        assert torch.equal(out[k], ref[k]), k
