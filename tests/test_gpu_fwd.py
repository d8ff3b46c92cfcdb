"""GPU parity of the chunkwise forward pass and the decode step against the
fp64 oracle, through the C ABI.

Tolerances (relative L2): 1e-4 for fp32 inputs and 2e-2 for bf16 inputs, on o
and on the final state, over the whole tensor and over every (sequence, head)
pair, and 2.5 times that over every 64-token chunk of every pair
(tests/parity.py).  The oracle reads exactly the bits the GPU reads (bf16
values upcast to fp64).  The full-size workloads are compared on every pair.
"""
import ctypes

import pytest
import torch

import chunkwise_delta_rule_wy_amd as dn
import parity
from chunkwise_delta_rule_wy_amd import synth
from chunkwise_delta_rule_wy_amd.synth import Shape, make_inputs, rel_l2

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def gpu_fwd(x):
    d = to_dev(x)
    o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"])
    torch.cuda.synchronize()
    return o.cpu(), hT.cpu()


def check_fwd(x, dtype, oracle_lib, label="", chunk=64):
    if chunk == 64:
        o, hT = gpu_fwd(x)
    else:
        d = to_dev(x)
        o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"], chunk=chunk)
        torch.cuda.synchronize()
        o, hT = o.cpu(), hT.cpu()
    oo, ho = oracle_lib.fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["cu_seqlens"])
    parity.check_fwd_outputs(o, hT, oo, ho, x["cu_seqlens"], TOL[dtype], label)
    return o, hT


SMALL = [
    # B, T, H, Dk, Dv, dtype, gated, h0
    (1, 256, 1, 64, 64, torch.float32, False, False),    # the fp32 parity workload itself
    (2, 190, 2, 64, 128, torch.float32, True, True),
    (2, 200, 3, 128, 128, torch.bfloat16, False, False),
    (2, 300, 2, 128, 256, torch.bfloat16, True, True),
    (1, 130, 2, 64, 192, torch.bfloat16, True, True),
    (3, 64, 1, 128, 64, torch.bfloat16, True, False),
    (1, 1, 2, 128, 128, torch.bfloat16, True, True),
    (1, 65, 9, 128, 128, torch.bfloat16, True, True),   # N*H not a multiple of 8
    (1, 130, 1, 128, 1024, torch.bfloat16, True, True),  # the largest d_v, ragged tail
    (1, 100, 1, 64, 1024, torch.float32, True, True),    # the largest d_v in fp32
    # N*H a multiple of 8: the XCD-aware workgroup placement of the full-size shapes
    (2, 200, 4, 128, 256, torch.bfloat16, True, True),
    (4, 130, 4, 128, 128, torch.bfloat16, False, False),
    (2, 77, 8, 64, 192, torch.bfloat16, True, True),
    (2, 150, 4, 64, 64, torch.float32, True, True),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: "B%dT%dH%dk%dv%d-%s-g%d-h%d" % (
    c[0], c[1], c[2], c[3], c[4], str(c[5]).split(".")[-1], c[6], c[7]))
def test_fwd_parity_small(oracle_lib, cfg):
    B, T, H, Dk, Dv, dtype, gated, h0 = cfg
    x = make_inputs(Shape(B, T, H, Dk, Dv, dtype, gated, h0), seed=7 + T + Dv)
    check_fwd(x, dtype, oracle_lib, str(cfg))


def test_fwd_varlen_ragged(oracle_lib):
    lens = (1, 63, 64, 65, 0, 127, 200, 5)
    sh = Shape(1, sum(lens), 2, 128, 128, torch.bfloat16, True, True, lengths=lens)
    x = make_inputs(sh, seed=21)
    o, hT = check_fwd(x, torch.bfloat16, oracle_lib, "varlen")
    # the empty sequence passes its initial state through unchanged
    assert torch.equal(hT[4], x["h0"][4])
    # varlen equals separate runs of each sequence
    cu = x["cu_seqlens"]
    for n in (0, 3, 6):
        s, e = int(cu[n]), int(cu[n + 1])
        xs = dict(q=x["q"][:, s:e].contiguous(), k=x["k"][:, s:e].contiguous(),
                  v=x["v"][:, s:e].contiguous(), beta=x["beta"][:, s:e].contiguous(),
                  g=x["g"][:, s:e].contiguous(), h0=x["h0"][n:n + 1].contiguous(), cu_seqlens=None)
        on, hn = gpu_fwd(xs)
        assert torch.equal(on, o[:, s:e]) and torch.equal(hn[0], hT[n])


def test_fwd_varlen_xcd_placement(oracle_lib):
    # 4 packed sequences x 4 heads (N*H = 16, the XCD-aware placement), d_v 256
    lens = (200, 65, 1, 130)
    sh = Shape(1, sum(lens), 4, 128, 256, torch.bfloat16, True, True, lengths=lens)
    check_fwd(make_inputs(sh, seed=23), torch.bfloat16, oracle_lib, "varlen N*H=16")


def test_fwd_zero_length(oracle_lib):
    sh = Shape(2, 0, 2, 128, 128, torch.bfloat16, True, True)
    x = make_inputs(sh, seed=3)
    o, hT = gpu_fwd(x)
    assert o.numel() == 0
    assert torch.equal(hT, x["h0"])


def test_fwd_no_write_special_case(oracle_lib):
    sh = Shape(2, 150, 2, 128, 128, torch.bfloat16, True, True)
    x = make_inputs(sh, seed=5, beta_override=0.0)
    o, hT = check_fwd(x, torch.bfloat16, oracle_lib, "beta=0")
    x0 = dict(x)
    x0["h0"] = None
    o0, h0 = gpu_fwd(x0)
    assert not o0.float().abs().max() and not h0.abs().max()


def test_fwd_orthonormal_keys_recall(oracle_lib):
    # beta = 1 with orthonormal keys: the state recalls every value exactly
    T, Dk, Dv = 64, 64, 64  # fp32 path: d_k = 64
    gen = torch.Generator().manual_seed(0)
    Qm, _ = torch.linalg.qr(torch.randn(Dk, Dk, generator=gen, dtype=torch.float64))
    k = Qm[:T].float().reshape(1, T, 1, Dk)
    q = torch.randn(1, T, 1, Dk, generator=gen)
    v = torch.randn(1, T, 1, Dv, generator=gen)
    x = dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), beta=torch.ones(1, T, 1),
             g=None, h0=None, cu_seqlens=None)
    o, hT = check_fwd(x, torch.float32, oracle_lib, "orthonormal")
    recall = hT[0, 0].double().T @ k[0, :, 0].double().T  # S k_j for every j
    assert rel_l2(recall.T, v[0, :, 0]) < 1e-4


def test_fwd_deterministic_and_state_passing(oracle_lib):
    sh = Shape(2, 333, 2, 128, 256, torch.bfloat16, True, True)
    x = make_inputs(sh, seed=11)
    o1, h1 = gpu_fwd(x)
    for _ in range(3):
        o2, h2 = gpu_fwd(x)
        assert torch.equal(o1, o2) and torch.equal(h1, h2)
    # Split at a chunk boundary: each segment against the oracle run on the same
    # segment (the second from the first's GPU final state), and the two
    # segments together against one run.  The kernel carries the state scaled by
    # a running product of decays and feeds it to the MFMA in bf16, so the two
    # runs round it differently: they must agree to within one bf16 epsilon
    # (2^-8, about 4e-3; measured on MI355X: o 1.5e-3, hT 2.5e-3).
    T1 = 128
    seg = lambda a, b: {kk: (vv[:, a:b].contiguous() if kk in ("q", "k", "v", "beta", "g") else vv)
                        for kk, vv in x.items()}
    xa = seg(0, T1)
    oa, ha = check_fwd(xa, torch.bfloat16, oracle_lib, "segment 1")
    xb = seg(T1, None)
    xb["h0"] = ha
    ob, hb = check_fwd(xb, torch.bfloat16, oracle_lib, "segment 2")
    eh, eo = rel_l2(hb, h1), rel_l2(torch.cat([oa, ob], 1), o1)
    print("chained vs one run: o %.2e hT %.2e" % (eo, eh), flush=True)
    assert eh < 4e-3 and eo < 4e-3, (eo, eh)


def test_fwd_canary_no_out_of_bounds_writes():
    lib = dn.load_library()
    sh = Shape(1, 100, 2, 128, 128, torch.bfloat16, True, True)
    x = to_dev(make_inputs(sh, seed=13))
    pad = 4096
    n_o = 1 * 100 * 2 * 128
    n_h = 2 * 128 * 128
    obuf = torch.full((n_o + 2 * pad,), 7.0, dtype=torch.bfloat16, device=DEV)
    hbuf = torch.full((n_h + 2 * pad,), 7.0, dtype=torch.float32, device=DEV)
    s = dn._Shape(1, 100, 2, 128, 128, 1, 64, 1)
    P = ctypes.c_void_p
    st = lib.dn_chunk_fwd(ctypes.byref(s), P(x["q"].data_ptr()), P(x["k"].data_ptr()),
                          P(x["v"].data_ptr()), P(x["beta"].data_ptr()), P(x["g"].data_ptr()),
                          P(x["h0"].data_ptr()), None, P(obuf[pad:].data_ptr()),
                          P(hbuf[pad:].data_ptr()), None, 0,
                          P(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert (obuf[:pad] == 7.0).all() and (obuf[pad + n_o:] == 7.0).all()
    assert (hbuf[:pad] == 7.0).all() and (hbuf[pad + n_h:] == 7.0).all()
    o_ref, h_ref = dn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"])
    assert torch.equal(obuf[pad:pad + n_o], o_ref.flatten())


# ------------------------------------------------------------------- decode
@pytest.mark.parametrize("B,H,Dk,Dv,dtype,gated", [
    (256, 32, 128, 128, torch.bfloat16, True),   # the decode workload
    (3, 2, 64, 64, torch.float32, False),
    (5, 3, 128, 256, torch.bfloat16, True),
    (2, 2, 64, 192, torch.float32, True),
    (2, 1, 128, 1024, torch.bfloat16, True),     # the largest d_v
])
def test_step_parity(oracle_lib, B, H, Dk, Dv, dtype, gated):
    x = synth.decode_inputs(B, H, Dk, Dv, dtype, gated)
    d = to_dev(x)
    st = d["state"].clone()
    o = dn.recurrent_step(d["q"], d["k"], d["v"], d["beta"], d["g"], st)
    torch.cuda.synchronize()
    oo, so = oracle_lib.step(x["q"], x["k"], x["v"], x["beta"], x["g"], x["state"])
    # whole tensor and every (batch, head) pair
    parity.check("o", parity.state_errors(o.cpu().unsqueeze(-1), oo[..., None]), TOL[dtype], "decode")
    parity.check("state", parity.state_errors(st.cpu(), so), TOL[dtype], "decode")


def test_decode_steps_equal_chunk_forward():
    # fp32 keeps the comparison tight; decode and chunk paths share no kernel
    sh = Shape(2, 70, 2, 64, 128, torch.float32, True, True)
    x = make_inputs(sh, seed=17)
    o, hT = gpu_fwd(x)
    d = to_dev(x)
    st = d["h0"].clone()
    outs = []
    for t in range(70):
        outs.append(dn.recurrent_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                      d["v"][:, t].contiguous(), d["beta"][:, t].contiguous(),
                                      d["g"][:, t].contiguous(), st))
    torch.cuda.synchronize()
    assert rel_l2(torch.stack(outs, 1).cpu(), o) < 1e-5
    assert rel_l2(st.cpu(), hT) < 1e-5


# ------------------------------------------------------- full-size workloads
@pytest.mark.timeout(900)
@pytest.mark.parametrize("wid", [2, 3, 5])
def test_fwd_full_size_every_pair(oracle_lib, wid):
    """The forward workloads at full size, in the launch configuration the
    benchmark times: every (sequence, head) pair and every chunk against the
    oracle."""
    sh = synth.WORKLOADS[wid]
    x, (oo, ho), _ = parity.oracle_run(oracle_lib, wid)
    o, hT = gpu_fwd(x)
    parity.check_fwd_outputs(o, hT, oo, ho, x["cu_seqlens"], TOL[sh.dtype], "workload %d" % wid)


# ----------------------------------------------------------- 32-token chunks
C32_CASES = [
    # B, T, H, Dk, Dv, gated, h0
    (2, 200, 3, 128, 128, True, True),
    (1, 31, 2, 64, 64, False, False),
    (1, 33, 2, 128, 256, True, True),
    (3, 64, 1, 128, 64, False, True),
    (1, 1, 2, 128, 128, True, True),
    (2, 95, 2, 64, 192, True, False),
    (1, 130, 1, 128, 1024, True, True),
    (2, 200, 4, 128, 256, True, True),    # N*H = 8
    (4, 97, 4, 128, 128, False, False),   # N*H = 16
]


@pytest.mark.parametrize("cfg", C32_CASES, ids=lambda c: "B%dT%dH%dk%dv%d-g%d-h%d" % c)
def test_fwd_chunk32_parity(oracle_lib, cfg):
    """The 32-token-chunk forward kernel against the oracle (the chunk size does
    not change the result beyond rounding)."""
    B, T, H, Dk, Dv, gated, h0 = cfg
    sh = Shape(B, T, H, Dk, Dv, torch.bfloat16, gated, h0)
    x = make_inputs(sh, seed=300 + T + Dv)
    check_fwd(x, torch.bfloat16, oracle_lib, "chunk 32 %s" % (cfg,), chunk=32)


def test_fwd_chunk32_varlen_ragged(oracle_lib):
    lens = (1, 31, 32, 33, 0, 100, 5)
    sh = Shape(1, sum(lens), 2, 128, 128, torch.bfloat16, True, True, lengths=lens)
    x = make_inputs(sh, seed=333)
    o, hT = check_fwd(x, torch.bfloat16, oracle_lib, "chunk 32 varlen", chunk=32)
    # the empty sequence passes its state through
    assert torch.equal(hT[4], x["h0"][4])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wid", [2, 3, 5])
def test_fwd_chunk32_full_size_every_pair(oracle_lib, wid):
    """The forward workloads at full size with 32-token chunks: every
    (sequence, head) pair and every chunk against the oracle."""
    sh = synth.WORKLOADS[wid]
    x, (oo, ho), _ = parity.oracle_run(oracle_lib, wid)
    d = to_dev(x)
    o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"], chunk=32)
    torch.cuda.synchronize()
    parity.check_fwd_outputs(o.cpu(), hT.cpu(), oo, ho, x["cu_seqlens"], TOL[sh.dtype],
                             "chunk 32 workload %d" % wid)
