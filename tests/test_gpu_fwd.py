"""GPU parity of the chunkwise forward pass and the decode step against the
fp64 oracle, through the C ABI.

Tolerances (relative L2 over a whole output tensor): 1e-4 for fp32 inputs and
2e-2 for bf16 inputs, on o and on the final state.  The oracle reads exactly
the bits the GPU reads (bf16 values upcast to fp64).
"""
import ctypes

import numpy as np
import pytest
import torch

import chunkwise_delta_rule_wy_amd as dn
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


def check_fwd(x, dtype, oracle_lib, label=""):
    o, hT = gpu_fwd(x)
    oo, ho = oracle_lib.fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["cu_seqlens"])
    eo, eh = rel_l2(o, oo), rel_l2(hT, ho)
    print("%s rel-L2 o %.3e hT %.3e" % (label, eo, eh), flush=True)
    assert np.isfinite(o.float().numpy()).all()
    assert eo <= TOL[dtype], eo
    assert eh <= TOL[dtype], eh
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


def test_fwd_deterministic_and_state_passing():
    sh = Shape(2, 333, 2, 128, 256, torch.bfloat16, True, True)
    x = make_inputs(sh, seed=11)
    o1, h1 = gpu_fwd(x)
    for _ in range(3):
        o2, h2 = gpu_fwd(x)
        assert torch.equal(o1, o2) and torch.equal(h1, h2)
    # Split at a chunk boundary: two segments equal one run up to rounding.  The
    # kernel carries the state scaled by a running product of decays and feeds
    # it to the MFMA in bf16, so the two runs round it differently: they agree
    # to the bf16 level, far inside the parity tolerance.
    T1 = 128
    xa = {kk: (vv[:, :T1].contiguous() if kk in ("q", "k", "v", "beta", "g") else vv)
          for kk, vv in x.items()}
    oa, ha = gpu_fwd(xa)
    xb = {kk: (vv[:, T1:].contiguous() if kk in ("q", "k", "v", "beta", "g") else vv)
          for kk, vv in x.items()}
    xb["h0"] = ha
    ob, hb = gpu_fwd(xb)
    assert rel_l2(hb, h1) < 1e-2
    assert rel_l2(torch.cat([oa, ob], 1), o1) < 1e-2


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
    eo, es = rel_l2(o.cpu(), oo), rel_l2(st.cpu(), so)
    print("decode rel-L2 o %.3e state %.3e" % (eo, es), flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


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
def sample_pairs(N, H, k, seed):
    rng = np.random.default_rng(seed)
    idx = rng.choice(N * H, size=min(k, N * H), replace=False)
    return [(int(i) // H, int(i) % H) for i in idx]


@pytest.mark.parametrize("wid", [2, 3, 5])
def test_fwd_full_size_sampled(oracle_lib, wid):
    sh = synth.WORKLOADS[wid]
    x = synth.workload_inputs(wid)
    o, hT = gpu_fwd(x)
    assert np.isfinite(o.float().numpy()).all()
    cu = x["cu_seqlens"]
    pairs = sample_pairs(sh.n_seqs, sh.H, 6, wid)
    if wid == 5:
        # the longest sequence, plus a random sample
        pairs = [(2, 0)] + pairs[:4]
    for n, h in pairs:
        if cu is None:
            b, s, e = n, 0, sh.T
        else:
            b, s, e = 0, int(cu[n]), int(cu[n + 1])
        sl = lambda t: t[b:b + 1, s:e, h:h + 1].contiguous()
        oo, ho = oracle_lib.fwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["beta"]),
                                None if x["g"] is None else sl(x["g"]),
                                None if x["h0"] is None else x["h0"][n:n + 1, h:h + 1].contiguous())
        eo = rel_l2(o[b, s:e, h], oo[0, :, 0])
        eh = rel_l2(hT[n, h], ho[0, 0])
        print("workload %d pair (%d,%d) rel-L2 o %.3e hT %.3e" % (wid, n, h, eo, eh), flush=True)
        assert eo <= TOL[sh.dtype] and eh <= TOL[sh.dtype]


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
]


@pytest.mark.parametrize("cfg", C32_CASES, ids=lambda c: "B%dT%dH%dk%dv%d-g%d-h%d" % c)
def test_fwd_chunk32_parity(oracle_lib, cfg):
    """The 32-token-chunk forward kernel against the oracle (the chunk size does
    not change the result beyond rounding)."""
    B, T, H, Dk, Dv, gated, h0 = cfg
    sh = Shape(B, T, H, Dk, Dv, torch.bfloat16, gated, h0)
    x = make_inputs(sh, seed=300 + T + Dv)
    d = to_dev(x)
    o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], chunk=32)
    torch.cuda.synchronize()
    oo, ho = oracle_lib.fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"])
    eo, eh = rel_l2(o.cpu(), oo), rel_l2(hT.cpu(), ho)
    print("chunk 32 %s rel-L2 o %.3e hT %.3e" % (cfg, eo, eh), flush=True)
    assert eo <= TOL[torch.bfloat16] and eh <= TOL[torch.bfloat16], (eo, eh)


def test_fwd_chunk32_varlen_ragged(oracle_lib):
    lens = (1, 31, 32, 33, 0, 100, 5)
    sh = Shape(1, sum(lens), 2, 128, 128, torch.bfloat16, True, True, lengths=lens)
    x = make_inputs(sh, seed=333)
    d = to_dev(x)
    o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"], chunk=32)
    torch.cuda.synchronize()
    oo, ho = oracle_lib.fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["cu_seqlens"])
    eo, eh = rel_l2(o.cpu(), oo), rel_l2(hT.cpu(), ho)
    print("chunk 32 varlen rel-L2 o %.3e hT %.3e" % (eo, eh), flush=True)
    assert eo <= TOL[torch.bfloat16] and eh <= TOL[torch.bfloat16], (eo, eh)
    # the empty sequence passes its state through
    assert torch.equal(hT[4].cpu(), x["h0"][4])


@pytest.mark.parametrize("wid", [2, 3])
def test_fwd_chunk32_full_size_sampled(oracle_lib, wid):
    """The forward workloads at full size with 32-token chunks: three
    (batch, head) pairs against the oracle."""
    sh = synth.WORKLOADS[wid]
    x = synth.workload_inputs(wid)
    d = to_dev(x)
    o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], chunk=32)
    torch.cuda.synchronize()
    o, hT = o.cpu(), hT.cpu()
    rng = np.random.default_rng(32 + wid)
    for idx in rng.choice(sh.B * sh.H, size=3, replace=False):
        b, h = int(idx) // sh.H, int(idx) % sh.H
        sl = lambda t: None if t is None else t[b:b + 1, :, h:h + 1].contiguous()
        st = lambda t: None if t is None else t[b:b + 1, h:h + 1].contiguous()
        oo, ho = oracle_lib.fwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["beta"]), sl(x["g"]), st(x["h0"]))
        eo, eh = rel_l2(o[b:b + 1, :, h:h + 1], oo), rel_l2(hT[b:b + 1, h:h + 1], ho)
        print("chunk 32 workload %d pair (%d,%d) rel-L2 o %.3e hT %.3e" % (wid, b, h, eo, eh), flush=True)
        assert eo <= TOL[torch.bfloat16] and eh <= TOL[torch.bfloat16], (eo, eh)
