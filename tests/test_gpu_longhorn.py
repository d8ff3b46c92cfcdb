"""GPU parity of the Longhorn recurrence (Gated DeltaNet review thread,
Table 1, row "Longhorn") against the fp64 oracle, through the C ABI.

The step size eps = beta / (1 + beta |k|^2) and its backward are plain fp32
arithmetic on exactly upcast inputs: within 1e-5 relative of the oracle.  The
recurrence runs in the chunkwise kernels at beta := eps (bf16 inputs): within
relative L2 2e-2 for o, hT and every gradient, like the delta rule.  Keys are
scaled to norms between 0.5 and 2 (except in the full-size case, which uses
the benchmark's unit keys), so that eps depends on |k|.
"""
import ctypes

import numpy as np
import pytest
import torch

import chunkwise_delta_rule_wy_amd as dn
import parity
from chunkwise_delta_rule_wy_amd import synth
from chunkwise_delta_rule_wy_amd.synth import Shape, make_inputs, rel_l2

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 2e-2
NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def scale_keys(x, seed):
    gen = torch.Generator("cpu").manual_seed(seed)
    k = x["k"]
    s = 0.5 + 1.5 * torch.rand(k.shape[:-1] + (1,), generator=gen)
    x["k"] = (k.float() * s).to(k.dtype).contiguous()
    x["beta"] = (x["beta"] * 3.0).contiguous()  # beta in (0, 3)
    return x


def max_rel(x, y):
    x = x.detach().double().cpu().numpy() if isinstance(x, torch.Tensor) else np.asarray(x)
    y = np.asarray(y, dtype=np.float64)
    return float(np.max(np.abs(x - y) / np.maximum(np.abs(y), 1e-30)))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("Dk", [64, 128])
def test_longhorn_eps_and_backward(oracle_lib, dtype, Dk):
    sh = Shape(2, 77, 3, Dk, 64, dtype, True, False, backward=True)
    x = scale_keys(make_inputs(sh, seed=50 + Dk), seed=51)
    d = to_dev(x)
    eps = dn.longhorn_eps(d["k"], d["beta"])
    torch.cuda.synchronize()
    assert max_rel(eps, oracle_lib.longhorn_eps(x["k"], x["beta"])) < 1e-5

    gen = torch.Generator("cpu").manual_seed(52)
    deps = torch.randn(x["beta"].shape, generator=gen)
    dk0 = torch.randn(x["k"].shape, generator=gen)
    dk = dk0.to(DEV)
    dbeta = dn.longhorn_eps_bwd(d["k"], d["beta"], deps.to(DEV), dk)
    torch.cuda.synchronize()
    ref_db, ref_dk = oracle_lib.longhorn_eps_bwd(x["k"], x["beta"], deps)
    assert max_rel(dbeta, ref_db) < 1e-5
    assert rel_l2(dk.cpu().double() - dk0.double(), ref_dk) < 1e-5

    # dbeta may overwrite deps in place
    lib = dn.load_library()
    dd = deps.to(DEV)
    dk2 = dk0.to(DEV)
    B, T, H = x["beta"].shape
    st = lib.dn_longhorn_eps_bwd(B, T, H, Dk, 1 if dtype == torch.bfloat16 else 0,
                                 ctypes.c_void_p(d["k"].data_ptr()), ctypes.c_void_p(d["beta"].data_ptr()),
                                 ctypes.c_void_p(dd.data_ptr()), ctypes.c_void_p(dd.data_ptr()),
                                 ctypes.c_void_p(dk2.data_ptr()),
                                 ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(dd, dbeta) and torch.equal(dk2, dk)


def test_longhorn_decode_step(oracle_lib):
    x = synth.decode_inputs(B=8, H=4, Dk=128, Dv=128)
    gen = torch.Generator("cpu").manual_seed(53)
    x["k"] = (x["k"].float() * (0.5 + 1.5 * torch.rand(8, 4, 1, generator=gen))).to(torch.bfloat16)
    d = to_dev(x)
    st = d["state"].clone()
    o = dn.recurrent_step(d["q"], d["k"], d["v"], dn.longhorn_eps(d["k"], d["beta"]), d["g"], st)
    torch.cuda.synchronize()
    ro, rst = oracle_lib.step(x["q"], x["k"], x["v"], oracle_lib.longhorn_eps(x["k"], x["beta"]),
                              x["g"], x["state"])
    assert rel_l2(o.cpu(), ro) < TOL and rel_l2(st.cpu(), rst) < 1e-4


CASES = [
    # B, T, H, Dk, Dv, gated, h0
    (2, 150, 2, 128, 128, False, False),
    (2, 131, 2, 128, 256, True, True),
    (1, 200, 3, 64, 64, False, True),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "B%dT%dH%dk%dv%d-g%d-h%d" % c)
def test_longhorn_fwd_bwd_parity(oracle_lib, cfg):
    B, T, H, Dk, Dv, gated, h0 = cfg
    sh = Shape(B, T, H, Dk, Dv, torch.bfloat16, gated, h0, backward=True)
    x = scale_keys(make_inputs(sh, seed=60 + T), seed=61)
    d = to_dev(x)
    o, hT = dn.longhorn_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])
    gr = dn.longhorn_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["dO"], d["dhT"])
    torch.cuda.synchronize()
    ro, rhT = oracle_lib.longhorn_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"])
    ref = oracle_lib.longhorn_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["dO"], x["dhT"])
    errs = {"o": rel_l2(o.cpu(), ro), "hT": rel_l2(hT.cpu(), rhT)}
    for name in NAMES:
        if ref[name] is None:
            assert gr[name] is None
            continue
        errs[name] = rel_l2(gr[name].cpu(), ref[name])
    print(cfg, " ".join("%s %.2e" % kv for kv in errs.items()), flush=True)
    for name, e in errs.items():
        assert e <= TOL, (name, e)


@pytest.mark.timeout(900)
def test_longhorn_full_size_every_pair(oracle_lib):
    """The benchmark's Longhorn step (B=4 T=4096 H=16 dk=128 dv=256, unit keys):
    every output and gradient of every (batch, head) pair and every chunk
    against the oracle."""
    x = synth.workload_inputs(4)
    d = to_dev(x)
    o, hT = dn.longhorn_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])
    gr = dn.longhorn_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["dO"], d["dhT"])
    torch.cuda.synchronize()
    o, hT = o.cpu(), hT.cpu()
    gr = {k: v.cpu() for k, v in gr.items()}
    del d
    ro, rhT = oracle_lib.longhorn_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"])
    ref = oracle_lib.longhorn_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["dO"], x["dhT"])
    parity.check_fwd_outputs(o, hT, ro, rhT, None, TOL, "longhorn workload 4")
    parity.check_grads(gr, ref, None, TOL, "longhorn workload 4")


FOLDED_CASES = [
    # B, T, H, Dk, Dv, gated, h0, lengths
    (2, 150, 2, 128, 128, True, True, None),
    (1, 200, 3, 64, 192, False, False, None),
    (1, 263, 2, 128, 256, True, True, (1, 63, 64, 0, 135)),
]


@pytest.mark.parametrize("cfg", FOLDED_CASES, ids=lambda c: "B%dT%dH%dk%dv%d-g%d-h%d-%s" % (
    c[:7] + ("packed" if c[7] else "fixed",)))
def test_longhorn_folded_backward(oracle_lib, cfg):
    """dn_chunk_bwd_longhorn (the step size's backward folded into the chunk-
    gradient kernel, after the state-saving forward pass at beta := eps)
    against dn_chunk_bwd_saved followed by dn_longhorn_eps_bwd: dq, dv, dg,
    dh0 bit for bit, dk and dbeta up to rounding; and against the oracle."""
    B, T, H, Dk, Dv, gated, h0, lens = cfg
    sh = Shape(B, T, H, Dk, Dv, torch.bfloat16, gated, h0, backward=True, lengths=lens)
    x = scale_keys(make_inputs(sh, seed=60 + T), seed=61)
    x["beta"][0, 2, 0] = 0.0  # a zero step
    d = to_dev(x)
    eps = dn.longhorn_eps(d["k"], d["beta"])
    ws = torch.empty(dn.bwd_workspace_bytes(B, T, H, Dk, Dv, sh.n_seqs), dtype=torch.uint8, device=DEV)
    o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], eps, d["g"], d["h0"], d["cu_seqlens"], save_workspace=ws)
    gr = dn.chunk_bwd(d["q"], d["k"], d["v"], eps, d["g"], d["h0"], d["dO"], d["dhT"], d["cu_seqlens"],
                      workspace=ws, saved=True)
    comp_db = dn.longhorn_eps_bwd(d["k"], d["beta"], gr["dbeta"], gr["dk"])
    fo = dn.chunk_bwd(d["q"], d["k"], d["v"], eps, d["g"], d["h0"], d["dO"], d["dhT"], d["cu_seqlens"],
                      workspace=ws, saved=True, longhorn_beta=d["beta"])
    torch.cuda.synchronize()
    for name in ("dq", "dv", "dg", "dh0"):
        if gr[name] is None:
            assert fo[name] is None
        else:
            assert torch.equal(fo[name], gr[name]), name
    for name, mine, ref in (("dk", fo["dk"], gr["dk"]), ("dbeta", fo["dbeta"], comp_db)):
        e = rel_l2(mine.cpu(), ref.cpu().double().numpy())
        print(cfg, name, "folded vs composed rel-L2 %.2e" % e, flush=True)
        assert e < 1e-5, (name, e)
    ref = oracle_lib.longhorn_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["dO"], x["dhT"],
                                  cu_seqlens=x["cu_seqlens"])
    for name in NAMES:
        if ref[name] is None:
            continue
        e = rel_l2(fo[name].cpu(), ref[name])
        print(cfg, name, "folded vs oracle rel-L2 %.2e" % e, flush=True)
        assert e <= TOL, (name, e)
