"""GPU parity of the depthwise causal short convolution (``dn_short_conv``)
and its backward (``dn_short_conv_bwd``) against the fp64 oracle, through the
C ABI.

The kernels compute in fp32 on exactly upcast inputs: y within relative L2
1e-6 of the oracle for fp32 and within one bf16 rounding (relative L2 4e-3)
when y is stored in bf16; dx within 1e-6; dw, a sum over every token in
fp32, within 1e-5.  Cases span several 32-token runs and 512-channel groups
with ragged tails, packed sequences with empty and one-token members, every
width 1..4, and the training shapes (B=4 T=4096 H=16 d=128, and the packed
65536-token, H=32 input) on every head.  The variant fused
with the per-head L2 normalisation is compared with the oracle's convolution
followed by its prologue normalisation, and a whole layer (projections through
the convolutions, the chunkwise passes and back) with the oracle's composition.
"""
import numpy as np
import pytest
import torch

import chunkwise_delta_rule_wy_amd as dn
import parity
from chunkwise_delta_rule_wy_amd.synth import conv_inputs, rel_l2

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
YTOL = {torch.float32: 1e-6, torch.bfloat16: 4e-3}


def run(x, w, dy, cu):
    d = lambda t: None if t is None else t.to(DEV)
    xd, wd, dyd, cud = d(x), d(w), d(dy), d(cu)
    y = dn.short_conv(xd, wd, cud)
    dx, dw = dn.short_conv_bwd(xd, wd, dyd, cud)
    torch.cuda.synchronize()
    return y.cpu(), dx.cpu(), dw.cpu()


def check(oracle_lib, inp):
    x, w, dy, cu = inp["x"], inp["w"], inp["dy"], inp["cu_seqlens"]
    y, dx, dw = run(x, w, dy, cu)
    ry = oracle_lib.short_conv(x, w, cu)
    rdx, rdw = oracle_lib.short_conv_bwd(x, w, dy, cu)
    # y and dx over the whole tensor, every (sequence, head) pair and every chunk
    parity.check("y", parity.token_errors(y, ry, cu), YTOL[x.dtype], "conv")
    parity.check("dx", parity.token_errors(dx, rdx, cu), 1e-6, "conv")
    edw = rel_l2(dw, rdw)
    print("conv rel-L2 dw %.2e" % edw, flush=True)
    assert edw <= 1e-5
    return y, dx, dw


@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_conv_parity_fixed_length(oracle_lib, W, dtype):
    # T = 300: nine 32-token runs and a ragged tail; C = 2 x 320 = 640: two channel groups, one partial
    check(oracle_lib, conv_inputs(3, 300, 2, 320, W, dtype, seed=1210 + W))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_conv_parity_packed(oracle_lib, dtype):
    lengths = [37, 0, 1, 130, 5, 64, 33]
    inp = conv_inputs(1, sum(lengths), 3, 24, 4, dtype, seed=1220, lengths=lengths)
    y, dx, _ = check(oracle_lib, inp)
    # nothing leaks across a boundary: the first token of each sequence sees only itself
    cu = inp["cu_seqlens"].tolist()
    x = inp["x"].double()
    for n, L in enumerate(lengths):
        if L:
            t = cu[n]
            ref = (inp["w"][:, :, -1].double() * x[0, t]).float()
            assert torch.allclose(y[0, t].float(), ref.to(y.dtype).float(), rtol=4e-3, atol=1e-6)


def test_conv_short_sequences_and_one_token(oracle_lib):
    # sequences shorter than the taps, and T = 1
    check(oracle_lib, conv_inputs(4, 2, 1, 8, 4, torch.float32, seed=1230))
    check(oracle_lib, conv_inputs(2, 1, 2, 16, 3, torch.bfloat16, seed=1231))


def test_conv_empty_input_clears_dw():
    w = torch.randn(2, 16, 4, device=DEV)
    x = torch.empty(1, 0, 2, 16, dtype=torch.bfloat16, device=DEV)
    dy = torch.empty(1, 0, 2, 16, device=DEV)
    assert dn.short_conv(x, w).shape == x.shape
    dx, dw = dn.short_conv_bwd(x, w, dy)
    torch.cuda.synchronize()
    assert dx.numel() == 0 and torch.count_nonzero(dw).item() == 0


def test_conv_repeat_calls_agree():
    # dw is cleared by every call: two calls give the same result up to summation order
    inp = conv_inputs(2, 500, 4, 128, 4, torch.bfloat16, seed=1240)
    _, dx1, dw1 = run(inp["x"], inp["w"], inp["dy"], None)
    _, dx2, dw2 = run(inp["x"], inp["w"], inp["dy"], None)
    assert torch.equal(dx1, dx2)
    assert rel_l2(dw1, dw2) < 1e-6


@pytest.mark.timeout(900)
def test_conv_full_size(oracle_lib):
    # the projections of the training shape: B=4 T=4096 H=16 d=128, W=4, every head
    check(oracle_lib, conv_inputs(4, 4096, 16, 128, 4, torch.bfloat16, seed=1250))


@pytest.mark.timeout(900)
def test_conv_full_size_packed(oracle_lib):
    from chunkwise_delta_rule_wy_amd.synth import VARLEN_LENGTHS
    inp = conv_inputs(1, sum(VARLEN_LENGTHS), 32, 128, 4, torch.bfloat16, seed=1251, lengths=list(VARLEN_LENGTHS))
    check(oracle_lib, inp)


def l2_reference(oracle_lib, x, w, dy, cu):
    """The fused pass as a composition of the oracle's pinned functions: the
    convolution, then the prologue's row normalisation (and their backward)."""
    z = oracle_lib.short_conv(x, w, cu)
    zeros = np.zeros(z.shape[:3])
    y = oracle_lib.prologue(z, z, zeros)[0]
    dz = oracle_lib.prologue_bwd(z, z, zeros, None, 1.0, dy, dy, zeros)[0]
    dx, dw = oracle_lib.short_conv_bwd(x, w, dz, cu)
    return y, dx, dw


def check_l2(oracle_lib, inp):
    x, w, dy, cu = inp["x"], inp["w"], inp["dy"], inp["cu_seqlens"]
    d = lambda t: None if t is None else t.to(DEV)
    y = dn.short_conv(d(x), d(w), d(cu), l2norm=True)
    dx, dw = dn.short_conv_bwd(d(x), d(w), d(dy), d(cu), l2norm=True)
    torch.cuda.synchronize()
    y, dx, dw = y.cpu(), dx.cpu(), dw.cpu()
    ry, rdx, rdw = l2_reference(oracle_lib, x, w, dy, cu)
    parity.check("y", parity.token_errors(y, ry, cu), YTOL[x.dtype], "conv l2")
    parity.check("dx", parity.token_errors(dx, rdx, cu), 1e-5, "conv l2")
    edw = rel_l2(dw, rdw)
    print("conv l2 rel-L2 dw %.2e" % edw, flush=True)
    assert edw <= 1e-5
    return y, dx, dw


@pytest.mark.parametrize("W", [1, 2, 4])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_conv_l2_parity(oracle_lib, W, D, dtype):
    inp = conv_inputs(2, 150, 5, D, W, dtype, seed=1260 + W + D)
    inp["w"][3] = 0.0  # head 3 convolves to zero rows: they stay zero, with zero gradients
    y, dx, dw = check_l2(oracle_lib, inp)
    assert torch.count_nonzero(y[:, :, 3]).item() == 0 and torch.count_nonzero(dx[:, :, 3]).item() == 0
    n = y[:, :, :3].double().norm(dim=-1)
    assert (n - 1).abs().max().item() < 1e-2  # unit rows (bf16 rounding included)


def test_conv_l2_packed(oracle_lib):
    lengths = [37, 0, 1, 130, 5, 64, 2]
    check_l2(oracle_lib, conv_inputs(1, sum(lengths), 4, 128, 4, torch.bfloat16, seed=1270, lengths=lengths))


@pytest.mark.timeout(900)
def test_conv_l2_full_size(oracle_lib):
    check_l2(oracle_lib, conv_inputs(4, 4096, 16, 128, 4, torch.bfloat16, seed=1271))


def test_layer_composition(oracle_lib):
    """Projections to gradients through the library: q, k by the fused
    convolution and normalisation, v by the plain convolution, the chunkwise
    forward and backward (bf16), then the convolutions' backward; against the
    same composition of the oracle's functions in fp64 (relative L2 2e-2, the
    bf16 recurrence's bar)."""
    B, T, H, D, W = 2, 150, 2, 64, 4
    xq = conv_inputs(B, T, H, D, W, torch.bfloat16, seed=1280)
    xk = conv_inputs(B, T, H, D, W, torch.bfloat16, seed=1281)
    xv = conv_inputs(B, T, H, D, W, torch.bfloat16, seed=1282)
    gen = torch.Generator("cpu").manual_seed(1283)
    beta = torch.sigmoid(torch.randn(B, T, H, generator=gen))
    g = -0.1 * torch.nn.functional.softplus(torch.randn(B, T, H, generator=gen))
    dO = torch.randn(B, T, H, D, generator=gen).to(torch.bfloat16)
    dv_ = lambda t: t.to(DEV)
    q = dn.short_conv(dv_(xq["x"]), dv_(xq["w"]), l2norm=True)
    k = dn.short_conv(dv_(xk["x"]), dv_(xk["w"]), l2norm=True)
    v = dn.short_conv(dv_(xv["x"]), dv_(xv["w"]))
    o, hT = dn.chunk_fwd(q, k, v, dv_(beta), dv_(g), None)
    gr = dn.chunk_bwd(q, k, v, dv_(beta), dv_(g), None, dv_(dO))
    dxq, dwq = dn.short_conv_bwd(dv_(xq["x"]), dv_(xq["w"]), gr["dq"], l2norm=True)
    dxk, dwk = dn.short_conv_bwd(dv_(xk["x"]), dv_(xk["w"]), gr["dk"], l2norm=True)
    dxv, dwv = dn.short_conv_bwd(dv_(xv["x"]), dv_(xv["w"]), gr["dv"])
    torch.cuda.synchronize()

    zeros = np.zeros((B, T, H))
    zq = oracle_lib.short_conv(xq["x"], xq["w"])
    zk = oracle_lib.short_conv(xk["x"], xk["w"])
    rq = oracle_lib.prologue(zq, zq, zeros)[0]
    rk = oracle_lib.prologue(zk, zk, zeros)[0]
    rv = oracle_lib.short_conv(xv["x"], xv["w"])
    ro, _ = oracle_lib.fwd(rq, rk, rv, beta, g, None)
    rg = oracle_lib.bwd(rq, rk, rv, beta, g, None, dO, None)
    rdzq = oracle_lib.prologue_bwd(zq, zq, zeros, None, 1.0, rg["dq"], rg["dq"], zeros)[0]
    rdzk = oracle_lib.prologue_bwd(zk, zk, zeros, None, 1.0, rg["dk"], rg["dk"], zeros)[0]
    rdxq, rdwq = oracle_lib.short_conv_bwd(xq["x"], xq["w"], rdzq)
    rdxk, rdwk = oracle_lib.short_conv_bwd(xk["x"], xk["w"], rdzk)
    rdxv, rdwv = oracle_lib.short_conv_bwd(xv["x"], xv["w"], rg["dv"])
    errs = {"o": rel_l2(o.cpu(), ro), "dxq": rel_l2(dxq.cpu(), rdxq), "dwq": rel_l2(dwq.cpu(), rdwq),
            "dxk": rel_l2(dxk.cpu(), rdxk), "dwk": rel_l2(dwk.cpu(), rdwk), "dxv": rel_l2(dxv.cpu(), rdxv),
            "dwv": rel_l2(dwv.cpu(), rdwv), "dbeta": rel_l2(gr["dbeta"].cpu(), rg["dbeta"]),
            "dg": rel_l2(gr["dg"].cpu(), rg["dg"])}
    print({k_: "%.2e" % e for k_, e in errs.items()}, flush=True)
    assert max(errs.values()) <= 2e-2


@pytest.mark.parametrize("l2norm", [False, True])
def test_conv_autograd(oracle_lib, l2norm):
    inp = conv_inputs(2, 70, 3, 64, 3, torch.float32, seed=1290)
    x = inp["x"].to(DEV).requires_grad_(True)
    w = inp["w"].to(DEV).requires_grad_(True)
    dy = inp["dy"].to(DEV)
    y = dn.short_conv_fn(x, w, l2norm=l2norm)
    (y * dy).sum().backward()
    torch.cuda.synchronize()
    if l2norm:
        _, rdx, rdw = l2_reference(oracle_lib, inp["x"], inp["w"], inp["dy"], None)
    else:
        rdx, rdw = oracle_lib.short_conv_bwd(inp["x"], inp["w"], inp["dy"])
    assert rel_l2(x.grad.cpu(), rdx) <= 1e-5 and rel_l2(w.grad.cpu(), rdw) <= 1e-5
