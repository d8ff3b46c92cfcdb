"""dn_chunk_bwd_noalloc (the recomputing backward pass with the library's
static scratch buffer in place of a workspace) through the C ABI, against
dn_chunk_bwd on the same inputs.  Both run the same kernels, so the gradients
must be equal bit for bit; they are also checked against the fp64 oracle
(relative L2 2e-2 per tensor and per (sequence, head) pair).  Two calls in a
row, the second with a smaller input, show that a call does not depend on
what the previous call left in the shared buffer."""
import ctypes

import pytest
import torch

import chunkwise_delta_rule_wy_amd as dn
import parity
from chunkwise_delta_rule_wy_amd.synth import Shape, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")
DN_ESCRATCH = 5
SCRATCH = 64 << 20


def _dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def _both(x, chunk=64):
    d = _dev(x)
    args = (d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["dO"], d["dhT"], d["cu_seqlens"])
    ref = dn.chunk_bwd(*args, chunk=chunk)
    got = dn.chunk_bwd_noalloc(*args, chunk=chunk)
    torch.cuda.synchronize()
    return ({k: (None if v is None else v.cpu()) for k, v in ref.items()},
            {k: (None if v is None else v.cpu()) for k, v in got.items()})


def _check(x, oracle_lib, label, chunk=64):
    ref, got = _both(x, chunk)
    for name in NAMES:
        if ref[name] is None:
            assert got[name] is None, name
        else:
            assert torch.equal(ref[name], got[name]), (label, name)
    o = oracle_lib.bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["dO"], x["dhT"],
                       cu_seqlens=x["cu_seqlens"])
    parity.check_grads(got, o, x["cu_seqlens"], 2e-2, label)


def test_noalloc_equals_workspace_entry_point_twice(oracle_lib):
    # first call: close to the largest shape the buffer holds (B 1, T 2048,
    # H 16, dk = dv = 128 needs 34.6 MB of the 64 MiB); second: smaller and packed
    big = Shape(1, 2048, 16, 128, 128, torch.bfloat16, True, True, backward=True)
    assert dn.bwd_workspace_bytes(1, 2048, 16, 128, 128) <= SCRATCH
    _check(make_inputs(big, seed=501), oracle_lib, "noalloc call 1")
    lens = (70, 0, 129, 5)
    small = Shape(1, sum(lens), 3, 128, 256, torch.bfloat16, True, False, backward=True, lengths=lens)
    _check(make_inputs(small, seed=502), oracle_lib, "noalloc call 2")


def test_noalloc_32_token_chunks(oracle_lib):
    # twice the chunk states of 64-token chunks; two calls, the second smaller and packed
    sh = Shape(1, 1024, 16, 128, 128, torch.bfloat16, True, True, backward=True)
    assert dn.bwd_workspace_bytes(1, 1024, 16, 128, 128, chunk=32) <= SCRATCH
    _check(make_inputs(sh, seed=511), oracle_lib, "noalloc C=32 call 1", chunk=32)
    lens = (31, 0, 33, 65)
    small = Shape(1, sum(lens), 2, 64, 128, torch.bfloat16, True, True, backward=True, lengths=lens)
    _check(make_inputs(small, seed=512), oracle_lib, "noalloc C=32 call 2", chunk=32)


def test_noalloc_ungated_after_gated(oracle_lib):
    sh = Shape(2, 200, 4, 64, 192, torch.bfloat16, False, True, backward=True)
    _check(make_inputs(sh, seed=503), oracle_lib, "noalloc ungated")


def test_noalloc_rejects_a_shape_beyond_the_buffer():
    sh = Shape(4, 4096, 16, 128, 256, torch.bfloat16, True, True, backward=True)
    assert dn.bwd_workspace_bytes(4, 4096, 16, 128, 256) > SCRATCH
    d = _dev(make_inputs(Shape(1, 64, 1, 128, 256, torch.bfloat16, True, True, backward=True), seed=1))
    s = dn._Shape(sh.B, sh.T, sh.H, sh.Dk, sh.Dv, sh.B, 64, 1)
    P = ctypes.c_void_p
    lib = dn.load_library()
    fake = P(d["q"].data_ptr())  # never read: the call returns before any launch
    st = lib.dn_chunk_bwd_noalloc(ctypes.byref(s), fake, fake, fake, fake, fake, fake, None, fake, fake,
                                  fake, fake, fake, fake, fake, fake, P(torch.cuda.current_stream().cuda_stream))
    assert st == DN_ESCRATCH
    assert lib.dn_status_str(st).decode().startswith("DN_ESCRATCH")
