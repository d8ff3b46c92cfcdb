"""Packed sequences are taken longest first by the sequential passes (an order
table the library builds on the device).  The order only decides which
workgroup runs when: every (sequence, head, d_v tile) and every (chunk, head)
is computed by the same arithmetic wherever it sits.  So permuting the
sequences of a pack must permute every output bit for bit: the forward pass,
the saving forward pass and both backward modes, for 64- and 32-token chunks.
Each pack mixes empty, single-token, boundary and long sequences, with the
longest placed first, last and in the middle.
"""
import pytest
import torch

import chunkwise_delta_rule_wy_amd as dn
from chunkwise_delta_rule_wy_amd.synth import Shape, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
LENS = (1, 130, 0, 700, 65, 64, 2100, 17)  # N * H = 32: the XCD-aware placement
H, DK, DV = 4, 128, 256
NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


def pack(x, lens, perm):
    """The inputs of the pack whose sequence i is sequence perm[i] of x."""
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    rows = lambda t: torch.cat([t[:, cu[j]:cu[j + 1]] for j in perm], dim=1).contiguous()
    y = {k: rows(x[k]) for k in ("q", "k", "v", "beta", "g", "dO")}
    y["h0"] = x["h0"][list(perm)].contiguous()
    y["dhT"] = x["dhT"][list(perm)].contiguous()
    new = [0]
    for j in perm:
        new.append(new[-1] + lens[j])
    y["cu_seqlens"] = torch.tensor(new, dtype=torch.int32)
    return y, cu, new


def run(y, chunk, mode):
    d = {k: v.to(DEV) for k, v in y.items()}
    if mode == "fwd":
        o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"], chunk=chunk)
        torch.cuda.synchronize()
        return {"o": o.cpu(), "hT": hT.cpu()}
    q = d["q"]
    ws = torch.empty(dn.bwd_workspace_bytes(1, q.shape[1], H, DK, DV, len(y["cu_seqlens"]) - 1, chunk=chunk),
                     dtype=torch.uint8, device=DEV)
    saved = mode == "saved"
    o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"], chunk=chunk,
                         save_workspace=ws if saved else None)
    gr = dn.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["dO"], d["dhT"], d["cu_seqlens"],
                      chunk=chunk, workspace=ws, saved=saved)
    torch.cuda.synchronize()
    out = {"o": o.cpu(), "hT": hT.cpu()}
    out.update({k: gr[k].cpu() for k in NAMES})
    return out


@pytest.mark.parametrize("mode", ["fwd", "saved", "recompute"])
@pytest.mark.parametrize("chunk", [64, 32])
def test_permuted_pack_permutes_every_output(mode, chunk):
    sh = Shape(1, sum(LENS), H, DK, DV, torch.bfloat16, True, True, backward=True, lengths=LENS)
    x = make_inputs(sh, seed=4242)
    ref = run(x, chunk, mode)
    for perm in ((6, 0, 1, 2, 3, 4, 5, 7), (7, 5, 4, 3, 2, 1, 0, 6), (0, 3, 6, 1, 4, 7, 2, 5)):
        y, cu, new = pack(x, LENS, perm)
        got = run(y, chunk, mode)
        for name, t in ref.items():
            if name in ("hT", "dh0"):
                assert torch.equal(got[name], t[list(perm)]), (name, perm)
                continue
            for i, j in enumerate(perm):
                a = got[name][:, new[i]:new[i + 1]]
                b = t[:, cu[j]:cu[j + 1]]
                assert torch.equal(a, b), (name, perm, i, j)
    print("mode %s, chunk %d: three permutations bit-identical" % (mode, chunk), flush=True)


@pytest.mark.parametrize("lens", [LENS, (5, 5, 0, 5, 64, 1, 64, 3), tuple(range(300, 0, -1)) + (0, 1000),
                                  tuple((7 * i) % 13 for i in range(2500))],  # several LDS tiles of lengths
                         ids=["pack", "ties", "302seqs", "2500seqs"])
def test_order_table_is_longest_first(lens):
    """dn_chunk_fwd leaves the order in the caller's workspace: the sequences
    by length, longest first, ties by index (checked through the C ABI)."""
    import ctypes
    h, dk, dv = 2, 64, 64
    sh = Shape(1, sum(lens), h, dk, dv, torch.bfloat16, True, True, lengths=lens)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in make_inputs(sh, seed=17).items()}
    lib = dn.load_library()
    s = dn._Shape(1, sum(lens), h, dk, dv, len(lens), 64, dn.DN_BF16)
    need = lib.dn_chunk_fwd_workspace(ctypes.byref(s))
    assert need >= 4 * len(lens)
    ws = torch.full((need // 4,), -1, dtype=torch.int32, device=DEV)
    o = torch.empty_like(d["v"])
    hT = torch.empty_like(d["h0"])
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.dn_chunk_fwd(ctypes.byref(s), P(d["q"]), P(d["k"]), P(d["v"]), P(d["beta"]), P(d["g"]), P(d["h0"]),
                          P(d["cu_seqlens"]), P(o), P(hT), P(ws), need,
                          ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    want = sorted(range(len(lens)), key=lambda i: (-lens[i], i))
    assert ws[:len(lens)].cpu().tolist() == want
    # and the outputs are those of the library's own call
    o2, hT2 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"])
    assert torch.equal(o, o2) and torch.equal(hT, hT2)
