"""The library's calls can be captured in a HIP graph: they only enqueue
kernels on the caller's stream (no allocation, no memset, no
synchronisation).  The training pair (forward storing the chunk states, the
backward reading them) and the short convolution's pair are captured once and
replayed three times, with other eager work and synchronisations between the
replays; every replay must reproduce the eager results (bit for bit for the
chunkwise passes and dx; dw, summed with atomic adds, to 1e-6)."""
import pytest
import torch

import chunkwise_delta_rule_wy_amd as dn
from chunkwise_delta_rule_wy_amd.synth import Shape, conv_inputs, make_inputs, rel_l2

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_training_pair_replays_in_a_graph():
    sh = Shape(2, 300, 2, 128, 128, torch.bfloat16, gated=True, has_h0=True, backward=True)
    x = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in make_inputs(sh, seed=1300).items()}
    ws = torch.empty(dn.bwd_workspace_bytes(sh.B, sh.T, sh.H, sh.Dk, sh.Dv), dtype=torch.uint8, device=DEV)
    cx = conv_inputs(2, 300, 2, 128, 4, torch.bfloat16, seed=1301)
    cx = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in cx.items()}

    def step():
        o, hT = dn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], save_workspace=ws)
        gr = dn.chunk_bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["dO"], x["dhT"],
                          workspace=ws, saved=True)
        y = dn.short_conv(cx["x"], cx["w"], l2norm=True)
        dxc, dwc = dn.short_conv_bwd(cx["x"], cx["w"], cx["dy"], l2norm=True)
        return [o, hT] + [gr[k] for k in ("dq", "dk", "dv", "dbeta", "dg", "dh0")] + [y, dxc, dwc]

    ref = [t.clone() for t in step()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    # other eager work in between: a call on different inputs, then a synchronisation
    other = make_inputs(sh, seed=1302)
    other = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in other.items()}
    for rep in range(3):
        dn.chunk_fwd(other["q"], other["k"], other["v"], other["beta"], other["g"], other["h0"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(out, ref)):
            if i == len(ref) - 1:  # dw: atomic adds
                assert rel_l2(a, b) < 1e-6, (rep, i)
            else:
                assert torch.equal(a, b), (rep, i)
        print("replay %d matches the eager results" % rep, flush=True)
