"""Run-to-run repeatability of the chunk kernels at the full workload sizes.

The kernels separate MFMA results from their later VALU and memory reads by
explicit wait states where control flow lies between them (the matrix pipeline
does not interlock such reads).  A missing wait state shows as a result that
changes from run to run, so every kernel is run repeatedly at the sizes and in
the launch configuration the benchmark uses (every workgroup placement, every
partial chunk of the packed workload) and each output is compared bit for bit
with the first run.  The kernels use no atomics, so any difference is an error.
"""
import pytest
import torch

import chunkwise_delta_rule_wy_amd as dn
from chunkwise_delta_rule_wy_amd import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
REPEATS = 8


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def assert_repeats(run, label):
    first = [t.clone() for t in run()]
    for rep in range(1, REPEATS):
        again = run()
        for i, (a, b) in enumerate(zip(first, again)):
            assert torch.equal(a, b), f"{label}: output {i} differs on repeat {rep}"
    print(f"{label}: {REPEATS} runs bit-identical", flush=True)


@pytest.mark.parametrize("wid", [2, 3, 5])
def test_forward_repeats(wid):
    d = to_dev(synth.workload_inputs(wid))

    def run():
        o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"])
        return o, hT

    assert_repeats(run, f"forward, workload {wid}")


def test_forward_32_token_chunks_repeats():
    d = to_dev(synth.workload_inputs(3))

    def run():
        return dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], chunk=32)

    assert_repeats(run, "forward, 32-token chunks, workload 3")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("wid,chunk", [(4, 64), (6, 64), (4, 32)])
@pytest.mark.parametrize("saved", [True, False])
def test_training_pair_repeats(wid, chunk, saved):
    d = to_dev(synth.workload_inputs(wid))
    q, v = d["q"], d["v"]
    N = q.shape[0] if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
    ws = torch.empty(dn.bwd_workspace_bytes(q.shape[0], q.shape[1], q.shape[2], q.shape[3], v.shape[-1], N,
                                            chunk=chunk), dtype=torch.uint8, device=DEV)
    names = ("dq", "dk", "dv", "dbeta", "dg", "dh0")

    def run():
        o, hT = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"], chunk=chunk,
                             save_workspace=ws if saved else None)
        gr = dn.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["dO"], d["dhT"],
                          d["cu_seqlens"], chunk=chunk, workspace=ws, saved=saved)
        return [o, hT] + [gr[n] for n in names]

    assert_repeats(run, f"forward + backward ({'saved states' if saved else 'recompute'}), workload {wid}, "
                        f"{chunk}-token chunks")


def test_decode_repeats():
    d = to_dev(synth.decode_inputs())
    s0 = d["state"].clone()

    def run():
        st = s0.clone()
        o = dn.recurrent_step(d["q"], d["k"], d["v"], d["beta"], d["g"], st)
        return o, st

    assert_repeats(run, "decode step")
