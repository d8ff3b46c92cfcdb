"""Benchmark of the chunkwise gated delta rule on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]

A step is one pass of the hot path over one batch of seeded synthetic input
already resident in HBM: for the default workload (gated delta rule, bf16,
B=4 T=4096 H=16 dk=128 dv=256) that is the chunkwise forward pass plus the
chunkwise backward pass (dq, dk, dv, dbeta, dg, dh0); workload 6 is the same for
the packed varlen input of workload 5.  Workloads 2, 3 and 5
are forward-only; "dec" is one decode step at batch 256, H=32, d=128.

Prints one JSON line: tokens/s and algorithmic TFLOP/s (with the fraction of
the bf16 MFMA peak) over the timed steps, every kernel's device time from HIP
events recorded on the launch stream inside the timed steps, the roofline
position of the dominant kernel (the chunk-gradient kernel of the backward
pass; the forward kernel for forward-only workloads), and the fp64 oracle's
throughput on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
# HBM bytes per launch of the chunk-gradient kernel at workload 4, from rocprofv3
# FETCH_SIZE and WRITE_SIZE scaled by what the same counters read for a copy of
# known size (commands and raw counts under profiles/); it describes the kernel as
# built when the counters were taken
CHUNK_GRAD_TRAFFIC_W4 = 1511.4e6
# the same for the forward kernel at the gated forward-only workload (B=4 T=4096
# H=16 dk=128 dv=256): 294.0 MB read + 142.6 MB written
FWD_TRAFFIC_W3 = 436.6e6
# the same for the short convolution's backward kernel (W = 4, B=4 T=4096 H=16 d=128,
# bf16): 214.3 MB read + 136.3 MB written
CONV_BWD_TRAFFIC = 350.7e6
MFMA_BF16_PEAK_TFS = 2500.0  # dense bf16 MFMA, TFLOP/s
PROBE_LIB = os.path.join(ROOT, "chunkwise_delta_rule_wy_amd", "libdnprobe.so")
_probe = None


def probe_lib():
    """libdnprobe.so (built beside libdn.so): machine probes and timing events."""
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_LIB):
            raise RuntimeError("%s is not built: run __graft_entry__.build()" % PROBE_LIB)
        lib = ctypes.CDLL(PROBE_LIB)
        vp = ctypes.c_void_p
        lib.dnp_event_create.argtypes = [ctypes.POINTER(vp)]
        lib.dnp_event_destroy.argtypes = [vp]
        lib.dnp_event_record.argtypes = [vp, vp]
        lib.dnp_event_elapsed_ms.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_float)]
        lib.dnp_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
        lib.dnp_mfma_loop_flops.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.dnp_mfma_loop_flops.restype = ctypes.c_double
        lib.dnp_clock.argtypes = [ctypes.c_ulonglong, vp, vp]
        lib.dnp_copy.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int, vp]
        _probe = lib
    return _probe


class TimingEvent:
    """A HIP event made for timing only: recording it takes a timestamp after
    the work enqueued before it on the stream, without the system-scope cache
    write-back and invalidation of a default event (torch.cuda.Event), which
    costs the kernels that follow it several microseconds per record.  The
    binding takes it wherever it takes a torch.cuda.Event (`cuda_event`)."""

    def __init__(self):
        h = ctypes.c_void_p()
        if probe_lib().dnp_event_create(ctypes.byref(h)) != 0:
            raise RuntimeError("dnp_event_create failed")
        self.cuda_event = h.value

    def record(self, stream):
        if probe_lib().dnp_event_record(ctypes.c_void_p(self.cuda_event), ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("dnp_event_record failed")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (waits for `end`)."""
        ms = ctypes.c_float()
        if probe_lib().dnp_event_elapsed_ms(ctypes.c_void_p(self.cuda_event), ctypes.c_void_p(end.cuda_event),
                                            ctypes.byref(ms)) != 0:
            raise RuntimeError("dnp_event_elapsed_ms failed")
        return ms.value

    def __del__(self):
        if _probe is not None and self.cuda_event:
            _probe.dnp_event_destroy(ctypes.c_void_p(self.cuda_event))
            self.cuda_event = None


def workload_bytes(sh, backward: bool) -> float:
    """Algorithmic HBM bytes: one read of every input, one write of every
    output, at their dtypes (no intermediate counted)."""
    es = 2 if str(sh.dtype).endswith("bfloat16") else 4
    th = sh.B * sh.T * sh.H
    st = sh.n_seqs * sh.H * sh.Dk * sh.Dv * 4
    fwd = th * (2 * sh.Dk * es + 2 * sh.Dv * es + 4 * (2 if sh.gated else 1))
    fwd += st * ((1 if sh.has_h0 else 0) + 1)
    if not backward:
        return float(fwd)
    bwd = th * (2 * sh.Dk * es + 2 * sh.Dv * es + 4 * (2 if sh.gated else 1)   # q k v dO beta g
                + 2 * sh.Dk * 4 + sh.Dv * 4 + 4 * (2 if sh.gated else 1))      # dq dk dv dbeta dg
    bwd += st * (1 + 1 + 1)                                                    # h0 dhT dh0
    return float(fwd + bwd)


def chunk_grad_bytes(sh) -> float:
    """Algorithmic HBM bytes of one launch of the chunk-gradient kernel: one
    read of each of its inputs (q, k, v, dO, beta, g) and one write of each of
    its outputs (dq, dk, dv, dbeta, dg in fp32) at their dtypes.  The bf16
    chunk states h and dh it also reads are intermediates of the backward
    pass and are not counted (they appear in the measured traffic)."""
    es = 2 if str(sh.dtype).endswith("bfloat16") else 4
    th = sh.B * sh.T * sh.H
    per_tok = (2 * sh.Dk * es + 2 * sh.Dv * es + 4 * (2 if sh.gated else 1)
               + 2 * sh.Dk * 4 + sh.Dv * 4 + 4 * (2 if sh.gated else 1))
    return float(th * per_tok)


def chunk_state_bytes(sh, chunk=64) -> float:
    """Bytes of the bf16 chunk states h and dh (d_k x d_v per (chunk, head)
    each) that the chunk-gradient kernel reads besides its inputs."""
    lengths = sh.lengths if sh.lengths is not None else [sh.T] * sh.B
    chunk_heads = sum((L + chunk - 1) // chunk for L in lengths) * sh.H
    return float(chunk_heads * 2 * sh.Dk * sh.Dv * 2)


def decode_bytes(B=256, H=32, Dk=128, Dv=128) -> float:
    """Algorithmic bytes of one decode step: the fp32 state read and written,
    q, k, v read and o written in bf16, beta and g read in fp32."""
    return float(B * H * Dk * Dv * 4 * 2 + B * H * (2 * Dk + 2 * Dv) * 2 + B * H * 8)


def decode_flops(B=256, H=32, Dk=128, Dv=128) -> float:
    """Algorithmic flops of one decode step: per state, the two matrix-vector
    products h^T k and h^T q and the rank-one update, 2 d_k d_v MACs each."""
    return 2.0 * 3 * Dk * Dv * B * H


def bwd_flops(sh) -> float:
    """Algorithmic flops of the backward pass without the recompute, per
    token-head (MACs): 6 dk dv for the state products, (C+1)/2 (5 dk + 4 dv)
    for the causal intra-chunk products, (C-1)/2 2 dk for the strict ones and
    2 C^2/3 for the two triangular substitutions."""
    C, dk, dv = 64, sh.Dk, sh.Dv
    mac = 6 * dk * dv + (C + 1) / 2 * (5 * dk + 4 * dv) + (C - 1) / 2 * 2 * dk + 2 * C * C / 3
    return 2.0 * mac * sh.B * sh.T * sh.H


def fwd_flops(sh) -> float:
    """Algorithmic flops of the chunkwise forward pass per token-head (MACs,
    triangular products at their exact half): K K^T strict (C-1)/2 d_k; the
    causal products Q K^T and T diag(gamma) K, (C+1)/2 d_k each, and T V and
    P V', (C+1)/2 d_v each; the state products K h, Q h and K^T V', d_k d_v
    each; the inverse of (I + A), C^2/6.  This is the method's count, with the
    WY factors W = T diag(gamma) K and U = T V formed; the library applies T to
    V - diag(gamma) K h instead and does fewer flops than it is credited with
    (the d_k term of the T product)."""
    C, dk, dv = 64, sh.Dk, sh.Dv
    mac = (C - 1) / 2 * dk + (C + 1) / 2 * (2 * dk + 2 * dv) + 3 * dk * dv + C * C / 6
    return 2.0 * mac * sh.B * sh.T * sh.H


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the clocks take some 40 steps of steady work to settle after a start
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default="4",
                    help="2, 3, 4, 5, 6 (numbered workloads), dec (decode step), conv (short "
                         "convolution) or chunksize (forward and training pair against the chunk size)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--chunk", type=int, choices=(32, 64), default=64,
                    help="chunk length (the folded prologue and Longhorn backward passes take 64)")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="after the timed steps, this many more steps each preceded by a 1 GiB "
                         "write that evicts the L2s and the 256 MB Infinity Cache; their per-kernel "
                         "event times are reported as kernel_us_cold (median, min)")
    ap.add_argument("--no-forward-configs", action="store_true",
                    help="skip the forward-only workloads and the decode step that the default "
                         "(training) run times after its own steps")
    ap.add_argument("--no-measured-peaks", action="store_true",
                    help="skip the probes of the machine's own peaks (HBM copy bandwidth, a bf16 "
                         "MFMA loop, the shader clock) reported beside the vendor figures")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy a 512 MiB fp32 tensor once (torch copy_): "
                         "the kernel of known size that calibrates rocprofv3 byte counters")
    ap.add_argument("--prologue", action="store_true",
                    help="start from the raw draws: the input prologue (L2-normalised q, k; "
                         "sigmoid beta; -0.1 softplus gate) runs before the passes and its backward "
                         "after them (folded into the chunk-gradient kernel with --bwd-mode saved)")
    ap.add_argument("--bwd-mode", choices=("saved", "recompute"), default="saved",
                    help="saved: the forward pass stores the bf16 chunk states and the backward "
                         "pass reads them (dn_chunk_fwd_save + dn_chunk_bwd_saved); recompute: "
                         "the backward pass recomputes them (dn_chunk_bwd)")
    ap.add_argument("--variant", choices=("delta", "longhorn"), default="delta",
                    help="longhorn: the step size eps = beta / (1 + beta |k|^2) of Table 1's "
                         "Longhorn row, computed (and differentiated) around the same passes")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(every (sequence, head) pair is independent, so several GPUs would each take a "
              "share of the pairs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import chunkwise_delta_rule_wy_amd as dn
    from chunkwise_delta_rule_wy_amd import synth

    dev = torch.device("cuda:0")
    wid = args.workload
    if wid == "dec":
        return bench_decode(args, dn, synth, dev)
    if wid == "conv":
        return bench_conv(args, dn, synth, dev)
    if wid == "chunksize":
        return bench_chunk_sizes(args, dn, synth, dev)
    wid = int(wid)
    sh = synth.WORKLOADS[wid]
    backward = sh.backward
    x = synth.workload_inputs(wid, raw=args.prologue)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    torch.cuda.synchronize()

    ws = None
    if backward:
        ws = torch.empty(dn.bwd_workspace_bytes(sh.B, sh.T, sh.H, sh.Dk, sh.Dv, sh.n_seqs,
                                                sh.dtype, chunk=args.chunk), dtype=torch.uint8, device=dev)

    # every timed step records HIP events on the stream the kernels run on
    # (torch's current stream, which the binding hands to the library)
    stream = torch.cuda.current_stream(dev)
    mk = TimingEvent
    nev = max(args.steps, 1) + max(args.cold_steps, 0)
    longhorn = args.variant == "longhorn"
    saved = backward and args.bwd_mode == "saved"
    fev = [(mk(), mk()) for _ in range(nev)]
    # the saved-state backward starts where the forward ends (nothing runs in
    # between): its first two events are not recorded and the forward's end
    # event starts the scan, four records per step instead of six
    bev = ([[None, None, mk(), mk()] if saved else [mk() for _ in range(4)] for _ in range(nev)]
           if backward else None)
    if backward and args.chunk != 64 and (args.prologue or longhorn):
        print("the folded prologue and Longhorn backward passes run 64-token chunks only", file=sys.stderr)
        sys.exit(2)
    lev = [(mk(), mk()) for _ in range(nev)]

    pev = [(mk(), mk()) for _ in range(nev)]
    pbev = [(mk(), mk()) for _ in range(nev)]

    def step(i=None):
        if args.prologue:
            if i is not None:
                pev[i][0].record(stream)
            q, k, b0, g = dn.prologue(d["q_in"], d["k_in"], d["b_in"], d["x_in"], d["gate_scale"])
            if i is not None:
                pev[i][1].record(stream)
        else:
            q, k, b0, g = d["q"], d["k"], d["beta"], d["g"]
        if i is not None:
            fev[i][0].record(stream)
        beta = dn.longhorn_eps(k, b0) if longhorn else b0
        o, hT = dn.chunk_fwd(q, k, d["v"], beta, g, d["h0"], d["cu_seqlens"], chunk=args.chunk,
                             save_workspace=ws if saved else None)
        if i is not None:
            fev[i][1].record(stream)
        if backward:
            # the recomputing backward pass keeps nothing from the forward pass and
            # recomputes eps; the saved-state pair keeps eps beside the states and
            # folds the step size's backward into the chunk-gradient kernel
            if not saved:
                beta = dn.longhorn_eps(k, b0) if longhorn else b0
            fused = saved and args.prologue and not longhorn
            pro = (d["q_in"], d["k_in"], d["x_in"], d["gate_scale"]) if fused else None
            gr = dn.chunk_bwd(q, k, d["v"], beta, g, d["h0"], d["dO"], d["dhT"],
                              d["cu_seqlens"], chunk=args.chunk, workspace=ws,
                              events=bev[i] if i is not None else None,
                              saved=saved, prologue_inputs=pro,
                              longhorn_beta=b0 if (longhorn and saved) else None)
            if longhorn and not saved:
                if i is not None:
                    lev[i][0].record(stream)
                gr["dbeta"] = dn.longhorn_eps_bwd(k, b0, gr["dbeta"], gr["dk"])
                if i is not None:
                    lev[i][1].record(stream)
            if args.prologue and not fused:
                if i is not None:
                    pbev[i][0].record(stream)
                dn.prologue_bwd(d["q_in"], d["k_in"], d["b_in"], d["x_in"], d["gate_scale"],
                                gr["dq"], gr["dk"], gr["dbeta"], gr["dg"])
                if i is not None:
                    pbev[i][1].record(stream)
        return o

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / max(args.steps, 1)
    tokens = sh.B * sh.T
    value = tokens / (ms_per_step * 1e-3)

    # cold steps: a 1 GiB write before each evicts what the previous step left in
    # the caches; they are timed by their events only, outside the timed region
    cold = range(args.steps, args.steps + max(args.cold_steps, 0))
    if len(cold):
        scratch = torch.empty(256 * 1024 * 1024, dtype=torch.float32, device=dev)
        for i in cold:
            scratch.fill_(float(i))
            step(i)
        torch.cuda.synchronize()
        del scratch

    def stage_times(idx):
        """Per-kernel device times (us) of the steps in idx, from their events."""
        us = lambda pairs: [a.elapsed_time(b) * 1e3 for a, b in pairs]
        t = {"fwd": us([fev[i] for i in idx])}
        if backward:
            for j, name in enumerate(("recompute", "state_grad_scan", "chunk_grad")):
                if j == 0 and saved:
                    continue  # the forward pass stored the states
                start = (lambda i: fev[i][1]) if (j == 1 and saved) else (lambda i: bev[i][j])
                t[name] = us([(start(i), bev[i][j + 1]) for i in idx])
            if longhorn and not saved:
                t["longhorn_eps_bwd"] = us([lev[i] for i in idx])
            if args.prologue and not (saved and not longhorn):
                t["prologue_bwd"] = us([pbev[i] for i in idx])
        if args.prologue:
            t["prologue"] = us([pev[i] for i in idx])
        return t

    # per-kernel device time, averaged over the timed steps
    warm_t = stage_times(range(args.steps))
    stage_us = {k: sum(v) / len(v) for k, v in warm_t.items()}
    med = lambda v: sorted(v)[len(v) // 2]
    cold_t = stage_times(cold) if len(cold) else {}
    flops = fwd_flops(sh) + (bwd_flops(sh) if backward else 0.0)
    if backward:
        kname, kus, kbytes = "dn::bwd_chunk_kernel", stage_us["chunk_grad"], chunk_grad_bytes(sh)
    else:
        kname = "dn::fwd_bf16_kernel" if args.chunk == 64 else "dn::fwd32_kernel"
        kus, kbytes = stage_us["fwd"], workload_bytes(sh, False)
    achieved = kbytes / (kus * 1e-6) / 1e9
    traffic = (CHUNK_GRAD_TRAFFIC_W4 if (backward and wid == 4 and args.chunk == 64) else
               FWD_TRAFFIC_W3 if (wid == 3 and args.chunk == 64 and not args.prologue and not longhorn)
               else None)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": kname, "kernel_us": round(kus, 2), "bytes_per_launch": kbytes,
                "timing": "warm: mean of the kernel's live event times over the timed steps, "
                          "which run back to back on resident inputs"}
    if traffic is not None:
        roofline["traffic_over_algorithmic"] = round(traffic / kbytes, 3)
    if backward:
        roofline["chunk_state_bytes"] = chunk_state_bytes(sh, args.chunk)
    step_tflops = flops / (ms_per_step * 1e-3) / 1e12

    out = {
        "metric": "tokens/s & TFLOP/s (fraction of MFMA peak), gated delta-rule fwd+bwd",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if sh.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded, L2-normalised q/k, sigmoid beta, -softplus*0.1 gate)",
        "config": {"workload": synth.WORKLOAD_NAMES[wid], "B": sh.B, "T": sh.T, "H": sh.H,
                   "Dk": sh.Dk, "Dv": sh.Dv, "chunk": args.chunk, "passes": "fwd+bwd" if backward else "fwd",
                   "n_seqs": sh.n_seqs, "variant": args.variant, "prologue": args.prologue,
                   "bwd_mode": args.bwd_mode if backward else None},
        "roofline": roofline,
        "tflops": round(step_tflops, 2),
        "mfma_frac": round(step_tflops / MFMA_BF16_PEAK_TFS, 4),
        "step_gbs": round(workload_bytes(sh, backward) / (ms_per_step * 1e-3) / 1e9, 1),
        "kernel_us": {k: round(v, 2) for k, v in stage_us.items()},
        "kernel_us_median_min": {k: [round(med(v), 2), round(min(v), 2)] for k, v in warm_t.items()},
    }
    if cold_t:
        out["kernel_us_cold"] = {k: {"median": round(med(v), 2), "min": round(min(v), 2)}
                                 for k, v in cold_t.items()}
        ck = "chunk_grad" if backward else "fwd"
        cmed = med(cold_t[ck])
        roofline["frac_cold"] = round(kbytes / (cmed * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        roofline["kernel_us_cold_median"] = round(cmed, 2)
    mp = None
    if not args.no_measured_peaks:
        mp = measured_peaks(torch, dev, stream)
        if mp is not None:
            out["measured_peaks"] = mp
            roofline["frac_of_measured"] = round(achieved / mp["hbm_copy_GBs"], 4)
            out["mfma_frac_of_measured"] = round(step_tflops / mp["mfma_bf16_TFs"], 4)
    if args.copy_calibration:
        a = torch.empty(128 * 1024 * 1024, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        e0, e1 = mk(), mk()
        e0.record(stream)
        b.copy_(a)
        e1.record(stream)
        out["copy_512MiB_us"] = round(e0.elapsed_time(e1) * 1e3, 1)
        del a, b
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, sh, backward, args.cpu_seconds, args.variant)
    if not args.no_forward_configs and wid == 4 and not args.prologue and args.variant == "delta":
        del d, ws, x
        torch.cuda.empty_cache()
        out["forward_configs"] = forward_configs(dn, synth, dev, stream, mp)
    print(json.dumps(out), flush=True)


# Algorithmic HBM floors of the forward workloads at 8 TB/s (one read of every
# input and one write of every output): the denominators of their roofline
# fractions
FWD_WORKLOADS = (2, 3, 5)


WARM_MS = 60.0


def _settle(fn, stream, warm_ms=WARM_MS):
    """Untimed calls for about `warm_ms` of device time (at least 20): the
    shader clock takes tens of milliseconds of steady work to settle after the
    GPU has idled, e.g. while the host built the next workload's inputs."""
    import torch
    e0, e1 = TimingEvent(), TimingEvent()
    e0.record(stream)
    for _ in range(5):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    per_call_ms = max(e0.elapsed_time(e1) / 5, 1e-3)
    for _ in range(min(5000, max(20, int(warm_ms / per_call_ms) + 1))):
        fn()


def _cold_times(fn, stream, reps=20, evict="write"):
    """The cold protocol: untimed calls until the clocks settle, then `reps`
    calls, each after a 1 GiB pass over a buffer of its own that evicts the
    L2s and the 256 MB Infinity Cache (reads and writes both allocate there),
    timed by events on the launch stream.  Returns the list of times (us).
    evict="write" fills the buffer: the caches then hold the fill's dirty
    lines, whose write-back the timed call pays for.  evict="read" sums it:
    the lines left are clean, and the timed call pays for its own traffic
    only (writes it leaves in the Infinity Cache reach HBM after it)."""
    import torch
    dev = torch.device("cuda:0")
    scratch = torch.empty(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    if evict == "read":
        scratch.fill_(1.0)
    _settle(fn, stream)
    times = []
    for i in range(reps):
        if evict == "read":
            torch.sum(scratch, 0, out=sink)
        else:
            scratch.fill_(float(i))
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record(stream)
        fn()
        e1.record(stream)
        times.append((e0, e1))
    torch.cuda.synchronize()
    del scratch
    return [a.elapsed_time(b) * 1e3 for a, b in times]


def _warm_times(fn, stream, reps=20):
    """Back-to-back calls on resident inputs (a loop's steady state): untimed
    calls until the clocks settle, then `reps` calls timed by events.  Returns
    times (us)."""
    import torch
    _settle(fn, stream)
    ev = [(TimingEvent(), TimingEvent()) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def forward_configs(dn, synth, dev, stream, peaks=None):
    """The forward-only workloads (2, 3 and 5) and the decode step, each timed
    warm (back to back on resident inputs) and cold (a 1 GiB eviction before
    every call; 20 timed calls, median and minimum), with the fraction of the
    HBM roofline at its algorithmic bytes, its algorithmic TFLOP/s and GB/s
    (warm), and, given the machine's measured peaks, the warm fractions of the
    measured copy bandwidth and bf16 MFMA rate."""
    import torch
    res = {}
    med = lambda v: sorted(v)[len(v) // 2]

    def entry(name, nbytes, tokens, warm, cold, cold_rd, flops):
        floor = nbytes / (HBM_PEAK_GBS * 1e9) * 1e6
        wmean = sum(warm) / len(warm)
        extra = {"tflops_warm": round(flops / (wmean * 1e-6) / 1e12, 2),
                 "gbs_warm": round(nbytes / (wmean * 1e-6) / 1e9, 1)}
        if peaks is not None:
            extra["frac_warm_of_measured_copy"] = round(extra["gbs_warm"] / peaks["hbm_copy_GBs"], 4)
            extra["mfma_frac_warm_of_measured"] = round(extra["tflops_warm"] / peaks["mfma_bf16_TFs"], 4)
        res[name] = {
            "bytes": nbytes, "floor_us": round(floor, 2),
            "warm_us": {"mean": round(sum(warm) / len(warm), 2), "median": round(med(warm), 2),
                        "min": round(min(warm), 2)},
            "cold_us": {"median": round(med(cold), 2), "min": round(min(cold), 2)},
            "cold_read_evict_us": {"median": round(med(cold_rd), 2), "min": round(min(cold_rd), 2)},
            "frac_warm": round(floor / (sum(warm) / len(warm)), 4),
            "frac_cold": round(floor / med(cold), 4),
            "frac_cold_read_evict": round(floor / med(cold_rd), 4),
            "tokens_per_s_cold": round(tokens / (med(cold) * 1e-6), 1),
            **extra,
        }

    for wid in FWD_WORKLOADS:
        sh = synth.WORKLOADS[wid]
        x = synth.workload_inputs(wid)
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
        del x
        fn = lambda: dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu_seqlens"])
        warm = _warm_times(fn, stream)
        cold = _cold_times(fn, stream)
        cold_rd = _cold_times(fn, stream, evict="read")
        entry(synth.WORKLOAD_NAMES[wid], workload_bytes(sh, False), sh.B * sh.T, warm, cold, cold_rd, fwd_flops(sh))
        del d
        torch.cuda.empty_cache()
    x = synth.decode_inputs()
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    fn = lambda: dn.recurrent_step(d["q"], d["k"], d["v"], d["beta"], d["g"], d["state"])
    warm = _warm_times(fn, stream)
    cold = _cold_times(fn, stream)
    cold_rd = _cold_times(fn, stream, evict="read")
    entry("decode-B256-H32-d128", decode_bytes(), 256, warm, cold, cold_rd, decode_flops())
    res["how"] = ("warm: untimed calls for %.0f ms of device time (at least 20), then 20 timed "
                  "back-to-back calls on resident inputs; cold: the same untimed calls, then 20 "
                  "timed calls each after a 1 GiB write (median, min); cold_read_evict: the same "
                  "with a 1 GiB read (a sum) in place of the write, which leaves no dirty lines "
                  "for the timed call to write back; " % WARM_MS +
                  "frac = the HBM floor at 8 TB/s of the algorithmic bytes over the time; tflops_warm and gbs_warm = the algorithmic flops and bytes over the warm mean, of_measured against the machine's measured copy and MFMA rates; "
                  "tokens_per_s_cold counts the decode batch as tokens")
    return res


def measured_peaks(torch, dev, stream):
    """The machine's own peaks, measured after the timed steps: HBM bandwidth of
    a 1 GiB device copy (bytes read + written over time), the bf16 rate of a
    plain MFMA loop (16x16x32 MFMAs on registers, four waves per SIMD) and the
    shader clock (a wave spinning on the clock counter, against HIP events)."""
    lib = probe_lib()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(fn, reps):
        fn()
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        return e0.elapsed_time(e1) * 1e-3 / reps

    a = torch.empty(256 * 1024 * 1024, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    t_torch = timed(lambda: b.copy_(a), 5)

    def copy():
        if lib.dnp_copy(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), a.numel() * 4,
                        256 * 16, sp) != 0:
            raise RuntimeError("dnp_copy failed")
    t_copy = timed(copy, 5)
    copy_gbs = 2 * a.numel() * 4 / min(t_copy, t_torch) / 1e9
    del a, b
    grid, iters = 256 * 4, 2000
    sink = torch.empty(grid * 256, dtype=torch.float32, device=dev)

    def mfma():
        if lib.dnp_mfma_loop(grid, iters, ctypes.c_void_p(sink.data_ptr()), sp) != 0:
            raise RuntimeError("dnp_mfma_loop failed")
    t_mfma = timed(mfma, 3)
    mfma_tfs = lib.dnp_mfma_loop_flops(grid, iters) / t_mfma / 1e12
    cyc = torch.zeros(1, dtype=torch.int64, device=dev)
    want = 20_000_000

    def clock():
        if lib.dnp_clock(want, ctypes.c_void_p(cyc.data_ptr()), sp) != 0:
            raise RuntimeError("dnp_clock failed")
    t_clock = timed(clock, 1)
    sclk_mhz = int(cyc.item()) / t_clock / 1e6
    return {"hbm_copy_GBs": round(copy_gbs, 1), "mfma_bf16_TFs": round(mfma_tfs, 1),
            "sclk_MHz": round(sclk_mhz, 1), "mclk_MHz": memory_clock_mhz(),
            "how": "1 GiB device copy, the faster of a streaming copy kernel and torch copy_ "
                   "(read + write bytes); 16x16x32 bf16 MFMA loop on "
                   "registers, 1024 workgroups x 4 waves; one wave spinning %d shader-clock "
                   "cycles against HIP events" % want}


def memory_clock_mhz():
    """The HBM clock that rocm-smi reports for the first GPU (None if it cannot
    be read); HBM3E at 2000 MHz is the part's 8 TB/s."""
    import re
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        m = re.search(r'"mclk clock speed:":\s*"\((\d+)\s*Mhz\)"', r.stdout)
        return int(m.group(1)) if m else None
    except (OSError, subprocess.SubprocessError):
        return None


def cpu_baseline(x, sh, backward, budget_s, variant="delta"):
    """The fp64 oracle on a bounded sample: whole sequences of a few heads."""
    import oracle
    ofwd = oracle.longhorn_fwd if variant == "longhorn" else oracle.fwd
    obwd = oracle.longhorn_bwd if variant == "longhorn" else oracle.bwd
    cores = len(os.sched_getaffinity(0))
    nthr = int(os.environ.get("OMP_NUM_THREADS", cores) or cores)
    nthr = max(1, min(nthr, cores))
    # sample: the first `npairs` (batch, head) pairs over the full sequence
    # length; grow until the budget is roughly used
    npairs, elapsed, T = nthr, 0.0, sh.T
    while True:
        b_idx = [i // sh.H for i in range(npairs)]
        h_idx = [i % sh.H for i in range(npairs)]
        import torch
        sel = lambda t: torch.stack([t[b, :, h] for b, h in zip(b_idx, h_idx)], 0).unsqueeze(2)
        xs = dict(q=sel(x["q"]), k=sel(x["k"]), v=sel(x["v"]), beta=sel(x["beta"]),
                  g=None if x["g"] is None else sel(x["g"]))
        h0 = None if x["h0"] is None else torch.stack([x["h0"][b, h] for b, h in zip(b_idx, h_idx)]).unsqueeze(1)
        if sh.lengths is not None:
            # packed input: sample whole heads of the first sequence
            L = sh.lengths[0]
            xs = {k: (v[:, :L] if v is not None else None) for k, v in xs.items()}
            h0 = h0[:, :1] if h0 is not None else None
            T = L
        t0 = time.perf_counter()
        ofwd(xs["q"], xs["k"], xs["v"], xs["beta"], xs["g"], h0, nthreads=nthr)
        if backward:
            dO = sel(x["dO"])
            if sh.lengths is not None:
                dO = dO[:, :T]
            dhT = torch.stack([x["dhT"][b, h] for b, h in zip(b_idx, h_idx)]).unsqueeze(1)
            obwd(xs["q"], xs["k"], xs["v"], xs["beta"], xs["g"], h0, dO, dhT, nthreads=nthr)
        elapsed = time.perf_counter() - t0
        if elapsed * 4 > budget_s or npairs >= sh.B * sh.H:
            break
        npairs = min(npairs * 4, sh.B * sh.H)
    token_heads = npairs * T
    # the same oracle on one thread, over one pair of the sample
    one = {k: (v[:1] if v is not None else None) for k, v in xs.items()}
    h01 = h0[:1] if h0 is not None else None
    t0 = time.perf_counter()
    ofwd(one["q"], one["k"], one["v"], one["beta"], one["g"], h01, nthreads=1)
    if backward:
        obwd(one["q"], one["k"], one["v"], one["beta"], one["g"], h01, dO[:1], dhT[:1], nthreads=1)
    t1 = time.perf_counter() - t0
    return {"value": round(token_heads / sh.H / elapsed, 1), "unit": "tokens/s",
            "cores": nthr, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d (batch, head) pairs x %d tokens (%s), %.1f s on %d threads; tokens/s counts "
                      "a token as all %d heads" % (npairs, T, "fwd+bwd" if backward else "fwd", elapsed,
                                                   nthr, sh.H),
            "one_thread": {"value": round(T / sh.H / t1, 1), "unit": "tokens/s", "seconds": round(t1, 2),
                           "sample": "1 (batch, head) pair x %d tokens on 1 thread" % T}}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def bench_chunk_sizes(args, dn, synth, dev):
    """The chunk-size comparison of the DeltaNet rebuttal (answer Q1: forward
    and backward time against the chunk size, at sequence length 4096, batch
    2, head dimension 128, 16 heads), on the ungated delta rule in bf16: the
    forward pass and the training pair (the forward pass storing the chunk
    states, then the backward pass reading them) with 32- and 64-token
    chunks, each timed warm and cold."""
    import torch
    sh = synth.Shape(2, 4096, 16, 128, 128, torch.bfloat16, gated=False, has_h0=False, backward=True)
    x = synth.make_inputs(sh, seed=1301)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    stream = torch.cuda.current_stream(dev)
    med = lambda v: sorted(v)[len(v) // 2]
    res = {}
    for C in (32, 64):
        fn = lambda: dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], None, None, chunk=C)
        warm, cold = _warm_times(fn, stream), _cold_times(fn, stream)
        res["fwd_C%d" % C] = {"warm_us": round(sum(warm) / len(warm), 2), "cold_median_us": round(med(cold), 2),
                              "cold_min_us": round(min(cold), 2)}
    for C in (32, 64):
        ws = torch.empty(dn.bwd_workspace_bytes(sh.B, sh.T, sh.H, sh.Dk, sh.Dv, chunk=C), dtype=torch.uint8,
                         device=dev)

        def train():
            dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], None, None, chunk=C, save_workspace=ws)
            dn.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], None, None, d["dO"], d["dhT"], chunk=C, workspace=ws,
                         saved=True)
        warm, cold = _warm_times(train, stream), _cold_times(train, stream)
        res["fwd+bwd_C%d" % C] = {"warm_us": round(sum(warm) / len(warm), 2),
                                  "cold_median_us": round(med(cold), 2), "cold_min_us": round(min(cold), 2)}
        del ws
    th = sh.B * sh.T * sh.H
    res["chunk_state_bytes_C64"] = 2 * (th // 64) * sh.Dk * sh.Dv * 2
    res["chunk_state_bytes_C32"] = 2 * (th // 32) * sh.Dk * sh.Dv * 2
    print(json.dumps({"metric": "chunk-size comparison (DeltaNet rebuttal, answer Q1 setting)",
                      "config": {"workload": "deltanet-B2-T4096-H16-d128-ungated", "dtype": "bf16"},
                      "results": res, "how": "warm: mean of 20 back-to-back calls after untimed calls for "
                      "%.0f ms of device time; cold: 20 calls each after a 1 GiB write (median, min); "
                      "chunk_state_bytes: the bf16 states h and dh the training pair stores and reads per "
                      "chunk size" % WARM_MS}), flush=True)


def bench_decode(args, dn, synth, dev):
    import torch
    x = synth.decode_inputs()
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    st = d["state"]
    for _ in range(args.warmup):
        dn.recurrent_step(d["q"], d["k"], d["v"], d["beta"], d["g"], st)
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        dn.recurrent_step(d["q"], d["k"], d["v"], d["beta"], d["g"], st)
    ev1.record(stream)
    us = ev0.elapsed_time(ev1) * 1e3 / args.steps
    B, H, Dk, Dv = 256, 32, 128, 128
    nbytes = B * H * Dk * Dv * 4 * 2 + B * H * (2 * Dk + 2 * Dv) * 2 + B * H * 8
    gbs = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({"metric": "decode step", "value": round(B / (us * 1e-6), 1),
                      "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": round(us / 1e3, 5), "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                      "data": "synthetic", "config": {"workload": "decode-B256-H32-d128"},
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                   "traffic": None}}), flush=True)


def bench_conv(args, dn, synth, dev):
    """The short convolution (W = 4) over the q projection of the training
    shape (B=4 T=4096 H=16 d=128, bf16): forward and backward per step (the
    timed steps); then the same with the L2 normalisation fused in, timed by
    its events only."""
    import torch
    B, T, H, D, W = 4, 4096, 16, 128, 4
    x = synth.conv_inputs(B, T, H, D, W, torch.bfloat16, seed=1250)
    xd, wd, dyd = x["x"].to(dev), x["w"].to(dev), x["dy"].to(dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        dn.short_conv(xd, wd)
        dn.short_conv_bwd(xd, wd, dyd)
    torch.cuda.synchronize()
    ev = [[TimingEvent() for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(stream)
        dn.short_conv(xd, wd)
        e[1].record(stream)
        dn.short_conv_bwd(xd, wd, dyd)
        e[2].record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    fus = sum(e[0].elapsed_time(e[1]) for e in ev) * 1e3 / args.steps
    bus = sum(e[1].elapsed_time(e[2]) for e in ev) * 1e3 / args.steps
    # the same with the per-head L2 normalisation fused in (how q and k are prepared)
    for _ in range(args.warmup):
        dn.short_conv(xd, wd, l2norm=True)
        dn.short_conv_bwd(xd, wd, dyd, l2norm=True)
    ev2 = [[TimingEvent() for _ in range(3)] for _ in range(args.steps)]
    for e in ev2:
        e[0].record(stream)
        dn.short_conv(xd, wd, l2norm=True)
        e[1].record(stream)
        dn.short_conv_bwd(xd, wd, dyd, l2norm=True)
        e[2].record(stream)
    torch.cuda.synchronize()
    lfus = sum(e[0].elapsed_time(e[1]) for e in ev2) * 1e3 / args.steps
    lbus = sum(e[1].elapsed_time(e[2]) for e in ev2) * 1e3 / args.steps
    if args.copy_calibration:  # the kernel of known size for the byte counters
        a = torch.empty(128 * 1024 * 1024, dtype=torch.float32, device=dev).fill_(1.0)
        torch.empty_like(a).copy_(a)
        torch.cuda.synchronize()
        del a
    n = B * T * H * D
    fbytes = n * (2 + 2) + H * D * W * 4            # x read, y written (bf16), taps
    bbytes = n * (2 + 4 + 4) + 2 * H * D * W * 4    # x, dy read, dx written, taps, dw
    fg, bg = fbytes / (fus * 1e-6) / 1e9, bbytes / (bus * 1e-6) / 1e9
    print(json.dumps({"metric": "short convolution fwd+bwd", "value": round(B * T / (ms * 1e-3), 1),
                      "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
                      "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "short-conv-W4-B4-T4096-H16-d128"},
                      "kernel_us": {"conv_fwd": round(fus, 2), "conv_bwd": round(bus, 2),
                                    "conv_l2_fwd": round(lfus, 2), "conv_l2_bwd": round(lbus, 2)},
                      "roofline": {"bound": "hbm", "achieved": round(bg, 1), "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": round(bg / HBM_PEAK_GBS, 4),
                                   "traffic": CONV_BWD_TRAFFIC, "kernel": "dn::conv_bwd_kernel",
                                   "bytes_per_launch": bbytes},
                      "fwd_roofline": {"achieved": round(fg, 1), "frac": round(fg / HBM_PEAK_GBS, 4),
                                       "bytes_per_launch": fbytes}}), flush=True)


if __name__ == "__main__":
    main()
