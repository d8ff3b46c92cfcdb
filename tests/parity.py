"""Parity helpers of the GPU tests (no test collected here).

Errors are relative L2 norms in fp64 (the tolerance metric of every parity
test): over a whole tensor, over every (sequence, head) pair, and over every
64-token chunk of every pair, so that a wrong tile or a wrong pair cannot hide
inside a whole-tensor norm.  ``oracle_run`` computes the fp64 oracle of a
numbered workload once per test session.
"""
from __future__ import annotations

import numpy as np
import torch

from chunkwise_delta_rule_wy_amd import synth

# A chunk holds 64 tokens x d values of one head, so its norm sums far fewer
# rounding errors than a whole tensor's and fluctuates more; its bound is the
# tensor bound times 2.5.  A chunk whose reference norm is below 1e-6 of its
# tensor's RMS chunk norm (a gradient that is zero there) is measured
# absolutely against that RMS instead.  Pairs and chunks of fewer than 64
# values (a short tail of a per-token scalar such as dbeta or dg) are left to
# the whole-tensor bound: the relative error of a handful of values is that of
# single elements, whose rounding is amplified wherever the value is a
# difference of larger terms.
CHUNK_FACTOR = 2.5
MIN_VALUES = 64


def _segments(shape_B, T, cu):
    """(batch row, first token, end token) of every sequence."""
    if cu is None:
        return [(b, 0, T) for b in range(shape_B)]
    c = [int(x) for x in (cu.tolist() if isinstance(cu, torch.Tensor) else cu)]
    return [(0, c[n], c[n + 1]) for n in range(len(c) - 1)]


def _as64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def token_errors(mine, ref, cu=None, chunk=64):
    """Errors of a token tensor ([B, T, H, D] or [B, T, H]) against the oracle.

    Returns dict(total, pair [N, H], chunk_max, chunk_at (n, h, c)) where pair
    is the relative L2 of each (sequence, head) pair (0 for a pair of fewer
    than MIN_VALUES values) and chunk_max the largest relative L2 of any
    64-token chunk of any pair (of at least MIN_VALUES values)."""
    B, T, H = mine.shape[:3]
    segs = _segments(B, T, cu)
    num = np.zeros((len(segs), H))
    den = np.zeros((len(segs), H))
    per_token = int(np.prod(tuple(mine.shape[3:])))
    small = np.zeros((len(segs), H), dtype=bool)
    cnum, cden, cidx, csmall = [], [], [], []
    for n, (b, s, e) in enumerate(segs):
        if e == s:
            small[n] = True
            continue
        x = _as64(mine[b, s:e])
        y = _as64(ref[b, s:e])
        d2 = (x - y) ** 2
        y2 = y ** 2
        if d2.ndim == 3:
            d2, y2 = d2.sum(-1), y2.sum(-1)
        L = e - s
        nc = (L + chunk - 1) // chunk
        pad = nc * chunk - L
        d2 = np.pad(d2, ((0, pad), (0, 0))).reshape(nc, chunk, H).sum(1)
        y2 = np.pad(y2, ((0, pad), (0, 0))).reshape(nc, chunk, H).sum(1)
        num[n] = d2.sum(0)
        den[n] = y2.sum(0)
        small[n] = L * per_token < MIN_VALUES
        cnum.append(d2)
        cden.append(y2)
        cidx.append(n)
        tokens = np.minimum(chunk, L - chunk * np.arange(nc))
        csmall.append(np.repeat((tokens * per_token < MIN_VALUES)[:, None], H, 1))
    total = float(np.sqrt(num.sum() / den.sum())) if den.sum() > 0 else float(np.sqrt(num.sum()))
    with np.errstate(divide="ignore", invalid="ignore"):
        pair = np.where(den > 0, np.sqrt(num / np.where(den > 0, den, 1.0)), np.sqrt(num))
    pair = np.where(small, 0.0, pair)  # left to the whole-tensor bound
    chunk_max, chunk_at = 0.0, None
    if cnum:
        mean = float(np.mean(np.concatenate([c.ravel() for c in cden])))
        floor = 1e-12 * mean
        for n, d2, y2, sm in zip(cidx, cnum, cden, csmall):
            r = np.sqrt(d2 / np.where(y2 > floor, y2, max(mean, 1e-300)))
            r = np.where(sm, 0.0, r)
            i = np.unravel_index(int(np.argmax(r)), r.shape)
            if r[i] > chunk_max:
                chunk_max, chunk_at = float(r[i]), (n, int(i[1]), int(i[0]))
    return dict(total=total, pair=pair, chunk_max=chunk_max, chunk_at=chunk_at)


def state_errors(mine, ref):
    """Errors of a state tensor [N, H, Dk, Dv]: total and per pair [N, H]."""
    x, y = _as64(mine), _as64(ref)
    num = ((x - y) ** 2).sum((2, 3))
    den = (y ** 2).sum((2, 3))
    total = float(np.sqrt(num.sum() / den.sum())) if den.sum() > 0 else float(np.sqrt(num.sum()))
    with np.errstate(divide="ignore", invalid="ignore"):
        pair = np.where(den > 0, np.sqrt(num / np.where(den > 0, den, 1.0)), np.sqrt(num))
    return dict(total=total, pair=pair, chunk_max=None, chunk_at=None)


def check(name, errs, tol, label=""):
    """Assert the whole-tensor, every-pair and every-chunk bounds; print the
    worst pair and chunk."""
    pair = errs["pair"]
    worst = np.unravel_index(int(np.argmax(pair)), pair.shape)
    msg = "%s %s rel-L2 total %.2e worst pair %s %.2e" % (label, name, errs["total"], tuple(int(i) for i in worst),
                                                          float(pair[worst]))
    if errs["chunk_max"] is not None:
        msg += " worst chunk %s %.2e" % (errs["chunk_at"], errs["chunk_max"])
    print(msg, flush=True)
    assert errs["total"] <= tol, (name, "total", errs["total"])
    assert float(pair[worst]) <= tol, (name, "pair", worst, float(pair[worst]))
    if errs["chunk_max"] is not None:
        assert errs["chunk_max"] <= CHUNK_FACTOR * tol, (name, "chunk", errs["chunk_at"], errs["chunk_max"])


def check_fwd_outputs(o, hT, oo, ho, cu, tol, label=""):
    check("o", token_errors(o, oo, cu), tol, label)
    check("hT", state_errors(hT, ho), tol, label)


GRAD_NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


def check_grads(gr, ref, cu, tol, label=""):
    for name in GRAD_NAMES:
        if ref[name] is None:
            assert gr[name] is None, name
            continue
        assert gr[name] is not None, name
        errs = state_errors(gr[name], ref[name]) if name == "dh0" else token_errors(gr[name], ref[name], cu)
        check(name, errs, tol, label)


_CACHE = {}


def oracle_run(oracle_lib, wid):
    """(inputs, oracle forward (o, hT), oracle backward dict or None) of a
    numbered workload, computed once per session."""
    if wid not in _CACHE:
        x = synth.workload_inputs(wid)
        fw = oracle_lib.fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["cu_seqlens"])
        bw = None
        if synth.WORKLOADS[wid].backward:
            bw = oracle_lib.bwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["dO"], x["dhT"],
                                cu_seqlens=x["cu_seqlens"])
        _CACHE[wid] = (x, fw, bw)
    return _CACHE[wid]
