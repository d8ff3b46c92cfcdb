"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle (``oracle/``) against something other than
itself: brute-force products of explicit transition matrices, closed forms of
special cases (no write, linear attention with orthonormal keys, overwrite),
the online-learning objective whose minimiser the update is, linearity and
state passing, finite differences for every gradient, and a hand-worked
example.  A dropped term, a wrong sign or index, or a transposed operand in
the oracle fails at least one of them.
"""
import os

import numpy as np
import pytest

import chunk_model

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_inputs(rng, B, T, H, Dk, Dv, gated=True, h0=True, beta=None, unit=True):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    bt = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H)))) if beta is None \
        else np.full((B, T, H), float(beta))
    g = -np.log1p(np.exp(rng.standard_normal((B, T, H)))) * 0.3 if gated else None
    hh = rng.standard_normal((B, H, Dk, Dv)) * 0.3 if h0 else None
    return q, k, v, bt, g, hh


def rel(x, y):
    d = np.linalg.norm(np.ravel(y))
    return np.linalg.norm(np.ravel(x - y)) / (d if d > 0 else 1.0)


# ---------------------------------------------------------------- brute force
def brute_force(q, k, v, beta, g, h0):
    """One (sequence, head): every transition as a dense matrix.

    S_t = S_0 prod_{l<=t} (alpha_l M_l) + sum_{j<=t} beta_j v_j k_j^T
          prod_{j<l<=t} (alpha_l M_l),  M_l = I - beta_l k_l k_l^T
    """
    T, Dk = k.shape
    Dv = v.shape[1]
    S0 = np.zeros((Dv, Dk)) if h0 is None else h0.T
    alpha = np.ones(T) if g is None else np.exp(g)
    Ms = [alpha[t] * (np.eye(Dk) - beta[t] * np.outer(k[t], k[t])) for t in range(T)]
    o = np.zeros((T, Dv))
    S = None
    for t in range(T):
        P = np.eye(Dk)
        for l in range(t + 1):
            P = P @ Ms[l]
        S = S0 @ P
        for j in range(t + 1):
            Pj = np.eye(Dk)
            for l in range(j + 1, t + 1):
                Pj = Pj @ Ms[l]
            S = S + beta[j] * np.outer(v[j], k[j]) @ Pj
        o[t] = S @ q[t]
    return o, (S.T if S is not None else S0.T)


@pytest.mark.parametrize("gated,use_h0", [(False, False), (True, True), (True, False)])
def test_p1_brute_force(oracle_lib, gated, use_h0):
    rng = np.random.default_rng(11)
    B, T, H, Dk, Dv = 2, 9, 2, 5, 4
    q, k, v, bt, g, h0 = rand_inputs(rng, B, T, H, Dk, Dv, gated, use_h0)
    o, hT = oracle_lib.fwd(q, k, v, bt, g, h0)
    for b in range(B):
        for h in range(H):
            ob, hb = brute_force(q[b, :, h], k[b, :, h], v[b, :, h], bt[b, :, h],
                                 None if g is None else g[b, :, h],
                                 None if h0 is None else h0[b, h])
            assert rel(o[b, :, h], ob) < 1e-12
            assert rel(hT[b, h], hb) < 1e-12


def test_p1_brute_force_nonunit_keys(oracle_lib):
    # the rule does not need unit keys; keep beta |k|^2 < 2 for stability
    rng = np.random.default_rng(12)
    q, k, v, bt, g, h0 = rand_inputs(rng, 1, 7, 1, 3, 6, True, True, unit=False)
    k *= 0.5
    o, hT = oracle_lib.fwd(q, k, v, bt, g, h0)
    ob, hb = brute_force(q[0, :, 0], k[0, :, 0], v[0, :, 0], bt[0, :, 0], g[0, :, 0], h0[0, 0])
    assert rel(o[0, :, 0], ob) < 1e-12 and rel(hT[0, 0], hb) < 1e-12


# ------------------------------------------------------------- hand-worked
def test_golden_handworked(oracle_lib):
    rows, hT_ref = [], None
    with open(os.path.join(HERE, "golden", "handworked_2d.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "hT":
                hT_ref = np.array([float(x) for x in parts[1:]]).reshape(2, 2)
            else:
                rows.append([float(x) for x in parts[1:]])
    rows = np.array(rows)
    T = len(rows)
    k = rows[:, 0:2].reshape(1, T, 1, 2)
    v = rows[:, 2:4].reshape(1, T, 1, 2)
    bt = rows[:, 4].reshape(1, T, 1)
    g = np.log(rows[:, 5]).reshape(1, T, 1)
    q = rows[:, 6:8].reshape(1, T, 1, 2)
    o_ref = rows[:, 8:10]
    o, hT = oracle_lib.fwd(q, k, v, bt, g, None)
    np.testing.assert_allclose(o[0, :, 0], o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(hT[0, 0], hT_ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------ special cases
def test_p2_no_write_only_decays(oracle_lib):
    rng = np.random.default_rng(2)
    B, T, H, Dk, Dv = 2, 40, 3, 6, 5
    q, k, v, _, g, h0 = rand_inputs(rng, B, T, H, Dk, Dv, True, True)
    bt = np.zeros((B, T, H))
    o, hT = oracle_lib.fwd(q, k, v, bt, g, h0)
    bcum = np.cumsum(g, axis=1)  # [B,T,H]
    np.testing.assert_allclose(hT, np.exp(bcum[:, -1])[:, :, None, None] * h0, rtol=1e-12, atol=0)
    o_ref = np.exp(bcum)[..., None] * np.einsum("bhkv,bthk->bthv", h0, q)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-14)
    # with no initial state nothing is ever written: exactly zero
    o0, hT0 = oracle_lib.fwd(q, k, v, bt, g, None)
    assert not o0.any() and not hT0.any()


def test_p3_orthonormal_keys_reduce_to_decayed_linear_attention(oracle_lib):
    # beta = 1 and orthonormal keys: each write lands in its own direction, so
    # the rule reduces to (decayed) linear attention, Table 1 rows LA / Mamba2:
    # o = ((Q K^T) * D) V with D_rj = exp(b_r - b_j) [j <= r]
    rng = np.random.default_rng(3)
    T, Dk, Dv = 12, 16, 7
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    k = Qm[:T].reshape(1, T, 1, Dk)
    q = rng.standard_normal((1, T, 1, Dk))
    v = rng.standard_normal((1, T, 1, Dv))
    for gated in (False, True):
        g = (-np.abs(rng.standard_normal((1, T, 1))) * 0.2) if gated else None
        bt = np.ones((1, T, 1))
        o, hT = oracle_lib.fwd(q, k, v, bt, g, None)
        b = np.cumsum(g[0, :, 0]) if gated else np.zeros(T)
        D = np.tril(np.exp(b[:, None] - b[None, :]))
        o_ref = ((q[0, :, 0] @ k[0, :, 0].T) * D) @ v[0, :, 0]
        np.testing.assert_allclose(o[0, :, 0], o_ref, rtol=1e-12, atol=1e-12)
        # exact recall: S_T k_j = (prod_{l>j} alpha_l) v_j
        S = hT[0, 0].T
        for j in range(T):
            np.testing.assert_allclose(S @ k[0, j, 0], np.exp(b[-1] - b[j]) * v[0, j, 0],
                                       rtol=1e-12, atol=1e-12)


def test_p4_overwrite(oracle_lib):
    rng = np.random.default_rng(4)
    Dk, Dv = 8, 5
    kk = rng.standard_normal(Dk)
    kk /= np.linalg.norm(kk)
    others = rng.standard_normal((3, Dk))
    others /= np.linalg.norm(others, axis=1, keepdims=True)
    keys = np.stack([kk, others[0], others[1], others[2], kk])
    vals = rng.standard_normal((5, Dv))
    bt = np.array([1.0, 0.4, 0.7, 0.2, 1.0])
    T = 5
    o, hT = oracle_lib.fwd(np.zeros((1, T, 1, Dk)), keys.reshape(1, T, 1, Dk),
                           vals.reshape(1, T, 1, Dv), bt.reshape(1, T, 1), None, None)
    # whatever was stored under kk is replaced by the last value written there
    np.testing.assert_allclose(hT[0, 0].T @ kk, vals[-1], rtol=1e-12, atol=1e-12)


def test_p5_update_minimises_table1_objective(oracle_lib):
    # Gated DeltaNet row of Table 1: S_t minimises
    # L(S) = ||S - a S_{t-1}||_F^2 - 2 <S k, beta (v - a S_{t-1} k)>.
    rng = np.random.default_rng(5)
    B, H, Dk, Dv = 2, 2, 5, 4
    state = rng.standard_normal((B, H, Dk, Dv)) * 0.5
    for _ in range(3):
        q = rng.standard_normal((B, H, Dk))
        k = rng.standard_normal((B, H, Dk))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((B, H, Dv))
        bt = rng.uniform(0.1, 0.9, (B, H))
        g = -rng.uniform(0.0, 0.5, (B, H))
        _, new = oracle_lib.step(q, k, v, bt, g, state)
        for b in range(B):
            for h in range(H):
                a = np.exp(g[b, h])
                Sp = state[b, h].T
                St = new[b, h].T
                kk, vv, be = k[b, h], v[b, h], bt[b, h]

                def L(S):
                    return (np.sum((S - a * Sp) ** 2)
                            - 2.0 * np.dot(S @ kk, be * (vv - a * Sp @ kk)))
                # central differences of a quadratic are exact up to rounding
                eps = 1e-3
                grad = np.zeros_like(St)
                for i in range(Dv):
                    for j in range(Dk):
                        E = np.zeros_like(St)
                        E[i, j] = eps
                        grad[i, j] = (L(St + E) - L(St - E)) / (2 * eps)
                assert np.abs(grad).max() < 1e-9
                for _ in range(5):
                    d = rng.standard_normal(St.shape) * 0.1
                    assert L(St + d) > L(St)
        state = new


def test_p6_linearity_and_state_passing(oracle_lib):
    rng = np.random.default_rng(6)
    B, T, H, Dk, Dv = 2, 50, 2, 6, 5
    q, k, v, bt, g, h0 = rand_inputs(rng, B, T, H, Dk, Dv, True, True)
    v2 = rng.standard_normal(v.shape)
    h02 = rng.standard_normal(h0.shape)
    a1, a2 = 0.7, -1.3
    o1, s1 = oracle_lib.fwd(q, k, v, bt, g, h0)
    o2, s2 = oracle_lib.fwd(q, k, v2, bt, g, h02)
    o3, s3 = oracle_lib.fwd(q, k, a1 * v + a2 * v2, bt, g, a1 * h0 + a2 * h02)
    assert rel(o3, a1 * o1 + a2 * o2) < 1e-12
    assert rel(s3, a1 * s1 + a2 * s2) < 1e-12
    # state passing: [0, T1) then [T1, T) from the carried state == one run
    T1 = 23
    oa, sa = oracle_lib.fwd(q[:, :T1], k[:, :T1], v[:, :T1], bt[:, :T1], g[:, :T1], h0)
    ob, sb = oracle_lib.fwd(q[:, T1:], k[:, T1:], v[:, T1:], bt[:, T1:], g[:, T1:], sa)
    assert rel(np.concatenate([oa, ob], axis=1), o1) < 1e-13
    assert rel(sb, s1) < 1e-13


def test_p7_varlen_equals_separate_runs_and_decode_steps(oracle_lib):
    rng = np.random.default_rng(7)
    lens = [1, 63, 64, 65, 0, 130, 7]
    Ttot = sum(lens)
    H, Dk, Dv = 2, 6, 4
    q, k, v, bt, g, _ = rand_inputs(rng, 1, Ttot, H, Dk, Dv, True, False)
    N = len(lens)
    h0 = rng.standard_normal((N, H, Dk, Dv)) * 0.3
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, hT = oracle_lib.fwd(q, k, v, bt, g, h0, cu_seqlens=cu)
    for n in range(N):
        s, e = cu[n], cu[n + 1]
        on, hn = oracle_lib.fwd(q[:, s:e], k[:, s:e], v[:, s:e], bt[:, s:e], g[:, s:e],
                                h0[n:n + 1]) if e > s else (np.zeros((1, 0, H, Dv)), h0[n:n + 1])
        assert np.array_equal(o[:, s:e], on)
        assert np.array_equal(hT[n:n + 1], hn)
    # an empty sequence returns its initial state
    assert np.array_equal(hT[4], h0[4])
    # T decode steps equal the whole forward pass
    n = 5
    s, e = cu[n], cu[n + 1]
    state = h0[n][None].copy()
    outs = []
    for t in range(s, e):
        ot, state = oracle_lib.step(q[:, t], k[:, t], v[:, t], bt[:, t], g[:, t], state)
        outs.append(ot)
    assert rel(np.stack(outs, axis=1), o[:, s:e]) < 1e-13
    assert rel(state[0], hT[n]) < 1e-13


@pytest.mark.parametrize("C", [1, 2, 16, 32, 64, 100, 1000])
@pytest.mark.parametrize("gated", [False, True])
def test_p8_chunk_algebra_matches_oracle(oracle_lib, C, gated):
    rng = np.random.default_rng(80 + C)
    T, Dk, Dv = 150, 12, 10
    q, k, v, bt, g, h0 = rand_inputs(rng, 1, T, 1, Dk, Dv, gated, True)
    o, hT = oracle_lib.fwd(q, k, v, bt, g, h0)
    om, hm, _ = chunk_model.fwd_seq(q[0, :, 0], k[0, :, 0], v[0, :, 0], bt[0, :, 0],
                                    None if g is None else g[0, :, 0], h0[0, 0], C)
    assert rel(om, o[0, :, 0]) < 1e-12
    assert rel(hm, hT[0, 0]) < 1e-12


def test_p8_forward_substitution_inverts():
    rng = np.random.default_rng(81)
    K = rng.standard_normal((64, 32))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    bt = rng.uniform(0, 1, 64)
    g = -rng.uniform(0, 0.1, 64)
    _, _, _, A, R = chunk_model.chunk_prep(K, bt, g)
    assert np.abs((np.eye(64) + A) @ R - np.eye(64)).max() < 1e-13
    assert np.allclose(R, np.linalg.inv(np.eye(64) + A), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ backward
def loss(oracle_lib, x, dO, dhT):
    o, hT = oracle_lib.fwd(x["q"], x["k"], x["v"], x["beta"], x.get("g"), x.get("h0"))
    return float(np.sum(o * dO) + np.sum(hT * dhT))


@pytest.mark.parametrize("gated", [False, True])
def test_p9_backward_finite_differences(oracle_lib, gated):
    rng = np.random.default_rng(9)
    B, T, H, Dk, Dv = 2, 6, 2, 3, 2
    q, k, v, bt, g, h0 = rand_inputs(rng, B, T, H, Dk, Dv, gated, True)
    dO = rng.standard_normal((B, T, H, Dv))
    dhT = rng.standard_normal((B, H, Dk, Dv))
    grads = oracle_lib.bwd(q, k, v, bt, g, h0, dO, dhT)
    x = dict(q=q, k=k, v=v, beta=bt, h0=h0)
    names = dict(q="dq", k="dk", v="dv", beta="dbeta", h0="dh0")
    if gated:
        x["g"] = g
        names["g"] = "dg"
    eps = 1e-6
    for name, gname in names.items():
        fd = np.zeros_like(x[name])
        it = np.nditer(x[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = {kk: vv.copy() for kk, vv in x.items()}
            xm = {kk: vv.copy() for kk, vv in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd[idx] = (loss(oracle_lib, xp, dO, dhT) - loss(oracle_lib, xm, dO, dhT)) / (2 * eps)
        assert rel(grads[gname], fd) < 1e-7, (gname, rel(grads[gname], fd))
    if not gated:
        assert grads["dg"] is None


def test_p9_backward_directional_derivative(oracle_lib):
    rng = np.random.default_rng(19)
    B, T, H, Dk, Dv = 1, 150, 2, 16, 12
    q, k, v, bt, g, h0 = rand_inputs(rng, B, T, H, Dk, Dv, True, True)
    dO = rng.standard_normal((B, T, H, Dv))
    dhT = rng.standard_normal((B, H, Dk, Dv))
    gr = oracle_lib.bwd(q, k, v, bt, g, h0, dO, dhT)
    x = dict(q=q, k=k, v=v, beta=bt, g=g, h0=h0)
    gmap = dict(q="dq", k="dk", v="dv", beta="dbeta", g="dg", h0="dh0")
    d = {kk: rng.standard_normal(vv.shape) for kk, vv in x.items()}
    eps = 1e-5
    xp = {kk: x[kk] + eps * d[kk] for kk in x}
    xm = {kk: x[kk] - eps * d[kk] for kk in x}
    fd = (loss(oracle_lib, xp, dO, dhT) - loss(oracle_lib, xm, dO, dhT)) / (2 * eps)
    an = sum(float(np.sum(gr[gmap[kk]] * d[kk])) for kk in x)
    assert abs(fd - an) < 1e-7 * max(1.0, abs(an))


def test_p10_no_write_gradient_closed_form(oracle_lib):
    rng = np.random.default_rng(10)
    B, T, H, Dk, Dv = 2, 30, 2, 5, 4
    q, k, v, _, g, h0 = rand_inputs(rng, B, T, H, Dk, Dv, True, True)
    bt = np.zeros((B, T, H))
    dO = rng.standard_normal((B, T, H, Dv))
    dhT = rng.standard_normal((B, H, Dk, Dv))
    o, hT = oracle_lib.fwd(q, k, v, bt, g, h0)
    gr = oracle_lib.bwd(q, k, v, bt, g, h0, dO, dhT)
    per_t = np.sum(dO * o, axis=-1)  # [B,T,H]
    tail = np.cumsum(per_t[:, ::-1], axis=1)[:, ::-1]
    dg_ref = tail + np.sum(dhT * hT, axis=(-1, -2))[:, None, :]
    np.testing.assert_allclose(gr["dg"], dg_ref, rtol=1e-11, atol=1e-12)
    assert not gr["dv"].any()
    bc = np.cumsum(g, axis=1)
    dq_ref = np.exp(bc)[..., None] * np.einsum("bhkv,bthv->bthk", h0, dO)
    np.testing.assert_allclose(gr["dq"], dq_ref, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("C", [1, 16, 32, 64, 100])
@pytest.mark.parametrize("gated", [False, True])
def test_p8_chunk_backward_matches_oracle(oracle_lib, C, gated):
    rng = np.random.default_rng(90 + C)
    T, Dk, Dv = 150, 10, 8
    q, k, v, bt, g, h0 = rand_inputs(rng, 1, T, 1, Dk, Dv, gated, True)
    dO = rng.standard_normal((1, T, 1, Dv))
    dhT = rng.standard_normal((1, 1, Dk, Dv))
    gr = oracle_lib.bwd(q, k, v, bt, g, h0, dO, dhT)
    dq, dk, dv, db, dg, dh0 = chunk_model.bwd_seq(
        q[0, :, 0], k[0, :, 0], v[0, :, 0], bt[0, :, 0], None if g is None else g[0, :, 0],
        h0[0, 0], dO[0, :, 0], dhT[0, 0], C)
    assert rel(dq, gr["dq"][0, :, 0]) < 1e-11
    assert rel(dk, gr["dk"][0, :, 0]) < 1e-11
    assert rel(dv, gr["dv"][0, :, 0]) < 1e-11
    assert rel(db, gr["dbeta"][0, :, 0]) < 1e-11
    assert rel(dh0, gr["dh0"][0, 0]) < 1e-11
    if gated:
        assert rel(dg, gr["dg"][0, :, 0]) < 1e-11


def test_p9_varlen_backward_equals_separate_runs(oracle_lib):
    rng = np.random.default_rng(29)
    lens = [5, 0, 70, 64]
    H, Dk, Dv = 2, 4, 3
    q, k, v, bt, g, _ = rand_inputs(rng, 1, sum(lens), H, Dk, Dv, True, False)
    N = len(lens)
    h0 = rng.standard_normal((N, H, Dk, Dv))
    dO = rng.standard_normal(v.shape)
    dhT = rng.standard_normal((N, H, Dk, Dv))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    gr = oracle_lib.bwd(q, k, v, bt, g, h0, dO, dhT, cu_seqlens=cu)
    for n in range(N):
        s, e = cu[n], cu[n + 1]
        if e == s:
            assert np.array_equal(gr["dh0"][n], dhT[n])
            continue
        gn = oracle_lib.bwd(q[:, s:e], k[:, s:e], v[:, s:e], bt[:, s:e], g[:, s:e],
                            h0[n:n + 1], dO[:, s:e], dhT[n:n + 1])
        for key in ("dq", "dk", "dv", "dbeta", "dg"):
            assert np.array_equal(gr[key][:, s:e], gn[key])
        assert np.array_equal(gr["dh0"][n:n + 1], gn["dh0"])


def test_p11_state_norm_bound(oracle_lib):
    # unit keys, beta in (0,1), alpha <= 1: each transition has spectral norm
    # <= 1, so ||S_T||_2 <= ||S_0||_2 + sum_t beta_t ||v_t||
    rng = np.random.default_rng(111)
    B, T, H, Dk, Dv = 1, 300, 3, 8, 8
    q, k, v, bt, g, h0 = rand_inputs(rng, B, T, H, Dk, Dv, True, True)
    _, hT = oracle_lib.fwd(q, k, v, bt, g, h0)
    for h in range(H):
        bound = np.linalg.norm(h0[0, h], 2) + np.sum(bt[0, :, h] * np.linalg.norm(v[0, :, h], axis=-1))
        assert np.linalg.norm(hT[0, h], 2) <= bound * (1 + 1e-12)


def test_oracle_rejects_bad_dims(oracle_lib):
    z = np.zeros((1, 4, 1, 2))
    with pytest.raises(ValueError):
        # varlen with B != 1
        oracle_lib.fwd(np.zeros((2, 4, 1, 2)), np.zeros((2, 4, 1, 2)), np.zeros((2, 4, 1, 2)),
                       np.zeros((2, 4, 1)), None, None, cu_seqlens=np.array([0, 4], np.int32))
    with pytest.raises(ValueError):
        # dg requested without a gate is impossible: bwd with g=None gives dg None,
        # so exercise the C check through a gated dg/g mismatch at the C level
        lib = oracle_lib._load()
        import ctypes
        p = z.ctypes.data_as(ctypes.c_void_p)
        rc = lib.oracle_bwd(1, 4, 1, 2, 2, 1, None, p, p, p, p, None, None, p, None,
                            p, p, p, p, p, None, 1)
        if rc:
            raise ValueError(rc)
