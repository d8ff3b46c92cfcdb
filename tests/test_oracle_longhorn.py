"""Pins of the oracle's Longhorn recurrence (Gated DeltaNet review thread,
Table 1, row "Longhorn": the delta-rule update at the step size
eps_t = beta_t / (1 + beta_t k_t^T k_t)).

- The update is the exact minimiser of the row's online-regression objective
  ||S - S_{t-1}||_F^2 + beta ||S k - v||^2 (checked by central differences of
  the objective at the oracle's state, with keys of non-unit norm, so a step
  size without the |k|^2 term or with it misplaced fails).
- A very large beta makes the write an exact overwrite: S_t k_t = v_t.
- Every gradient, including those through eps (dbeta and the extra key
  term), matches central differences of <dO, o> + <dhT, hT>.
"""
import numpy as np
import pytest

from test_oracle_pins import rand_inputs, rel


def test_longhorn_update_minimises_objective(oracle_lib):
    rng = np.random.default_rng(41)
    Dk, Dv = 5, 4
    S = rng.standard_normal((Dv, Dk)) * 0.5
    for _ in range(4):
        q = rng.standard_normal((1, 1, 1, Dk))
        k = rng.standard_normal((1, 1, 1, Dk)) * rng.uniform(0.3, 2.0)
        v = rng.standard_normal((1, 1, 1, Dv))
        be = rng.uniform(0.2, 3.0, (1, 1, 1))
        _, hT = oracle_lib.longhorn_fwd(q, k, v, be, None, S.T[None, None].copy())
        St = hT[0, 0].T
        kk, vv, b = k[0, 0, 0], v[0, 0, 0], float(be[0, 0, 0])

        def L(X):
            r = X @ kk - vv
            return np.sum((X - S) ** 2) + b * np.dot(r, r)
        h = 1e-3
        grad = np.zeros_like(St)
        for i in range(Dv):
            for j in range(Dk):
                E = np.zeros_like(St)
                E[i, j] = h
                grad[i, j] = (L(St + E) - L(St - E)) / (2 * h)
        assert np.abs(grad).max() < 1e-9
        for _ in range(5):
            d = rng.standard_normal(St.shape) * 0.1
            assert L(St + d) > L(St)
        S = St


def test_longhorn_large_beta_overwrites(oracle_lib):
    rng = np.random.default_rng(42)
    B, T, H, Dk, Dv = 1, 7, 2, 6, 3
    q, k, v, _, _, h0 = rand_inputs(rng, B, T, H, Dk, Dv, gated=False, h0=True, unit=False)
    bt = np.full((B, T, H), 1e9)
    for t in range(1, T + 1):
        _, hT = oracle_lib.longhorn_fwd(q[:, :t], k[:, :t], v[:, :t], bt[:, :t], None, h0)
        for h in range(H):
            recall = hT[0, h].T @ k[0, t - 1, h]
            assert rel(recall, v[0, t - 1, h]) < 1e-7


def _loss(oracle_lib, x, dO, dhT):
    o, hT = oracle_lib.longhorn_fwd(x["q"], x["k"], x["v"], x["beta"], x.get("g"), x.get("h0"))
    return float(np.sum(o * dO) + np.sum(hT * dhT))


@pytest.mark.parametrize("gated", [False, True])
def test_longhorn_backward_finite_differences(oracle_lib, gated):
    rng = np.random.default_rng(43)
    B, T, H, Dk, Dv = 2, 5, 2, 3, 2
    q, k, v, bt, g, h0 = rand_inputs(rng, B, T, H, Dk, Dv, gated, True, unit=False)
    bt = bt * 2.0
    dO = rng.standard_normal((B, T, H, Dv))
    dhT = rng.standard_normal((B, H, Dk, Dv))
    grads = oracle_lib.longhorn_bwd(q, k, v, bt, g, h0, dO, dhT)
    x = dict(q=q, k=k, v=v, beta=bt, h0=h0)
    names = dict(q="dq", k="dk", v="dv", beta="dbeta", h0="dh0")
    if gated:
        x["g"] = g
        names["g"] = "dg"
    h = 1e-6
    for name, gname in names.items():
        fd = np.zeros_like(x[name])
        it = np.nditer(x[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = {kk: vv.copy() for kk, vv in x.items()}
            xm = {kk: vv.copy() for kk, vv in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            fd[idx] = (_loss(oracle_lib, xp, dO, dhT) - _loss(oracle_lib, xm, dO, dhT)) / (2 * h)
        assert rel(grads[gname], fd) < 1e-7, (gname, rel(grads[gname], fd))
